// Attainable peaks of the chip, measured by kernels that do nothing else, as
// the measured denominators beside the published ones (MI355X: dense fp16
// MFMA 2.5 PFLOP/s, fp32 MFMA 157.3 TFLOP/s, HBM 8 TB/s).  Not part of the
// quantization path; built into its own library (libgptq_peaks.so).
//
//   which 0: v_mfma_f32_32x32x16_f16 stream, 1: v_mfma_f32_32x32x2_f32
//   stream (eight independent accumulators per wave, operands from random
//   bits so the matrix pipe sees realistic toggling); 2: HBM read (16-byte
//   loads, eight in flight per thread, grid-stride); 3: HBM copy (16-byte
//   loads and stores).
//
// int gptq_peaks_launch(int which, const void* src, void* dst, size_t bytes,
//                       int iters, int grid, void* stream)
//   src: which 0/1: at least 256 * grid * 16 bytes of random bits; 2/3: the
//   buffer read (bytes, a multiple of 16).  dst: which 0/1: grid * 256
//   floats; 2: grid * 256 words; 3: bytes to write.  iters: MFMA passes of
//   16 instructions per wave (0/1 only).  Returns the hipError_t of the
//   launch; -1 for an unknown which or a bad size.
#include <hip/hip_runtime.h>

#include <cstdint>

namespace {

typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef _Float16 half8 __attribute__((ext_vector_type(8)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

template <int KIND>
__global__ __launch_bounds__(256) void mfma_stream_kernel(const u32x4* bits, float* out, int iters) {
  const int tid = threadIdx.x, lane = tid & 63;
  const u32x4 r = bits[blockIdx.x * 256 + tid];
  f32x16 acc[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) acc[i] = f32x16{};
  if (KIND == 0) {
    // fp16 magnitudes below 1 (exponent field at most 14): finite sums
    const u32x4 a = r & 0x3BFF3BFFu, b = (r >> 1) & 0x3BFF3BFFu;
    const half8 ha = __builtin_bit_cast(half8, a), hb = __builtin_bit_cast(half8, b);
    for (int it = 0; it < iters; ++it) {
#pragma unroll
      for (int i = 0; i < 16; ++i) acc[i & 7] = __builtin_amdgcn_mfma_f32_32x32x16_f16(ha, hb, acc[i & 7], 0, 0, 0);
    }
  } else {
    const float fa = __builtin_bit_cast(float, (r.x & 0x007FFFFFu) | 0x3F000000u);  // [0.5, 1)
    const float fb = __builtin_bit_cast(float, (r.y & 0x007FFFFFu) | 0x3F000000u);
    for (int it = 0; it < iters; ++it) {
#pragma unroll
      for (int i = 0; i < 16; ++i) acc[i & 7] = __builtin_amdgcn_mfma_f32_32x32x2f32(fa, fb, acc[i & 7], 0, 0, 0);
    }
  }
  float s = 0.f;
#pragma unroll
  for (int i = 0; i < 8; ++i) s += acc[i][lane & 15];
  out[blockIdx.x * 256 + tid] = s;
}

__global__ __launch_bounds__(256) void read_stream_kernel(const u32x4* p, int64_t n16, uint32_t* out) {
  const int64_t stride = (int64_t)gridDim.x * 256;
  int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  u32x4 acc = {0u, 0u, 0u, 0u};
  for (; i + 7 * stride < n16; i += 8 * stride) {
    u32x4 v[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) v[u] = __builtin_nontemporal_load(p + i + u * stride);
#pragma unroll
    for (int u = 0; u < 8; ++u) acc ^= v[u];
  }
  for (; i < n16; i += stride) acc ^= p[i];
  out[(int64_t)blockIdx.x * 256 + threadIdx.x] = acc.x ^ acc.y ^ acc.z ^ acc.w;
}

__global__ __launch_bounds__(256) void copy_stream_kernel(const u32x4* src, u32x4* dst, int64_t n16) {
  const int64_t stride = (int64_t)gridDim.x * 256;
  int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  for (; i + 3 * stride < n16; i += 4 * stride) {
    u32x4 v[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) v[u] = __builtin_nontemporal_load(src + i + u * stride);
#pragma unroll
    for (int u = 0; u < 4; ++u) __builtin_nontemporal_store(v[u], dst + i + u * stride);
  }
  for (; i < n16; i += stride) dst[i] = src[i];
}

}  // namespace

extern "C" int gptq_peaks_launch(int which, const void* src, void* dst, size_t bytes, int iters, int grid,
                                 void* stream) {
  hipStream_t s = (hipStream_t)stream;
  if (grid < 1 || (which >= 2 && (bytes == 0 || bytes % 16 != 0))) return -1;
  switch (which) {
    case 0:
      hipLaunchKernelGGL(mfma_stream_kernel<0>, dim3(grid), dim3(256), 0, s, (const u32x4*)src, (float*)dst, iters);
      break;
    case 1:
      hipLaunchKernelGGL(mfma_stream_kernel<1>, dim3(grid), dim3(256), 0, s, (const u32x4*)src, (float*)dst, iters);
      break;
    case 2:
      hipLaunchKernelGGL(read_stream_kernel, dim3(grid), dim3(256), 0, s, (const u32x4*)src, (int64_t)(bytes / 16),
                         (uint32_t*)dst);
      break;
    case 3:
      hipLaunchKernelGGL(copy_stream_kernel, dim3(grid), dim3(256), 0, s, (const u32x4*)src, (u32x4*)dst,
                         (int64_t)(bytes / 16));
      break;
    default:
      return -1;
  }
  return (int)hipGetLastError();
}
