// Elementwise steps of the network-level loop over MLP blocks (one layer at
// a time, each layer's calibration inputs computed by the network as
// quantized so far: "Part 3: Adaptive Rounding: GPTQ", 'Algorithm GPTQ'; the
// English GPTQ second-order quantization post, 'Calibration for a multimodal
// or VLA backbone').  The block is x <- x + W_down (silu(W_gate x) * (W_up x));
// the three products run in gptq_dequant_matmul, these kernels do the rest:
//   swiglu:        A = silu(G) * U, silu(v) = v / (1 + e^-v), in fp32, one
//                  rounding to the activations' dtype;
//   residual add:  X <- X + Y in fp32, one rounding.
// HBM-bound: 8 elements (16 bytes) per thread and access when rows allow.
#include <cmath>

#include "common.hpp"
#include "internal.hpp"

namespace gptq {

namespace {

template <int DT>
__device__ __forceinline__ float ld1(const void* p, int64_t i) {
  return Elem<DT>::load(p, i);
}

template <int DT>
__device__ __forceinline__ void unpack8(u32x4 v, float (&f)[8]) {
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    const uint32_t w = v[e];  // copied: a bit cast of the vector element itself would read element 0
    if (DT == 0) {
      f[2 * e] = (float)__builtin_bit_cast(_Float16, (uint16_t)(w & 0xFFFFu));
      f[2 * e + 1] = (float)__builtin_bit_cast(_Float16, (uint16_t)(w >> 16));
    } else {
      f[2 * e] = __builtin_bit_cast(float, w << 16);
      f[2 * e + 1] = __builtin_bit_cast(float, w & 0xFFFF0000u);
    }
  }
}

template <int DT>
__device__ __forceinline__ u32x4 pack8(const float (&f)[8]) {
  u32x4 v;
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    uint32_t lo, hi;
    if (DT == 0) {
      lo = __builtin_bit_cast(uint16_t, (_Float16)f[2 * e]);
      hi = __builtin_bit_cast(uint16_t, (_Float16)f[2 * e + 1]);
    } else {
      lo = f32_to_bf16(f[2 * e]);
      hi = f32_to_bf16(f[2 * e + 1]);
    }
    v[e] = lo | (hi << 16);
  }
  return v;
}

__device__ __forceinline__ float silu_mul(float g, float u) { return g / (1.0f + expf(-g)) * u; }

// OP 0: out = silu(a) * b;  OP 1: out = a + b (out may be a)
template <int DT, int OP>
__global__ __launch_bounds__(256) void ew8_kernel(const void* a, const void* b, void* out, int64_t rows, int64_t cols,
                                                  int64_t ld) {
  const int64_t per_row = cols / 8;
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i >= rows * per_row) return;
  const int64_t r = i / per_row, c = (i - r * per_row) * 8;
  const int64_t off = r * ld + c;
  float fa[8], fb[8], fo[8];
  unpack8<DT>(*(const u32x4*)((const uint16_t*)a + off), fa);
  unpack8<DT>(*(const u32x4*)((const uint16_t*)b + off), fb);
#pragma unroll
  for (int e = 0; e < 8; ++e) fo[e] = OP == 0 ? silu_mul(fa[e], fb[e]) : fa[e] + fb[e];
  *(u32x4*)((uint16_t*)out + off) = pack8<DT>(fo);
}

template <int DT, int OP>
__global__ __launch_bounds__(256) void ew1_kernel(const void* a, const void* b, void* out, int64_t rows, int64_t cols,
                                                  int64_t ld) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i >= rows * cols) return;
  const int64_t r = i / cols, off = r * ld + (i - r * cols);
  const float x = ld1<DT>(a, off), y = ld1<DT>(b, off);
  Elem<DT>::store(out, off, OP == 0 ? silu_mul(x, y) : x + y);
}

template <int OP>
hipError_t ew_launch(const void* a, const void* b, void* out, int dt, int64_t rows, int64_t cols, int64_t ld,
                     hipStream_t st) {
  const bool vec = cols % 8 == 0 && ld % 8 == 0 && ((((uintptr_t)a) | ((uintptr_t)b) | ((uintptr_t)out)) & 15) == 0;
  const int64_t items = vec ? rows * (cols / 8) : rows * cols;
  const dim3 grid((unsigned)cdiv(items, 256));
  if (vec) {
    if (dt == 0) hipLaunchKernelGGL((ew8_kernel<0, OP>), grid, dim3(256), 0, st, a, b, out, rows, cols, ld);
    else hipLaunchKernelGGL((ew8_kernel<1, OP>), grid, dim3(256), 0, st, a, b, out, rows, cols, ld);
  } else {
    if (dt == 0) hipLaunchKernelGGL((ew1_kernel<0, OP>), grid, dim3(256), 0, st, a, b, out, rows, cols, ld);
    else hipLaunchKernelGGL((ew1_kernel<1, OP>), grid, dim3(256), 0, st, a, b, out, rows, cols, ld);
  }
  return hipGetLastError();
}

}  // namespace

hipError_t swiglu(const void* G, const void* U, void* A, int dt, int64_t rows, int64_t cols, int64_t ld,
                  hipStream_t st) {
  return ew_launch<0>(G, U, A, dt, rows, cols, ld, st);
}

hipError_t residual_add(void* X, const void* Y, int dt, int64_t rows, int64_t cols, int64_t ld, hipStream_t st) {
  return ew_launch<1>(X, Y, X, dt, rows, cols, ld, st);
}

}  // namespace gptq
