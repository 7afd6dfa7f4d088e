// Fixed rotation before GPTQ, in place on the rows of a matrix:
// M <- M R with R = blockdiag(H_b, ..., H_b) / sqrt(b), H_b the
// Sylvester-ordered Hadamard matrix of order b (a power of two, 16 <= b <=
// 4096, dividing the row length).  Rotating both the weights (W' = W R) and
// the calibration activations (X' = X R) leaves the layer output unchanged
// and gives H' = R^T H R; GPTQ then quantizes W' (OptRot, abstract and
// Figure 1: the rotation folds into the previous layer, and spreading weight
// outliers lowers the error bound of its Theorem 3.1, which grows with the
// weight incoherence).
//
// How: a workgroup takes 4096 consecutive elements of the segment sequence
// (4096 / b segments), 16 per thread, and runs the fast Walsh-Hadamard
// transform in fp32: the butterflies (a, c) -> (a + c, a - c) on bit k of
// the in-segment index pair elements k apart.  Bits 0-3 are done in
// registers on the thread's 16 contiguous elements; two transposes through
// LDS (rows of 16 floats padded to 17, so every access pattern used hits
// distinct banks) put bits 4-7 and then 8-11 into the registers; a third
// puts the elements back for 16-byte stores.  Only the bits below log2(b)
// are transformed.  HBM-bound: each element is read and written once.
#include "common.hpp"
#include "internal.hpp"

namespace gptq {

namespace {

constexpr int RV = 4096;   // elements per workgroup
constexpr int RPAD = 17;   // LDS floats per 16 elements

// butterflies of register bits 0..nb-1 (nb <= 4; uniform)
__device__ __forceinline__ void butterflies(float (&r)[16], int nb) {
#pragma unroll
  for (int s = 0; s < 4; ++s) {
    if (s < nb) {
      const int h = 1 << s;
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        if (!(i & h)) {
          const float a = r[i], c = r[i + h];
          r[i] = a + c;
          r[i + h] = a - c;
        }
      }
    }
  }
}

template <int DT>
__device__ __forceinline__ void load16(const void* base, int64_t off, bool ok, float (&r)[16]) {
  if (DT == 2) {
    const f32x4* p = (const f32x4*)((const float*)base + off);
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const f32x4 v = ok ? p[q] : f32x4{0.f, 0.f, 0.f, 0.f};
      r[4 * q] = v[0]; r[4 * q + 1] = v[1]; r[4 * q + 2] = v[2]; r[4 * q + 3] = v[3];
    }
  } else {
    const u32x4* p = (const u32x4*)((const uint16_t*)base + off);
#pragma unroll
    for (int q = 0; q < 2; ++q) {
      const u32x4 v = ok ? p[q] : u32x4{0u, 0u, 0u, 0u};
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const uint32_t w = v[e];  // copy first: a bit cast of the element itself would read element 0
        const uint32_t lo = w & 0xFFFFu, hi = w >> 16;
        if (DT == 0) {
          r[8 * q + 2 * e] = (float)__builtin_bit_cast(_Float16, (uint16_t)lo);
          r[8 * q + 2 * e + 1] = (float)__builtin_bit_cast(_Float16, (uint16_t)hi);
        } else {
          r[8 * q + 2 * e] = __builtin_bit_cast(float, lo << 16);
          r[8 * q + 2 * e + 1] = __builtin_bit_cast(float, hi << 16);
        }
      }
    }
  }
}

template <int DT>
__device__ __forceinline__ void store16(void* base, int64_t off, const float (&r)[16]) {
  if (DT == 2) {
    f32x4* p = (f32x4*)((float*)base + off);
#pragma unroll
    for (int q = 0; q < 4; ++q) p[q] = f32x4{r[4 * q], r[4 * q + 1], r[4 * q + 2], r[4 * q + 3]};
  } else {
    u32x4* p = (u32x4*)((uint16_t*)base + off);
#pragma unroll
    for (int q = 0; q < 2; ++q) {
      u32x4 v;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        uint32_t lo, hi;
        if (DT == 0) {
          lo = __builtin_bit_cast(uint16_t, (_Float16)r[8 * q + 2 * e]);
          hi = __builtin_bit_cast(uint16_t, (_Float16)r[8 * q + 2 * e + 1]);
        } else {
          lo = f32_to_bf16(r[8 * q + 2 * e]);
          hi = f32_to_bf16(r[8 * q + 2 * e + 1]);
        }
        v[e] = lo | (hi << 16);
      }
      p[q] = v;
    }
  }
}

template <int DT>
__global__ __launch_bounds__(256) void hadamard_rows_kernel(void* M, int64_t rows, int64_t n, int64_t ld, int lb,
                                                            float scale) {
  __shared__ float sm[256 * RPAD];
  const int t = threadIdx.x;
  const int64_t spr = n >> lb;  // segments per row
  const int64_t nseg = rows * spr;
  const int64_t g = (int64_t)blockIdx.x * (RV >> lb) + ((16 * t) >> lb);  // this thread's segment
  const bool ok = g < nseg;
  const int64_t row = ok ? g / spr : 0;
  const int64_t off = row * ld + ((ok ? g - row * spr : 0) << lb) + ((16 * t) & ((1 << lb) - 1));
  float r[16];
  load16<DT>(M, off, ok, r);
  butterflies(r, min(lb, 4));  // in-segment bits 0..3
  if (lb > 4) {
    // bits 4..7: thread t takes v = (t >> 4) << 8 | j << 4 | (t & 15)
    const int p2 = RPAD * ((t >> 4) << 4) + (t & 15);
#pragma unroll
    for (int j = 0; j < 16; ++j) sm[RPAD * t + j] = r[j];
    __syncthreads();
#pragma unroll
    for (int j = 0; j < 16; ++j) r[j] = sm[p2 + RPAD * j];
    butterflies(r, min(lb - 4, 4));
    // every position is read by one thread only, so each writes back its own
#pragma unroll
    for (int j = 0; j < 16; ++j) sm[p2 + RPAD * j] = r[j];
    if (lb > 8) {
      // bits 8..11: thread t takes v = j << 8 | t
      const int p3 = RPAD * (t >> 4) + (t & 15);
      __syncthreads();
#pragma unroll
      for (int j = 0; j < 16; ++j) r[j] = sm[p3 + 16 * RPAD * j];
      butterflies(r, lb - 8);
#pragma unroll
      for (int j = 0; j < 16; ++j) sm[p3 + 16 * RPAD * j] = r[j];
    }
    __syncthreads();
#pragma unroll
    for (int j = 0; j < 16; ++j) r[j] = sm[RPAD * t + j];
  }
#pragma unroll
  for (int j = 0; j < 16; ++j) r[j] *= scale;
  if (ok) store16<DT>(M, off, r);
}

}  // namespace

int rotation_block(int64_t n, int64_t block) {
  if (block > 0) return (int)block;
  int b = 1;
  while (n % (2 * b) == 0 && 2 * b <= RV) b *= 2;
  return b;
}

bool rotation_supported(int64_t n, int64_t block) {
  const int64_t b = rotation_block(n, block);
  return b >= 16 && b <= RV && (b & (b - 1)) == 0 && n % b == 0;
}

hipError_t rotate_hadamard(void* M, int dt, int64_t rows, int64_t n, int64_t ld, int64_t block, hipStream_t st) {
  if (rows == 0) return hipSuccess;
  const int b = rotation_block(n, block);
  int lb = 0;
  while ((1 << lb) < b) ++lb;
  const int64_t wgs = cdiv(rows * (n / b), RV / b);
  if (wgs >= ((int64_t)1 << 31)) return hipErrorInvalidValue;
  const float scale = 1.0f / sqrtf((float)b);
  const dim3 grid((unsigned)wgs);
  if (dt == 0) hipLaunchKernelGGL(hadamard_rows_kernel<0>, grid, dim3(256), 0, st, M, rows, n, ld, lb, scale);
  else if (dt == 1) hipLaunchKernelGGL(hadamard_rows_kernel<1>, grid, dim3(256), 0, st, M, rows, n, ld, lb, scale);
  else hipLaunchKernelGGL(hadamard_rows_kernel<2>, grid, dim3(256), 0, st, M, rows, n, ld, lb, scale);
  return hipGetLastError();
}

}  // namespace gptq
