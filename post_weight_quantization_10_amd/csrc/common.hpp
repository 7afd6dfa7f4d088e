// Shared device helpers for the gfx950 (CDNA4) GPTQ kernels.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace gptq {

typedef _Float16 half8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

// Output layout of every 32x32 MFMA (16 fp32 per lane): accumulator r of lane
// l holds C[row][col] with col = l % 32 and row = 8*(r/4) + 4*(l/32) + r%4.
__device__ __forceinline__ int mfma32_row(int r, int lane) { return 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3); }
__device__ __forceinline__ int mfma32_col(int lane) { return lane & 31; }

__device__ __forceinline__ f32x16 zero16() {
  f32x16 z;
#pragma unroll
  for (int i = 0; i < 16; ++i) z[i] = 0.f;
  return z;
}

// Broadcast lane `src` (0..15, compile-time) of each 16-lane DPP row to the
// whole row.
template <int SRC>
__device__ __forceinline__ float row_bcast(float v) {
  return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), 0x150 + SRC, 0xF, 0xF, false));
}

// Min / max over the 16 lanes of a DPP row (xor 1, xor 2 inside quads, then
// rotations by 4 and 8 inside the row); every lane receives the result.
__device__ __forceinline__ float row_min16(float v) {
  v = fminf(v, __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, v), 0xB1, 0xF, 0xF, false)));
  v = fminf(v, __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, v), 0x4E, 0xF, 0xF, false)));
  v = fminf(v, __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, v), 0x124, 0xF, 0xF, false)));
  v = fminf(v, __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, v), 0x128, 0xF, 0xF, false)));
  return v;
}
__device__ __forceinline__ float row_max16(float v) {
  v = fmaxf(v, __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, v), 0xB1, 0xF, 0xF, false)));
  v = fmaxf(v, __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, v), 0x4E, 0xF, 0xF, false)));
  v = fmaxf(v, __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, v), 0x124, 0xF, 0xF, false)));
  v = fmaxf(v, __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, v), 0x128, 0xF, 0xF, false)));
  return v;
}

// Element conversions for the weight / activation dtypes.
__device__ __forceinline__ float bf16_to_f32(uint16_t b) { return __builtin_bit_cast(float, (uint32_t)b << 16); }
__device__ __forceinline__ uint16_t f32_to_bf16(float f) {
  uint32_t u = __builtin_bit_cast(uint32_t, f);
  if ((u & 0x7F800000u) == 0x7F800000u && (u & 0x7FFFFFu)) return (uint16_t)((u >> 16) | 0x40);  // quiet NaN
  u += 0x7FFFu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}

template <int DT> struct Elem;
template <> struct Elem<0> {  // fp16
  typedef _Float16 T;
  __device__ static float load(const void* p, int64_t i) { return (float)((const _Float16*)p)[i]; }
  __device__ static void store(void* p, int64_t i, float v) { ((_Float16*)p)[i] = (_Float16)v; }
};
template <> struct Elem<1> {  // bf16
  typedef uint16_t T;
  __device__ static float load(const void* p, int64_t i) { return bf16_to_f32(((const uint16_t*)p)[i]); }
  __device__ static void store(void* p, int64_t i, float v) { ((uint16_t*)p)[i] = f32_to_bf16(v); }
};
template <> struct Elem<2> {  // fp32
  typedef float T;
  __device__ static float load(const void* p, int64_t i) { return ((const float*)p)[i]; }
  __device__ static void store(void* p, int64_t i, float v) { ((float*)p)[i] = v; }
};

__host__ __device__ inline int64_t cdiv(int64_t a, int64_t b) { return (a + b - 1) / b; }

// Quantizer parameters (s, z) from the range [lo, hi] of a group or row:
// x_lo = min(0, lo), x_hi = max(0, hi) (an all-zero range becomes [0, 1]),
// s = (x_hi - x_lo) / maxq, z = rint(-x_lo / s).  Taken in fp64 (s then
// rounded to fp32): for 16-bit weights the extremes of a row or group are
// often exact negatives of each other, and then -x_lo / s is exactly the
// half-integer maxq / 2 in exact arithmetic, so the integer z would be
// decided by the last bit of the division; fp64 takes that decision the same
// way as an fp64 computation of the same formula does.
__device__ __forceinline__ void qparams(float lo, float hi, int maxq, float& s, float& z) {
  double l = fmin((double)lo, 0.0), h = fmax((double)hi, 0.0);
  if (h == l) { l = 0.0; h = 1.0; }
  const double s64 = (h - l) / (double)maxq;
  s = (float)s64;
  z = (float)rint(-l / s64);
}


// ---------------------------------------------------------------------------- LDS-DMA staging

#define LDS_AS __attribute__((address_space(3)))

typedef int i32x4 __attribute__((ext_vector_type(4)));

// One 16-byte-per-lane global -> LDS copy: lane l's 16 bytes at byte offset
// voff of the buffer described by rs land at LDS address lds_addr + 16 l
// (bounds-checked: past num_records they read as zero).  Written as inline
// assembly so that the compiler does not treat the asynchronous LDS write as
// aliasing every LDS read (it would then wait for all copies in flight before
// each stage); ordering is explicit instead: wait_vmcnt before the stage's
// barrier.  Nothing else in these kernels uses M0.  The instruction has no
// register result.
__device__ __forceinline__ void dma16(i32x4 rs, uint32_t lds_addr, int voff) {
  const uint32_t m0v = __builtin_amdgcn_readfirstlane(lds_addr);  // wave-uniform by construction
  asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tbuffer_load_dwordx4 %1, %2, 0 offen lds" ::"s"(m0v), "v"(voff),
               "s"(rs));
}

__device__ __forceinline__ i32x4 make_rsrc(const void* base, uint32_t nbytes) {
  const uint64_t b = (uint64_t)base;
  return i32x4{(int)(uint32_t)b, (int)((b >> 32) & 0xFFFFu), (int)nbytes, 0x00020000};
}

// Workgroup barrier without the release/acquire fences of __syncthreads():
// the only cross-wave data here are the stage DMAs, which every wave has
// already waited for with wait_vmcnt, and LDS reads of a stage are consumed
// before the wave reaches the next barrier.  The memory clobber keeps the
// compiler from moving LDS accesses across it.
__device__ __forceinline__ void stage_barrier() { asm volatile("s_barrier" ::: "memory"); }

// vmcnt-only wait (expcnt and lgkmcnt left at their "no wait" maxima)
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  __builtin_amdgcn_s_waitcnt((N & 0xF) | ((N >> 4) << 14) | (0x7 << 4) | (0xF << 8));
}

}  // namespace gptq
