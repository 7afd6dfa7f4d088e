// fp32 GEMM on the CDNA4 matrix cores (v_mfma_f32_32x32x2_f32).
//
// Used for every dense contraction after the Hessian: the lazy trailing
// update of the column sweep (V[:, i2:] -= E U[i:i2, i2:], the single matrix
// product of "Part 3: Adaptive Rounding: GPTQ", 'Algorithm GPTQ'), and the
// panel solves, trailing updates and inverse products of the factorization.
// The sweep's compensation must stay fp32-accurate, so no 16-bit operands.
//
// Tile: 128x128 per workgroup of 256 threads (4 wave64s, each 64x64 = 2x2
// MFMA 32x32 blocks), K staged through LDS 32 at a time, double-buffered,
// 16-byte global loads where aligned; two workgroups per CU.
#include "common.hpp"
#include "internal.hpp"

namespace gptq {

namespace {

constexpr int BM = 128, BN = 128, BK = 32, PAD = 4;
constexpr int LDT = BM + PAD;  // LDS row pitch (floats); BM == BN

// Load a BK x 128 slab of op(X) into registers.  ALONG_K: X[i*ld + k] (k
// contiguous, the tile is stored transposed into LDS); else X[k*ld + i].
// Each thread moves 4 float4 groups; VEC uses 16-byte loads where the group
// lies fully in bounds.
template <bool ALONG_K, bool VEC>
__device__ __forceinline__ void load_slab(const float* __restrict__ X, int64_t ld, int i0, int iEnd, int k0, int kEnd,
                                          int tid, f32x4 (&r)[4]) {
#pragma unroll
  for (int u = 0; u < 4; ++u) {
    int i, k;
    if (ALONG_K) { k = (tid & 7) * 4; i = (tid >> 3) + 32 * u; }
    else { i = (tid & 31) * 4; k = (tid >> 5) + 8 * u; }
    const int gi = i0 + i, gk = k0 + k;
    f32x4 v = {0.f, 0.f, 0.f, 0.f};
    if (ALONG_K) {
      const float* p = X + (int64_t)gi * ld + gk;
      if (gi < iEnd) {
        if (VEC && gk + 3 < kEnd) v = *(const f32x4*)p;
        else {
#pragma unroll
          for (int e = 0; e < 4; ++e) v[e] = (gk + e < kEnd) ? p[e] : 0.f;
        }
      }
    } else {
      const float* p = X + (int64_t)gk * ld + gi;
      if (gk < kEnd) {
        if (VEC && gi + 3 < iEnd) v = *(const f32x4*)p;
        else {
#pragma unroll
          for (int e = 0; e < 4; ++e) v[e] = (gi + e < iEnd) ? p[e] : 0.f;
        }
      }
    }
    r[u] = v;
  }
}

template <bool ALONG_K>
__device__ __forceinline__ void store_slab(float (*T)[LDT], int tid, const f32x4 (&r)[4]) {
#pragma unroll
  for (int u = 0; u < 4; ++u) {
    if (ALONG_K) {
      const int k = (tid & 7) * 4, i = (tid >> 3) + 32 * u;
      T[k + 0][i] = r[u][0];
      T[k + 1][i] = r[u][1];
      T[k + 2][i] = r[u][2];
      T[k + 3][i] = r[u][3];
    } else {
      const int i = (tid & 31) * 4, k = (tid >> 5) + 8 * u;
      *(f32x4*)&T[k][i] = r[u];
    }
  }
}

template <bool TRANS_A, bool TRANS_B, bool VEC>
__global__ __launch_bounds__(256, 2) void gemm_f32_kernel(GemmDesc d) {
  if (d.info && *d.info != 0) return;
  __shared__ __attribute__((aligned(16))) float As[2][BK][LDT];
  __shared__ __attribute__((aligned(16))) float Bs[2][BK][LDT];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int wr = wave >> 1, wc = wave & 1;

  int tm, tn;
  if (d.flags & GEMM_LOWER_TILES) {
    // linear index over the lower triangle of tiles: t = tm*(tm+1)/2 + tn
    const int t = blockIdx.x;
    int r = (int)((sqrtf(8.f * (float)t + 1.f) - 1.f) * 0.5f);
    while ((r + 1) * (r + 2) / 2 <= t) ++r;
    while (r * (r + 1) / 2 > t) --r;
    tm = r;
    tn = t - r * (r + 1) / 2;
  } else {
    tm = blockIdx.x;
    tn = blockIdx.y;
  }
  const int r0 = tm * BM, c0 = tn * BN;
  if (r0 >= d.M || c0 >= d.N) return;

  const int64_t z = blockIdx.z;
  const float* __restrict__ A = d.A + z * d.strideA;
  const float* __restrict__ B = d.B + z * d.strideB;
  float* C = d.C + z * d.strideC;

  int kLo = 0, kHi = d.K;
  if (d.flags & GEMM_A_LOWER) kHi = min(kHi, r0 + BM);
  if (d.flags & GEMM_B_LOWER) kLo = c0;

  f32x16 acc[2][2];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j) acc[i][j] = zero16();

  // beta != 0: fetch this lane's C values now, so their latency overlaps the K loop
  const float alpha = d.alpha, beta = d.beta;
  f32x16 cpre[2][2];
  if (beta != 0.f) {
#pragma unroll
    for (int mb = 0; mb < 2; ++mb)
#pragma unroll
      for (int nb = 0; nb < 2; ++nb)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int row = r0 + wr * 64 + mb * 32 + mfma32_row(r, lane);
          const int col = c0 + wc * 64 + nb * 32 + mfma32_col(lane);
          cpre[mb][nb][r] = (row < d.M && col < d.N) ? C[(int64_t)row * d.ldc + col] : 0.f;
        }
  }

  f32x4 ra[4], rb[4];
  if (kLo < kHi) {
    load_slab<!TRANS_A, VEC>(A, d.lda, r0, d.M, kLo, kHi, tid, ra);
    load_slab<TRANS_B, VEC>(B, d.ldb, c0, d.N, kLo, kHi, tid, rb);
    store_slab<!TRANS_A>(As[0], tid, ra);
    store_slab<TRANS_B>(Bs[0], tid, rb);
    __syncthreads();
    int buf = 0;
    for (int k0 = kLo; k0 < kHi; k0 += BK) {
      const bool more = k0 + BK < kHi;
      if (more) {
        load_slab<!TRANS_A, VEC>(A, d.lda, r0, d.M, k0 + BK, kHi, tid, ra);
        load_slab<TRANS_B, VEC>(B, d.ldb, c0, d.N, k0 + BK, kHi, tid, rb);
      }
      const int kr = lane >> 5;
      const int cl = lane & 31;
#pragma unroll
      for (int kk = 0; kk < BK; kk += 2) {
        const float a0 = As[buf][kk + kr][wr * 64 + cl];
        const float a1 = As[buf][kk + kr][wr * 64 + 32 + cl];
        const float b0 = Bs[buf][kk + kr][wc * 64 + cl];
        const float b1 = Bs[buf][kk + kr][wc * 64 + 32 + cl];
        acc[0][0] = __builtin_amdgcn_mfma_f32_32x32x2f32(a0, b0, acc[0][0], 0, 0, 0);
        acc[0][1] = __builtin_amdgcn_mfma_f32_32x32x2f32(a0, b1, acc[0][1], 0, 0, 0);
        acc[1][0] = __builtin_amdgcn_mfma_f32_32x32x2f32(a1, b0, acc[1][0], 0, 0, 0);
        acc[1][1] = __builtin_amdgcn_mfma_f32_32x32x2f32(a1, b1, acc[1][1], 0, 0, 0);
      }
      if (more) {
        store_slab<!TRANS_A>(As[buf ^ 1], tid, ra);
        store_slab<TRANS_B>(Bs[buf ^ 1], tid, rb);
      }
      __syncthreads();
      buf ^= 1;
    }
  }

#pragma unroll
  for (int mb = 0; mb < 2; ++mb)
#pragma unroll
    for (int nb = 0; nb < 2; ++nb)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int row = r0 + wr * 64 + mb * 32 + mfma32_row(r, lane);
        const int col = c0 + wc * 64 + nb * 32 + mfma32_col(lane);
        if (row < d.M && col < d.N) {
          const float v = alpha * acc[mb][nb][r];
          C[(int64_t)row * d.ldc + col] = (beta == 0.f) ? v : fmaf(beta, cpre[mb][nb][r], v);
        }
      }
}

template <bool TA, bool TB>
void launch(const GemmDesc& d, dim3 grid, hipStream_t s) {
  const bool vec = d.lda % 4 == 0 && d.ldb % 4 == 0 && d.strideA % 4 == 0 && d.strideB % 4 == 0 &&
                   ((uintptr_t)d.A & 15) == 0 && ((uintptr_t)d.B & 15) == 0;
  if (vec) hipLaunchKernelGGL((gemm_f32_kernel<TA, TB, true>), grid, dim3(256), 0, s, d);
  else hipLaunchKernelGGL((gemm_f32_kernel<TA, TB, false>), grid, dim3(256), 0, s, d);
}

}  // namespace

hipError_t gemm_f32(const GemmDesc& d, bool transA, bool transB, hipStream_t s) {
  if (d.M <= 0 || d.N <= 0 || d.batch <= 0) return hipSuccess;
  dim3 grid;
  const int tM = (int)cdiv(d.M, BM), tN = (int)cdiv(d.N, BN);
  if (d.flags & GEMM_LOWER_TILES) grid = dim3((unsigned)(tM * (tM + 1) / 2), 1, (unsigned)d.batch);
  else grid = dim3((unsigned)tM, (unsigned)tN, (unsigned)d.batch);
  if (!transA && !transB) launch<false, false>(d, grid, s);
  else if (!transA && transB) launch<false, true>(d, grid, s);
  else if (transA && !transB) launch<true, false>(d, grid, s);
  else launch<true, true>(d, grid, s);
  return hipGetLastError();
}

}  // namespace gptq
