// fp32 GEMM on the CDNA4 matrix cores (v_mfma_f32_32x32x2_f32).
//
// Used for every dense contraction after the Hessian: the lazy trailing
// update of the column sweep (V[:, i2:] -= E U[i:i2, i2:], the single matrix
// product of "Part 3: Adaptive Rounding: GPTQ", 'Algorithm GPTQ'), and the
// panel solves, trailing updates and inverse products of the factorization.
// The sweep's compensation must stay fp32-accurate, so no 16-bit operands.
//
// Tile: 128x128 per workgroup of 256 threads (4 wave64s, each 64x64 = 2x2
// MFMA 32x32 blocks), K staged through LDS 16 at a time, double-buffered.
#include "common.hpp"
#include "internal.hpp"

namespace gptq {

namespace {

constexpr int BM = 128, BN = 128, BK = 16, PAD = 4;
constexpr int LDT = BM + PAD;  // LDS row pitch (floats); BM == BN

template <bool TRANS_A, bool TRANS_B>
__global__ __launch_bounds__(256) void gemm_f32_kernel(GemmDesc d) {
  if (d.info && *d.info != 0) return;
  __shared__ float As[2][BK][LDT];
  __shared__ float Bs[2][BK][LDT];

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

  float ra[8], rb[8];

  // global -> registers for the chunk starting at k0
  auto load = [&](int k0) {
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      if (TRANS_A) {  // A[k][i]: contiguous along i
        const int i = tid & 127, kk = (tid >> 7) + 2 * u;
        const int gi = r0 + i, gk = k0 + kk;
        ra[u] = (gi < d.M && gk < kHi) ? A[(int64_t)gk * d.lda + gi] : 0.f;
      } else {  // A[i][k]: contiguous along k
        const int kk = tid & 15, i = (tid >> 4) + 16 * u;
        const int gi = r0 + i, gk = k0 + kk;
        ra[u] = (gi < d.M && gk < kHi) ? A[(int64_t)gi * d.lda + gk] : 0.f;
      }
      if (!TRANS_B) {  // B[k][j]: contiguous along j
        const int j = tid & 127, kk = (tid >> 7) + 2 * u;
        const int gj = c0 + j, gk = k0 + kk;
        rb[u] = (gj < d.N && gk < kHi) ? B[(int64_t)gk * d.ldb + gj] : 0.f;
      } else {  // B[j][k]: contiguous along k
        const int kk = tid & 15, j = (tid >> 4) + 16 * u;
        const int gj = c0 + j, gk = k0 + kk;
        rb[u] = (gj < d.N && gk < kHi) ? B[(int64_t)gj * d.ldb + gk] : 0.f;
      }
    }
  };
  auto store = [&](int buf) {
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      if (TRANS_A) As[buf][(tid >> 7) + 2 * u][tid & 127] = ra[u];
      else As[buf][tid & 15][(tid >> 4) + 16 * u] = ra[u];
      if (!TRANS_B) Bs[buf][(tid >> 7) + 2 * u][tid & 127] = rb[u];
      else Bs[buf][tid & 15][(tid >> 4) + 16 * u] = rb[u];
    }
  };

  if (kLo < kHi) {
    load(kLo);
    store(0);
    __syncthreads();
    int buf = 0;
    for (int k0 = kLo; k0 < kHi; k0 += BK) {
      const bool more = k0 + BK < kHi;
      if (more) load(k0 + BK);
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
      if (more) store(buf ^ 1);
      __syncthreads();
      buf ^= 1;
    }
  }

  const float alpha = d.alpha, beta = d.beta;
#pragma unroll
  for (int mb = 0; mb < 2; ++mb)
#pragma unroll
    for (int nb = 0; nb < 2; ++nb)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int row = r0 + wr * 64 + mb * 32 + mfma32_row(r, lane);
        const int col = c0 + wc * 64 + nb * 32 + mfma32_col(lane);
        if (row < d.M && col < d.N) {
          float* p = C + (int64_t)row * d.ldc + col;
          const float v = alpha * acc[mb][nb][r];
          *p = (beta == 0.f) ? v : fmaf(beta, *p, v);
        }
      }
}

}  // namespace

hipError_t gemm_f32(const GemmDesc& d, bool transA, bool transB, hipStream_t s) {
  if (d.M <= 0 || d.N <= 0 || d.batch <= 0) return hipSuccess;
  dim3 grid;
  const int tM = (int)cdiv(d.M, BM), tN = (int)cdiv(d.N, BN);
  if (d.flags & GEMM_LOWER_TILES) grid = dim3((unsigned)(tM * (tM + 1) / 2), 1, (unsigned)d.batch);
  else grid = dim3((unsigned)tM, (unsigned)tN, (unsigned)d.batch);
  if (!transA && !transB) hipLaunchKernelGGL((gemm_f32_kernel<false, false>), grid, dim3(256), 0, s, d);
  else if (!transA && transB) hipLaunchKernelGGL((gemm_f32_kernel<false, true>), grid, dim3(256), 0, s, d);
  else if (transA && !transB) hipLaunchKernelGGL((gemm_f32_kernel<true, false>), grid, dim3(256), 0, s, d);
  else hipLaunchKernelGGL((gemm_f32_kernel<true, true>), grid, dim3(256), 0, s, d);
  return hipGetLastError();
}

}  // namespace gptq
