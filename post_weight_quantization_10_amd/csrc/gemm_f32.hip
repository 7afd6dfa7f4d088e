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
#include <algorithm>

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

// ---------------------------------------------------------------------------- NN, LDS-DMA path
//
// C = alpha A B + beta C with A [M x K] and B [K x N] row-major, K-range
// multiples of 32 (the sweep's block flushes and the doubling products of the
// triangular inverse).  Both slabs of a 32-deep K step move HBM -> LDS with
// buffer_load_dwordx4 ... lds (no VGPR staging, bounds-checked, so no edge
// branches): A as 128 rows x 128 B, B as 32 rows x 512 B, their 16-byte chunks
// XOR-swizzled so that the MFMA operand reads (one float per lane) spread over
// the banks.  Two stages in a ring, two workgroups per CU; every operand read
// sits between two MFMAs, two k pairs ahead of its use.

constexpr int DBK = 32;                       // K per stage
constexpr int DSTAGE_F = BM * DBK + DBK * BN;  // floats per stage (A then B): 32 KiB

__device__ __forceinline__ int swzA(int row) { return (row >> 1) & 7; }  // chunk XOR for A rows
__device__ __forceinline__ int swzB(int k) { return (k & 1) << 3; }      // chunk XOR for B rows

// Split-K (nsplit > 1): blockIdx.z = batch entry * nsplit + chunk; the chunk's
// product (no alpha, no beta) goes to part[(z * tiles + tile)][128 x 128].
__global__ __launch_bounds__(256, 2) void gemm_nn_dma_kernel(GemmDesc d, int nsplit, int chunk, float* part) {
  if (d.info && *d.info != 0) return;
  __shared__ __attribute__((aligned(1024))) float stg0[DSTAGE_F];
  __shared__ __attribute__((aligned(1024))) float stg1[DSTAGE_F];
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wr = wave >> 1, wc = wave & 1;
  const int tm = blockIdx.x, tn = blockIdx.y;
  const int r0 = tm * BM, c0 = tn * BN;
  if (r0 >= d.M || c0 >= d.N) return;
  const int64_t z = blockIdx.z / nsplit;
  const int split = blockIdx.z % nsplit;
  const float* A = d.A + z * d.strideA;
  const float* B = d.B + z * d.strideB;
  float* C = d.C + z * d.strideC;
  int kLo = 0, kHi = d.K;
  if (d.flags & GEMM_A_LOWER) kHi = min(kHi, r0 + BM);
  if (d.flags & GEMM_B_LOWER) kLo = c0;
  if (nsplit > 1) {
    kLo += split * chunk;
    kHi = min(kHi, kLo + chunk);
    if (kLo >= kHi) return;  // the reduction skips chunks past the tile's K range
  }
  const int nst = (kHi - kLo) / DBK;
  const int mrows = min(BM, d.M - r0), ncols = min(BN, d.N - c0);

  // this lane's copies of one stage: 4 for A (rows 32w + 8q + l/8), 4 for B
  // (rows 8w + 2q + l/32); byte offsets relative to the stage's buffer bases
  int voffA[4], voffB[4];
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const int ra = 32 * wave + 8 * q + (lane >> 3);
    voffA[q] = (int)((int64_t)ra * d.lda * 4) + ((((lane & 7) ^ swzA(ra))) << 4);
    const int rb = 8 * wave + 2 * q + (lane >> 5);
    voffB[q] = (int)((int64_t)rb * d.ldb * 4) + ((((lane & 31) ^ swzB(rb))) << 4);
  }
  const uint32_t aBytes = (uint32_t)(((int64_t)(mrows - 1) * d.lda + DBK) * 4);
  const uint32_t bBytes = (uint32_t)(((int64_t)(DBK - 1) * d.ldb + ncols) * 4);
  auto issue = [&](int st, float* stg) {
    const int kc = kLo + st * DBK;
    const i32x4 ra = make_rsrc(A + (int64_t)r0 * d.lda + kc, aBytes);
    const i32x4 rb = make_rsrc(B + (int64_t)kc * d.ldb + c0, bBytes);
    const uint32_t sb = (uint32_t)(uintptr_t)((float LDS_AS*)stg);
#pragma unroll
    for (int q = 0; q < 4; ++q) dma16(ra, sb + (uint32_t)((32 * wave + 8 * q) * DBK * 4), voffA[q]);
#pragma unroll
    for (int q = 0; q < 4; ++q) dma16(rb, sb + (uint32_t)((BM * DBK + (8 * wave + 2 * q) * BN) * 4), voffB[q]);
  };

  // C of this wave's 64 x 64 quadrant, fetched first (interior tiles: one base
  // plus constant offsets; edge tiles: clamped addresses, entries past M or N
  // are never stored)
  const float alpha = d.alpha, beta = d.beta;
  const bool interior = mrows == BM && ncols == BN;
  const int rl = wr * 64 + 4 * (lane >> 5), cl0 = wc * 64 + (lane & 31);
  f32x16 cp[2][2];
#pragma unroll
  for (int mb = 0; mb < 2; ++mb)
#pragma unroll
    for (int nb = 0; nb < 2; ++nb) cp[mb][nb] = zero16();
  if (beta != 0.f && nsplit == 1) {
    if (interior) {
      const float* base = C + (int64_t)(r0 + rl) * d.ldc + c0 + cl0;
#pragma unroll
      for (int mb = 0; mb < 2; ++mb)
#pragma unroll
        for (int nb = 0; nb < 2; ++nb)
#pragma unroll
          for (int r = 0; r < 16; ++r)
            cp[mb][nb][r] = base[(int64_t)(32 * mb + 8 * (r >> 2) + (r & 3)) * d.ldc + 32 * nb];
    } else {
#pragma unroll
      for (int mb = 0; mb < 2; ++mb)
#pragma unroll
        for (int nb = 0; nb < 2; ++nb) {
          const float* colp = C + min(c0 + cl0 + 32 * nb, d.N - 1);
#pragma unroll
          for (int r = 0; r < 16; ++r)
            cp[mb][nb][r] = colp[(int64_t)min(r0 + rl + 32 * mb + 8 * (r >> 2) + (r & 3), d.M - 1) * d.ldc];
        }
    }
  }

  f32x16 acc[2][2];
#pragma unroll
  for (int mb = 0; mb < 2; ++mb)
#pragma unroll
    for (int nb = 0; nb < 2; ++nb) acc[mb][nb] = zero16();
  const int kr = lane >> 5, cl = lane & 31;
  // operand reads of one k pair (k = 2 kk + kr) from a stage
  auto rdA = [&](const float* sA, int row, int k) { return sA[row * DBK + ((((k >> 2) ^ swzA(row))) << 2) + (k & 3)]; };
  auto rdB = [&](const float* sB, int k, int col) { return sB[k * BN + ((((col >> 2) ^ swzB(k))) << 2) + (col & 3)]; };
  auto compute = [&](const float* stg) {
    const float* sA = stg;
    const float* sB = stg + BM * DBK;
    // operands of k pair kk in slot kk % 3, read two pairs (eight MFMAs) ahead
    float fa0[3], fa1[3], fb0[3], fb1[3];
    auto rdk = [&](int kk, int sl) {
      const int k = 2 * kk + kr;
      fa0[sl] = rdA(sA, wr * 64 + cl, k); fa1[sl] = rdA(sA, wr * 64 + 32 + cl, k);
      fb0[sl] = rdB(sB, k, wc * 64 + cl); fb1[sl] = rdB(sB, k, wc * 64 + 32 + cl);
    };
    rdk(0, 0);
    rdk(1, 1);
#pragma unroll
    for (int kk = 0; kk < DBK / 2; ++kk) {
      const int s = kk % 3, sn = (kk + 2) % 3, kn = 2 * (kk + 2) + kr;
      const bool more = kk + 2 < DBK / 2;
      acc[0][0] = __builtin_amdgcn_mfma_f32_32x32x2f32(fa0[s], fb0[s], acc[0][0], 0, 0, 0);
      if (more) fa0[sn] = rdA(sA, wr * 64 + cl, kn);
      acc[0][1] = __builtin_amdgcn_mfma_f32_32x32x2f32(fa0[s], fb1[s], acc[0][1], 0, 0, 0);
      if (more) fa1[sn] = rdA(sA, wr * 64 + 32 + cl, kn);
      acc[1][0] = __builtin_amdgcn_mfma_f32_32x32x2f32(fa1[s], fb0[s], acc[1][0], 0, 0, 0);
      if (more) fb0[sn] = rdB(sB, kn, wc * 64 + cl);
      acc[1][1] = __builtin_amdgcn_mfma_f32_32x32x2f32(fa1[s], fb1[s], acc[1][1], 0, 0, 0);
      if (more) fb1[sn] = rdB(sB, kn, wc * 64 + 32 + cl);
    }
#pragma unroll
    for (int kk = 0; kk < DBK / 2 - 2; ++kk)
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // one MFMA
        __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);  // one LDS read
      }
    __builtin_amdgcn_sched_group_barrier(0x008, 8, 0);
  };

  // two-stage ring: the copy of step s+1 is in flight while step s computes
  if (nst > 0) {
    issue(0, stg0);
    for (int st = 0; st < nst; st += 2) {
      if (st + 1 < nst) { issue(st + 1, stg1); wait_vmcnt<8>(); } else wait_vmcnt<0>();
      stage_barrier();  // step st visible to every wave
      compute(stg0);
      stage_barrier();  // everyone is done with stg0
      if (st + 1 >= nst) break;
      if (st + 2 < nst) { issue(st + 2, stg0); wait_vmcnt<8>(); } else wait_vmcnt<0>();
      stage_barrier();
      compute(stg1);
      stage_barrier();
    }
  }

  if (nsplit > 1) {
    float* P = part + ((int64_t)blockIdx.z * gridDim.x * gridDim.y + (int64_t)tn * gridDim.x + tm) * (BM * BN);
#pragma unroll
    for (int mb = 0; mb < 2; ++mb)
#pragma unroll
      for (int nb = 0; nb < 2; ++nb)
#pragma unroll
        for (int r = 0; r < 16; ++r) P[(rl + 32 * mb + 8 * (r >> 2) + (r & 3)) * BN + cl0 + 32 * nb] = acc[mb][nb][r];
    return;
  }
  if (interior) {
    float* base = C + (int64_t)(r0 + rl) * d.ldc + c0 + cl0;
#pragma unroll
    for (int mb = 0; mb < 2; ++mb)
#pragma unroll
      for (int nb = 0; nb < 2; ++nb)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const float v = alpha * acc[mb][nb][r];
          base[(int64_t)(32 * mb + 8 * (r >> 2) + (r & 3)) * d.ldc + 32 * nb] =
              (beta == 0.f) ? v : fmaf(beta, cp[mb][nb][r], v);
        }
    return;
  }
#pragma unroll
  for (int mb = 0; mb < 2; ++mb)
#pragma unroll
    for (int nb = 0; nb < 2; ++nb)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int row = r0 + rl + 32 * mb + 8 * (r >> 2) + (r & 3);
        const int col = c0 + cl0 + 32 * nb;
        if (row < d.M && col < d.N) {
          const float v = alpha * acc[mb][nb][r];
          C[(int64_t)row * d.ldc + col] = (beta == 0.f) ? v : fmaf(beta, cp[mb][nb][r], v);
        }
      }
}

// ---------------------------------------------------------------------------- NN, 64 x 64 tiles
//
// The same staging for products whose 128 x 128 tile grid would leave the GPU
// under-filled, such as the doubling products of a triangular inverse, where a
// triangular operand also gives the tiles K ranges from 64 to K: 64 x 64
// tiles, four waves of 32 x 32 (2 x 2 blocks of v_mfma_f32_16x16x4f32), a ring
// of three 32-deep K stages with one barrier per stage.  One linear grid over
// (tile, batch entry) is ordered longest K range first, so the short tiles
// fill in behind the long ones and no split-K partial sums are needed.

constexpr int SB = 64, SNS = 3;
constexpr int SSTAGE_F = 2 * SB * DBK;  // floats per stage (A then B): 16 KiB
__device__ __forceinline__ int swzB4(int k) { return (k & 3) << 2; }  // chunk XOR for the 64-wide B rows

__global__ __launch_bounds__(256, 2) void gemm_nn_dma64_kernel(GemmDesc d, int tM, int tN) {
  if (d.info && *d.info != 0) return;
  __shared__ __attribute__((aligned(1024))) float stg[SNS * SSTAGE_F];
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wr = wave >> 1, wc = wave & 1;
  const int z = (int)(blockIdx.x % (unsigned)d.batch), rank = (int)(blockIdx.x / (unsigned)d.batch);
  int tm, tn;
  if (d.flags & GEMM_A_LOWER) {  // the K range grows with the tile row
    tm = tM - 1 - rank / tN;
    tn = rank % tN;
  } else if (d.flags & GEMM_B_LOWER) {  // and shrinks with the tile column
    tn = rank / tM;
    tm = rank % tM;
  } else {
    tm = rank / tN;
    tn = rank % tN;
  }
  const int r0 = tm * SB, c0 = tn * SB;
  const float* A = d.A + z * d.strideA;
  const float* B = d.B + z * d.strideB;
  float* C = d.C + z * d.strideC;
  int kLo = 0, kHi = d.K;
  if (d.flags & GEMM_A_LOWER) kHi = min(kHi, r0 + SB);
  if (d.flags & GEMM_B_LOWER) kLo = c0;
  const int nst = kHi > kLo ? (kHi - kLo) / DBK : 0;
  const int mrows = min(SB, d.M - r0), ncols = min(SB, d.N - c0);

  // this lane's copies of one stage: A rows 16w + 8q + l/8 (eight 16-byte
  // chunks each), B rows 8w + 4q + l/16 (sixteen chunks each)
  int voffA[2], voffB[2];
#pragma unroll
  for (int q = 0; q < 2; ++q) {
    const int ra = 16 * wave + 8 * q + (lane >> 3);
    voffA[q] = (int)((int64_t)ra * d.lda * 4) + (((lane & 7) ^ swzA(ra)) << 4);
    const int rb = 8 * wave + 4 * q + (lane >> 4);
    voffB[q] = (int)((int64_t)rb * d.ldb * 4) + (((lane & 15) ^ swzB4(rb)) << 4);
  }
  const uint32_t aBytes = (uint32_t)(((int64_t)(mrows - 1) * d.lda + DBK) * 4);
  const uint32_t bBytes = (uint32_t)(((int64_t)(DBK - 1) * d.ldb + ncols) * 4);
  auto issue = [&](int st) {
    const int kc = kLo + st * DBK;
    const i32x4 ra = make_rsrc(A + (int64_t)r0 * d.lda + kc, aBytes);
    const i32x4 rb = make_rsrc(B + (int64_t)kc * d.ldb + c0, bBytes);
    const uint32_t sb = (uint32_t)(uintptr_t)((float LDS_AS*)(stg + (st % SNS) * SSTAGE_F));
#pragma unroll
    for (int q = 0; q < 2; ++q) dma16(ra, sb + (uint32_t)((16 * wave + 8 * q) * DBK * 4), voffA[q]);
#pragma unroll
    for (int q = 0; q < 2; ++q) dma16(rb, sb + (uint32_t)((SB * DBK + (8 * wave + 4 * q) * SB) * 4), voffB[q]);
  };

  f32x4 acc[2][2];
#pragma unroll
  for (int mb = 0; mb < 2; ++mb)
#pragma unroll
    for (int nb = 0; nb < 2; ++nb) acc[mb][nb] = f32x4{0.f, 0.f, 0.f, 0.f};
  // v_mfma_f32_16x16x4f32: lane l gives A[l%16][k] and B[k][l%16] with
  // k = 4kk + l/16; result register r is row 4(l/16) + r, column l%16
  const int l16 = lane & 15, kq = lane >> 4;
  auto compute = [&](const float* s) {
    const float* sA = s;
    const float* sB = s + SB * DBK;
#pragma unroll
    for (int kk = 0; kk < DBK / 4; ++kk) {
      const int k = 4 * kk + kq;
      float a[2], b[2];
#pragma unroll
      for (int mb = 0; mb < 2; ++mb) {
        const int row = 32 * wr + 16 * mb + l16;
        a[mb] = sA[row * DBK + ((kk ^ swzA(row)) << 2) + kq];
      }
#pragma unroll
      for (int nb = 0; nb < 2; ++nb) {
        const int col = 32 * wc + 16 * nb + l16;
        b[nb] = sB[k * SB + (((col >> 2) ^ swzB4(k)) << 2) + (col & 3)];
      }
#pragma unroll
      for (int mb = 0; mb < 2; ++mb)
#pragma unroll
        for (int nb = 0; nb < 2; ++nb)
          acc[mb][nb] = __builtin_amdgcn_mfma_f32_16x16x4f32(a[mb], b[nb], acc[mb][nb], 0, 0, 0);
    }
  };

  // this lane's 16 entries of C, fetched before the K loop when beta != 0
  // (rows and columns past M or N read the last valid one, never stored):
  // loaded one by one behind the store's bounds test they would be 16
  // dependent memory round trips at the end.  They are issued before the
  // first stage's copies, so the in-order vmcnt waits below also cover them.
  const float alpha = d.alpha, beta = d.beta;
  f32x4 cp[2][2];
#pragma unroll
  for (int mb = 0; mb < 2; ++mb)
#pragma unroll
    for (int nb = 0; nb < 2; ++nb) cp[mb][nb] = f32x4{0.f, 0.f, 0.f, 0.f};
  if (beta != 0.f) {
#pragma unroll
    for (int mb = 0; mb < 2; ++mb)
#pragma unroll
      for (int nb = 0; nb < 2; ++nb) {
        const float* colp = C + min(c0 + 32 * wc + 16 * nb + l16, d.N - 1);
#pragma unroll
        for (int r = 0; r < 4; ++r)
          cp[mb][nb][r] = colp[(int64_t)min(r0 + 32 * wr + 16 * mb + 4 * kq + r, d.M - 1) * d.ldc];
      }
  }

  // three-stage ring: stages st + 1 and st + 2 are in flight while st computes
  if (nst > 0) issue(0);
  if (nst > 1) issue(1);
  for (int st = 0; st < nst; ++st) {
    if (st + 1 < nst) wait_vmcnt<4>(); else wait_vmcnt<0>();
    stage_barrier();  // stage st visible to every wave; every wave is done with stage st - 1
    if (st + 2 < nst) issue(st + 2);
    compute(stg + (st % SNS) * SSTAGE_F);
  }

#pragma unroll
  for (int mb = 0; mb < 2; ++mb)
#pragma unroll
    for (int nb = 0; nb < 2; ++nb)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int row = r0 + 32 * wr + 16 * mb + 4 * kq + r, col = c0 + 32 * wc + 16 * nb + l16;
        if (row < d.M && col < d.N) {
          const float v = alpha * acc[mb][nb][r];
          C[(int64_t)row * d.ldc + col] = (beta == 0.f) ? v : fmaf(beta, cp[mb][nb][r], v);
        }
      }
}

// C tile = alpha * (sum of its chunks in chunk order) + beta * C; chunks past
// the tile's K range were never computed and are skipped.
__global__ __launch_bounds__(256) void gemm_split_reduce_kernel(GemmDesc d, int nsplit, int chunk, const float* part) {
  if (d.info && *d.info != 0) return;
  const int tm = blockIdx.x, tn = blockIdx.y;
  const int r0 = tm * BM, c0 = tn * BN;
  const int64_t z = blockIdx.z;
  float* C = d.C + z * d.strideC;
  int kLo = 0, kHi = d.K;
  if (d.flags & GEMM_A_LOWER) kHi = min(kHi, r0 + BM);
  if (d.flags & GEMM_B_LOWER) kLo = c0;
  const int nvalid = kHi > kLo ? min(nsplit, (kHi - kLo + chunk - 1) / chunk) : 0;
  const int64_t tstride = (int64_t)gridDim.x * gridDim.y * (BM * BN);
  const float* P = part + ((z * nsplit) * gridDim.x * gridDim.y + (int64_t)tn * gridDim.x + tm) * (BM * BN);
  const int tid = threadIdx.x;
#pragma unroll 4
  for (int u = 0; u < BM * BN / (4 * 256); ++u) {
    const int e = 4 * (tid + 256 * u);
    const int row = e / BN, col = e % BN;
    f32x4 sum = {0.f, 0.f, 0.f, 0.f};
    for (int s = 0; s < nvalid; ++s) sum += *(const f32x4*)(P + s * tstride + e);
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int gr = r0 + row, gc = c0 + col + q;
      if (gr < d.M && gc < d.N) {
        float* pc = C + (int64_t)gr * d.ldc + gc;
        const float v = d.alpha * sum[q];
        *pc = (d.beta == 0.f) ? v : fmaf(d.beta, *pc, v);
      }
    }
  }
}

bool nn_dma_ok(const GemmDesc& d) {
  const auto al16 = [](const void* p) { return ((uintptr_t)p & 15) == 0; };
  return d.K % DBK == 0 && d.lda % 4 == 0 && d.ldb % 4 == 0 && d.N % 4 == 0 && d.strideA % 4 == 0 &&
         d.strideB % 4 == 0 && al16(d.A) && al16(d.B) && !(d.flags & GEMM_LOWER_TILES) &&
         (int64_t)(BM - 1) * d.lda * 4 + 4096 < ((int64_t)1 << 31) && (int64_t)(DBK - 1) * d.ldb * 4 + 4096 < ((int64_t)1 << 31);
}

// Whether 64 x 64 tiles finish a full-K product (no triangular operand) in
// fewer rounds of resident workgroups than 128 x 128 tiles: a 128-tile does
// four times the work of a 64-tile, two of either fit on a CU, and a round of
// 64-tiles is taken as 15 % less efficient (more operand traffic per flop).
// True for the narrow late flushes of a sweep, whose 128-tile grid leaves
// most CUs idle.
bool small_tiles_pay(const GemmDesc& d, int tM, int tN, int sM, int sN) {
  if (d.flags & (GEMM_A_LOWER | GEMM_B_LOWER)) return false;
  const int64_t slots = (int64_t)2 * device_cus();
  const int64_t r128 = cdiv((int64_t)tM * tN * d.batch, slots), r64 = cdiv((int64_t)sM * sN * d.batch, slots);
  return 20 * r64 < 17 * 4 * r128;
}

template <bool TA, bool TB>
void launch(const GemmDesc& d, dim3 grid, hipStream_t s) {
  const bool vec = d.lda % 4 == 0 && d.ldb % 4 == 0 && d.strideA % 4 == 0 && d.strideB % 4 == 0 &&
                   ((uintptr_t)d.A & 15) == 0 && ((uintptr_t)d.B & 15) == 0;
  if (vec) hipLaunchKernelGGL((gemm_f32_kernel<TA, TB, true>), grid, dim3(256), 0, s, d);
  else hipLaunchKernelGGL((gemm_f32_kernel<TA, TB, false>), grid, dim3(256), 0, s, d);
}

}  // namespace

int device_cus() {
  static const int cus = [] {
    int dev = 0, c = 0;
    if (hipGetDevice(&dev) != hipSuccess || hipDeviceGetAttribute(&c, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || c <= 0)
      c = 256;
    return c;
  }();
  return cus;
}

hipError_t gemm_f32(const GemmDesc& d, bool transA, bool transB, hipStream_t s) {
  if (d.M <= 0 || d.N <= 0 || d.batch <= 0) return hipSuccess;
  dim3 grid;
  const int tM = (int)cdiv(d.M, BM), tN = (int)cdiv(d.N, BN);
  if (d.flags & GEMM_LOWER_TILES) grid = dim3((unsigned)(tM * (tM + 1) / 2), 1, (unsigned)d.batch);
  else grid = dim3((unsigned)tM, (unsigned)tN, (unsigned)d.batch);
  const int sM = (int)cdiv(d.M, SB), sN = (int)cdiv(d.N, SB);
  if (!transA && !transB && nn_dma_ok(d) && ((d.flags & GEMM_SMALL_TILES) || small_tiles_pay(d, tM, tN, sM, sN))) {
    hipLaunchKernelGGL(gemm_nn_dma64_kernel, dim3((unsigned)((int64_t)sM * sN * d.batch)), dim3(256), 0, s, d, sM, sN);
  } else if (!transA && !transB && nn_dma_ok(d)) {
    // split K when the tiles alone would give fewer than about four work
    // items per CU (the triangular products have K ranges from 128 to K, so
    // balance needs more items than workgroup slots) and K is long: chunks of
    // at least 256, multiples of 32, as many as the scratch holds
    const int64_t tiles = (int64_t)tM * tN * d.batch;
    int nsplit = 1, chunk = d.K;
    if (d.ws && d.K >= 512 && tiles < 1024) {
      int64_t want = std::min<int64_t>((1024 + tiles - 1) / tiles, d.K / 256);
      want = std::min<int64_t>(want, d.ws_floats / (tiles * BM * BN));
      if (want > 1) {
        chunk = (int)cdiv(cdiv(d.K, want), DBK) * DBK;
        nsplit = (int)cdiv(d.K, chunk);
      }
    }
    if (nsplit > 1) {
      const dim3 g2(grid.x, grid.y, grid.z * nsplit);
      hipLaunchKernelGGL(gemm_nn_dma_kernel, g2, dim3(256), 0, s, d, nsplit, chunk, d.ws);
      hipLaunchKernelGGL(gemm_split_reduce_kernel, grid, dim3(256), 0, s, d, nsplit, chunk, (const float*)d.ws);
    } else {
      hipLaunchKernelGGL(gemm_nn_dma_kernel, grid, dim3(256), 0, s, d, 1, d.K, (float*)nullptr);
    }
  } else if (!transA && !transB) launch<false, false>(d, grid, s);
  else if (!transA && transB) launch<false, true>(d, grid, s);
  else if (transA && !transB) launch<true, false>(d, grid, s);
  else launch<true, true>(d, grid, s);
  return hipGetLastError();
}

}  // namespace gptq
