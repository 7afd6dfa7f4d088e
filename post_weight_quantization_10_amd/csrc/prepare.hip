// Damping and the upper Cholesky factor of the damped inverse Hessian.
//
// What is computed: lambda = damp * mean(diag H) (the English GPTQ
// second-order quantization post, '3. Cholesky reformulation') and U upper
// with (H + lambda I)^{-1} = U^T U ("Part 3: Adaptive Rounding: GPTQ",
// 'Observation 3: The Cholesky Reformulation').
//
// How: if J is the reversal permutation and L' = chol(J H_d J) (lower), then
// H_d = (J L' J)(J L' J)^T with J L' J upper, so H_d^{-1} = U^T U with
// U = J L'^{-1} J.  By uniqueness of the Cholesky factor this is the same U as
// "invert, then factor the inverse", for one Cholesky and one triangular
// inverse (2n^3/3 flops) instead of four factor-sized steps (4n^3/3).
//
//   1. reversed copy + damping  A = J H J + lambda I             (HBM-bound)
//   2. blocked Cholesky of A in NB = 64 column blocks, two levels: panels of
//      PB = 4 blocks.  One launch per block column k of a panel: workgroup 0
//      takes the next diagonal block (it applies the update from block column
//      k to it, factors it and inverts the factor, Dinv_{k+1}); the other
//      workgroups own 128 x 128 lower tiles of the panel's remaining columns:
//      they solve the slabs they need on the fly, L21 = A21 Dinv_k^T (MFMA,
//      fp32), apply A22 <- A22 - L21 L21^T (MFMA, fp32), and the tiles of the
//      first tile column store their slab of L21 to L.  After the panel, one
//      rank-256 update from the stored panel of L: the launch that factors the
//      next panel's first diagonal block (its update taken from L) applies it
//      to the next panel's columns, and the rest of it is dealt out over the
//      next panel's launches.  So each diagonal block is factored while tiles
//      run, and the trailing matrix moves through memory once per 256
//      columns instead of once per 64.
//   3. triangular inverse in place by recursive doubling: with the NB-block
//      inverses on the diagonal, for block sizes s = NB, 2NB, ...:
//        L21^{-} = -L22^{-1} (L21 L11^{-1})   (two batched MFMA GEMMs)
//   4. U[i][j] = A[n-1-i][n-1-j] for i <= j, 0 below the diagonal.
#include <algorithm>

#include "common.hpp"
#include "internal.hpp"

namespace gptq {

namespace {

constexpr int NB = 64;

__global__ __launch_bounds__(1024) void damp_mean_kernel(const float* H, int64_t n, float damp, float* lam_ws,
                                                         float* lambda_out, int32_t* info) {
  __shared__ double part[1024];
  const int tid = threadIdx.x;
  double s = 0.0;
  for (int64_t i = tid; i < n; i += 1024) s += (double)H[i * n + i];
  part[tid] = s;
  __syncthreads();
  for (int w = 512; w > 0; w >>= 1) {
    if (tid < w) part[tid] += part[tid + w];
    __syncthreads();
  }
  if (tid == 0) {
    const float lam = (float)((double)damp * part[0] / (double)n);
    *lam_ws = lam;
    *lambda_out = lam;
    *info = 0;
  }
}

// A = J H J + lambda I   (A[i][j] = H[n-1-i][n-1-j])
__global__ __launch_bounds__(256) void reverse_damp_kernel(const float* H, float* A, int64_t n, const float* lam_ws) {
  const int64_t i = blockIdx.y;
  const float lam = *lam_ws;
  const float* src = H + (n - 1 - i) * n + (n - 1);
  float* dst = A + i * n;
  for (int64_t j = blockIdx.x * 256 + threadIdx.x; j < n; j += (int64_t)gridDim.x * 256) {
    float v = src[-j];
    if (j == i) v += lam;
    dst[j] = v;
  }
}

// The same with 16-byte accesses (n % 4 == 0, 16-byte aligned rows): A[i][j..j+3]
// is the reversed float4 H[n-1-i][n-4-j .. n-1-j].
__global__ __launch_bounds__(256) void reverse_damp4_kernel(const float* H, float* A, int64_t n, const float* lam_ws) {
  const float lam = *lam_ws;
  for (int64_t i = blockIdx.y; i < n; i += gridDim.y) {
    const float* src = H + (n - 1 - i) * n;
    for (int64_t j = 4 * ((int64_t)blockIdx.x * 256 + threadIdx.x); j < n; j += (int64_t)gridDim.x * 1024) {
      const f32x4 x = *(const f32x4*)(src + n - 4 - j);
      f32x4 y = {x[3], x[2], x[1], x[0]};
#pragma unroll
      for (int e = 0; e < 4; ++e)
        if (j + e == i) y[e] += lam;
      *(f32x4*)(A + i * n + j) = y;
    }
  }
}

constexpr int TB = 128;          // trailing-update tile
constexpr int PB = 4;            // block columns per panel of the two-level Cholesky
constexpr int64_t TWO_LEVEL_MIN = 4096;  // trailing columns below which a panel runs to the end
constexpr int LP = 65;           // LDS pitch of 64-column leaf matrices (floats)
constexpr int LLP = 68;          // LDS pitch of the leaf factor: 16-byte aligned rows
constexpr int PP = 68;           // LDS pitch of the leaf's product operands: 16-byte aligned rows
constexpr int SMEM = 20480;      // floats of LDS per workgroup (80 KiB)
static_assert(64 * LP + 2 * 64 * PP + 64 * LLP + 65 <= SMEM, "leaf LDS layout");
static_assert(64 * LLP + 32 * 33 <= 2 * 64 * PP, "the inverse and the doubling products fit over the product buffers");
static_assert(64 * 64 + 2 * 128 * 64 <= SMEM, "tile LDS layout");

__device__ __forceinline__ f32x16 mfma_f32(float a, float b, const f32x16& c) {
  return __builtin_amdgcn_mfma_f32_32x32x2f32(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ float readlane_f(float v, int l) {
  return __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), l));
}

// Diagonal block J = [j0, j0 + kb) (workgroup-wide, 256 threads).
//
// If kp >= 0, first the update from block column K = [kp, kp + NB):
//   Lrow = A[J, K] Dinv_K^T   (the rows J of that block column of the factor)
//   D    = A[J, J] - Lrow Lrow^T
// (two 64 x 64 x 64 MFMA products).  If lnk > 0 instead, the update from lnk
// block columns of the factor stored in L from column lk0 on:
//   D    = A[J, J] - sum_c L[J, lk0 + 64c] L[J, lk0 + 64c]^T
// (one 64 x 64 x 64 product per slab).  Else D = A[J, J].  Then D = L L^T and
// Dinv_J = L^{-1}, written to dinv_out (NB x NB, zero outside the kb x kb
// lower triangle).  Rows and columns past kb are padded with the identity.
//
// The factorization is blocked in four panels of PW = 16 columns: wave 0
// factors a panel (lane i holds the panel's part of row i in registers; at
// column j the pivot comes from lane j and each later panel column is updated
// with a readlane of l: at most 15 FMAs per column, no LDS, no branch), then
// all four waves apply the panel to the rest of the block with
// v_mfma_f32_16x16x4f32.  The inverse: one wave inverts the four 16 x 16
// diagonal blocks at once (lane = block, column; forward substitution), then
// two levels of recursive doubling, X21 = -X22 (L21 X11), with MFMA products.
// (A single wave issues an independent VALU op only every ~7 cycles, so the
// work that is not on the column chain goes to the matrix cores.)
__device__ __forceinline__ void leaf_block(const float* __restrict__ A, int64_t n, int64_t j0, int64_t kp,
                                        const float* __restrict__ dinv_prev, float* __restrict__ dinv_out,
                                        int32_t* info, float* smem, const float* __restrict__ Lsrc = nullptr,
                                        int64_t lk0 = 0, int lnk = 0) {
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int kb = (int)min<int64_t>(NB, n - j0);
  float* sD = smem;              // 64 x LP
  float* sP = sD + 64 * LP;      // 64 x PP
  float* sQ = sP + 64 * PP;      // 64 x PP
  float* sL = sQ + 64 * PP;      // 64 x LLP: the factor (above the diagonal only zeros and unread values)
  float* sX = sP;                // 64 x LLP over sP and sQ once the update is applied: the inverse
  float* sT = sP + 64 * LLP;     // 32 x 33: products of the doubling steps
  float* rinv = sL + 64 * LLP;   // 64: 1 / L[j][j]
  int* failed = (int*)(rinv + 64);

  // All loads in flight together, then to LDS.  (The empty asm makes every
  // load unconditional; otherwise the compiler moves each load under its
  // select, one wait per load.)
  if (kb == NB && (n & 3) == 0) {  // full block: 16-byte loads
    f32x4 v[4], pv[4], qv[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int e = tid + 256 * u;
      const int r = e >> 4, c = 4 * (e & 15);
      v[u] = *(const f32x4*)&A[(j0 + r) * n + j0 + c];
      if (kp >= 0) {
        pv[u] = *(const f32x4*)&A[(j0 + r) * n + kp + c];
        qv[u] = *(const f32x4*)&dinv_prev[r * NB + c];
      }
    }
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      asm volatile("" : "+v"(v[u]));
      const int e = tid + 256 * u;
      const int r = e >> 4, c = 4 * (e & 15);
#pragma unroll
      for (int q = 0; q < 4; ++q) sD[r * LP + c + q] = (c + q <= r) ? v[u][q] : 0.f;
      if (kp >= 0) {
        asm volatile("" : "+v"(pv[u]));
        *(f32x4*)&sP[r * PP + c] = pv[u];
        *(f32x4*)&sQ[r * PP + c] = qv[u];
      }
    }
  } else {  // the last, partial block (or n not a multiple of 4): clamped addresses, then selects
    constexpr int NU = NB * NB / 256;
    float v[NU], pv[NU], qv[NU];
#pragma unroll
    for (int u = 0; u < NU; ++u) {
      const int e = tid + 256 * u;
      const int r = e >> 6, c = e & 63;
      const int rc = min(r, kb - 1), cc = min(c, kb - 1);
      v[u] = A[(j0 + rc) * n + j0 + cc];
      if (kp >= 0) {
        pv[u] = A[(j0 + rc) * n + kp + c];
        qv[u] = dinv_prev[r * NB + c];
      }
    }
#pragma unroll
    for (int u = 0; u < NU; ++u) {
      asm volatile("" : "+v"(v[u]));
      const int e = tid + 256 * u;
      const int r = e >> 6, c = e & 63;
      sD[r * LP + c] = (r < kb && c < kb) ? ((c <= r) ? v[u] : 0.f) : ((r == c) ? 1.f : 0.f);
      if (kp >= 0) {
        asm volatile("" : "+v"(pv[u]));
        sP[r * PP + c] = (r < kb) ? pv[u] : 0.f;
        sQ[r * PP + c] = qv[u];
      }
    }
  }
  if (tid == 0) *failed = 0;
  __syncthreads();

  // The products with v_mfma_f32_16x16x4f32 (lane l: A[l%16][l/16],
  // B[l/16][l%16]; result register r is row 4(l/16) + r, column l%16) on
  // 16 x 16 output blocks.  MFMA step 4t + q of a K = 64 sum gives lane
  // quarter kq = l/16 the index k = 16t + 4kq + q: one 16-byte read per
  // operand and group t, and a block that needs only k < 16(t+1) stops there.
  const int i16 = lane & 15, kq = lane >> 4;
  // D -= S S^T for the 64 x 64 slab S in sP, on the ten lower 16 x 16 blocks:
  // 3, 3, 2, 2 of them per wave.  Blocks (bi, bj): wave 0 (0,0) (1,0) (1,1);
  // wave 1 (2,0) (2,1) (2,2); wave 2 (3,0) (3,1); wave 3 (3,2) (3,3)
  auto dupd = [&]() {
    const int nblk = wave < 2 ? 3 : 2;
    const int bi0 = wave == 0 ? 0 : (wave == 1 ? 2 : 3);
#pragma unroll
    for (int b = 0; b < 3; ++b) {
      if (b < nblk) {
        const int bi = wave == 0 ? (b == 0 ? 0 : 1) : bi0;
        const int bj = wave == 0 ? (b == 0 ? 0 : b - 1) : (wave == 3 ? 2 + b : b);
        f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int t = 0; t < 4; ++t) {
          const f32x4 av = *(const f32x4*)&sP[(16 * bi + i16) * PP + 16 * t + 4 * kq];
          const f32x4 bv = *(const f32x4*)&sP[(16 * bj + i16) * PP + 16 * t + 4 * kq];
#pragma unroll
          for (int q = 0; q < 4; ++q) acc = __builtin_amdgcn_mfma_f32_16x16x4f32(av[q], bv[q], acc, 0, 0, 0);
        }
#pragma unroll
        for (int r = 0; r < 4; ++r) sD[(16 * bi + 4 * kq + r) * LP + 16 * bj + i16] -= acc[r];
      }
    }
  };
  if (kp >= 0) {
    {  // Lrow rows 16w.. = P[16w.., :] Dinv_K^T; column block bj needs k < 16(bj+1) (Dinv_K is lower)
      f32x4 acc[4];
#pragma unroll
      for (int bj = 0; bj < 4; ++bj) acc[bj] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        const f32x4 av = *(const f32x4*)&sP[(16 * wave + i16) * PP + 16 * t + 4 * kq];
#pragma unroll
        for (int bj = t; bj < 4; ++bj) {
          const f32x4 bv = *(const f32x4*)&sQ[(16 * bj + i16) * PP + 16 * t + 4 * kq];
#pragma unroll
          for (int q = 0; q < 4; ++q) acc[bj] = __builtin_amdgcn_mfma_f32_16x16x4f32(av[q], bv[q], acc[bj], 0, 0, 0);
        }
      }
      __syncthreads();  // every wave is done reading A[J, K]
#pragma unroll
      for (int bj = 0; bj < 4; ++bj)
#pragma unroll
        for (int r = 0; r < 4; ++r) sP[(16 * wave + 4 * kq + r) * PP + 16 * bj + i16] = acc[bj][r];
    }
    __syncthreads();
    dupd();
    __syncthreads();
  }
  if (lnk > 0) {
    // the slabs L[J, lk0 + 64c] in turn through sP (rows past kb zero)
    const bool v16 = (n & 3) == 0;
    for (int c = 0; c < lnk; ++c) {
      const float* src = Lsrc + lk0 + (int64_t)NB * c;
      f32x4 lv[4];
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const int e = tid + 256 * u;
        const int r = e >> 4, c4 = 4 * (e & 15);
        const float* q = src + (j0 + min(r, kb - 1)) * n + c4;
        lv[u] = v16 ? *(const f32x4*)q : f32x4{q[0], q[1], q[2], q[3]};
      }
      if (c > 0) __syncthreads();  // every wave is done with the previous slab
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const int e = tid + 256 * u;
        const int r = e >> 4, c4 = 4 * (e & 15);
        *(f32x4*)&sP[r * PP + c4] = r < kb ? lv[u] : f32x4{0.f, 0.f, 0.f, 0.f};
      }
      __syncthreads();
      dupd();
    }
    __syncthreads();
  }

  // sX is free now (the update is applied): waves 1..3 zero it while wave 0
  // factors the first panel, so that its upper blocks read as zero in the
  // doubling products
  if (wave > 0)
    for (int e = tid - 64; e < 64 * LLP; e += 192) sX[e] = 0.f;

  // ---- factor, PW-column panels.  Panel p: wave 0 applies panel p-1 to the
  // panel's own 16 columns and factors them (lane i holds row i of the panel
  // in registers; at column j the pivot comes from lane j and each later
  // panel column is updated with a readlane of l: no LDS, no branch), while
  // waves 1..3 apply panel p-1 to the column blocks after it.  One barrier
  // per panel.
  constexpr int PW = 16;
  const int l16 = lane & 15, g16 = lane >> 4;
  // D[16bi.., 16bj..] -= L[16bi.., q0:q0+16] L[16bj.., q0:q0+16]^T: a 16 x 16
  // block, v_mfma_f32_16x16x4f32 (lane l: A[l%16][l/16], B[l/16][l%16];
  // result register r is row 4(l/16) + r, column l%16)
  auto upd = [&](int bi, int bj, int q0) {
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int k = 0; k < PW; k += 4)
      acc = __builtin_amdgcn_mfma_f32_16x16x4f32(sL[(16 * bi + l16) * LLP + q0 + k + g16],
                                                  sL[(16 * bj + l16) * LLP + q0 + k + g16], acc, 0, 0, 0);
#pragma unroll
    for (int r = 0; r < 4; ++r) sD[(16 * bi + 4 * g16 + r) * LP + 16 * bj + l16] -= acc[r];
  };
#pragma unroll 1
  for (int p = 0; p < NB / PW; ++p) {
    const int c0 = PW * p;
    if (wave == 0) {
      for (int bi = p; p > 0 && bi < NB / 16; ++bi) upd(bi, p, c0 - PW);
      float a[PW];
#pragma unroll
      for (int k = 0; k < PW; ++k) a[k] = sD[lane * LP + c0 + k];
      // Per column only the pivot's readlane, its 1/sqrt and the scaling sit
      // on the chain.  Rows above the pivot are scaled too: those entries (the
      // upper part of the panel's own 16 x 16 block; rows of earlier panels
      // stay exactly 0) are never read, as later panels, the substitution and
      // the doubling products read only the strictly lower part of that block.
      // The next column's pivot is taken from pn = a[jj+1] - l^2, which in
      // lane c0 + jj + 1 is exactly that lane's updated a[jj+1] (there the
      // broadcast l is its own), so no readlane of l sits on the chain.
      float rsv[PW];
      float piv = readlane_f(a[0], c0);
#pragma unroll
      for (int jj = 0; jj < PW; ++jj) {
        const float rs = __builtin_amdgcn_rsqf(piv);  // not finite after a failure: the rest is discarded
        rsv[jj] = rs;
        const float l = a[jj] * rs;  // lane c0 + jj: piv rs = sqrt(piv)
        a[jj] = l;
        if (jj + 1 < PW) piv = readlane_f(fmaf(-l, l, a[jj + 1]), c0 + jj + 1);
#pragma unroll
        for (int k = jj + 1; k < PW; ++k) a[k] = fmaf(-l, readlane_f(l, c0 + k), a[k]);
      }
      if (lane == 0) {
#pragma unroll
        for (int k = 0; k < PW; k += 4) *(f32x4*)&rinv[c0 + k] = f32x4{rsv[k], rsv[k + 1], rsv[k + 2], rsv[k + 3]};
      }
#pragma unroll
      for (int k = 0; k < PW; ++k) sL[lane * LLP + c0 + k] = a[k];
    } else if (p > 0) {
      // lower blocks (bi, bj) with p < bj <= bi, one per wave in turn
      const int nb = NB / 16 - 1 - p;
      for (int t = wave - 1; t < nb * (nb + 1) / 2; t += 3) {
        int bi = 0;
        while ((bi + 1) * (bi + 2) / 2 <= t) ++bi;
        const int bj = t - bi * (bi + 1) / 2;
        upd(p + 1 + bi, p + 1 + bj, c0 - PW);
      }
    }
    __syncthreads();
  }
  // the first column whose pivot is not positive and finite, i.e. whose
  // 1/sqrt is not positive and finite (0 for an infinite pivot, infinite for
  // 0, NaN below 0); padding columns past kb have pivot 1
  if (wave == 0) {
    const float r = rinv[lane];
    const uint64_t badm = __ballot(!(r > 0.f && r < INFINITY));
    if (badm != 0 && lane == 0) {
      atomicCAS(info, 0, (int32_t)(n - (j0 + (int)__builtin_ctzll(badm))));
      *failed = 1;
    }
  }

  // ---- inverse.  The four 16 x 16 diagonal blocks: lane = (block g16,
  // column l16) forward-substitutes its column of the block's inverse.
  if (wave == 0) {
    const int base = 16 * g16;
    float x[16];
#pragma unroll
    for (int j = 0; j < 16; ++j) {
      f32x4 v[4];
#pragma unroll
      for (int g = 0; 4 * g < j; ++g) v[g] = *(const f32x4*)&sL[(base + j) * LLP + base + 4 * g];
      float s0 = (l16 == j) ? 1.f : 0.f, s1 = 0.f;
#pragma unroll
      for (int q = 0; q < j; ++q) {
        if (q & 1) s1 = fmaf(-v[q >> 2][q & 3], x[q], s1);
        else s0 = fmaf(-v[q >> 2][q & 3], x[q], s0);
      }
      x[j] = (s0 + s1) * rinv[base + j];
    }
#pragma unroll
    for (int j = 0; j < 16; ++j) sX[(base + j) * LLP + base + l16] = x[j];
  }
  __syncthreads();

  // 16 x 16 output block (row r0, column s0) of -X[r0.., kr..] T or of
  // L[r0.., k..] X[k.., s0..]: C = sum over K of A[r][k] B[k][c]
  auto prod16 = [&](const float* Am, int lda_, int ar, int ac, const float* Bm, int ldb_, int br, int bc_,
                    int K) {
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
    for (int k = 0; k < K; k += 4)
      acc = __builtin_amdgcn_mfma_f32_16x16x4f32(Am[(ar + l16) * lda_ + ac + k + g16],
                                                  Bm[(br + k + g16) * ldb_ + bc_ + l16], acc, 0, 0, 0);
    return acc;
  };
  // doubling, 16 -> 32: pairs (0, 1) and (2, 3), wave 0 and wave 1
  if (wave < 2) {
    const int b0 = 32 * wave;  // X[b0+16.., b0..] = -X[b0+16.., b0+16..] (L[b0+16.., b0..] X[b0.., b0..])
    const f32x4 t = prod16(sL, LLP, b0 + 16, b0, sX, LLP, b0, b0, 16);
#pragma unroll
    for (int r = 0; r < 4; ++r) sT[(16 * wave + 4 * g16 + r) * 33 + l16] = t[r];
  }
  __syncthreads();
  if (wave < 2) {
    const int b0 = 32 * wave;
    const f32x4 t = prod16(sX, LLP, b0 + 16, b0 + 16, sT + 16 * wave * 33, 33, 0, 0, 16);
#pragma unroll
    for (int r = 0; r < 4; ++r) sX[(b0 + 16 + 4 * g16 + r) * LLP + b0 + l16] = -t[r];
  }
  __syncthreads();
  // doubling, 32 -> 64: X[32.., ..32] = -X[32.., 32..] (L[32.., ..32] X[..32, ..32]);
  // wave w computes the 16 x 16 block (w >> 1, w & 1) of each product
  {
    const int br = 16 * (wave >> 1), bcol = 16 * (wave & 1);
    const f32x4 t = prod16(sL, LLP, 32 + br, 0, sX, LLP, 0, bcol, 32);
#pragma unroll
    for (int r = 0; r < 4; ++r) sT[(br + 4 * g16 + r) * 33 + bcol + l16] = t[r];
  }
  __syncthreads();
  {
    const int br = 16 * (wave >> 1), bcol = 16 * (wave & 1);
    const f32x4 t = prod16(sX, LLP, 32 + br, 32, sT, 33, 0, bcol, 32);
#pragma unroll
    for (int r = 0; r < 4; ++r) sX[(32 + br + 4 * g16 + r) * LLP + bcol + l16] = -t[r];
  }
  __syncthreads();
  if (*failed == 0) {
#pragma unroll
    for (int u = 0; u < NB * NB / 256; ++u) {
      const int e = tid + 256 * u;
      const int r = e >> 6, c = e & 63;
      dinv_out[r * NB + c] = (r < kb && c < kb) ? sX[r * LLP + c] : 0.f;
    }
  }
}

__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(1, 1))) void chol_first_kernel(const float* A, int64_t n, float* dinv, int32_t* info) {
  if (*info != 0) return;
  __shared__ __attribute__((aligned(16))) float smem[SMEM];
  leaf_block(A, n, 0, -1, nullptr, dinv, info, smem);
}

// Panel layout in LDS: [rows][64] floats, 16-byte groups XOR-swizzled by row.
__device__ __forceinline__ int pidx(int r, int k) { return r * 64 + (k ^ ((r & 15) << 2)); }

template <bool VEC>
__device__ __forceinline__ f32x4 ld4(const float* p) {
  return VEC ? *(const f32x4*)p : f32x4{p[0], p[1], p[2], p[3]};
}

// K order of the 32 steps of a K = 64 product with v_mfma_f32_32x32x2f32:
// step s gives lane half kr (lanes 32 kr ..) the index
// k = 32 (s / 16) + 16 kr + s % 16, so each lane walks contiguous runs of k
// (16-byte LDS reads, four steps per read) and steps 0..15 see only k < 32.
// Any order is the same sum; the first operand and the second use the same one.
__device__ __forceinline__ int kgroup(int g, int kr) { return 32 * (g >> 2) + 16 * kr + 4 * (g & 3); }  // g = s / 4

// Rows 32w..32w+31 of S (a 64-column panel in LDS) times Dinv^T, both 32-wide
// output blocks, for this wave.  The operands of steps 4g+4.. are read while
// the MFMAs of steps 4g.. run.
__device__ __forceinline__ void panel_solve(const float* S, const float* sD, int w, int lane, f32x16 (&o)[2]) {
  const int kr = lane >> 5, cl = lane & 31;
  o[0] = zero16();
  o[1] = zero16();
  f32x4 av[2], d0[2], d1[2];
  auto ld = [&](int g, int b) {
    const int k = kgroup(g, kr);
    av[b] = *(const f32x4*)&S[pidx(32 * w + cl, k)];
    if (g < 4) d0[b] = *(const f32x4*)&sD[pidx(cl, k)];  // Dinv is lower triangular: columns 0..31 need k < 32
    d1[b] = *(const f32x4*)&sD[pidx(32 + cl, k)];
  };
  ld(0, 0);
#pragma unroll
  for (int g = 0; g < 8; ++g) {
    const int b = g & 1;
    if (g + 1 < 8) ld(g + 1, b ^ 1);
    __builtin_amdgcn_sched_barrier(0);  // keeps the reads ahead of this group's MFMAs
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      if (g < 4) o[0] = mfma_f32(av[b][q], d0[b][q], o[0]);
      o[1] = mfma_f32(av[b][q], d1[b][q], o[1]);
    }
    __builtin_amdgcn_sched_barrier(0);
  }
}

// Tile lists.  A region [R0, n) x [R0, cend) of the trailing matrix is cut
// into 128 x 128 tiles, nr tile rows and nc <= nr tile columns; its lower
// tiles (tm >= tn) are listed column by column, so column j starts at
// C(j) = j nr - j (j - 1) / 2.
__device__ __forceinline__ void region_tile(int t, int nr, int& tm, int& tn) {
  const float b = 2.f * (float)nr + 1.f;
  int j = (int)((b - sqrtf(fmaxf(b * b - 8.f * (float)t, 0.f))) * 0.5f);
  auto C = [nr](int c) { return c * nr - c * (c - 1) / 2; };
  while (j > 0 && C(j) > t) --j;
  while (C(j + 1) <= t) ++j;
  tn = j;
  tm = j + (t - C(j));
}

// One 128 x 128 lower tile (tm, tn) of the region [R0, n) x [R0, cend):
//   C -= sum over slabs S of S[rows] S[cols]^T,
// S a 64-column block column of the factor.  SOLVE: one slab, solved here
// from A's block column at k0 (S = A21 Dinv_k^T, MFMA fp32), and the tiles of
// the first tile column store their rows of it to L.  Else nk slabs read from
// L's columns k0 + 64 c, the next slab's loads in flight while the current
// one's MFMAs run.  skip00: the first 64 x 64 quadrant of tile (0, 0) is a
// diagonal block that workgroup 0 updates itself.
template <bool VEC, bool SOLVE>
__device__ __forceinline__ void tile_update(float* __restrict__ A, float* __restrict__ L,
                                            const float* __restrict__ dinv_k, int64_t n, int64_t k0, int nk,
                                            int64_t R0, int64_t cend, int tm, int tn, bool skip00, float* smem) {
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  float* sD = smem;            // 64 x 64: Dinv_k (SOLVE)
  float* sR = sD + 64 * 64;    // 128 x 64: the tile's row slab (SOLVE: A21, then L21)
  float* sC = sR + 128 * 64;   // 128 x 64: the same for the column slab
  const int64_t r0 = R0 + (int64_t)tm * TB, c0 = R0 + (int64_t)tn * TB;
  const bool dg = tm == tn;
  const int wr = wave >> 1, wc = wave & 1;
  // Nothing to do for a quadrant of a diagonal tile above the diagonal, for
  // one whose columns all lie past cend, and for the skipped diagonal block.
  const bool active =
      !(dg && wr < wc) && c0 + 64 * wc < cend && !(skip00 && tm == 0 && tn == 0 && wr == 0 && wc == 0);
  const uint32_t n32 = (uint32_t)n;
  const float* P = SOLVE ? (const float*)A : (const float*)L;

  // Rows of the tile's row and column slabs at column col, all loads in
  // flight together.  Rows past n are clamped: they only reach outputs that
  // are never stored.
  f32x4 pr[8], pc[8];
  auto load_slabs = [&](int64_t col) {
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const int e = tid + 256 * u;
      const int r = e >> 4, g = 4 * (e & 15);
      pr[u] = ld4<VEC>(P + min(r0 + r, n - 1) * n + col + g);
      if (!dg) pc[u] = ld4<VEC>(P + min(c0 + r, n - 1) * n + col + g);
    }
  };
  auto store_slabs = [&]() {
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const int e = tid + 256 * u;
      const int r = e >> 4, g = 4 * (e & 15);
      *(f32x4*)&sR[pidx(r, g)] = pr[u];
      if (!dg) *(f32x4*)&sC[pidx(r, g)] = pc[u];
    }
  };
  const int cl = lane & 31, kr = lane >> 5;

  // C of this wave's 64 x 64 quadrant through a buffer resource over the
  // tile's rows inside the matrix and 32-bit lane offsets (the tile spans
  // fewer than 128 n elements, n < 2^22).  Loads past the last row read as
  // zero and entries past n or cend are never stored, so edge tiles need no
  // clamping; a store that must not happen gets an offset past the buffer and
  // is dropped, so no store is behind a branch.
  const bool interior = r0 + TB <= n && c0 + TB <= cend;
  const uint32_t lr0 = (uint32_t)(64 * wr + 4 * (lane >> 5)), lc0 = (uint32_t)(64 * wc + (lane & 31));
  const uint32_t rlim = (uint32_t)(min<int64_t>(TB, n - r0) - 1), clim = (uint32_t)(min<int64_t>(TB, cend - c0) - 1);
  const __amdgpu_buffer_rsrc_t trs =
      __builtin_amdgcn_make_buffer_rsrc(A + (r0 * n + c0), 0, (int)((rlim + 1) * n32 * 4u), 0x00020000);
  const uint32_t loff = (lr0 * n32 + lc0) * 4u;
  auto coff = [&](int mb, int nb, int r) {
    return loff + ((uint32_t)(32 * mb + 8 * (r >> 2) + (r & 3)) * n32 + (uint32_t)(32 * nb)) * 4u;
  };
  f32x16 cp[2][2];
  auto load_c = [&]() {
#pragma unroll
    for (int mb = 0; mb < 2; ++mb)
#pragma unroll
      for (int nb = 0; nb < 2; ++nb) {
        cp[mb][nb] = zero16();
        if (active) {
#pragma unroll
          for (int r = 0; r < 16; ++r)
            cp[mb][nb][r] = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(trs, coff(mb, nb, r), 0, 0));
        }
      }
  };

  f32x16 acc[2][2];
#pragma unroll
  for (int mb = 0; mb < 2; ++mb)
#pragma unroll
    for (int nb = 0; nb < 2; ++nb) acc[mb][nb] = zero16();
  const float* sB = dg ? sR : sC;
  // acc += (rows of sR) (rows of sB)^T over the slab's 64 columns; the
  // operands of steps 4g+4.. are read while the MFMAs of steps 4g.. run
  auto rank_update = [&]() {
    f32x4 a0[2], a1[2], b0[2], b1[2];
    auto ld = [&](int g, int b) {
      const int k = kgroup(g, kr);
      a0[b] = *(const f32x4*)&sR[pidx(64 * wr + cl, k)];
      a1[b] = *(const f32x4*)&sR[pidx(64 * wr + 32 + cl, k)];
      b0[b] = *(const f32x4*)&sB[pidx(64 * wc + cl, k)];
      b1[b] = *(const f32x4*)&sB[pidx(64 * wc + 32 + cl, k)];
    };
    ld(0, 0);
#pragma unroll
    for (int g = 0; g < 8; ++g) {
      const int b = g & 1;
      if (g + 1 < 8) ld(g + 1, b ^ 1);
      __builtin_amdgcn_sched_barrier(0);  // keeps the reads ahead of this group's MFMAs
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        acc[0][0] = mfma_f32(a0[b][q], b0[b][q], acc[0][0]);
        acc[0][1] = mfma_f32(a0[b][q], b1[b][q], acc[0][1]);
        acc[1][0] = mfma_f32(a1[b][q], b0[b][q], acc[1][0]);
        acc[1][1] = mfma_f32(a1[b][q], b1[b][q], acc[1][1]);
      }
      __builtin_amdgcn_sched_barrier(0);
    }
  };

  if constexpr (SOLVE) {
    {
      f32x4 dv[4];
      load_slabs(k0);
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const int e = tid + 256 * u;
        dv[u] = *(const f32x4*)&dinv_k[(e >> 4) * NB + 4 * (e & 15)];
      }
      store_slabs();
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const int e = tid + 256 * u;
        *(f32x4*)&sD[pidx(e >> 4, 4 * (e & 15))] = dv[u];
      }
    }
    __syncthreads();
    // L21 slabs; each wave reads and then overwrites only its own 32 rows.
    // The first tile column stores its slab of L21: rows past n fall outside
    // this buffer and are dropped.
    const __amdgpu_buffer_rsrc_t lrs = __builtin_amdgcn_make_buffer_rsrc(
        L + (r0 * n + k0), 0, (int)((uint32_t)min<int64_t>(TB, n - r0) * n32 * 4u), 0x00020000);
    // The solved rows go back in place.  Output register r of a 32 x 32 block
    // is row 32w + 4kr + 8(r/4) + r%4 (column cl), so its swizzled LDS index is
    // a lane term plus a constant: (row & 15) = 4kr | (8(r/4 % 2) + r%4).
    auto put = [&](float* S, const f32x16 (&v)[2]) {
#pragma unroll
      for (int nb = 0; nb < 2; ++nb) {
        const int lc = (32 * nb + cl) ^ (kr << 4);
        float* base = S + (32 * wave + 4 * kr) * 64;
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int rc = 8 * (r >> 2) + (r & 3);
          base[rc * 64 + (lc ^ ((rc & 15) << 2))] = v[nb][r];
        }
      }
    };
    f32x16 o[2];
    panel_solve(sR, sD, wave, lane, o);
    put(sR, o);
    if (tn == 0) {  // row 32w + 4kr + rc of the slab: a lane term plus a uniform multiple of n
      const uint32_t lb = (uint32_t)(32 * wave + 4 * kr) * n32 + (uint32_t)cl;
#pragma unroll
      for (int nb = 0; nb < 2; ++nb)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const float v = o[nb][r];  // (a bit cast of the vector element itself reads element 0)
          __builtin_amdgcn_raw_buffer_store_b32(__builtin_bit_cast(int, v), lrs,
                                                (lb + (uint32_t)(8 * (r >> 2) + (r & 3)) * n32 + 32u * nb) * 4u, 0, 0);
        }
    }
    if (!dg) {
      panel_solve(sC, sD, wave, lane, o);
      put(sC, o);
    }
    load_c();  // fetched only now, so that it is not live during the panel solves
    __syncthreads();
    if (active) rank_update();
  } else {
    // the next slab's loads (or, with the last slab, C's) in flight during
    // the current slab's MFMAs: never both sets of registers live at once
    load_slabs(k0);
    for (int c = 0; c + 1 < nk; ++c) {
      if (c > 0) __syncthreads();  // every wave is done with the previous slabs
      store_slabs();
      __syncthreads();
      load_slabs(k0 + (int64_t)NB * (c + 1));
      if (active) rank_update();
    }
    if (nk > 1) __syncthreads();
    store_slabs();
    __syncthreads();
    load_c();
    if (active) rank_update();
  }
  if (!active) return;

  // lower part only
  if (interior && !dg) {
#pragma unroll
    for (int mb = 0; mb < 2; ++mb)
#pragma unroll
      for (int nb = 0; nb < 2; ++nb)
#pragma unroll
        for (int r = 0; r < 16; ++r)
          __builtin_amdgcn_raw_buffer_store_b32(__builtin_bit_cast(int, cp[mb][nb][r] - acc[mb][nb][r]), trs,
                                                coff(mb, nb, r), 0, 0);
    return;
  }
#pragma unroll
  for (int mb = 0; mb < 2; ++mb)
#pragma unroll
    for (int nb = 0; nb < 2; ++nb)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const uint32_t lr = lr0 + (uint32_t)(32 * mb + 8 * (r >> 2) + (r & 3)), lc = lc0 + (uint32_t)(32 * nb);
        // inside the matrix and the region, and on or below the diagonal of
        // a diagonal tile (there r0 = c0)
        const bool st = lr <= rlim && lc <= clim && (!dg || lc <= lr);
        __builtin_amdgcn_raw_buffer_store_b32(__builtin_bit_cast(int, cp[mb][nb][r] - acc[mb][nb][r]), trs,
                                              st ? coff(mb, nb, r) : 0x80000000u, 0, 0);
      }
}

// Rows [r0, r0 + 128) of the block column at k0 of the factor,
// L21 = A21 Dinv_k^T, written to L (rows past n dropped).
template <bool VEC>
__device__ __forceinline__ void solve_slab(const float* __restrict__ A, float* __restrict__ L,
                                           const float* __restrict__ dinv_k, int64_t n, int64_t k0, int64_t r0,
                                           float* smem) {
  float* sD = smem;          // 64 x 64
  float* sR = sD + 64 * 64;  // 128 x 64
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  {
    f32x4 pr[8], dv[4];
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const int e = tid + 256 * u;
      pr[u] = ld4<VEC>(A + min(r0 + (e >> 4), n - 1) * n + k0 + 4 * (e & 15));
    }
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int e = tid + 256 * u;
      dv[u] = *(const f32x4*)&dinv_k[(e >> 4) * NB + 4 * (e & 15)];
    }
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const int e = tid + 256 * u;
      *(f32x4*)&sR[pidx(e >> 4, 4 * (e & 15))] = pr[u];
    }
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int e = tid + 256 * u;
      *(f32x4*)&sD[pidx(e >> 4, 4 * (e & 15))] = dv[u];
    }
  }
  __syncthreads();
  f32x16 o[2];
  panel_solve(sR, sD, wave, lane, o);
  const uint32_t n32 = (uint32_t)n;
  const __amdgpu_buffer_rsrc_t lrs = __builtin_amdgcn_make_buffer_rsrc(
      L + (r0 * n + k0), 0, (int)((uint32_t)min<int64_t>(TB, n - r0) * n32 * 4u), 0x00020000);
  const int cl = lane & 31, kr = lane >> 5;
  const uint32_t lb = (uint32_t)(32 * wave + 4 * kr) * n32 + (uint32_t)cl;
#pragma unroll
  for (int nb = 0; nb < 2; ++nb)
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const float v = o[nb][r];  // (a bit cast of the vector element itself reads element 0)
      __builtin_amdgcn_raw_buffer_store_b32(__builtin_bit_cast(int, v), lrs,
                                            (lb + (uint32_t)(8 * (r >> 2) + (r & 3)) * n32 + 32u * nb) * 4u, 0, 0);
    }
}

// One launch of the blocked Cholesky, three kinds of workgroup, in this
// order of blockIdx:
//  - workgroup 0 factors the diagonal block at leaf_j0 (leaf_mode 1: after
//    the update from the block column at leaf_kp, from A and that block's
//    inverse; 2: after the update from leaf_nk block columns of L starting at
//    column leaf_kp; 0: no leaf in this launch);
//  - lt1 - lt0 workgroups update tiles [lt0, lt1) of the lower tile list of
//    [lR0, n) x [lR0, lcend) from lnk block columns of L starting at lk0
//    (lskip00: not the diagonal block at lR0, which workgroup 0 updates);
//  - nstrip workgroups update the tiles of [sk0 + 64, n) x [sk0 + 64, send)
//    (the rest of a panel's columns) from the block column at sk0, solving it
//    on the fly and storing it to L; or, with no strip, nsolve workgroups
//    solve and store that block column's 128-row slabs.
struct StepArgs {
  float* A;
  float* L;
  float* dinv;
  int32_t* info;
  int64_t n;
  int64_t leaf_j0, leaf_kp;
  int leaf_mode, leaf_nk;
  int64_t sk0, send;
  int s_nr, nstrip, nsolve;
  int64_t lk0, lR0, lcend;
  int lnk, l_nr, lt0, lt1, lskip00;
};

template <bool VEC>
__global__ __launch_bounds__(256, 2) void chol_step_kernel(StepArgs a) {
  if (*a.info != 0) return;
  __shared__ __attribute__((aligned(16))) float smem[SMEM];
  int b = (int)blockIdx.x;
  if (b == 0) {
    if (a.leaf_mode == 1)
      leaf_block(a.A, a.n, a.leaf_j0, a.leaf_kp, a.dinv + (a.leaf_kp / NB) * NB * NB,
                 a.dinv + (a.leaf_j0 / NB) * NB * NB, a.info, smem);
    else if (a.leaf_mode == 2)
      leaf_block(a.A, a.n, a.leaf_j0, -1, nullptr, a.dinv + (a.leaf_j0 / NB) * NB * NB, a.info, smem, a.L,
                 a.leaf_kp, a.leaf_nk);
    return;
  }
  // The longest workgroups go out first: the rank-256 tiles from L (about
  // three times a strip tile), then the strip tiles, then the slab solves,
  // which fill the CUs the long tiles leave idle at the launch's end.
  b -= 1;
  if (b < a.lt1 - a.lt0) {
    int tm, tn;
    region_tile(a.lt0 + b, a.l_nr, tm, tn);
    tile_update<VEC, false>(a.A, a.L, nullptr, a.n, a.lk0, a.lnk, a.lR0, a.lcend, tm, tn, a.lskip00 != 0, smem);
    return;
  }
  b -= a.lt1 - a.lt0;
  const float* dk = a.dinv + (a.sk0 / NB) * NB * NB;
  if (b < a.nstrip) {
    int tm, tn;
    region_tile(b, a.s_nr, tm, tn);
    tile_update<VEC, true>(a.A, a.L, dk, a.n, a.sk0, 1, a.sk0 + NB, a.send, tm, tn, true, smem);
    return;
  }
  b -= a.nstrip;
  if (b < a.nsolve) solve_slab<VEC>(a.A, a.L, dk, a.n, a.sk0, a.sk0 + NB + (int64_t)TB * b, smem);
}

// Zero the strict upper triangle and put the NB-block inverses on the diagonal.
__global__ __launch_bounds__(256) void trtri_init_kernel(float* A, int64_t n, const float* Dinv, const int32_t* info) {
  if (*info != 0) return;
  const int64_t i = blockIdx.y;
  const int64_t bi = i / NB;
  for (int64_t j = blockIdx.x * 256 + threadIdx.x; j < n; j += (int64_t)gridDim.x * 256) {
    if (j > i) A[i * n + j] = 0.f;
    else if (j / NB == bi) A[i * n + j] = Dinv[bi * NB * NB + (i - bi * NB) * NB + (j - bi * NB)];
  }
}

// 16-byte variants (n % 4 == 0, 16-byte aligned rows; block boundaries never
// split a float4 since NB % 4 == 0).
__global__ __launch_bounds__(256) void trtri_init4_kernel(float* A, int64_t n, const float* Dinv, const int32_t* info) {
  if (*info != 0) return;
  for (int64_t i = blockIdx.y; i < n; i += gridDim.y) {
    const int64_t bi = i / NB;
    const float* drow = Dinv + bi * NB * NB + (i - bi * NB) * NB - bi * NB;  // + j
    for (int64_t j = 4 * ((int64_t)blockIdx.x * 256 + threadIdx.x); j < n; j += (int64_t)gridDim.x * 1024) {
      float* dst = A + i * n + j;
      if (j > i) {
        *(f32x4*)dst = f32x4{0.f, 0.f, 0.f, 0.f};
      } else if (j / NB == bi) {
        if (j + 3 <= i) *(f32x4*)dst = *(const f32x4*)(drow + j);
        else {
#pragma unroll
          for (int e = 0; e < 4; ++e) dst[e] = (j + e > i) ? 0.f : drow[j + e];
        }
      }
    }
  }
}

__global__ __launch_bounds__(256) void write_u4_kernel(const float* A, float* U, int64_t n, const int32_t* info) {
  if (*info != 0) return;
  for (int64_t i = blockIdx.y; i < n; i += gridDim.y) {
    const float* src = A + (n - 1 - i) * n;
    for (int64_t j = 4 * ((int64_t)blockIdx.x * 256 + threadIdx.x); j < n; j += (int64_t)gridDim.x * 1024) {
      f32x4 y = {0.f, 0.f, 0.f, 0.f};
      if (j + 3 >= i) {
        const f32x4 x = *(const f32x4*)(src + n - 4 - j);
#pragma unroll
        for (int e = 0; e < 4; ++e) y[e] = (j + e >= i) ? x[3 - e] : 0.f;
      }
      *(f32x4*)(U + i * n + j) = y;
    }
  }
}

// U[i][j] = Linv[n-1-i][n-1-j] for i <= j, 0 below the diagonal.
__global__ __launch_bounds__(256) void write_u_kernel(const float* A, float* U, int64_t n, const int32_t* info) {
  if (*info != 0) return;
  const int64_t i = blockIdx.y;
  const float* src = A + (n - 1 - i) * n + (n - 1);
  for (int64_t j = blockIdx.x * 256 + threadIdx.x; j < n; j += (int64_t)gridDim.x * 256)
    U[i * n + j] = (j >= i) ? src[-j] : 0.f;
}

inline size_t align256(size_t b) { return (b + 255) & ~(size_t)255; }

struct PrepWs {
  float* A;     // damped, reversed H; its trailing part is updated in place
  float* L;     // the factor, then its inverse
  float* dinv;  // inverses of the NB x NB diagonal blocks of the factor
  float* lam;
};

PrepWs carve(void* ws, int64_t n) {
  char* p = (char*)ws;
  PrepWs w;
  w.A = (float*)p;
  p += align256((size_t)n * n * 4);
  w.L = (float*)p;
  p += align256((size_t)n * n * 4);
  w.dinv = (float*)p;
  p += align256((size_t)cdiv(n, NB) * NB * NB * 4);
  w.lam = (float*)p;
  return w;
}

dim3 row_grid(int64_t n) { return dim3((unsigned)std::min<int64_t>(cdiv(n, 256), 64), (unsigned)n); }
dim3 row_grid4(int64_t n) {
  return dim3((unsigned)std::min<int64_t>(cdiv(n, 1024), 64), (unsigned)std::min<int64_t>(n, 65535));
}

}  // namespace

size_t prepare_workspace_bytes(int64_t n) {
  if (n < 1) return 0;
  return 2 * align256((size_t)n * n * 4) + align256((size_t)cdiv(n, NB) * NB * NB * 4) + 256;
}

hipError_t prepare_hinv(const float* H, int64_t n, float damp, float* U, int32_t* info, float* lambda_out, void* ws,
                        hipStream_t s) {
  PrepWs w = carve(ws, n);
  hipLaunchKernelGGL(damp_mean_kernel, dim3(1), dim3(1024), 0, s, H, n, damp, w.lam, lambda_out, info);
  const bool v4 = n % 4 == 0 && ((uintptr_t)H & 15) == 0 && ((uintptr_t)U & 15) == 0;
  if (v4) hipLaunchKernelGGL(reverse_damp4_kernel, row_grid4(n), dim3(256), 0, s, H, w.A, n, (const float*)w.lam);
  else hipLaunchKernelGGL(reverse_damp_kernel, row_grid(n), dim3(256), 0, s, H, w.A, n, (const float*)w.lam);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;

  // Blocked Cholesky of A (lower), two levels while the trailing matrix is
  // large: panels of PB block columns of NB.  Inside a panel, block column k
  // is applied (right-looking) only to the panel's later columns while
  // workgroup 0 factors block k + 1; at the panel's end one rank-PB*NB update
  // reads the panel back from L.  Its part on the next panel's columns runs
  // in the launch that factors the next panel's first block; the rest of it
  // is dealt out over the next panel's launches, where it fills the CUs the
  // serial diagonal blocks leave idle (it touches neither that panel's
  // columns nor its diagonal blocks).  So the trailing matrix moves through
  // memory once per PB*NB columns instead of once per NB.  Once fewer than
  // TWO_LEVEL_MIN columns would remain after a panel, the last panel runs to
  // the end: one launch per block column updating the whole trailing matrix,
  // where a launch is bound by the diagonal block's factorization rather
  // than by memory and a rank-256 tile (at least 14 us of MFMA on one CU)
  // would only lengthen it.  The factor's off-diagonal blocks go to L, the
  // inverses of its diagonal blocks to dinv.
  hipLaunchKernelGGL(chol_first_kernel, dim3(1), dim3(256), 0, s, (const float*)w.A, n, w.dinv, info);
  {
    const int64_t nb = cdiv(n, NB);
    const bool vec = n % 4 == 0;
    auto lower_tiles = [](int64_t nr, int64_t nc) { return nc * nr - nc * (nc - 1) / 2; };  // nc <= nr
    auto panel_end = [&](int64_t b0) {
      const int64_t b1 = std::min(b0 + PB, nb);
      return n - b1 * NB < TWO_LEVEL_MIN ? nb : b1;
    };
    auto launch = [&](const StepArgs& a, int64_t grid) {
      if (vec) hipLaunchKernelGGL((chol_step_kernel<true>), dim3((unsigned)grid), dim3(256), 0, s, a);
      else hipLaunchKernelGGL((chol_step_kernel<false>), dim3((unsigned)grid), dim3(256), 0, s, a);
    };
    StepArgs base{};
    base.A = w.A; base.L = w.L; base.dinv = w.dinv; base.info = info; base.n = n;
    // Workgroups of the launch for block column k of the panel ending at b1
    // besides its share of the previous panel's far update: strip tiles
    // (k + 1 < b1) or slab solves (the panel's last column).
    auto own_tiles = [&](int64_t k, int64_t b1, int64_t& nstrip, int64_t& nsolve) {
      nstrip = nsolve = 0;
      if (k + 1 < b1) {
        const int64_t send = std::min(b1 * NB, n);
        nstrip = lower_tiles(cdiv(n - (k + 1) * NB, TB), cdiv(send - (k + 1) * NB, TB));
      } else {
        nsolve = cdiv(n - (k + 1) * NB, TB);
      }
    };
    // The far update's tiles are dealt over the panel's launches so that
    // every launch but the last fills whole rounds of one tile per CU (two
    // share a CU at half speed each): an even split leaves each launch with a
    // partly filled last round.  Counted in far-tile times: a strip tile
    // (rank 64 with its slab solves) about 2/3, a slab solve 1/4, the
    // diagonal block one.
    const int64_t cus = device_cus();
    int64_t far_cut[PB + 1] = {};
    auto deal_far = [&](int64_t p0, int64_t p1, int64_t F) {
      const int64_t m = p1 - p0;
      int64_t own[PB];
      int64_t total = 3 * F;  // in thirds of a far tile
      for (int64_t i = 0; i < m; ++i) {
        int64_t ns, nv;
        own_tiles(p0 + i, p1, ns, nv);
        own[i] = 3 + 2 * ns + cdiv(3 * nv, 4);
        total += own[i];
      }
      const int64_t rounds = cdiv(total, 3 * cus);
      far_cut[0] = 0;
      for (int64_t i = 0; i < m; ++i) {
        const int64_t h = rounds / m + (i < rounds % m ? 1 : 0);
        const int64_t f = i + 1 < m ? std::max<int64_t>(0, (3 * cus * h - own[i]) / 3) : F;
        far_cut[i + 1] = std::min(F, far_cut[i] + f);
      }
    };
    int64_t far_R0 = 0, far_k0 = 0, far_tiles = 0;  // the previous panel's update past this panel
    for (int64_t b0 = 0; b0 < nb;) {
      const int64_t b1 = panel_end(b0), np = b1 - b0;
      for (int64_t k = b0; k < b1 && k + 1 < nb; ++k) {
        StepArgs a = base;
        a.sk0 = k * NB;
        if (k + 1 < b1) {
          a.leaf_mode = 1; a.leaf_j0 = (k + 1) * NB; a.leaf_kp = k * NB;
          a.send = std::min(b1 * NB, n);
          const int64_t nr = cdiv(n - (k + 1) * NB, TB), nc = cdiv(a.send - (k + 1) * NB, TB);
          a.s_nr = (int)nr; a.nstrip = (int)lower_tiles(nr, nc);
        } else {
          a.nsolve = (int)cdiv(n - (k + 1) * NB, TB);
        }
        if (far_tiles > 0) {
          a.lk0 = far_k0; a.lnk = PB; a.lR0 = far_R0; a.lcend = n; a.l_nr = (int)cdiv(n - far_R0, TB);
          a.lt0 = (int)far_cut[k - b0]; a.lt1 = (int)far_cut[k - b0 + 1];
        }
        launch(a, 1 + (int64_t)a.nstrip + a.nsolve + (a.lt1 - a.lt0));
      }
      far_tiles = 0;
      if (b1 < nb) {  // the panel's update: block b1 factored, the next panel's columns updated
        const int64_t nb1 = panel_end(b1);
        StepArgs a = base;
        a.leaf_mode = 2; a.leaf_j0 = b1 * NB; a.leaf_kp = b0 * NB; a.leaf_nk = (int)np;
        a.lk0 = b0 * NB; a.lnk = (int)np; a.lR0 = b1 * NB; a.lcend = std::min(nb1 * NB, n); a.lskip00 = 1;
        const int64_t nr = cdiv(n - a.lR0, TB), nc = cdiv(a.lcend - a.lR0, TB);
        a.l_nr = (int)nr; a.lt0 = 0; a.lt1 = (int)lower_tiles(nr, nc);
        launch(a, 1 + (int64_t)a.lt1);
        if (nb1 < nb) {
          far_R0 = nb1 * NB; far_k0 = b0 * NB;
          const int64_t nt = cdiv(n - far_R0, TB);
          far_tiles = lower_tiles(nt, nt);
          deal_far(b1, nb1, far_tiles);
        }
      }
      b0 = b1;
    }
  }
  if ((e = hipGetLastError()) != hipSuccess) return e;

  // triangular inverse of the factor, in place, by recursive doubling
  if (v4) hipLaunchKernelGGL(trtri_init4_kernel, row_grid4(n), dim3(256), 0, s, w.L, n, (const float*)w.dinv, (const int32_t*)info);
  else hipLaunchKernelGGL(trtri_init_kernel, row_grid(n), dim3(256), 0, s, w.L, n, (const float*)w.dinv, (const int32_t*)info);
  for (int64_t bs = NB; bs < n; bs *= 2) {
    const int64_t full = n / (2 * bs);  // pairs of two complete bs-blocks
    const int64_t a_part = full * 2 * bs;
    const int64_t s2_part = n - a_part - bs;  // > 0: a trailing pair with a short second block
    for (int pass = 0; pass < 2; ++pass) {
      const int64_t count = pass == 0 ? full : (s2_part > 0 ? 1 : 0);
      if (count == 0) continue;
      const int64_t a = pass == 0 ? 0 : a_part;
      const int64_t s2 = pass == 0 ? bs : s2_part;
      const int64_t stride = 2 * bs * n + 2 * bs;
      GemmDesc g1{};  // tmp = L21 * Linv11
      g1.A = w.L + (a + bs) * n + a; g1.lda = n; g1.strideA = stride;
      g1.B = w.L + a * n + a; g1.ldb = n; g1.strideB = stride;
      g1.C = w.A; g1.ldc = bs; g1.strideC = bs * bs;
      g1.M = (int)s2; g1.N = (int)bs; g1.K = (int)bs; g1.batch = (int)count;
      g1.alpha = 1.f; g1.beta = 0.f; g1.flags = GEMM_B_LOWER | GEMM_SMALL_TILES; g1.info = info;
      // split-K scratch: the rest of A past the product buffer (at least n^2/2 floats)
      const int64_t tmp_floats = (count * bs * bs + 63) / 64 * 64;
      g1.ws = w.A + tmp_floats; g1.ws_floats = n * n - tmp_floats;
      if ((e = gemm_f32(g1, false, false, s)) != hipSuccess) return e;
      GemmDesc g2{};  // Linv21 = -Linv22 * tmp
      g2.A = w.L + (a + bs) * n + (a + bs); g2.lda = n; g2.strideA = stride;
      g2.B = w.A; g2.ldb = bs; g2.strideB = bs * bs;
      g2.C = w.L + (a + bs) * n + a; g2.ldc = n; g2.strideC = stride;
      g2.M = (int)s2; g2.N = (int)bs; g2.K = (int)s2; g2.batch = (int)count;
      g2.alpha = -1.f; g2.beta = 0.f; g2.flags = GEMM_A_LOWER | GEMM_SMALL_TILES; g2.info = info;
      g2.ws = g1.ws; g2.ws_floats = g1.ws_floats;
      if ((e = gemm_f32(g2, false, false, s)) != hipSuccess) return e;
    }
  }
  if (v4) hipLaunchKernelGGL(write_u4_kernel, row_grid4(n), dim3(256), 0, s, (const float*)w.L, U, n, (const int32_t*)info);
  else hipLaunchKernelGGL(write_u_kernel, row_grid(n), dim3(256), 0, s, (const float*)w.L, U, n, (const int32_t*)info);
  return hipGetLastError();
}

}  // namespace gptq
