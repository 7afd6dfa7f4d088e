// The sweep's lazy trailing updates, V[:, c0:c0+N] -= E U[r0:r0+K, c0:c0+N],
// as three bf16 products on the 16-bit matrix cores with fp32 accumulation.
//
// "Part 3: Adaptive Rounding: GPTQ", 'Observation 2: Lazy Batch Updates' and
// 'Algorithm GPTQ': after a batch of columns is swept, its errors are applied
// to every later column with one matrix product (the Vietnamese edition of
// the English GPTQ second-order quantization post, 'Lazy batch update',
// writes it W[:, B:] <- W[:, B:] - E R[B, B:]).
//
// Precision: each fp32 operand x is split into x_hi = bf16(x) and
// x_lo = bf16(x - x_hi) (x - x_hi is exact in fp32), and
//   E U ~ E_hi U_hi + E_hi U_lo + E_lo U_hi,
// every product accumulated in fp32: each term keeps about 16 bits of its
// operands (the dropped E_lo U_lo and the rounding of the lo parts are about
// 2^-16 of the term).  E's rows hold [E_hi | E_lo] (written so by the
// sweep kernels); U is split and transposed once per layer into
// Ut = [U_hi | U_lo]^T, so that both operands are contiguous along K, and
// every flush reads its factor rows from there.  Each K stage loads the four
// panels once and runs the three products on them.
#include "common.hpp"
#include "internal.hpp"

namespace gptq {

namespace {

constexpr int XT = 128;         // output tile (rows and columns)
constexpr int XK = 64;          // K per stage (bf16)
constexpr int XP = XK + 8;      // LDS pitch of a stage row (bf16): 144 bytes
constexpr int TT = 64;          // transpose tile
constexpr int NXCD = 8;         // MI355X: 8 XCDs, workgroups dealt round-robin
constexpr int GB = 8;           // tile rows per band of the tile order

// Ut[j][k], Ut[j][n + k] = hi, lo of U[k][j] (rows of ldu bf16): 64 x 64
// tiles through LDS, read along U's rows, written along Ut's rows.  A flush
// reads only entries whose row k lies in an earlier granule (of gran
// columns: the flushes' factor rows end at a granule boundary at or before
// their first column), so every other tile is skipped.
__global__ __launch_bounds__(256) void split_t_kernel(const float* U, int64_t n, uint16_t* Ut, int64_t ldu,
                                                      int64_t gran) {
  __shared__ float t[TT][TT + 1];
  const int64_t j0 = (int64_t)blockIdx.x * TT, k0 = (int64_t)blockIdx.y * TT;
  if (k0 / gran >= j0 / gran) return;
  const int tid = threadIdx.x;
  for (int e = tid; e < TT * TT; e += 256) {
    const int i = e / TT, jj = e % TT;  // row k0 + i of U, column j0 + jj
    t[i][jj] = (k0 + i < n && j0 + jj < n) ? U[(k0 + i) * n + j0 + jj] : 0.f;
  }
  __syncthreads();
  // four consecutive k per thread, 8-byte stores (n is a multiple of 4, so a
  // run of four is inside or outside the matrix as a whole)
  for (int e = tid; e < TT * TT / 4; e += 256) {
    const int jj = e / (TT / 4), i = 4 * (e % (TT / 4));
    if (k0 + i < n && j0 + jj < n) {
      uint32_t hi[4], lo[4];
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const float u = t[i + r][jj];
        const uint16_t h = f32_to_bf16(u);
        hi[r] = h;
        lo[r] = f32_to_bf16(u - bf16_to_f32(h));
      }
      uint16_t* row = Ut + (j0 + jj) * ldu + k0 + i;
      *(uint2*)row = make_uint2(hi[0] | (hi[1] << 16), hi[2] | (hi[3] << 16));
      *(uint2*)(row + n) = make_uint2(lo[0] | (lo[1] << 16), lo[2] | (lo[3] << 16));
    }
  }
}

// C[M x N] (fp32, leading dimension ldc) -= A_hi Bt_hi^T + A_hi Bt_lo^T +
// A_lo Bt_hi^T over K (a multiple of XK), all operands bf16 and contiguous
// along K: row r of A_hi at A + r lda, of A_lo alo elements further; row j of
// Bt_hi at Bt + j ldb, of Bt_lo blo elements further.
// 128 x 128 tiles, four waves of 64 x 64 on v_mfma_f32_32x32x16_bf16 (lane l
// supplies row / column l % 32 and k = 8 (l / 32) .. + 7 of a 16-deep step;
// accumulator r of lane l is row 8 (r / 4) + 4 (l / 32) + r % 4, column
// l % 32).  A stage of 64 k holds the four panels (72 KiB of LDS, two
// workgroups per CU); the next stage's panels are loaded into registers while
// the current one is multiplied, then stored between two barriers, and C's
// tile is loaded while the last stage is multiplied.  Rows past M or N load
// the last valid row (never stored).
__global__ __launch_bounds__(256, 2) void gemm_x3_kernel(const uint16_t* __restrict__ A, int64_t lda, int64_t alo,
                                                         int K, const uint16_t* __restrict__ Bt, int64_t ldb,
                                                         int64_t blo, float* __restrict__ C, int64_t ldc, int M,
                                                         int N) {
  __shared__ __attribute__((aligned(16))) uint16_t lds[4][XT * XP];  // A_hi, A_lo, Bt_hi, Bt_lo
  const int tN = (N + XT - 1) / XT, tM = (M + XT - 1) / XT;
  // Tile order: XCD x (workgroup x mod 8) takes tiles [x P, (x + 1) P) of an
  // order that walks bands of GB tile rows column by column, so the
  // workgroups resident on one XCD share a few row panels of A and column
  // panels of Bt in its L2 instead of streaming all of Bt per tile row.
  const int T = tM * tN, P = (T + NXCD - 1) / NXCD;
  const int t = (blockIdx.x % NXCD) * P + blockIdx.x / NXCD;
  if (t >= T) return;  // the grid is NXCD * P workgroups
  const int band = t / (GB * tN), rows = min(GB, tM - band * GB), within = t - band * GB * tN;
  const int tm = band * GB + within % rows, tn = within / rows;
  const int r0 = tm * XT, c0 = tn * XT;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wr = wave >> 1, wc = wave & 1;

  // loader: chunk q = tid + 256 e (e < 4) of each panel's stage is row q / 8,
  // 16-byte piece q % 8 of that row's 64 k
  const uint16_t* pa[4];
  const uint16_t* pb[4];
  int lo_[4];
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    const int q = tid + 256 * e, row = q >> 3, c8 = q & 7;
    pa[e] = A + (int64_t)min(r0 + row, M - 1) * lda + 8 * c8;
    pb[e] = Bt + (int64_t)min(c0 + row, N - 1) * ldb + 8 * c8;
    lo_[e] = row * XP + 8 * c8;
  }
  u32x4 rah[4], ral[4], rbh[4], rbl[4];
  auto gload = [&](int k0) {
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      rah[e] = *(const u32x4*)(pa[e] + k0);
      ral[e] = *(const u32x4*)(pa[e] + alo + k0);
      rbh[e] = *(const u32x4*)(pb[e] + k0);
      rbl[e] = *(const u32x4*)(pb[e] + blo + k0);
    }
  };
  auto lstore = [&]() {
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      *(u32x4*)(&lds[0][lo_[e]]) = rah[e];
      *(u32x4*)(&lds[1][lo_[e]]) = ral[e];
      *(u32x4*)(&lds[2][lo_[e]]) = rbh[e];
      *(u32x4*)(&lds[3][lo_[e]]) = rbl[e];
    }
  };

  f32x16 acc[2][2];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j) acc[i][j] = zero16();

  const int arow = (wr * 64 + (lane & 31)) * XP, brow = (wc * 64 + (lane & 31)) * XP;
  auto stage = [&]() {
#pragma unroll
    for (int ks = 0; ks < XK / 16; ++ks) {
      const int kk = 16 * ks + 8 * (lane >> 5);
      bf16x8 ah[2], al[2], bh[2], bl[2];
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        ah[h] = __builtin_bit_cast(bf16x8, *(const u32x4*)(&lds[0][arow + 32 * h * XP + kk]));
        al[h] = __builtin_bit_cast(bf16x8, *(const u32x4*)(&lds[1][arow + 32 * h * XP + kk]));
        bh[h] = __builtin_bit_cast(bf16x8, *(const u32x4*)(&lds[2][brow + 32 * h * XP + kk]));
        bl[h] = __builtin_bit_cast(bf16x8, *(const u32x4*)(&lds[3][brow + 32 * h * XP + kk]));
      }
      // four independent accumulators between two products into the same one
#pragma unroll
      for (int mb = 0; mb < 2; ++mb)
#pragma unroll
        for (int nb = 0; nb < 2; ++nb)
          acc[mb][nb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ah[mb], bh[nb], acc[mb][nb], 0, 0, 0);
#pragma unroll
      for (int mb = 0; mb < 2; ++mb)
#pragma unroll
        for (int nb = 0; nb < 2; ++nb)
          acc[mb][nb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ah[mb], bl[nb], acc[mb][nb], 0, 0, 0);
#pragma unroll
      for (int mb = 0; mb < 2; ++mb)
#pragma unroll
        for (int nb = 0; nb < 2; ++nb)
          acc[mb][nb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(al[mb], bh[nb], acc[mb][nb], 0, 0, 0);
    }
  };

  gload(0);
  lstore();
  __syncthreads();
  for (int k0 = XK; k0 < K; k0 += XK) {
    gload(k0);
    stage();
    __syncthreads();  // every wave is done with this stage
    lstore();
    __syncthreads();  // the next stage is visible
  }
  // the last stage, with this lane's part of C (rows and columns past M or N
  // read the last valid one, never stored) loaded ahead of its products, in
  // the registers the stage loads no longer need
  float cv[2][2][16];
#pragma unroll
  for (int mb = 0; mb < 2; ++mb)
#pragma unroll
    for (int nb = 0; nb < 2; ++nb) {
      const float* colp = C + min(c0 + wc * 64 + nb * 32 + mfma32_col(lane), N - 1);
#pragma unroll
      for (int r = 0; r < 16; ++r)
        cv[mb][nb][r] = colp[(int64_t)min(r0 + wr * 64 + mb * 32 + mfma32_row(r, lane), M - 1) * ldc];
    }
  __builtin_amdgcn_sched_barrier(0);  // every load issued before the stage's products
  stage();

#pragma unroll
  for (int mb = 0; mb < 2; ++mb)
#pragma unroll
    for (int nb = 0; nb < 2; ++nb)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int row = r0 + wr * 64 + mb * 32 + mfma32_row(r, lane);
        const int col = c0 + wc * 64 + nb * 32 + mfma32_col(lane);
        if (row < M && col < N) C[(int64_t)row * ldc + col] = cv[mb][nb][r] - acc[mb][nb][r];
      }
}

}  // namespace

// Ut (n rows of 2n bf16) = [U_hi | U_lo]^T of the n x n factor U, the part
// above the diagonal blocks of gran columns (a multiple of 64) that the
// flushes read; n a multiple of 4.
hipError_t split_ut_x3(const float* U, int64_t n, uint16_t* Ut, int64_t gran, hipStream_t s) {
  if (n <= 0) return hipSuccess;
  if (n % 4 != 0 || gran <= 0 || gran % TT != 0 || (((uintptr_t)Ut) & 15) != 0 || cdiv(n, TT) > INT32_MAX)
    return hipErrorInvalidValue;
  hipLaunchKernelGGL(split_t_kernel, dim3((unsigned)cdiv(n, TT), (unsigned)cdiv(n, TT)), dim3(256), 0, s, U, n, Ut,
                     2 * n, gran);
  return hipGetLastError();
}

// V[:, c0:c0+N] -= E U[r0:r0+K, c0:c0+N] for m rows (V leading dimension n)
// as three bf16 products: row r of E holds E_hi at Ecat + r lde and E_lo alo
// elements further; the factor comes split from split_ut_x3 (row j of Ut:
// hi of U[:, j] at Ut + 2n j, lo n elements further), and the flush reads
// only its rows [r0, r0 + K), which must end at a boundary of that split's
// granules at or before its first column c0.  K and r0 must be multiples
// of 64.
hipError_t flush_x3(const uint16_t* Ecat, int64_t lde, int64_t alo, const uint16_t* Ut, int64_t n, int64_t r0,
                    int K, int64_t c0, int64_t N, float* V, int64_t m, hipStream_t s) {
  if (N <= 0 || m <= 0 || K <= 0) return hipSuccess;
  if (K % XK != 0 || r0 % XK != 0 || alo < K || lde < alo + K || (lde % 8) != 0 || (alo % 8) != 0 || n % 4 != 0 ||
      (((uintptr_t)Ecat) & 15) != 0 || (((uintptr_t)Ut) & 15) != 0 || m > INT32_MAX || N > INT32_MAX ||
      c0 + N > n || r0 + K > c0)
    return hipErrorInvalidValue;
  const int64_t ldu = 2 * n;
  const int64_t tiles = cdiv(m, XT) * cdiv(N, XT);
  hipLaunchKernelGGL(gemm_x3_kernel, dim3((unsigned)(NXCD * cdiv(tiles, NXCD))), dim3(256), 0, s, Ecat, lde, alo, K,
                     Ut + c0 * ldu + r0, ldu, n, V + c0, n, (int)m, (int)N);
  return hipGetLastError();
}

}  // namespace gptq
