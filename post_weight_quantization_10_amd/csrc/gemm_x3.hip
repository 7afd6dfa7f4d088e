// The trailing update past a superblock, V[:, c0:] -= E U[r0:r0+K, c0:], as
// three bf16 products on the 16-bit matrix cores with fp32 accumulation.
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
// 2^-16 of the term).  The three products are one bf16 product with
// K' = 3K over the concatenations A = [E_hi | E_hi | E_lo] (rows of E,
// written so by the superblock sweep kernel) and Bt = [U_hi | U_lo | U_hi]^T
// (columns of U's rows r0.., transposed here so that both operands are
// contiguous along K).
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

// Bt[j][k], Bt[j][K + k], Bt[j][2K + k] = hi, lo, hi of U[r0 + k][c0 + j]
// for j < N, k < K (leading dimension ldb): 64 x 64 tiles through LDS, read
// along U's rows, written along Bt's rows.
__global__ __launch_bounds__(256) void split_t_kernel(const float* U, int64_t n, int64_t r0, int K, int64_t c0, int N,
                                                      uint16_t* Bt, int64_t ldb) {
  __shared__ float t[TT][TT + 1];
  const int j0 = blockIdx.x * TT, k0 = blockIdx.y * TT;
  const int tid = threadIdx.x;
  for (int e = tid; e < TT * TT; e += 256) {
    const int i = e / TT, jj = e % TT;  // row k0 + i of the slice, column j0 + jj
    t[i][jj] = (k0 + i < K && j0 + jj < N) ? U[(r0 + k0 + i) * n + c0 + j0 + jj] : 0.f;
  }
  __syncthreads();
  for (int e = tid; e < TT * TT; e += 256) {
    const int jj = e / TT, i = e % TT;
    if (k0 + i < K && j0 + jj < N) {
      const float u = t[i][jj];
      const uint16_t hi = f32_to_bf16(u);
      const uint16_t lo = f32_to_bf16(u - bf16_to_f32(hi));
      uint16_t* row = Bt + (int64_t)(j0 + jj) * ldb + k0 + i;
      row[0] = hi;
      row[K] = lo;
      row[2 * K] = hi;
    }
  }
}

// C[M x N] (fp32, leading dimension ldc) -= A[M x K3] Bt[N x K3]^T, both bf16
// and contiguous along K (leading dimensions lda, ldb), K3 = 3 K with K a
// multiple of XK.  A's three K-segments (hi, hi, lo) start aseg elements
// apart in each row, so a stage never straddles two of them.
// 128 x 128 tiles, four waves of 64 x 64 on v_mfma_f32_32x32x16_bf16 (lane l
// supplies row / column l % 32 and k = 8 (l / 32) .. + 7 of a 16-deep step;
// accumulator r of lane l is row 8 (r / 4) + 4 (l / 32) + r % 4, column
// l % 32).  Stages of 64 k move global -> registers -> LDS, double buffered;
// rows past M or N load the last valid row (never stored).
__global__ __launch_bounds__(256, 2) void gemm_x3_kernel(const uint16_t* __restrict__ A, int64_t lda, int64_t aseg,
                                                         int K, const uint16_t* __restrict__ Bt, int64_t ldb,
                                                         float* __restrict__ C, int64_t ldc, int M, int N) {
  const int K3 = 3 * K;
  __shared__ __attribute__((aligned(16))) uint16_t lds[2][2][XT * XP];
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

  // loader: chunk q = tid + 256 e (e < 4) of each operand's stage is row
  // q / 8, 16-byte piece q % 8 of that row's 64 k
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
  u32x4 ra[4], rb[4];
  auto gload = [&](int k0) {
    const int seg = k0 / K;
    const int64_t ak = seg * aseg + (k0 - seg * K);
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      ra[e] = *(const u32x4*)(pa[e] + ak);
      rb[e] = *(const u32x4*)(pb[e] + k0);
    }
  };
  auto lstore = [&](int buf) {
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      *(u32x4*)(&lds[buf][0][lo_[e]]) = ra[e];
      *(u32x4*)(&lds[buf][1][lo_[e]]) = rb[e];
    }
  };

  f32x16 acc[2][2];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j) acc[i][j] = zero16();

  gload(0);
  lstore(0);
  __syncthreads();
  int buf = 0;
  for (int k0 = 0; k0 < K3; k0 += XK) {
    const bool more = k0 + XK < K3;
    if (more) gload(k0 + XK);
    const uint16_t* Ta = lds[buf][0];
    const uint16_t* Tb = lds[buf][1];
#pragma unroll
    for (int ks = 0; ks < XK / 16; ++ks) {
      const int kk = 16 * ks + 8 * (lane >> 5);
      u32x4 av[2], bv[2];
#pragma unroll
      for (int mb = 0; mb < 2; ++mb) av[mb] = *(const u32x4*)(Ta + (wr * 64 + mb * 32 + (lane & 31)) * XP + kk);
#pragma unroll
      for (int nb = 0; nb < 2; ++nb) bv[nb] = *(const u32x4*)(Tb + (wc * 64 + nb * 32 + (lane & 31)) * XP + kk);
#pragma unroll
      for (int mb = 0; mb < 2; ++mb)
#pragma unroll
        for (int nb = 0; nb < 2; ++nb)
          acc[mb][nb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, av[mb]),
                                                               __builtin_bit_cast(bf16x8, bv[nb]), acc[mb][nb], 0, 0, 0);
    }
    if (more) lstore(buf ^ 1);
    __syncthreads();
    buf ^= 1;
  }

#pragma unroll
  for (int mb = 0; mb < 2; ++mb)
#pragma unroll
    for (int nb = 0; nb < 2; ++nb)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int row = r0 + wr * 64 + mb * 32 + mfma32_row(r, lane);
        const int col = c0 + wc * 64 + nb * 32 + mfma32_col(lane);
        if (row < M && col < N) C[(int64_t)row * ldc + col] -= acc[mb][nb][r];
      }
}

}  // namespace

// V[:, c0:c0+N] -= E_cat U_cat for m rows (V leading dimension n): E_cat's
// row r holds E_hi, E_hi, E_lo of the K errors at Ecat + r lde, + aseg,
// + 2 aseg; U_cat is the hi / lo / hi split of U's rows [r0, r0 + K),
// columns [c0, c0 + N), written transposed to the scratch Bt (N x ldb bf16,
// ldb >= 3K).  K must be a multiple of 64.
hipError_t flush_x3(const uint16_t* Ecat, int64_t lde, int64_t aseg, const float* U, int64_t n, int64_t r0, int K,
                    int64_t c0, int64_t N, float* V, int64_t m, uint16_t* Bt, int64_t ldb, hipStream_t s) {
  if (N <= 0 || m <= 0 || K <= 0) return hipSuccess;
  if (K % XK != 0 || aseg < K || lde < 2 * aseg + K || ldb < 3 * (int64_t)K || (lde % 8) != 0 || (aseg % 8) != 0 ||
      (ldb % 8) != 0 || (((uintptr_t)Ecat) & 15) != 0 || (((uintptr_t)Bt) & 15) != 0 || m > INT32_MAX ||
      N > INT32_MAX || c0 + N > n || r0 + K > n)
    return hipErrorInvalidValue;
  hipLaunchKernelGGL(split_t_kernel, dim3((unsigned)cdiv(N, TT), (unsigned)cdiv(K, TT)), dim3(256), 0, s, U, n, r0, K,
                     c0, (int)N, Bt, ldb);
  const int64_t tiles = cdiv(m, XT) * cdiv(N, XT);
  hipLaunchKernelGGL(gemm_x3_kernel, dim3((unsigned)(NXCD * cdiv(tiles, NXCD))), dim3(256), 0, s, Ecat, lde, aseg, K,
                     (const uint16_t*)Bt, ldb, V + c0, n, (int)m, (int)N);
  return hipGetLastError();
}

}  // namespace gptq
