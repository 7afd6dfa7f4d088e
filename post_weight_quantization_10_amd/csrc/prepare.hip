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
//   2. blocked right-looking Cholesky of A, panels of NB = 64:
//        leaf kernel: one workgroup factors the NB x NB diagonal block and
//        inverts it in the same pass (registers + LDS broadcasts);
//        panel solve  A21 <- A21 L11^{-T}  (MFMA GEMM with the leaf inverse)
//        trailing     A22 <- A22 - A21 A21^T  (MFMA GEMM, lower tiles only)
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

// Factor the kb x kb diagonal block at (k0, k0) of A in place (lower) and
// write its inverse to Dinv (NB x NB, zero above the diagonal), in one pass.
//
// Thread (ty, tx) of a 16 x 16 grid keeps a 4 x 4 tile (rows 4ty.., columns
// 4tx..) of the block being factored (Am) and of the running inverse (Tm) in
// registers.  Step j, right-looking: d = A[j][j]; column j of L is
// A[r][j]/sqrt(d); row j of L^{-1} is R[j][:]/sqrt(d); then
//   A[r][c] -= L[r][j] L[c][j]        (r, c > j)
//   R[r][c] -= L[r][j] Linv[j][c]     (r > j, c <= j)
// with R = I initially (so that R[r][:] becomes row r of L^{-1} times L[r][r]).
// The raw column j+1 of A and row j+1 of R are published to double-buffered
// LDS by their owners, so each step needs one barrier.  Rows/columns past kb
// are padded with the identity, which factors trivially.
__global__ __launch_bounds__(256) void chol_leaf_kernel(float* A, int64_t lda, int64_t k0, int kb, float* Dinv,
                                                        int32_t* info, int64_t n) {
  if (*info != 0) return;
  __shared__ __attribute__((aligned(16))) float colbuf[2][NB];
  __shared__ __attribute__((aligned(16))) float rowbuf[2][NB];
  const int tid = threadIdx.x;
  const int ty = tid >> 4, tx = tid & 15;
  float Am[4][4], Tm[4][4];
#pragma unroll
  for (int a = 0; a < 4; ++a)
#pragma unroll
    for (int b = 0; b < 4; ++b) {
      const int r = 4 * ty + a, c = 4 * tx + b;
      float v = 0.f;
      if (r < kb && c < kb) { if (c <= r) v = A[(k0 + r) * lda + k0 + c]; }
      else if (r == c) v = 1.f;
      Am[a][b] = v;
      Tm[a][b] = (r == c) ? 1.f : 0.f;
    }
  if (tx == 0)
#pragma unroll
    for (int a = 0; a < 4; ++a) colbuf[0][4 * ty + a] = Am[a][0];
  if (ty == 0)
#pragma unroll
    for (int b = 0; b < 4; ++b) rowbuf[0][4 * tx + b] = Tm[0][b];
  __syncthreads();

  for (int jb = 0; jb < NB / 4; ++jb) {
#pragma unroll
    for (int jj = 0; jj < 4; ++jj) {
      const int j = 4 * jb + jj;
      const float* cb = colbuf[j & 1];
      const float* rb = rowbuf[j & 1];
      const float d = cb[j];
      if (!(d > 0.f) || !(d < INFINITY)) {  // uniform: every thread read the same d
        if (tid == 0) atomicCAS(info, 0, (int32_t)(n - (k0 + j)));
        return;
      }
      const float rs = __builtin_amdgcn_rsqf(d);
      const float sd = d * rs;
      const f32x4 cr = *(const f32x4*)&cb[4 * ty];
      const f32x4 cc = *(const f32x4*)&cb[4 * tx];
      const f32x4 rr = *(const f32x4*)&rb[4 * tx];
      float lr[4], lc[4], tc[4];
#pragma unroll
      for (int a = 0; a < 4; ++a) lr[a] = (4 * ty + a > j) ? cr[a] * rs : 0.f;
#pragma unroll
      for (int b = 0; b < 4; ++b) {
        lc[b] = (4 * tx + b > j) ? cc[b] * rs : 0.f;
        tc[b] = (4 * tx + b <= j) ? rr[b] * rs : 0.f;
      }
      if (4 * ty + 3 > j) {
#pragma unroll
        for (int a = 0; a < 4; ++a)
#pragma unroll
          for (int b = 0; b < 4; ++b) {
            Am[a][b] = fmaf(-lr[a], lc[b], Am[a][b]);
            Tm[a][b] = fmaf(-lr[a], tc[b], Tm[a][b]);
          }
      }
      if (tx == jb) {  // column j of L
#pragma unroll
        for (int a = 0; a < 4; ++a) {
          const int r = 4 * ty + a;
          Am[a][jj] = (r > j) ? lr[a] : (r == j ? sd : Am[a][jj]);
        }
      }
      if (ty == jb) {  // row j of L^{-1}
#pragma unroll
        for (int b = 0; b < 4; ++b) Tm[jj][b] = tc[b];
      }
      if (j + 1 < NB) {
        const int jn = j + 1, jnb = jn >> 2, jnj = (jj + 1) & 3;
        if (tx == jnb)
#pragma unroll
          for (int a = 0; a < 4; ++a) colbuf[jn & 1][4 * ty + a] = Am[a][jnj];
        if (ty == jnb)
#pragma unroll
          for (int b = 0; b < 4; ++b) rowbuf[jn & 1][4 * tx + b] = Tm[jnj][b];
      }
      __syncthreads();
    }
  }
#pragma unroll
  for (int a = 0; a < 4; ++a)
#pragma unroll
    for (int b = 0; b < 4; ++b) {
      const int r = 4 * ty + a, c = 4 * tx + b;
      if (r < kb && c <= r) A[(k0 + r) * lda + k0 + c] = Am[a][b];
      Dinv[r * NB + c] = (r < kb && c <= r) ? Tm[a][b] : 0.f;
    }
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
  float* A;
  float* tmp;
  float* dinv;
  float* lam;
};

PrepWs carve(void* ws, int64_t n) {
  char* p = (char*)ws;
  PrepWs w;
  w.A = (float*)p;
  p += align256((size_t)n * n * 4);
  w.tmp = (float*)p;
  p += align256((size_t)n * ((n + 1) / 2) * 4);
  w.dinv = (float*)p;
  p += align256((size_t)cdiv(n, NB) * NB * NB * 4);
  w.lam = (float*)p;
  return w;
}

dim3 row_grid(int64_t n) { return dim3((unsigned)std::min<int64_t>(cdiv(n, 256), 64), (unsigned)n); }

}  // namespace

size_t prepare_workspace_bytes(int64_t n) {
  if (n < 1) return 0;
  return align256((size_t)n * n * 4) + align256((size_t)n * ((n + 1) / 2) * 4) +
         align256((size_t)cdiv(n, NB) * NB * NB * 4) + 256;
}

hipError_t prepare_hinv(const float* H, int64_t n, float damp, float* U, int32_t* info, float* lambda_out, void* ws,
                        hipStream_t s) {
  PrepWs w = carve(ws, n);
  hipLaunchKernelGGL(damp_mean_kernel, dim3(1), dim3(1024), 0, s, H, n, damp, w.lam, lambda_out, info);
  hipLaunchKernelGGL(reverse_damp_kernel, row_grid(n), dim3(256), 0, s, H, w.A, n, (const float*)w.lam);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;

  // blocked right-looking Cholesky of A (lower)
  for (int64_t k0 = 0; k0 < n; k0 += NB) {
    const int kb = (int)std::min<int64_t>(NB, n - k0);
    float* dblk = w.dinv + (k0 / NB) * NB * NB;
    hipLaunchKernelGGL(chol_leaf_kernel, dim3(1), dim3(256), 0, s, w.A, n, k0, kb, dblk, info, n);
    const int64_t rest = n - k0 - kb;
    if (rest > 0) {
      float* P = w.A + (k0 + kb) * n + k0;
      GemmDesc g{};
      g.A = P; g.lda = n;
      g.B = dblk; g.ldb = NB;
      g.C = P; g.ldc = n;
      g.M = (int)rest; g.N = kb; g.K = kb; g.batch = 1;
      g.alpha = 1.f; g.beta = 0.f; g.info = info;
      if ((e = gemm_f32(g, false, true, s)) != hipSuccess) return e;
      GemmDesc t{};
      t.A = P; t.lda = n;
      t.B = P; t.ldb = n;
      t.C = w.A + (k0 + kb) * n + (k0 + kb); t.ldc = n;
      t.M = (int)rest; t.N = (int)rest; t.K = kb; t.batch = 1;
      t.alpha = -1.f; t.beta = 1.f; t.flags = GEMM_LOWER_TILES; t.info = info;
      if ((e = gemm_f32(t, false, true, s)) != hipSuccess) return e;
    }
    if ((e = hipGetLastError()) != hipSuccess) return e;
  }

  // triangular inverse of the factor, in place, by recursive doubling
  hipLaunchKernelGGL(trtri_init_kernel, row_grid(n), dim3(256), 0, s, w.A, n, (const float*)w.dinv, (const int32_t*)info);
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
      g1.A = w.A + (a + bs) * n + a; g1.lda = n; g1.strideA = stride;
      g1.B = w.A + a * n + a; g1.ldb = n; g1.strideB = stride;
      g1.C = w.tmp; g1.ldc = bs; g1.strideC = bs * bs;
      g1.M = (int)s2; g1.N = (int)bs; g1.K = (int)bs; g1.batch = (int)count;
      g1.alpha = 1.f; g1.beta = 0.f; g1.flags = GEMM_B_LOWER; g1.info = info;
      if ((e = gemm_f32(g1, false, false, s)) != hipSuccess) return e;
      GemmDesc g2{};  // Linv21 = -Linv22 * tmp
      g2.A = w.A + (a + bs) * n + (a + bs); g2.lda = n; g2.strideA = stride;
      g2.B = w.tmp; g2.ldb = bs; g2.strideB = bs * bs;
      g2.C = w.A + (a + bs) * n + a; g2.ldc = n; g2.strideC = stride;
      g2.M = (int)s2; g2.N = (int)bs; g2.K = (int)s2; g2.batch = (int)count;
      g2.alpha = -1.f; g2.beta = 0.f; g2.flags = GEMM_A_LOWER; g2.info = info;
      if ((e = gemm_f32(g2, false, false, s)) != hipSuccess) return e;
    }
  }
  hipLaunchKernelGGL(write_u_kernel, row_grid(n), dim3(256), 0, s, (const float*)w.A, U, n, (const int32_t*)info);
  return hipGetLastError();
}

}  // namespace gptq
