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
//        leaf kernel: one workgroup factors the NB x NB diagonal block in
//        LDS and also inverts it;
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
// write its inverse to Dinv (NB x NB, zero above the diagonal).
__global__ __launch_bounds__(256) void chol_leaf_kernel(float* A, int64_t lda, int64_t k0, int kb, float* Dinv,
                                                        int32_t* info, int64_t n) {
  if (*info != 0) return;
  __shared__ float S[NB][NB + 1];
  __shared__ float T[NB][NB + 1];
  __shared__ float col[NB];
  const int tid = threadIdx.x;
  for (int idx = tid; idx < NB * NB; idx += 256) {
    const int r = idx / NB, c = idx % NB;
    S[r][c] = (r < kb && c < kb && c <= r) ? A[(k0 + r) * lda + k0 + c] : 0.f;
    T[r][c] = (r == c) ? 1.f : 0.f;
  }
  __syncthreads();
  const int tr = tid >> 4, tc = tid & 15;
  for (int j = 0; j < kb; ++j) {
    const float d = S[j][j];
    if (!(d > 0.f) || !(d < INFINITY)) {  // uniform: every thread read the same d
      if (tid == 0) atomicCAS(info, 0, (int32_t)(n - (k0 + j)));
      return;
    }
    const float sd = sqrtf(d);
    if (tid < kb) col[tid] = (tid > j) ? S[tid][j] / sd : 0.f;
    __syncthreads();
    if (tid < kb && tid > j) S[tid][j] = col[tid];
    if (tid == j) S[j][j] = sd;
    for (int r = j + 1 + tr; r < kb; r += 16) {
      const float cr = col[r];
      for (int c = j + 1 + tc; c <= r; c += 16) S[r][c] -= cr * col[c];
    }
    __syncthreads();
  }
  // inverse of the lower-triangular factor, row by row: T <- L^{-1}
  for (int k = 0; k < kb; ++k) {
    const float dk = S[k][k];
    if (tid <= k) T[k][tid] = T[k][tid] / dk;
    __syncthreads();
    for (int r = k + 1 + tr; r < kb; r += 16) {
      const float l = S[r][k];
      for (int c = tc; c <= k; c += 16) T[r][c] -= l * T[k][c];
    }
    __syncthreads();
  }
  for (int idx = tid; idx < NB * NB; idx += 256) {
    const int r = idx / NB, c = idx % NB;
    if (r < kb && c <= r) A[(k0 + r) * lda + k0 + c] = S[r][c];
    Dinv[idx] = (r < kb && c < kb && c <= r) ? T[r][c] : 0.f;
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
