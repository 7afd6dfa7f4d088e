// The column sweep of GPTQ: per-block quantize-and-compensate, plus the
// conversion, parameter, packing and dequantization kernels around it.
//
// "Part 3: Adaptive Rounding: GPTQ", 'Algorithm GPTQ' and 'Observation 2:
// Lazy Batch Updates': a block of B columns is processed on chip; each column
// is rounded, its error (scaled by the diagonal of the factor) is stored in E
// and compensated into the later columns of the block, and the block's E is
// flushed to all later columns with one matrix product afterwards (the GEMM in
// gemm_f32.hip).  The Vietnamese edition of the English GPTQ second-order
// quantization post ('Lazy batch update') states the flush as
// W[:, B:] <- W[:, B:] - E R[B, B:].
//
// Mapping on gfx950: 16 lanes (one DPP row) own one weight row of the block,
// 8 consecutive columns per lane in registers; a wave holds 4 rows and a
// 256-thread workgroup 16 rows.  The block's factor rows, pre-divided by their
// diagonal, sit in LDS (128 x 128 fp32).  Per column the owning lane's value
// is broadcast across its row with one DPP row_newbcast, every lane rounds it
// redundantly (so scale, zero and error need no further exchange), and each
// lane updates its own 8 columns.  Group minimum / maximum at a group start
// are DPP reductions over the row.
#include <algorithm>

#include "common.hpp"
#include "internal.hpp"

namespace gptq {

namespace {

constexpr int BMAX = 128;
constexpr int UP_PITCH = BMAX + 4;

struct SweepArgs {
  const float* U;
  float* V;
  int64_t n, m;
  int64_t i;  // first column of the block
  int w;      // block width (<= 128)
  int maxq;
  int64_t group;  // group size (<= 0: per row)
  int inblock;    // 1: group starts are taken inside the block (0 < group <= B)
  int64_t G;
  float* S;
  int32_t* Z;
  uint8_t* Q8;   // [m x n] codes
  float* E;      // [m x 128] scaled errors of this block
  float* err_sq; // [m] or null
};

template <int P>
__device__ __forceinline__ float bcast_col(const float (&v)[8]) {
  return row_bcast<(P >> 3)>(v[P & 7]);
}

// Quantizer parameters (s, z) from the range [lo, hi] of a group or row.
__device__ __forceinline__ void qparams(float lo, float hi, int maxq, float& s, float& z) {
  lo = fminf(lo, 0.f);
  hi = fmaxf(hi, 0.f);
  if (hi == lo) { lo = 0.f; hi = 1.f; }
  s = (hi - lo) / (float)maxq;
  z = rintf(-lo / s);
}

template <int P>
__device__ __forceinline__ void sweep_step(const SweepArgs& a, float (&v)[8], float (&ek)[8], float (&qk)[8],
                                           float& s, float& inv_s, float& z, float& eacc, int& gcount, int l16,
                                           bool active, int64_t r, const float (*Up)[UP_PITCH], const float* invd) {
  if (a.inblock) {
    if (gcount == 0) {  // first column of a group: (s, z) from the group's current values
      float lo = INFINITY, hi = -INFINITY;
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const int c = 8 * l16 + e;
        if (c >= P && c < P + a.group && c < a.w) {
          lo = fminf(lo, v[e]);
          hi = fmaxf(hi, v[e]);
        }
      }
      lo = row_min16(lo);
      hi = row_max16(hi);
      qparams(lo, hi, a.maxq, s, z);
      inv_s = 1.f / s;
      if (l16 == 0 && active) {
        const int64_t gi = (a.i + P) / a.group;
        a.S[r * a.G + gi] = s;
        a.Z[r * a.G + gi] = (int32_t)z;
      }
      gcount = (int)a.group;
    }
    --gcount;
  }
  const float vp = bcast_col<P>(v);
  const float qz = __builtin_amdgcn_fmed3f(rintf(vp * inv_s), -z, (float)a.maxq - z);
  const float err = fmaf(-s, qz, vp);
  const float e = err * invd[P];
  if (l16 == (P >> 3)) {
    ek[P & 7] = e;
    qk[P & 7] = qz + z;
  }
  eacc = fmaf(e, e, eacc);
  const f32x4 u0 = *(const f32x4*)&Up[P][8 * l16];
  const f32x4 u1 = *(const f32x4*)&Up[P][8 * l16 + 4];
  v[0] = fmaf(-err, u0[0], v[0]);
  v[1] = fmaf(-err, u0[1], v[1]);
  v[2] = fmaf(-err, u0[2], v[2]);
  v[3] = fmaf(-err, u0[3], v[3]);
  v[4] = fmaf(-err, u1[0], v[4]);
  v[5] = fmaf(-err, u1[1], v[5]);
  v[6] = fmaf(-err, u1[2], v[6]);
  v[7] = fmaf(-err, u1[3], v[7]);
}

template <int P>
struct Steps {
  __device__ __forceinline__ static void run(const SweepArgs& a, float (&v)[8], float (&ek)[8], float (&qk)[8],
                                             float& s, float& inv_s, float& z, float& eacc, int& gcount, int l16,
                                             bool active, int64_t r, const float (*Up)[UP_PITCH], const float* invd) {
    if (P >= a.w) return;
    sweep_step<P>(a, v, ek, qk, s, inv_s, z, eacc, gcount, l16, active, r, Up, invd);
    Steps<P + 1>::run(a, v, ek, qk, s, inv_s, z, eacc, gcount, l16, active, r, Up, invd);
  }
};
template <>
struct Steps<BMAX> {
  __device__ __forceinline__ static void run(const SweepArgs&, float (&)[8], float (&)[8], float (&)[8], float&,
                                             float&, float&, float&, int&, int, bool, int64_t,
                                             const float (*)[UP_PITCH], const float*) {}
};

__global__ __launch_bounds__(256) void sweep_block_kernel(SweepArgs a) {
  __shared__ __attribute__((aligned(16))) float Up[BMAX][UP_PITCH];
  __shared__ float invd[BMAX];
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int l16 = lane & 15;
  const int64_t r = (int64_t)blockIdx.x * 16 + (tid >> 4);
  const bool active = r < a.m;
  const int w = a.w;
  const int64_t i = a.i;

  if (tid < BMAX) invd[tid] = (tid < w) ? 1.f / a.U[(i + tid) * a.n + i + tid] : 0.f;
  __syncthreads();
  for (int idx = tid; idx < BMAX * BMAX; idx += 256) {
    const int p = idx >> 7, j = idx & (BMAX - 1);
    float u = 0.f;
    if (p < w && j < w && j > p) u = a.U[(i + p) * a.n + i + j] * invd[p];
    Up[p][j] = u;
  }

  float v[8], ek[8], qk[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    const int c = 8 * l16 + e;
    v[e] = (active && c < w) ? a.V[r * a.n + i + c] : 0.f;
    ek[e] = 0.f;
    qk[e] = 0.f;
  }
  float s = 1.f, z = 0.f;
  if (!a.inblock && active) {
    const int64_t gi = a.group <= 0 ? 0 : i / a.group;
    s = a.S[r * a.G + gi];
    z = (float)a.Z[r * a.G + gi];
  }
  float inv_s = 1.f / s;
  float eacc = 0.f;
  int gcount = 0;
  __syncthreads();

  Steps<0>::run(a, v, ek, qk, s, inv_s, z, eacc, gcount, l16, active, r, Up, invd);

  if (active) {
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const int c = 8 * l16 + e;
      if (c < w) {
        a.E[r * BMAX + c] = ek[e];
        a.Q8[r * a.n + i + c] = (uint8_t)(int)qk[e];
      }
    }
    if (l16 == 0 && a.err_sq) a.err_sq[r] += eacc;
  }
}

// V = fp32 copy of W (row-major, leading dimension n).
template <int DT>
__global__ __launch_bounds__(256) void to_f32_kernel(const void* W, int64_t ldw, float* V, int64_t m, int64_t n) {
  for (int64_t r = blockIdx.y; r < m; r += gridDim.y)
    for (int64_t c = blockIdx.x * 256 + threadIdx.x; c < n; c += (int64_t)gridDim.x * 256)
      V[r * n + c] = Elem<DT>::load(W, r * ldw + c);
}

// (s, z) of columns [c0, c0 + width) of each row, one wave per row.
__global__ __launch_bounds__(256) void row_params_kernel(const float* V, int64_t m, int64_t n, int64_t c0,
                                                         int64_t width, int maxq, float* S, int32_t* Z, int64_t G,
                                                         int64_t gidx) {
  const int64_t r = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  if (r >= m) return;  // whole wave
  float lo = INFINITY, hi = -INFINITY;
  const int64_t c1 = std::min<int64_t>(n, c0 + width);
  for (int64_t c = c0 + lane; c < c1; c += 64) {
    const float x = V[r * n + c];
    lo = fminf(lo, x);
    hi = fmaxf(hi, x);
  }
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) {
    lo = fminf(lo, __shfl_xor(lo, o, 64));
    hi = fmaxf(hi, __shfl_xor(hi, o, 64));
  }
  if (lane == 0) {
    float s, z;
    qparams(lo, hi, maxq, s, z);
    S[r * G + gidx] = s;
    Z[r * G + gidx] = (int32_t)z;
  }
}

__global__ __launch_bounds__(256) void zero_f32_kernel(float* p, int64_t count) {
  for (int64_t k = (int64_t)blockIdx.x * 256 + threadIdx.x; k < count; k += (int64_t)gridDim.x * 256) p[k] = 0.f;
}

// Pack codes into per-row little-endian bit-streams: one thread per output word.
__global__ __launch_bounds__(256) void pack_kernel(const uint8_t* Q8, int64_t m, int64_t n, int bits,
                                                   uint32_t* out, int64_t words) {
  for (int64_t r = blockIdx.y; r < m; r += gridDim.y)
  for (int64_t wd = (int64_t)blockIdx.x * 256 + threadIdx.x; wd < words; wd += (int64_t)gridDim.x * 256) {
    const int64_t bit0 = wd * 32;
    const int64_t j0 = bit0 / bits;
    const int64_t j1 = std::min<int64_t>(n - 1, (bit0 + 31) / bits);
    uint32_t word = 0;
    for (int64_t j = j0; j <= j1; ++j) {
      const uint32_t q = Q8[r * n + j];
      const int64_t sh = j * bits - bit0;
      word |= (sh >= 0) ? (q << sh) : (q >> (-sh));
    }
    out[r * words + wd] = word;
  }
}

// W <- s (q - z) in W's dtype.
template <int DT>
__global__ __launch_bounds__(256) void dequant_kernel(void* W, int64_t ldw, const uint8_t* Q8, const float* S,
                                                      const int32_t* Z, int64_t m, int64_t n, int64_t group,
                                                      int64_t G) {
  for (int64_t r = blockIdx.y; r < m; r += gridDim.y)
  for (int64_t c = (int64_t)blockIdx.x * 256 + threadIdx.x; c < n; c += (int64_t)gridDim.x * 256) {
    const int64_t g = group <= 0 ? 0 : c / group;
    const float s = S[r * G + g];
    const float z = (float)Z[r * G + g];
    Elem<DT>::store(W, r * ldw + c, s * ((float)Q8[r * n + c] - z));
  }
}

inline size_t align256(size_t b) { return (b + 255) & ~(size_t)255; }

dim3 rows_grid(int64_t cols, int64_t rows) {
  return dim3((unsigned)std::min<int64_t>(cdiv(cols, 256), 64), (unsigned)std::min<int64_t>(rows, 65535));
}

}  // namespace

size_t quantize_workspace_bytes(int64_t m, int64_t n) {
  if (m < 1 || n < 1) return 0;
  return align256((size_t)m * n * 4) + align256((size_t)m * n) + align256((size_t)m * BMAX * 4);
}

hipError_t quantize_layer(void* W, int dt, int64_t m, int64_t n, int64_t ldw, const float* U, int bits,
                          int64_t group, int64_t B, uint32_t* qcodes, float* S, int32_t* Z, float* err_sq,
                          int write_dequant, void* ws, hipStream_t st) {
  char* p = (char*)ws;
  float* V = (float*)p;
  p += align256((size_t)m * n * 4);
  uint8_t* Q8 = (uint8_t*)p;
  p += align256((size_t)m * n);
  float* E = (float*)p;

  const int maxq = (1 << bits) - 1;
  const int64_t G = group <= 0 ? 1 : cdiv(n, group);
  const int inblock = (group > 0 && group <= B) ? 1 : 0;
  const dim3 rg = rows_grid(n, m);

  if (dt == 0) hipLaunchKernelGGL((to_f32_kernel<0>), rg, dim3(256), 0, st, W, ldw, V, m, n);
  else if (dt == 1) hipLaunchKernelGGL((to_f32_kernel<1>), rg, dim3(256), 0, st, W, ldw, V, m, n);
  else hipLaunchKernelGGL((to_f32_kernel<2>), rg, dim3(256), 0, st, W, ldw, V, m, n);
  const unsigned prow = (unsigned)cdiv(m, 4);
  if (group <= 0)
    hipLaunchKernelGGL(row_params_kernel, dim3(prow), dim3(256), 0, st, (const float*)V, m, n, (int64_t)0, n, maxq, S,
                       Z, G, (int64_t)0);
  if (err_sq)
    hipLaunchKernelGGL(zero_f32_kernel, dim3((unsigned)std::min<int64_t>(cdiv(m, 256), 1024)), dim3(256), 0, st,
                       err_sq, m);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;

  for (int64_t i = 0; i < n; i += B) {
    const int w = (int)std::min<int64_t>(B, n - i);
    if (group > B && i % group == 0)
      hipLaunchKernelGGL(row_params_kernel, dim3(prow), dim3(256), 0, st, (const float*)V, m, n, i, group, maxq, S,
                         Z, G, i / group);
    SweepArgs a{U, V, n, m, i, w, maxq, group, inblock, G, S, Z, Q8, E, err_sq};
    hipLaunchKernelGGL(sweep_block_kernel, dim3((unsigned)cdiv(m, 16)), dim3(256), 0, st, a);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    if (i + w < n) {
      GemmDesc g{};
      g.A = E; g.lda = BMAX;
      g.B = U + i * n + i + w; g.ldb = n;
      g.C = V + i + w; g.ldc = n;
      g.M = (int)m; g.N = (int)(n - i - w); g.K = w; g.batch = 1;
      g.alpha = -1.f; g.beta = 1.f;
      if ((e = gemm_f32(g, false, false, st)) != hipSuccess) return e;
    }
  }
  const int64_t words = cdiv(n * bits, 32);
  hipLaunchKernelGGL(pack_kernel, rows_grid(words, m), dim3(256), 0, st, (const uint8_t*)Q8, m, n, bits, qcodes, words);
  if (write_dequant) {
    if (dt == 0) hipLaunchKernelGGL((dequant_kernel<0>), rg, dim3(256), 0, st, W, ldw, (const uint8_t*)Q8, (const float*)S, (const int32_t*)Z, m, n, group, G);
    else if (dt == 1) hipLaunchKernelGGL((dequant_kernel<1>), rg, dim3(256), 0, st, W, ldw, (const uint8_t*)Q8, (const float*)S, (const int32_t*)Z, m, n, group, G);
    else hipLaunchKernelGGL((dequant_kernel<2>), rg, dim3(256), 0, st, W, ldw, (const uint8_t*)Q8, (const float*)S, (const int32_t*)Z, m, n, group, G);
  }
  return hipGetLastError();
}

}  // namespace gptq
