// OBQ's greedy-order quantization of a layer ([OBQ] "Greedy Search"): each
// row quantizes, one weight at a time, the unquantized weight whose rounding
// adds the least to the proxy loss, dL_p = (what_p - w_p)^2 / [H^-1]_pp,
// moves the others by the OBS compensation ([OBQ] "Generalized Weight
// Update") and removes p from its own copy of H^-1 by the rank-one downdate
// H^-1 - H^-1_{:,p} H^-1_{p,:} / [H^-1]_pp ([OBQ] "The OBS / GPTQ Trick").
// Rows pick different weights, so each needs its own H^-1 ([OBQ] "Limitations
// of OBQ", item 2): here one workgroup owns one row at a time and keeps that
// row's H^-1 as a packed lower triangle, in LDS for rows of up to NL weights
// (157 KB of the CU's 160 KB) and in a per-workgroup slice of the workspace
// beyond that.
//
// Unquantized weights always occupy positions 0..R-1: after weight p is
// chosen it is swapped with position R-1 (row and column of the triangle,
// the weight, its column index), so the downdate only touches the leading
// (R-1)-triangle, which stays contiguous in the packed layout.  Every group's
// grid (s, z) is fixed once from the original row, since the order jumps
// across groups; equal scores go to the smaller column index.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <algorithm>

#include "common.hpp"

namespace gptq {
namespace {

constexpr int GT = 256;     // threads per workgroup (4 waves)
constexpr int GWV = GT / 64;
constexpr int NL = 280;     // longest row whose packed H^-1 fits in LDS
constexpr int NMAX = 4096;  // longest row of the workspace-resident path
constexpr int GMIN = 16;    // smallest group (bounds the per-group tables)
constexpr int GRID_G = 512; // workgroups (and workspace slices) of the workspace path

__host__ __device__ constexpr int tri(int i) { return i * (i + 1) / 2; }  // start of packed row i

template <int N, int TF>
struct GreedySmem {
  float T[TF > 0 ? TF : 1];  // packed lower triangle of the row's H^-1 (LDS path)
  float w[N];                // current weights by position
  float c[N];                // the eliminated weight's H^-1 column (downdate vector)
  int perm[N];               // original column of each position
  float gs[N / GMIN + 1], gis[N / GMIN + 1], gz[N / GMIN + 1];  // per-group s, 1/s, z
  uint64_t rkey[GWV];        // per-wave best candidate
  float rerr[GWV], rd[GWV];
  int rcode[GWV];
  uint8_t code[N];           // chosen codes by original column
};

struct GreedyArgs {
  const void* W;
  const float* Hp;  // packed H^-1 (tri(n) floats)
  float* Tws;       // workspace slices (workspace path)
  int64_t ldw, m;
  int n, bits, gsz, G, words;
  uint32_t* Q;
  float* S;
  int32_t* Z;
  int32_t* order;
  float* loss;
};

__device__ __forceinline__ float wave_min(float v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v = fminf(v, __shfl_xor(v, o));
  return v;
}
__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v = fmaxf(v, __shfl_xor(v, o));
  return v;
}

// H^-1 = U^T U (U upper) as a packed lower triangle: Hp[tri(i) + j] for j <= i.
__global__ __launch_bounds__(256) void hinv_pack_kernel(const float* __restrict__ U, int n, float* __restrict__ Hp) {
  const int64_t e = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (e >= (int64_t)tri(n)) return;
  int i = (int)((sqrt(8.0 * (double)e + 1.0) - 1.0) * 0.5);
  while ((int64_t)tri(i + 1) <= e) ++i;
  while ((int64_t)tri(i) > e) --i;
  const int j = (int)(e - tri(i));
  float acc = 0.f;
  for (int k = 0; k <= j; ++k) acc = fmaf(U[(int64_t)k * n + i], U[(int64_t)k * n + j], acc);
  Hp[e] = acc;
}

template <int DT, bool INLDS>
__global__ __launch_bounds__(GT) void greedy_kernel(GreedyArgs a) {
  constexpr int N = INLDS ? NL : NMAX;
  __shared__ __attribute__((aligned(16))) GreedySmem<N, INLDS ? tri(NL) : 0> sm;
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const int n = a.n, P = tri(n);
  const int maxq = (1 << a.bits) - 1;
  float* T;
  if constexpr (INLDS) {
    T = sm.T;
  } else {
    T = a.Tws + (int64_t)blockIdx.x * (((int64_t)P + 63) & ~(int64_t)63);
  }

  for (int64_t row = blockIdx.x; row < a.m; row += gridDim.x) {
    for (int e = tid; e < P; e += GT) T[e] = a.Hp[e];
    for (int k = tid; k < n; k += GT) {
      sm.w[k] = Elem<DT>::load(a.W, row * a.ldw + k);
      sm.perm[k] = k;
    }
    __syncthreads();
    // The grid of every group from the original row.
    for (int g = wv; g < a.G; g += GWV) {
      const int c0 = g * a.gsz, c1 = min(n, c0 + a.gsz);
      float lo = INFINITY, hi = -INFINITY;
      for (int c = c0 + lane; c < c1; c += 64) {
        lo = fminf(lo, sm.w[c]);
        hi = fmaxf(hi, sm.w[c]);
      }
      lo = wave_min(lo);
      hi = wave_max(hi);
      float s, z;
      qparams(lo, hi, maxq, s, z);
      if (lane == 0) {
        sm.gs[g] = s;
        sm.gis[g] = 1.f / s;
        sm.gz[g] = z;
        a.S[row * a.G + g] = s;
        a.Z[row * a.G + g] = (int32_t)z;
      }
    }
    __syncthreads();

    double loss = 0.0;
    for (int R = n; R >= 1; --R) {
      const int last = R - 1;
      // Scores of the unquantized weights; the smallest (score, column) wins.
      uint64_t best = ~0ull;
      float berr = 0.f, bd = 1.f;
      int bcode = 0;
      for (int k = tid; k < R; k += GT) {
        const int col = sm.perm[k];
        const int g = col / a.gsz;
        const float s = sm.gs[g], z = sm.gz[g];
        const float wk = sm.w[k];
        const float qz = __builtin_amdgcn_fmed3f(rintf(wk * sm.gis[g]), -z, (float)maxq - z);
        const float err = s * qz - wk;
        const float d = T[tri(k) + k];
        const float sc = err * err / d;
        const uint64_t key = ((uint64_t)__float_as_uint(sc) << 32) | ((uint64_t)col << 16) | (uint64_t)k;
        if (key < best) {
          best = key;
          berr = err;
          bd = d;
          bcode = (int)(qz + z);
        }
      }
      uint64_t wmin = best;
#pragma unroll
      for (int o = 32; o >= 1; o >>= 1) {
        const uint64_t t = __shfl_xor(wmin, o);
        wmin = t < wmin ? t : wmin;
      }
      if (wmin == ~0ull) {
        if (lane == 0) sm.rkey[wv] = ~0ull;
      } else if (best == wmin) {  // the one lane holding the wave's winner
        sm.rkey[wv] = wmin;
        sm.rerr[wv] = berr;
        sm.rd[wv] = bd;
        sm.rcode[wv] = bcode;
      }
      __syncthreads();
      int bw = 0;
      uint64_t kk = sm.rkey[0];
#pragma unroll
      for (int i = 1; i < GWV; ++i) {
        const uint64_t t = sm.rkey[i];
        if (t < kk) {
          kk = t;
          bw = i;
        }
      }
      const int p = (int)(kk & 0xFFFF), colp = (int)((kk >> 16) & 0xFFFF);
      const float err = sm.rerr[bw], d = sm.rd[bw];
      if (tid == 0) {
        sm.code[colp] = (uint8_t)sm.rcode[bw];
        if (a.order) a.order[row * n + (n - R)] = colp;
        loss += (double)(err * err / d);
      }
      // Compensation w_k += (what_p - w_p) H^-1_pk / H^-1_pp, and the swap of
      // positions p and R-1; c receives the H^-1 column of the eliminated weight.
      const float f = err / d;
      for (int k = tid; k < R; k += GT) {
        if (k == p) continue;
        const int ipk = p > k ? tri(p) + k : tri(k) + p;
        const float av = T[ipk];
        if (k != last) {
          if (p != last) {
            const int ilk = tri(last) + k;
            T[ipk] = T[ilk];
            T[ilk] = av;
          }
          sm.w[k] += f * av;
          sm.c[k] = av;
        } else {  // position p takes over the last unquantized weight
          sm.w[p] = sm.w[last] + f * av;
          sm.perm[p] = sm.perm[last];
          T[tri(p) + p] = T[tri(last) + last];
          sm.c[p] = av;
        }
      }
      __syncthreads();
      // Rank-one downdate of the leading (R-1)-triangle.  Rows r and R-2-r
      // are paired (r + 1 and R-1-r entries, R in all) and one wave sweeps a
      // pair with its lanes.
      const int Rr = last;
      const float dinv = 1.f / d;
      const int npair = (Rr + 1) / 2;
      for (int r = wv; r < npair; r += GWV) {
        const int r2 = Rr - 1 - r;
        const int len = r == r2 ? r + 1 : Rr + 1;
        const float cr = sm.c[r] * dinv, cr2 = sm.c[r2] * dinv;
        const int b1 = tri(r), b2 = tri(r2) - r - 1;
        for (int x0 = 0; x0 < len; x0 += 256) {
          float tv[4], cv[4];
          int ev[4];
#pragma unroll
          for (int u = 0; u < 4; ++u) {
            const int x = x0 + lane + 64 * u;
            const bool first = x <= r;
            const int j = first ? x : x - r - 1;
            ev[u] = x < len ? (first ? b1 : b2) + x : -1;
            cv[u] = x < len ? sm.c[j] * (first ? cr : cr2) : 0.f;
            tv[u] = x < len ? T[ev[u]] : 0.f;
          }
#pragma unroll
          for (int u = 0; u < 4; ++u)
            if (ev[u] >= 0) T[ev[u]] = tv[u] - cv[u];
        }
      }
      __syncthreads();
    }

    for (int wd = tid; wd < a.words; wd += GT) {
      const int b0 = wd * 32;
      const int j0 = b0 / a.bits, j1 = min(n - 1, (b0 + 31) / a.bits);
      uint64_t acc = 0;
      for (int j = j0; j <= j1; ++j) {
        const int off = j * a.bits - b0;
        const uint64_t cv = sm.code[j];
        acc |= off >= 0 ? (cv << off) : (cv >> -off);
      }
      a.Q[row * a.words + wd] = (uint32_t)acc;
    }
    if (tid == 0 && a.loss) a.loss[row] = (float)loss;
    __syncthreads();
  }
}

int64_t slice_floats(int64_t n) { return ((int64_t)tri((int)n) + 63) & ~(int64_t)63; }

template <int DT>
void launch_greedy(const GreedyArgs& a, hipStream_t st) {
  if (a.n <= NL) {
    const int grid = (int)std::min<int64_t>(a.m, 65535);
    hipLaunchKernelGGL((greedy_kernel<DT, true>), dim3(grid), dim3(GT), 0, st, a);
  } else {
    const int grid = (int)std::min<int64_t>(a.m, GRID_G);
    hipLaunchKernelGGL((greedy_kernel<DT, false>), dim3(grid), dim3(GT), 0, st, a);
  }
}

}  // namespace

bool greedy_supported(int64_t n, int64_t group) { return n <= NMAX && (group <= 0 || group >= GMIN); }

size_t greedy_workspace_bytes(int64_t m, int64_t n) {
  if (m < 1 || n < 1 || n > NMAX) return 0;
  const int64_t slices = n <= NL ? 0 : std::min<int64_t>(m, GRID_G);
  return (size_t)(slice_floats(n) * (1 + slices)) * sizeof(float);
}

hipError_t quantize_greedy(const void* W, int dt, int64_t m, int64_t n, int64_t ldw, const float* U, int bits,
                           int64_t group, uint32_t* qcodes, float* S, int32_t* Z, int32_t* order, float* loss, void* ws,
                           hipStream_t st) {
  float* Hp = (float*)ws;
  const int64_t P = tri((int)n);
  hipLaunchKernelGGL(hinv_pack_kernel, dim3((unsigned)cdiv(P, 256)), dim3(256), 0, st, U, (int)n, Hp);
  GreedyArgs a;
  a.W = W;
  a.Hp = Hp;
  a.Tws = Hp + slice_floats(n);
  a.ldw = ldw;
  a.m = m;
  a.n = (int)n;
  a.bits = bits;
  a.gsz = group > 0 ? (int)std::min<int64_t>(group, n) : (int)n;
  a.G = group > 0 ? (int)cdiv(n, group) : 1;
  a.words = (int)cdiv(n * bits, 32);
  a.Q = qcodes;
  a.S = S;
  a.Z = Z;
  a.order = order;
  a.loss = loss;
  switch (dt) {
    case 0: launch_greedy<0>(a, st); break;
    case 1: launch_greedy<1>(a, st); break;
    default: launch_greedy<2>(a, st); break;
  }
  return hipGetLastError();
}

}  // namespace gptq
