// OBQ's greedy-order quantization of a layer ([OBQ] "Greedy Search"): each
// row quantizes, one weight at a time, the unquantized weight whose rounding
// adds the least to the proxy loss, dL_p = (what_p - w_p)^2 / [H^-1]_pp,
// moves the others by the OBS compensation ([OBQ] "Generalized Weight
// Update") and removes p from its own copy of H^-1 by the rank-one downdate
// H^-1 - H^-1_{:,p} H^-1_{p,:} / [H^-1]_pp ([OBQ] "The OBS / GPTQ Trick").
// Rows pick different weights, so each needs its own H^-1 ([OBQ] "Limitations
// of OBQ", item 2): here one workgroup owns one row at a time and keeps that
// row's H^-1 as a packed lower triangle.  Rows of up to NLZ weights defer
// their downdates (greedy_lazy_kernel; the base in LDS up to NLB weights,
// with four rows per CU up to NS, else in a per-workgroup slice of the
// workspace); longer rows downdate a workspace slice every step
// (greedy_kernel).
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

constexpr int NS = 128;     // longest row of the four-rows-per-CU variant
constexpr int NMAX = 4096;  // longest row of the workspace-resident path
constexpr int GMIN = 16;    // smallest group (bounds the per-group tables)
constexpr int GRID_G = 256; // workgroups (and workspace slices) of the workspace path
constexpr int RB = 4;       // full rows per downdate batch


__host__ __device__ constexpr int tri(int i) { return i * (i + 1) / 2; }  // start of packed row i

// Floats per packed copy of H^-1: the triangle, then 64 spare entries that
// lanes past the end of a downdate row read and write instead of branching.
__host__ __device__ constexpr int64_t slice_floats(int64_t n) { return ((n * (n + 1) / 2 + 64) + 63) & ~(int64_t)63; }

template <int N, int NW>
struct GreedySmem {
  float w[N];                     // current weights by position
  float c[N];                     // the eliminated weight's H^-1 column (downdate vector)
  float e2[N];                    // squared rounding error of each position's weight
  float ps[N], pis[N], pz[N];     // each position's grid: s, 1/s, z
  int perm[N];                    // original column of each position
  uint16_t ord[N];                // column quantized at each step
  float gs[N / GMIN + 1], gis[N / GMIN + 1], gz[N / GMIN + 1];  // per-group s, 1/s, z
  uint64_t rkey[NW];              // per-wave best candidate
  float rerr[NW], rd[NW];
  int rcode[NW];
  uint8_t code[N];                // chosen codes by original column
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

template <int CTRL, int ROWS>
__device__ __forceinline__ uint32_t dpp_u(uint32_t old, uint32_t src) {
  return (uint32_t)__builtin_amdgcn_update_dpp((int)old, (int)src, CTRL, ROWS, 0xF, false);
}

// Unsigned minimum over the 64 lanes by DPP (within quads, across each
// 16-lane row, then row_bcast:15 and row_bcast:31 carry it to lane 63).
__device__ __forceinline__ uint32_t wave_min_u32(uint32_t v) {
  v = min(v, dpp_u<0xB1, 0xF>(v, v));   // quad_perm [1,0,3,2]
  v = min(v, dpp_u<0x4E, 0xF>(v, v));   // quad_perm [2,3,0,1]
  v = min(v, dpp_u<0x124, 0xF>(v, v));  // row_ror:4
  v = min(v, dpp_u<0x128, 0xF>(v, v));  // row_ror:8
  v = min(v, dpp_u<0x142, 0xA>(v, v));  // row_bcast:15 into rows 1 and 3
  v = min(v, dpp_u<0x143, 0xC>(v, v));  // row_bcast:31 into rows 2 and 3
  return (uint32_t)__builtin_amdgcn_readlane((int)v, 63);
}

// Rounding of w on the grid (s, 1/s, z): returns what - w, sets the code.
__device__ __forceinline__ float round_err(float w, float s, float is, float z, int maxq, int& code) {
  const float qz = __builtin_amdgcn_fmed3f(rintf(w * is), -z, (float)maxq - z);
  code = (int)(qz + z);
  return s * qz - w;
}

// A score's bit pattern orders like the score for every non-negative value
// (NaN after +inf); all ones is kept for "no candidate".
__device__ __forceinline__ uint32_t score_bits(float e2, float d) {
  return min(__float_as_uint(e2 * __builtin_amdgcn_rcpf(d)), 0xFFFFFFFEu);
}

// Candidate (score, column, position, H^-1 diagonal) of one lane.
struct Cand {
  uint32_t sc;
  int col, pos;
  float d;
  __device__ __forceinline__ void init() {
    sc = 0xFFFFFFFFu;
    col = 0xFFFF;
    pos = 0;
    d = 1.f;
  }
  __device__ __forceinline__ void offer(uint32_t s, int c, int p, float dd) {
    if (s < sc || (s == sc && c < col)) {
      sc = s;
      col = c;
      pos = p;
      d = dd;
    }
  }
};

// The wave's smallest (score, column); its lane posts it with the rounding
// error and code of that position's weight.
template <typename SM, typename ErrF>
__device__ __forceinline__ void post_wave_best(SM& sm, const Cand& b, int lane, int wv, ErrF errf) {
  const uint32_t wmin = wave_min_u32(b.sc);
  if (wmin == 0xFFFFFFFFu) {
    if (lane == 0) sm.rkey[wv] = ~0ull;
    return;
  }
  uint64_t tied = __ballot(b.sc == wmin);
  int wl = __builtin_ctzll(tied);
  if (tied & (tied - 1)) {  // equal scores: the smallest column
    int wc = 0x10000;
    while (tied) {
      const int l = __builtin_ctzll(tied);
      tied &= tied - 1;
      const int cl = __builtin_amdgcn_readlane(b.col, l);
      if (cl < wc) {
        wc = cl;
        wl = l;
      }
    }
  }
  if (lane == wl) {
    const int k = b.pos;
    int code;
    const float err = errf(k, code);
    sm.rkey[wv] = ((uint64_t)b.sc << 32) | ((uint64_t)b.col << 16) | (uint64_t)k;
    sm.rerr[wv] = err;
    sm.rd[wv] = b.d;
    sm.rcode[wv] = code;
  }
}

// Smallest of the NW per-wave posts: every 16-lane row holds them (repeated
// when NW < 16) and a DPP minimum over the row finds it; bw receives the
// posting wave.
template <int NW, typename SM>
__device__ __forceinline__ uint64_t min_post(SM& sm, int lane, int& bw) {
  static_assert(NW == 4 || NW == 8 || NW == 16, "the posts fit one 16-lane DPP row");
  const uint64_t mine = sm.rkey[lane & (NW - 1)];
  uint32_t hi = (uint32_t)(mine >> 32), lo = (uint32_t)mine;
#define GREEDY_MIN_STEP(CTRL)                                                                  \
  {                                                                                          \
    const uint32_t oh = (uint32_t)__builtin_amdgcn_mov_dpp((int)hi, CTRL, 0xF, 0xF, false);  \
    const uint32_t ol = (uint32_t)__builtin_amdgcn_mov_dpp((int)lo, CTRL, 0xF, 0xF, false);  \
    const bool take = oh < hi || (oh == hi && ol < lo);                                      \
    hi = take ? oh : hi;                                                                     \
    lo = take ? ol : lo;                                                                     \
  }
  GREEDY_MIN_STEP(0xB1)                 // quad_perm [1,0,3,2]
  GREEDY_MIN_STEP(0x4E)                 // quad_perm [2,3,0,1]
  if constexpr (NW >= 8) GREEDY_MIN_STEP(0x124)   // row_ror:4
  if constexpr (NW >= 16) GREEDY_MIN_STEP(0x128)  // row_ror:8
#undef GREEDY_MIN_STEP
  const uint64_t kk = ((uint64_t)(uint32_t)__builtin_amdgcn_readlane((int)hi, 0) << 32) |
                      (uint32_t)__builtin_amdgcn_readlane((int)lo, 0);
  bw = __builtin_ctzll(__ballot(lane < NW && mine == kk) | (1ull << 63));
  bw = bw > NW - 1 ? 0 : bw;
  return kk;
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

// One step is two phases separated by barriers: (1) every thread reads the
// winner (position p) from the per-wave posts; the other weights are
// compensated, p is swapped with the last unquantized position, and each
// moved weight's squared rounding error is refreshed; (2) the rank-one
// downdate of the leading (R-1)-triangle, in which the lane that updates a
// diagonal entry also scores that position for the next step.  Lanes that
// fall past the end of the triangle read and write spare entries instead of
// branching.
//
// It takes the rows longer than the deferred-downdate kernel does, with the
// row's H^-1 in a workspace slice (1024 threads).
template <int DT>
__global__ __launch_bounds__(1024) void greedy_kernel(GreedyArgs a) {
  constexpr int N = NMAX, NT = 1024, NW = NT / 64;
  __shared__ __attribute__((aligned(16))) GreedySmem<N, NW> sm;
  const int tid = threadIdx.x, lane = tid & 63, wv = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int n = a.n, P = tri(n);
  const int maxq = (1 << a.bits) - 1;
  const int spare = P + lane;  // where lanes past the end of a row read and write
  float* T = a.Tws + (int64_t)blockIdx.x * slice_floats(n);
  auto errf = [&](int k, int& code) { return round_err(sm.w[k], sm.ps[k], sm.pis[k], sm.pz[k], maxq, code); };

  for (int64_t row = blockIdx.x; row < a.m; row += gridDim.x) {
    for (int e = tid; e < P; e += NT) T[e] = a.Hp[e];
    for (int k = tid; k < n; k += NT) {
      sm.w[k] = Elem<DT>::load(a.W, row * a.ldw + k);
      sm.perm[k] = k;
    }
    __syncthreads();
    // The grid of every group from the original row.
    for (int g = wv; g < a.G; g += NW) {
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
    // Each position's grid, and the scores of the first step.
    Cand b;
    b.init();
    for (int k = tid; k < n; k += NT) {
      const int g = k / a.gsz;
      const float s = sm.gs[g], is = sm.gis[g], z = sm.gz[g];
      sm.ps[k] = s;
      sm.pis[k] = is;
      sm.pz[k] = z;
      int code;
      const float err = round_err(sm.w[k], s, is, z, maxq, code);
      sm.e2[k] = err * err;
      const float d = T[tri(k) + k];
      b.offer(score_bits(err * err, d), k, k, d);
    }
    post_wave_best(sm, b, lane, wv, errf);
    __syncthreads();

    double loss = 0.0;
    for (int R = n; R >= 1; --R) {
      const int last = R - 1;
      int bw;
      const uint64_t kk = min_post<NW>(sm, lane, bw);
      const int p = (int)(kk & 0xFFFF), colp = (int)((kk >> 16) & 0xFFFF);
      const float err = sm.rerr[bw], d = sm.rd[bw];
      if (tid == 0) {
        sm.code[colp] = (uint8_t)sm.rcode[bw];
        sm.ord[n - R] = (uint16_t)colp;
        loss += (double)(err * err / d);
      }
      // Compensation w_k += (what_p - w_p) H^-1_pk / H^-1_pp, and the swap of
      // positions p and R-1; c receives the H^-1 column of the eliminated weight.
      const float f = err / d;
      for (int k = tid; k < R; k += NT) {
        if (k == p) continue;
        const int ipk = p > k ? tri(p) + k : tri(k) + p;
        const float av = T[ipk];
        int code;
        if (k != last) {
          if (p != last) {
            const int ilk = tri(last) + k;
            T[ipk] = T[ilk];
            T[ilk] = av;
          }
          const float wn = sm.w[k] + f * av;
          sm.w[k] = wn;
          sm.c[k] = av;
          const float e = round_err(wn, sm.ps[k], sm.pis[k], sm.pz[k], maxq, code);
          sm.e2[k] = e * e;
        } else {  // position p takes over the last unquantized weight
          const float wn = sm.w[last] + f * av;
          const float s = sm.ps[last], is = sm.pis[last], z = sm.pz[last];
          sm.w[p] = wn;
          sm.perm[p] = sm.perm[last];
          sm.ps[p] = s;
          sm.pis[p] = is;
          sm.pz[p] = z;
          T[tri(p) + p] = T[tri(last) + last];
          sm.c[p] = av;
          const float e = round_err(wn, s, is, z, maxq, code);
          sm.e2[p] = e * e;
        }
      }
      __syncthreads();
      if (R == 1) break;
      // Rank-one downdate of the leading (R-1)-triangle.  Lanes take columns
      // (64 at a time), waves take rows round robin; the lane whose column
      // meets the diagonal also scores that position for the next step.
      const int Rr = last;
      const float dinv = 1.f / d;
      b.init();
      for (int j0 = 0; j0 < Rr; j0 += 64) {
        const int j = j0 + lane;
        const bool jok = j < Rr;
        const int jc = jok ? j : 0;
        const float cj = sm.c[jc] * dinv;
        const float e2j = sm.e2[jc];
        const int pj = sm.perm[jc];
        // Rows j0..j0+63 cross the diagonal (64 / NW per wave, 4 at a time):
        // lanes right of it, and rows past the end, use the spare entries.
        float dj = 0.f;  // new diagonal entry of column j, if this wave owns row j
#pragma unroll
        for (int ub = 0; ub < 64 / NW; ub += 4) {
          float tv[4], ci[4];
          int ev[4];
#pragma unroll
          for (int u = 0; u < 4; ++u) {
            const int ii = j0 + wv + (ub + u) * NW;
            const bool ok = ii < Rr;
            ci[u] = sm.c[ok ? ii : 0];
            ev[u] = ok && j <= ii ? tri(ii) + j : spare;  // j <= ii < Rr: inside the triangle
            tv[u] = T[ev[u]];
          }
#pragma unroll
          for (int u = 0; u < 4; ++u) {
            const float nv = tv[u] - ci[u] * cj;
            T[ev[u]] = nv;
            dj = j == j0 + wv + (ub + u) * NW ? nv : dj;
          }
        }
        // Full rows below: every lane is inside the triangle.
        int i = j0 + 64 + wv;
        for (; i + (RB - 1) * NW < Rr; i += RB * NW) {
          float tv[RB], ci[RB];
          int ev[RB];
#pragma unroll
          for (int u = 0; u < RB; ++u) {
            ci[u] = sm.c[i + u * NW];
            ev[u] = tri(i + u * NW) + j;
            tv[u] = T[ev[u]];
          }
#pragma unroll
          for (int u = 0; u < RB; ++u) T[ev[u]] = tv[u] - ci[u] * cj;
        }
        for (; i < Rr; i += NW) {
          const int e = tri(i) + j;
          T[e] = T[e] - sm.c[i] * cj;
        }
        if (jok && ((j - j0) & (NW - 1)) == wv) b.offer(score_bits(e2j, dj), pj, j, dj);
      }
      post_wave_best(sm, b, lane, wv, errf);
      __syncthreads();
    }

    for (int wd = tid; wd < a.words; wd += NT) {
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
    if (a.order)
      for (int k = tid; k < n; k += NT) a.order[row * n + k] = sm.ord[k];
    if (tid == 0 && a.loss) a.loss[row] = (float)loss;
    __syncthreads();
  }
}

// Rows of up to NLZ weights defer the rank-one downdates, with the base
// H^-1 in LDS up to NLB weights and in the workspace beyond: the true H^-1
// is the stored base minus sum_t c_t c_t^T / d_t over the (at most KD) most
// recent eliminations,
// whose columns c_t sit in LDS.  A step needs only the true row of the
// chosen weight (base row minus the deferred terms) and the diagonal, which
// is kept current in LDS; every KD steps the deferred columns are folded
// into the base by one rank-KD update, so the base is read and written once
// per KD steps instead of every step.  Positions are swapped as in
// greedy_kernel: in the base, the deferred columns and the diagonal alike.
constexpr int NLZ = 1024;  // longest row of the deferred-downdate path
constexpr int NLB = 256;   // longest row whose base H^-1 stays in LDS on that path

// Deferred-downdate variants: rows of up to NS weights, base in LDS, 4 waves
// (four rows per CU); up to NLB, base in LDS, 16 waves; up to NLZ, base in
// the workspace, 16 waves.
template <int LV> struct LVar;
// KD downdates are deferred per base update: 8 with the base in LDS, 16 with
// it in the workspace, where each base update is a pass over HBM.
template <> struct LVar<0> { static constexpr int N = NS, NT = 256, TF = NS * (NS + 1) / 2, KD = 8; };
template <> struct LVar<1> { static constexpr int N = NLB, NT = 1024, TF = NLB * (NLB + 1) / 2, KD = 8; };
template <> struct LVar<2> { static constexpr int N = NLZ, NT = 1024, TF = 0, KD = 16; };

template <int N, int TF, int NW, int KD>
struct LazySmem {
  float T[TF > 0 ? TF + 64 : 1];  // packed base H^-1 (+ 64 spare entries) when it fits in LDS
  float w[N];         // current weights by position
  float e2[N];        // squared rounding error of each position's weight
  float dg[N];        // diagonal of the true H^-1 by position
  float C[KD][N];     // deferred columns of H^-1 by position
  float cdv[KD];      // 1 / d of each deferred column
  int perm[N];        // original column of each position
  uint16_t gpos[N];   // group of each position's weight
  uint16_t ord[N];    // column quantized at each step
  float gs[N / GMIN + 1], gis[N / GMIN + 1], gz[N / GMIN + 1];
  uint64_t rkey[NW];
  float rerr[NW], rd[NW];
  int rcode[NW];
  uint8_t code[N];    // chosen codes by original column
};

template <int DT, int LV>
__global__ __launch_bounds__(LVar<LV>::NT) void greedy_lazy_kernel(GreedyArgs a) {
  constexpr int N = LVar<LV>::N, NT = LVar<LV>::NT, NW = NT / 64, KD = LVar<LV>::KD;
  constexpr bool BASE_LDS = LVar<LV>::TF > 0;
  static_assert(N <= NT, "one position per thread");
  __shared__ __attribute__((aligned(16))) LazySmem<N, LVar<LV>::TF, NW, KD> sm;
  const int tid = threadIdx.x, lane = tid & 63, wv = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int n = a.n, P = tri(n);
  const int maxq = (1 << a.bits) - 1;
  const int spare = P + lane;
  float* T;
  if constexpr (BASE_LDS) {
    T = sm.T;
  } else {
    T = a.Tws + (int64_t)blockIdx.x * slice_floats(n);
  }
  auto errf = [&](int k, int& code) {
    const int g = sm.gpos[k];
    return round_err(sm.w[k], sm.gs[g], sm.gis[g], sm.gz[g], maxq, code);
  };
  const int j = tid;  // this thread's position

  for (int64_t row = blockIdx.x; row < a.m; row += gridDim.x) {
    for (int e = tid; e < P; e += NT) T[e] = a.Hp[e];
    if (j < n) {
      sm.w[j] = Elem<DT>::load(a.W, row * a.ldw + j);
      sm.perm[j] = j;
    }
    __syncthreads();
    for (int g = wv; g < a.G; g += NW) {
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
    Cand b;
    b.init();
    if (j < n) {
      sm.gpos[j] = (uint16_t)(j / a.gsz);
      int code;
      const float err = errf(j, code);
      sm.e2[j] = err * err;
      const float d = T[tri(j) + j];
      sm.dg[j] = d;
      b.offer(score_bits(err * err, d), j, j, d);
    }
    post_wave_best(sm, b, lane, wv, errf);
    __syncthreads();

    double loss = 0.0;
    int kd = 0;  // deferred columns
    for (int R = n; R >= 1; --R) {
      const int last = R - 1;
      int bw;
      const uint64_t kk = min_post<NW>(sm, lane, bw);
      const int p = (int)(kk & 0xFFFF), colp = (int)((kk >> 16) & 0xFFFF);
      const float err = sm.rerr[bw], d = sm.rd[bw];
      if (tid == 0) {
        sm.code[colp] = (uint8_t)sm.rcode[bw];
        sm.ord[n - R] = (uint16_t)colp;
        loss += (double)(err * err / d);
      }
      // The true H^-1 entry (p, j), and the base entries the swap moves.
      const bool mine = j < R && j != p;
      float tp = 0.f, tl = 0.f, rp = 0.f;
      if (mine) {
        tp = T[p > j ? tri(p) + j : tri(j) + p];
        tl = T[tri(last) + j];  // j == last: the base diagonal of the last position
        rp = tp;
        for (int t = 0; t < kd; ++t) rp -= sm.C[t][p] * sm.cdv[t] * sm.C[t][j];
      }
      __syncthreads();
      const float f = err / d;
      if (mine) {
        int code;
        if (j != last) {
          if (p != last) {
            T[p > j ? tri(p) + j : tri(j) + p] = tl;
            T[tri(last) + j] = tp;
          }
          sm.w[j] += f * rp;
          sm.dg[j] -= rp * rp / d;
          sm.C[kd][j] = rp;
          const float e = errf(j, code);
          sm.e2[j] = e * e;
        } else {  // position p takes over the last unquantized weight
          sm.w[p] = sm.w[last] + f * rp;
          sm.perm[p] = sm.perm[last];
          sm.gpos[p] = sm.gpos[last];
          sm.dg[p] = sm.dg[last] - rp * rp / d;
          T[tri(p) + p] = tl;
          for (int t = 0; t < kd; ++t) sm.C[t][p] = sm.C[t][last];
          sm.C[kd][p] = rp;
          const float e = errf(p, code);
          sm.e2[p] = e * e;
        }
      }
      if (tid == 0) sm.cdv[kd] = 1.f / d;
      __syncthreads();
      if (R == 1) break;
      const int Rr = last;
      ++kd;
      if (kd == KD) {
        // Fold the deferred columns into the base: lanes take columns, waves rows.
        for (int j0 = 0; j0 < Rr; j0 += 64) {
          const int jj = j0 + lane;
          const int jc = jj < Rr ? jj : 0;
          float cj[KD];
#pragma unroll
          for (int t = 0; t < KD; ++t) cj[t] = sm.C[t][jc] * sm.cdv[t];
#pragma unroll
          for (int ub = 0; ub < 64 / NW; ub += 4) {
            float tv[4];
            int ev[4], ic[4];
#pragma unroll
            for (int u = 0; u < 4; ++u) {
              const int ii = j0 + wv + (ub + u) * NW;
              const bool ok = ii < Rr;
              ic[u] = ok ? ii : 0;
              ev[u] = ok && jj <= ii ? tri(ii) + jj : spare;  // jj <= ii < Rr: inside the triangle
              tv[u] = T[ev[u]];
            }
#pragma unroll
            for (int u = 0; u < 4; ++u) {
              float v = tv[u];
#pragma unroll
              for (int t = 0; t < KD; ++t) v -= sm.C[t][ic[u]] * cj[t];
              T[ev[u]] = v;
            }
          }
          int i = j0 + 64 + wv;
          for (; i + (RB - 1) * NW < Rr; i += RB * NW) {
            float tv[RB];
            int ev[RB];
#pragma unroll
            for (int u = 0; u < RB; ++u) {
              ev[u] = tri(i + u * NW) + jj;
              tv[u] = T[ev[u]];
            }
#pragma unroll
            for (int u = 0; u < RB; ++u) {
              float v = tv[u];
#pragma unroll
              for (int t = 0; t < KD; ++t) v -= sm.C[t][i + u * NW] * cj[t];
              T[ev[u]] = v;
            }
          }
          for (; i < Rr; i += NW) {
            const int e = tri(i) + jj;
            float v = T[e];
#pragma unroll
            for (int t = 0; t < KD; ++t) v -= sm.C[t][i] * cj[t];
            T[e] = v;
          }
        }
        kd = 0;
      }
      // Scores for the next step from the kept diagonal.
      b.init();
      if (j < Rr) b.offer(score_bits(sm.e2[j], sm.dg[j]), sm.perm[j], j, sm.dg[j]);
      post_wave_best(sm, b, lane, wv, errf);
      __syncthreads();
    }

    for (int wd = tid; wd < a.words; wd += NT) {
      const int b0 = wd * 32;
      const int j0 = b0 / a.bits, j1 = min(n - 1, (b0 + 31) / a.bits);
      uint64_t acc = 0;
      for (int jj = j0; jj <= j1; ++jj) {
        const int off = jj * a.bits - b0;
        const uint64_t cv = sm.code[jj];
        acc |= off >= 0 ? (cv << off) : (cv >> -off);
      }
      a.Q[row * a.words + wd] = (uint32_t)acc;
    }
    if (a.order && j < n) a.order[row * n + j] = sm.ord[j];
    if (tid == 0 && a.loss) a.loss[row] = (float)loss;
    __syncthreads();
  }
}

template <int DT>
void launch_greedy(const GreedyArgs& a, hipStream_t st) {
  const int grid = (int)std::min<int64_t>(a.m, a.n <= NLB ? 65535 : GRID_G);
  if (a.n <= NS)
    hipLaunchKernelGGL((greedy_lazy_kernel<DT, 0>), dim3(grid), dim3(LVar<0>::NT), 0, st, a);
  else if (a.n <= NLB)
    hipLaunchKernelGGL((greedy_lazy_kernel<DT, 1>), dim3(grid), dim3(LVar<1>::NT), 0, st, a);
  else if (a.n <= NLZ)
    hipLaunchKernelGGL((greedy_lazy_kernel<DT, 2>), dim3(grid), dim3(LVar<2>::NT), 0, st, a);
  else
    hipLaunchKernelGGL((greedy_kernel<DT>), dim3(grid), dim3(1024), 0, st, a);
}

}  // namespace

bool greedy_supported(int64_t n, int64_t group) { return n <= NMAX && (group <= 0 || group >= GMIN); }

size_t greedy_workspace_bytes(int64_t m, int64_t n) {
  if (m < 1 || n < 1 || n > NMAX) return 0;
  const int64_t slices = n <= NLB ? 0 : std::min<int64_t>(m, GRID_G);
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
