// Hessian accumulation H += 2 X X^T on the CDNA4 matrix cores.
//
// The proxy Hessian of the layer objective ||WX - What X||^2 is 2 X X^T (the
// English GPTQ second-order quantization post, 'The objective is layer
// output, not weight distance').  X arrives token-major ([tokens x n]), so the
// contraction index (tokens) is the strided one: every 8x8 block of
// (token, feature) values is transposed in registers on its way into LDS, so
// each lane can feed the MFMA 8 consecutive tokens of one feature.
//
// Work decomposition: the lower triangle of H is cut into 256x256 tiles; each
// workgroup (256 threads, 4 wave64s of 128x128) accumulates one tile over one
// contiguous slice of tokens ("split"), with fp16/bf16 products exact in the
// fp32 accumulators of v_mfma_f32_32x32x16_{f16,bf16}.  Partial tiles go to
// the workspace; a second kernel sums the splits in a fixed order, scales by
// 2, adds to H and writes both triangles, so results are deterministic.
#include <algorithm>

#include "common.hpp"
#include "internal.hpp"

namespace gptq {

namespace {

constexpr int TILE = 256;
constexpr int KC16 = 64;   // tokens per LDS stage, 16-bit inputs
constexpr int KC32 = 16;   // tokens per LDS stage, fp32 inputs
constexpr int PITCH16 = KC16;      // halfs per feature row in LDS (128 B, 8 slots of 16 B)
constexpr int PITCH32 = TILE + 4;  // floats per token row in LDS
constexpr int NXCD = 8;            // MI355X: 8 XCDs, workgroups dealt round-robin
constexpr int SB_H = 8, SB_W = 4;  // tile regions of 8 x 4 tiles (share 12 feature blocks)

// LDS slot of 16-byte token group `slot` (0..7) in feature row `row`: XOR
// swizzled by row bits 0-2 (eight consecutive rows read by the MFMA fragment
// loads land on distinct banks) and bits 3-5 (the transposed stores of eight
// feature octets land on distinct banks).
__device__ __forceinline__ int swz(int row, int slot) { return slot ^ (row & 7) ^ ((row >> 3) & 7); }

__device__ __forceinline__ void tile_of(int t, int& bi, int& bj) {
  int r = (int)((sqrtf(8.f * (float)t + 1.f) - 1.f) * 0.5f);
  while ((r + 1) * (r + 2) / 2 <= t) ++r;
  while (r * (r + 1) / 2 > t) --r;
  bi = r;
  bj = t - r * (r + 1) / 2;
}

// The t-th lower tile when tiles are listed region by region (8 tile-rows by
// 4 tile-columns, each region row-major), so that consecutive tiles share
// feature blocks.
__device__ __forceinline__ void region_tile(int t, int nt1, int& bi, int& bj) {
  for (int si = 0; si * SB_H < nt1; ++si) {
    const int r0 = si * SB_H, r1 = min(nt1, r0 + SB_H);
    for (int sj = 0; sj * SB_W < r1; ++sj) {
      const int c0 = sj * SB_W;
      int cnt = 0;
      for (int r = r0; r < r1; ++r) cnt += max(0, min(r + 1, c0 + SB_W) - c0);
      if (t < cnt) {
        for (int r = r0; r < r1; ++r) {
          const int w = max(0, min(r + 1, c0 + SB_W) - c0);
          if (t < w) { bi = r; bj = c0 + t; return; }
          t -= w;
        }
      }
      t -= cnt;
    }
  }
  bi = bj = 0;
}

struct SyrkArgs {
  const void* X;
  int64_t ldx;
  int n;
  int64_t tokens;
  int ntiles;
  int nsplit;
  int64_t nchunks;
  int64_t per_xcd;  // work items per XCD (items = nsplit * ntiles, padded to a multiple of NXCD)
  float* partial;   // [nsplit][ntiles][256][256]
};

// Work item of this workgroup: XCD x (= blockIdx.x % 8) takes items
// [x * per_xcd, (x + 1) * per_xcd) in order, item = split * ntiles + region
// tile, so the workgroups resident on one XCD share token ranges and tiles.
__device__ __forceinline__ bool syrk_item(const SyrkArgs& a, int& split, int& tlin, int& bi, int& bj) {
  const int64_t item = (int64_t)(blockIdx.x % NXCD) * a.per_xcd + blockIdx.x / NXCD;
  if (item >= (int64_t)a.nsplit * a.ntiles) return false;
  split = (int)(item / a.ntiles);
  const int nt1 = (int)cdiv(a.n, TILE);
  region_tile((int)(item % a.ntiles), nt1, bi, bj);
  tlin = bi * (bi + 1) / 2 + bj;
  return true;
}

// ---------------------------------------------------------------------------- 16-bit inputs

template <int DT, bool VEC>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(1, 1)))
void syrk16_kernel(SyrkArgs a) {
  __shared__ __attribute__((aligned(16))) uint16_t lds[2][2][TILE * PITCH16];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wr = wave >> 1, wc = wave & 1;
  int split, tlin, bi, bj;
  if (!syrk_item(a, split, tlin, bi, bj)) return;
  const bool diag = (bi == bj);
  const int64_t cb = (int64_t)split * a.nchunks / a.nsplit;
  const int64_t ce = (int64_t)(split + 1) * a.nchunks / a.nsplit;
  const uint16_t* __restrict__ X = (const uint16_t*)a.X;

  // loader role: operand (0: rows bi, 1: rows bj), feature octet, token octet
  const int op = tid >> 7;
  const int fo = tid & 31;
  const int to = (tid >> 5) & 3;  // token octets to, to + 4 of the 64-token stage
  const int fbase = (op == 0 ? bi : bj) * TILE + fo * 8;
  const bool loader = !(diag && op == 1) && fbase < a.n;

  u32x4 rg[16];
  auto gload = [&](int64_t chunk) {
    const int64_t t0 = chunk * KC16;
    const bool full = t0 + KC16 <= a.tokens;
    if (VEC && full) {
      if (loader) {
#pragma unroll
        for (int e = 0; e < 16; ++e) {
          const int64_t t = t0 + (to + 4 * (e >> 3)) * 8 + (e & 7);
          rg[e] = *(const u32x4*)(X + t * a.ldx + fbase);
        }
      } else {
#pragma unroll
        for (int e = 0; e < 16; ++e) rg[e] = u32x4{0u, 0u, 0u, 0u};
      }
      return;
    }
#pragma unroll
    for (int e = 0; e < 16; ++e) {
      const int64_t t = t0 + (to + 4 * (e >> 3)) * 8 + (e & 7);
      u32x4 v = {0u, 0u, 0u, 0u};
      if (loader && t < a.tokens) {
        const uint16_t* p = X + t * a.ldx + fbase;
        if (VEC) {
          v = *(const u32x4*)p;
        } else {
          uint32_t h[8];
#pragma unroll
          for (int f = 0; f < 8; ++f) h[f] = (fbase + f < a.n) ? (uint32_t)p[f] : 0u;
          v = u32x4{h[0] | (h[1] << 16), h[2] | (h[3] << 16), h[4] | (h[5] << 16), h[6] | (h[7] << 16)};
        }
      }
      rg[e] = v;
    }
  };
  // 8x8 (token, feature) -> (feature, token) transposes, then 16-byte LDS stores
  auto lstore = [&](int buf) {
    if (diag && op == 1) return;
    uint16_t* T = lds[buf][op];
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const int slot = to + 4 * h;
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        uint32_t lo[4], hi[4];
#pragma unroll
        for (int d = 0; d < 4; ++d) {
          const uint32_t x0 = rg[8 * h + 2 * d][c], x1 = rg[8 * h + 2 * d + 1][c];
          lo[d] = (x0 & 0xFFFFu) | (x1 << 16);          // feature 2c, tokens 2d, 2d+1
          hi[d] = (x0 >> 16) | (x1 & 0xFFFF0000u);      // feature 2c+1
        }
        const int r0 = fo * 8 + 2 * c, r1 = r0 + 1;
        *(u32x4*)(T + r0 * PITCH16 + swz(r0, slot) * 8) = u32x4{lo[0], lo[1], lo[2], lo[3]};
        *(u32x4*)(T + r1 * PITCH16 + swz(r1, slot) * 8) = u32x4{hi[0], hi[1], hi[2], hi[3]};
      }
    }
  };

  f32x16 acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = zero16();

  if (cb < ce) {
    gload(cb);
    lstore(0);
    __syncthreads();
    int buf = 0;
    for (int64_t c = cb; c < ce; ++c) {
      const bool more = c + 1 < ce;
      if (more) gload(c + 1);
      const uint16_t* Ti = lds[buf][0];
      const uint16_t* Tj = diag ? lds[buf][0] : lds[buf][1];
#pragma unroll
      for (int ks = 0; ks < KC16 / 16; ++ks) {
        const int slot = ks * 2 + (lane >> 5);
        u32x4 av[4], bv[4];
#pragma unroll
        for (int mb = 0; mb < 4; ++mb) {
          const int row = wr * 128 + mb * 32 + (lane & 31);
          av[mb] = *(const u32x4*)(Ti + row * PITCH16 + swz(row, slot) * 8);
        }
#pragma unroll
        for (int nb = 0; nb < 4; ++nb) {
          const int row = wc * 128 + nb * 32 + (lane & 31);
          bv[nb] = *(const u32x4*)(Tj + row * PITCH16 + swz(row, slot) * 8);
        }
#pragma unroll
        for (int mb = 0; mb < 4; ++mb)
#pragma unroll
          for (int nb = 0; nb < 4; ++nb) {
            if (DT == 0)
              acc[mb][nb] = __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(half8, av[mb]),
                                                                  __builtin_bit_cast(half8, bv[nb]), acc[mb][nb], 0, 0, 0);
            else
              acc[mb][nb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, av[mb]),
                                                                   __builtin_bit_cast(bf16x8, bv[nb]), acc[mb][nb], 0, 0, 0);
          }
      }
      if (more) lstore(buf ^ 1);
      __syncthreads();
      buf ^= 1;
    }
  }

  float* out = a.partial + ((int64_t)split * a.ntiles + tlin) * (TILE * TILE);
#pragma unroll
  for (int mb = 0; mb < 4; ++mb)
#pragma unroll
    for (int nb = 0; nb < 4; ++nb)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int row = wr * 128 + mb * 32 + mfma32_row(r, lane);
        const int col = wc * 128 + nb * 32 + mfma32_col(lane);
        out[row * TILE + col] = acc[mb][nb][r];
      }
}

// ---------------------------------------------------------------------------- fp32 inputs

__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(1, 1)))
void syrk32_kernel(SyrkArgs a) {
  __shared__ float lds[2][2][KC32 * PITCH32];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wr = wave >> 1, wc = wave & 1;
  int split, tlin, bi, bj;
  if (!syrk_item(a, split, tlin, bi, bj)) return;
  const bool diag = (bi == bj);
  const int64_t cb = (int64_t)split * a.nchunks / a.nsplit;
  const int64_t ce = (int64_t)(split + 1) * a.nchunks / a.nsplit;
  const float* __restrict__ X = (const float*)a.X;

  float rg[2][KC32];
  auto gload = [&](int64_t chunk) {
#pragma unroll
    for (int op = 0; op < 2; ++op) {
      const int f = (op == 0 ? bi : bj) * TILE + tid;
#pragma unroll
      for (int kk = 0; kk < KC32; ++kk) {
        const int64_t t = chunk * KC32 + kk;
        rg[op][kk] = (f < a.n && t < a.tokens && !(diag && op == 1)) ? X[t * a.ldx + f] : 0.f;
      }
    }
  };
  auto lstore = [&](int buf) {
#pragma unroll
    for (int op = 0; op < 2; ++op)
#pragma unroll
      for (int kk = 0; kk < KC32; ++kk) lds[buf][op][kk * PITCH32 + tid] = rg[op][kk];
  };

  f32x16 acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = zero16();

  if (cb < ce) {
    gload(cb);
    lstore(0);
    __syncthreads();
    int buf = 0;
    for (int64_t c = cb; c < ce; ++c) {
      const bool more = c + 1 < ce;
      if (more) gload(c + 1);
      const float* Xi = lds[buf][0];
      const float* Xj = diag ? lds[buf][0] : lds[buf][1];
#pragma unroll
      for (int kk = 0; kk < KC32; kk += 2) {
        const int k = kk + (lane >> 5);
        float av[4], bv[4];
#pragma unroll
        for (int mb = 0; mb < 4; ++mb) av[mb] = Xi[k * PITCH32 + wr * 128 + mb * 32 + (lane & 31)];
#pragma unroll
        for (int nb = 0; nb < 4; ++nb) bv[nb] = Xj[k * PITCH32 + wc * 128 + nb * 32 + (lane & 31)];
#pragma unroll
        for (int mb = 0; mb < 4; ++mb)
#pragma unroll
          for (int nb = 0; nb < 4; ++nb)
            acc[mb][nb] = __builtin_amdgcn_mfma_f32_32x32x2f32(av[mb], bv[nb], acc[mb][nb], 0, 0, 0);
      }
      if (more) lstore(buf ^ 1);
      __syncthreads();
      buf ^= 1;
    }
  }

  float* out = a.partial + ((int64_t)split * a.ntiles + tlin) * (TILE * TILE);
#pragma unroll
  for (int mb = 0; mb < 4; ++mb)
#pragma unroll
    for (int nb = 0; nb < 4; ++nb)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int row = wr * 128 + mb * 32 + mfma32_row(r, lane);
        const int col = wc * 128 + nb * 32 + mfma32_col(lane);
        out[row * TILE + col] = acc[mb][nb][r];
      }
}

// ---------------------------------------------------------------------------- split reduction + mirror

// One workgroup per 64x64 sub-block of a lower tile: H <- H + 2 * sum_s P_s,
// written to both triangles (the upper one through an LDS transpose).
__global__ __launch_bounds__(256) void syrk_reduce_kernel(float* H, int n, const float* partial, int ntiles,
                                                          int nsplit) {
  __shared__ float t[64][65];
  const int tile = blockIdx.x;
  const int sub = blockIdx.y;  // 0..15
  const int sr = sub >> 2, sc = sub & 3;
  int bi, bj;
  tile_of(tile, bi, bj);
  const bool diag = (bi == bj);
  const int tid = threadIdx.x;
  const int c = tid & 63;
#pragma unroll 4
  for (int u = 0; u < 16; ++u) {
    const int r = (tid >> 6) + 4 * u;
    const int li = sr * 64 + r, lj = sc * 64 + c;
    const int gi = bi * TILE + li, gj = bj * TILE + lj;
    float sum = 0.f;
    for (int s = 0; s < nsplit; ++s) sum += partial[((int64_t)s * ntiles + tile) * (TILE * TILE) + li * TILE + lj];
    float h = 0.f;
    if (gi < n && gj < n && (!diag || gi >= gj)) {
      float* p = H + (int64_t)gi * n + gj;
      h = *p + 2.f * sum;
      *p = h;
      if (diag && gi != gj) H[(int64_t)gj * n + gi] = h;
    }
    t[r][c] = h;
  }
  if (diag) return;  // uniform per block
  __syncthreads();
#pragma unroll 4
  for (int u = 0; u < 16; ++u) {
    const int r = (tid >> 6) + 4 * u;  // row of the mirrored block = column of the lower block
    const int gi = bj * TILE + sc * 64 + r;
    const int gj = bi * TILE + sr * 64 + c;
    if (gi < n && gj < n) H[(int64_t)gi * n + gj] = t[c][r];
  }
}

int syrk_splits(int64_t n, int64_t tokens, int kc, int& ntiles, int64_t& nchunks) {
  const int64_t nt1 = cdiv(n, TILE);
  ntiles = (int)(nt1 * (nt1 + 1) / 2);
  nchunks = cdiv(tokens, kc);
  // about 8 rounds of 256 workgroups, each split at least 4 stages long
  int64_t s = 2048 / ntiles;
  s = std::min<int64_t>(s, nchunks / 4);
  if (s < 1) s = 1;
  if (s > 64) s = 64;
  return (int)s;
}

}  // namespace

size_t syrk_workspace_bytes(int64_t n, int64_t tokens, int dtype) {
  if (n < 1 || tokens < 1) return 0;
  int ntiles;
  int64_t nchunks;
  const int s = syrk_splits(n, tokens, dtype == 2 ? KC32 : KC16, ntiles, nchunks);
  return (size_t)s * (size_t)ntiles * TILE * TILE * sizeof(float);
}

hipError_t syrk_accumulate(float* H, int64_t n, const void* X, int dtype, int64_t tokens, int64_t ldx, void* ws,
                           hipStream_t stream) {
  int ntiles;
  int64_t nchunks;
  const int kc = dtype == 2 ? KC32 : KC16;
  const int s = syrk_splits(n, tokens, kc, ntiles, nchunks);
  const int64_t items = (int64_t)s * ntiles;
  const int64_t per_xcd = cdiv(items, NXCD);
  SyrkArgs a{X, ldx, (int)n, tokens, ntiles, s, nchunks, per_xcd, (float*)ws};
  dim3 grid((unsigned)(per_xcd * NXCD));
  if (dtype == 2) {
    hipLaunchKernelGGL(syrk32_kernel, grid, dim3(256), 0, stream, a);
  } else {
    const bool vec = (n % 8 == 0) && (ldx % 8 == 0) && (((uintptr_t)X & 15) == 0);
    if (dtype == 0) {
      if (vec) hipLaunchKernelGGL((syrk16_kernel<0, true>), grid, dim3(256), 0, stream, a);
      else hipLaunchKernelGGL((syrk16_kernel<0, false>), grid, dim3(256), 0, stream, a);
    } else {
      if (vec) hipLaunchKernelGGL((syrk16_kernel<1, true>), grid, dim3(256), 0, stream, a);
      else hipLaunchKernelGGL((syrk16_kernel<1, false>), grid, dim3(256), 0, stream, a);
    }
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(syrk_reduce_kernel, dim3((unsigned)ntiles, 16), dim3(256), 0, stream, H, (int)n,
                     (const float*)ws, ntiles, s);
  return hipGetLastError();
}

}  // namespace gptq
