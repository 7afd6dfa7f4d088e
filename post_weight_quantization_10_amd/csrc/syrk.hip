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

// ---------------------------------------------------------------------------- 16-bit inputs, DMA path
//
// Same tiles and work order as above, but X moves global -> LDS with
// buffer_load_dwordx4 ... lds (no VGPR staging) through a ring of NSTAGE = 5
// 32-token stages (all 160 KiB of LDS): three stages in flight while one is
// consumed.  LDS keeps
// X token-major (as in HBM): per stage and operand, 32 token rows of 512 B,
// the 16-byte chunks of row t XOR-swizzled by h(t & 3) = {0, 6, 10, 12},
// which keeps every fragment read bank-conflict-free whether the LDS serves
// 16 lanes x 8 B or 32 lanes x 8 B per cycle.  MFMA operands are
// read with ds_read_b64_tr_b16: within a 16-lane group, source lane j points
// at [token t0 + j/4][features F + 4*(j%4)], and lane i receives feature F+i
// for tokens t0..t0+3, i.e. the K-contiguous fragment the MFMA wants.
// Tokens past the end of X read as zero (buffer bounds); features past n only
// reach outputs that are never written.

constexpr int DKC = 32;                        // tokens per stage
constexpr int NSTAGE = 5;
constexpr int OPB = DKC * TILE * 2;            // bytes per operand per stage (16 KiB)
constexpr int STB = 2 * OPB;                   // bytes per stage

typedef __fp16 fp16x4_t __attribute__((__vector_size__(4 * sizeof(__fp16))));
typedef __bf16 bf16x4_t __attribute__((__vector_size__(4 * sizeof(__bf16))));

template <int DT>
__device__ __forceinline__ uint2 tr_read(const char LDS_AS* p) {
  if (DT == 0) {
    fp16x4_t v = __builtin_amdgcn_ds_read_tr16_b64_v4f16((fp16x4_t LDS_AS*)p);
    return __builtin_bit_cast(uint2, v);
  } else {
    bf16x4_t v = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((bf16x4_t LDS_AS*)p);
    return __builtin_bit_cast(uint2, v);
  }
}

__device__ __forceinline__ int dswz(int r) { return (0xCA60 >> (4 * (r & 3))) & 0xF; }  // {0, 6, 10, 12}

// Fragment read order within one K16 step, matched to the order in which the
// MFMAs (mb-major over the 4 x 4 block grid) consume them: A0, B0..B3, A1..A3,
// each as its two 4-token halves.
__device__ __forceinline__ constexpr int rd_isb(int i) { return (i >= 2 && i < 10) ? 1 : 0; }
__device__ __forceinline__ constexpr int rd_blk(int i) { return i < 2 ? 0 : (i < 10 ? (i - 2) >> 1 : 1 + ((i - 10) >> 1)); }
__device__ __forceinline__ constexpr int rd_half(int i) { return i & 1; }

// IDLE: the wave of a diagonal tile whose 128 x 128 block lies strictly above
// the diagonal (never read by the reduction): it takes its share of the ring
// refills and every barrier, and reads and multiplies nothing.
template <int DT, bool DIAG, bool IDLE>
__device__ __forceinline__ void syrk16_dma_body(const SyrkArgs& a, int split, int tlin, int bi, int bj, char* st0,
                                                char* st1, char* st2, char* st3, char* st4) {
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wr = wave >> 1, wc = wave & 1;
  const int64_t cb = (int64_t)split * a.nchunks / a.nsplit;
  const int64_t ce = (int64_t)(split + 1) * a.nchunks / a.nsplit;
  const uint16_t* X = (const uint16_t*)a.X;
  const int64_t row_bytes = a.ldx * 2;

  // This lane's share of one stage: for each operand, 4 copies of 1 KiB (two
  // token rows each).  The byte offset within the stage's rows and the LDS
  // destination are fixed per lane and copy; only the buffer base moves.
  int voff[2][4];
#pragma unroll
  for (int op = 0; op < 2; ++op)
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int fb = (op == 0 ? bi : bj) * TILE;
      const int r = 2 * (4 * wave + q) + (lane >> 5);  // token row within the stage
      const int c = (lane & 31) ^ dswz(r);             // logical 16-byte chunk held at this lane's slot
      voff[op][q] = (int)(r * row_bytes) + (fb + 8 * c) * 2;
    }
  auto rsrc_of = [&](int64_t chunk) {
    const int64_t t0 = chunk * DKC;
    const int64_t rows = min<int64_t>(DKC, a.tokens - t0);
    return make_rsrc(X + t0 * a.ldx, (uint32_t)(rows * row_bytes));
  };
  auto dma1 = [&](const i32x4& rs, char* stage, int k) {  // copy k of 8 (4 if DIAG)
    const int op = k >> 2, q = k & 3;
    const uint32_t sbase = (uint32_t)(uintptr_t)((char LDS_AS*)stage);
    dma16(rs, sbase + op * OPB + (2 * (4 * wave + q)) * 512, voff[op][q]);
  };
  constexpr int NCOPY = DIAG ? 4 : 8;
  auto issue = [&](int64_t chunk, char* stage) {
    const i32x4 rs = rsrc_of(chunk);
#pragma unroll
    for (int k = 0; k < NCOPY; ++k) dma1(rs, stage, k);
  };

  f32x16 acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = zero16();

  // fragment addressing (see the comment above)
  const int g = lane >> 4, j16 = lane & 15;
  const int fa = wr * 128 + 16 * (g & 1) + 4 * (j16 & 3);   // + mb * 32
  const int fbb = wc * 128 + 16 * (g & 1) + 4 * (j16 & 3);  // + nb * 32
  const int trow = 8 * (g >> 1) + (j16 >> 2);               // + 16 * ks (+ 4 for the upper half)

  struct Frag {
    uint4 a[4], b[4];
  };
  // read i (0..15) of the K16 step ks of stage st into F
  auto rd1 = [&](const char* st, int ks, Frag& F, int i) {
    if constexpr (IDLE) return;
    const int isb = rd_isb(i), blk = rd_blk(i), h = rd_half(i);
    const char* T = (isb && !DIAG) ? st + OPB : st;
    const int r = 16 * ks + trow + 4 * h;
    const int f = (isb ? fbb : fa) + blk * 32;
    const uint2 x = tr_read<DT>((const char LDS_AS*)(T + r * 512 + (((f >> 3) ^ dswz(r)) << 4) + ((f & 4) << 1)));
    uint4& d = isb ? F.b[blk] : F.a[blk];
    if (h == 0) { d.x = x.x; d.y = x.y; } else { d.z = x.x; d.w = x.y; }
  };
  auto rd = [&](const char* st, int ks, Frag& F) {
#pragma unroll
    for (int i = 0; i < 16; ++i) rd1(st, ks, F, i);
  };
  auto mfma1 = [&](const Frag& F, int i) {
    if constexpr (IDLE) return;
    const int mb = i >> 2, nb = i & 3;
    if (DT == 0)
      acc[mb][nb] = __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(half8, F.a[mb]),
                                                          __builtin_bit_cast(half8, F.b[nb]), acc[mb][nb], 0, 0, 0);
    else
      acc[mb][nb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, F.a[mb]),
                                                           __builtin_bit_cast(bf16x8, F.b[nb]), acc[mb][nb], 0, 0, 0);
  };
  auto mma = [&](const Frag& F) {
#pragma unroll
    for (int i = 0; i < 16; ++i) mfma1(F, i);
  };
  // wait until this wave's copies of the oldest stage in flight have landed,
  // `ahead` later stages still in flight
  auto wait_stage = [&](int64_t ahead) {
    if (DIAG) {
      if (ahead >= 3) wait_vmcnt<12>(); else if (ahead == 2) wait_vmcnt<8>(); else if (ahead == 1) wait_vmcnt<4>();
      else wait_vmcnt<0>();
    } else {
      if (ahead >= 3) wait_vmcnt<24>(); else if (ahead == 2) wait_vmcnt<16>(); else if (ahead == 1) wait_vmcnt<8>();
      else wait_vmcnt<0>();
    }
  };

  // Software pipeline over stages (two K16 steps each).  The barrier that
  // publishes stage c+1 sits between the two MFMA batches of stage c.  In the
  // steady state every LDS fragment read is issued between two MFMAs (the
  // second half of stage c is read under the first half's MFMAs, the first
  // half of stage c+1 under the second half's), so with one wave per SIMD the
  // read latency stays hidden behind the matrix pipe; the copies that refill
  // the ring go out between the MFMAs of the second half.
  Frag F0, F1;
  auto step_ss = [&](int64_t c, const char* cur, const char* nx, char* fill) {
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      mfma1(F0, i);
      rd1(cur, 1, F1, i);
    }
    if constexpr (!IDLE) {
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // one MFMA
        __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);  // one LDS read
      }
    }
    wait_stage(2);
    stage_barrier();  // stage c+1 visible; stage c-1 no longer read by anyone
    const i32x4 rs = rsrc_of(c + NSTAGE - 1);
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      mfma1(F1, i);
      rd1(nx, 0, F0, i);
      if ((i & 1) && (i >> 1) < NCOPY) dma1(rs, fill, i >> 1);
    }
    if constexpr (!IDLE) {
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
        __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
      }
    }
  };
  // general step (pipeline fill and drain)
  auto step = [&](int64_t c, const char* cur, const char* nx, char* fill) {
    mma(F0);
    rd(cur, 1, F1);
    if (c + 1 < ce) {
      wait_stage(min<int64_t>(2, ce - 2 - c));
      stage_barrier();
      if (c + NSTAGE - 1 < ce) issue(c + NSTAGE - 1, fill);
    }
    mma(F1);
    if (c + 1 < ce) rd(nx, 0, F0);
  };

  if (cb < ce) {
    issue(cb, st0);
    if (cb + 1 < ce) issue(cb + 1, st1);
    if (cb + 2 < ce) issue(cb + 2, st2);
    if (cb + 3 < ce) issue(cb + 3, st3);
    wait_stage(min<int64_t>(3, ce - 1 - cb));
    stage_barrier();
    rd(st0, 0, F0);
  }
  int64_t c = cb;
  // steady state: all five steps of a ring turn refill (c + 8 < ce)
  for (; c + 2 * NSTAGE - 2 < ce; c += NSTAGE) {
    step_ss(c, st0, st1, st4);
    step_ss(c + 1, st1, st2, st0);
    step_ss(c + 2, st2, st3, st1);
    step_ss(c + 3, st3, st4, st2);
    step_ss(c + 4, st4, st0, st3);
  }
  for (; c < ce; c += NSTAGE) {
    step(c, st0, st1, st4);
    if (c + 1 < ce) step(c + 1, st1, st2, st0);
    if (c + 2 < ce) step(c + 2, st2, st3, st1);
    if (c + 3 < ce) step(c + 3, st3, st4, st2);
    if (c + 4 < ce) step(c + 4, st4, st0, st3);
  }

  if constexpr (IDLE) return;
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

template <int DT>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(1, 1)))
void syrk16_dma_kernel(SyrkArgs a) {
  // one LDS object per stage, so the compiler can tell the stage being read
  // from the stages the DMA is still writing
  __shared__ __attribute__((aligned(1024))) char st0[STB];
  __shared__ __attribute__((aligned(1024))) char st1[STB];
  __shared__ __attribute__((aligned(1024))) char st2[STB];
  __shared__ __attribute__((aligned(1024))) char st3[STB];
  __shared__ __attribute__((aligned(1024))) char st4[STB];
  int split, tlin, bi, bj;
  if (!syrk_item(a, split, tlin, bi, bj)) return;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  if (bi != bj) syrk16_dma_body<DT, false, false>(a, split, tlin, bi, bj, st0, st1, st2, st3, st4);
  else if (wave == 1) syrk16_dma_body<DT, true, true>(a, split, tlin, bi, bj, st0, st1, st2, st3, st4);
  else syrk16_dma_body<DT, true, false>(a, split, tlin, bi, bj, st0, st1, st2, st3, st4);
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
// written to both triangles (the upper one through an LDS transpose).  Each
// thread owns 4 rows x 4 columns and sums the splits in split order, with
// 16-byte loads of four splits in flight per row (16 per thread).
__global__ __launch_bounds__(256) void syrk_reduce_kernel(float* H, int n, const float* partial, int ntiles,
                                                          int nsplit) {
  __shared__ float t[64][65];
  const int tile = blockIdx.x;
  const int sub = blockIdx.y;  // 0..15
  const int sr = sub >> 2, sc = sub & 3;
  int bi, bj;
  tile_of(tile, bi, bj);
  const bool diag = (bi == bj);
  if (diag && sc > sr) return;  // the diagonal tile's upper half mirrors its lower half
  const int tid = threadIdx.x;
  const int c4 = (tid & 15) * 4, r16 = tid >> 4;
  const int64_t pstride = (int64_t)ntiles * (TILE * TILE);
  const float* P = partial + (int64_t)tile * (TILE * TILE) + (sr * 64 + r16) * TILE + sc * 64 + c4;
  f32x4 sum[4];
#pragma unroll
  for (int u = 0; u < 4; ++u) sum[u] = f32x4{0.f, 0.f, 0.f, 0.f};
  int s = 0;
  for (; s + 4 <= nsplit; s += 4) {
    f32x4 p[4][4];
#pragma unroll
    for (int v = 0; v < 4; ++v)
#pragma unroll
      for (int u = 0; u < 4; ++u) p[v][u] = *(const f32x4*)(P + (s + v) * pstride + 16 * u * TILE);
#pragma unroll
    for (int v = 0; v < 4; ++v)
#pragma unroll
      for (int u = 0; u < 4; ++u) sum[u] += p[v][u];
  }
  for (; s < nsplit; ++s)
#pragma unroll
    for (int u = 0; u < 4; ++u) sum[u] += *(const f32x4*)(P + s * pstride + 16 * u * TILE);
#pragma unroll
  for (int u = 0; u < 4; ++u) {
    const int r = r16 + 16 * u;
    const int gi = bi * TILE + sr * 64 + r;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int gj = bj * TILE + sc * 64 + c4 + e;
      float h = 0.f;
      if (gi < n && gj < n && (!diag || gi >= gj)) {
        float* ph = H + (int64_t)gi * n + gj;
        h = *ph + 2.f * sum[u][e];
        *ph = h;
        if (diag && gi != gj) H[(int64_t)gj * n + gi] = h;
      }
      t[r][c4 + e] = h;
    }
  }
  if (diag) return;  // uniform per block
  __syncthreads();
  const int c = tid & 63;
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
  // the smallest stage size gives the most splits, so this bounds every path
  const int s = syrk_splits(n, tokens, dtype == 2 ? KC32 : DKC, ntiles, nchunks);
  return (size_t)s * (size_t)ntiles * TILE * TILE * sizeof(float);
}

hipError_t syrk_accumulate(float* H, int64_t n, const void* X, int dtype, int64_t tokens, int64_t ldx, void* ws,
                           hipStream_t stream) {
  int ntiles;
  int64_t nchunks;
  const bool vec = dtype != 2 && (n % 8 == 0) && (ldx % 8 == 0) && (((uintptr_t)X & 15) == 0);
  const int kc = dtype == 2 ? KC32 : (vec ? DKC : KC16);
  const int s = syrk_splits(n, tokens, kc, ntiles, nchunks);
  const int64_t items = (int64_t)s * ntiles;
  const int64_t per_xcd = cdiv(items, NXCD);
  SyrkArgs a{X, ldx, (int)n, tokens, ntiles, s, nchunks, per_xcd, (float*)ws};
  dim3 grid((unsigned)(per_xcd * NXCD));
  if (dtype == 2) hipLaunchKernelGGL(syrk32_kernel, grid, dim3(256), 0, stream, a);
  else if (vec && dtype == 0) hipLaunchKernelGGL((syrk16_dma_kernel<0>), grid, dim3(256), 0, stream, a);
  else if (vec) hipLaunchKernelGGL((syrk16_dma_kernel<1>), grid, dim3(256), 0, stream, a);
  else if (dtype == 0) hipLaunchKernelGGL((syrk16_kernel<0, false>), grid, dim3(256), 0, stream, a);
  else hipLaunchKernelGGL((syrk16_kernel<1, false>), grid, dim3(256), 0, stream, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(syrk_reduce_kernel, dim3((unsigned)ntiles, 16), dim3(256), 0, stream, H, (int)n,
                     (const float*)ws, ntiles, s);
  return hipGetLastError();
}

}  // namespace gptq
