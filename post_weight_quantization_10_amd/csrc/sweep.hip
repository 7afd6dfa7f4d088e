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
#include <utility>

#include "common.hpp"
#include "internal.hpp"

namespace gptq {

namespace {

constexpr int BMAX = 128;  // widest block
constexpr int LA = 2;          // blocks per lazy flush on the look-ahead path
constexpr int SBW = 8 * BMAX;  // columns per superblock of the look-ahead path's two-level flush
constexpr int ELD = SBW;       // leading dimension of the E buffer: the errors of one superblock

// Layout of a block's factor rows for the sweep kernel.  Lane lr (of the LPR
// lanes that share a weight row) holds the block columns c = lr + LPR j,
// j = 0..7, in register j, so step p (column p) changes only registers
// j >= J = p / LPR: the columns left of p are final.  Row p of the factor
// block (divided by its diagonal, zero on and left of it) keeps just those
// registers, cut into the segments one load each reads (4, 2 or 1 floats:
// registers 0-3 / 4-7 as float4 where all four are needed, else the pairs and
// singles that remain), every segment stored as LPR consecutive vectors (lane
// lr's at lr * len): the LPR lanes of a row read consecutive bytes
// (bank-conflict-free, the same addresses for every row of the wave), and no
// load brings a register the step does not use.
template <int LPR>
struct BlockLayout {
  static constexpr int NSTEP = 8 * LPR;           // columns per block
  static constexpr int USZ = 36 * LPR * LPR;      // floats: sum over rows of LPR (8 - J)
  static constexpr int STRIDE = USZ + NSTEP;      // per block in the workspace: the rows, then 1/U_pp
  // segments of a row with first live register J: (first register, length)
  static constexpr int NSEG[8] = {2, 3, 2, 2, 1, 2, 1, 1};
  static constexpr int SEG[8][3][2] = {{{0, 4}, {4, 4}, {0, 0}}, {{1, 1}, {2, 2}, {4, 4}}, {{2, 2}, {4, 4}, {0, 0}},
                                       {{3, 1}, {4, 4}, {0, 0}}, {{4, 4}, {0, 0}, {0, 0}}, {{5, 1}, {6, 2}, {0, 0}},
                                       {{6, 2}, {0, 0}, {0, 0}}, {{7, 1}, {0, 0}, {0, 0}}};
  __host__ __device__ static constexpr int row_off(int p) {
    const int K = p / LPR, t = p % LPR;
    return LPR * (LPR * (8 * K - K * (K - 1) / 2) + t * (8 - K));
  }
  // offset of segment s of row p (lane 0)
  __host__ __device__ static constexpr int seg_off(int p, int s) {
    const int J = p / LPR;
    int o = row_off(p);
    for (int k = 0; k < s; ++k) o += LPR * SEG[J][k][1];
    return o;
  }
};

struct SweepArgs {
  const float* U;
  float* V;
  int64_t n, m;
  int64_t i;  // first column of the block
  int w;      // block width (<= 128)
  int maxq;
  int64_t group;  // group size (<= 0: per row)
  int64_t G;
  float* S;
  int32_t* Z;
  uint8_t* Q8;    // [m x n] codes, or null when the codes are packed here
  uint32_t* Qw;   // packed codes [m x words] (bit-streams), or null
  int64_t words;  // uint32 words per row of Qw
  int bits;
  void* Wout;     // dequantized weights written here (W's dtype), or null
  int wdt;
  int64_t ldw;
  float* E;       // scaled errors of this block (leading dimension ELD)
  float* err_sq;  // [m] or null
  const float* Dblk;  // this block's factor rows in BlockLayout order, then 1/U_pp [NSTEP]
  // look-ahead: errors of the kpend columns swept since the last flush
  // (E buffer from column 0) and the factor rows of those columns restricted
  // to this block's columns (U + r * n + i, leading dimension n)
  const float* Ep;
  int kpend;
  const float* Upend;
  // superblock launches: nblk consecutive blocks of width w (the last one
  // wlast wide) swept by one launch, each first taking the errors of the
  // launch's earlier blocks (Upend: the factor rows from the launch's first
  // column, at this block's columns)
  int nblk;
  int wlast;
  // flushes as three bf16 products: the errors as E_hi, E_lo bf16 in two
  // segments SBW apart per row (leading dimension 2 SBW), at this
  // block's column of its superblock (superblock launches: at the
  // superblock's first column, and written instead of E); null otherwise
  uint16_t* Ecat;
};

// Lanes-per-row variants: 16 lanes (one DPP row) x 8 columns = 128 columns,
// or 4 lanes (one DPP quad) x 8 columns = 32 columns.
template <int LPR>
struct RowOps;
template <>
struct RowOps<16> {
  template <int SRC>
  __device__ __forceinline__ static float bcast(float v) {
    return __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, v), 0x150 + SRC, 0xF, 0xF, false));
  }
  __device__ __forceinline__ static float rmin(float v) { return row_min16(v); }
  __device__ __forceinline__ static float rmax(float v) { return row_max16(v); }
  __device__ __forceinline__ static float rsum(float v) {
    v += __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, v), 0xB1, 0xF, 0xF, false));
    v += __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, v), 0x4E, 0xF, 0xF, false));
    v += __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, v), 0x124, 0xF, 0xF, false));
    return v + __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, v), 0x128, 0xF, 0xF, false));
  }
};
template <>
struct RowOps<4> {
  template <int SRC>
  __device__ __forceinline__ static float bcast(float v) {
    return __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, v),
                                                              SRC | (SRC << 2) | (SRC << 4) | (SRC << 6), 0xF, 0xF, false));
  }
  __device__ __forceinline__ static float rmin(float v) {
    v = fminf(v, __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, v), 0xB1, 0xF, 0xF, false)));
    return fminf(v, __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, v), 0x4E, 0xF, 0xF, false)));
  }
  __device__ __forceinline__ static float rmax(float v) {
    v = fmaxf(v, __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, v), 0xB1, 0xF, 0xF, false)));
    return fmaxf(v, __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, v), 0x4E, 0xF, 0xF, false)));
  }
  __device__ __forceinline__ static float rsum(float v) {
    v += __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, v), 0xB1, 0xF, 0xF, false));
    return v + __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, v), 0x4E, 0xF, 0xF, false));
  }
};

struct GroupState {
  float s, inv_s, nz, mz;  // scale, 1/scale, -z, maxq - z
  float z;
};

__device__ __forceinline__ GroupState make_group(float s, float z, int maxq) {
  GroupState g;
  g.s = s;
  g.z = z;
  g.inv_s = 1.f / s;
  g.nz = -z;
  g.mz = (float)maxq - z;
  return g;
}

// (s, z) of block columns [c0, c1) of the row: this lane's values there
// (column of register k: lr + LPR k), reduced over the row's lanes.
template <int LPR>
__device__ __forceinline__ GroupState group_params(const float (&v)[8], int lr, int c0, int c1, int maxq) {
  float lo = INFINITY, hi = -INFINITY;
#pragma unroll
  for (int k = 0; k < 8; ++k) {
    const int c = lr + LPR * k;
    const bool in = c >= c0 && c < c1;
    lo = fminf(lo, in ? v[k] : INFINITY);
    hi = fmaxf(hi, in ? v[k] : -INFINITY);
  }
  lo = RowOps<LPR>::rmin(lo);
  hi = RowOps<LPR>::rmax(hi);
  float s, z;
  qparams(lo, hi, maxq, s, z);
  return make_group(s, z, maxq);
}

template <int LPR>
__device__ __attribute__((noinline)) GroupState group_params_call(float v0, float v1, float v2, float v3, float v4,
                                                                  float v5, float v6, float v7, int lr, int c0, int c1,
                                                                  int maxq) {
  const float v[8] = {v0, v1, v2, v3, v4, v5, v6, v7};
  return group_params<LPR>(v, lr, c0, c1, maxq);
}

__device__ __forceinline__ void store_params(const SweepArgs& a, const GroupState& g, int64_t r, int64_t col,
                                             bool writer) {
  if (writer) {
    const int64_t gi = col / a.group;
    a.S[r * a.G + gi] = g.s;
    a.Z[r * a.G + gi] = (int32_t)g.z;
  }
}

// The errors of the pending columns (swept since the last flush) applied to
// this block's 128 columns for the workgroup's 16 rows, with
// v_mfma_f32_16x16x4f32: wave w computes output column blocks 2w, 2w+1.  The
// sum over the KP pending columns is taken in an order that gives every lane
// contiguous errors: at MFMA step t, lane quarter g takes k = (KP / 4) g + t.
// Every operand is loaded straight from global memory (the errors as float4
// runs, the factor rows one float per lane, 16 lanes per 64-byte row piece),
// all of them before the first MFMA, so the workgroup waits for one round of
// loads.  The result lands in `upd` (16 x 132 in LDS).
constexpr int UPITCH = BMAX + 4;
template <int KP>
__device__ __forceinline__ void pending_update(const SweepArgs& a, int64_t r0, float* upd) {
  constexpr int K4 = KP / 4;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int l16 = lane & 15, g16 = lane >> 4;
  const int64_t erow = min<int64_t>(r0 + l16, a.m - 1);  // rows past m: results never used
  const f32x4* __restrict__ ep = (const f32x4*)(a.Ep + erow * ELD + K4 * g16);
  f32x4 ev[K4 / 4];
#pragma unroll
  for (int u = 0; u < K4 / 4; ++u) ev[u] = ep[u];
  // w is a multiple of 4 on this path, so a column block is either inside the block or past it
  float bv[2][K4];
#pragma unroll
  for (int q = 0; q < 2; ++q) {
    const int col = 16 * (2 * wave + q) + l16;
    const bool in = col < a.w;
    const float* __restrict__ up = a.Upend + (int64_t)(K4 * g16) * a.n + (in ? col : 0);
#pragma unroll
    for (int t = 0; t < K4; ++t) bv[q][t] = up[(int64_t)t * a.n];
    if (!in) {
#pragma unroll
      for (int t = 0; t < K4; ++t) bv[q][t] = 0.f;
    }
  }
  f32x4 acc[2] = {{0.f, 0.f, 0.f, 0.f}, {0.f, 0.f, 0.f, 0.f}};
#pragma unroll
  for (int t = 0; t < K4; ++t) {
    const float av = ev[t / 4][t % 4];
#pragma unroll
    for (int q = 0; q < 2; ++q) acc[q] = __builtin_amdgcn_mfma_f32_16x16x4f32(av, bv[q][t], acc[q], 0, 0, 0);
  }
#pragma unroll
  for (int q = 0; q < 2; ++q)
#pragma unroll
    for (int rr = 0; rr < 4; ++rr) upd[(4 * g16 + rr) * UPITCH + 16 * (2 * wave + q) + l16] = acc[q][rr];
  __syncthreads();  // upd complete
}

// Inside a superblock launch the pending updates run on four waves of their
// own (waves 4..7 of a 512-thread workgroup) while waves 0..3 sweep: wave
// 4 + w accumulates output column blocks 2w, 2w + 1 of
//   acc += E[:, k0 : k0 + 64 nch] U[s0 + k0 .., ib + (0..wblk)]
// for the workgroup's 16 rows, the errors from LDS (Elds, pitch ELP), the
// factor rows from global memory in chunks of 64 rows with the next chunk's
// loads in flight while the current chunk's 32 MFMAs run.  Inside a chunk,
// lane quarter g takes k = 64 c + 16 g + t at step t.
constexpr int ELP = SBW + 4;
struct PendingOps {
  const float* Elds;
  const float* ubase;  // factor row a.i + k0, column ib
  int64_t n;
  int k0;
  uint32_t loff[2];    // per-lane byte offsets: the lane's k quarter and column
  int l16, g16;
  // per-lane offsets from a row pointer that is the same for the whole wave,
  // so the loads take a scalar base and one 32-bit offset register each
  __device__ __forceinline__ PendingOps(const SweepArgs& a, const float* E_, int k0_, int64_t ib, int wblk)
      : Elds(E_), ubase(a.U + (a.i + k0_) * a.n + ib), n(a.n), k0(k0_) {
    const int lane = threadIdx.x & 63, wq = (threadIdx.x >> 6) - 4;
    l16 = lane & 15;
    g16 = lane >> 4;
#pragma unroll
    for (int q = 0; q < 2; ++q) {
      const int col = 16 * (2 * wq + q) + l16;
      loff[q] = (uint32_t)((16 * g16 * n + (col < wblk ? col : 0)) * 4);  // past the block: computed, never read
    }
  }
  __device__ __forceinline__ void load(int c, float (&u)[2][16]) const {
#pragma unroll
    for (int t = 0; t < 16; ++t) {
      const char* __restrict__ row = (const char*)(ubase + (int64_t)(64 * c + t) * n);
#pragma unroll
      for (int q = 0; q < 2; ++q) u[q][t] = *(const float*)(row + loff[q]);
    }
  }
  __device__ __forceinline__ void mul(int c, const float (&u)[2][16], f32x4 (&acc)[2]) const {
    f32x4 e4[4];
#pragma unroll
    for (int v4 = 0; v4 < 4; ++v4) e4[v4] = *(const f32x4*)&Elds[l16 * ELP + k0 + 64 * c + 16 * g16 + 4 * v4];
#pragma unroll
    for (int t = 0; t < 16; ++t) {
#pragma unroll
      for (int q = 0; q < 2; ++q) acc[q] = __builtin_amdgcn_mfma_f32_16x16x4f32(e4[t / 4][t % 4], u[q][t], acc[q], 0, 0, 0);
    }
  }
};

__device__ __forceinline__ void pending_acc(const SweepArgs& a, const float* Elds, int k0, int nch, int64_t ib,
                                            int wblk, f32x4 (&acc)[2]) {
  if (nch <= 0) return;
  const PendingOps op(a, Elds, k0, ib, wblk);
  float ua[2][16], ub[2][16];
  op.load(0, ua);
  for (int c = 0; c < nch; c += 2) {
    if (c + 1 < nch) op.load(c + 1, ub);
    op.mul(c, ua, acc);
    if (c + 1 < nch) {
      if (c + 2 < nch) op.load(c + 2, ua);
      op.mul(c + 1, ub, acc);
    }
  }
}

// One block of the sweep.  GMODE: 0 = (s, z) fixed for the whole block
// (per-row, or a group spanning several blocks); 8..128 = group size known at
// compile time, groups start inside the block; -1 = any other in-block group
// size (runtime).  Codes and errors of a lane's columns are taken after the
// last step from the registers, which keep each column's value from its own
// step on (the factor row of a later step is zero there); groups narrower than
// the lanes of a row, and runtime group sizes, capture them at their step.
// Three workgroups per CU for the look-ahead kernel (at most 168 VGPRs, which
// its pending update's operands otherwise just exceed); the narrow-group
// variants hold several groups' state and would spill, so they keep one.
// A barrier that orders only LDS: global stores and loads in flight (the
// previous block's outputs, the next block's operands) stay in flight.  The
// waves of a superblock launch hand each other data through LDS only.
__device__ __forceinline__ void lds_barrier() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}

// What a block's sweep reads from global memory first: its factor rows and
// 1/U_pp (prepared once per layer by diag_blocks_kernel) and the rows' values.
template <int LPR>
struct BlockLoads {
  using LY = BlockLayout<LPR>;
  static constexpr int Q4 = LY::USZ / 4, NQ = (Q4 + 255) / 256;
  f32x4 ublk[NQ];
  float invd_t;
  float v[8];
  __device__ __forceinline__ void load(const SweepArgs& a) {
    const int tid = threadIdx.x, lr = tid & (LPR - 1);
    const int64_t r = (int64_t)blockIdx.x * (256 / LPR) + tid / LPR;
    const bool active = r < a.m;
    const f32x4* src = (const f32x4*)a.Dblk;
#pragma unroll
    for (int u = 0; u < NQ; ++u) {
      const int q = tid + 256 * u;
      ublk[u] = (Q4 % 256 == 0 || q < Q4) ? src[q] : f32x4{0.f, 0.f, 0.f, 0.f};
    }
    invd_t = tid < LY::NSTEP ? a.Dblk[LY::USZ + tid] : 0.f;
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      const int c = lr + LPR * k;
      v[k] = (active && c < a.w) ? a.V[r * a.n + a.i + c] : 0.f;
    }
  }
};

template <int LPR>
struct SweepSmem {
  using LY = BlockLayout<LPR>;
  float* Us;                                        // LY::USZ floats, 16-byte aligned
  float* invd;                                      // LY::NSTEP
  uint8_t (*codes8)[LY::NSTEP];                     // [256 / LPR][NSTEP], 8-byte aligned
  float* Elds;                                      // superblock launches: [16][ELP] errors, else null
  float* upd;                                       // superblock launches: [16][UPITCH] pending update
};

// SBM: the block is block `sbt` of a superblock launch (its pending errors
// from Elds, its own errors also kept there at column sbt * w).
template <int LPR, int GMODE, bool LOOK, bool SBM>
__device__ __forceinline__ void sweep_block_body(const SweepArgs& a, const SweepSmem<LPR>& sm, int ecol,
                                                 BlockLoads<LPR>* pre = nullptr, const SweepArgs* next = nullptr) {
  using LY = BlockLayout<LPR>;
  constexpr int NSTEP = LY::NSTEP;
  constexpr int ROWS = 256 / LPR;
  constexpr bool CAPTURE = GMODE < 0 || (GMODE > 0 && GMODE < LPR);
  constexpr int NG = (GMODE > 0 && !CAPTURE) ? NSTEP / GMODE : 1;  // groups of the block kept for the end
  constexpr int USZ = LY::USZ;
  static_assert(!(LOOK || SBM) || (LPR == 16 && 16 * UPITCH <= USZ), "look-ahead needs the 128-column layout");
  float* const Us = sm.Us;
  float* const invd = sm.invd;
  uint8_t (*const codes8)[NSTEP] = sm.codes8;
  const int tid = threadIdx.x;
  const int lr = tid & (LPR - 1);
  const int rl = tid / LPR;  // row within the workgroup
  const int64_t r = (int64_t)blockIdx.x * ROWS + rl;
  const bool active = r < a.m;
  const int w = a.w;
  const int64_t i = a.i;
  // every load of the block's start in flight at once (in a superblock
  // launch they were issued during the previous block)
  constexpr int Q4 = BlockLoads<LPR>::Q4, NQ = BlockLoads<LPR>::NQ;
  BlockLoads<LPR> ld;
  if constexpr (SBM) ld = *pre;
  else ld.load(a);
  f32x4 (&ublk)[NQ] = ld.ublk;
  const float invd_t = ld.invd_t;
  float (&v)[8] = ld.v;
  if constexpr (LOOK && !SBM) {
    if (a.kpend > 0) {
      if (a.kpend == BMAX) pending_update<BMAX>(a, (int64_t)blockIdx.x * ROWS, Us);
      else pending_update<BMAX / 2>(a, (int64_t)blockIdx.x * ROWS, Us);
#pragma unroll
      for (int k = 0; k < 8; ++k) v[k] -= Us[rl * UPITCH + lr + LPR * k];
      __syncthreads();  // upd consumed before the factor block overwrites it
    }
  }
#pragma unroll
  for (int u = 0; u < NQ; ++u) {
    const int q = tid + 256 * u;
    if (Q4 % 256 == 0 || q < Q4) ((f32x4*)Us)[q] = ublk[u];
  }
  if (tid < NSTEP) invd[tid] = invd_t;
  if constexpr (SBM) {
    // B1: the factor block is in LDS and the MFMA waves have put this block's
    // pending update in `upd` (they take the same barrier whether or not
    // anything is pending; they write `upd` again only after the next block's
    // B0, when every sweeping wave has read it)
    lds_barrier();
    if (a.kpend > 0) {
#pragma unroll
      for (int k = 0; k < 8; ++k) v[k] -= sm.upd[rl * UPITCH + lr + LPR * k];
    }
  }

  GroupState g = make_group(1.f, 0.f, a.maxq);
  if (GMODE == 0 && active) {
    const int64_t gi = a.group <= 0 ? 0 : i / a.group;
    g = make_group(a.S[r * a.G + gi], (float)a.Z[r * a.G + gi], a.maxq);
  }
  GroupState gk[NG];
#pragma unroll
  for (int k = 0; k < NG; ++k) gk[k] = g;
  float ek[8], qk[8], sk[8], zk[8];  // CAPTURE only: error, qz, scale and zero point of the column
#pragma unroll
  for (int k = 0; k < 8; ++k) {
    ek[k] = 0.f;
    qk[k] = 0.f;
    sk[k] = 1.f;
    zk[k] = 0.f;
  }
  int next_group = 0;  // GMODE == -1: block-local column of the next group start
  const bool writer = active && lr == 0;
  if constexpr (!SBM) __syncthreads();

  // factor rows prefetched D steps ahead into a ring of registers (only the
  // live registers J..7 of each row)
  constexpr int D = 4;
  float u[D + 1][8];
  auto load_row = [&](auto PC) {
    constexpr int P = decltype(PC)::value;
    constexpr int J = P / LPR;
    [&]<int... S>(std::integer_sequence<int, S...>) {
      (
          [&] {
            constexpr int R0 = LY::SEG[J][S][0], LEN = LY::SEG[J][S][1];
            constexpr int O = LY::seg_off(P, S);
            if constexpr (LEN == 4) {
              const f32x4 x = *(const f32x4*)&Us[O + 4 * lr];
              u[P % (D + 1)][R0] = x[0]; u[P % (D + 1)][R0 + 1] = x[1];
              u[P % (D + 1)][R0 + 2] = x[2]; u[P % (D + 1)][R0 + 3] = x[3];
            } else if constexpr (LEN == 2) {
              const float2 x = *(const float2*)&Us[O + 2 * lr];
              u[P % (D + 1)][R0] = x.x; u[P % (D + 1)][R0 + 1] = x.y;
            } else {
              u[P % (D + 1)][R0] = Us[O + lr];
            }
          }(),
          ...);
    }(std::make_integer_sequence<int, LY::NSEG[J]>{});
  };
  [&]<int... P>(std::integer_sequence<int, P...>) {
    (load_row(std::integral_constant<int, P>{}), ...);
  }(std::make_integer_sequence<int, D>{});

  // one column per step, fully unrolled so that register and DPP lane
  // indices are compile-time constants
  [&]<int... P>(std::integer_sequence<int, P...>) {
    (
        [&] {
          if constexpr (P + D < NSTEP) load_row(std::integral_constant<int, P + D>{});
          // keep the prefetch where it is: the scheduler would otherwise sink
          // the loads next to their use, D steps later
          __builtin_amdgcn_sched_barrier(0);
          if constexpr (GMODE > 0) {
            if constexpr (P % GMODE == 0) {
              g = group_params<LPR>(v, lr, P, P + GMODE < w ? P + GMODE : w, a.maxq);
              store_params(a, g, r, i + P, writer && P < w);
              if constexpr (!CAPTURE) gk[P / GMODE] = g;
            }
          } else if constexpr (GMODE < 0) {
            if (P == next_group && P < w) {
              const int c1 = (int)((int64_t)P + a.group < (int64_t)w ? P + a.group : w);
              g = group_params_call<LPR>(v[0], v[1], v[2], v[3], v[4], v[5], v[6], v[7], lr, P, c1, a.maxq);
              store_params(a, g, r, i + P, writer);
              next_group += (int)a.group;
            }
          }
          constexpr int J = P / LPR;  // register of column P (registers below are final)
          const float vp = RowOps<LPR>::template bcast<P % LPR>(v[J]);
          const float qz = __builtin_amdgcn_fmed3f(rintf(vp * g.inv_s), g.nz, g.mz);
          const float err = fmaf(-g.s, qz, vp);
          if constexpr (CAPTURE) {
            if (lr == P % LPR) {
              ek[J] = err;
              qk[J] = qz;
              sk[J] = g.s;
              zk[J] = g.z;
            }
          }
#pragma unroll
          for (int k = J; k < 8; ++k) v[k] = fmaf(-err, u[P % (D + 1)][k], v[k]);
        }(),
        ...);
  }(std::make_integer_sequence<int, NSTEP>{});

  if constexpr (SBM) {
    if (next) pre->load(*next);  // the next block's operands arrive while this one is written out
  }
  // codes, errors and dequantized weights of this lane's columns
  float eacc = 0.f;
  float ws_[8], qz_[8];
#pragma unroll
  for (int k = 0; k < 8; ++k) {
    const int c = lr + LPR * k;
    float err, qz, s;
    if constexpr (CAPTURE) {
      err = ek[k];
      qz = qk[k];
      s = sk[k];
    } else {
      const GroupState& gc = gk[GMODE > 0 ? (LPR * k) / GMODE : 0];
      qz = __builtin_amdgcn_fmed3f(rintf(v[k] * gc.inv_s), gc.nz, gc.mz);
      err = fmaf(-gc.s, qz, v[k]);
      s = gc.s;
    }
    const float e = err * invd[c];
    ek[k] = e;
    qz_[k] = qz;
    ws_[k] = s;
    eacc = fmaf(e, e, eacc);
  }
  eacc = RowOps<LPR>::rsum(eacc);
  if constexpr (SBM) {
    // the errors go to LDS first: from the barrier on, the MFMA waves apply
    // them to the next block while this one is written out
    if (active) {
#pragma unroll
      for (int k = 0; k < 8; ++k) {
        const int c = lr + LPR * k;
        if (c < w) sm.Elds[rl * ELP + ecol + c] = ek[k];
      }
    }
    if (next) lds_barrier();  // B0 of the next block
  }
  if (active) {
    // one branch on the output type for the whole row, not one per column
    const bool full = w == NSTEP;
    if (a.Ecat) {  // also keep E itself on the paired path, whose look-ahead reads it
      uint16_t* erow = a.Ecat + r * (2 * SBW) + (SBM ? ecol : 0);
#pragma unroll
      for (int k = 0; k < 8; ++k) {
        const int c = lr + LPR * k;
        if (full || c < w) {
          const uint16_t hi = f32_to_bf16(ek[k]);
          const uint16_t lo = f32_to_bf16(ek[k] - bf16_to_f32(hi));
          erow[c] = hi;
          erow[SBW + c] = lo;
        }
      }
    }
    if (!SBM || !a.Ecat) {
#pragma unroll
      for (int k = 0; k < 8; ++k) {
        const int c = lr + LPR * k;
        if (full || c < w) a.E[r * ELD + c] = ek[k];
      }
    }
    if (a.Wout) {
      if (a.wdt == 0) {
#pragma unroll
        for (int k = 0; k < 8; ++k) {
          const int c = lr + LPR * k;
          if (full || c < w) ((_Float16*)a.Wout)[r * a.ldw + i + c] = (_Float16)(ws_[k] * qz_[k]);
        }
      } else if (a.wdt == 1) {
#pragma unroll
        for (int k = 0; k < 8; ++k) {
          const int c = lr + LPR * k;
          if (full || c < w) ((uint16_t*)a.Wout)[r * a.ldw + i + c] = f32_to_bf16(ws_[k] * qz_[k]);
        }
      } else {
#pragma unroll
        for (int k = 0; k < 8; ++k) {
          const int c = lr + LPR * k;
          if (full || c < w) ((float*)a.Wout)[r * a.ldw + i + c] = ws_[k] * qz_[k];
        }
      }
    }
    // blocks run one after another, so each row's sum is taken in block order
    if (lr == 0 && a.err_sq) atomicAdd(a.err_sq + r, eacc);
  }
  // codes: q = qz + z, as bytes (fallback layout) or packed per row
  float zc[8];
#pragma unroll
  for (int k = 0; k < 8; ++k) {
    if constexpr (CAPTURE) {
      zc[k] = zk[k];
    } else {
      zc[k] = gk[GMODE > 0 ? (LPR * k) / GMODE : 0].z;
    }
  }
  if (a.Qw == nullptr) {
    if (active) {
#pragma unroll
      for (int k = 0; k < 8; ++k) {
        const int c = lr + LPR * k;
        if (c < w) a.Q8[r * a.n + i + c] = (uint8_t)(int)(qz_[k] + zc[k]);
      }
    }
    return;
  }
  // the row's codes as bytes (0 past w), then each lane packs 8 consecutive
  // codes into one dense segment of 8 bits: the row's bit-stream is the
  // segments of its LPR lanes in order
#pragma unroll
  for (int k = 0; k < 8; ++k) {
    const int c = lr + LPR * k;
    codes8[rl][c] = c < w ? (uint8_t)(int)(qz_[k] + zc[k]) : (uint8_t)0;
  }
  // the row's codes were written by lanes of this wave only: wait for the
  // wave's LDS writes before its lanes read each other's bytes
  asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
  __builtin_amdgcn_wave_barrier();
  const int bits = a.bits;
  uint64_t seg = 0;
  {
    const uint64_t b8 = *(const uint64_t*)&codes8[rl][8 * lr];
#pragma unroll
    for (int k = 0; k < 8; ++k) seg |= ((b8 >> (8 * k)) & 0xFFu) << (bits * k);
  }
  const int nwords = (w * bits + 31) / 32;
  uint32_t* dst = a.Qw + r * a.words + (i * bits) / 32;
  if (bits == 4 || bits == 8) {  // a segment is whole words: store it
    if (active) {
      if (bits == 4) {
        if (lr < nwords) dst[lr] = (uint32_t)seg;
      } else {
        if (2 * lr < nwords) dst[2 * lr] = (uint32_t)seg;
        if (2 * lr + 1 < nwords) dst[2 * lr + 1] = (uint32_t)(seg >> 32);
      }
    }
    return;
  }
  // the segments replace the row's bytes (NSTEP bytes = LPR segments); the
  // wave's read of the bytes is issued before this write
  uint64_t* segs = (uint64_t*)&codes8[rl][0];
  segs[lr] = seg;
  asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
  __builtin_amdgcn_wave_barrier();
  if (!active) return;
  // word wd = bits [32 wd, 32 wd + 32) of the row: the segments of 8 bits
  // each that overlap it (at most 3 for bits >= 2)
  const int sb = 8 * bits;
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    const int wd = lr + LPR * h;
    const int bit0 = 32 * wd;
    const int s0 = bit0 / sb;
    uint64_t word = 0;
#pragma unroll
    for (int t = 0; t < 3; ++t) {
      const int sg = s0 + t;
      const int off = sg * sb - bit0;  // position of the segment's bit 0 in the word
      if (sg < LPR && off < 32) {
        const uint64_t v = segs[sg];
        word |= off >= 0 ? (v << off) : (v >> (-off));
      }
    }
    if (wd < nwords) dst[wd] = (uint32_t)word;
  }
}

template <int LPR, int GMODE, bool LOOK>
__global__ __launch_bounds__(256, (LOOK && (GMODE <= 0 || GMODE >= 64)) ? 3 : 1) void sweep_block_kernel(SweepArgs a) {
  using LY = BlockLayout<LPR>;
  __shared__ __attribute__((aligned(16))) float Us[LY::USZ];
  __shared__ float invd[LY::NSTEP];
  __shared__ __attribute__((aligned(8))) uint8_t codes8[256 / LPR][LY::NSTEP];
  const SweepSmem<LPR> sm{Us, invd, codes8, nullptr, nullptr};
  sweep_block_body<LPR, GMODE, LOOK, false>(a, sm, 0);
}

// A whole superblock (up to SBW columns) in one launch, one workgroup per CU,
// 512 threads.  Waves 0..3 sweep the blocks one after another (16 rows, as
// above); waves 4..7 apply the pending updates on the matrix cores beside
// them: while block t is swept they accumulate the errors of blocks 0..t-1
// onto block t + 1's columns, and once block t's errors are in LDS they add
// those and hand the update over.  Rows are independent, so nothing is
// exchanged between workgroups; what the launch replaces is one launch per
// block and the product flushes inside the superblock.
//
// Barriers per block, taken by all eight waves: B0 (t > 0: block t - 1's
// errors in Elds, taken by the sweeping waves before they write that block
// out; the MFMA waves' partial sums done) and B1 (the update in `upd`, the
// factor block in LDS).
template <int GMODE>
__global__ __launch_bounds__(512, 1) void sweep_superblock_kernel(SweepArgs a) {
  using LY = BlockLayout<16>;
  __shared__ __attribute__((aligned(16))) float Us[LY::USZ];
  __shared__ float invd[LY::NSTEP];
  __shared__ __attribute__((aligned(8))) uint8_t codes8[16][LY::NSTEP];
  __shared__ __attribute__((aligned(16))) float Elds[16 * ELP];
  __shared__ __attribute__((aligned(16))) float upd[16 * UPITCH];
  const SweepSmem<16> sm{Us, invd, codes8, Elds, upd};
  const int B = a.w;
  if (threadIdx.x < 256) {
    auto block_args = [&](int t) {
      SweepArgs b = a;
      b.i = a.i + (int64_t)t * B;
      b.w = t + 1 < a.nblk ? B : a.wlast;
      b.E = a.E + (int64_t)t * B;
      b.Dblk = a.Dblk + (int64_t)t * LY::STRIDE;
      b.kpend = t * B;
      return b;
    };
    BlockLoads<16> pre;
    SweepArgs b = block_args(0);
    pre.load(b);
    for (int t = 0; t < a.nblk; ++t) {
      // (B0 of block t + 1 is taken inside block t's write-out, once its
      // errors are in Elds)
      const SweepArgs bn = block_args(t + 1 < a.nblk ? t + 1 : t);
      sweep_block_body<16, GMODE, false, true>(b, sm, t * B, &pre, t + 1 < a.nblk ? &bn : nullptr);
      b = bn;
    }
  } else {
    const int lane = threadIdx.x & 63, wq = (threadIdx.x >> 6) - 4;
    const int l16 = lane & 15, g16 = lane >> 4;
    const int nb = B / 64;  // 64-row chunks per block (1 or 2)
    f32x4 acc[2] = {{0.f, 0.f, 0.f, 0.f}, {0.f, 0.f, 0.f, 0.f}};
    float bu[2][2][16];     // factor rows of the previous block, for its errors onto this one (loaded early)
    for (int t = 0; t < a.nblk; ++t) {
      const int wt = t + 1 < a.nblk ? B : a.wlast;  // width of block t
      if (t > 0) {
        lds_barrier();  // B0: block t - 1's errors are in Elds
        const PendingOps op(a, Elds, (t - 1) * B, a.i + (int64_t)t * B, wt);
        op.mul(0, bu[0], acc);
        if (nb > 1) op.mul(1, bu[1], acc);
#pragma unroll
        for (int q = 0; q < 2; ++q)
#pragma unroll
          for (int rr = 0; rr < 4; ++rr)
            upd[(4 * g16 + rr) * UPITCH + 16 * (2 * wq + q) + l16] = 16 * (2 * wq + q) + l16 < wt ? acc[q][rr] : 0.f;
      }
      lds_barrier();  // B1
      acc[0] = f32x4{0.f, 0.f, 0.f, 0.f};
      acc[1] = f32x4{0.f, 0.f, 0.f, 0.f};
      if (t + 1 < a.nblk) {
        // while block t is swept: blocks 0..t-1 onto block t + 1, then the
        // factor rows of block t for block t + 1's columns (its errors follow)
        const int wn = t + 2 < a.nblk ? B : a.wlast;
        const int64_t ibn = a.i + (int64_t)(t + 1) * B;
        pending_acc(a, Elds, 0, t * nb, ibn, wn, acc);
        const PendingOps op(a, Elds, t * B, ibn, wn);
        op.load(0, bu[0]);
        if (nb > 1) op.load(1, bu[1]);
      }
    }
  }
}

// Per block of B columns starting at i = blk * B: the factor rows p of
// U[i:i+w, i:i+w] divided by U_pp, zero on and left of the diagonal, in
// BlockLayout<LPR> order, then 1/U_pp (0 past w).  One thread per (row p,
// lane lr), writing the row's live registers of that lane.
template <int LPR>
__global__ __launch_bounds__(256) void diag_blocks_kernel(const float* U, int64_t n, int64_t B, float* out) {
  using LY = BlockLayout<LPR>;
  const int64_t i = (int64_t)blockIdx.x * B;
  const int w = (int)std::min<int64_t>(B, n - i);
  float* dst = out + (int64_t)blockIdx.x * LY::STRIDE;
  const int t = blockIdx.y * 256 + threadIdx.x;
  const int p = t / LPR, lr = t % LPR;
  if (p < LY::NSTEP) {
    const int J = p / LPR;
    const bool prow = p < w;
    const float d = prow ? U[(i + p) * n + i + p] : 1.f;
    for (int s = 0; s < LY::NSEG[J]; ++s) {
      const int r0 = LY::SEG[J][s][0], len = LY::SEG[J][s][1];
      const int o = LY::seg_off(p, s) + len * lr;
      for (int k = 0; k < len; ++k) {
        const int c = lr + LPR * (r0 + k);
        dst[o + k] = (prow && c < w && c > p) ? U[(i + p) * n + i + c] / d : 0.f;
      }
    }
    if (lr == 0) dst[LY::USZ + p] = prow ? 1.f / d : 0.f;
  }
}

void launch_sweep_sb(const SweepArgs& a, int gmode, hipStream_t st) {
  const dim3 grid((unsigned)cdiv(a.m, 16)), block(512);
  switch (gmode) {
    case 0: hipLaunchKernelGGL((sweep_superblock_kernel<0>), grid, block, 0, st, a); break;
    case 8: hipLaunchKernelGGL((sweep_superblock_kernel<8>), grid, block, 0, st, a); break;
    case 16: hipLaunchKernelGGL((sweep_superblock_kernel<16>), grid, block, 0, st, a); break;
    case 32: hipLaunchKernelGGL((sweep_superblock_kernel<32>), grid, block, 0, st, a); break;
    case 64: hipLaunchKernelGGL((sweep_superblock_kernel<64>), grid, block, 0, st, a); break;
    case 128: hipLaunchKernelGGL((sweep_superblock_kernel<128>), grid, block, 0, st, a); break;
    default: hipLaunchKernelGGL((sweep_superblock_kernel<-1>), grid, block, 0, st, a);
  }
}

template <int LPR, bool LOOK>
void launch_sweep(const SweepArgs& a, int gmode, hipStream_t st) {
  const dim3 grid((unsigned)cdiv(a.m, 256 / LPR)), block(256);
  switch (gmode) {
    case 0: hipLaunchKernelGGL((sweep_block_kernel<LPR, 0, LOOK>), grid, block, 0, st, a); break;
    case 8: hipLaunchKernelGGL((sweep_block_kernel<LPR, 8, LOOK>), grid, block, 0, st, a); break;
    case 16: hipLaunchKernelGGL((sweep_block_kernel<LPR, 16, LOOK>), grid, block, 0, st, a); break;
    case 32: hipLaunchKernelGGL((sweep_block_kernel<LPR, 32, LOOK>), grid, block, 0, st, a); break;
    default:
      if constexpr (LPR == 16) {
        if (gmode == 64) { hipLaunchKernelGGL((sweep_block_kernel<LPR, 64, LOOK>), grid, block, 0, st, a); break; }
        if (gmode == 128) { hipLaunchKernelGGL((sweep_block_kernel<LPR, 128, LOOK>), grid, block, 0, st, a); break; }
      }
      hipLaunchKernelGGL((sweep_block_kernel<LPR, -1, LOOK>), grid, block, 0, st, a);
  }
}

// V = fp32 copy of W (row-major, leading dimension n).
template <int DT>
__global__ __launch_bounds__(256) void to_f32_kernel(const void* W, int64_t ldw, float* V, int64_t m, int64_t n) {
  for (int64_t r = blockIdx.y; r < m; r += gridDim.y)
    for (int64_t c = blockIdx.x * 256 + threadIdx.x; c < n; c += (int64_t)gridDim.x * 256)
      V[r * n + c] = Elem<DT>::load(W, r * ldw + c);
}

// The same, 8 elements per thread with 16-byte accesses (n % 8 == 0,
// ldw % 8 == 0, 16-byte aligned W).
template <int DT>
__global__ __launch_bounds__(256) void to_f32x8_kernel(const void* W, int64_t ldw, float* V, int64_t m, int64_t n) {
  for (int64_t r = blockIdx.y; r < m; r += gridDim.y)
    for (int64_t c = 8 * ((int64_t)blockIdx.x * 256 + threadIdx.x); c < n; c += (int64_t)gridDim.x * 2048) {
      float x[8];
      if (DT == 2) {
        const f32x4 a = *(const f32x4*)((const float*)W + r * ldw + c), b = *(const f32x4*)((const float*)W + r * ldw + c + 4);
        x[0] = a[0]; x[1] = a[1]; x[2] = a[2]; x[3] = a[3]; x[4] = b[0]; x[5] = b[1]; x[6] = b[2]; x[7] = b[3];
      } else {
        const uint4 q = *(const uint4*)((const uint16_t*)W + r * ldw + c);
        const uint32_t wv[4] = {q.x, q.y, q.z, q.w};
#pragma unroll
        for (int k = 0; k < 4; ++k) {
          const uint16_t lo = (uint16_t)(wv[k] & 0xFFFFu), hi = (uint16_t)(wv[k] >> 16);
          if (DT == 0) {
            x[2 * k] = (float)__builtin_bit_cast(_Float16, lo);
            x[2 * k + 1] = (float)__builtin_bit_cast(_Float16, hi);
          } else {
            x[2 * k] = bf16_to_f32(lo);
            x[2 * k + 1] = bf16_to_f32(hi);
          }
        }
      }
      *(f32x4*)(V + r * n + c) = f32x4{x[0], x[1], x[2], x[3]};
      *(f32x4*)(V + r * n + c + 4) = f32x4{x[4], x[5], x[6], x[7]};
    }
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

inline size_t align256(size_t b) { return (b + 255) & ~(size_t)255; }

dim3 rows_grid(int64_t cols, int64_t rows) {
  return dim3((unsigned)std::min<int64_t>(cdiv(cols, 256), 64), (unsigned)std::min<int64_t>(rows, 65535));
}

}  // namespace

// Workspace: fp32 working copy V [m x n], codes [m x n] bytes (used only when
// a block's codes do not fill whole 32-bit words), E [m x 256], then the
// prepared diagonal factor blocks.
inline int64_t dstride_for(int64_t B) { return B <= 32 ? BlockLayout<4>::STRIDE : BlockLayout<16>::STRIDE; }
inline size_t dblk_bytes(int64_t n, int64_t B) { return (size_t)cdiv(n, B) * (size_t)dstride_for(B) * 4; }

// Rows up to X3_MAX_N columns run their trailing products as three bf16
// products (the reason for the limit is given where quantize_layer decides).
constexpr int64_t X3_MAX_N = 16384;

// Then, for the flushes as bf16 products: the errors as [E_hi | E_lo]
// [m x 2 SBW] and the factor split and transposed once, [U_hi | U_lo]^T
// [n x 2n], bf16 (none past X3_MAX_N columns).
inline size_t x3_bytes(int64_t m, int64_t n) {
  if (n > X3_MAX_N) return 0;
  return align256((size_t)m * 2 * SBW * 2) + align256((size_t)n * 2 * n * 2);
}

size_t quantize_workspace_bytes(int64_t m, int64_t n, int64_t B) {
  if (m < 1 || n < 1 || B < 1) return 0;
  return align256((size_t)m * n * 4) + align256((size_t)m * n) + align256((size_t)m * ELD * 4) +
         align256(dblk_bytes(n, B)) + x3_bytes(m, n);
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
  p += align256((size_t)m * ELD * 4);
  float* Dblk = (float*)p;
  p += align256(dblk_bytes(n, B));
  uint16_t* Ecat = (uint16_t*)p;  // Ecat and Ut only when n <= X3_MAX_N
  p += align256((size_t)m * 2 * SBW * 2);
  uint16_t* Ut = (uint16_t*)p;
  const int64_t dstride = dstride_for(B);
  // every block starts on a word boundary of the packed rows: the sweep packs its own codes
  const bool packed = (B * bits) % 32 == 0;
  const int64_t words = cdiv(n * bits, 32);

  const int maxq = (1 << bits) - 1;
  const int64_t G = group <= 0 ? 1 : cdiv(n, group);
  const bool inblock = group > 0 && group <= B;
  const bool pow2 = group >= 8 && group <= 128 && (group & (group - 1)) == 0;
  const int gmode = !inblock ? 0 : (pow2 && group <= (B <= 32 ? 32 : 128) ? (int)group : -1);
  const dim3 rg = rows_grid(n, m);

  const bool x8 = n % 8 == 0 && ldw % 8 == 0 && ((uintptr_t)W & 15) == 0;
  const dim3 rg8 = rows_grid(cdiv(n, 8), m);
  if (x8 && dt == 0) hipLaunchKernelGGL((to_f32x8_kernel<0>), rg8, dim3(256), 0, st, W, ldw, V, m, n);
  else if (x8 && dt == 1) hipLaunchKernelGGL((to_f32x8_kernel<1>), rg8, dim3(256), 0, st, W, ldw, V, m, n);
  else if (x8) hipLaunchKernelGGL((to_f32x8_kernel<2>), rg8, dim3(256), 0, st, W, ldw, V, m, n);
  else if (dt == 0) hipLaunchKernelGGL((to_f32_kernel<0>), rg, dim3(256), 0, st, W, ldw, V, m, n);
  else if (dt == 1) hipLaunchKernelGGL((to_f32_kernel<1>), rg, dim3(256), 0, st, W, ldw, V, m, n);
  else hipLaunchKernelGGL((to_f32_kernel<2>), rg, dim3(256), 0, st, W, ldw, V, m, n);
  const unsigned prow = (unsigned)cdiv(m, 4);
  if (group <= 0)
    hipLaunchKernelGGL(row_params_kernel, dim3(prow), dim3(256), 0, st, (const float*)V, m, n, (int64_t)0, n, maxq, S,
                       Z, G, (int64_t)0);
  if (err_sq)
    hipLaunchKernelGGL(zero_f32_kernel, dim3((unsigned)std::min<int64_t>(cdiv(m, 256), 1024)), dim3(256), 0, st,
                       err_sq, m);
  if (B <= 32)
    hipLaunchKernelGGL((diag_blocks_kernel<4>), dim3((unsigned)cdiv(n, B), (unsigned)cdiv(32 * 4, 256)), dim3(256), 0,
                       st, U, n, B, Dblk);
  else
    hipLaunchKernelGGL((diag_blocks_kernel<16>), dim3((unsigned)cdiv(n, B), (unsigned)cdiv(128 * 16, 256)), dim3(256),
                       0, st, U, n, B, Dblk);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;

  const bool look = B % 64 == 0 && (group <= 0 || group <= B) && n % 4 == 0;
  // on the look-ahead paths the flushes run as three bf16 products (the
  // sweep kernels write the errors split into E_hi and E_lo as well, and
  // the factor is split once, here); a flush whose K is not a multiple of
  // 64 (a short last block) stays fp32.
  // Rows longer than X3_MAX_N stay fp32 too: every column takes the errors of
  // all earlier superblocks, and at 49152 columns the products' error moved
  // 0.11 % of the codes (99.89 % identical against 99.96 % in fp32), at
  // 12288 columns and below it moves none beyond the near-tie band.
  const bool x3 = look && n <= X3_MAX_N;
  // superblock launches (below) flush only past whole superblocks; the
  // paired blocks flush past every 64-column multiple
  const bool sb = look && cdiv(m, 16) <= device_cus();
  if (x3 && (e = split_ut_x3(U, n, Ut, sb ? SBW : 64, st)) != hipSuccess) return e;

  // sweep one block [i, i + w) with its errors written at column eoff of E;
  // on the look-ahead path the kpend columns before it (from column g0, their
  // errors at column epair of E) are still to be applied to it
  auto sweep_block = [&](int64_t i, int w, int eoff, bool la, int64_t g0, int epair) -> hipError_t {
    if (group > B && i % group == 0)
      hipLaunchKernelGGL(row_params_kernel, dim3(prow), dim3(256), 0, st, (const float*)V, m, n, i, group, maxq, S,
                         Z, G, i / group);
    SweepArgs a{U, V, n, m, i, w, maxq, group, G, S, Z, packed ? nullptr : Q8, packed ? qcodes : nullptr, words,
                bits, write_dequant ? W : nullptr, dt, ldw, E + eoff, err_sq, Dblk + (i / B) * dstride,
                E + epair, (int)(i - g0), U + g0 * n + i, 1, w, x3 && la ? Ecat + eoff : nullptr};
    if (B <= 32) launch_sweep<4, false>(a, gmode, st);
    else if (la) launch_sweep<16, true>(a, gmode, st);
    else launch_sweep<16, false>(a, gmode, st);
    return hipGetLastError();
  };
  // V[:, c0:c0+N] -= E[:, ec:ec+K] U[r0:r0+K, c0:c0+N]
  auto flush = [&](int ec, int64_t r0, int K, int64_t c0, int64_t N) -> hipError_t {
    if (N <= 0) return hipSuccess;
    GemmDesc g{};
    g.A = E + ec; g.lda = ELD;
    g.B = U + r0 * n + c0; g.ldb = n;
    g.C = V + c0; g.ldc = n;
    g.M = (int)m; g.N = (int)N; g.K = K; g.batch = 1;
    g.alpha = -1.f; g.beta = 1.f;
    return gemm_f32(g, false, false, st);
  };
  // (pending K = t B is a multiple of the 64-row chunks; rows of V 16-byte aligned)
  auto flushx = [&](int ec, int64_t r0, int K, int64_t c0, int64_t N) -> hipError_t {
    if (N <= 0) return hipSuccess;
    if (x3 && K % 64 == 0) return flush_x3(Ecat + ec, 2 * SBW, SBW, Ut, n, r0, K, c0, N, V, m, st);
    return flush(ec, r0, K, c0, N);
  };
  // Superblock launches while the rows fit the GPU in one round of one
  // workgroup (16 rows) per CU: each superblock of SBW columns is swept by one
  // launch (every block taking the errors of the superblock's earlier blocks
  // inside the kernel), then one product brings the rest of the row up to
  // date.
  if (sb) {
    for (int64_t s0 = 0; s0 < n; s0 += SBW) {
      const int64_t s1 = std::min<int64_t>(s0 + SBW, n);
      const int nblk = (int)cdiv(s1 - s0, B);
      // the flush past the superblock: three bf16 products up to X3_MAX_N
      // columns (its errors written as [E_hi | E_lo] by the sweep kernel
      // instead of E), else fp32 from E
      SweepArgs a{U, V, n, m, s0, (int)B, maxq, group, G, S, Z, packed ? nullptr : Q8, packed ? qcodes : nullptr,
                  words, bits, write_dequant ? W : nullptr, dt, ldw, E, err_sq, Dblk + (s0 / B) * dstride,
                  nullptr, 0, U + s0 * n + s0, nblk, (int)(s1 - s0 - (int64_t)(nblk - 1) * B),
                  x3 && s1 < n ? Ecat : nullptr};
      launch_sweep_sb(a, gmode, st);
      if ((e = hipGetLastError()) != hipSuccess) return e;
      if ((e = flushx(0, s0, (int)(s1 - s0), s1, n - s1)) != hipSuccess) return e;
    }
  } else if (look) {
    // Look-ahead: LA blocks per flush.  Block t of a group first takes the
    // errors of blocks 0..t-1 of its group (inside the sweep kernel, K = t B,
    // on MFMA), then is swept; after the group, one GEMM with K = LA B brings
    // the rest of its superblock (SBW columns) up to date, and after the
    // superblock one GEMM with K = SBW the rest of the row: a quarter of the
    // passes over V of flushing every group to the end, and long K for most
    // of the flops.  Every column still gets each earlier column's error once
    // before it is swept.  (Groups wider than a block would need V updated
    // past the block before their scales are taken, so they stay on the path
    // below.)
    for (int64_t s0 = 0; s0 < n; s0 += SBW) {
      const int64_t s1 = std::min<int64_t>(s0 + SBW, n);  // SBW is a multiple of B: no block straddles
      for (int64_t g0 = s0; g0 < s1;) {
        int64_t i = g0;
        for (int t = 0; t < LA && i < s1; ++t) {
          const int w = (int)std::min<int64_t>(B, s1 - i);
          if ((e = sweep_block(i, w, (int)(i - s0), true, g0, (int)(g0 - s0))) != hipSuccess) return e;
          i += w;
        }
        if ((e = flushx((int)(g0 - s0), g0, (int)(i - g0), i, s1 - i)) != hipSuccess) return e;
        g0 = i;
      }
      if ((e = flushx(0, s0, (int)(s1 - s0), s1, n - s1)) != hipSuccess) return e;
    }
  } else {
    for (int64_t i = 0; i < n; i += B) {
      const int w = (int)std::min<int64_t>(B, n - i);
      if ((e = sweep_block(i, w, 0, false, i, 0)) != hipSuccess) return e;
      if ((e = flush(0, i, w, i + w, n - i - w)) != hipSuccess) return e;
    }
  }
  if (!packed)
    hipLaunchKernelGGL(pack_kernel, rows_grid(words, m), dim3(256), 0, st, (const uint8_t*)Q8, m, n, bits, qcodes, words);
  return hipGetLastError();
}

}  // namespace gptq
