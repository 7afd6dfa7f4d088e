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
constexpr int ELD = LA * BMAX;  // leading dimension of the E buffer: the errors of LA consecutive blocks

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
  uint8_t* Q8;    // [m x n] codes
  float* E;       // [m x 128] scaled errors of this block
  float* err_sq;  // [m] or null
  const float* Dblk;  // this block's factor rows divided by their diagonal ([NSTEP][NSTEP]), then 1/U_pp [NSTEP]
  // look-ahead: errors of the kpend columns swept since the last flush
  // (E buffer from column 0) and the factor rows of those columns restricted
  // to this block's columns (U + r * n + i, leading dimension n)
  const float* Ep;
  int kpend;
  const float* Upend;
};

// Lanes-per-row variants: 16 lanes (one DPP row) x 8 columns = 128 columns,
// or 4 lanes (one DPP quad) x 8 columns = 32 columns.
template <int LPR>
struct RowOps;
template <>
struct RowOps<16> {
  template <int SRC>
  __device__ __forceinline__ static float bcast(float v) { return row_bcast<SRC>(v); }
  __device__ __forceinline__ static float rmin(float v) { return row_min16(v); }
  __device__ __forceinline__ static float rmax(float v) { return row_max16(v); }
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
};


struct GroupState {
  float s, inv_s, nz, mz;  // scale, 1/scale, -z, maxq - z
  float z;
};

// Range of columns [c0, c1) of this lane's 8 values (block-local column of
// value k is 8*lane + k), reduced over the row's lanes, then (s, z).
template <int LPR>
__device__ __forceinline__ GroupState group_params(const float (&v)[8], int lr, int c0, int c1, int maxq) {
  float lo = INFINITY, hi = -INFINITY;
#pragma unroll
  for (int k = 0; k < 8; ++k) {
    const int c = 8 * lr + k;
    const bool in = c >= c0 && c < c1;
    lo = fminf(lo, in ? v[k] : INFINITY);
    hi = fmaxf(hi, in ? v[k] : -INFINITY);
  }
  lo = RowOps<LPR>::rmin(lo);
  hi = RowOps<LPR>::rmax(hi);
  GroupState g;
  qparams(lo, hi, maxq, g.s, g.z);
  g.inv_s = 1.f / g.s;
  g.nz = -g.z;
  g.mz = (float)maxq - g.z;
  return g;
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

// GMODE: 0 = (s, z) fixed for the whole block (per-row, or a group spanning
// several blocks); 8..128 = group size known at compile time, groups start
// inside the block; -1 = any other in-block group size (runtime).
// The errors of the pending columns (swept since the last flush) applied to
// this block's 128 columns for the workgroup's 16 rows, with
// v_mfma_f32_16x16x4f32: wave w computes output column blocks 2w, 2w+1; the
// factor rows stream through the Up buffer (64 at a time, pitch 144, which
// keeps the operand reads bank-conflict-free).  The result lands in upd
// (16 x 132) for the lanes' V loads.
constexpr int KPMAX = (LA - 1) * BMAX;
constexpr int EPITCH = KPMAX + 4;
constexpr int CPITCH = 144;
__device__ __forceinline__ void pending_update(const SweepArgs& a, int64_t r0, float* chunk, float* sE, float* upd) {
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int l16 = lane & 15, g16 = lane >> 4;
  const int kp = a.kpend;
  f32x4 acc[2] = {{0.f, 0.f, 0.f, 0.f}, {0.f, 0.f, 0.f, 0.f}};
  // 64 factor rows x 128 columns per chunk, 8 float4 per thread; the next
  // chunk is loaded while the current one is multiplied
  f32x4 xr[8];
  auto load_chunk = [&](int k0) {
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const int e = tid + 256 * u;
      const int kr = e >> 5, c4 = 4 * (e & 31);  // w is a multiple of 4 on this path
      xr[u] = c4 < a.w ? *(const f32x4*)&a.Upend[(int64_t)(k0 + kr) * a.n + c4] : f32x4{0.f, 0.f, 0.f, 0.f};
    }
  };
  load_chunk(0);
  for (int e = tid; e < 16 * kp; e += 256) {
    const int rr = e / kp, k = e % kp;
    const int64_t row = min<int64_t>(r0 + rr, a.m - 1);  // rows past m: their results are never used
    sE[rr * EPITCH + k] = a.Ep[row * ELD + k];
  }
  for (int k0 = 0; k0 < kp; k0 += 64) {
    __syncthreads();  // the previous chunk is consumed (and sE is written)
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const int e = tid + 256 * u;
      *(f32x4*)&chunk[(e >> 5) * CPITCH + 4 * (e & 31)] = xr[u];
    }
    if (k0 + 64 < kp) load_chunk(k0 + 64);
    __syncthreads();
#pragma unroll
    for (int kk = 0; kk < 16; ++kk) {
      const float av = sE[l16 * EPITCH + k0 + 4 * kk + g16];
#pragma unroll
      for (int q = 0; q < 2; ++q)
        acc[q] = __builtin_amdgcn_mfma_f32_16x16x4f32(av, chunk[(4 * kk + g16) * CPITCH + 16 * (2 * wave + q) + l16],
                                                       acc[q], 0, 0, 0);
    }
  }
#pragma unroll
  for (int q = 0; q < 2; ++q)
#pragma unroll
    for (int rr = 0; rr < 4; ++rr) upd[(4 * g16 + rr) * (BMAX + 4) + 16 * (2 * wave + q) + l16] = acc[q][rr];
  __syncthreads();  // upd complete; chunk (the Up buffer) free
}

template <int LPR, int GMODE, bool LOOK>
__global__ __launch_bounds__(256) void sweep_block_kernel(SweepArgs a) {
  constexpr int NSTEP = 8 * LPR;
  constexpr int PITCH = NSTEP + 4;
  constexpr int ROWS = 256 / LPR;
  static_assert(!LOOK || (LPR == 16 && 64 * CPITCH <= NSTEP * PITCH), "look-ahead needs the 128-column layout");
  __shared__ __attribute__((aligned(16))) float Up[NSTEP * PITCH];
  __shared__ float invd[NSTEP];
  __shared__ __attribute__((aligned(16))) float sE[LOOK ? 16 * EPITCH : 1];
  __shared__ float upd[LOOK ? 16 * (BMAX + 4) : 1];
  const int tid = threadIdx.x;
  const int lr = tid & (LPR - 1);
  const int64_t r = (int64_t)blockIdx.x * ROWS + tid / LPR;
  const bool active = r < a.m;
  const int w = a.w;
  const int64_t i = a.i;
  const float* __restrict__ U = a.U;
  if constexpr (LOOK) {
    if (a.kpend > 0) pending_update(a, (int64_t)blockIdx.x * ROWS, Up, sE, upd);
  }

  // this block's factor rows divided by their diagonal (zero on and below it)
  // and 1/U_pp, prepared once per layer by diag_blocks_kernel
  {
    constexpr int Q = NSTEP * NSTEP / 4;  // float4 groups
    const f32x4* src = (const f32x4*)a.Dblk;
    f32x4 t[Q / 256];
#pragma unroll
    for (int u = 0; u < Q / 256; ++u) t[u] = src[tid + 256 * u];
#pragma unroll
    for (int u = 0; u < Q / 256; ++u) {
      const int q = tid + 256 * u;
      const int p = q / (NSTEP / 4), j4 = q % (NSTEP / 4);
      *(f32x4*)&Up[p * PITCH + 4 * j4] = t[u];
    }
    if (tid < NSTEP) invd[tid] = a.Dblk[NSTEP * NSTEP + tid];
  }
  (void)U;

  float v[8], ek[8], qk[8];
  const bool vec = ((a.n | i) & 3) == 0;  // 16-byte aligned rows of V
  if (vec && active && 8 * lr + 8 <= w) {
    const f32x4 x0 = *(const f32x4*)&a.V[r * a.n + i + 8 * lr];
    const f32x4 x1 = *(const f32x4*)&a.V[r * a.n + i + 8 * lr + 4];
    v[0] = x0[0]; v[1] = x0[1]; v[2] = x0[2]; v[3] = x0[3];
    v[4] = x1[0]; v[5] = x1[1]; v[6] = x1[2]; v[7] = x1[3];
  } else {
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      const int c = 8 * lr + k;
      v[k] = (active && c < w) ? a.V[r * a.n + i + c] : 0.f;
    }
  }
  if constexpr (LOOK) {
    if (a.kpend > 0) {
#pragma unroll
      for (int k = 0; k < 8; ++k) {
        const int c = 8 * lr + k;
        if (c < w) v[k] -= upd[(tid / LPR) * (BMAX + 4) + c];
      }
    }
  }
#pragma unroll
  for (int k = 0; k < 8; ++k) {
    ek[k] = 0.f;
    qk[k] = 0.f;
  }
  GroupState g;
  g.s = 1.f;
  g.z = 0.f;
  if (GMODE == 0 && active) {
    const int64_t gi = a.group <= 0 ? 0 : i / a.group;
    g.s = a.S[r * a.G + gi];
    g.z = (float)a.Z[r * a.G + gi];
  }
  g.inv_s = 1.f / g.s;
  g.nz = -g.z;
  g.mz = (float)a.maxq - g.z;
  int next_group = 0;  // GMODE == -1: block-local column of the next group start
  const bool writer = active && lr == 0;
  __syncthreads();

  // factor row p of this lane's 8 columns, prefetched two columns ahead
  f32x4 ua[3], ub[3];
  ua[0] = *(const f32x4*)&Up[0 * PITCH + 8 * lr];
  ub[0] = *(const f32x4*)&Up[0 * PITCH + 8 * lr + 4];
  ua[1] = *(const f32x4*)&Up[1 * PITCH + 8 * lr];
  ub[1] = *(const f32x4*)&Up[1 * PITCH + 8 * lr + 4];

  // one column per step, fully unrolled so that register and DPP lane
  // indices are compile-time constants
  [&]<int... P>(std::integer_sequence<int, P...>) {
    (
        [&] {
          if constexpr (P + 2 < NSTEP) {
            ua[(P + 2) % 3] = *(const f32x4*)&Up[(P + 2) * PITCH + 8 * lr];
            ub[(P + 2) % 3] = *(const f32x4*)&Up[(P + 2) * PITCH + 8 * lr + 4];
          }
          if constexpr (GMODE > 0) {
            if constexpr (P % GMODE == 0) {
              g = group_params<LPR>(v, lr, P, P + GMODE < w ? P + GMODE : w, a.maxq);
              store_params(a, g, r, i + P, writer && P < w);
            }
          } else if constexpr (GMODE < 0) {
            if (P == next_group && P < w) {
              const int c1 = (int)((int64_t)P + a.group < (int64_t)w ? P + a.group : w);
              g = group_params_call<LPR>(v[0], v[1], v[2], v[3], v[4], v[5], v[6], v[7], lr, P, c1, a.maxq);
              store_params(a, g, r, i + P, writer);
              next_group += (int)a.group;
            }
          }
          const float vp = RowOps<LPR>::template bcast<(P >> 3)>(v[P & 7]);
          const float qz = __builtin_amdgcn_fmed3f(rintf(vp * g.inv_s), g.nz, g.mz);
          const float err = fmaf(-g.s, qz, vp);
          if (lr == (P >> 3)) {  // the owner keeps the error and the code of its column
            ek[P & 7] = err;
            qk[P & 7] = qz + g.z;
          }
          const f32x4 u0 = ua[P % 3], u1 = ub[P % 3];
          v[0] = fmaf(-err, u0[0], v[0]);
          v[1] = fmaf(-err, u0[1], v[1]);
          v[2] = fmaf(-err, u0[2], v[2]);
          v[3] = fmaf(-err, u0[3], v[3]);
          v[4] = fmaf(-err, u1[0], v[4]);
          v[5] = fmaf(-err, u1[1], v[5]);
          v[6] = fmaf(-err, u1[2], v[6]);
          v[7] = fmaf(-err, u1[3], v[7]);
        }(),
        ...);
  }(std::make_integer_sequence<int, NSTEP>{});

  // scaled errors e = err / U_pp of this lane's columns, their squares summed over the row
  float eacc = 0.f;
#pragma unroll
  for (int k = 0; k < 8; ++k) {
    ek[k] *= invd[8 * lr + k];
    eacc = fmaf(ek[k], ek[k], eacc);
  }
  if constexpr (LPR == 16) {
    eacc += __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, eacc), 0xB1, 0xF, 0xF, false));
    eacc += __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, eacc), 0x4E, 0xF, 0xF, false));
    eacc += __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, eacc), 0x124, 0xF, 0xF, false));
    eacc += __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, eacc), 0x128, 0xF, 0xF, false));
  } else {
    eacc += __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, eacc), 0xB1, 0xF, 0xF, false));
    eacc += __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, eacc), 0x4E, 0xF, 0xF, false));
  }

  if (active) {
    if (8 * lr + 8 <= w) {
      *(f32x4*)&a.E[r * ELD + 8 * lr] = f32x4{ek[0], ek[1], ek[2], ek[3]};
      *(f32x4*)&a.E[r * ELD + 8 * lr + 4] = f32x4{ek[4], ek[5], ek[6], ek[7]};
      uint32_t lo = 0, hi = 0;
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        lo |= (uint32_t)(int)qk[k] << (8 * k);
        hi |= (uint32_t)(int)qk[k + 4] << (8 * k);
      }
      uint8_t* q = a.Q8 + r * a.n + i + 8 * lr;
      if ((((uintptr_t)q) & 7) == 0) {
        *(uint2*)q = make_uint2(lo, hi);
      } else {
#pragma unroll
        for (int k = 0; k < 8; ++k) q[k] = (uint8_t)(int)qk[k];
      }
    } else {
#pragma unroll
      for (int k = 0; k < 8; ++k) {
        const int c = 8 * lr + k;
        if (c < w) {
          a.E[r * ELD + c] = ek[k];
          a.Q8[r * a.n + i + c] = (uint8_t)(int)qk[k];
        }
      }
    }
    if (lr == 0 && a.err_sq) a.err_sq[r] += eacc;
  }
}

// Per block of B columns starting at i = blk * B: rows p of U[i:i+w, i:i+w]
// divided by U_pp, zero on and below the diagonal, padded to NSTEP x NSTEP,
// followed by 1/U_pp (0 past w).
template <int NSTEP>
// One workgroup per (block, 8 rows of it): every load of the workgroup in
// flight at once.
__global__ __launch_bounds__(256) void diag_blocks_kernel(const float* U, int64_t n, int64_t B, float* out) {
  const int64_t i = (int64_t)blockIdx.x * B;
  const int w = (int)std::min<int64_t>(B, n - i);
  float* dst = out + (int64_t)blockIdx.x * (NSTEP * NSTEP + NSTEP);
  const int p0 = 8 * blockIdx.y;
  constexpr int PER = 8 * NSTEP / 256;  // elements per thread
  float u[PER], d[PER];
#pragma unroll
  for (int k = 0; k < PER; ++k) {
    const int idx = threadIdx.x + 256 * k;
    const int p = p0 + idx / NSTEP, j = idx % NSTEP;
    const bool in = p < w && j < w && j > p;
    u[k] = in ? U[(i + p) * n + i + j] : 0.f;
    d[k] = in ? U[(i + p) * n + i + p] : 1.f;
  }
#pragma unroll
  for (int k = 0; k < PER; ++k) {
    const int idx = threadIdx.x + 256 * k;
    dst[(p0 + idx / NSTEP) * NSTEP + idx % NSTEP] = u[k] / d[k];
  }
  if (threadIdx.x < 8) {
    const int p = p0 + threadIdx.x;
    dst[NSTEP * NSTEP + p] = (p < w) ? 1.f / U[(i + p) * n + i + p] : 0.f;
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

// The same, 8 elements per thread (n % 8 == 0, ldw % 8 == 0, 16-byte aligned W).
template <int DT>
__global__ __launch_bounds__(256) void dequant_x8_kernel(void* W, int64_t ldw, const uint8_t* Q8, const float* S,
                                                         const int32_t* Z, int64_t m, int64_t n, int64_t group,
                                                         int64_t G) {
  for (int64_t r = blockIdx.y; r < m; r += gridDim.y)
    for (int64_t c = 8 * ((int64_t)blockIdx.x * 256 + threadIdx.x); c < n; c += (int64_t)gridDim.x * 2048) {
      const uint2 q = *(const uint2*)(Q8 + r * n + c);
      float y[8];
#pragma unroll
      for (int k = 0; k < 8; ++k) {
        const int64_t g = group <= 0 ? 0 : (c + k) / group;
        const uint32_t qb = ((k < 4 ? q.x : q.y) >> (8 * (k & 3))) & 0xFFu;
        y[k] = S[r * G + g] * ((float)qb - (float)Z[r * G + g]);
      }
      if (DT == 2) {
        *(f32x4*)((float*)W + r * ldw + c) = f32x4{y[0], y[1], y[2], y[3]};
        *(f32x4*)((float*)W + r * ldw + c + 4) = f32x4{y[4], y[5], y[6], y[7]};
      } else {
        uint32_t wv[4];
#pragma unroll
        for (int k = 0; k < 4; ++k) {
          uint16_t lo, hi;
          if (DT == 0) {
            lo = __builtin_bit_cast(uint16_t, (_Float16)y[2 * k]);
            hi = __builtin_bit_cast(uint16_t, (_Float16)y[2 * k + 1]);
          } else {
            lo = f32_to_bf16(y[2 * k]);
            hi = f32_to_bf16(y[2 * k + 1]);
          }
          wv[k] = (uint32_t)lo | ((uint32_t)hi << 16);
        }
        *(uint4*)((uint16_t*)W + r * ldw + c) = uint4{wv[0], wv[1], wv[2], wv[3]};
      }
    }
}

inline size_t align256(size_t b) { return (b + 255) & ~(size_t)255; }

dim3 rows_grid(int64_t cols, int64_t rows) {
  return dim3((unsigned)std::min<int64_t>(cdiv(cols, 256), 64), (unsigned)std::min<int64_t>(rows, 65535));
}

}  // namespace

// Workspace: fp32 working copy V [m x n], codes [m x n] bytes, E [m x 128],
// then the prepared diagonal factor blocks.
inline int nstep_for(int64_t B) { return B <= 32 ? 32 : BMAX; }
inline size_t dblk_bytes(int64_t n, int64_t B) {
  const int64_t ns = nstep_for(B);
  return (size_t)cdiv(n, B) * (size_t)(ns * ns + ns) * 4;
}

size_t quantize_workspace_bytes(int64_t m, int64_t n, int64_t B) {
  if (m < 1 || n < 1 || B < 1) return 0;
  return align256((size_t)m * n * 4) + align256((size_t)m * n) + align256((size_t)m * ELD * 4) + align256(dblk_bytes(n, B));
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
  const int nstep = nstep_for(B);
  const int64_t dstride = (int64_t)nstep * nstep + nstep;

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
  if (nstep == 32) hipLaunchKernelGGL((diag_blocks_kernel<32>), dim3((unsigned)cdiv(n, B), 32 / 8), dim3(256), 0, st, U, n, B, Dblk);
  else hipLaunchKernelGGL((diag_blocks_kernel<BMAX>), dim3((unsigned)cdiv(n, B), BMAX / 8), dim3(256), 0, st, U, n, B, Dblk);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;

  // sweep one block [i, i + w) with its errors written at column eoff of E;
  // on the look-ahead path the kpend columns before it (from column g0) are
  // still to be applied to it
  auto sweep_block = [&](int64_t i, int w, int eoff, bool look, int64_t g0) -> hipError_t {
    if (group > B && i % group == 0)
      hipLaunchKernelGGL(row_params_kernel, dim3(prow), dim3(256), 0, st, (const float*)V, m, n, i, group, maxq, S,
                         Z, G, i / group);
    SweepArgs a{U, V, n, m, i, w, maxq, group, G, S, Z, Q8, E + eoff, err_sq, Dblk + (i / B) * dstride,
                E, (int)(i - g0), U + g0 * n + i};
    if (B <= 32) launch_sweep<4, false>(a, gmode, st);
    else if (look) launch_sweep<16, true>(a, gmode, st);
    else launch_sweep<16, false>(a, gmode, st);
    return hipGetLastError();
  };
  // V[:, c0:c0+N] -= E[:, 0:K] U[r0:r0+K, c0:c0+N]
  auto flush = [&](int64_t r0, int K, int64_t c0, int64_t N) -> hipError_t {
    if (N <= 0) return hipSuccess;
    GemmDesc g{};
    g.A = E; g.lda = ELD;
    g.B = U + r0 * n + c0; g.ldb = n;
    g.C = V + c0; g.ldc = n;
    g.M = (int)m; g.N = (int)N; g.K = K; g.batch = 1;
    g.alpha = -1.f; g.beta = 1.f;
    return gemm_f32(g, false, false, st);
  };
  // (pending K = t B is a multiple of the 64-row chunks; rows of V 16-byte aligned)
  const bool look = B % 64 == 0 && (group <= 0 || group <= B) && n % 4 == 0;
  if (look) {
    // Look-ahead: LA blocks per flush.  Block t of a group first takes the
    // errors of blocks 0..t-1 of its group (inside the sweep kernel, K = t B,
    // on MFMA), then is swept; after the group, one GEMM with K = LA B brings
    // the rest of the row up to date: a quarter of the passes over V and long
    // K per GEMM tile.  (Groups wider than a block would need V updated past
    // the block before their scales are taken, so they stay on the path below.)
    for (int64_t g0 = 0; g0 < n;) {
      int64_t i = g0;
      for (int t = 0; t < LA && i < n; ++t) {
        const int w = (int)std::min<int64_t>(B, n - i);
        if ((e = sweep_block(i, w, (int)(i - g0), true, g0)) != hipSuccess) return e;
        i += w;
      }
      if ((e = flush(g0, (int)(i - g0), i, n - i)) != hipSuccess) return e;
      g0 = i;
    }
  } else {
    for (int64_t i = 0; i < n; i += B) {
      const int w = (int)std::min<int64_t>(B, n - i);
      if ((e = sweep_block(i, w, 0, false, i)) != hipSuccess) return e;
      if ((e = flush(i, w, i + w, n - i - w)) != hipSuccess) return e;
    }
  }
  const int64_t words = cdiv(n * bits, 32);
  hipLaunchKernelGGL(pack_kernel, rows_grid(words, m), dim3(256), 0, st, (const uint8_t*)Q8, m, n, bits, qcodes, words);
  if (write_dequant) {
    if (x8 && dt == 0) hipLaunchKernelGGL((dequant_x8_kernel<0>), rg8, dim3(256), 0, st, W, ldw, (const uint8_t*)Q8, (const float*)S, (const int32_t*)Z, m, n, group, G);
    else if (x8 && dt == 1) hipLaunchKernelGGL((dequant_x8_kernel<1>), rg8, dim3(256), 0, st, W, ldw, (const uint8_t*)Q8, (const float*)S, (const int32_t*)Z, m, n, group, G);
    else if (x8) hipLaunchKernelGGL((dequant_x8_kernel<2>), rg8, dim3(256), 0, st, W, ldw, (const uint8_t*)Q8, (const float*)S, (const int32_t*)Z, m, n, group, G);
    else if (dt == 0) hipLaunchKernelGGL((dequant_kernel<0>), rg, dim3(256), 0, st, W, ldw, (const uint8_t*)Q8, (const float*)S, (const int32_t*)Z, m, n, group, G);
    else if (dt == 1) hipLaunchKernelGGL((dequant_kernel<1>), rg, dim3(256), 0, st, W, ldw, (const uint8_t*)Q8, (const float*)S, (const int32_t*)Z, m, n, group, G);
    else hipLaunchKernelGGL((dequant_kernel<2>), rg, dim3(256), 0, st, W, ldw, (const uint8_t*)Q8, (const float*)S, (const int32_t*)Z, m, n, group, G);
  }
  return hipGetLastError();
}

}  // namespace gptq
