// Causal multi-head softmax attention for the network-level loop (one layer
// at a time, each layer's calibration inputs computed by the network as
// quantized so far: "Part 3: Adaptive Rounding: GPTQ", 'Algorithm GPTQ'; the
// English GPTQ second-order quantization post, 'Calibration for a multimodal
// or VLA backbone').  Between the quantized q/k/v projections and the
// quantized o projection of a block:
//
//   O[i, h] = sum_{j <= i, same sequence} p_ij V[j, h],
//   p_ij = softmax_j (Q[i, h] . K[j, h] / sqrt(dh))
//
// for every head h (columns h dh .. h dh + dh - 1 of the activations).  fp32
// throughout, one rounding of O to the activations' dtype.
//
// One wave per 64 (64-dim heads) or 32 (128-dim heads) consecutive queries of
// one head (a query block never straddles a sequence: the sequence length is a
// multiple of 64); a lane owns 64 dims of one query's scaled query and output
// rows in registers (16-byte loads and stores: 16-byte aligned rows).  Keys and
// values stream through LDS in tiles of 32 (fp32); per tile every lane takes
// its 32 scores (masked past its own position), rescales its output once by
// e^(m_old - m_new) with the tile's running maximum (the online softmax), and
// adds p V.  VALU-bound: 2 dh FMAs per (query, key) pair.
#include <cmath>

#include "common.hpp"
#include "internal.hpp"

namespace gptq {

namespace {

constexpr int AQ = 64;  // queries per workgroup (one wave)
constexpr int AK = 32;  // keys per LDS tile

struct AttnArgs {
  const void* Q;
  const void* K;
  const void* V;
  void* O;
  int64_t T, S, heads, ld;
};

// 8 16-bit values (one 16-byte word) <-> floats
template <int DT>
__device__ __forceinline__ void h8_to_f(u32x4 v, float* f) {
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    const uint32_t w = v[e];
    if (DT == 0) {
      f[2 * e] = (float)__builtin_bit_cast(_Float16, (uint16_t)(w & 0xFFFFu));
      f[2 * e + 1] = (float)__builtin_bit_cast(_Float16, (uint16_t)(w >> 16));
    } else {
      f[2 * e] = __builtin_bit_cast(float, w << 16);
      f[2 * e + 1] = __builtin_bit_cast(float, w & 0xFFFF0000u);
    }
  }
}
template <int DT>
__device__ __forceinline__ u32x4 f_to_h8(const float* f) {
  u32x4 v;
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    uint16_t lo, hi;
    if (DT == 0) {
      lo = __builtin_bit_cast(uint16_t, (_Float16)f[2 * e]);
      hi = __builtin_bit_cast(uint16_t, (_Float16)f[2 * e + 1]);
    } else {
      lo = f32_to_bf16(f[2 * e]);
      hi = f32_to_bf16(f[2 * e + 1]);
    }
    v[e] = (uint32_t)lo | ((uint32_t)hi << 16);
  }
  return v;
}

// LQ = DH / 64 adjacent lanes per query (a 128-dim head is split over two
// lanes, 64 dims each, their partial scores added with one DPP swap), so a
// lane holds 64 query and 64 output values; a wave takes 64 / LQ queries.
template <int DT, int DH>
__global__ __launch_bounds__(AQ) void attention_kernel(AttnArgs a) {
  constexpr int LQ = DH / 64, DL = DH / LQ, QW = AQ / LQ;  // lanes per query, dims per lane, queries per wave
  __shared__ __attribute__((aligned(16))) float ks[AK][DH];
  __shared__ __attribute__((aligned(16))) float vs[AK][DH];
  const int lane = threadIdx.x;
  const int64_t q0 = (int64_t)blockIdx.x * QW;
  const int64_t hc = (int64_t)blockIdx.y * DH;  // first column of the head
  const int64_t i = q0 + lane / LQ;
  const int dl0 = DL * (lane % LQ);  // this lane's first dim of the head
  const bool valid = i < a.T;
  const int64_t seq0 = (q0 / a.S) * a.S;
  const float scale = 1.f / sqrtf((float)DH);
  const uint16_t* Qp = (const uint16_t*)a.Q;
  const uint16_t* Kp = (const uint16_t*)a.K;
  const uint16_t* Vp = (const uint16_t*)a.V;

  float q[DL], o[DL];
  {
    const int64_t ii = valid ? i : a.T - 1;
#pragma unroll
    for (int d = 0; d < DL; d += 8) h8_to_f<DT>(*(const u32x4*)(Qp + ii * a.ld + hc + dl0 + d), q + d);
#pragma unroll
    for (int d = 0; d < DL; ++d) {
      q[d] *= scale;
      o[d] = 0.f;
    }
  }
  float m = -INFINITY, l = 0.f;
  const int64_t kend = min<int64_t>(q0 + QW, a.T);  // keys past the block's last query are masked for all
  for (int64_t kb = seq0; kb < kend; kb += AK) {
    __syncthreads();  // the previous tile is consumed
    // tile: AK keys x DH of K and of V, 16-byte words, AK * DH / 8 / AQ per lane each
#pragma unroll
    for (int u = 0; u < AK * DH / 8 / AQ; ++u) {
      const int e = lane + AQ * u;
      const int jj = e / (DH / 8), d = 8 * (e % (DH / 8));
      const int64_t j = min<int64_t>(kb + jj, a.T - 1);  // keys past T are masked below
      float f[8];
      h8_to_f<DT>(*(const u32x4*)(Kp + j * a.ld + hc + d), f);
      *(f32x4*)&ks[jj][d] = f32x4{f[0], f[1], f[2], f[3]};
      *(f32x4*)&ks[jj][d + 4] = f32x4{f[4], f[5], f[6], f[7]};
      h8_to_f<DT>(*(const u32x4*)(Vp + j * a.ld + hc + d), f);
      *(f32x4*)&vs[jj][d] = f32x4{f[0], f[1], f[2], f[3]};
      *(f32x4*)&vs[jj][d + 4] = f32x4{f[4], f[5], f[6], f[7]};
    }
    __syncthreads();
    float s[AK];
    float mt = -INFINITY;
#pragma unroll
    for (int jj = 0; jj < AK; ++jj) {
      float dot = 0.f;
#pragma unroll
      for (int d = 0; d < DL; d += 4) {
        const f32x4 k4 = *(const f32x4*)&ks[jj][dl0 + d];
        dot = fmaf(q[d], k4[0], dot);
        dot = fmaf(q[d + 1], k4[1], dot);
        dot = fmaf(q[d + 2], k4[2], dot);
        dot = fmaf(q[d + 3], k4[3], dot);
      }
      if constexpr (LQ == 2)  // the partner lane's half (lanes 2q, 2q + 1)
        dot += __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, dot), 0xB1, 0xF, 0xF, false));
      s[jj] = (kb + jj <= i) ? dot : -INFINITY;
      mt = fmaxf(mt, s[jj]);
    }
    // the first tile always holds a visible key (key seq0 <= i), so after it
    // the running maximum is finite; before it c = e^-inf = 0
    const float mn = fmaxf(m, mt);
    const float c = expf(m - mn);
    float ps = 0.f;
#pragma unroll
    for (int jj = 0; jj < AK; ++jj) {
      s[jj] = expf(s[jj] - mn);  // masked keys: e^-inf = 0
      ps += s[jj];
    }
    l = fmaf(l, c, ps);
#pragma unroll
    for (int d = 0; d < DL; ++d) o[d] *= c;
#pragma unroll
    for (int jj = 0; jj < AK; ++jj) {
#pragma unroll
      for (int d = 0; d < DL; d += 4) {
        const f32x4 v4 = *(const f32x4*)&vs[jj][dl0 + d];
        o[d] = fmaf(s[jj], v4[0], o[d]);
        o[d + 1] = fmaf(s[jj], v4[1], o[d + 1]);
        o[d + 2] = fmaf(s[jj], v4[2], o[d + 2]);
        o[d + 3] = fmaf(s[jj], v4[3], o[d + 3]);
      }
    }
    m = mn;
  }
  if (!valid) return;
  const float inv = 1.f / l;
#pragma unroll
  for (int d = 0; d < DL; ++d) o[d] *= inv;
  uint16_t* Op = (uint16_t*)a.O;
#pragma unroll
  for (int d = 0; d < DL; d += 8) *(u32x4*)(Op + i * a.ld + hc + dl0 + d) = f_to_h8<DT>(o + d);
}

}  // namespace

bool attention_supported(int64_t seq_len, int64_t head_dim) {
  return (head_dim == 64 || head_dim == 128) && seq_len % AQ == 0;
}

hipError_t attention(const void* Q, const void* K, const void* V, void* O, int dt, int64_t T, int64_t S,
                     int64_t heads, int64_t dh, int64_t ld, hipStream_t st) {
  if (T == 0) return hipSuccess;
  AttnArgs a{Q, K, V, O, T, S, heads, ld};
  const dim3 grid((unsigned)cdiv(T, AQ / (dh / 64)), (unsigned)heads);
  if (dt == 0 && dh == 64) hipLaunchKernelGGL((attention_kernel<0, 64>), grid, dim3(AQ), 0, st, a);
  else if (dt == 0) hipLaunchKernelGGL((attention_kernel<0, 128>), grid, dim3(AQ), 0, st, a);
  else if (dh == 64) hipLaunchKernelGGL((attention_kernel<1, 64>), grid, dim3(AQ), 0, st, a);
  else hipLaunchKernelGGL((attention_kernel<1, 128>), grid, dim3(AQ), 0, st, a);
  return hipGetLastError();
}

}  // namespace gptq
