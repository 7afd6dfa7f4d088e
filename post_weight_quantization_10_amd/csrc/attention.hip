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
// accuracy throughout, one rounding of O to the activations' dtype.
//
// On the matrix cores: a workgroup takes 64 consecutive queries of one head
// (a query block never straddles a sequence: the sequence length is a multiple
// of 64) and walks the sequence's keys in tiles of 64 up to its diagonal.
// Wave (wq, wk) owns queries 32 wq .. and keys 32 wk .. of each tile:
//   * S^T = K Q^T with v_mfma_f32_32x32x16_{f16,bf16}: 16-bit inputs, so every
//     product is exact and the sums are fp32; a lane holds one query's scores
//     for 16 keys (its query's Q operand stays in registers for all tiles);
//   * online softmax in fp32: the tile's maximum per query over both key
//     halves through LDS, the output rescaled once per tile;
//   * O += P V with v_mfma_f32_32x32x2f32 (fp32 probabilities, V converted
//     exactly from 16 bits, staged per tile in LDS as fp32): the MFMA step
//     that lane half h feeds key 8 (s / 4) + 4 h + s % 4 takes the lane's own
//     probability register s, so P never moves between lanes.
// The two key halves' outputs and sums meet in LDS at the end.
#include <cmath>

#include "common.hpp"
#include "internal.hpp"

namespace gptq {

namespace {

struct AttnArgs {
  const void* Q;
  const void* K;
  const void* V;
  void* O;
  int64_t T, S, heads, ld;
};

// 8 16-bit values (one 16-byte word) -> floats
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
__device__ __forceinline__ f32x16 mfma_qk(u32x4 a, u32x4 b, const f32x16& c) {
  if constexpr (DT == 0)
    return __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(half8, a), __builtin_bit_cast(half8, b), c, 0,
                                                  0, 0);
  else
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a), __builtin_bit_cast(bf16x8, b), c,
                                                   0, 0, 0);
}

template <int DT, int DH>
__global__ __launch_bounds__(256) void attention_kernel(AttnArgs a) {
  constexpr int NS = DH / 16;  // S^T MFMA steps over the head's dims
  constexpr int NB = DH / 32;  // 32-dim blocks of the output
  constexpr int VP = DH + 4;   // LDS pitch of a staged V row (floats)
  static_assert(2 * NB * 16 * 64 <= 64 * VP, "the end's exchange fits over the V tile");
  __shared__ __attribute__((aligned(16))) float vs[64 * VP];
  __shared__ float mx[2][2][32];  // [wq][wk][query]: a tile's maximum of each key half
  __shared__ float cb[4][32];     // per wave: this tile's rescale factor of each query
  __shared__ float lb[2][32];     // [wq][query]: the second key half's sum of p
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wq = wave >> 1, wk = wave & 1;
  const int lq = lane & 31, h = lane >> 5;
  const int64_t q0 = (int64_t)blockIdx.x * 64;
  const int64_t hc = (int64_t)blockIdx.y * DH;  // first column of the head
  const int64_t seq0 = (q0 / a.S) * a.S;
  const int64_t myq = q0 + 32 * wq + lq;  // this lane's query (a column of S^T)
  const float scale = 1.f / sqrtf((float)DH);
  const uint16_t* Qp = (const uint16_t*)a.Q;
  const uint16_t* Kp = (const uint16_t*)a.K;
  const uint16_t* Vp = (const uint16_t*)a.V;

  // B operand of S^T = K Q^T: lane l gives Q^T[dims 16 s + 8 h .. + 7][query lq]
  u32x4 qop[NS];
#pragma unroll
  for (int s = 0; s < NS; ++s) qop[s] = *(const u32x4*)(Qp + myq * a.ld + hc + 16 * s + 8 * h);

  f32x16 o[NB];
#pragma unroll
  for (int b = 0; b < NB; ++b) o[b] = zero16();
  float m = -INFINITY, lsum = 0.f;  // running maximum of this lane's query; this lane's share of the sum
  for (int64_t kb = seq0; kb <= q0; kb += 64) {
    // A operand: lane l gives K[key kb + 32 wk + lq][dims 16 s + 8 h .. + 7]
    u32x4 kop[NS];
    const int64_t mykey = kb + 32 * wk + lq;
#pragma unroll
    for (int s = 0; s < NS; ++s) kop[s] = *(const u32x4*)(Kp + mykey * a.ld + hc + 16 * s + 8 * h);
    // the tile of V, 16-byte words
    constexpr int VW = 64 * DH / 8 / 256;  // words per thread
    u32x4 vv[VW];
#pragma unroll
    for (int u = 0; u < VW; ++u) {
      const int e = tid + 256 * u;
      vv[u] = *(const u32x4*)(Vp + (kb + e / (DH / 8)) * a.ld + hc + 8 * (e % (DH / 8)));
    }
    __syncthreads();  // every wave is done with the previous tile's V and maxima
#pragma unroll
    for (int u = 0; u < VW; ++u) {
      const int e = tid + 256 * u;
      float f[8];
      h8_to_f<DT>(vv[u], f);
      float* dst = vs + (e / (DH / 8)) * VP + 8 * (e % (DH / 8));
      *(f32x4*)dst = f32x4{f[0], f[1], f[2], f[3]};
      *(f32x4*)(dst + 4) = f32x4{f[4], f[5], f[6], f[7]};
    }
    // scores: st[r] = S^T[key kb + 32 wk + 8 (r / 4) + 4 h + r % 4][query myq]
    f32x16 st = zero16();
#pragma unroll
    for (int s = 0; s < NS; ++s) st = mfma_qk<DT>(kop[s], qop[s], st);
    float mt = -INFINITY;
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int64_t key = kb + 32 * wk + 8 * (r >> 2) + 4 * h + (r & 3);
      st[r] = key <= myq ? st[r] * scale : -INFINITY;
      mt = fmaxf(mt, st[r]);
    }
    mt = fmaxf(mt, __shfl_xor(mt, 32));  // the query's other 16 keys of this key half
    if (h == 0) mx[wq][wk][lq] = mt;
    __syncthreads();  // V staged, both key halves' maxima published
    // every query of the block sees key seq0 <= itself, so after the first tile
    // the maximum is finite; before it the factor is e^-inf = 0
    const float mn = fmaxf(m, fmaxf(mt, mx[wq][wk ^ 1][lq]));
    const float c = expf(m - mn);
    float ps = 0.f;
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      st[r] = expf(st[r] - mn);  // masked keys: e^-inf = 0
      ps += st[r];
    }
    lsum = fmaf(lsum, c, ps);
    m = mn;
    // the output's registers hold queries 8 (r / 4) + 4 h + r % 4: their factors through LDS
    if (h == 0) cb[wave][lq] = c;  // read back by this wave only, in order
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const float cr = cb[wave][8 * (r >> 2) + 4 * h + (r & 3)];
#pragma unroll
      for (int b = 0; b < NB; ++b) o[b][r] *= cr;
    }
    // O += P V: step s takes key 8 (s / 4) + 4 h + s % 4 of this key half from
    // lane half h (A[query lq][h] = its probability register s) and the
    // matching row of V (B[h][dim 32 b + lq])
#pragma unroll
    for (int s = 0; s < 16; ++s) {
      const float* vrow = vs + (32 * wk + 8 * (s >> 2) + 4 * h + (s & 3)) * VP + lq;
#pragma unroll
      for (int b = 0; b < NB; ++b)
        o[b] = __builtin_amdgcn_mfma_f32_32x32x2f32(st[s], vrow[32 * b], o[b], 0, 0, 0);
    }
  }

  // the two key halves: O = (o_0 + o_1) / (l_0 + l_1), with the same running
  // maxima on both sides
  const float lw = lsum + __shfl_xor(lsum, 32);  // this wave's sum for query lq
  __syncthreads();  // the last tile's V is consumed: its space takes the exchange
  float* ox = vs + wq * (NB * 16 * 64);
  if (wk == 1) {
#pragma unroll
    for (int b = 0; b < NB; ++b)
#pragma unroll
      for (int r = 0; r < 16; ++r) ox[(b * 16 + r) * 64 + lane] = o[b][r];
    if (h == 0) lb[wq][lq] = lw;
  }
  __syncthreads();
  if (wk == 1) return;
  if (h == 0) cb[wave][lq] = lw + lb[wq][lq];  // the query's whole sum (read back by this wave)
  uint16_t* Op = (uint16_t*)a.O;
#pragma unroll
  for (int r = 0; r < 16; ++r) {
    const int ql = 8 * (r >> 2) + 4 * h + (r & 3);
    const float inv = 1.f / cb[wave][ql];
    const int64_t q = q0 + 32 * wq + ql;
#pragma unroll
    for (int b = 0; b < NB; ++b) {
      const float v = (o[b][r] + ox[(b * 16 + r) * 64 + lane]) * inv;
      Op[q * a.ld + hc + 32 * b + lq] = DT == 0 ? __builtin_bit_cast(uint16_t, (_Float16)v) : f32_to_bf16(v);
    }
  }
}

}  // namespace

bool attention_supported(int64_t seq_len, int64_t head_dim) {
  return (head_dim == 64 || head_dim == 128) && seq_len % 64 == 0;
}

hipError_t attention(const void* Q, const void* K, const void* V, void* O, int dt, int64_t T, int64_t S,
                     int64_t heads, int64_t dh, int64_t ld, hipStream_t st) {
  if (T == 0) return hipSuccess;
  AttnArgs a{Q, K, V, O, T, S, heads, ld};
  const dim3 grid((unsigned)(T / 64), (unsigned)heads);  // T is a multiple of S, itself a multiple of 64
  if (dt == 0 && dh == 64) hipLaunchKernelGGL((attention_kernel<0, 64>), grid, dim3(256), 0, st, a);
  else if (dt == 0) hipLaunchKernelGGL((attention_kernel<0, 128>), grid, dim3(256), 0, st, a);
  else if (dh == 64) hipLaunchKernelGGL((attention_kernel<1, 64>), grid, dim3(256), 0, st, a);
  else hipLaunchKernelGGL((attention_kernel<1, 128>), grid, dim3(256), 0, st, a);
  return hipGetLastError();
}

}  // namespace gptq
