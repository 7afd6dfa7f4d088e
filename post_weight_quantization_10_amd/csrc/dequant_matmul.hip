// Runtime use of a packed layer: Y = X What^T with What = s (q - z), the
// b-bit codes unpacked and dequantized next to 16-bit activations (the
// weight-only path of the English GPTQ second-order quantization post, 'What
// the original results established': speed comes from moving fewer weight
// bytes with a kernel that unpacks them efficiently; its Vietnamese edition
// ends on the same point: the artifact needs a packed INT4 kernel for the
// target device).
//
// How (4-bit codes, fp16 or bf16 activations):
//   * A workgroup owns 64 rows of W (16 per wave) and up to 64 tokens, and
//     walks 512-column slices of K.  A wave's codes for a slice (16 rows x
//     256 bytes) are requested first, 16 bytes per lane; the slice of X goes
//     to LDS meanwhile.
//   * Zero points are folded out of the products.  For a 32-bit word of eight
//     codes, ((w >> 4i) & 0x000F000F) | 0x64006400 is the fp16 pair
//     (1024 + q_i, 1024 + q_{i+4}), and one packed fp16 subtraction of 1024
//     leaves (q_i, q_{i+4}), both exact (bf16: 0x43004300 gives 128 + q, kept
//     as it is: b = 128, else b = 0).  The MFMA
//     v_mfma_f32_16x16x32_{f16,bf16} sums (b + q) x over a 128-column piece
//     (every product is exact in fp32), and once per group and row
//     Y += s (acc - (b + z) sum(x)).  Codes are never turned into weights one
//     by one: about a dozen VALU operations per word of eight codes.
//   * K order: in piece p, lane quarter g of a wave takes words 4g..4g+3 of
//     the piece's 16 (one 16-byte load), one word per MFMA step; X is staged
//     in LDS with the same pair order inside each eight-column word, so the
//     two operands agree.
//   * When rows x token groups alone would leave the GPU under-filled, K is
//     cut into strided sets of slices whose fp32 partial outputs a second
//     kernel sums in a fixed order (deterministic) and converts to X's dtype.
#include <algorithm>

#include "common.hpp"
#include "internal.hpp"

namespace gptq {

namespace {

constexpr int DQ_ROWS = 64;           // rows of W per workgroup, 16 per wave
constexpr int DQ_KR = 512;            // columns per K slice (4 pieces of 128)
constexpr int DQ_TOK = 64;            // tokens per workgroup (4 MFMA column blocks)
constexpr int DQ_XP = DQ_KR + 8;      // LDS pitch of a staged X row (halves): rows 4 banks apart
constexpr int DQ_SLOTS = 512;         // workgroups that fill the GPU (2 per CU)

typedef _Float16 half8_t __attribute__((ext_vector_type(8)));
typedef _Float16 half2_t __attribute__((ext_vector_type(2)));
typedef __bf16 bf168_t __attribute__((ext_vector_type(8)));

struct DqArgs {
  const void* X;
  int64_t ldx, T;
  const uint32_t* Q;
  int64_t W;  // uint32 words per row of codes
  const float* S;
  const int32_t* Z;
  int64_t G, group;  // group <= 0: one group per row
  int64_t m, n;
  float* P;  // partials [KS][T][m], or null: Y written directly
  void* Y;
  int64_t ldy;
  int KS;
};

__device__ __forceinline__ float half_bits_to_f32(uint32_t h, int dt) {
  return dt == 0 ? (float)__builtin_bit_cast(_Float16, (uint16_t)h) : __builtin_bit_cast(float, h << 16);
}

template <int DT>
__global__ __launch_bounds__(256, 2) void dqmm4_kernel(DqArgs a) {
  __shared__ __attribute__((aligned(16))) uint16_t xs[DQ_TOK * DQ_XP];
  __shared__ float xsum[DQ_TOK][DQ_KR / 128];
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int g4 = lane >> 4, l16 = lane & 15;
  const int64_t rbase = (int64_t)blockIdx.x * DQ_ROWS;
  const int64_t t0 = (int64_t)blockIdx.z * DQ_TOK;
  const int nt = (int)min<int64_t>(DQ_TOK, a.T - t0);
  const int ntc = (nt + 15) >> 4;  // 16-token column blocks with work
  constexpr uint32_t MAGIC = DT == 0 ? 0x64006400u : 0x43004300u;
  // fp16: the magic 1024 is taken off again in fp16 (exact), so the sums
  // carry q x only; bf16: 128 + q stays and is folded out with z
  constexpr float BIAS = DT == 0 ? 0.f : 128.f;
  const half2_t m1024 = {(_Float16)1024.f, (_Float16)1024.f};
  auto unbias = [&](uint32_t h) -> uint32_t {
    return DT == 0 ? __builtin_bit_cast(uint32_t, __builtin_bit_cast(half2_t, h) - m1024) : h;
  };

  // codes of this workgroup's rows; rows past m and words past the end read as zero
  const int64_t rows_here = min<int64_t>(DQ_ROWS, a.m - rbase);
  const __amdgpu_buffer_rsrc_t qrs = __builtin_amdgcn_make_buffer_rsrc(
      (void*)(a.Q + rbase * a.W), 0, (int)(rows_here * a.W * 4), 0x00020000);
  const uint32_t qrow = (uint32_t)(16 * wave + l16) * (uint32_t)a.W;

  // output rows of this lane (MFMA result register v: row 4 g4 + v of the wave's 16)
  const int64_t orow0 = rbase + 16 * wave + 4 * g4;
  float tot[4][4];  // [column block][v]
#pragma unroll
  for (int c = 0; c < 4; ++c)
#pragma unroll
    for (int v = 0; v < 4; ++v) tot[c][v] = 0.f;

  const int64_t nslices = cdiv(a.n, DQ_KR);
  for (int64_t ks = blockIdx.y; ks < nslices; ks += a.KS) {
    const int64_t k0 = ks * DQ_KR;
    // this lane's words: k0/8 + 16p + 4 g4 .. +3 for the four pieces p
    u32x4 qw[4];
    const uint32_t qoff = (qrow + (uint32_t)(k0 / 8) + 4u * g4) * 4u;
#pragma unroll
    for (int p = 0; p < 4; ++p) qw[p] = __builtin_amdgcn_raw_buffer_load_b128(qrs, qoff + 64u * p, 0, 0);

    // stage X[t0 .. t0+63][k0 .. k0+511] with the pair order of the unpacked
    // codes inside each 8-column word, and the sum of every 128-column piece
    __syncthreads();  // the previous slice's LDS reads are done
    {
      const int t = tid >> 2, qq = tid & 3;
      float sum = 0.f;
      const bool tok = t < nt;
      const uint16_t* xrow = (const uint16_t*)a.X + (t0 + (tok ? t : 0)) * a.ldx;
#pragma unroll 4
      for (int w = 0; w < 16; ++w) {
        const int64_t c = k0 + 128 * qq + 8 * w;
        u32x4 d = {0u, 0u, 0u, 0u};
        if (tok && c < a.n) d = *(const u32x4*)(xrow + c);
        const u32x4 e = {__builtin_amdgcn_perm(d.z, d.x, 0x05040100u), __builtin_amdgcn_perm(d.z, d.x, 0x07060302u),
                         __builtin_amdgcn_perm(d.w, d.y, 0x05040100u), __builtin_amdgcn_perm(d.w, d.y, 0x07060302u)};
        *(u32x4*)&xs[t * DQ_XP + 128 * qq + 8 * w] = e;
#pragma unroll
        for (int h = 0; h < 4; ++h)
          sum += half_bits_to_f32(d[h] & 0xFFFFu, DT) + half_bits_to_f32(d[h] >> 16, DT);
      }
      xsum[t][qq] = sum;
    }
    __syncthreads();

    // pieces of 128 columns; a group is one or more whole pieces (or the whole
    // row), so a piece never straddles two groups
    f32x4 acc[4];
    float xs_g[4];
#pragma unroll
    for (int p = 0; p < 4; ++p) {
      const int64_t c0 = k0 + 128 * p;
      if (c0 >= a.n) break;  // nothing past the last column (the piece before it closed its group)
      const bool first = p == 0 || (a.group > 0 && c0 % a.group == 0);
      const bool last = p == 3 || c0 + 128 >= a.n || (a.group > 0 && (c0 + 128) % a.group == 0);
      if (first) {
#pragma unroll
        for (int c = 0; c < 4; ++c) {
          acc[c] = f32x4{0.f, 0.f, 0.f, 0.f};
          xs_g[c] = 0.f;
        }
      }
#pragma unroll
      for (int c = 0; c < 4; ++c)
        if (c < ntc) xs_g[c] += xsum[16 * c + l16][p];
#pragma unroll
      for (int st = 0; st < 4; ++st) {
        const uint32_t w = qw[p][st];
        u32x4 ai;
        ai.x = unbias((w & 0x000F000Fu) | MAGIC);
        ai.y = unbias(((w >> 4) & 0x000F000Fu) | MAGIC);
        ai.z = unbias(((w >> 8) & 0x000F000Fu) | MAGIC);
        ai.w = unbias(((w >> 12) & 0x000F000Fu) | MAGIC);
        const int col = 128 * p + 8 * (4 * g4 + st);
#pragma unroll
        for (int c = 0; c < 4; ++c) {
          if (c < ntc) {
            const u32x4 bi = *(const u32x4*)&xs[(16 * c + l16) * DQ_XP + col];
            if (DT == 0)
              acc[c] = __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(half8_t, ai),
                                                             __builtin_bit_cast(half8_t, bi), acc[c], 0, 0, 0);
            else
              acc[c] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf168_t, ai),
                                                              __builtin_bit_cast(bf168_t, bi), acc[c], 0, 0, 0);
          }
        }
      }
      if (last) {  // Y += s (acc - (b + z) sum(x)) for this group, per output row
        const int64_t gi = a.group > 0 ? c0 / a.group : 0;
#pragma unroll
        for (int v = 0; v < 4; ++v) {
          const int64_t r = min<int64_t>(orow0 + v, a.m - 1);
          const float s = a.S[r * a.G + gi];
          const float b = BIAS + (float)a.Z[r * a.G + gi];
#pragma unroll
          for (int c = 0; c < 4; ++c)
            if (c < ntc) tot[c][v] = fmaf(s, fmaf(-b, xs_g[c], acc[c][v]), tot[c][v]);
        }
      }
    }
  }

#pragma unroll
  for (int c = 0; c < 4; ++c) {
    const int64_t t = t0 + 16 * c + l16;
    if (c >= ntc || t >= a.T) continue;
#pragma unroll
    for (int v = 0; v < 4; ++v) {
      const int64_t r = orow0 + v;
      if (r >= a.m) continue;
      if (a.P) a.P[((int64_t)blockIdx.y * a.T + t) * a.m + r] = tot[c][v];
      else Elem<DT>::store(a.Y, t * a.ldy + r, tot[c][v]);
    }
  }
}

// Decode-sized batches (tokens <= 16): every wave streams its own task, 16
// rows over a range of K, with the codes of four 256-column chunks in flight
// and X read straight from L2 (it is small and shared by every wave) two
// chunks ahead; no LDS, no barrier.  X's eight columns of a word are put in
// the pair order of the unpacked codes with four byte permutes.  fp16: the
// zero point leaves with the bias, (1024 + q) - (1024 + z) = q - z exactly,
// so the sums carry (q - z) x and Y += s acc per group.  bf16 (no packed
// bf16 subtract): 128 + q stays, a second MFMA with all-ones weights gives
// sum(x) for the same columns, and Y += s (acc - (128 + z) sum(x)).
// fp16 pairs a - b (exact here: both are 1024 + a small integer); bf16: a
template <int DT>
__device__ __forceinline__ uint32_t hsub(uint32_t a, uint32_t b) {
  if (DT != 0) return a;
  const half2_t d = __builtin_bit_cast(half2_t, a) - __builtin_bit_cast(half2_t, b);
  return __builtin_bit_cast(uint32_t, d);
}

constexpr int DS_CH = 256;      // columns per chunk (two 128-column pieces)
constexpr int DS_AHEAD = 4;     // chunks of codes in flight per wave
constexpr int DS_XAHEAD = 2;    // chunks of X in flight per wave
constexpr int DS_WAVES = 3072;  // waves that keep HBM busy (12 per CU)

// G128: groups of exactly one 128-column piece (the usual g128), so every
// piece opens and closes its group and no bookkeeping is needed.  FULL: n is
// a multiple of 256, so no chunk runs past the end of a row and X needs no
// masking.
template <int DT, bool G128, bool FULL>
__global__ __launch_bounds__(256) void dqmm4_stream_kernel(DqArgs a, int64_t KR) {
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int g4 = lane >> 4, l16 = lane & 15;
  const int64_t task = (int64_t)blockIdx.x * 4 + wave;
  const int64_t RB = cdiv(a.m, 16);
  if (task >= RB * a.KS) return;  // the whole wave: there is no barrier in this kernel
  const int64_t rb = task / a.KS, ks = task % a.KS;
  const int64_t kb = ks * KR, ke = min<int64_t>(a.n, kb + KR);
  const int nch = (int)cdiv(ke - kb, DS_CH);
  constexpr uint32_t MAGIC = DT == 0 ? 0x64006400u : 0x43004300u;

  const int64_t rows_here = min<int64_t>(16, a.m - 16 * rb);
  const __amdgpu_buffer_rsrc_t qrs = __builtin_amdgcn_make_buffer_rsrc(
      (void*)(a.Q + 16 * rb * a.W), 0, (int)(rows_here * a.W * 4), 0x00020000);
  // this lane's words of chunk j: kb/8 + 32 j + 16 p + 4 g4 .. +3 of row l16
  const uint32_t qoff = ((uint32_t)l16 * (uint32_t)a.W + (uint32_t)(kb / 8) + 4u * g4) * 4u;
  // X through a buffer over its T rows: lanes of tokens past T read zeros
  const __amdgpu_buffer_rsrc_t xrs =
      __builtin_amdgcn_make_buffer_rsrc((void*)a.X, 0, (int)(a.T * a.ldx * 2), 0x00020000);
  const uint32_t xoff = (uint32_t)(l16 * a.ldx + kb + 32 * g4) * 2u;
  const int64_t rA = min<int64_t>(16 * rb + l16, a.m - 1);  // row of this lane's codes
  const int64_t rO = 16 * rb + 4 * g4;                      // first of this lane's four output rows
  // scales and zero points through buffers with 32-bit offsets (m G < 2^29)
  const __amdgpu_buffer_rsrc_t srs = __builtin_amdgcn_make_buffer_rsrc((void*)a.S, 0, (int)(a.m * a.G * 4), 0x00020000);
  const __amdgpu_buffer_rsrc_t zrs = __builtin_amdgcn_make_buffer_rsrc((void*)a.Z, 0, (int)(a.m * a.G * 4), 0x00020000);
  const uint32_t zoffA = (uint32_t)(rA * a.G) * 4u;
  uint32_t poff[4];
#pragma unroll
  for (int v = 0; v < 4; ++v) poff[v] = (uint32_t)(min<int64_t>(rO + v, a.m - 1) * a.G) * 4u;
  // 128-column pieces, counted from the wave's first one (kb is a multiple
  // of 256); a group is gp whole pieces (gp = 0: the whole row).  32-bit
  // bookkeeping only: piece P of the range is global piece pb + P.
  const uint32_t pb = (uint32_t)(kb >> 7);
  const int npc = (int)cdiv(ke - kb, 128);
  const uint32_t gp = a.group > 0 ? (uint32_t)(a.group >> 7) : 0u;
  const uint32_t gmax = (uint32_t)(a.G - 1);
  auto group_of = [&](int P) -> uint32_t {
    if (G128) return pb + (uint32_t)P;
    if (gp == 0) return 0u;
    const uint32_t g = gp == 1 ? pb + (uint32_t)P : (pb + (uint32_t)P) / gp;
    return g < gmax ? g : gmax;
  };
  auto starts_group = [&](int P) { return P == 0 || (gp != 0 && (gp == 1 || (pb + (uint32_t)P) % gp == 0)); };
  auto ends_group = [&](int P) {
    return P == npc - 1 || (gp != 0 && (gp == 1 || (pb + (uint32_t)P + 1) % gp == 0));
  };

  u32x4 qb[DS_AHEAD][2];
  u32x4 xb[DS_XAHEAD][8];
  // Every load below is issued unconditionally: past the range they read
  // other rows' values, or zeros past the buffer, and are never used.
  auto load_q = [&](int slot, int j) {
#pragma unroll
    for (int p = 0; p < 2; ++p)
      qb[slot][p] = __builtin_amdgcn_raw_buffer_load_b128(qrs, qoff + 128u * j + 64u * p, 0, 0);
  };
  // Columns past the range (the range's last chunk only): zero, so that
  // whatever the codes there are, they add nothing.
  const int xlim = (int)(ke - kb) - 32 * g4;
  const int nfull = (int)((ke - kb) / DS_CH);  // chunks entirely inside the range
  auto load_x = [&](int slot, int j) {
#pragma unroll
    for (int e = 0; e < 8; ++e) {  // piece e / 4, word e % 4
      const int c = DS_CH * j + 128 * (e >> 2) + 8 * (e & 3);
      xb[slot][e] = __builtin_amdgcn_raw_buffer_load_b128(xrs, xoff + 2u * (uint32_t)c, 0, 0);
    }
    if (!FULL && j >= nfull) {  // uniform
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const int c = DS_CH * j + 128 * (e >> 2) + 8 * (e & 3);
        if (c >= xlim) xb[slot][e] = u32x4{0u, 0u, 0u, 0u};
      }
    }
  };
  // group parameters of the two pieces of a chunk, two chunks ahead: the zero
  // point of this lane's code row; scales (and bf16 zero points) of its four
  // output rows
  int zA[2][2];
  float sO[2][2][4];
  int zO[2][2][4];
  auto load_par = [&](int slot, int j) {
#pragma unroll
    for (int p = 0; p < 2; ++p) {
      const uint32_t gi4 = 4u * group_of(2 * j + p);
      if (DT == 0) zA[slot][p] = __builtin_amdgcn_raw_buffer_load_b32(zrs, zoffA + gi4, 0, 0);
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        sO[slot][p][v] = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(srs, poff[v] + gi4, 0, 0));
        if (DT != 0) zO[slot][p][v] = __builtin_amdgcn_raw_buffer_load_b32(zrs, poff[v] + gi4, 0, 0);
      }
    }
  };
#pragma unroll
  for (int d = 0; d < DS_AHEAD; ++d) load_q(d, d);
#pragma unroll
  for (int d = 0; d < DS_XAHEAD; ++d) load_x(d, d);
  load_par(0, 0);
  load_par(1, 1);

  f32x4 tot = {0.f, 0.f, 0.f, 0.f}, acc = {0.f, 0.f, 0.f, 0.f}, acc1 = {0.f, 0.f, 0.f, 0.f};
  const u32x4 ones = {0x3F803F80u, 0x3F803F80u, 0x3F803F80u, 0x3F803F80u};  // bf16 1.0
  for (int j0 = 0; j0 < nch; j0 += DS_AHEAD) {
#pragma unroll
    for (int d = 0; d < DS_AHEAD; ++d) {
      const int j = j0 + d;
      if (j >= nch) break;
      const int xs = d % DS_XAHEAD;  // DS_AHEAD is a multiple of DS_XAHEAD
#pragma unroll
      for (int p = 0; p < 2; ++p) {
        const int P = 2 * j + p;
        if (!FULL && P >= npc) break;
        const bool first = G128 || starts_group(P);
        const bool last = G128 || ends_group(P);
        if (first) {
          acc = f32x4{0.f, 0.f, 0.f, 0.f};
          acc1 = f32x4{0.f, 0.f, 0.f, 0.f};
        }
        const int ps = d & 1;  // parameter slot of chunk j
        uint32_t zb = 0;       // fp16 (1024 + z, 1024 + z) of this lane's row
        if (DT == 0) {
          const uint32_t z = (uint32_t)zA[ps][p];
          zb = MAGIC | z | (z << 16);
        }
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const uint32_t w = qb[d][p][i];
          // (no bit cast of a vector element below: it would read element 0)
          const uint32_t h0 = hsub<DT>((w & 0x000F000Fu) | MAGIC, zb);
          const uint32_t h1 = hsub<DT>(((w >> 4) & 0x000F000Fu) | MAGIC, zb);
          const uint32_t h2 = hsub<DT>(((w >> 8) & 0x000F000Fu) | MAGIC, zb);
          const uint32_t h3 = hsub<DT>(((w >> 12) & 0x000F000Fu) | MAGIC, zb);
          const u32x4 ai = {h0, h1, h2, h3};
          const u32x4 xv = xb[xs][4 * p + i];
          const u32x4 bi = {__builtin_amdgcn_perm(xv.z, xv.x, 0x05040100u), __builtin_amdgcn_perm(xv.z, xv.x, 0x07060302u),
                            __builtin_amdgcn_perm(xv.w, xv.y, 0x05040100u), __builtin_amdgcn_perm(xv.w, xv.y, 0x07060302u)};
          if (DT == 0) {
            acc = __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(half8_t, ai), __builtin_bit_cast(half8_t, bi),
                                                         acc, 0, 0, 0);
          } else {
            acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf168_t, ai),
                                                          __builtin_bit_cast(bf168_t, bi), acc, 0, 0, 0);
            acc1 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf168_t, ones),
                                                           __builtin_bit_cast(bf168_t, bi), acc1, 0, 0, 0);
          }
        }
        if (last) {
#pragma unroll
          for (int v = 0; v < 4; ++v) {
            const float sc = sO[ps][p][v];
            if (DT == 0) tot[v] = fmaf(sc, acc[v], tot[v]);
            else tot[v] = fmaf(sc, fmaf(-(128.f + (float)zO[ps][p][v]), acc1[v], acc[v]), tot[v]);
          }
        }
      }
      load_q(d, j + DS_AHEAD);
      load_x(xs, j + DS_XAHEAD);
      load_par(d & 1, j + 2);
    }
  }

  const int64_t t = l16;
  if (t < a.T) {
#pragma unroll
    for (int v = 0; v < 4; ++v) {
      const int64_t r = rO + v;
      if (r >= a.m) continue;
      if (a.P) a.P[(ks * a.T + t) * a.m + r] = tot[v];
      else Elem<DT>::store(a.Y, t * a.ldy + r, tot[v]);
    }
  }
}

// Y[t][r] = sum over the K sets of the partials, in set order, in X's dtype.
template <int DT>
__global__ __launch_bounds__(256) void dqmm_reduce_kernel(const float* P, int KS, int64_t T, int64_t m, void* Y,
                                                          int64_t ldy) {
  for (int64_t t = blockIdx.y; t < T; t += gridDim.y)
    for (int64_t r = (int64_t)blockIdx.x * 256 + threadIdx.x; r < m; r += (int64_t)gridDim.x * 256) {
      float s = 0.f;
      for (int k = 0; k < KS; ++k) s += P[((int64_t)k * T + t) * m + r];
      Elem<DT>::store(Y, t * ldy + r, s);
    }
}

// K sets and the columns of each: the staged kernel for more than 16 tokens
// (slices of 512), the streaming kernel for up to 16 (ranges of whole
// 256-column chunks, enough waves to keep HBM busy, at least 512 columns
// each)
struct DqSplit {
  int ks;
  int64_t kr;
};
DqSplit dq_split(int64_t T, int64_t m, int64_t n) {
  if (T > 16) {
    const int64_t base = cdiv(m, DQ_ROWS) * cdiv(T, DQ_TOK);
    if (base >= DQ_SLOTS) return {1, cdiv(n, DQ_KR) * DQ_KR};
    return {(int)std::min<int64_t>(cdiv(n, DQ_KR), cdiv(DQ_SLOTS, base)), DQ_KR};
  }
  const int64_t rb = cdiv(m, 16);
  const int64_t want = std::max<int64_t>(1, std::min<int64_t>(cdiv(DS_WAVES, rb), cdiv(n, 512)));
  const int64_t kr = cdiv(cdiv(n, want), DS_CH) * DS_CH;
  return {(int)cdiv(n, kr), kr};
}

}  // namespace

size_t dequant_matmul_workspace_bytes(int64_t tokens, int64_t m, int64_t n) {
  if (tokens < 1 || m < 1 || n < 1) return 0;
  const int ks = dq_split(tokens, m, n).ks;
  return ks > 1 ? (size_t)ks * (size_t)tokens * (size_t)m * 4 : 0;
}

bool dequant_matmul_supported(int bits, int64_t n, int64_t group) {
  return bits == 4 && n % 32 == 0 && (group <= 0 || group % 128 == 0);
}

hipError_t dequant_matmul(const void* X, int dt, int64_t T, int64_t ldx, const uint32_t* Q, const float* S,
                          const int32_t* Z, int64_t m, int64_t n, int64_t group, void* Y, int64_t ldy, void* ws,
                          hipStream_t st) {
  if (T == 0) return hipSuccess;
  DqArgs a{};
  a.X = X; a.ldx = ldx; a.T = T;
  a.Q = Q; a.W = cdiv(n * 4, 32);
  a.S = S; a.Z = Z; a.group = group; a.G = group > 0 ? cdiv(n, group) : 1;
  a.m = m; a.n = n; a.Y = Y; a.ldy = ldy;
  const DqSplit sp = dq_split(T, m, n);
  a.KS = sp.ks;
  a.P = a.KS > 1 ? (float*)ws : nullptr;
  if (T <= 16) {
    const dim3 grid((unsigned)cdiv(cdiv(m, 16) * a.KS, 4));
    const bool g128 = group == 128, full = n % DS_CH == 0;
#define DQ_STREAM(D, G, F) hipLaunchKernelGGL((dqmm4_stream_kernel<D, G, F>), grid, dim3(256), 0, st, a, sp.kr)
    if (dt == 0) {
      if (g128) { if (full) DQ_STREAM(0, true, true); else DQ_STREAM(0, true, false); }
      else { if (full) DQ_STREAM(0, false, true); else DQ_STREAM(0, false, false); }
    } else {
      if (g128) { if (full) DQ_STREAM(1, true, true); else DQ_STREAM(1, true, false); }
      else { if (full) DQ_STREAM(1, false, true); else DQ_STREAM(1, false, false); }
    }
#undef DQ_STREAM
  } else {
    const dim3 grid((unsigned)cdiv(m, DQ_ROWS), (unsigned)a.KS, (unsigned)cdiv(T, DQ_TOK));
    if (dt == 0) hipLaunchKernelGGL(dqmm4_kernel<0>, grid, dim3(256), 0, st, a);
    else hipLaunchKernelGGL(dqmm4_kernel<1>, grid, dim3(256), 0, st, a);
  }
  if (a.KS > 1) {
    const dim3 rg((unsigned)std::min<int64_t>(cdiv(m, 256), 64), (unsigned)std::min<int64_t>(T, 65535));
    if (dt == 0) hipLaunchKernelGGL(dqmm_reduce_kernel<0>, rg, dim3(256), 0, st, (const float*)a.P, a.KS, T, m, Y, ldy);
    else hipLaunchKernelGGL(dqmm_reduce_kernel<1>, rg, dim3(256), 0, st, (const float*)a.P, a.KS, T, m, Y, ldy);
  }
  return hipGetLastError();
}

}  // namespace gptq
