// Runtime use of a packed layer: Y = X What^T with What = s (q - z), the
// b-bit codes unpacked and dequantized next to 16-bit activations (the
// weight-only path of the English GPTQ second-order quantization post, 'What
// the original results established': speed comes from moving fewer weight
// bytes with a kernel that unpacks them efficiently; its Vietnamese edition
// ends on the same point: the artifact needs a packed INT4 kernel for the
// target device).
//
// How (4-bit and 3-bit codes, fp16 or bf16 activations; 3-bit rows are
// bit-streams whose codes straddle words, turned into the 4-bit layout in
// registers right after their load):
//   * Up to 16 tokens (decode): a workgroup takes 64 rows of W over one K
//     range of 512 or 1024 columns; each wave requests all of its codes at
//     once while the workgroup stages X and the group parameters in LDS.
//     More tokens, fp16, at least 128 tiles of 128 tokens x 128 rows: a
//     GEMM-shaped kernel (X staged in LDS, codes unpacked in registers as the
//     MFMA's other operand).  Otherwise a workgroup owns 64 rows and up to 64
//     tokens and walks
//     512-column slices of K; a wave's codes for a slice (16 rows x 256
//     bytes) are requested first, 16 bytes per lane; the slice of X goes to
//     LDS meanwhile.
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
//   * When K is cut (always for decode; for more tokens when rows x token
//     groups alone would leave the GPU under-filled), the fp32 partial
//     outputs of the K sets are summed by a second kernel in a fixed order
//     (deterministic) and converted to X's dtype.
#include <algorithm>
#include <mutex>

#include "common.hpp"
#include "internal.hpp"

// Fixed device buffer for the partial sums of dequant_matmul_static (callers
// that cannot allocate).  Each GPU the library runs on holds its own copy
// until the process ends; host code reaches it only through the address
// hipGetSymbolAddress returns for the current device (the array's name is a
// host-side stand-in, not a device address).
static __device__ __align__(256) unsigned char scratch[gptq::kStaticScratchBytes];

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
typedef uint32_t u32x3 __attribute__((ext_vector_type(3)));

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

// 32 3-bit codes (a little-endian 96-bit stream w0 w1 w2, code c at bit 3c)
// as four words of eight 4-bit codes (code 8i + k at bits 4k of word i): the
// layout the 4-bit path unpacks.  Per word, the 24-bit window of its eight
// codes is spread 3 -> 4 bits in three mask-and-shift steps.
__device__ __forceinline__ u32x4 spread3(uint32_t w0, uint32_t w1, uint32_t w2) {
  const uint32_t win[4] = {w0 & 0xFFFFFFu, __builtin_amdgcn_alignbit(w1, w0, 24) & 0xFFFFFFu,
                           __builtin_amdgcn_alignbit(w2, w1, 16) & 0xFFFFFFu, w2 >> 8};
  u32x4 out;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const uint32_t t = win[i];
    const uint32_t x = (t & 0xFFFu) | ((t & 0xFFF000u) << 4);         // codes 0-3 | 4-7 at bits 0 | 16, 3 apart
    const uint32_t y = (x & 0x003F003Fu) | ((x & 0x0FC00FC0u) << 2);  // pairs at bits 0 | 8 | 16 | 24, 3 apart
    out[i] = (y & 0x07070707u) | ((y & 0x38383838u) << 1);           // 4 apart
  }
  return out;
}

// BITS = 3: a lane's 32 codes of a piece are three words (a 12-byte load),
// turned into the 4-bit layout by spread3.
template <int DT, int BITS>
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
    // this lane's words of the four pieces p: 4 bits: k0/8 + 16p + 4 g4 .. +3;
    // 3 bits: 3 k0/32 + 12p + 3 g4 .. +2, spread to the 4-bit layout
    u32x4 qw[4];
    const uint32_t qoff = (qrow + (uint32_t)(k0 * BITS / 32) + (uint32_t)BITS * g4) * 4u;
#pragma unroll
    for (int p = 0; p < 4; ++p) {
      if constexpr (BITS == 4) {
        qw[p] = __builtin_amdgcn_raw_buffer_load_b128(qrs, qoff + 64u * p, 0, 0);
      } else {
        const u32x3 c = __builtin_amdgcn_raw_buffer_load_b96(qrs, qoff + 48u * p, 0, 0);
        qw[p] = spread3(c.x, c.y, c.z);
      }
    }

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

// fp16 pairs a - b (exact here: both are 1024 + a small integer); bf16: a
template <int DT>
__device__ __forceinline__ uint32_t hsub(uint32_t a, uint32_t b) {
  if (DT != 0) return a;
  const half2_t d = __builtin_bit_cast(half2_t, a) - __builtin_bit_cast(half2_t, b);
  return __builtin_bit_cast(uint32_t, d);
}

// Decode-sized batches (tokens <= 16), one task per workgroup: 64 rows of W
// (16 per wave) over a range of KR columns.  Each wave asks for all of its
// codes at once (KR / 128 loads of 16 bytes per lane: 8 KiB per wave at
// KR = 1024), so a CU keeps tens of KiB of codes in flight with no loop and
// no wait inside a wave; meanwhile the workgroup stages the range's slice of
// X (in the pair order of the unpacked codes) and the scale and zero point
// of each (row, piece) in LDS.  Lane
// (g4, l16) holds words 4 g4 .. 4 g4 + 3 of row l16 in every 128-column
// piece, one word per MFMA step, and reads the same columns of token l16 of
// the staged X.  fp16: the zero point leaves with the bias,
// (1024 + q) - (1024 + z) = q - z exactly, so the sums carry (q - z) x and
// Y += s acc per group.  bf16 (no packed bf16 subtract): 128 + q stays, a
// second MFMA with all-ones weights gives sum(x) for the same columns, and
// Y += s (acc - (128 + z) sum(x)).  Tokens past T read whatever the staged
// rows hold: they only reach output columns that are never written.  Columns
// past n are staged as zeros, so the codes there (another row's, or zeros
// past the buffer) add nothing.
// BITS = 3: each lane's 32 codes of a piece are three words (a 12-byte load)
// turned into the 4-bit layout by spread3; everything else as for 4 bits.
template <int DT, bool G128, int KR, int TT, int BITS>
__global__ __launch_bounds__(256) void dqmm4_task_kernel(DqArgs a) {
  constexpr int NP = KR / 128;     // pieces per range
  constexpr int XP = KR * 2 + 16;  // LDS bytes per staged token row (rows 4 banks apart)
  constexpr int NXW = TT * KR / 8 / 256;  // staged 8-column words per thread (upper bound)
  static_assert(NP % 4 == 0 && NXW >= 1, "range of whole groups of four pieces");
  __shared__ __attribute__((aligned(16))) char xs[TT * XP];
  __shared__ float ps[64][NP + 1];
  __shared__ int pz[64][NP + 1];
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int g4 = lane >> 4, l16 = lane & 15;
  // consecutive workgroups take consecutive row blocks of one K range
  const int64_t nrb = cdiv(a.m, 64);
  const int64_t rb = blockIdx.x % nrb, ks = blockIdx.x / nrb;
  const int64_t kb = ks * KR;
  const int64_t r0 = rb * 64;
  const int64_t rw = r0 + 16 * wave;
  constexpr uint32_t MAGIC = DT == 0 ? 0x64006400u : 0x43004300u;

  // group of piece P of the range (clamped: pieces past n add nothing)
  const uint32_t pb = (uint32_t)(kb >> 7);
  const uint32_t gp = a.group > 0 ? (uint32_t)(a.group >> 7) : 0u;
  const uint32_t gmax = (uint32_t)(a.G - 1);
  auto group_of = [&](int P) -> uint32_t {
    uint32_t g;
    if (G128) g = pb + (uint32_t)P;
    else if (gp == 0) g = 0u;
    else g = gp == 1 ? pb + (uint32_t)P : (pb + (uint32_t)P) / gp;
    return g < gmax ? g : gmax;
  };

  // 1. parameters: thread e = tid + 256 u takes (row e / NP, piece e % NP)
  const __amdgpu_buffer_rsrc_t srs = __builtin_amdgcn_make_buffer_rsrc((void*)a.S, 0, (int)(a.m * a.G * 4), 0x00020000);
  const __amdgpu_buffer_rsrc_t zrs = __builtin_amdgcn_make_buffer_rsrc((void*)a.Z, 0, (int)(a.m * a.G * 4), 0x00020000);
  uint32_t sv[NP / 4], zv[NP / 4];
#pragma unroll
  for (int u = 0; u < NP / 4; ++u) {
    const int e = tid + 256 * u;
    const int64_t r = min<int64_t>(r0 + e / NP, a.m - 1);
    const uint32_t off = (uint32_t)(r * a.G + group_of(e % NP)) * 4u;
    sv[u] = __builtin_amdgcn_raw_buffer_load_b32(srs, off, 0, 0);
    zv[u] = __builtin_amdgcn_raw_buffer_load_b32(zrs, off, 0, 0);
  }
  // 2. X: the range's columns of tokens < min(T, TT), one 8-column word per
  // load, zero past n
  const int tst = (int)min<int64_t>(a.T, TT);
  const int nw = (int)((min<int64_t>(a.n, kb + KR) - kb) >> 3);  // words of the range inside the row
  const __amdgpu_buffer_rsrc_t xrs =
      __builtin_amdgcn_make_buffer_rsrc((void*)a.X, 0, (int)(a.T * a.ldx * 2), 0x00020000);
  u32x4 xv[NXW];
#pragma unroll
  for (int u = 0; u < NXW; ++u) {
    const int e = tid + 256 * u;
    const int t = e / (KR / 8), w = e % (KR / 8);
    const bool ok = t < tst && w < nw;
    xv[u] = __builtin_amdgcn_raw_buffer_load_b128(xrs, ok ? (uint32_t)(t * a.ldx + kb + 8 * w) * 2u : 0x80000000u, 0, 0);
  }
  __builtin_amdgcn_sched_barrier(0);  // the codes go out after X and the parameters
  // 3. this wave's codes: piece P, words 4 g4 .. 4 g4 + 3 of row rw + l16
  const int64_t rows_here = max<int64_t>(0, min<int64_t>(16, a.m - rw));
  const __amdgpu_buffer_rsrc_t qrs = __builtin_amdgcn_make_buffer_rsrc(
      (void*)(a.Q + min<int64_t>(rw, a.m - 1) * a.W), 0, (int)(rows_here * a.W * 4), 0x00020000);
  // a piece is 128 columns: 16 words at 4 bits, 12 at 3; lane quarter g4
  // takes its 32 columns
  const uint32_t qoff = ((uint32_t)l16 * (uint32_t)a.W + (uint32_t)(kb * BITS / 32) + (uint32_t)BITS * g4) * 4u;
  u32x4 qv[BITS == 4 ? NP : 1];
  u32x3 q3[BITS == 3 ? NP : 1];
#pragma unroll
  for (int P = 0; P < NP; ++P) {
    if constexpr (BITS == 4) qv[P] = __builtin_amdgcn_raw_buffer_load_b128(qrs, qoff + 64u * P, 0, 0);
    else q3[P] = __builtin_amdgcn_raw_buffer_load_b96(qrs, qoff + 48u * P, 0, 0);
  }
  __builtin_amdgcn_sched_barrier(0);

  // 4. stage parameters and X (X's eight columns in pair order)
#pragma unroll
  for (int u = 0; u < NP / 4; ++u) {
    const int e = tid + 256 * u;
    ps[e / NP][e % NP] = __builtin_bit_cast(float, sv[u]);
    pz[e / NP][e % NP] = (int)zv[u];
  }
#pragma unroll
  for (int u = 0; u < NXW; ++u) {
    const int e = tid + 256 * u;
    const int t = e / (KR / 8), w = e % (KR / 8);
    if (t < tst) {
      const u32x4 x = xv[u];
      const u32x4 pr = {__builtin_amdgcn_perm(x.z, x.x, 0x05040100u), __builtin_amdgcn_perm(x.z, x.x, 0x07060302u),
                        __builtin_amdgcn_perm(x.w, x.y, 0x05040100u), __builtin_amdgcn_perm(x.w, x.y, 0x07060302u)};
      *(u32x4*)(xs + t * XP + 16 * w) = pr;
    }
  }
  __syncthreads();

  // 5. products
  const char* xrow = xs + min(l16, TT - 1) * XP + 64 * g4;
  const int prA = 16 * wave + l16;     // LDS row of this lane's codes
  const int prO = 16 * wave + 4 * g4;  // LDS rows of this lane's four outputs
  f32x4 tot = {0.f, 0.f, 0.f, 0.f}, acc = {0.f, 0.f, 0.f, 0.f}, acc1 = {0.f, 0.f, 0.f, 0.f};
  const u32x4 ones = {0x3F803F80u, 0x3F803F80u, 0x3F803F80u, 0x3F803F80u};  // bf16 1.0
#pragma unroll
  for (int P = 0; P < NP; ++P) {
    uint32_t zb = 0;  // fp16 (1024 + z, 1024 + z) of this lane's row
    if (DT == 0) {
      const uint32_t z = (uint32_t)pz[prA][P];
      zb = MAGIC | z | (z << 16);
    }
    u32x4 words;
    if constexpr (BITS == 4) {
      words = qv[P];
    } else {
      const u32x3 c = q3[P];
      const uint32_t c0 = c.x, c1 = c.y, c2 = c.z;
      words = spread3(c0, c1, c2);
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const uint32_t w = words[i];
      const uint32_t h0 = hsub<DT>((w & 0x000F000Fu) | MAGIC, zb);
      const uint32_t h1 = hsub<DT>(((w >> 4) & 0x000F000Fu) | MAGIC, zb);
      const uint32_t h2 = hsub<DT>(((w >> 8) & 0x000F000Fu) | MAGIC, zb);
      const uint32_t h3 = hsub<DT>(((w >> 12) & 0x000F000Fu) | MAGIC, zb);
      const u32x4 ai = {h0, h1, h2, h3};
      const u32x4 bi = *(const u32x4*)(xrow + 256 * P + 16 * i);
      if (DT == 0) {
        acc = __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(half8_t, ai), __builtin_bit_cast(half8_t, bi),
                                                     acc, 0, 0, 0);
      } else {
        acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf168_t, ai), __builtin_bit_cast(bf168_t, bi),
                                                      acc, 0, 0, 0);
        acc1 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf168_t, ones),
                                                       __builtin_bit_cast(bf168_t, bi), acc1, 0, 0, 0);
      }
    }
    if (G128 || P == NP - 1 || group_of(P + 1) != group_of(P)) {
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        const float sc = ps[prO + v][P];
        if (DT == 0) tot[v] = fmaf(sc, acc[v], tot[v]);
        else tot[v] = fmaf(sc, fmaf(-(128.f + (float)pz[prO + v][P]), acc1[v], acc[v]), tot[v]);
      }
      acc = f32x4{0.f, 0.f, 0.f, 0.f};
      acc1 = f32x4{0.f, 0.f, 0.f, 0.f};
    }
  }

  const int64_t t = l16;
  if (t < a.T) {
#pragma unroll
    for (int v = 0; v < 4; ++v) {
      const int64_t r = rw + 4 * g4 + v;
      if (r >= a.m) continue;
      if (a.P) a.P[(ks * a.T + t) * a.m + r] = tot[v];
      else Elem<DT>::store(a.Y, t * a.ldy + r, tot[v]);
    }
  }
}

// Many tokens, fp16 activations (prefill and calibration forward passes): a
// GEMM-shaped workgroup of 128 tokens x 128 rows of W, four waves of 64 x 64
// (2 x 2 blocks of v_mfma_f32_32x32x16_f16), K in steps of 64 columns.  The
// A operand is X, staged once per step in LDS (double-buffered, one barrier
// per step) in the pair order of the unpacked codes; the B operand is the
// codes themselves, one 8-code word per lane and MFMA step, unpacked in
// registers to exact fp16 (q - z) with the magic-number subtraction, so every
// product is exact in fp32.  Lane half g of a wave takes words 4g .. 4g+3 of
// a row's step (one 16-byte load); MFMA step s sums over words s and 4 + s.
// Per group, Y += s acc for each output row.  Each code is unpacked once per
// 128-token tile (the 64-token staged kernel above: once per 64 tokens, and
// with 16 x 16 MFMA blocks re-reading X from LDS four times as often).
constexpr int GM = 128, GN = 128, GK = 64;
constexpr int GXP = GK + 8;  // LDS pitch of a staged X row (halves): 144 bytes

template <int BITS>
__global__ __launch_bounds__(256, 2) void dqmm4_gemm_kernel(DqArgs a) {
  __shared__ __attribute__((aligned(16))) uint16_t xs[2][GM * GXP];
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave >> 1, wn = wave & 1;
  const int l32 = lane & 31, g = lane >> 5;
  const int64_t t0 = (int64_t)blockIdx.x * GM;  // first token of the tile
  const int64_t r0 = (int64_t)blockIdx.y * GN;  // first row of W
  constexpr uint32_t MAGIC = 0x64006400u;

  // this lane's two code rows (one per 32-row block of the wave)
  const int64_t rw = r0 + 64 * wn;
  const int64_t rows_here = max<int64_t>(0, min<int64_t>(64, a.m - rw));
  const __amdgpu_buffer_rsrc_t qrs = __builtin_amdgcn_make_buffer_rsrc(
      (void*)(a.Q + min<int64_t>(rw, a.m - 1) * a.W), 0, (int)(rows_here * a.W * 4), 0x00020000);
  uint32_t qoff[2];
  int64_t zrow[2];
#pragma unroll
  for (int nb = 0; nb < 2; ++nb) {
    qoff[nb] = ((uint32_t)(32 * nb + l32) * (uint32_t)a.W + (uint32_t)BITS * g) * 4u;
    zrow[nb] = min<int64_t>(rw + 32 * nb + l32, a.m - 1);
  }
  // X staging: thread -> (token tid / 2, 32-column half tid % 2), four words
  const int xt = tid >> 1, xh = tid & 1;
  const bool xok = t0 + xt < a.T;
  const uint16_t* xrow = (const uint16_t*)a.X + (t0 + (xok ? xt : 0)) * a.ldx;
  auto load_x = [&](int64_t k0, u32x4 (&r)[4]) {
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      const int64_t c = k0 + 32 * xh + 8 * w;
      r[w] = (xok && c < a.n) ? *(const u32x4*)(xrow + c) : u32x4{0u, 0u, 0u, 0u};
    }
  };
  auto store_x = [&](int buf, const u32x4 (&r)[4]) {
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      const u32x4 d = r[w];
      const u32x4 e = {__builtin_amdgcn_perm(d.z, d.x, 0x05040100u), __builtin_amdgcn_perm(d.z, d.x, 0x07060302u),
                       __builtin_amdgcn_perm(d.w, d.y, 0x05040100u), __builtin_amdgcn_perm(d.w, d.y, 0x07060302u)};
      *(u32x4*)&xs[buf][xt * GXP + 32 * xh + 8 * w] = e;
    }
  };
  // a step's 64 columns are 8 words at 4 bits (lane half g: 4 g .. 4 g + 3) and
  // 6 at 3 bits (3 g .. 3 g + 2, spread to the 4-bit layout)
  auto load_q = [&](int64_t k0, u32x4 (&q)[2]) {
#pragma unroll
    for (int nb = 0; nb < 2; ++nb) {
      const uint32_t off = qoff[nb] + (uint32_t)(k0 * BITS / 32) * 4u;
      if constexpr (BITS == 4) {
        q[nb] = __builtin_amdgcn_raw_buffer_load_b128(qrs, off, 0, 0);
      } else {
        const u32x3 c = __builtin_amdgcn_raw_buffer_load_b96(qrs, off, 0, 0);
        q[nb] = spread3(c.x, c.y, c.z);
      }
    }
  };

  f32x16 acc[2][2], tot[2][2];
#pragma unroll
  for (int mb = 0; mb < 2; ++mb)
#pragma unroll
    for (int nb = 0; nb < 2; ++nb) {
      acc[mb][nb] = zero16();
      tot[mb][nb] = zero16();
    }
  const int64_t nsteps = cdiv(a.n, GK);
  const int64_t gsteps = a.group > 0 ? a.group / GK : nsteps;  // steps per group (groups are multiples of 128)
  uint32_t zb[2];
  float sc[2];
  auto params = [&](int64_t gi) {
#pragma unroll
    for (int nb = 0; nb < 2; ++nb) {
      const uint32_t z = (uint32_t)a.Z[zrow[nb] * a.G + gi];
      zb[nb] = MAGIC | z | (z << 16);
      sc[nb] = a.S[zrow[nb] * a.G + gi];
    }
  };

  u32x4 xr[4], qc[2], qn[2];
  load_x(0, xr);
  load_q(0, qc);
  params(0);
  store_x(0, xr);
  __syncthreads();
  for (int64_t ks = 0; ks < nsteps; ++ks) {
    const int buf = (int)(ks & 1);
    const bool more = ks + 1 < nsteps;
    if (more) {
      load_x((ks + 1) * GK, xr);
      load_q((ks + 1) * GK, qn);
    }
    const uint16_t* xa = xs[buf] + (64 * wm + l32) * GXP + 32 * g;
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      u32x4 bq[2];
#pragma unroll
      for (int nb = 0; nb < 2; ++nb) {
        const uint32_t w = qc[nb][s];
        bq[nb] = u32x4{hsub<0>((w & 0x000F000Fu) | MAGIC, zb[nb]), hsub<0>(((w >> 4) & 0x000F000Fu) | MAGIC, zb[nb]),
                       hsub<0>(((w >> 8) & 0x000F000Fu) | MAGIC, zb[nb]),
                       hsub<0>(((w >> 12) & 0x000F000Fu) | MAGIC, zb[nb])};
      }
#pragma unroll
      for (int mb = 0; mb < 2; ++mb) {
        const u32x4 ax = *(const u32x4*)(xa + mb * 32 * GXP + 8 * s);
#pragma unroll
        for (int nb = 0; nb < 2; ++nb)
          acc[mb][nb] = __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(half8_t, ax),
                                                              __builtin_bit_cast(half8_t, bq[nb]), acc[mb][nb], 0, 0, 0);
      }
    }
    // a group ends after this step: fold its sums in with the scale of each output row
    if (!more || (ks + 1) % gsteps == 0) {
#pragma unroll
      for (int mb = 0; mb < 2; ++mb)
#pragma unroll
        for (int nb = 0; nb < 2; ++nb) {
#pragma unroll
          for (int r = 0; r < 16; ++r) tot[mb][nb][r] = fmaf(sc[nb], acc[mb][nb][r], tot[mb][nb][r]);
          acc[mb][nb] = zero16();
        }
      if (more) params(a.group > 0 ? (ks + 1) / gsteps : 0);
    }
    if (more) {
      store_x(buf ^ 1, xr);
      qc[0] = qn[0];
      qc[1] = qn[1];
    }
    __syncthreads();
  }

  // Y[t][r]: MFMA output element r of lane l is token 8(r/4) + 4(l/32) + r%4 of
  // the block and row l%32; 32 lanes store 32 consecutive rows of one token
#pragma unroll
  for (int mb = 0; mb < 2; ++mb)
#pragma unroll
    for (int nb = 0; nb < 2; ++nb) {
      const int64_t row = rw + 32 * nb + l32;
      if (row >= a.m) continue;
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int64_t t = t0 + 64 * wm + 32 * mb + mfma32_row(r, lane);
        if (t < a.T) Elem<0>::store(a.Y, t * a.ldy + row, tot[mb][nb][r]);
      }
    }
}

// Y[t][r] = sum over the K sets of the partials, in set order, in X's dtype.
// A thread takes four consecutive rows of one token (16-byte loads when m is
// a multiple of 4), all KS loads in flight at once.
template <int DT>
__global__ __launch_bounds__(256) void dqmm_reduce_kernel(const float* P, int KS, int64_t T, int64_t m, void* Y,
                                                          int64_t ldy) {
  const int64_t r = ((int64_t)blockIdx.x * 256 + threadIdx.x) * 4;
  if (r >= m) return;
  for (int64_t t = blockIdx.y; t < T; t += gridDim.y) {
    f32x4 s = {0.f, 0.f, 0.f, 0.f};
    if ((m & 3) == 0) {
      constexpr int U = 8;  // loads in flight per pass
      for (int k0 = 0; k0 < KS; k0 += U) {
        f32x4 v[U];
#pragma unroll
        for (int u = 0; u < U; ++u)
          if (k0 + u < KS) v[u] = *(const f32x4*)(P + ((int64_t)(k0 + u) * T + t) * m + r);
#pragma unroll
        for (int u = 0; u < U; ++u)
          if (k0 + u < KS) s += v[u];
      }
    } else {
      for (int k = 0; k < KS; ++k)
#pragma unroll
        for (int e = 0; e < 4; ++e)
          if (r + e < m) s[e] += P[((int64_t)k * T + t) * m + r + e];
    }
#pragma unroll
    for (int e = 0; e < 4; ++e)
      if (r + e < m) Elem<DT>::store(Y, t * ldy + r + e, s[e]);
  }
}

// K sets and the columns of each: the staged kernel for more than 16 tokens
// (slices of 512), the task kernel for up to 16 (ranges of 512 or 1024); the
// GEMM-shaped kernel never cuts K (its partial-sum workspace is unused)
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
  // ranges of 1024 columns while that still gives about four workgroups per
  // CU, else 512
  const int64_t kr = cdiv(m, 64) * cdiv(n, 1024) >= 1024 ? 1024 : 512;
  return {(int)cdiv(n, kr), kr};
}

template <int DT, bool G128, int BITS>
void launch_task_g(const DqArgs& a, int64_t kr, int64_t T, dim3 grid, hipStream_t st) {
  if (kr == 1024) {
    if (T <= 4) hipLaunchKernelGGL((dqmm4_task_kernel<DT, G128, 1024, 4, BITS>), grid, dim3(256), 0, st, a);
    else hipLaunchKernelGGL((dqmm4_task_kernel<DT, G128, 1024, 16, BITS>), grid, dim3(256), 0, st, a);
  } else {
    if (T <= 4) hipLaunchKernelGGL((dqmm4_task_kernel<DT, G128, 512, 4, BITS>), grid, dim3(256), 0, st, a);
    else hipLaunchKernelGGL((dqmm4_task_kernel<DT, G128, 512, 16, BITS>), grid, dim3(256), 0, st, a);
  }
}
template <int DT>
void launch_task(const DqArgs& a, bool g128, int bits, int64_t kr, int64_t T, dim3 grid, hipStream_t st) {
  if (bits == 3) {
    if (g128) launch_task_g<DT, true, 3>(a, kr, T, grid, st);
    else launch_task_g<DT, false, 3>(a, kr, T, grid, st);
  } else {
    if (g128) launch_task_g<DT, true, 4>(a, kr, T, grid, st);
    else launch_task_g<DT, false, 4>(a, kr, T, grid, st);
  }
}

}  // namespace

size_t dequant_matmul_workspace_bytes(int64_t tokens, int64_t m, int64_t n) {
  if (tokens < 1 || m < 1 || n < 1) return 0;
  const int ks = dq_split(tokens, m, n).ks;
  return ks > 1 ? (size_t)ks * (size_t)tokens * (size_t)m * 4 : 0;
}

bool dequant_matmul_supported(int bits, int64_t n, int64_t group, int64_t tokens) {
  return (bits == 4 || bits == 3) && n % 32 == 0 && (group <= 0 || group % 128 == 0);
}

hipError_t dequant_matmul(const void* X, int dt, int64_t T, int64_t ldx, const uint32_t* Q, int bits, const float* S,
                          const int32_t* Z, int64_t m, int64_t n, int64_t group, void* Y, int64_t ldy, void* ws,
                          hipStream_t st) {
  if (T == 0) return hipSuccess;
  DqArgs a{};
  a.X = X; a.ldx = ldx; a.T = T;
  a.Q = Q; a.W = cdiv(n * bits, 32);
  a.S = S; a.Z = Z; a.group = group; a.G = group > 0 ? cdiv(n, group) : 1;
  a.m = m; a.n = n; a.Y = Y; a.ldy = ldy;
  const DqSplit sp = dq_split(T, m, n);
  a.KS = sp.ks;
  a.P = a.KS > 1 ? (float*)ws : nullptr;
  if (T <= 16) {
    const dim3 grid((unsigned)(cdiv(m, 64) * a.KS));
    if (dt == 0) launch_task<0>(a, group == 128, bits, sp.kr, T, grid, st);
    else launch_task<1>(a, group == 128, bits, sp.kr, T, grid, st);
  } else if (dt == 0 && cdiv(T, GM) * cdiv(m, GN) >= 128) {
    // enough 128 x 128 tiles to fill the GPU without cutting K
    a.KS = 1;
    a.P = nullptr;
    const dim3 grid((unsigned)cdiv(T, GM), (unsigned)cdiv(m, GN));
    if (bits == 4) hipLaunchKernelGGL((dqmm4_gemm_kernel<4>), grid, dim3(256), 0, st, a);
    else hipLaunchKernelGGL((dqmm4_gemm_kernel<3>), grid, dim3(256), 0, st, a);
  } else {
    const dim3 grid((unsigned)cdiv(m, DQ_ROWS), (unsigned)a.KS, (unsigned)cdiv(T, DQ_TOK));
    if (dt == 0 && bits == 4) hipLaunchKernelGGL((dqmm4_kernel<0, 4>), grid, dim3(256), 0, st, a);
    else if (dt == 0) hipLaunchKernelGGL((dqmm4_kernel<0, 3>), grid, dim3(256), 0, st, a);
    else if (bits == 4) hipLaunchKernelGGL((dqmm4_kernel<1, 4>), grid, dim3(256), 0, st, a);
    else hipLaunchKernelGGL((dqmm4_kernel<1, 3>), grid, dim3(256), 0, st, a);
  }
  if (a.KS > 1) {
    const dim3 rg((unsigned)cdiv(m, 1024), (unsigned)std::min<int64_t>(T, 65535));
    if (dt == 0) hipLaunchKernelGGL(dqmm_reduce_kernel<0>, rg, dim3(256), 0, st, (const float*)a.P, a.KS, T, m, Y, ldy);
    else hipLaunchKernelGGL(dqmm_reduce_kernel<1>, rg, dim3(256), 0, st, (const float*)a.P, a.KS, T, m, Y, ldy);
  }
  return hipGetLastError();
}

namespace {
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};
}  // namespace

// Device address of `scratch` on the device `stream` belongs to (the current
// device for the null stream), looked up once per device with that device
// current and kept.
hipError_t static_scratch(hipStream_t stream, void** out) {
  int cur = 0;
  hipError_t e = hipGetDevice(&cur);
  if (e != hipSuccess) return e;
  int dev = cur;
  if (stream != nullptr) {
    hipDevice_t d = 0;
    if ((e = hipStreamGetDevice(stream, &d)) != hipSuccess) return e;
    dev = (int)d;
  }
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (g_scratch_ptr[dev] == nullptr) {
    if (dev != cur && (e = hipSetDevice(dev)) != hipSuccess) return e;
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (dev != cur) {
      const hipError_t e2 = hipSetDevice(cur);
      if (e == hipSuccess) e = e2;
    }
    if (e != hipSuccess) return e;
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return hipSuccess;
}

}  // namespace gptq

