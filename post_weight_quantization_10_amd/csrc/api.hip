// C ABI of the library: argument validation on the host, then the launch
// sequences of the three GPTQ stages (declared in include/gptq.h).
#include <cmath>

#include "../../include/gptq.h"
#include "common.hpp"
#include "internal.hpp"

namespace gptq {
size_t syrk_workspace_bytes(int64_t n, int64_t tokens, int dtype);
hipError_t syrk_accumulate(float* H, int64_t n, const void* X, int dtype, int64_t tokens, int64_t ldx, void* ws,
                           hipStream_t stream);
size_t prepare_workspace_bytes(int64_t n);
hipError_t prepare_hinv(const float* H, int64_t n, float damp, float* U, int32_t* info, float* lambda_out, void* ws,
                        hipStream_t s);
size_t quantize_workspace_bytes(int64_t m, int64_t n, int64_t B);
hipError_t quantize_layer(void* W, int dt, int64_t m, int64_t n, int64_t ldw, const float* U, int bits, int64_t group,
                          int64_t B, uint32_t* qcodes, float* S, int32_t* Z, float* err_sq, int write_dequant,
                          void* ws, hipStream_t st);
size_t dequant_matmul_workspace_bytes(int64_t tokens, int64_t m, int64_t n);
bool dequant_matmul_supported(int bits, int64_t n, int64_t group, int64_t tokens);
hipError_t dequant_matmul(const void* X, int dt, int64_t T, int64_t ldx, const uint32_t* Q, int bits, const float* S,
                          const int32_t* Z, int64_t m, int64_t n, int64_t group, void* Y, int64_t ldy, void* ws,
                          hipStream_t st);
int rotation_block(int64_t n, int64_t block);
bool rotation_supported(int64_t n, int64_t block);
hipError_t rotate_hadamard(void* M, int dt, int64_t rows, int64_t n, int64_t ld, int64_t block, hipStream_t st);
hipError_t swiglu(const void* G, const void* U, void* A, int dt, int64_t rows, int64_t cols, int64_t ld,
                  hipStream_t st);
hipError_t residual_add(void* X, const void* Y, int dt, int64_t rows, int64_t cols, int64_t ld, hipStream_t st);
bool attention_supported(int64_t seq_len, int64_t head_dim);
hipError_t attention(const void* Q, const void* K, const void* V, void* O, int dt, int64_t T, int64_t S,
                     int64_t heads, int64_t dh, int64_t ld, hipStream_t st);
bool greedy_supported(int64_t n, int64_t group);
size_t greedy_workspace_bytes(int64_t m, int64_t n);
hipError_t quantize_greedy(const void* W, int dt, int64_t m, int64_t n, int64_t ldw, const float* U, int bits,
                           int64_t group, uint32_t* qcodes, float* S, int32_t* Z, int32_t* order, float* loss, void* ws,
                           hipStream_t st);
}  // namespace gptq

namespace {
constexpr int64_t kMaxDim = 65535;  // grid-dimension limit of the per-row launches
inline bool dtype_ok(int32_t d) { return d == GPTQ_F16 || d == GPTQ_BF16 || d == GPTQ_F32; }
}  // namespace

extern "C" {

const char* gptq_status_string(int32_t s) {
  switch (s) {
    case GPTQ_OK: return "GPTQ_OK";
    case GPTQ_ERR_INVALID_ARG: return "GPTQ_ERR_INVALID_ARG";
    case GPTQ_ERR_UNSUPPORTED: return "GPTQ_ERR_UNSUPPORTED";
    case GPTQ_ERR_WORKSPACE: return "GPTQ_ERR_WORKSPACE";
    case GPTQ_ERR_HIP: return "GPTQ_ERR_HIP";
    case GPTQ_ERR_SCRATCH_LIMIT: return "GPTQ_ERR_SCRATCH_LIMIT";
    default: return "GPTQ_UNKNOWN_STATUS";
  }
}

int32_t gptq_version(void) { return 100; }

size_t gptq_hessian_workspace_bytes(int64_t n, int64_t tokens) {
  // the fp32 path stages fewer tokens per step and may use more splits
  const size_t a = gptq::syrk_workspace_bytes(n, tokens, GPTQ_F16);
  const size_t b = gptq::syrk_workspace_bytes(n, tokens, GPTQ_F32);
  return a > b ? a : b;
}

gptq_status gptq_hessian_accumulate(float* H, int64_t n, const void* X, int32_t x_dtype, int64_t tokens, int64_t ldx,
                                    void* workspace, size_t ws_bytes, void* stream) {
  if (n < 1 || n > kMaxDim || tokens < 0 || ldx < n || !dtype_ok(x_dtype) || H == nullptr) return GPTQ_ERR_INVALID_ARG;
  if (tokens == 0) return GPTQ_OK;
  if (X == nullptr) return GPTQ_ERR_INVALID_ARG;
  const size_t need = gptq::syrk_workspace_bytes(n, tokens, x_dtype);
  if (workspace == nullptr || ws_bytes < need) return GPTQ_ERR_WORKSPACE;
  hipError_t e = gptq::syrk_accumulate(H, n, X, x_dtype, tokens, ldx, workspace, (hipStream_t)stream);
  return e == hipSuccess ? GPTQ_OK : GPTQ_ERR_HIP;
}

size_t gptq_prepare_workspace_bytes(int64_t n) { return gptq::prepare_workspace_bytes(n); }

gptq_status gptq_prepare_hinv(const float* H, int64_t n, float damp, float* U, int32_t* info, float* lambda_out,
                              void* workspace, size_t ws_bytes, void* stream) {
  if (n < 1 || n > kMaxDim || !(damp >= 0.f) || !std::isfinite(damp) || H == nullptr || U == nullptr ||
      info == nullptr || lambda_out == nullptr)
    return GPTQ_ERR_INVALID_ARG;
  if (workspace == nullptr || ws_bytes < gptq::prepare_workspace_bytes(n)) return GPTQ_ERR_WORKSPACE;
  hipError_t e = gptq::prepare_hinv(H, n, damp, U, info, lambda_out, workspace, (hipStream_t)stream);
  return e == hipSuccess ? GPTQ_OK : GPTQ_ERR_HIP;
}

size_t gptq_quantize_workspace_bytes(int64_t m, int64_t n, int64_t block_size) {
  return gptq::quantize_workspace_bytes(m, n, block_size);
}

gptq_status gptq_quantize_layer(void* W, int32_t w_dtype, int64_t m, int64_t n, int64_t ldw, const float* U,
                                int32_t bits, int64_t group_size, int64_t block_size, uint32_t* qcodes, float* scales,
                                int32_t* zeros, float* err_sq, int32_t write_dequant, void* workspace, size_t ws_bytes,
                                void* stream) {
  if (m < 1 || n < 1 || n > kMaxDim || ldw < n || !dtype_ok(w_dtype) || bits < 2 || bits > 8 || block_size < 1 ||
      block_size > 128)
    return GPTQ_ERR_INVALID_ARG;
  if (group_size > 0 && !(group_size % block_size == 0 || block_size % group_size == 0)) return GPTQ_ERR_INVALID_ARG;
  if (W == nullptr || U == nullptr || qcodes == nullptr || scales == nullptr || zeros == nullptr)
    return GPTQ_ERR_INVALID_ARG;
  if (workspace == nullptr || ws_bytes < gptq::quantize_workspace_bytes(m, n, block_size)) return GPTQ_ERR_WORKSPACE;
  hipError_t e = gptq::quantize_layer(W, w_dtype, m, n, ldw, U, bits, group_size, block_size, qcodes, scales, zeros,
                                      err_sq, write_dequant, workspace, (hipStream_t)stream);
  return e == hipSuccess ? GPTQ_OK : GPTQ_ERR_HIP;
}

size_t gptq_quantize_greedy_workspace_bytes(int64_t m, int64_t n) { return gptq::greedy_workspace_bytes(m, n); }

gptq_status gptq_quantize_greedy(const void* W, int32_t w_dtype, int64_t m, int64_t n, int64_t ldw, const float* U,
                                 int32_t bits, int64_t group_size, uint32_t* qcodes, float* scales, int32_t* zeros,
                                 int32_t* order, float* loss, void* workspace, size_t ws_bytes, void* stream) {
  if (m < 1 || n < 1 || ldw < n || !dtype_ok(w_dtype) || bits < 2 || bits > 8) return GPTQ_ERR_INVALID_ARG;
  if (W == nullptr || U == nullptr || qcodes == nullptr || scales == nullptr || zeros == nullptr)
    return GPTQ_ERR_INVALID_ARG;
  if (!gptq::greedy_supported(n, group_size)) return GPTQ_ERR_UNSUPPORTED;
  if (workspace == nullptr || ws_bytes < gptq::greedy_workspace_bytes(m, n)) return GPTQ_ERR_WORKSPACE;
  hipError_t e = gptq::quantize_greedy(W, w_dtype, m, n, ldw, U, bits, group_size, qcodes, scales, zeros, order, loss,
                                       workspace, (hipStream_t)stream);
  return e == hipSuccess ? GPTQ_OK : GPTQ_ERR_HIP;
}

size_t gptq_dequant_matmul_workspace_bytes(int64_t tokens, int64_t m, int64_t n) {
  return gptq::dequant_matmul_workspace_bytes(tokens, m, n);
}

// Argument checks shared by the two dequant-matmul entry points; GPTQ_OK
// means "run it" (tokens > 0).
static gptq_status dequant_matmul_check(const void* X, int32_t x_dtype, int64_t tokens, int64_t ldx,
                                        const uint32_t* qcodes, const float* scales, const int32_t* zeros, int64_t m,
                                        int64_t n, int32_t bits, int64_t group_size, void* Y, int64_t ldy) {
  if (m < 1 || n < 1 || tokens < 0 || tokens > ((int64_t)1 << 31) || ldx < n || ldy < m ||
      !(x_dtype == GPTQ_F16 || x_dtype == GPTQ_BF16) || bits < 2 || bits > 8)
    return GPTQ_ERR_INVALID_ARG;
  if (tokens == 0) return GPTQ_OK;
  if (X == nullptr || qcodes == nullptr || scales == nullptr || zeros == nullptr || Y == nullptr)
    return GPTQ_ERR_INVALID_ARG;
  const auto al16 = [](const void* p) { return ((uintptr_t)p & 15) == 0; };
  const int64_t G = group_size > 0 ? (n + group_size - 1) / group_size : 1;
  const int64_t lim = (int64_t)1 << 31;  // byte ranges addressed with 32-bit buffer offsets
  if (!gptq::dequant_matmul_supported(bits, n, group_size, tokens) || ldx % 8 != 0 || !al16(X) || !al16(qcodes) ||
      (int64_t)64 * n * 4 >= lim || m * G * 4 >= lim || (int64_t)16 * ldx * 2 >= lim)
    return GPTQ_ERR_UNSUPPORTED;
  return GPTQ_OK;
}

gptq_status gptq_dequant_matmul(const void* X, int32_t x_dtype, int64_t tokens, int64_t ldx, const uint32_t* qcodes,
                                const float* scales, const int32_t* zeros, int64_t m, int64_t n, int32_t bits,
                                int64_t group_size, void* Y, int64_t ldy, void* workspace, size_t ws_bytes,
                                void* stream) {
  const gptq_status c = dequant_matmul_check(X, x_dtype, tokens, ldx, qcodes, scales, zeros, m, n, bits, group_size,
                                             Y, ldy);
  if (c != GPTQ_OK || tokens == 0) return c;
  const size_t need = gptq::dequant_matmul_workspace_bytes(tokens, m, n);
  if (need > 0 && (workspace == nullptr || ws_bytes < need)) return GPTQ_ERR_WORKSPACE;
  hipError_t e = gptq::dequant_matmul(X, x_dtype, tokens, ldx, qcodes, bits, scales, zeros, m, n, group_size, Y, ldy,
                                      workspace, (hipStream_t)stream);
  return e == hipSuccess ? GPTQ_OK : GPTQ_ERR_HIP;
}

size_t gptq_static_scratch_bytes(void) { return gptq::kStaticScratchBytes; }

gptq_status gptq_dequant_matmul_static(const void* X, int32_t x_dtype, int64_t tokens, int64_t ldx,
                                       const uint32_t* qcodes, const float* scales, const int32_t* zeros, int64_t m,
                                       int64_t n, int32_t bits, int64_t group_size, void* Y, int64_t ldy,
                                       void* stream) {
  const gptq_status c = dequant_matmul_check(X, x_dtype, tokens, ldx, qcodes, scales, zeros, m, n, bits, group_size,
                                             Y, ldy);
  if (c != GPTQ_OK || tokens == 0) return c;
  const size_t need = gptq::dequant_matmul_workspace_bytes(tokens, m, n);
  if (need > gptq::kStaticScratchBytes) return GPTQ_ERR_SCRATCH_LIMIT;
  void* ws = nullptr;
  hipError_t e = gptq::static_scratch((hipStream_t)stream, &ws);
  if (e != hipSuccess) return GPTQ_ERR_HIP;
  e = gptq::dequant_matmul(X, x_dtype, tokens, ldx, qcodes, bits, scales, zeros, m, n, group_size, Y, ldy, ws,
                           (hipStream_t)stream);
  return e == hipSuccess ? GPTQ_OK : GPTQ_ERR_HIP;
}

gptq_status gptq_rotate_hadamard(void* M, int32_t dtype, int64_t rows, int64_t n, int64_t ld, int64_t block,
                                 void* stream) {
  if (rows < 0 || n < 1 || ld < n || !dtype_ok(dtype) || block < 0) return GPTQ_ERR_INVALID_ARG;
  if (block > 0 && ((block & (block - 1)) != 0 || n % block != 0)) return GPTQ_ERR_INVALID_ARG;
  if (rows == 0) return GPTQ_OK;
  if (M == nullptr) return GPTQ_ERR_INVALID_ARG;
  const int64_t per16 = dtype == GPTQ_F32 ? 4 : 8;  // elements per 16 bytes
  if (!gptq::rotation_supported(n, block) || ld % per16 != 0 || ((uintptr_t)M & 15) != 0 ||
      rows * (n / gptq::rotation_block(n, block)) / (4096 / gptq::rotation_block(n, block)) >= ((int64_t)1 << 31) - 1)
    return GPTQ_ERR_UNSUPPORTED;
  hipError_t e = gptq::rotate_hadamard(M, dtype, rows, n, ld, block, (hipStream_t)stream);
  return e == hipSuccess ? GPTQ_OK : GPTQ_ERR_HIP;
}

gptq_status gptq_swiglu(const void* G, const void* Uo, void* A, int32_t dtype, int64_t tokens, int64_t f,
                        int64_t ld, void* stream) {
  if (tokens < 0 || f < 1 || ld < f || !(dtype == GPTQ_F16 || dtype == GPTQ_BF16)) return GPTQ_ERR_INVALID_ARG;
  if (tokens == 0) return GPTQ_OK;
  if (G == nullptr || Uo == nullptr || A == nullptr || tokens * (ld / f + 1) * f >= ((int64_t)1 << 40))
    return GPTQ_ERR_INVALID_ARG;
  hipError_t e = gptq::swiglu(G, Uo, A, dtype, tokens, f, ld, (hipStream_t)stream);
  return e == hipSuccess ? GPTQ_OK : GPTQ_ERR_HIP;
}

gptq_status gptq_residual_add(void* X, const void* Y, int32_t dtype, int64_t tokens, int64_t d, int64_t ld,
                              void* stream) {
  if (tokens < 0 || d < 1 || ld < d || !(dtype == GPTQ_F16 || dtype == GPTQ_BF16)) return GPTQ_ERR_INVALID_ARG;
  if (tokens == 0) return GPTQ_OK;
  if (X == nullptr || Y == nullptr || tokens * (ld / d + 1) * d >= ((int64_t)1 << 40)) return GPTQ_ERR_INVALID_ARG;
  hipError_t e = gptq::residual_add(X, Y, dtype, tokens, d, ld, (hipStream_t)stream);
  return e == hipSuccess ? GPTQ_OK : GPTQ_ERR_HIP;
}

gptq_status gptq_attention(const void* Q, const void* K, const void* V, void* O, int32_t dtype, int64_t tokens,
                           int64_t seq_len, int64_t heads, int64_t head_dim, int64_t ld, void* stream) {
  if (tokens < 0 || seq_len < 1 || heads < 1 || head_dim < 1 || ld < heads * head_dim ||
      !(dtype == GPTQ_F16 || dtype == GPTQ_BF16) || (tokens > 0 && tokens % seq_len != 0) ||
      heads > 65535 || tokens >= ((int64_t)1 << 37))
    return GPTQ_ERR_INVALID_ARG;
  if (tokens == 0) return GPTQ_OK;
  if (Q == nullptr || K == nullptr || V == nullptr || O == nullptr) return GPTQ_ERR_INVALID_ARG;
  const auto al16 = [](const void* p) { return ((uintptr_t)p & 15) == 0; };
  if (!gptq::attention_supported(seq_len, head_dim) || ld % 8 != 0 || !al16(Q) || !al16(K) || !al16(V) || !al16(O))
    return GPTQ_ERR_UNSUPPORTED;
  hipError_t e = gptq::attention(Q, K, V, O, dtype, tokens, seq_len, heads, head_dim, ld, (hipStream_t)stream);
  return e == hipSuccess ? GPTQ_OK : GPTQ_ERR_HIP;
}

}  // extern "C"
