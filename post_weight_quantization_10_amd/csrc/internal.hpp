// Internal launchers shared between the HIP translation units of the library.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace gptq {

// Size of the fixed partial-sum buffer behind gptq_dequant_matmul_static.
constexpr size_t kStaticScratchBytes = (size_t)32 << 20;

// Device address of that buffer on the device of `stream`.
hipError_t static_scratch(hipStream_t stream, void** out);

// Flags for gemm_f32.
enum : int {
  GEMM_LOWER_TILES = 1,  // C square; only 128x128 tiles on or below the diagonal are computed
  GEMM_A_LOWER = 2,      // op(A)[i][k] == 0 for k > i (skip those K chunks)
  GEMM_B_LOWER = 4,      // op(B)[k][j] == 0 for k < j (skip those K chunks)
  GEMM_SMALL_TILES = 8,  // NN products on 64x64 tiles, longest K range first, never split (for grids of few
                         // 128x128 tiles with triangular operands)
};

struct GemmDesc {
  const float* A;
  const float* B;
  float* C;
  int64_t lda, ldb, ldc;
  int64_t strideA, strideB, strideC;  // per batch entry (blockIdx.z)
  int M, N, K, batch;
  float alpha, beta;
  int flags;
  const int32_t* info;  // if non-null and *info != 0 the kernel does nothing
  // Optional scratch for a split-K launch (K cut into chunks whose partial
  // tiles are summed in chunk order by a second kernel: deterministic).  Used
  // only when the tile grid alone would leave the GPU under-filled.
  float* ws;
  int64_t ws_floats;
};

// C = alpha * op(A) * op(B) + beta * C in fp32 on the MFMA pipe.
// op(A) is M x K: A[i*lda + k] (transA = false) or A[k*lda + i] (true).
// op(B) is K x N: B[k*ldb + j] (transB = false) or B[j*ldb + k] (true).
// beta == 0 never reads C.  C may alias A only when N <= 128 (each tile row
// then reads all of its A rows before writing them).
hipError_t gemm_f32(const GemmDesc& d, bool transA, bool transB, hipStream_t s);

// Compute units of the current device (256 if the query fails), read once.
int device_cus();

// The factor split for the trailing updates as three bf16 products
// (gemm_x3.hip): Ut (n rows of 2n bf16, 16-byte aligned) = [U_hi | U_lo]^T
// above the diagonal blocks of gran columns (a multiple of 64); n a
// multiple of 4.
hipError_t split_ut_x3(const float* U, int64_t n, uint16_t* Ut, int64_t gran, hipStream_t s);

// A trailing update V[:, c0:c0+N] -= E U[r0:r0+K, c0:c0+N] as three bf16
// products: row r of E given as E_hi at Ecat + r lde and E_lo alo elements
// further, U as split by split_ut_x3 (rows [r0, r0 + K) ending at one of its
// granule boundaries, at or before c0); K and r0 multiples of 64.
hipError_t flush_x3(const uint16_t* Ecat, int64_t lde, int64_t alo, const uint16_t* Ut, int64_t n, int64_t r0,
                    int K, int64_t c0, int64_t N, float* V, int64_t m, hipStream_t s);

}  // namespace gptq
