// C++ interfaces between the library's translation units (internal header,
// not part of the C ABI).
#pragma once

#include "tdp_common.h"

namespace tdp {

// Epilogues of gemm(): acc = (A B)[m][n], B given as B^T [N][K].
enum GemmEpi : int {
  kEpiBf16 = 0,       // c[m][n] = bf16(acc)
  kEpiF32 = 1,        // c[m][n] = acc
  kEpiGeluBf16 = 2,   // c[m][n] = bf16(gelu_tanh(acc))
  kEpiSiluBf16 = 3,   // c[m][n] = bf16(acc * sigmoid(acc))
  kEpiResid = 4,      // c[m][n] += acc            (c float)
  kEpiResidGate = 5,  // c[m][n] += gate(m, n) acc (c float)
};

// C[M][N] (+)= A[M][K] B[K][N].  bf16 operands, fp32 accumulation.
// Requirements: N % 128 == 0, K % 64 == 0, M >= 1, rows and pointers 16-byte
// aligned.  A is row-major (lda elements per row) unless a_head_dim > 0: then
// A is head-major, row R of segment s = R / a_seg_rows holding the features
// of head h at ((s * a_heads + h) * a_seg_rows + R % a_seg_rows) * a_head_dim
// (K = a_heads * a_head_dim, a_head_dim 64 or 128).
// gate(m, n) = g0[(m / rows_per_batch) * g0_stride + n] + g1[n] (either term
// may be absent).
struct GemmDesc {
  const bf16 *a = nullptr;
  int64_t lda = 0;
  int64_t a_seg_rows = 0;
  int32_t a_heads = 0, a_head_dim = 0;
  const bf16 *bt = nullptr;
  int64_t ldb = 0;
  int64_t M = 0;
  int32_t N = 0, K = 0;
  void *c = nullptr;
  int64_t ldc = 0;
  const float *g0 = nullptr;
  int64_t g0_stride = 0;
  const float *g1 = nullptr;
  int64_t rows_per_batch = 1;
};

// Launches the GEMM on `stream`; TDP_ERR_UNSUPPORTED for shapes outside the
// requirements, TDP_ERR_HIP for a failed launch.
tdp_status gemm(int epi, const GemmDesc &d, hipStream_t stream);

}  // namespace tdp
