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
  // A zeroed counter the persistent large form may use for a claimed tail of
  // tiles (each launch leaves it zero again); null: every tile assigned
  // statically.  Launches that share a counter must not overlap.
  uint32_t *tail_ctr = nullptr;
};

// Launches the GEMM on `stream`; TDP_ERR_UNSUPPORTED for shapes outside the
// requirements, TDP_ERR_HIP for a failed launch.
tdp_status gemm(int epi, const GemmDesc &d, hipStream_t stream);

// The attention core driven from row-major projections (the transformer
// block).  `desc` and the tile arguments are those of the tdp_attn_* calls;
// the workspace is sized by tdp_tile_attention_workspace.
// Block table of the padded row space, K-norm maxima cleared.
tdp_status attn_tables(const tdp_attn_desc *desc, int32_t n_tiles, const int64_t *trb,
                       int32_t max_rows, int64_t n_rows, void *ws, size_t ws_bytes,
                       hipStream_t stream);
// Tile rows of src ([B][n_rows][ld]; Q, K, V of head h at columns
// {q,k,v}_col + h * head_dim, negative = absent) into the core's layouts, with
// RoPE when row_pos is given; or (text) rows of text_src ([B][n_audio][text_ld])
// into the second key segment (K and V only, no rotation).
tdp_status attn_rows_to_heads(const tdp_attn_desc *desc, int32_t n_tiles, const int64_t *trb,
                              int32_t max_rows, int64_t n_rows, const bf16 *src, int64_t ld,
                              int32_t q_col, int32_t k_col, int32_t v_col, const float *row_pos,
                              bool text, const bf16 *text_src, int64_t text_ld, void *ws,
                              size_t ws_bytes, hipStream_t stream);
// The core over the tile's keys then the second segment's (tile_keys), or the
// second segment's only (cross-attention; no queries from that segment).
tdp_status attn_core_run(const tdp_attn_desc *desc, int32_t n_tiles, const int64_t *trb,
                         int32_t max_rows, int64_t n_rows, void *ws, size_t ws_bytes,
                         bool tile_keys, hipStream_t stream);
// The core's output O, head-major [B][heads][n_rows][head_dim] (nullptr for a bad desc).
const bf16 *attn_output(const tdp_attn_desc *desc, int32_t n_tiles, int64_t n_rows, void *ws);
// The attention workspace's tail-claim counter: zeroed by attn_tables, left
// zero by every launch that uses it (the core's, and GEMMs given it).
uint32_t *attn_tail_counter(const tdp_attn_desc *desc, int32_t n_tiles, int64_t n_rows, void *ws);

}  // namespace tdp
