/*
 * tdp.h - C ABI of libtdp.so: one Tiled Data Parallelism (TDP) upscale step on
 * one MI355X (gfx950), the GPU holding every tile.
 *
 * The method is the one on the "Tiled Data Parallelism (TDP)" design page:
 * split the patchified (frames, height, width) latent into overlapping tiles
 * ("What it is"), shift each tile's positions so its generated tokens start at
 * zero ("Position normalization"), keep the conditioning tokens that overlap a
 * tile plus every negative-time reference token ("Shared negative (reference)
 * positions"), run the denoiser on every tile, and sum the mask-weighted tile
 * outputs into the global latent.  On one GPU that sum replaces the page's
 * single all_reduce.
 *
 * Conventions for every call:
 *  - Every call returns a tdp_status; nothing throws, nothing aborts.
 *  - The library never allocates memory.  Host arrays, device buffers, the
 *    workspace and the stream are the caller's.
 *  - Pointers marked "host" are read or written before the call returns.
 *    Pointers marked "device" are HBM addresses (hipMalloc'd, e.g. the
 *    data_ptr() of a torch tensor on cuda:0) and must be 16-byte aligned.
 *  - Device work is enqueued on `hip_stream` (a hipStream_t; NULL = the
 *    default stream) and runs asynchronously.  Arguments are validated on the
 *    host before anything is launched: an invalid call launches nothing.  A
 *    launch failure returns TDP_ERR_HIP; faults show at the caller's sync.
 *  - Calls hold no global state and may be made from several threads; calls
 *    whose device buffers overlap must be ordered by the caller (one stream).
 *  - Layouts are row-major, innermost index last.  "bf16" is IEEE binary32
 *    truncated to its upper 16 bits in storage (round to nearest even when
 *    the library produces it).
 */
#ifndef TDP_H
#define TDP_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  TDP_OK = 0,
  TDP_ERR_NULL = -1,        /* a required pointer is NULL                          */
  TDP_ERR_ARG = -2,         /* a count, size or tiling is out of range             */
  TDP_ERR_SHAPE = -3,       /* sizes disagree with each other (e.g. plan vs desc)  */
  TDP_ERR_UNSUPPORTED = -4, /* a valid but unsupported shape or dtype              */
  TDP_ERR_BUFFER = -5,      /* a caller buffer or the workspace is too small       */
  TDP_ERR_HIP = -6,         /* a HIP launch or runtime call failed                 */
  TDP_ERR_ALIGN = -7        /* a device pointer is not 16-byte aligned             */
} tdp_status;

typedef enum { TDP_F32 = 0, TDP_BF16 = 1 } tdp_dtype;

/* Static string naming a status (never NULL). */
const char *tdp_status_string(int32_t status);

/* ------------------------------------------------------------------------ */
/* Plan (host only)                                                          */
/* ------------------------------------------------------------------------ */

/* One dimension's tiling: a tile COUNT and an overlap in latent grid units
 * ("API / Tiling config": counts, not sizes).  Boxes: the dimension [0, L) is
 * split into num_tiles cores [c_i, c_{i+1}), c_i = floor(i L / num_tiles); core
 * i is widened by floor(overlap/2) on the left and ceil(overlap/2) on the
 * right, clipped to [0, L), so neighbours overlap by exactly `overlap`.
 * Requires 1 <= num_tiles <= L and, for num_tiles > 1,
 * 0 <= overlap <= smallest core length; num_tiles == 1 ignores overlap. */
typedef struct {
  int32_t num_tiles;
  int32_t overlap;
} tdp_dim_tiling;

typedef struct {
  int32_t grid[3];            /* (F, H, W) patchified latent grid, each >= 1        */
  tdp_dim_tiling tiling[3];   /* frames, height, width                              */
  int32_t n_cond;             /* M >= 0 conditioning tokens, appended after the
                                 N = F*H*W generated tokens                         */
  const float *cond_pos;      /* host [M][3][2]: (start, end) per dim (t, h, w), in
                                 latent units; NULL iff M == 0; finite values       */
  int32_t normalize_positions;/* 1 (default) or 0 ("Position normalization")        */
  int32_t world_size, rank;   /* round-robin share: tile t belongs to rank
                                 t mod world_size ("What it is"); (1, 0) = all     */
  int32_t assignment;         /* 0 (default): the page's round robin above;
                                 1: longest first -- tiles by attention cost
                                 rows^2 (rows = generated + kept conditioning),
                                 largest first (ties: lower index), each to the
                                 rank with the least cost so far (ties: lower
                                 rank).  A rank's tiles are listed in ascending
                                 index either way.                                 */
} tdp_plan_desc;

typedef struct {
  int32_t n_tiles_total;      /* T = product of the tile counts                    */
  int32_t n_tiles_local;      /* tiles of this rank                                */
  int32_t max_tile_rows;      /* largest local tile (generated + kept cond rows)   */
  int32_t n_gen_total;        /* N                                                 */
  int64_t n_rows;             /* sum of local tile rows                            */
  int64_t n_dst_rows;         /* N + M                                             */
} tdp_plan_sizes;

/* Caller-owned host arrays, sized from tdp_plan_sizes.  Tile order: global
 * tile index t = (i_f * n_h + i_h) * n_w + i_w, local tiles ascending.  A
 * tile's rows are its generated tokens, row-major over its box (w fastest),
 * then its kept conditioning tokens in ascending j. */
typedef struct {
  int32_t *tile_id;           /* [n_tiles_local] global tile index                 */
  int32_t *tile_box;          /* [n_tiles_local][3][2] box [a, b) per dim          */
  float *tile_offset;         /* [n_tiles_local][3] subtracted positions (0 if off)*/
  int64_t *tile_row_begin;    /* [n_tiles_local + 1] CSR of rows over tiles        */
  int32_t *tile_n_gen;        /* [n_tiles_local] generated rows of each tile       */
  int32_t *row_src;           /* [n_rows] global token: (f*H + h)*W + w, or N + j  */
  float *row_weight;          /* [n_rows] trapezoid mask product, or 1/k_j         */
  float *row_pos;             /* [n_rows][3][2] normalized (start, end)            */
  int32_t *cond_keep_count;   /* [M] k_j = tiles (of all ranks) keeping token j    */
  int64_t *dst_row_begin;     /* [n_dst_rows + 1] inverse CSR over global tokens   */
  int32_t *dst_rows;          /* [n_rows] rows feeding each token, ascending       */
} tdp_plan_out;

/* Sizes of a rank's plan.  Errors: TDP_ERR_NULL, TDP_ERR_ARG (bad grid,
 * tiling, M < 0, world_size < 1, rank outside [0, world_size)). */
tdp_status tdp_plan_query(const tdp_plan_desc *desc, tdp_plan_sizes *sizes);

/* Fill a rank's plan.
 *  Masks ("What it is": trapezoidal masks summing to one): along a dimension,
 *  at the k-th position (k = 0..o-1) of the overlap between tiles i-1 and i,
 *  tile i weighs (2k+1)/(2o) and tile i-1 weighs (2o-2k-1)/(2o), each a
 *  float32 quotient; 1 elsewhere, grid edges included.  A generated row's
 *  weight is the float32 product (w_f * w_h) * w_w.
 *  Positions ("Position normalization"): generated token (f, h, w) has the
 *  intervals [f, f+1), [h, h+1), [w, w+1).  A tile's offset per dim is the
 *  smallest start of its generated tokens (0 when normalize_positions == 0)
 *  and is subtracted from both ends of all its rows.
 *  Keep rule ("Shared negative (reference) positions"): token j is kept by a
 *  tile when its time start is < 0, or when in all three dims
 *  start < tile_end and end > tile_start (the tile's generated extent, in
 *  global units).  Its weight is 1.0f / k_j; a token no tile keeps gets no
 *  row.  `sizes` must be the values tdp_plan_query returned for `desc`
 *  (TDP_ERR_SHAPE otherwise).  All out arrays are required (TDP_ERR_NULL). */
tdp_status tdp_plan(const tdp_plan_desc *desc, const tdp_plan_sizes *sizes,
                    tdp_plan_out *out);

/* Tile counts for a balanced 2D (height x width) grid of n tiles, one per
 * rank of a group ("Usage": the full-resolution stage asks for such a split of
 * the group size; the page does not define it).  Writes the factor pair
 * h * w = n with h <= w and w - h smallest: h is the largest divisor of n not
 * above sqrt(n).  Host only; both outputs are caller-owned.
 * Errors: TDP_ERR_NULL (an output is NULL), TDP_ERR_ARG (n < 1). */
tdp_status tdp_balanced_tile_split(int32_t n, int32_t *h_tiles, int32_t *w_tiles);

/* ------------------------------------------------------------------------ */
/* Gather (device)                                                           */
/* ------------------------------------------------------------------------ */

/* x_tiles[b][r][:] = x_global[b][row_src[r]][:] ("What it is": each tile is a
 * piece of the latent; kept conditioning rows follow the generated ones).
 *  x_global: device [batch][n_src_rows][C], dtype `dtype`.
 *  row_src:  device [n_rows] int32, each in [0, n_src_rows) (rows outside are
 *            written as zeros, never read out of bounds).
 *  x_tiles:  device [batch][n_rows][C], same dtype.
 * C must be a positive multiple of 8.  n_rows == 0 is a no-op. */
tdp_status tdp_gather_tiles(const void *x_global, int32_t dtype, int32_t batch,
                            int64_t n_src_rows, int32_t C, const int32_t *row_src,
                            int64_t n_rows, void *x_tiles, void *hip_stream);

/* ------------------------------------------------------------------------ */
/* Per-tile attention (device)                                               */
/* ------------------------------------------------------------------------ */

/* The denoiser run on every tile ("What it is": each rank applies the whole
 * denoising network to the tiles it holds; "When to use it": the cost of
 * attention grows with the square of a tile's token count).  It is one multi-head self-attention layer, no bias,
 * no norm, no residual:  per tile t and batch b, with S = [tile rows ; audio
 * rows] (audio untiled, attended on every tile forward),
 *   Q = S Wq, K = S Wk, V = S Wv          (bf16 operands, fp32 accumulation)
 *   3D RoPE on the Q and K of tile rows at their normalized positions
 *     ("Position normalization"): head_dim/2 interleaved pairs (2i, 2i+1),
 *     p = head_dim/6 pairs per axis: pairs [0,p) time, [p,2p) height,
 *     [2p,3p) width, the rest unrotated; pair j of an axis turns by
 *     m * rope_base^(-j/p), m = (start + end)/2 of the row's interval.
 *     Audio rows are not rotated.
 *   O_h = softmax(Q_h K_h^T / sqrt(head_dim)) V_h, bidirectional, no mask
 *   Y = [O_1 .. O_heads] Wo
 * Tile rows of Y go to y_tiles, audio rows to y_audio_tiles[t]. */
typedef struct {
  int32_t batch;              /* B >= 1                                           */
  int32_t C;                  /* channels; must be 128                            */
  int32_t heads;              /* >= 1                                             */
  int32_t head_dim;           /* 64 or 128                                        */
  int32_t n_audio;            /* A >= 0 audio tokens                              */
  int32_t x_dtype;            /* dtype of x_tiles and x_audio (TDP_F32/TDP_BF16)  */
  int32_t y_dtype;            /* dtype of y_tiles                                 */
  float rope_base;            /* > 0; 10000 in the workloads                      */
  int32_t kv_splits;          /* 0: chosen from the launch size; 1: never split;
                               * 2..8: the keys of every query block of the core
                               * are split into this many parts, each part's
                               * partial softmax sums (fp32, in the workspace) are
                               * combined afterwards.  Splitting fills the GPU
                               * when there are few query blocks (the sequence-
                               * parallel share: all tokens, few heads).  0 splits
                               * only such launches; self-attention launches of
                               * 256 or more query blocks (d = 128) never split.
                               * With 0, an unsplit launch of two rounds or more
                               * also leaves its last ~1/12 of the query blocks
                               * to whichever workgroups reach them first (the
                               * XCDs run at different clocks); with 1 every
                               * block's workgroup is fixed.  The results are
                               * bitwise the same either way. */
} tdp_attn_desc;

/* Workspace bytes tdp_tile_attention needs for these sizes.  Errors as
 * tdp_tile_attention's shape checks.  When desc->kv_splits asks for key parts
 * (or 0 chooses them for a launch of few query blocks) the bytes include the
 * parts' fp32 partial results: (query blocks x parts x rows) x (4 head_dim + 8). */
tdp_status tdp_tile_attention_workspace(const tdp_attn_desc *desc, int32_t n_tiles,
                                        int64_t n_rows, size_t *bytes);

/*  tile_row_begin: device [n_tiles + 1] int64 CSR (from tdp_plan): non-
 *                  decreasing, [0] = 0, [n_tiles] = n_rows, every tile at most
 *                  max_tile_rows rows.  (A violation gives wrong results but
 *                  every access stays inside the caller's buffers and the
 *                  workspace.)
 *  x_tiles:   device [B][n_rows][C] (x_dtype), e.g. from tdp_gather_tiles.
 *  row_pos:   device [n_rows][3][2] float32 normalized positions (tdp_plan).
 *  wq, wk, wv: device [C][heads*head_dim] bf16;  wo: device [heads*head_dim][C]
 *             bf16 (row-major [in][out]).
 *  x_audio:   device [B][A][C] (x_dtype), NULL iff A == 0.
 *  y_tiles:   device [B][n_rows][C] (y_dtype), overwritten.
 *  y_audio_tiles: device [n_tiles][B][A][C] float32, NULL iff A == 0.
 *  workspace: device, >= tdp_tile_attention_workspace bytes; scratch, its
 *             contents are overwritten. */
tdp_status tdp_tile_attention(const tdp_attn_desc *desc, int32_t n_tiles,
                              const int64_t *tile_row_begin, int32_t max_tile_rows,
                              int64_t n_rows, const void *x_tiles, const float *row_pos,
                              const void *wq, const void *wk, const void *wv,
                              const void *wo, const void *x_audio, void *y_tiles,
                              float *y_audio_tiles, void *workspace,
                              size_t workspace_bytes, void *hip_stream);

/* The same step split into its three stages, for callers that time or
 * schedule them separately.  tdp_tile_attention == prepare; qkv_rope;
 * core; out_proj, on one stream with the same arguments and workspace.
 *  prepare:  transposed weights and the tile -> 128-row block table.
 *  qkv_rope: the Q/K/V projection with RoPE, into the workspace.
 *  core:     softmax(QK^T/sqrt(d))V per tile, head and batch, into the
 *            workspace (bf16 O); with key parts (desc->kv_splits), the
 *            parts' partial sums and then their combination.
 *  out_proj: Y = O Wo into y_tiles and y_audio_tiles. */
tdp_status tdp_attn_prepare(const tdp_attn_desc *desc, int32_t n_tiles,
                            const int64_t *tile_row_begin, int32_t max_tile_rows,
                            int64_t n_rows, const void *wq, const void *wk,
                            const void *wv, const void *wo, void *workspace,
                            size_t workspace_bytes, void *hip_stream);
tdp_status tdp_attn_qkv_rope(const tdp_attn_desc *desc, int32_t n_tiles,
                             const int64_t *tile_row_begin, int32_t max_tile_rows,
                             int64_t n_rows, const void *x_tiles, const float *row_pos,
                             const void *x_audio, void *workspace,
                             size_t workspace_bytes, void *hip_stream);
tdp_status tdp_attn_core(const tdp_attn_desc *desc, int32_t n_tiles,
                         const int64_t *tile_row_begin, int32_t max_tile_rows,
                         int64_t n_rows, void *workspace, size_t workspace_bytes,
                         void *hip_stream);
tdp_status tdp_attn_out_proj(const tdp_attn_desc *desc, int32_t n_tiles,
                             const int64_t *tile_row_begin, int32_t max_tile_rows,
                             int64_t n_rows, void *y_tiles, float *y_audio_tiles,
                             void *workspace, size_t workspace_bytes, void *hip_stream);

/* For callers that cannot allocate device memory (code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc): the
 * tdp_tile_attention layer with the same arguments minus the workspace, which
 * comes from a scratch array inside the library instead.  That array has
 * TDP_NOALLOC_SCRATCH_BYTES bytes; every GPU the library runs on holds its own
 * copy from the first use until the process ends.  The call allocates
 * nothing and uses the current device's copy (make the stream's device
 * current).  Every call on one GPU shares that copy: calls that overlap on one
 * GPU (other streams, other threads) race and give wrong results; calls in
 * one stream are ordered.  Results equal tdp_tile_attention's bit for bit.
 * Errors: those of tdp_tile_attention; TDP_ERR_BUFFER when
 * tdp_tile_attention_workspace for these sizes exceeds
 * TDP_NOALLOC_SCRATCH_BYTES (checked before any device work);
 * TDP_ERR_HIP when the scratch address cannot be found. */
#define TDP_NOALLOC_SCRATCH_BYTES (64u << 20)
tdp_status tdp_tile_attention_noalloc(const tdp_attn_desc *desc, int32_t n_tiles,
                                      const int64_t *tile_row_begin, int32_t max_tile_rows,
                                      int64_t n_rows, const void *x_tiles,
                                      const float *row_pos, const void *wq, const void *wk,
                                      const void *wv, const void *wo, const void *x_audio,
                                      void *y_tiles, float *y_audio_tiles, void *hip_stream);

/* ------------------------------------------------------------------------ */
/* Blend (device) - the on-device stand-in for the multi-GPU all_reduce      */
/* ------------------------------------------------------------------------ */

/* y_global[b][n][:] (+)= sum over k in [dst_row_begin[n], dst_row_begin[n+1])
 *                         of row_weight[r] * y_tiles[b][r][:],  r = dst_rows[k]
 * ("What it is": masked tiles summed into the result; "Shared negative
 * (reference) positions": conditioning rows weigh 1/k).  Rows are summed in
 * the order dst_rows lists them (ascending tile), in float32.  One thread
 * writes each output element: deterministic, no atomics.
 *  y_tiles:       device [batch][n_rows][C] (dtype `dtype`).
 *  dst_row_begin: device [n_dst_rows + 1] int64 (tdp_plan), non-decreasing,
 *                 last entry <= n_rows.
 *  dst_rows:      device int32 row ids in [0, n_rows) (others are skipped).
 *  row_weight:    device [n_rows] float32.
 *  y_global:      device [batch][n_dst_rows][C] float32; overwritten when
 *                 accumulate == 0, added to when accumulate == 1 (the sum over
 *                 ranks of a multi-rank plan).
 * C must be a positive multiple of 8. */
tdp_status tdp_blend_accumulate(const void *y_tiles, int32_t dtype, int32_t batch,
                                int64_t n_rows, int32_t C, const int64_t *dst_row_begin,
                                const int32_t *dst_rows, const float *row_weight,
                                int64_t n_dst_rows, float *y_global, int32_t accumulate,
                                void *hip_stream);

/* Audio average ("What it is": the audio stream is not cut into tiles; it
 * enters each tile's forward pass, and the tiles' audio results are then
 * averaged):
 *   y_audio[b][a][:] (+)= sum_t (1 / n_tiles_total) * y_audio_tiles[t][b][a][:]
 * over the n_tiles_local tiles given, in ascending t, float32.
 *  y_audio_tiles: device [n_tiles_local][batch][A][C] float32.
 *  y_audio:       device [batch][A][C] float32. */
tdp_status tdp_audio_accumulate(const float *y_audio_tiles, int32_t n_tiles_local,
                                int32_t n_tiles_total, int32_t batch, int32_t n_audio,
                                int32_t C, float *y_audio, int32_t accumulate,
                                void *hip_stream);

/* ------------------------------------------------------------------------ */
/* Per-tile transformer block (device)                                       */
/* ------------------------------------------------------------------------ */

/* The TDP page ("What it is") has each rank apply the whole denoising
 * network to its tiles and describes no part of it.  This library's reading is L blocks of
 *   h = rms(x)(1 + scale_a) + shift_a;  x += gate_a * SelfAttn(h)
 *   h = rms(x);                         x += CrossAttn(h, text)
 *   h = rms(x)(1 + scale_f) + shift_f;  x += gate_f * FFN(h)
 * around x_0 = X W_in and y = rms(x_L) W_out, per tile and batch entry, with
 *  rms(x) = x / sqrt(mean(x^2) + 1e-6) (no weight);
 *  (shift_a, scale_a, gate_a, shift_f, scale_f, gate_f) = table_l +
 *    silu(emb(tau_b) Wt1) Wt2 split into six D-vectors, emb(tau) =
 *    [cos(tau w_i), sin(tau w_i)], w_i = 10000^(-i/(time_dim/2));
 *  SelfAttn = the tdp_tile_attention layer at width D = heads * head_dim
 *    (3D RoPE on row_pos, softmax(Q K^T / sqrt(d)) V, no bias);
 *  CrossAttn: queries from the tile rows, keys and values from the batch
 *    entry's n_text text tokens (width D), no rotation, no mask;
 *  FFN(h) = gelu_tanh(h W1) W2, width 4D.  No biases.
 * The residual stream is float32, matrix operands bf16. */
typedef struct {
  int32_t batch, C;            /* C must be 128 */
  int32_t heads, head_dim;     /* head_dim 64 or 128; D = heads * head_dim, a multiple of 128 */
  int32_t n_text, layers;      /* n_text >= 1, layers >= 0 */
  int32_t time_dim;            /* timestep embedding width, a multiple of 64 (256) */
  int32_t x_dtype, y_dtype;    /* tdp_dtype of x_tiles and y_tiles */
  float rope_base;             /* 10000 */
} tdp_block_desc;

/* One block's weights: device pointers, bf16 matrices stored [out][in]
 * row-major (the transpose of x W); every pointer 16-byte aligned
 * (TDP_ERR_ALIGN otherwise). */
typedef struct {
  const void *wqkv;            /* [3D][D]: rows of Wq^T, then Wk^T, then Wv^T */
  const void *wo;              /* [D][D] */
  const void *cq;              /* [D][D]  cross-attention query */
  const void *ckv;             /* [2D][D] cross-attention key rows, then value rows */
  const void *co;              /* [D][D] */
  const void *w1;              /* [4D][D] */
  const void *w2;              /* [D][4D] */
  const float *table;          /* [6][D] float32 modulation table */
} tdp_block_layer;

typedef struct {
  const void *w_in;            /* [D][C] */
  const void *w_out;           /* [C][D] */
  const void *wt1;             /* [D][time_dim] */
  const void *wt2;             /* [6D][D] */
  const tdp_block_layer *layers;   /* host array of `layers` entries */
} tdp_block_weights;

/* Workspace bytes of tdp_block_forward.  Errors: TDP_ERR_NULL, TDP_ERR_ARG,
 * TDP_ERR_UNSUPPORTED (C, head_dim, D or dtypes outside the above). */
tdp_status tdp_block_workspace(const tdp_block_desc *desc, int32_t n_tiles, int64_t n_rows,
                               size_t *bytes);

/* y_tiles = the per-tile transformer of x_tiles, for every tile of a rank's
 * plan (the tile arguments are those of tdp_tile_attention).
 *  x_tiles:  device [batch][n_rows][C], x_dtype.
 *  row_pos:  device [n_rows][3][2] float32 (tdp_plan's normalized positions).
 *  text:     device [batch][n_text][D] bf16.
 *  tau:      device [batch] float32 timesteps.
 *  y_tiles:  device [batch][n_rows][C], y_dtype.
 * Asynchronous on hip_stream; the library allocates nothing.  Errors:
 * TDP_ERR_NULL, TDP_ERR_ARG, TDP_ERR_UNSUPPORTED, TDP_ERR_BUFFER (workspace
 * too small), TDP_ERR_ALIGN, TDP_ERR_HIP. */
tdp_status tdp_block_forward(const tdp_block_desc *desc, int32_t n_tiles,
                             const int64_t *tile_row_begin, int32_t max_tile_rows,
                             int64_t n_rows, const void *x_tiles, const float *row_pos,
                             const void *text, const float *tau, const tdp_block_weights *weights,
                             void *y_tiles, void *workspace, size_t workspace_bytes,
                             void *hip_stream);

/* ------------------------------------------------------------------------ */

/* The upscale loop.  TDP page, "When to use it" (the note on stages): TDP is
 * the upscale stage, run on a first stage's full-frame result; it re-injects
 * noise up to a first sigma, then denoises, and its tiles drift apart more as
 * that sigma grows; conditioning on the stage-1 result at negative time
 * indices keeps them together.  The page names no sampler.  This library's
 * reading is the flow-matching form:
 *  - a latent at noise level sigma in [0, 1] is (1 - sigma) x0 + sigma eps;
 *  - the blend of the tile outputs is the velocity v (eps - x0);
 *  - one step from sigma_i to sigma_{i+1}: x += (sigma_{i+1} - sigma_i) v,
 *    on the generated rows only; conditioning rows keep their clean tokens;
 *  - the transformer's timestep is tau = 1000 sigma;
 *  - seam spread of a step: over the batch entries and the generated tokens
 *    that two or more of the given rows cover, S2 = sum_r w_r |y_r - v|^2 and
 *    S0 = sum |v|^2; reported as {S2, S0, sqrt(S2 / S0)} (0 when S0 = 0). */

/* sigmas[i] = sigma0 (1 - i / n_steps), i = 0..n_steps, computed in double and
 * rounded once to float; sigmas[0] = sigma0 when n_steps = 0.  Host array of
 * n_steps + 1 floats, caller-owned.  Errors: TDP_ERR_NULL, TDP_ERR_ARG
 * (n_steps < 0, sigma0 outside [0, 1]). */
tdp_status tdp_linear_sigmas(float sigma0, int32_t n_steps, float *sigmas);

/* x[b][n] = (1 - sigma0) x_stage1[b][n] + sigma0 noise[b][n] for generated
 * rows n < n_gen, x_stage1[b][n] for the conditioning rows [n_gen, n_dst_rows).
 *  x_stage1, x: device [batch][n_dst_rows][C] float32 (x may be x_stage1).
 *  noise:       device [batch][n_gen][C] float32.
 * C a multiple of 4; buffers 16-byte aligned.  Asynchronous on hip_stream.
 * Errors: TDP_ERR_ARG, TDP_ERR_NULL, TDP_ERR_ALIGN, TDP_ERR_HIP. */
tdp_status tdp_renoise(const float *x_stage1, const float *noise, int32_t batch, int64_t n_gen,
                       int64_t n_dst_rows, int32_t C, float sigma0, float *x,
                       void *hip_stream);

/* Workspace bytes tdp_blend_euler needs when it reports the seam spread. */
tdp_status tdp_blend_euler_workspace(int32_t batch, int64_t n_gen, int32_t C, size_t *bytes);

/* One Euler step on the blended tile outputs: for every generated token
 * n < n_gen, v = the tdp_blend_accumulate sum of its rows (same order), and
 * x[b][n] += (sigma_next - sigma) v; rows [n_gen, n_dst_rows) of x are not
 * touched.  The blended v is not stored.
 *  y_tiles:   device [batch][n_rows][C] (dtype), the tile outputs.
 *  dst_row_begin / dst_rows / row_weight: tdp_plan's inverse map and weights
 *             on the device.
 *  x:         device [batch][n_dst_rows][C] float32, updated in place.
 *  seam:      device double[3] receiving {S2, S0, sqrt(S2 / S0)} of this step,
 *             or NULL; then workspace may be NULL.
 *  workspace: device, tdp_blend_euler_workspace bytes (partial sums).
 * Asynchronous on hip_stream.  Errors: TDP_ERR_ARG, TDP_ERR_UNSUPPORTED,
 * TDP_ERR_NULL, TDP_ERR_BUFFER, TDP_ERR_ALIGN, TDP_ERR_HIP. */
tdp_status tdp_blend_euler(const void *y_tiles, int32_t dtype, int32_t batch, int64_t n_rows,
                           int32_t C, const int64_t *dst_row_begin, const int32_t *dst_rows,
                           const float *row_weight, int64_t n_gen, float *x, int64_t n_dst_rows,
                           float sigma, float sigma_next, double *seam, void *workspace,
                           size_t workspace_bytes, void *hip_stream);

/* A rank's plan (tdp_plan's arrays) copied to the device, for the loop. */
typedef struct {
  int32_t n_tiles, max_tile_rows;
  int64_t n_rows;              /* tile rows of all local tiles */
  int64_t n_gen;               /* N = F * H * W generated tokens */
  int64_t n_dst_rows;          /* N + M */
  const int64_t *tile_row_begin;   /* [n_tiles + 1] */
  const int32_t *row_src;          /* [n_rows] */
  const float *row_weight;         /* [n_rows] */
  const float *row_pos;            /* [n_rows][3][2] */
  const int64_t *dst_row_begin;    /* [n_dst_rows + 1] */
  const int32_t *dst_rows;         /* [n_rows] */
} tdp_plan_dev;

/* Workspace bytes of tdp_upscale_loop (the block's workspace, float32 tile
 * buffers, partial sums).  desc->x_dtype and y_dtype must be TDP_F32
 * (TDP_ERR_UNSUPPORTED otherwise). */
tdp_status tdp_upscale_workspace(const tdp_block_desc *desc, const tdp_plan_dev *plan,
                                 size_t *bytes);

/* n_steps steps of the upscale loop on x, the re-noised latent (tdp_renoise):
 * for i = 0 .. n_steps - 1, tau = 1000 sigmas[i]; x_tiles = gather(x);
 * y_tiles = tdp_block_forward(x_tiles, tau); tdp_blend_euler(y_tiles, sigmas[i],
 * sigmas[i + 1]).
 *  sigmas: host float[n_steps + 1], each in [0, 1] (tdp_linear_sigmas).
 *  x:      device [batch][n_dst_rows][C] float32, in place; holds the result.
 *  seam:   device double[n_steps][3] (per step, as tdp_blend_euler) or NULL.
 *  text, weights: as tdp_block_forward.
 * Asynchronous on hip_stream; the library allocates nothing.  Errors: those
 * of tdp_block_forward, TDP_ERR_ARG (a sigma outside [0, 1]). */
tdp_status tdp_upscale_loop(const tdp_block_desc *desc, const tdp_plan_dev *plan,
                            const tdp_block_weights *weights, const void *text,
                            const float *sigmas, int32_t n_steps, float *x, double *seam,
                            void *workspace, size_t workspace_bytes, void *hip_stream);

/* ------------------------------------------------------------------------ */

/* Sequence parallelism (SP) for the first stage: the head exchange.  LTX-2
 * sequence-parallel guide (how a denoising step is split; the all2all
 * kernel): the W ranks hold equal contiguous slices of the (padded) tokens;
 * before self-attention an exchange gives every rank all tokens of H/W of
 * the heads (rank s: heads [s H/W, (s+1) H/W)), and after it the inverse
 * exchange returns each rank's token slice with the outputs of all heads.
 * These calls are one rank's half of each exchange, as direct copies into
 * (or out of) every rank's buffer: pointers to this GPU's memory, or to peer
 * buffers mapped into the process.  Cross-GPU completion signalling is the
 * caller's (not needed on one GPU).
 *
 * Layouts (row-major, dtype elements): this rank's slice [t_loc][heads][d];
 * each rank's head buffer [world t_loc][heads / world][d], token t of rank r
 * at row r t_loc + t.  Constraints: 1 <= world <= 16, heads % world == 0,
 * (heads / world) d a multiple of 16 bytes; 16-byte aligned buffers.  The
 * exchange moves bytes only: tdp_sp_gather_heads after tdp_sp_send_heads
 * returns the slice bit for bit.  Asynchronous on hip_stream.  Errors:
 * TDP_ERR_ARG, TDP_ERR_UNSUPPORTED, TDP_ERR_NULL, TDP_ERR_ALIGN, TDP_ERR_HIP. */

/* dst[s] rows [rank t_loc, (rank+1) t_loc) <- src's heads of rank s.
 * dst: host array of `world` device pointers. */
tdp_status tdp_sp_send_heads(const void *src, int32_t dtype, int64_t t_loc, int32_t heads,
                             int32_t head_dim, int32_t world, int32_t rank, void *const *dst,
                             void *hip_stream);

/* dst's heads of rank s <- src[s] rows [rank t_loc, (rank+1) t_loc).
 * src: host array of `world` device pointers. */
tdp_status tdp_sp_gather_heads(const void *const *src, int32_t dtype, int64_t t_loc,
                               int32_t heads, int32_t head_dim, int32_t world, int32_t rank,
                               void *dst, void *hip_stream);

#ifdef __cplusplus
}
#endif

#endif /* TDP_H */
