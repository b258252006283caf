// Per-tile multi-head self-attention with 3D RoPE on gfx950 (MI355X).
//
// "Tiled Data Parallelism (TDP)" page: "What it is" - every tile runs the
// denoiser with only its own rows (plus the untiled audio tokens); "When to
// use it" - attention is quadratic in a tile's token count, which is where the
// time goes; "Position normalization" - RoPE sees each tile's normalized
// positions.  The denoiser is one attention layer (see tdp.h).
//
// Stages (one stream):
//   prepare   W^T copies of the weights; a table mapping every 128-row block
//             of the padded row space to (tile, first row).
//   qkv_rope  Q, K (row-major per token) and V^T (keys contiguous) in bf16,
//             RoPE applied to the fp32 accumulator; tiles padded to 256 rows
//             with zero rows so every K/V block load is aligned and finite.
//   core      flash attention per (batch, head, 256-query block): S^T = K Q^T
//             and O^T += V^T P^T on v_mfma_f32_32x32x16_bf16.  With keys on
//             the MFMA rows, a lane holds one query's scores, so the online
//             softmax needs one cross-half exchange per 64-key block, and P
//             stays in registers as the B operand of the second MFMA.
//   out_proj  Y = O Wo on MFMA, into y_tiles / y_audio_tiles.
#include <algorithm>
#include <cmath>
#include <mutex>
#include <type_traits>

#include "tdp_common.h"
#include "tdp_internal.h"

// Waves (of 32 query rows each) per attention workgroup, 4 or 8, and keys
// per iteration, 64 or 128; 0 = per head dim (measured best: 8 waves and
// 128-key blocks at head_dim 128, one workgroup per CU; 4 waves and 64-key
// blocks at head_dim 64).
#ifndef TDP_ATTN_WAVES
#define TDP_ATTN_WAVES 0
#endif
#ifndef TDP_ATTN_BN
#define TDP_ATTN_BN 0
#endif
// Keys per compute part of a block without the pipeline (32, 64 or 128;
// 0 = the whole block; measured: parts of 32 or 64 keys, with their lower
// register use, run within 1% of whole blocks).  TDP_ATTN_SUB_HI is the part
// size of the upper half of a workgroup's waves (0 = 64): the two waves that
// share a SIMD (wave w and w + kWaves/2) then reach their MFMA-heavy and
// exp-heavy stretches at different times (measured 2% faster at head_dim 128).
#ifndef TDP_ATTN_SUB
#define TDP_ATTN_SUB 0
#endif
#ifndef TDP_ATTN_SUB_HI
#define TDP_ATTN_SUB_HI 0
#endif
// Query groups of 32 per wave (1 or 2): 2 halves the LDS fragment reads and
// the K/V staging per flop, at one wave per SIMD.
#ifndef TDP_ATTN_NG
#define TDP_ATTN_NG 1
#endif

namespace tdp {
namespace {

typedef __attribute__((address_space(1))) void gvoid_t;   // global pointer for direct LDS loads
typedef __attribute__((address_space(3))) void lvoid_t;   // LDS pointer

constexpr int kC = 128;       // channels per token row
constexpr int kBlk = 128;     // rows per block of the padded row space (one QKV workgroup)
constexpr int kUnit = 256;    // tiles are padded to whole units of this many rows
constexpr int kThreads = 256;
constexpr float kLazy = 8.0f; // log2 headroom before the running softmax max is moved
static_assert(kUnit % kBlk == 0, "tile padding covers whole blocks");
constexpr int kNG = TDP_ATTN_NG;

// Shape of the attention core for one head dim.
template <int D>
struct CoreShape {
  static constexpr int kBN = TDP_ATTN_BN ? TDP_ATTN_BN : (D >= 128 ? 128 : 64);   // keys per iteration
  static constexpr int kKT = kBN / 32;                                            // 32-key MFMA tiles
  static constexpr int kWaves = TDP_ATTN_WAVES ? TDP_ATTN_WAVES : (D >= 128 ? 8 : 4);
  static constexpr int kRowsWG = kWaves * 32 * kNG;   // query rows per workgroup
  // tiles per compute part of a block without the pipeline
  static constexpr int kSubKT = (TDP_ATTN_SUB && TDP_ATTN_SUB / 32 < kKT) ? TDP_ATTN_SUB / 32 : kKT;
  static constexpr int kSubHi = (TDP_ATTN_SUB_HI ? TDP_ATTN_SUB_HI : 64) / 32;
  static constexpr int kSubKTHi = kSubHi < kKT ? kSubHi : kKT;   // ... for the upper half of the waves
  static_assert(kBN == 64 || kBN == 128, "64- or 128-key blocks");
  static_assert(kUnit % kBN == 0, "tile padding covers whole key blocks");
  static_assert(kUnit % kRowsWG == 0, "a 256-row unit is split over whole workgroups");
};

__host__ __device__ inline int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }
size_t align256(size_t x) { return (x + 255) & ~static_cast<size_t>(255); }

// Workspace layout (byte offsets, each 256-aligned).
struct Layout {
  int64_t npb = 0;    // 128-row blocks of the padded tile row space (upper bound, even)
  int64_t n_pad = 0;  // npb * 128 rows per (batch, head) slab
  int64_t a_pad = 0;  // audio rows padded to 256
  int32_t n_aqb = 0;  // 256-query audio units per tile
  int32_t hidden = 0;
  size_t off_wt = 0, off_wot = 0, off_pad_begin = 0, off_blk_tile = 0, off_blk_q0 = 0;
  size_t off_kmax = 0;  // [B][heads][T+1] largest squared K row norm per tile (slot T: audio)
  size_t off_pool = 0;  // the core's tail-claim counter (one word right after the maxima)
  int64_t vt_cols = 0;  // columns per V^T row: the padded tile rows, then the padded audio rows
  size_t off_q = 0, off_k = 0, off_vt = 0, off_qa = 0, off_ka = 0;
  size_t off_o = 0, off_oa = 0, total = 0;
  int32_t kv_splits = 1;             // key parts per query slot of the core
  size_t off_op = 0, off_ml = 0;     // its partial results (kv_splits > 1)
};

constexpr int32_t kMaxKvSplits = 8;
constexpr int64_t kCUs = 256;        // compute units of the MI355X

// Core workgroups resident at once: d = 128 is held to one per CU by its
// 131 KB of LDS; d = 64 (4 waves, 32 KB of LDS, ~128 VGPRs) fits four.
int64_t core_resident(int head_dim) { return kCUs * (head_dim == 64 ? 4 : 1); }

// Key parts per query slot when the slots alone leave compute units idle.
// Cost of S parts, in key-block times of a full chip:
//   rounds x (key blocks per part + 3) x (0.70 + 0.30 f) + 1.7 x S slots / resident
// with rounds = ceil(S slots / resident) and f = min(1, S slots / resident)
// the share of resident workgroups a round occupies.  The 3 blocks stand for
// a part's fixed cost (Q fragments, filling the K/V pipeline, partial
// stores); the f term for the shader clock, which falls as more compute
// units run MFMA (the power limit); the last term for the combine's traffic.
// The constants are fitted to the sequence-parallel shares measured on the
// MI355X (6144 keys, head dim 128, core + combine):
//   96 query blocks:  1 part 143-149 us, 2 parts 99-102, 4 parts 112, 8 parts 116;
//   192 query blocks: 1 part 167 us, 4 parts 184;
//   48 query blocks:  1 part 140 us, 5 parts 58.
// At most kMaxKvSplits parts and one per key block; ties keep fewer parts.
int32_t auto_kv_splits(int64_t slots, int64_t nkb, int64_t resident) {
  if (slots >= resident || nkb < 2) return 1;
  auto cost = [&](int64_t s) {
    const double used = static_cast<double>(slots * s) / static_cast<double>(resident);
    const double rounds = static_cast<double>(ceil_div(slots * s, resident));
    const double t = rounds * static_cast<double>(ceil_div(nkb, s) + 3) *
                     (0.70 + 0.30 * std::min(used, 1.0));
    return s > 1 ? t + 1.7 * used : t;
  };
  int32_t best = 1;
  for (int32_t s = 2; s <= kMaxKvSplits && s <= nkb; ++s)
    if (cost(s) < cost(best)) best = s;
  return best;
}

tdp_status make_layout(const tdp_attn_desc *d, int32_t n_tiles, int64_t n_rows, Layout *L) {
  if (!d) return TDP_ERR_NULL;
  if (d->batch < 1 || d->batch > 65535 || d->heads < 1 || d->n_audio < 0 || n_tiles < 1 ||
      n_tiles > (1 << 20) || n_rows < 1 || n_rows > INT32_MAX || !(d->rope_base > 0.0f) ||
      !std::isfinite(d->rope_base))
    return TDP_ERR_ARG;
  if (d->kv_splits < 0 || d->kv_splits > kMaxKvSplits) return TDP_ERR_ARG;
  if (d->C != kC || (d->head_dim != 64 && d->head_dim != 128)) return TDP_ERR_UNSUPPORTED;
  if ((d->x_dtype != TDP_F32 && d->x_dtype != TDP_BF16) ||
      (d->y_dtype != TDP_F32 && d->y_dtype != TDP_BF16))
    return TDP_ERR_UNSUPPORTED;
  const int64_t hidden = static_cast<int64_t>(d->heads) * d->head_dim;
  if (hidden > (1 << 16)) return TDP_ERR_UNSUPPORTED;
  L->hidden = static_cast<int32_t>(hidden);
  // Each tile takes ceil(rows/256) units of 256 rows: at most (rows + 255)/256.
  L->npb = (n_rows + static_cast<int64_t>(kUnit - 1) * n_tiles) / kUnit * (kUnit / kBlk);
  L->n_pad = L->npb * kBlk;
  L->a_pad = ceil_div(d->n_audio, kUnit) * kUnit;
  L->n_aqb = static_cast<int32_t>(L->a_pad / kUnit);
  L->vt_cols = L->n_pad + L->a_pad;
  // lane offsets into a (batch, head) slab of V^T are 32-bit byte offsets
  if (L->vt_cols * d->head_dim * 2 > static_cast<int64_t>(UINT32_MAX)) return TDP_ERR_UNSUPPORTED;
  const size_t B = d->batch, H = d->heads, D = d->head_dim, T = n_tiles, A = d->n_audio;
  size_t off = 0;
  auto take = [&off](size_t bytes) { const size_t o = off; off = align256(off + bytes); return o; };
  L->off_wt = take(3 * hidden * kC * 2);
  L->off_wot = take(kC * hidden * 2);
  L->off_pad_begin = take((T + 1) * 4);
  L->off_blk_tile = take(L->npb * 4);
  L->off_blk_q0 = take(L->npb * 4);
  L->off_kmax = take((B * H * (T + 1) + 1) * 4);
  L->off_pool = L->off_kmax + B * H * (T + 1) * 4;
  L->off_q = take(B * H * L->n_pad * D * 2);
  L->off_k = take(B * H * L->n_pad * D * 2);
  L->off_vt = take(B * H * static_cast<size_t>(L->vt_cols) * D * 2);
  L->off_qa = take(B * H * L->a_pad * D * 2);
  L->off_ka = take(B * H * L->a_pad * D * 2);
  L->off_o = take(B * static_cast<size_t>(n_rows) * hidden * 2);
  L->off_oa = take(T * B * A * hidden * 2);
  // key parts of the core, for the workspace: slots = workgroups of an
  // unsplit launch (upper bound), key blocks of the longest tile (at most
  // n_rows rows) + audio; the launch may take fewer parts (max_tile_rows)
  const int rows_wg = D == 64 ? CoreShape<64>::kRowsWG : CoreShape<128>::kRowsWG;
  const int bn = D == 64 ? CoreShape<64>::kBN : CoreShape<128>::kBN;
  const int64_t slots = (L->npb / (kUnit / kBlk) + static_cast<int64_t>(T) * L->n_aqb) *
                        static_cast<int64_t>(B * H) * (kUnit / rows_wg);
  const int64_t nkb = ceil_div(n_rows, bn) + ceil_div(d->n_audio, bn);
  L->kv_splits = d->kv_splits > 0 ? d->kv_splits : auto_kv_splits(slots, nkb, core_resident(D));
  if (L->kv_splits > 1) {
    const size_t parts = static_cast<size_t>(slots) * L->kv_splits * rows_wg;
    L->off_op = take(parts * D * 4);
    L->off_ml = take(parts * 8);
  }
  L->total = off;
  return TDP_OK;
}

template <typename T>
T *ws_at(void *ws, size_t off) { return reinterpret_cast<T *>(static_cast<char *>(ws) + off); }

// ---------------------------------------------------------------------------
// prepare
// ---------------------------------------------------------------------------

// dst[m][f][c] = src_m[c][f] for the three [C][hidden] input projections, and
// wot[c][f] = wo[f][c].  One thread per element (a few MB, once per call).
__global__ void transpose_weights_kernel(const bf16 *__restrict__ wq, const bf16 *__restrict__ wk,
                                         const bf16 *__restrict__ wv, const bf16 *__restrict__ wo,
                                         int32_t hidden, bf16 *__restrict__ wt,
                                         bf16 *__restrict__ wot) {
  const int64_t i = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
  const int64_t per = static_cast<int64_t>(hidden) * kC;
  if (i < 3 * per) {
    const int64_t m = i / per, rem = i - m * per;
    const int64_t f = rem / kC, c = rem - f * kC;
    const bf16 *src = m == 0 ? wq : (m == 1 ? wk : wv);
    wt[i] = src[c * hidden + f];
  } else if (i < 4 * per) {
    const int64_t j = i - 3 * per;
    const int64_t c = j / hidden, f = j - c * hidden;
    wot[j] = wo[f * kC + c];
  }
}

// Rows of tile t, clamped into [0, n_rows] and to max_rows.
__device__ inline void tile_rows(const int64_t *trb, int32_t t, int64_t n_rows, int32_t max_rows,
                                 int64_t *r0, int32_t *len) {
  int64_t a = trb[t], b = trb[t + 1];
  a = a < 0 ? 0 : (a > n_rows ? n_rows : a);
  b = b < a ? a : (b > n_rows ? n_rows : b);
  *r0 = a;
  *len = static_cast<int32_t>(min(b - a, static_cast<int64_t>(max_rows)));
}

// pad_begin[t] = first 128-row block of tile t in the padded row space, where
// each tile takes a whole number of 256-row units (clamped to npb);
// blk_tile/blk_q0 map each block to its tile and first tile row (-1 for blocks
// past the last tile); also clears the per-tile K norm maxima and, in the
// word after them, the core's tail-claim counter.  One workgroup.
__global__ __launch_bounds__(1024) void block_table_kernel(const int64_t *__restrict__ trb,
                                                           int32_t T, int64_t n_rows,
                                                           int32_t max_rows, int64_t npb,
                                                           int32_t *__restrict__ pad_begin,
                                                           int32_t *__restrict__ blk_tile,
                                                           int32_t *__restrict__ blk_q0,
                                                           uint32_t *__restrict__ kmax2,
                                                           int64_t n_kmax) {
  for (int64_t i = threadIdx.x; i < n_kmax; i += blockDim.x) kmax2[i] = 0u;
  for (int32_t t = threadIdx.x; t < T; t += blockDim.x) {
    int64_t r0;
    int32_t len;
    tile_rows(trb, t, n_rows, max_rows, &r0, &len);
    pad_begin[t + 1] = static_cast<int32_t>(ceil_div(len, kUnit) * (kUnit / kBlk));
  }
  __syncthreads();
  if (threadIdx.x == 0) {
    pad_begin[0] = 0;
    int64_t acc = 0;
    for (int32_t t = 0; t < T; ++t) {
      acc = min(acc + pad_begin[t + 1], npb);
      pad_begin[t + 1] = static_cast<int32_t>(acc);
    }
  }
  __syncthreads();
  const int32_t used = pad_begin[T];
  for (int64_t pb = threadIdx.x; pb < npb; pb += blockDim.x) {
    int32_t tile = -1, q0 = 0;
    if (pb < used) {
      int32_t lo = 0, hi = T - 1;  // last t with pad_begin[t] <= pb
      while (lo < hi) {
        const int32_t mid = (lo + hi + 1) >> 1;
        if (pad_begin[mid] <= pb) lo = mid; else hi = mid - 1;
      }
      tile = lo;
      q0 = static_cast<int32_t>((pb - pad_begin[lo]) * kBlk);
    }
    blk_tile[pb] = tile;
    blk_q0[pb] = q0;
  }
}

// ---------------------------------------------------------------------------
// qkv_rope
// ---------------------------------------------------------------------------

// Column of key x (x % 16 = position in its 16-key group) in V^T: the middle
// two quarters of every 16-key group are swapped, so the keys one lane half
// feeds a 16-key MFMA step of P V, {0..3, 8..11} or {4..7, 12..15}, are
// contiguous.  The map is its own inverse.  (Key blocks start at multiples
// of 16 in the padded row space.)
__device__ inline int vt_column(int x) {
  const int q = (x >> 2) & 3;
  const int q2 = (q == 1 || q == 2) ? 3 - q : q;
  return (x & ~12) | (q2 << 2);
}

// Q, K and V^T are written once with a non-temporal hint (measured on the
// 16-tile step: 3 GB in 0.65 ms instead of 0.93).  The attention core's O
// stays an ordinary store and load: the output projection reads it right
// after, and the part still in the last-level cache then hits (a
// non-temporal O read measured 0.55 ms instead of 0.34).
#ifndef TDP_STREAM_HINTS
#define TDP_STREAM_HINTS 1
#endif
__device__ __forceinline__ void store_stream(bf16x8 *p, bf16x8 v) {
#if TDP_STREAM_HINTS
  __builtin_nontemporal_store(v, p);
#else
  *p = v;
#endif
}

// Workgroup barrier ordering LDS only: waves exchange data through LDS, so
// outstanding global stores need not complete first (a plain __syncthreads
// would wait for them).
__device__ __forceinline__ void lds_barrier() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}

template <typename TX>
__device__ inline bf16x8 load_x8(const TX *p);
template <>
__device__ inline bf16x8 load_x8<bf16>(const bf16 *p) {
  return *reinterpret_cast<const bf16x8 *>(p);
}
template <>
__device__ inline bf16x8 load_x8<float>(const float *p) {
  const f32x4 a = *reinterpret_cast<const f32x4 *>(p);
  const f32x4 b = *reinterpret_cast<const f32x4 *>(p + 4);
  bf16x8 r;
  r[0] = static_cast<bf16>(a[0]); r[1] = static_cast<bf16>(a[1]);
  r[2] = static_cast<bf16>(a[2]); r[3] = static_cast<bf16>(a[3]);
  r[4] = static_cast<bf16>(b[0]); r[5] = static_cast<bf16>(b[1]);
  r[6] = static_cast<bf16>(b[2]); r[7] = static_cast<bf16>(b[3]);
  return r;
}

struct QkvArgs {
  const void *x;              // tile rows [B][x_rows][C] or audio [B][A][C]
  int64_t x_rows;
  const int32_t *blk_tile, *blk_q0, *pad_begin;
  const int64_t *trb;
  int64_t n_rows;
  int32_t max_rows;
  const float *row_pos;       // [n_rows][3][2]
  const bf16 *wt;             // [3][hidden][C]
  int32_t heads, hidden;
  int64_t n_pad;              // padded rows per (batch, head) slab of Q and K
  int64_t vt_cols;            // columns per V^T row
  int64_t vt_col0;            // first V^T column of this launch's rows (audio: after the tiles)
  float log2_theta_step;      // -log2(rope_base) / p
  float q_scale;              // log2(e) / sqrt(head_dim), applied to Q before rounding
  bf16 *q, *k, *vt;
  uint32_t *kmax2;            // [B][heads][T+1] float bits of the largest squared K norm
  int32_t n_tiles;
  int32_t chunks_per_wg;      // output chunks (of 3 * heads) per workgroup; blockIdx.z picks the range
};

// One workgroup = 128 token rows (4 waves x 32) of one batch entry and the
// output chunks [z c, z c + c) of the 3*heads chunks of head_dim features,
// z = blockIdx.z, c = chunks_per_wg (small launches split the chunks over
// more workgroups so the chip fills).  D[feature][token] = W^T X^T on
// MFMA, so a lane owns one token and groups of 4 consecutive features: RoPE
// pairs (2i, 2i+1) sit in one lane and cos/sin depend on that lane's token,
// computed once and reused by every Q and K head.
#ifndef TDP_QKV_TARGET_WGS
#define TDP_QKV_TARGET_WGS 1024
#endif
constexpr int64_t kQkvTargetWgs = TDP_QKV_TARGET_WGS;

template <typename TX, int D, bool AUDIO>
__global__ __launch_bounds__(kThreads, 2) void qkv_rope_kernel(QkvArgs a) {
  constexpr int kFT = D / 32;            // 32-feature MFMA tiles per head
  constexpr int kPairs = D / 4;          // rotation pairs held per lane
  // Waves 0-1 load W^T chunks, waves 2-3 copy output tiles out, so a wave
  // waiting for its loads (vmcnt counts stores too) never waits for stores.
  constexpr int kWUnits = D * kC * 2 / 1024 / 2;   // 1 KB direct loads per loader wave per chunk
  // staged output rows, +8 bytes each: 8-byte aligned, lane rows hit distinct banks
  constexpr int kVtRow = kBlk + 4;       // bf16 per staged V^T row (128 tokens)
  constexpr int kQkRow = D + 4;          // bf16 per staged Q/K row (one token)
  // W^T chunk [D][128]: unpadded 256-byte rows, 16-byte chunk p of row r holds
  // channel chunk p ^ (r % 16) (conflict-free fragment reads).  sOut: the
  // 128-token output tile of one head, [token][D] for Q/K, [D][token] for V^T.
  __shared__ __attribute__((aligned(16))) bf16 sW[D * kC];
  __shared__ __attribute__((aligned(16))) bf16 sOut[(kBlk * kQkRow > D * kVtRow) ? kBlk * kQkRow
                                                                                  : D * kVtRow];

  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int l32 = lane & 31, hh = lane >> 5;
  const int uwave = __builtin_amdgcn_readfirstlane(wave);
  const int64_t b = blockIdx.y;
  const int64_t pb = blockIdx.x;

  int64_t src0 = 0, pad_row0 = 0;
  int32_t nvalid = 0, tile = 0;
  if (AUDIO) {
    src0 = pb * kBlk;
    pad_row0 = pb * kBlk;
    nvalid = static_cast<int32_t>(min(static_cast<int64_t>(kBlk), a.x_rows - src0));
  } else {
    tile = a.blk_tile[pb];
    if (tile < 0) return;
    const int32_t q0 = a.blk_q0[pb];
    int64_t r0;
    int32_t len;
    tile_rows(a.trb, tile, a.n_rows, a.max_rows, &r0, &len);
    src0 = r0 + q0;
    pad_row0 = static_cast<int64_t>(a.pad_begin[tile]) * kBlk + q0;
    nvalid = len - q0;
  }
  const int my = wave * 32 + l32;
  const bool valid = my < nvalid;

  // W^T chunk (m, h) = rows [m*hidden + h*D, +D) of wt, straight into LDS.
  uint32_t woff[kWUnits];
#pragma unroll
  for (int i = 0; i < kWUnits; ++i) {
    const int byte = (i * 2 + (uwave & 1)) * 1024 + 16 * lane;
    const int r = byte / 256, p = (byte % 256) / 16;
    woff[i] = static_cast<uint32_t>(r * 256 + 16 * (p ^ (r % 16)));
  }
  auto load_w = [&](int chunk) {
    const int m = chunk / a.heads, h = chunk - m * a.heads;
    const char *src = reinterpret_cast<const char *>(
        a.wt + (static_cast<int64_t>(m) * a.hidden + static_cast<int64_t>(h) * D) * kC);
#pragma unroll
    for (int i = 0; i < kWUnits; ++i)
      __builtin_amdgcn_global_load_lds((gvoid_t *)(src + woff[i]),
                                       (lvoid_t *)(sW + (i * 2 + uwave) * 512), 16, 0, 0);
  };
  // this lane's fragment offsets: row 32 ft + l32, channel chunk 2 s + hh
  int32_t wro[kC / 16];
#pragma unroll
  for (int st = 0; st < kC / 16; ++st) wro[st] = l32 * kC + 8 * ((2 * st + hh) ^ (l32 % 16));

  const int n_chunks = 3 * a.heads;
  const int c_begin = static_cast<int>(blockIdx.z) * a.chunks_per_wg;
  const int c_end = min(c_begin + a.chunks_per_wg, n_chunks);
  if (uwave < 2) load_w(c_begin);

  // X fragments: token `my`, channels 16s + 8hh + 0..7 (B operand of
  // W^T X^T, A operand of X W).
  bf16x8 xf[kC / 16];
  const TX *xrow = static_cast<const TX *>(a.x) + (b * a.x_rows + src0 + (valid ? my : 0)) * kC;
#pragma unroll
  for (int s = 0; s < kC / 16; ++s) {
    xf[s] = valid ? load_x8<TX>(xrow + 16 * s + 8 * hh) : bf16x8{};
  }

  // cos/sin of the lane's rotation pairs: pair j = 16 ft + 4 g + 2 hh + e.
  float rc[kPairs], rs[kPairs];
  if (!AUDIO) {
    constexpr int p = D / 6;
    float mid[3] = {0.f, 0.f, 0.f};
    if (valid) {
      const float *pp = a.row_pos + (src0 + my) * 6;
#pragma unroll
      for (int ax = 0; ax < 3; ++ax) mid[ax] = 0.5f * (pp[2 * ax] + pp[2 * ax + 1]);
    }
#pragma unroll
    for (int i = 0; i < kPairs; ++i) {
      const int ft = i / 8, g = (i / 2) % 4, e = i % 2;
      const int j = 16 * ft + 4 * g + 2 * hh + e;
      const int ax = j / p;
      float c = 1.f, s = 0.f;
      if (ax < 3) {
        const float theta = exp2f(static_cast<float>(j - ax * p) * a.log2_theta_step);
        const float mv = ax == 0 ? mid[0] : (ax == 1 ? mid[1] : mid[2]);   // no indexed array
        sincosf(mv * theta, &s, &c);
      }
      rc[i] = c;
      rs[i] = s;
    }
  }
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  __syncthreads();

  // The chunk loop is compiled twice: loader waves (W^T direct loads, which
  // the compiler must wait for before LDS reads) and copy waves (global
  // stores only), so copy waves never wait for their stores.  Both copies
  // pass the same barriers.
  auto chunk_loop = [&](auto loader_tag) {
  constexpr bool loader = decltype(loader_tag)::value;
  for (int chunk = c_begin; chunk < c_end; ++chunk) {
    const int m = chunk / a.heads, h = chunk - m * a.heads;
    const int64_t slab = b * a.heads + h;
    float kss = 0.f;   // squared norm of this lane's (rounded) K row of head h
    if (m < 2) {
#pragma unroll
      for (int ft = 0; ft < kFT; ++ft) {
        f32x16 acc = {};
#pragma unroll
        for (int s = 0; s < kC / 16; ++s) {
          const bf16x8 w = *reinterpret_cast<const bf16x8 *>(sW + 32 * ft * kC + wro[s]);
          acc = mfma32(w, xf[s], acc);
        }
        // acc[v]: feature 32 ft + 8 (v/4) + 4 hh + v%4 of token `my`
        if (!AUDIO) {
#pragma unroll
          for (int g = 0; g < 4; ++g) {
#pragma unroll
            for (int e = 0; e < 2; ++e) {
              const int i = ft * 8 + g * 2 + e, v = 4 * g + 2 * e;
              const float x0 = acc[v], x1 = acc[v + 1];
              acc[v] = x0 * rc[i] - x1 * rs[i];
              acc[v + 1] = x0 * rs[i] + x1 * rc[i];
            }
          }
        }
        // Q carries the softmax scale in log2 units, so Q K^T is log2 of the
        // unnormalized attention weight.
        if (m == 0) {
#pragma unroll
          for (int v = 0; v < 16; ++v) acc[v] *= a.q_scale;
        }
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          bf16x4 v4;
          v4[0] = static_cast<bf16>(acc[4 * g + 0]);
          v4[1] = static_cast<bf16>(acc[4 * g + 1]);
          v4[2] = static_cast<bf16>(acc[4 * g + 2]);
          v4[3] = static_cast<bf16>(acc[4 * g + 3]);
          *reinterpret_cast<bf16x4 *>(sOut + my * kQkRow + 32 * ft + 8 * g + 4 * hh) = v4;
          if (m == 1) {
#pragma unroll
            for (int e = 0; e < 4; ++e) {
              const float r = static_cast<float>(v4[e]);
              kss = fmaf(r, r, kss);
            }
          }
        }
      }
    } else {
      // V = X Wv with tokens on the MFMA rows: lane holds head-dim row
      // 32 ft + l32 of V^T and 4 consecutive tokens per group (vt_column keeps
      // a quarter's order).
#pragma unroll
      for (int ft = 0; ft < kFT; ++ft) {
        f32x16 acc = {};
#pragma unroll
        for (int s = 0; s < kC / 16; ++s) {
          const bf16x8 w = *reinterpret_cast<const bf16x8 *>(sW + 32 * ft * kC + wro[s]);
          acc = mfma32(xf[s], w, acc);
        }
        // acc[v]: token wave*32 + 8 (v/4) + 4 hh + v%4, head dim 32 ft + l32
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          bf16x4 v4;
          v4[0] = static_cast<bf16>(acc[4 * g + 0]);
          v4[1] = static_cast<bf16>(acc[4 * g + 1]);
          v4[2] = static_cast<bf16>(acc[4 * g + 2]);
          v4[3] = static_cast<bf16>(acc[4 * g + 3]);
          *reinterpret_cast<bf16x4 *>(sOut + (32 * ft + l32) * kVtRow +
                                      vt_column(wave * 32 + 8 * g + 4 * hh)) = v4;
        }
      }
    }
    if (m == 1) {
      // Largest squared K row norm of the block for this head and tile; the
      // float bits of non-negative floats order like unsigned integers, so the
      // maximum over workgroups is an integer atomic max (order-independent).
      kss += __shfl_xor(kss, 32);
#pragma unroll
      for (int off = 1; off < 32; off <<= 1) kss = fmaxf(kss, __shfl_xor(kss, off));
      if (lane == 0)
        atomicMax(a.kmax2 + slab * (a.n_tiles + 1) + (AUDIO ? a.n_tiles : tile),
                  __float_as_uint(kss));
    }
    lds_barrier();                          // sW read, sOut complete
    if (loader && chunk + 1 < c_end) load_w(chunk + 1);
    // Copy the tile out in 16-byte pieces: consecutive threads, consecutive bytes.
    const int ct = threadIdx.x - 128;      // copy thread of waves 2-3
    if constexpr (loader) {
      // nothing to copy
    } else if (m < 2) {
      bf16 *dst = (m == 0 ? a.q : a.k) + (slab * a.n_pad + pad_row0) * D;
#pragma unroll
      for (int i = 0; i < kBlk * D / 8 / 128; ++i) {
        const int piece = ct + i * 128;
        const int r = piece / (D / 8), col = (piece % (D / 8)) * 8;
        const bf16 *src = sOut + r * kQkRow + col;
        const bf16x4 lo = *reinterpret_cast<const bf16x4 *>(src);
        const bf16x4 hi = *reinterpret_cast<const bf16x4 *>(src + 4);
        store_stream(reinterpret_cast<bf16x8 *>(dst + r * D + col),
                     bf16x8{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]});
      }
    } else {
      bf16 *dst = a.vt + slab * D * a.vt_cols + a.vt_col0 + pad_row0;
#pragma unroll
      for (int i = 0; i < D * kBlk / 8 / 128; ++i) {
        const int piece = ct + i * 128;
        const int d = piece / (kBlk / 8), col = (piece % (kBlk / 8)) * 8;
        const bf16 *src = sOut + d * kVtRow + col;
        const bf16x4 lo = *reinterpret_cast<const bf16x4 *>(src);
        const bf16x4 hi = *reinterpret_cast<const bf16x4 *>(src + 4);
        store_stream(reinterpret_cast<bf16x8 *>(dst + d * a.vt_cols + col),
                     bf16x8{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]});
      }
    }
    if (loader) asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    lds_barrier();                          // W(chunk+1) landed, sOut free
  }
  };
  if (uwave < 2) chunk_loop(std::true_type{});
  else chunk_loop(std::false_type{});
}

// ---------------------------------------------------------------------------
// rows_to_heads: row-major Q / K / V columns into the core's layouts
// ---------------------------------------------------------------------------

// For callers that compute the projections with a general GEMM (the per-tile
// transformer block).  The source holds, per row, head h's features of Q, K
// and V at columns q_col + h D, k_col + h D and v_col + h D (a part is absent
// when its column is negative).  The arithmetic after the projection is that
// of the QKV stage above: RoPE of Q and K from the row's normalized interval
// midpoints (when `rope`), Q times log2(e)/sqrt(D), one bf16 rounding, the
// largest squared K row norm per (batch, head, tile), V^T with vt_column's
// order, zeros in padded rows.
struct HeadsArgs {
  const bf16 *src;             // [B][src_rows][ld]
  int64_t ld, src_rows;
  int32_t q_col, k_col, v_col;
  const float *row_pos;        // [n_rows][3][2], tile rows only
  int32_t rope;
  float log2_theta_step, q_scale;
  bf16 *q, *k, *vt;            // the core's layouts (text rows: the second segment's)
  int64_t n_pad, vt_cols, vt_col0;
  uint32_t *kmax2;
  int32_t n_tiles, heads;
  const int32_t *blk_tile, *blk_q0, *pad_begin;
  const int64_t *trb;
  int64_t n_rows;
  int32_t max_rows;
  int32_t heads_per_wg;        // heads [z h, z h + h) for blockIdx.z = z
};

// One workgroup = 128 rows of the padded row space of one batch entry (tile
// rows: one block of the block table; TEXT: one 128-row block of the text
// rows) and heads_per_wg of the heads (blockIdx.z); thread = (row, half of
// the head dims).
template <int D, bool TEXT>
__global__ __launch_bounds__(256) void rows_to_heads_kernel(HeadsArgs a) {
  constexpr int kHalf = D / 2;        // head dims per thread
  constexpr int kPairs = D / 4;       // rotation pairs per thread
  constexpr int kRow = D + 8;         // staged V row (bf16)
  __shared__ __attribute__((aligned(16))) bf16 sV[kBlk * kRow];
  const int r = threadIdx.x >> 1, half = threadIdx.x & 1;
  const int lane = threadIdx.x & 63;
  const int64_t b = blockIdx.y, pb = blockIdx.x;
  int64_t src0 = 0, pad_row0 = 0;
  int32_t nvalid = 0, tile = a.n_tiles;
  if (TEXT) {
    src0 = pb * kBlk;
    pad_row0 = pb * kBlk;
    nvalid = static_cast<int32_t>(min(static_cast<int64_t>(kBlk), a.src_rows - src0));
  } else {
    tile = a.blk_tile[pb];
    if (tile < 0) return;
    const int32_t q0 = a.blk_q0[pb];
    int64_t r0;
    int32_t len;
    tile_rows(a.trb, tile, a.n_rows, a.max_rows, &r0, &len);
    src0 = r0 + q0;
    pad_row0 = static_cast<int64_t>(a.pad_begin[tile]) * kBlk + q0;
    nvalid = len - q0;
  }
  const bool valid = r < nvalid;
  const bf16 *row = a.src + (b * a.src_rows + src0 + (valid ? r : 0)) * a.ld;

  float rc[kPairs], rs[kPairs];
#pragma unroll
  for (int i = 0; i < kPairs; ++i) { rc[i] = 1.f; rs[i] = 0.f; }
  if (!TEXT && a.rope && valid) {
    constexpr int p = D / 6;
    const float *pp = a.row_pos + (src0 + r) * 6;
    const float mid[3] = {0.5f * (pp[0] + pp[1]), 0.5f * (pp[2] + pp[3]), 0.5f * (pp[4] + pp[5])};
#pragma unroll
    for (int i = 0; i < kPairs; ++i) {
      const int j = half * kPairs + i;
      const int ax = j / p;
      if (ax < 3) {
        const float theta = exp2f(static_cast<float>(j - ax * p) * a.log2_theta_step);
        const float mv = ax == 0 ? mid[0] : (ax == 1 ? mid[1] : mid[2]);
        sincosf(mv * theta, &rs[i], &rc[i]);
      }
    }
  }
  // one part of one head of this thread's row: rotate (Q, K), scale (Q), round
  auto rotated = [&](int col, float scale, bool rot, bf16x8 (&out)[kHalf / 8], float *kss) {
#pragma unroll
    for (int c = 0; c < kHalf / 8; ++c) {
      const bf16x8 in = valid ? *reinterpret_cast<const bf16x8 *>(row + col + half * kHalf + 8 * c)
                              : bf16x8{};
#pragma unroll
      for (int e = 0; e < 8; e += 2) {
        const int i = 4 * c + e / 2;
        float x0 = static_cast<float>(in[e]), x1 = static_cast<float>(in[e + 1]);
        if (rot) {
          const float y0 = x0 * rc[i] - x1 * rs[i];
          const float y1 = x0 * rs[i] + x1 * rc[i];
          x0 = y0;
          x1 = y1;
        }
        out[c][e] = static_cast<bf16>(x0 * scale);
        out[c][e + 1] = static_cast<bf16>(x1 * scale);
        if (kss) {
          const float r0 = static_cast<float>(out[c][e]), r1 = static_cast<float>(out[c][e + 1]);
          *kss = fmaf(r0, r0, fmaf(r1, r1, *kss));
        }
      }
    }
  };
  const int h_end = min(a.heads, static_cast<int>(blockIdx.z + 1) * a.heads_per_wg);
  for (int h = static_cast<int>(blockIdx.z) * a.heads_per_wg; h < h_end; ++h) {
    const int64_t slab = b * a.heads + h;
    bf16x8 out[kHalf / 8];
    if (a.q_col >= 0) {
      rotated(a.q_col + h * D, a.q_scale, !TEXT && a.rope, out, nullptr);
      bf16 *dst = a.q + (slab * a.n_pad + pad_row0 + r) * D + half * kHalf;
#pragma unroll
      for (int c = 0; c < kHalf / 8; ++c) *reinterpret_cast<bf16x8 *>(dst + 8 * c) = out[c];
    }
    if (a.k_col >= 0) {
      float kss = 0.f;
      rotated(a.k_col + h * D, 1.f, !TEXT && a.rope, out, &kss);
      bf16 *dst = a.k + (slab * a.n_pad + pad_row0 + r) * D + half * kHalf;
#pragma unroll
      for (int c = 0; c < kHalf / 8; ++c) *reinterpret_cast<bf16x8 *>(dst + 8 * c) = out[c];
      kss += __shfl_xor(kss, 1);
#pragma unroll
      for (int off = 2; off < 64; off <<= 1) kss = fmaxf(kss, __shfl_xor(kss, off));
      if (lane == 0)
        atomicMax(a.kmax2 + slab * (a.n_tiles + 1) + tile, __float_as_uint(kss));
    }
    if (a.v_col >= 0) {
      rotated(a.v_col + h * D, 1.f, false, out, nullptr);
#pragma unroll
      for (int c = 0; c < kHalf / 8; ++c)
        *reinterpret_cast<bf16x8 *>(sV + r * kRow + half * kHalf + 8 * c) = out[c];
      __syncthreads();
      // V^T row d, columns 8 c8 .. 8 c8 + 7 of the block: key vt_column(col)
      bf16 *vdst = a.vt + slab * D * a.vt_cols + a.vt_col0 + pad_row0;
#pragma unroll
      for (int i = 0; i < D * (kBlk / 8) / 256; ++i) {
        const int piece = threadIdx.x + 256 * i;
        const int d = piece / (kBlk / 8), c8 = piece % (kBlk / 8);
        bf16x8 v8;
#pragma unroll
        for (int e = 0; e < 8; ++e) v8[e] = sV[vt_column(8 * c8 + e) * kRow + d];
        *reinterpret_cast<bf16x8 *>(vdst + d * a.vt_cols + 8 * c8) = v8;
      }
      __syncthreads();
    }
  }
}

// ---------------------------------------------------------------------------
// core
// ---------------------------------------------------------------------------

struct CoreArgs {
  const bf16 *q, *k, *vt, *qa, *ka;   // vt: [B*H][D][vt_cols], tile columns then audio columns
  bf16 *o, *oa;
  const int32_t *blk_tile, *blk_q0, *pad_begin;
  const int64_t *trb;
  int64_t n_units, n_pad, a_pad, vt_cols, n_rows, units_per_bh, total_units;
  int32_t T, heads, batch, A, n_aqb, max_rows, hidden;
  const uint32_t *kmax2;      // [B][heads][T+1] float bits of the largest squared K norm
  int32_t tile_keys;           // 0: attend the second key segment only (cross-attention)
  // Key-split launches only: S parts per query slot, the unnormalized fp32
  // partial O [slot][S][rows per workgroup][D] and its (m, l) per row.
  int32_t kv_splits;
  float *op;
  float2 *ml;
  // Unsplit two-group launches: units assigned per XCD, then the claimed tail
  // (see attn_core2_kernel).
  int64_t per_xcd;
  uint32_t pool_claims;
  uint32_t *pool_ctr;
};

// What one query slot of the core covers: (batch, head), tile, first query
// row and the number of queries from there (the caller clamps it to its
// rows).  False when the slot holds no queries.
struct CoreSlot {
  int64_t bh, b, r0, pad0;
  int32_t h, t, q0, len0, nq;
  bool audio_q;
};

template <int kRowsWG>
__device__ __forceinline__ bool core_slot(const CoreArgs &a, int64_t lid, CoreSlot &s) {
  constexpr int kSplit = kUnit / kRowsWG;   // workgroups per 256-row unit
  const int64_t item = lid / kSplit;
  const int part = static_cast<int>(lid - item * kSplit);
  s.bh = item / a.units_per_bh;
  const int64_t u = item - s.bh * a.units_per_bh;
  s.b = s.bh / a.heads;
  s.h = static_cast<int>(s.bh - s.b * a.heads);
  if (u < a.n_units) {
    s.t = a.blk_tile[u * (kUnit / kBlk)];
    if (s.t < 0) return false;
    s.q0 = a.blk_q0[u * (kUnit / kBlk)];
    s.audio_q = false;
  } else {
    const int64_t ua = u - a.n_units;
    s.t = static_cast<int32_t>(ua / a.n_aqb);
    s.q0 = static_cast<int32_t>((ua - static_cast<int64_t>(s.t) * a.n_aqb) * kUnit);
    s.audio_q = true;
  }
  s.q0 += part * kRowsWG;
  tile_rows(a.trb, s.t, a.n_rows, a.max_rows, &s.r0, &s.len0);
  s.pad0 = static_cast<int64_t>(a.pad_begin[s.t]) * kBlk;
  s.len0 = static_cast<int32_t>(min(static_cast<int64_t>(s.len0),
                                    static_cast<int64_t>(a.pad_begin[s.t + 1]) * kBlk - s.pad0));
  s.nq = s.audio_q ? (a.A - s.q0) : (s.len0 - s.q0);
  return s.nq > 0;
}

// LDS staging of one kBN-key block, unpadded rows with an XOR swizzle of the
// 16-byte chunks inside a row (the layout; the kernel declares the buffers):
//   K   [kBN keys][D]: chunk p of row r holds head-dim chunk p ^ ksw(r)
//   V^T [D][kBN keys]: chunk p of row d holds key chunk p ^ vsw(d)
// Both swizzles make the 16 lanes of an LDS read phase hit 16 different
// 16-byte bank groups.  Blocks arrive by direct global->LDS loads: each
// 16-byte load of a wave lands at LDS base + 16 * lane, so each lane fetches
// the global chunk that belongs at its LDS position.
template <int D>
struct CoreSmem {
  static constexpr int kRB = 2 * D;                 // bytes per K row
  static constexpr int kCPR = D / 8;                // 16-byte chunks per K row
  __device__ static int ksw(int r) { return (r / (256 / kRB)) % kCPR; }
  // V^T rows of kBN keys: 128 / kBN rows share one 256-byte bank window
  static constexpr int kBN = CoreShape<D>::kBN;
  __device__ static int vsw(int d) { return (d / (128 / kBN)) % (kBN / 8); }
};


template <int D>
struct DirectStage {
  static constexpr int kWaves = CoreShape<D>::kWaves;
  static constexpr int kBN = CoreShape<D>::kBN;
  static constexpr int kKUnits = kBN * D * 2 / 1024 / kWaves;   // 1 KB loads per wave, K block
  static constexpr int kVUnits = D * kBN * 2 / 1024 / kWaves;   // 1 KB loads per wave, V^T block
  uint32_t koff[kKUnits];                 // byte offset of this lane's chunk in a K block
  uint32_t voff[kVUnits];                 // ... in a V^T block (rows of vstr columns)
  int wave;                               // wave-uniform

  __device__ DirectStage(int wave_, int lane, uint32_t vstr) : wave(wave_) {
#pragma unroll
    for (int i = 0; i < kKUnits; ++i) {
      const int byte = (i * kWaves + wave) * 1024 + 16 * lane;
      const int r = byte / CoreSmem<D>::kRB, p = (byte % CoreSmem<D>::kRB) / 16;
      koff[i] = 2u * static_cast<uint32_t>(r * D + 8 * (p ^ CoreSmem<D>::ksw(r)));
    }
#pragma unroll
    for (int i = 0; i < kVUnits; ++i) {
      const int byte = (i * kWaves + wave) * 1024 + 16 * lane;
      const int d = byte / (2 * kBN), p = (byte % (2 * kBN)) / 16;
      const uint32_t col = 8 * (p ^ CoreSmem<D>::vsw(d));
      voff[i] = 2u * (static_cast<uint32_t>(d) * vstr + col);
    }
  }
  // kblk / vblk: wave-uniform block bases; lane offsets are 32-bit.
  __device__ void load_k(const bf16 *kblk, bf16 *kbuf) const {
    const char *base = reinterpret_cast<const char *>(kblk);
#pragma unroll
    for (int i = 0; i < kKUnits; ++i)
      __builtin_amdgcn_global_load_lds((gvoid_t *)(base + koff[i]),
                                       (lvoid_t *)(kbuf + (i * kWaves + wave) * 512), 16, 0, 0);
  }
  __device__ void load_v(const bf16 *vblk, bf16 *vbuf) const {
    const char *base = reinterpret_cast<const char *>(vblk);
#pragma unroll
    for (int i = 0; i < kVUnits; ++i)
      __builtin_amdgcn_global_load_lds((gvoid_t *)(base + voff[i]),
                                       (lvoid_t *)(vbuf + (i * kWaves + wave) * 512), 16, 0, 0);
  }
};

// Wait for this wave's direct loads, then the workgroup barrier.
__device__ __forceinline__ void loads_landed_barrier() {
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  __syncthreads();
}

typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

// Per-lane element offsets of the MFMA fragments in the swizzled buffers.
template <int D>
struct FragOffsets {
  int32_t k[D / 16];     // K row l32, head-dim chunk 2 st + hh  (+32 D per 32-key tile)
  static constexpr int kBN = CoreShape<D>::kBN, kKT = CoreShape<D>::kKT;
  int32_t v[kKT][2];     // V^T row l32, key chunk 4 kt + 2 u + hh (+32*kBN per 32-row tile)
  __device__ FragOffsets(int l32, int hh) {
    const int ks = CoreSmem<D>::ksw(l32), vs = CoreSmem<D>::vsw(l32);
#pragma unroll
    for (int st = 0; st < D / 16; ++st) k[st] = l32 * D + 8 * ((2 * st + hh) ^ ks);
#pragma unroll
    for (int kt = 0; kt < kKT; ++kt)
#pragma unroll
      for (int u = 0; u < 2; ++u) v[kt][u] = l32 * kBN + 8 * ((4 * kt + 2 * u + hh) ^ vs);
  }
};

// S^T[key][query] = K Q^T for one kBN-key block and NG groups of 32 queries:
// keys on the MFMA rows, so lane l owns query l%32 of each group and, in
// s[g][kt][v], key 32 kt + 8 (v/4) + 4 hh + v%4.  Each K fragment read from
// LDS feeds all NG groups.
// Tiles KT0 .. KT0+NKT-1 of the block; s[g][i] holds tile KT0 + i.
template <int D, int NG, int KT0 = 0, int NKT = CoreShape<D>::kKT>
__device__ __forceinline__ void qk_block(const bf16 *__restrict__ ks,
                                         const bf16x8 (&qf)[NG][D / 16], f32x16 (&s)[NG][NKT],
                                         const FragOffsets<D> &fo) {
#pragma unroll
  for (int i = 0; i < NKT; ++i) {
    constexpr int kt0 = KT0;
    const int kt = kt0 + i;
#pragma unroll
    for (int g = 0; g < NG; ++g) s[g][i] = f32x16{};
#pragma unroll
    for (int st = 0; st < D / 16; ++st) {
      const bf16x8 kf = *reinterpret_cast<const bf16x8 *>(ks + 32 * kt * D + fo.k[st]);
#pragma unroll
      for (int g = 0; g < NG; ++g) s[g][i] = mfma32(kf, qf[g][st], s[g][i]);
    }
  }
}

// Largest score of the block for this lane's query (both half-waves).
template <int kKT>
__device__ __forceinline__ float block_max(const f32x16 (&s)[kKT]) {
  float mx = s[0][0];
#pragma unroll
  for (int kt = 0; kt < kKT; ++kt)
#pragma unroll
    for (int v = 0; v < 16; v += 2) mx = fmaxf(mx, fmaxf(s[kt][v], s[kt][v + 1]));
  return fmaxf(mx, __shfl_xor(mx, 32));
}

// P = 2^(s - m) (SHIFT) or 2^s rounded to bf16 and packed as the B operands
// of O^T += V^T P^T; step (kt, u) holds keys 32 kt + 16 u + {4 hh + 0..3,
// 8 + 4 hh + 0..3} = s[kt][8u .. 8u+7].  Returns the sum of the bf16 values.
template <bool SHIFT, int kKT>
__device__ __forceinline__ float exp_pack(const f32x16 (&s)[kKT], float m, bf16x8 (&pf)[kKT][2]) {
  const bf16x2 ones = {static_cast<bf16>(1.0f), static_cast<bf16>(1.0f)};
  float lsum = 0.f;
#pragma unroll
  for (int kt = 0; kt < kKT; ++kt) {
#pragma unroll
    for (int v = 0; v < 16; v += 2) {
      const float p0 = __builtin_amdgcn_exp2f(SHIFT ? s[kt][v] - m : s[kt][v]);
      const float p1 = __builtin_amdgcn_exp2f(SHIFT ? s[kt][v + 1] - m : s[kt][v + 1]);
      const bf16x2 pp = {static_cast<bf16>(p0), static_cast<bf16>(p1)};
      pf[kt][v / 8][v % 8] = pp[0];
      pf[kt][v / 8][v % 8 + 1] = pp[1];
      lsum = __builtin_amdgcn_fdot2_f32_bf16(pp, ones, lsum, false);
    }
  }
  return lsum;
}

// O^T[d][query] += V^T P^T for NG groups.  The V^T chunk a lane reads holds
// exactly the keys of its P operand, in the same order (see vt_column), and
// feeds all NG groups.
// Tiles KT0 .. KT0+NKT-1 of the block; pf[g][i] holds tile KT0 + i.
template <int D, int NG, int KT0 = 0, int NKT = CoreShape<D>::kKT>
__device__ __forceinline__ void pv_block(const bf16 *__restrict__ vs,
                                         const bf16x8 (&pf)[NG][NKT][2],
                                         f32x16 (&o)[NG][D / 32], const FragOffsets<D> &fo) {
  constexpr int kBN = CoreShape<D>::kBN;
#pragma unroll
  for (int dt = 0; dt < D / 32; ++dt) {
#pragma unroll
    for (int i = 0; i < NKT; ++i) {
#pragma unroll
      for (int uu = 0; uu < 2; ++uu) {
        const bf16x8 vf = *reinterpret_cast<const bf16x8 *>(vs + 32 * dt * kBN + fo.v[KT0 + i][uu]);
#pragma unroll
        for (int g = 0; g < NG; ++g) o[g][dt] = mfma32(vf, pf[g][i][uu], o[g][dt]);
      }
    }
  }
}

// Keys >= kvalid among this lane's keys of a kBN-key block (8 i + 4 hh + 0..3).
template <int kBN>
__device__ __forceinline__ int padded_keys(int kvalid, int hh) {
  int n = 0;
#pragma unroll
  for (int i = 0; i < kBN / 8; ++i) n += min(max(8 * i + 4 * hh + 4 - kvalid, 0), 4);
  return n;
}

// Scores of keys >= kvalid (the zero rows padding a segment's last block)
// set to -inf, so they take no part in the block maximum and get p = 0.  The
// lane's score v of 32-key tile i belongs to key 32 i + 8 (v/4) + 4 hh + v%4.
template <int NG, int N>
__device__ __forceinline__ void mask_padded(f32x16 (&s)[NG][N], int kvalid, int hh) {
  const int kv = kvalid - 4 * hh;   // compared with compile-time key offsets
#pragma unroll
  for (int g = 0; g < NG; ++g)
#pragma unroll
    for (int i = 0; i < N; ++i)
#pragma unroll
      for (int v = 0; v < 16; ++v)
        s[g][i][v] = (32 * i + 8 * (v / 4) + v % 4 >= kv) ? -INFINITY : s[g][i][v];
}

// 1: S of block j+1 is computed while block j is exponentiated (two S sets);
// 0: each block's S is computed in its own step (one S set; with two query
// groups the second group's S overlaps the first group's exp).
// -1: 1 for 64-key blocks at head_dim 128 with one group, else 0 (measured:
// at head_dim 64 the second S set costs more occupancy than the overlap
// gains; with 128-key blocks it does not fit the registers).
#ifndef TDP_ATTN_PIPE
#define TDP_ATTN_PIPE (-1)
#endif
template <int D>
constexpr bool kPipeFor = TDP_ATTN_PIPE < 0 ? (D >= 128 && kNG == 1 && CoreShape<D>::kBN == 64)
                                            : TDP_ATTN_PIPE != 0;

// One workgroup = kWaves waves x kNG x 32 query rows of one (batch, head,
// tile) against all keys of the tile, then the audio keys; a 256-row unit of
// the padded row space is split over kUnit / kRowsWG workgroups.  SPLIT: each
// such query slot gets kv_splits workgroups, workgroup sp taking key blocks
// [nkb sp / S, nkb (sp + 1) / S) of the same sequence and leaving its
// unnormalized O and (m, l) for attn_combine_kernel; the rest is the same
// code (the unsplit instantiation compiles as if the split did not exist).
//
// Per kBN-key block j the wave (1) issues the direct loads of K(j+1) and
// V(j+1) into the LDS buffers of block j-1, (2) computes S(j) on MFMA, turns
// it into bf16 P on the VALU and accumulates O += V(j) P(j), and (3) waits for
// its loads and meets the others at the barrier.  With the pipeline (an
// option for 64-key blocks) step j instead loads K(j+2) and V(j+1) and
// computes S(j+1) while the VALU works on S(j); K is then staged one block
// ahead of V.  Either way two K and two V^T buffers suffice.  Head dim 128
// runs 128-key blocks in 8-wave workgroups (256 queries share each staged
// block, one workgroup per CU), head dim 64 runs 64-key blocks in 4-wave
// workgroups.
//
// Softmax: shift-free with a static per-query bound when it allows (below),
// else the exact online softmax for the whole workgroup.
//
// Keys past the end of a segment are the zero rows the QKV stage writes into
// the padding: score exactly 0, V row 0.  On the shift-free path each adds
// p = 1 to the row sum of the lane holding it, taken off again after the
// loop; when a lane's sum is then below 2^-6 of what was taken off (every
// real score of the query far below 0), that difference has lost precision
// and the workgroup runs the exact path instead.  The exact path masks them
// (score -inf, p = 0).
//
// Work items of one (batch, head) are contiguous: the units of every tile in
// tile order, then the audio query units of every tile.  Consecutive
// workgroup ids go to the 8 XCDs in turn; the id is remapped so each XCD
// walks a contiguous range of work items and the workgroups sharing a tile's
// K/V run together on one L2.
template <int D, bool SPLIT>
__global__ __launch_bounds__(64 * CoreShape<D>::kWaves, 8 / (CoreShape<D>::kWaves * kNG))
void attn_core_kernel(CoreArgs a) {
  constexpr int kBN = CoreShape<D>::kBN;
  constexpr int kKT = CoreShape<D>::kKT;
  constexpr int kCoreRowsWG = CoreShape<D>::kRowsWG;
  constexpr int kSubKT = CoreShape<D>::kSubKT;
  // Two K and two V^T buffers, as four separate arrays: a direct load into one
  // and fragment reads from another are then provably disjoint, so the
  // compiler does not make the reads wait for the loads.  Every buffer choice
  // below is a compile-time parity.
  __shared__ __attribute__((aligned(16))) bf16 sk0[kBN * D], sk1[kBN * D];
  __shared__ __attribute__((aligned(16))) bf16 sv0[D * kBN], sv1[D * kBN];
  auto kbuf = [&](auto par) -> bf16 * {
    if constexpr (decltype(par)::value) return sk1; else return sk0;
  };
  auto vbuf = [&](auto par) -> bf16 * {
    if constexpr (decltype(par)::value) return sv1; else return sv0;
  };
  using P0 = std::integral_constant<int, 0>;
  using P1 = std::integral_constant<int, 1>;
  constexpr int kSteps = D / 16;
  constexpr int kDT = D / 32;
  constexpr int NG = kNG;
  constexpr bool kPipe = kPipeFor<D>;
  constexpr int kSplit = kUnit / kCoreRowsWG;   // workgroups per 256-row unit

  const int64_t G = gridDim.x;
  const int64_t bid = blockIdx.x;
  int64_t lid = (bid % 8) * (G / 8) + bid / 8;   // gridDim.x is a multiple of 8
  int sp = 0;                                    // key split of the slot (SPLIT)
  if constexpr (SPLIT) {
    const int64_t slot = lid / a.kv_splits;
    sp = static_cast<int>(lid - slot * a.kv_splits);
    lid = slot;
  }
  if (lid >= a.total_units * kSplit) return;
  // (the same decode as core_slot, written out: the combine uses the helper)
  const int64_t item = lid / kSplit;
  const int part = static_cast<int>(lid - item * kSplit);
  const int64_t bh = item / a.units_per_bh;
  const int64_t u = item - bh * a.units_per_bh;
  const int64_t b = bh / a.heads;
  const int h = static_cast<int>(bh - b * a.heads);

  int32_t t, q0;
  bool audio_q;
  if (u < a.n_units) {
    t = a.blk_tile[u * (kUnit / kBlk)];
    if (t < 0) return;
    q0 = a.blk_q0[u * (kUnit / kBlk)];
    audio_q = false;
  } else {
    const int64_t ua = u - a.n_units;
    t = static_cast<int32_t>(ua / a.n_aqb);
    q0 = static_cast<int32_t>((ua - static_cast<int64_t>(t) * a.n_aqb) * kUnit);
    audio_q = true;
  }
  q0 += part * kCoreRowsWG;
  int64_t r0;
  int32_t len0;
  tile_rows(a.trb, t, a.n_rows, a.max_rows, &r0, &len0);
  const int64_t pad0 = static_cast<int64_t>(a.pad_begin[t]) * kBlk;
  len0 = static_cast<int32_t>(min(static_cast<int64_t>(len0),
                                  static_cast<int64_t>(a.pad_begin[t + 1]) * kBlk - pad0));
  const int32_t nq = audio_q ? (a.A - q0) : (len0 - q0);
  if (nq <= 0) return;

  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int l32 = lane & 31, hh = lane >> 5;

  // Q fragments (B operand of S^T = K Q^T): group g holds query row
  // wave*32*NG + 32 g + l32.
  const bf16 *qsrc = audio_q ? a.qa + ((bh * a.a_pad) + q0) * D
                             : a.q + ((bh * a.n_pad) + pad0 + q0) * D;
  bf16x8 qf[NG][kSteps];
#pragma unroll
  for (int g = 0; g < NG; ++g)
#pragma unroll
    for (int s = 0; s < kSteps; ++s)
      qf[g][s] = *reinterpret_cast<const bf16x8 *>(qsrc + (wave * 32 * NG + 32 * g + l32) * D +
                                                   16 * s + 8 * hh);

  // Segment 0: the tile's rows; segment 1: the audio rows.
  const bf16 *kseg0 = a.k + (bh * a.n_pad + pad0) * D;
  const bf16 *vseg0 = a.vt + bh * D * a.vt_cols + pad0;
  const bf16 *kseg1 = a.ka + bh * a.a_pad * D;
  const bf16 *vseg1 = a.vt + bh * D * a.vt_cols + a.n_pad;
  const int nkb0 = a.tile_keys ? static_cast<int>(ceil_div(len0, kBN)) : 0;
  const int nkb1 = static_cast<int>(ceil_div(a.A, kBN));
  const int nkb = nkb0 + nkb1;
  // Key blocks [jb, je) of this workgroup: all of them, or split part sp.
  int jb = 0, je = nkb;   // (the unsplit kernel uses 0 and nkb as written)
  if constexpr (SPLIT) {
    jb = static_cast<int>(static_cast<int64_t>(nkb) * sp / a.kv_splits);
    je = static_cast<int>(static_cast<int64_t>(nkb) * (sp + 1) / a.kv_splits);
    if (jb == je) {   // an empty part: l = 0 tells the combine to skip it
      const int64_t mrow = (lid * a.kv_splits + sp) * kCoreRowsWG;
      for (int r = threadIdx.x; r < min(nq, kCoreRowsWG); r += blockDim.x)
        a.ml[mrow + r] = make_float2(-INFINITY, 0.f);
      return;
    }
  }
  if (nkb == 0) return;
  // padded keys this lane holds in the last block of each segment
  // real keys in the last block of each segment, and the padded keys this
  // lane holds there
  const int kvalid0 = nkb0 > 0 ? len0 - (nkb0 - 1) * kBN : kBN;
  const int kvalid1 = nkb1 > 0 ? a.A - (nkb1 - 1) * kBN : kBN;
  const int nz0 = nkb0 > 0 ? padded_keys<kBN>(kvalid0, hh) : 0;
  const int nz1 = nkb1 > 0 ? padded_keys<kBN>(kvalid1, hh) : 0;

  const DirectStage<D> ds(__builtin_amdgcn_readfirstlane(wave), lane,
                          static_cast<uint32_t>(a.vt_cols));
  const FragOffsets<D> fo(l32, hh);
  // Block j (clamped to the last block of the range) of the tile-then-audio
  // key sequence, straight into an LDS buffer.
  auto load_k = [&](int j, bf16 *buf) __attribute__((always_inline)) {
    j = min(j, (SPLIT ? je : nkb) - 1);
    const bf16 *kb = j < nkb0 ? kseg0 + static_cast<int64_t>(j) * kBN * D
                              : kseg1 + static_cast<int64_t>(j - nkb0) * kBN * D;
    ds.load_k(kb, buf);
  };
  auto load_v = [&](int j, bf16 *buf) __attribute__((always_inline)) {
    j = min(j, (SPLIT ? je : nkb) - 1);
    const bool s0 = j < nkb0;
    ds.load_v(s0 ? vseg0 + j * kBN : vseg1 + (j - nkb0) * kBN, buf);
  };

  // Softmax without a running maximum.  Q carries log2(e)/sqrt(d), so a score
  // s = q.k is log2 of the unnormalized weight and, by Cauchy-Schwarz,
  // |s| <= U = |q| max|k| over the tile's and the audio keys (|q| from the
  // bf16 row in registers, max|k| from the QKV stage).  When U <= kNoShift
  // for every query of the workgroup, p = 2^s needs no shift: every p lies
  // in [2^-kNoShift, 2^kNoShift], normal in bf16 and fp32, the sums stay
  // finite, and the final division by l cancels the missing common factor.
  // Otherwise the workgroup runs the exact online softmax instead.
  constexpr float kNoShift = 64.f;
  bool need_exact = false;
  {
    const uint32_t *km = a.kmax2 + bh * (a.T + 1);
    float kk = nkb0 > 0 ? __uint_as_float(km[t]) : 0.f;
    if (nkb1 > 0) kk = fmaxf(kk, __uint_as_float(km[a.T]));
#pragma unroll
    for (int g = 0; g < NG; ++g) {
      float qq = 0.f;
#pragma unroll
      for (int st = 0; st < kSteps; ++st)
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const float x = static_cast<float>(qf[g][st][e]);
          qq = fmaf(x, x, qq);
        }
      qq += __shfl_xor(qq, 32);
      const float u = sqrtf(qq) * sqrtf(kk) * 1.0009765625f;
      need_exact = need_exact || !(u <= kNoShift);   // NaN included
    }
  }

  f32x16 o[NG][kDT];
  float m_run[NG], l_run[NG];
  f32x16 sa[NG][kKT], sb[NG][kKT];   // S of two consecutive blocks (sb unused without kPipe)

  // K(0), V(0), K(1) into LDS; S(0), then a barrier so that no wave's load of
  // K(2) into k[0] overtakes another wave's reads of K(0).  The caller has
  // passed a barrier since any earlier reads of these buffers.
  auto prologue = [&]() __attribute__((always_inline)) {
#pragma unroll
    for (int g = 0; g < NG; ++g) {
#pragma unroll
      for (int i = 0; i < kDT; ++i) o[g][i] = f32x16{};
      l_run[g] = 0.f;
    }
    load_k(SPLIT ? jb : 0, sk0);
    load_v(SPLIT ? jb : 0, sv0);
    if constexpr (kPipe) load_k(SPLIT ? jb + 1 : 1, sk1);
    loads_landed_barrier();
    if constexpr (kPipe) {
      qk_block<D, NG>(sk0, qf, sa, fo);
      // Step 0 loads K(2) into k[0]: every wave must have read K(0) first.
      __syncthreads();
    }
  };

  // Softmax of one part of a block (N 32-key tiles, scores sc) into bf16 P.
  // EXACT = false: p = 2^s (see above).  EXACT = true: the exact online
  // softmax with a lazily moved maximum (moved only when a part's max exceeds
  // it by more than kLazy, so p <= 2^kLazy; the O rescale is rare and sits on
  // a real branch).  kvalid: keys of the part below this index are real, the
  // rest are zero padding (score 0), which the exact path masks here (p = 0);
  // the shift-free path takes p = 1 per padded key off after the loop.
  auto soft = [&](auto exact_tag, auto &sc, auto &pf, int kvalid) __attribute__((always_inline)) {
    constexpr bool kExact = decltype(exact_tag)::value;
    constexpr int N = sizeof(sc[0]) / sizeof(f32x16);
    if constexpr (kExact) {
      if (kvalid < 32 * N) mask_padded<NG, N>(sc, kvalid, hh);
      float mb[NG];
      bool grow = false;
#pragma unroll
      for (int g = 0; g < NG; ++g) {
        mb[g] = block_max<N>(sc[g]);
        grow = grow || (mb[g] > m_run[g] + kLazy);
      }
      if (__builtin_expect(__ballot(grow) != 0, 0)) {
        // Rare after the first block; the empty asm keeps this a real branch.
        asm volatile("" ::: "memory");
#pragma unroll
        for (int g = 0; g < NG; ++g) {
          const float m_new = fmaxf(m_run[g], mb[g]);
          const float alpha = __builtin_amdgcn_exp2f(m_run[g] - m_new);
#pragma unroll
          for (int i = 0; i < kDT; ++i)
#pragma unroll
            for (int v = 0; v < 16; ++v) o[g][i][v] *= alpha;
          l_run[g] *= alpha;
          m_run[g] = m_new;
        }
      }
    }
#pragma unroll
    for (int g = 0; g < NG; ++g) {
      // (m_run is finite here: part 0 of every block holds the block's first
      // key, which is real; the guard keeps -inf - -inf out regardless)
      const float m = kExact ? (m_run[g] == -INFINITY ? 0.f : m_run[g]) : 0.f;
      l_run[g] += exp_pack<kExact, N>(sc[g], m, pf[g]);
    }
  };

  // One kBN-key block j.  Without the pipeline it loads K(j+1) and V(j+1)
  // into the buffers of block j-1, then works through the block in parts of
  // kSubKT tiles (QK, softmax, PV per part).  With the pipeline
  // (64-key blocks) K(j) and V(j-1) were consumed in block j-1, so their
  // buffers take K(j+2) and V(j+1), and S(j+1) is computed while block j is
  // exponentiated.  Loads run unconditionally so they share one basic block
  // with the exp; past the last block they re-read in-range data and the
  // results are dropped.  PAR = j % 2.
  auto step = [&](auto exact_tag, auto upper, auto par, int j, f32x16 (&scur)[NG][kKT],
                  f32x16 (&snext)[NG][kKT]) __attribute__((always_inline)) {
    constexpr int kPK = decltype(upper)::value ? CoreShape<D>::kSubKTHi : kSubKT;
    constexpr int kPar = decltype(par)::value;
    const std::integral_constant<int, kPar> cur{};
    const std::integral_constant<int, 1 - kPar> oth{};
    // real keys of this block (the last block of each segment is padded)
    const int kvalid = (j == nkb0 - 1) ? kvalid0 : ((j == nkb - 1 && nkb1 > 0) ? kvalid1 : kBN);
    if constexpr (!kPipe) {
      load_k(j + 1, kbuf(oth));
      load_v(j + 1, vbuf(oth));
      auto part = [&](auto part_tag) __attribute__((always_inline)) {
        constexpr int kT0 = decltype(part_tag)::value * kPK;
        f32x16 sp[NG][kPK];
        qk_block<D, NG, kT0, kPK>(kbuf(cur), qf, sp, fo);
        bf16x8 pf[NG][kPK][2];
        soft(exact_tag, sp, pf, kvalid - 32 * kT0);
        pv_block<D, NG, kT0, kPK>(vbuf(cur), pf, o, fo);
      };
      part(std::integral_constant<int, 0>{});
      if constexpr (kKT / kPK > 1) part(std::integral_constant<int, 1>{});
      if constexpr (kKT / kPK > 2) part(std::integral_constant<int, 2>{});
      if constexpr (kKT / kPK > 3) part(std::integral_constant<int, 3>{});
    } else {
      load_k(j + 2, kbuf(cur));
      load_v(j + 1, vbuf(oth));
      qk_block<D, NG>(kbuf(oth), qf, snext, fo);
      bf16x8 pf[NG][kKT][2];
      soft(exact_tag, scur, pf, kvalid);
      pv_block<D, NG>(vbuf(cur), pf, o, fo);
    }
    loads_landed_barrier();
  };

  auto run_half = [&](auto exact_tag, auto upper) __attribute__((always_inline)) {
    prologue();
    const int jend = SPLIT ? je : nkb;
    for (int j = SPLIT ? jb : 0; j < jend; j += 2) {
      if constexpr (kPipe) {
        step(exact_tag, upper, P0{}, j, sa, sb);
        if (j + 1 < jend) step(exact_tag, upper, P1{}, j + 1, sb, sa);
      } else {
        step(exact_tag, upper, P0{}, j, sa, sa);
        if (j + 1 < jend) step(exact_tag, upper, P1{}, j + 1, sa, sa);
      }
    }
  };
  // The upper half of the waves runs its own copy of the loop (different
  // part size); both copies pass the same barriers.
  const bool upper_half = __builtin_amdgcn_readfirstlane(wave) >= CoreShape<D>::kWaves / 2;
  auto run = [&](auto exact_tag) __attribute__((always_inline)) {
    if (CoreShape<D>::kSubKTHi != kSubKT && !kPipe && upper_half)
      run_half(exact_tag, std::true_type{});
    else
      run_half(exact_tag, std::false_type{});
  };
  float l_tot[NG];
  bool exact = __syncthreads_or(need_exact);
  if (!exact) {
    run(std::false_type{});
    // l >= 2^-kNoShift here unless the inputs hold Inf or NaN, or every real
    // score of a query lies so far below 0 that taking the padded keys'
    // weight off cancelled (a lane's sum under 2^-6 of that weight: its
    // rounding error may then exceed 2^-11 of the result); such workgroups
    // take the exact path, which masks the padded keys.
    bool bad = false;
    // padded keys of the segments whose last block lies in [jb, je)
    const float pad_ones = SPLIT ? static_cast<float>((jb < nkb0 && nkb0 <= je ? nz0 : 0) +
                                                      (je == nkb ? nz1 : 0))
                                 : static_cast<float>(nz0 + nz1);
#pragma unroll
    for (int g = 0; g < NG; ++g) {
      l_run[g] -= pad_ones;
      bad = bad || !(l_run[g] >= 0x1p-6f * pad_ones);
      l_tot[g] = l_run[g] + __shfl_xor(l_run[g], 32);
      bad = bad || !(l_tot[g] >= 0x1p-90f);
    }
    exact = __syncthreads_or(bad);
  }
  if (exact) {
#pragma unroll
    for (int g = 0; g < NG; ++g) m_run[g] = -INFINITY;
    run(std::true_type{});
#pragma unroll
    for (int g = 0; g < NG; ++g) l_tot[g] = l_run[g] + __shfl_xor(l_run[g], 32);
  }

  if constexpr (SPLIT) {
    // The part's unnormalized O (fp32) and its (m, l): O_true = 2^m O.
#pragma unroll
    for (int g = 0; g < NG; ++g) {
      const int row = wave * 32 * NG + 32 * g + l32;
      if (row < nq) {
        const int64_t prow = (lid * a.kv_splits + sp) * kCoreRowsWG + row;
        float *dst = a.op + prow * D + 4 * hh;
#pragma unroll
        for (int dt = 0; dt < kDT; ++dt)
#pragma unroll
          for (int gg = 0; gg < 4; ++gg)
            *reinterpret_cast<float4 *>(dst + 32 * dt + 8 * gg) =
                make_float4(o[g][dt][4 * gg + 0], o[g][dt][4 * gg + 1], o[g][dt][4 * gg + 2],
                            o[g][dt][4 * gg + 3]);
        if (hh == 0) a.ml[prow] = make_float2(exact ? m_run[g] : 0.f, l_tot[g]);
      }
    }
    return;
  }
#pragma unroll
  for (int g = 0; g < NG; ++g) {
    const float inv = 1.0f / l_tot[g];
    const int row = wave * 32 * NG + 32 * g + l32;
    if (row < nq) {
      bf16 *dst = audio_q
          ? a.oa + (((static_cast<int64_t>(t) * a.batch + b) * a.heads + h) * a.A + q0 + row) * D
          : a.o + ((b * a.heads + h) * a.n_rows + r0 + q0 + row) * D;
      dst += 4 * hh;
#pragma unroll
      for (int dt = 0; dt < kDT; ++dt) {
#pragma unroll
        for (int gg = 0; gg < 4; ++gg) {
          bf16x4 v4;
          v4[0] = static_cast<bf16>(o[g][dt][4 * gg + 0] * inv);
          v4[1] = static_cast<bf16>(o[g][dt][4 * gg + 1] * inv);
          v4[2] = static_cast<bf16>(o[g][dt][4 * gg + 2] * inv);
          v4[3] = static_cast<bf16>(o[g][dt][4 * gg + 3] * inv);
          *reinterpret_cast<bf16x4 *>(dst + 32 * dt + 8 * gg) = v4;
        }
      }
    }
  }
}


// ---------------------------------------------------------------------------
// core, two query groups per wave (head dim 64 and 128, unsplit launches)
// ---------------------------------------------------------------------------
//
// 4 waves x 64 queries (two groups of 32 per wave) = 256 queries of one
// (batch, head, tile) per workgroup, 128-key blocks; at head dim 128 one
// workgroup per CU and so one wave per SIMD (two at head dim 64).  Each K or V^T fragment a wave reads from LDS feeds
// the MFMAs of both its query groups: half the LDS reads per MFMA of the
// 8-wave form, whose 1 KB per MFMA (plus the K/V staging) would exceed the
// CU's LDS bandwidth before the MFMA rate is reached.
//
// With one wave per SIMD nothing else covers latency, so the block loop is a
// software pipeline over 32-key tiles tau in a fixed instruction order (a
// scheduling fence after each MFMA and its companions; within a step the
// MFMA issues first, then its LDS reads, then the rest).  Iteration tau:
//   phase 1: 16 MFMAs of O += V(tau-1) P(tau-1), with the reads of the K
//            fragments of tile tau+1 and the exponentials of group 0 of S(tau)
//   phase 2: 16 MFMAs of S(tau+1) = K(tau+1) Q^T, with the reads of the V
//            fragments of tile tau+1 and the exponentials of group 1 of S(tau)
// Fragments of a block are read in iterations 4j-1 .. 4j+2; at the start of
// iteration 4j+3 every wave waits for its share of block j+1's direct loads
// (issued one block earlier) and meets the others at the one barrier of the
// block, after which block j's buffers take block j+2.  The direct loads are
// buffer_load ... lds in inline assembly: the compiler does not track them,
// so its waits for fragment reads stay exact.
//
// Softmax: the shift-free form of attn_core_kernel when the Cauchy-Schwarz
// bound allows it; otherwise (and when taking the padded keys' weight off
// cancelled) a plain exact online softmax, tile by tile, without the
// pipeline.
typedef int i32x4 __attribute__((ext_vector_type(4)));

// Buffer descriptor of `bytes` bytes at `base` (wave-uniform): raw, stride 0.
__device__ __forceinline__ i32x4 buf_rsrc(const void *base, uint32_t bytes) {
  const uint64_t p = reinterpret_cast<uint64_t>(base);
  i32x4 r;
  r[0] = __builtin_amdgcn_readfirstlane(static_cast<int>(p & 0xffffffffu));
  r[1] = __builtin_amdgcn_readfirstlane(static_cast<int>((p >> 32) & 0xffffu));
  r[2] = __builtin_amdgcn_readfirstlane(static_cast<int>(bytes));
  r[3] = 0x00020000;
  return r;
}

__device__ __forceinline__ uint32_t lds_addr(const bf16 *p) {
  return static_cast<uint32_t>(
      reinterpret_cast<uintptr_t>((__attribute__((address_space(3))) const bf16 *)p));
}

// 16 bytes per lane at descriptor offset voff + soff (soff wave-uniform)
// into LDS: the wave's 64 lanes fill the 1 KB at LDS byte address m0
// (wave-uniform) in lane order.
__device__ __forceinline__ void lds_load16(i32x4 rsrc, uint32_t voff, uint32_t soff,
                                           uint32_t m0) {
  asm volatile("buffer_load_dwordx4 %0, %1, %2 offen lds"
               :
               : "v"(voff), "s"(rsrc), "s"(soff), "{m0}"(m0)
               : "memory");
}

#ifndef TDP_ATTN_NG2
#define TDP_ATTN_NG2 1
#endif
#define TDP_NG2_FENCE() __builtin_amdgcn_sched_barrier(0)
// Within each MFMA step of the key loop the MFMA issues first, then the
// step's LDS reads, then its other companions (accumulator reads,
// exponentials, packs, loads), in the matrix pipe's shadow.  Left to itself
// the scheduler sometimes puts a step's accumulator reads ahead of its
// MFMA, and the loop then takes about 2% more cycles.
#ifndef TDP_ATTN_PIN
#define TDP_ATTN_PIN 1
#endif
#if TDP_ATTN_PIN
#define TDP_NG2_MFMA_FIRST()                                                       \
  do {                                                                             \
    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);   /* MFMA */                 \
    __builtin_amdgcn_sched_group_barrier(0x100, 8, 0);   /* LDS reads */            \
    __builtin_amdgcn_sched_group_barrier(0x616, 256, 0); /* VALU SALU VMEM LDS-write trans */ \
  } while (0)
#else
#define TDP_NG2_MFMA_FIRST() \
  do {                       \
  } while (0)
#endif

// Fragment offsets of the two-group core (128-key blocks at either head
// dim): K row l32, head-dim chunk 2 st + hh, in CoreSmem's K swizzle; V^T
// row l32 of a 32-row group, key chunk 4 kt + 2 u + hh, rows of 128 keys
// swizzled by row % 16.
template <int D>
struct Frag2 {
  int32_t k[D / 16];
  int32_t v[4][2];
  __device__ Frag2(int l32, int hh) {
    const int ks = CoreSmem<D>::ksw(l32), vs = l32 % 16;
#pragma unroll
    for (int st = 0; st < D / 16; ++st) k[st] = l32 * D + 8 * ((2 * st + hh) ^ ks);
#pragma unroll
    for (int kt = 0; kt < 4; ++kt)
#pragma unroll
      for (int u = 0; u < 2; ++u) v[kt][u] = l32 * 128 + 8 * ((4 * kt + 2 * u + hh) ^ vs);
  }
};

// Head dim 128: one workgroup (and so one wave) per SIMD.  Head dim 64 needs
// half the registers and runs two workgroups per CU.
template <int D>
__global__ __launch_bounds__(256, D == 128 ? 1 : 2) void attn_core2_kernel(CoreArgs a) {
  static_assert(D == 128 || D == 64, "the two-group core is built for head dim 64 or 128");
  constexpr int kBN = 128, kKT = kBN / 32, kW = 4;
  constexpr int kSteps = D / 16, kDT = D / 32;
  constexpr int kLoads = kBN * D * 2 / 1024 / kW;       // 1 KB loads per wave, K or V^T block
  // MFMAs per phase of a 32-key tile: O += V P (phase 1), S = K Q^T (phase 2);
  // each phase also takes the 16 softmax steps of one group, kR1 / kR2 per MFMA
  constexpr int kP1 = 4 * kDT, kP2 = 2 * kSteps;
  constexpr int kR1 = 16 / kP1, kR2 = 16 / kP2;
  static_assert(kLoads == D / 16 && 2 * kLoads == kP2, "one direct load per phase-2 MFMA");
  // One LDS array: K buffers 0 and 1, then V^T buffers 0 and 1.  Fragment
  // reads address it as a per-lane byte offset plus a compile-time constant,
  // which the LDS read carries in its immediate offset field.
  __shared__ __attribute__((aligned(16))) bf16 smem[4 * kBN * D];
  constexpr int kBufEl = kBN * D;
  auto kbuf = [&](auto par) -> bf16 * { return smem + decltype(par)::value * kBufEl; };
  auto vbuf = [&](auto par) -> bf16 * { return smem + (2 + decltype(par)::value) * kBufEl; };
  bf16 *const sk0 = smem, *const sk1 = smem + kBufEl;
  bf16 *const sv0 = smem + 2 * kBufEl, *const sv1 = smem + 3 * kBufEl;
  (void)sv1;
  using P0 = std::integral_constant<int, 0>;
  using P1 = std::integral_constant<int, 1>;

  // One 256-row unit per workgroup.  Workgroup i runs on XCD i % 8, and XCD
  // x's first per_xcd workgroups take units x per_xcd, x per_xcd + 1, ... in
  // order, so the units of one (tile, head) share that XCD's L2.  Units from
  // 8 per_xcd on form a shared tail: every later workgroup claims the next
  // one from a counter, so the XCDs that run faster (their shader clocks
  // differ under load) take more of it, and claims past the last unit end
  // at once.  Each of the pool_claims tail workgroups claims exactly once;
  // the launch's last claim puts the counter back to zero for the next
  // launch (the prepare stage zeroes it first).
  const int64_t bid = blockIdx.x;
  const int64_t xcd = bid % 8, kx = bid / 8;
  int64_t lid;
  if (kx < a.per_xcd) {
    lid = xcd * a.per_xcd + kx;
  } else {
    __shared__ uint32_t ticket;
    if (threadIdx.x == 0) {
      const uint32_t tk = atomicAdd(a.pool_ctr, 1u);
      if (tk == a.pool_claims - 1u) atomicExch(a.pool_ctr, 0u);
      ticket = tk;
    }
    __syncthreads();
    lid = 8 * a.per_xcd + static_cast<int64_t>(ticket);
  }
  if (lid >= a.total_units) return;
  const int64_t bh = lid / a.units_per_bh;
  const int64_t u = lid - bh * a.units_per_bh;
  const int64_t b = bh / a.heads;
  const int h = static_cast<int>(bh - b * a.heads);
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int l32 = lane & 31, hh = lane >> 5;
  const int uwave = __builtin_amdgcn_readfirstlane(wave);

  // Q fragments first, before the unit's table lookups: group g holds query
  // row 64 wave + 32 g + l32.  A tile unit's rows start at row 256 u of the
  // (batch, head)'s padded slab (each tile takes whole 256-row units there);
  // an audio unit's at row 256 (u - units) % (audio units per tile).  Rows
  // of an empty unit (past the last tile) are in the slab and never used.
  bf16x8 qf[2][kSteps];
  {
    const bool tile_unit = u < a.n_units;
    const int64_t ua = u - a.n_units;
    const bf16 *qsrc = tile_unit ? a.q + (bh * a.n_pad + u * kUnit) * D
                                 : a.qa + (bh * a.a_pad + (ua % max(a.n_aqb, 1)) * kUnit) * D;
#pragma unroll
    for (int g = 0; g < 2; ++g)
#pragma unroll
      for (int st = 0; st < kSteps; ++st)
        qf[g][st] = *reinterpret_cast<const bf16x8 *>(qsrc + (64 * wave + 32 * g + l32) * D +
                                                      16 * st + 8 * hh);
  }
  int32_t t, q0;
  bool audio_q;
  if (u < a.n_units) {
    t = a.blk_tile[u * (kUnit / kBlk)];
    if (t < 0) return;
    q0 = a.blk_q0[u * (kUnit / kBlk)];
    audio_q = false;
  } else {
    const int64_t ua = u - a.n_units;
    t = static_cast<int32_t>(ua / a.n_aqb);
    q0 = static_cast<int32_t>((ua - static_cast<int64_t>(t) * a.n_aqb) * kUnit);
    audio_q = true;
  }
  int64_t r0;
  int32_t len0;
  tile_rows(a.trb, t, a.n_rows, a.max_rows, &r0, &len0);
  const int64_t pad0 = static_cast<int64_t>(a.pad_begin[t]) * kBlk;
  len0 = static_cast<int32_t>(min(static_cast<int64_t>(len0),
                                  static_cast<int64_t>(a.pad_begin[t + 1]) * kBlk - pad0));
  const int32_t nq = audio_q ? (a.A - q0) : (len0 - q0);
  if (nq <= 0) return;


  // key blocks: the tile's rows (segment 0), then the audio rows (segment 1)
  const int nkb0 = a.tile_keys ? static_cast<int>(ceil_div(len0, kBN)) : 0;
  const int nkb1 = static_cast<int>(ceil_div(a.A, kBN));
  const int nkb = nkb0 + nkb1;
  if (nkb == 0) return;
  const int kvalid0 = nkb0 > 0 ? len0 - (nkb0 - 1) * kBN : kBN;
  const int kvalid1 = nkb1 > 0 ? a.A - (nkb1 - 1) * kBN : kBN;
  const int nz = (nkb0 > 0 ? padded_keys<kBN>(kvalid0, hh) : 0) +
                 (nkb1 > 0 ? padded_keys<kBN>(kvalid1, hh) : 0);

  // Per-lane byte offsets of the direct loads: 1 KB unit i * 4 + wave of a
  // block, in the swizzled layouts (K rows of D in CoreSmem's swizzle, V^T
  // rows of 128 keys swizzled by row % 16, read from the slab's vt_cols
  // columns).  A K unit holds kKR rows, kKR (4 i + wave) + lane / kCPR; a V^T
  // unit 4 rows, 16 i + 4 wave + lane / 16.  Neither swizzle key depends on
  // i, so unit i's offset is unit 0's plus a wave-uniform step: 4 KB of K,
  // 16 V^T rows.
  constexpr int kCPR = D / 8, kKR = 64 / kCPR;
  static_assert(CoreSmem<D>::kCPR == kCPR, "16-byte chunks per K row");
  uint32_t koff0, voff0;
  {
    const int r = kKR * uwave + lane / kCPR, p = lane % kCPR;
    koff0 = 2u * static_cast<uint32_t>(r * D + 8 * (p ^ CoreSmem<D>::ksw(r)));
    const int vr = 4 * uwave + lane / 16, vp = lane % 16;
    voff0 = 2u * (static_cast<uint32_t>(vr) * static_cast<uint32_t>(a.vt_cols) +
                  static_cast<uint32_t>(8 * (vp ^ (vr % 16))));
  }
  const uint32_t vstep = 2u * 16u * static_cast<uint32_t>(a.vt_cols);   // bytes per 16 V^T rows
  const bf16 *kslab0 = a.k + (bh * a.n_pad + pad0) * D;
  const bf16 *kslab1 = a.ka + bh * a.a_pad * D;
  const bf16 *vslab = a.vt + bh * D * a.vt_cols;
  const uint32_t kbytes = kBN * D * 2;
  const uint32_t vbytes = static_cast<uint32_t>(((D - 1) * a.vt_cols + kBN) * 2);
  // Block j straight into LDS: kLoads of K, then kLoads of V^T; load i < 8
  // is of K, 8..15 of V^T.  Past the last block the descriptors hold no
  // bytes: those loads touch no memory and write zeros that are never read
  // (the unit's last wait then does not wait on memory).
  auto block_rsrc = [&](int j, i32x4 &kr, i32x4 &vr) __attribute__((always_inline)) {
    const bool live = j < nkb;
    j = min(j, nkb - 1);
    const bool s0 = j < nkb0;
    kr = buf_rsrc(s0 ? kslab0 + static_cast<int64_t>(j) * kBN * D
                     : kslab1 + static_cast<int64_t>(j - nkb0) * kBN * D, live ? kbytes : 0u);
    vr = buf_rsrc(vslab + (s0 ? pad0 + static_cast<int64_t>(j) * kBN
                              : a.n_pad + static_cast<int64_t>(j - nkb0) * kBN), live ? vbytes : 0u);
  };
  // The LDS destination of load i is the buffer's address + i * 4 KB + wb,
  // wb = the wave's 1 KB slot, taken afresh (through an opaque copy) for
  // every block: each destination is then one scalar add at its load
  // instead of one of 32 registers held through the whole loop.
  auto wave_slot = [&]() __attribute__((always_inline)) {
    uint32_t wb = static_cast<uint32_t>(uwave) * 1024u;
    asm volatile("" : "+s"(wb));
    return wb;
  };
  auto load_one = [&](int i, const i32x4 &kr, const i32x4 &vr, bf16 *kb, bf16 *vb, uint32_t wb)
      __attribute__((always_inline)) {
    if (i < kLoads)
      lds_load16(kr, koff0, static_cast<uint32_t>(i) * 4096u,
                 lds_addr(kb) + static_cast<uint32_t>(i * kW) * 1024u + wb);
    else
      lds_load16(vr, voff0, static_cast<uint32_t>(i - kLoads) * vstep,
                 lds_addr(vb) + static_cast<uint32_t>((i - kLoads) * kW) * 1024u + wb);
  };
  auto load_block = [&](int j, bf16 *kb, bf16 *vb) __attribute__((always_inline)) {
    i32x4 kr, vr;
    block_rsrc(j, kr, vr);
    const uint32_t wb = wave_slot();
#pragma unroll
    for (int i = 0; i < 2 * kLoads; ++i) load_one(i, kr, vr, kb, vb, wb);
  };

  // Blocks 0 and 1 go out before the Q-dependent check below, so their
  // latency overlaps that of the Q loads.  (The exact path reloads block 0
  // after waiting for every load: same data, same place.)
  load_block(0, sk0, sv0);
  load_block(1, sk1, sv1);

  // Cauchy-Schwarz bound of the shift-free softmax (see attn_core_kernel).
  constexpr float kNoShift = 64.f;
  bool need_exact = false;
  {
    const uint32_t *km = a.kmax2 + bh * (a.T + 1);
    float kk = nkb0 > 0 ? __uint_as_float(km[t]) : 0.f;
    if (nkb1 > 0) kk = fmaxf(kk, __uint_as_float(km[a.T]));
#pragma unroll
    for (int g = 0; g < 2; ++g) {
      float qq = 0.f;
#pragma unroll
      for (int st = 0; st < kSteps; ++st)
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const float x = static_cast<float>(qf[g][st][e]);
          qq = fmaf(x, x, qq);
        }
      qq += __shfl_xor(qq, 32);
      const float ub = sqrtf(qq) * sqrtf(kk) * 1.0009765625f;
      need_exact = need_exact || !(ub <= kNoShift);
    }
  }
  bool exact = __syncthreads_or(need_exact);

  // (at head dim 128 FragOffsets<128> holds the same offsets; it stays there,
  // as the register allocation of this kernel is sensitive to its form)
  using Frags = std::conditional_t<D == 128, FragOffsets<D>, Frag2<D>>;
  // The V^T offsets carry the V^T buffers' base (64 KB into the LDS array),
  // so that what a fragment read adds to them, at most 56 KB, fits the LDS
  // read's 16-bit immediate offset.
  Frags fo(l32, hh);
#pragma unroll
  for (int kt = 0; kt < kKT; ++kt)
#pragma unroll
    for (int x = 0; x < 2; ++x) {
      fo.v[kt][x] += 2 * kBufEl;
      asm volatile("" : "+v"(fo.v[kt][x]));   // (kept out of the constant folding)
    }
  f32x16 o[2][kDT];
  float l_tot[2];
  const bf16x2 ones = {static_cast<bf16>(1.0f), static_cast<bf16>(1.0f)};

  if (!exact) {
#pragma unroll
    for (int g = 0; g < 2; ++g)
#pragma unroll
      for (int i = 0; i < kDT; ++i) o[g][i] = f32x16{};
    f32x16 sc[2][2];        // [parity of the tile][group] scores
    bf16x8 pf[2][2][2];     // [parity][group][16-key half] bf16 P
    bf16x8 kf[kSteps];      // K fragments of the next tile (a few live at a time)
    bf16x8 vf[kDT][2];      // V^T fragments [32-row group of d][16-key half]
    // Row sums: at head dim 128 two fp32 partial sums of the exponentials per
    // group (the bf16 dot instruction co-issues worse with the MFMAs); at 64,
    // where registers are short, one dot2 over the packed pair.
    float lsum[2] = {0.f, 0.f}, lsum2[2] = {0.f, 0.f};
    float e0 = 0.f, e1 = 0.f;
    // P and V^T of "tile -1" are zero: the first PV step adds nothing.
#pragma unroll
    for (int g = 0; g < 2; ++g)
#pragma unroll
      for (int x = 0; x < 2; ++x) pf[1][g][x] = bf16x8{};
#pragma unroll
    for (int i = 0; i < kDT; ++i) vf[i][0] = vf[i][1] = bf16x8{};

    // wait for block 0 (block 1's loads may stay in flight); S(0) from tile
    // 0's K fragments
    if constexpr (2 * kLoads == 16) asm volatile("s_waitcnt vmcnt(16)" ::: "memory");
    else asm volatile("s_waitcnt vmcnt(8)" ::: "memory");
    lds_barrier();
#pragma unroll
    for (int st = 0; st < kSteps; ++st) {
      const bf16x8 k8 = *reinterpret_cast<const bf16x8 *>(sk0 + fo.k[st]);
      sc[0][0] = mfma32(k8, qf[0][st], st == 0 ? f32x16{} : sc[0][0]);
      sc[0][1] = mfma32(k8, qf[1][st], st == 0 ? f32x16{} : sc[0][1]);
    }

    // Softmax step q (0..15) of group g of S(tau): even q exponentiates
    // scores q, q+1; odd q packs them into P and adds them to the row sum.
    auto soft_step = [&](auto pc_tag, int g, int q) __attribute__((always_inline)) {
      constexpr int PC = decltype(pc_tag)::value;
      if (q % 2 == 0) {
        e0 = __builtin_amdgcn_exp2f(sc[PC][g][q]);
        e1 = __builtin_amdgcn_exp2f(sc[PC][g][q + 1]);
      } else {
        const int v = q - 1;
        const bf16x2 pp = {static_cast<bf16>(e0), static_cast<bf16>(e1)};
        pf[PC][g][v / 8][v % 8] = pp[0];
        pf[PC][g][v / 8][v % 8 + 1] = pp[1];
        if constexpr (D == 128) {
          lsum[g] += e0;
          lsum2[g] += e1;
        } else {
          lsum[g] = __builtin_amdgcn_fdot2_f32_bf16(pp, ones, lsum[g], false);
        }
      }
    };
    constexpr int kLead = kSteps == 8 ? 3 : 2;   // K fragment reads run this many k steps ahead

    // Iteration on tile tau = 4 j + T of block j (buffers of parity BP):
    //  phase 1: O += V(tau-1) P(tau-1), each V^T fragment refilled with
    //           tile tau's right after its last use; group 0 of P(tau);
    //  [T = 3: wait for block j+1, barrier, block j+2's loads go out]
    //  phase 2: S(tau+1) = K(tau+1) Q^T, K fragments read kLead steps
    //           ahead; group 1 of P(tau).
    auto iter = [&](auto t_tag, auto bp_tag, int j) __attribute__((always_inline)) {
      constexpr int T = decltype(t_tag)::value;
      constexpr int BP = decltype(bp_tag)::value;
      constexpr int PC = T % 2, PN = 1 - PC;          // parity of tau, of tau +- 1
      constexpr int TN = (T + 1) % kKT;               // tile index of tau + 1 in its block
      constexpr int NBP = T == kKT - 1 ? 1 - BP : BP; // its buffers
      const std::integral_constant<int, PC> pc{};
      const bf16 *kn = kbuf(std::integral_constant<int, NBP>{});
#pragma unroll
      for (int q = 0; q < kP1; ++q) {
        const int dt = q / 4, x = (q / 2) % 2, g = q % 2;
        o[g][dt] = mfma32(vf[dt][x], pf[PN][g][x], o[g][dt]);
        if (g == 1)   // both groups have read vf[dt][x]: tile tau's goes in
          vf[dt][x] = *reinterpret_cast<const bf16x8 *>(smem + (BP * kBufEl + 32 * dt * kBN) +
                                                        fo.v[T][x]);
#pragma unroll
        for (int r = 0; r < kR1; ++r) soft_step(pc, 0, kR1 * q + r);
        if constexpr (T != kKT - 1) {
          if (q >= kP1 - 2 * kLead && q % 2 == 0)
            kf[(q - (kP1 - 2 * kLead)) / 2] =
                *reinterpret_cast<const bf16x8 *>(kn + 32 * TN * D + fo.k[(q - (kP1 - 2 * kLead)) / 2]);
        }
        TDP_NG2_MFMA_FIRST();
        TDP_NG2_FENCE();
      }
      i32x4 kr, vr;
      uint32_t wb = 0;
      if constexpr (T == kKT - 1) {
        // block j + 1 landed (this wave's loads, then everyone's); every wave
        // is past its reads of block j, whose buffers now take block j + 2
        asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
        lds_barrier();
        block_rsrc(j + 2, kr, vr);
        wb = wave_slot();
#pragma unroll
        for (int st = 0; st < kLead; ++st)
          kf[st] = *reinterpret_cast<const bf16x8 *>(kn + 32 * TN * D + fo.k[st]);
        TDP_NG2_FENCE();
      }
#pragma unroll
      for (int q = 0; q < kP2; ++q) {
        const int st = q / 2, g = q % 2;
        sc[PN][g] = mfma32(kf[st], qf[g][st], st == 0 ? f32x16{} : sc[PN][g]);
        if (g == 1 && st + kLead < kSteps)
          kf[st + kLead] =
              *reinterpret_cast<const bf16x8 *>(kn + 32 * TN * D + fo.k[st + kLead]);
#pragma unroll
        for (int r = 0; r < kR2; ++r) soft_step(pc, 1, kR2 * q + r);
        if constexpr (T == kKT - 1) {
          load_one(q, kr, vr, kbuf(std::integral_constant<int, BP>{}),
                   vbuf(std::integral_constant<int, BP>{}), wb);
        }
        TDP_NG2_MFMA_FIRST();
        TDP_NG2_FENCE();
      }
    };
    auto block = [&](auto bp_tag, int j) __attribute__((always_inline)) {
      iter(std::integral_constant<int, 0>{}, bp_tag, j);
      iter(std::integral_constant<int, 1>{}, bp_tag, j);
      iter(std::integral_constant<int, 2>{}, bp_tag, j);
      iter(std::integral_constant<int, 3>{}, bp_tag, j);
    };
    for (int j = 0; j < nkb; j += 2) {
      block(P0{}, j);
      if (j + 1 < nkb) block(P1{}, j + 1);
    }
    // the last tile's P V (tau = 4 nkb - 1 has parity 1)
#pragma unroll
    for (int q = 0; q < kP1; ++q) {
      const int dt = q / 4, x = (q / 2) % 2, g = q % 2;
      o[g][dt] = mfma32(vf[dt][x], pf[1][g][x], o[g][dt]);
    }
    // every direct load done before the buffers are reused or the wave ends
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    // padded keys scored 0 (p = 1 each); see attn_core_kernel for the check
    bool bad = false;
#pragma unroll
    for (int g = 0; g < 2; ++g) {
      const float lr = (lsum[g] + lsum2[g]) - static_cast<float>(nz);
      bad = bad || !(lr >= 0x1p-6f * static_cast<float>(nz));
      l_tot[g] = lr + __shfl_xor(lr, 32);
      bad = bad || !(l_tot[g] >= 0x1p-90f);
    }
    exact = __syncthreads_or(bad);
  }

  if (exact) {
    // The exact online softmax, tile by tile (rare: a score bound above the
    // shift-free range, or a cancelled sum).  Padded keys are masked.
    float m_run[2] = {-INFINITY, -INFINITY}, l_run[2] = {0.f, 0.f};
#pragma unroll
    for (int g = 0; g < 2; ++g)
#pragma unroll
      for (int i = 0; i < kDT; ++i) o[g][i] = f32x16{};
    // (the buffers are free: every wave passed the check above after its
    // loads completed)
    auto xblock = [&](auto par, int j) __attribute__((always_inline)) {
      const bf16 *kb = kbuf(par);
      load_block(j + 1, kbuf(std::integral_constant<int, 1 - decltype(par)::value>{}),
                 vbuf(std::integral_constant<int, 1 - decltype(par)::value>{}));
      const int kvalid = (j == nkb0 - 1) ? kvalid0 : ((j == nkb - 1 && nkb1 > 0) ? kvalid1 : kBN);
#pragma unroll
      for (int i = 0; i < kKT; ++i) {
        f32x16 sx[2][1];
#pragma unroll
        for (int g = 0; g < 2; ++g) sx[g][0] = f32x16{};
#pragma unroll
        for (int st = 0; st < kSteps; ++st) {
          const bf16x8 k8 = *reinterpret_cast<const bf16x8 *>(kb + 32 * i * D + fo.k[st]);
          sx[0][0] = mfma32(k8, qf[0][st], sx[0][0]);
          sx[1][0] = mfma32(k8, qf[1][st], sx[1][0]);
        }
        if (kvalid - 32 * i < 32) mask_padded<2, 1>(sx, kvalid - 32 * i, hh);
        bf16x8 px[2][1][2];
#pragma unroll
        for (int g = 0; g < 2; ++g) {
          const float mb = block_max<1>(sx[g]);
          if (mb > m_run[g] + kLazy) {
            const float m_new = fmaxf(m_run[g], mb);
            const float alpha = __builtin_amdgcn_exp2f(m_run[g] - m_new);
#pragma unroll
            for (int dd = 0; dd < kDT; ++dd)
#pragma unroll
              for (int v = 0; v < 16; ++v) o[g][dd][v] *= alpha;
            l_run[g] *= alpha;
            m_run[g] = m_new;
          }
          const float m = m_run[g] == -INFINITY ? 0.f : m_run[g];
          l_run[g] += exp_pack<true, 1>(sx[g], m, px[g]);
        }
#pragma unroll
        for (int dt = 0; dt < kDT; ++dt)
#pragma unroll
          for (int x = 0; x < 2; ++x) {
            const bf16x8 v8 = *reinterpret_cast<const bf16x8 *>(
                smem + (decltype(par)::value * kBufEl + 32 * dt * kBN) + fo.v[i][x]);
            o[0][dt] = mfma32(v8, px[0][0][x], o[0][dt]);
            o[1][dt] = mfma32(v8, px[1][0][x], o[1][dt]);
          }
      }
      asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
      lds_barrier();
    };
    load_block(0, sk0, sv0);
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    lds_barrier();
    for (int j = 0; j < nkb; j += 2) {
      xblock(P0{}, j);
      if (j + 1 < nkb) xblock(P1{}, j + 1);
    }
#pragma unroll
    for (int g = 0; g < 2; ++g) l_tot[g] = l_run[g] + __shfl_xor(l_run[g], 32);
  }

#pragma unroll
  for (int g = 0; g < 2; ++g) {
    const float inv = 1.0f / l_tot[g];
    const int row = 64 * wave + 32 * g + l32;
    if (row < nq) {
      bf16 *dst = audio_q
          ? a.oa + (((static_cast<int64_t>(t) * a.batch + b) * a.heads + h) * a.A + q0 + row) * D
          : a.o + ((b * a.heads + h) * a.n_rows + r0 + q0 + row) * D;
      dst += 4 * hh;
#pragma unroll
      for (int dt = 0; dt < kDT; ++dt) {
#pragma unroll
        for (int gg = 0; gg < 4; ++gg) {
          bf16x4 v4;
          v4[0] = static_cast<bf16>(o[g][dt][4 * gg + 0] * inv);
          v4[1] = static_cast<bf16>(o[g][dt][4 * gg + 1] * inv);
          v4[2] = static_cast<bf16>(o[g][dt][4 * gg + 2] * inv);
          v4[3] = static_cast<bf16>(o[g][dt][4 * gg + 3] * inv);
          *reinterpret_cast<bf16x4 *>(dst + 32 * dt + 8 * gg) = v4;
        }
      }
    }
  }
}

// Key-split launches: O = sum_s 2^(m_s - m) O_s / sum_s 2^(m_s - m) l_s with
// m = max_s m_s, per query row of every slot, rounded to bf16 into the same
// place as the unsplit core's output.  Parts with l = 0 hold no keys and are
// skipped.  A workgroup takes kRPP rows of one slot, D/4 threads per row and
// 4 columns per thread; all of a thread's loads are issued together.
template <int D>
__global__ __launch_bounds__(256) void attn_combine_kernel(CoreArgs a) {
  constexpr int kRowsWG = CoreShape<D>::kRowsWG;
  constexpr int kTPR = D / 4;
  constexpr int kRPP = 256 / kTPR;            // rows per workgroup
  constexpr int kWGS = kRowsWG / kRPP;        // workgroups per slot
  const int64_t slot = blockIdx.x / kWGS;
  CoreSlot cs;
  if (!core_slot<kRowsWG>(a, slot, cs)) return;
  const int row = static_cast<int>(blockIdx.x % kWGS) * kRPP + static_cast<int>(threadIdx.x) / kTPR;
  if (row >= min(cs.nq, kRowsWG)) return;
  const int S = a.kv_splits;
  const int c4 = threadIdx.x % kTPR;
  const int64_t base = slot * S * kRowsWG + row;   // (part 0, this row)
  float2 e[kMaxKvSplits];
#pragma unroll
  for (int s = 0; s < kMaxKvSplits; ++s)
    e[s] = s < S ? a.ml[base + s * kRowsWG] : make_float2(0.f, 0.f);
  float4 v[kMaxKvSplits];
#pragma unroll
  for (int s = 0; s < kMaxKvSplits; ++s)
    v[s] = e[s].y > 0.f ? *reinterpret_cast<const float4 *>(a.op + (base + s * kRowsWG) * D + 4 * c4)
                        : make_float4(0.f, 0.f, 0.f, 0.f);
  float m = -INFINITY;
#pragma unroll
  for (int s = 0; s < kMaxKvSplits; ++s)
    if (e[s].y > 0.f) m = fmaxf(m, e[s].x);
  float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
  float l = 0.f;
#pragma unroll
  for (int s = 0; s < kMaxKvSplits; ++s) {
    if (!(e[s].y > 0.f)) continue;
    const float w = __builtin_amdgcn_exp2f(e[s].x - m);
    acc.x = fmaf(w, v[s].x, acc.x);
    acc.y = fmaf(w, v[s].y, acc.y);
    acc.z = fmaf(w, v[s].z, acc.z);
    acc.w = fmaf(w, v[s].w, acc.w);
    l = fmaf(w, e[s].y, l);
  }
  const float inv = 1.0f / l;
  bf16 *dst = cs.audio_q
      ? a.oa + (((static_cast<int64_t>(cs.t) * a.batch + cs.b) * a.heads + cs.h) * a.A + cs.q0 +
                row) * D
      : a.o + ((cs.b * a.heads + cs.h) * a.n_rows + cs.r0 + cs.q0 + row) * D;
  bf16x4 o4;
  o4[0] = static_cast<bf16>(acc.x * inv);
  o4[1] = static_cast<bf16>(acc.y * inv);
  o4[2] = static_cast<bf16>(acc.z * inv);
  o4[3] = static_cast<bf16>(acc.w * inv);
  *reinterpret_cast<bf16x4 *>(dst + 4 * c4) = o4;
}

// ---------------------------------------------------------------------------
// out_proj
// ---------------------------------------------------------------------------

// ---------------------------------------------------------------------------
// host side
// ---------------------------------------------------------------------------

struct Call {
  const tdp_attn_desc *d;
  int32_t n_tiles;
  const int64_t *trb;
  int32_t max_rows;
  int64_t n_rows;
  void *ws;
  size_t ws_bytes;
  Layout L;
};

tdp_status check_call(Call *c) {
  const tdp_status s = make_layout(c->d, c->n_tiles, c->n_rows, &c->L);
  if (s != TDP_OK) return s;
  if (c->max_rows < 1 || c->max_rows > c->n_rows) return TDP_ERR_ARG;
  if (!c->trb || !c->ws) return TDP_ERR_NULL;
  if (!aligned16(c->ws)) return TDP_ERR_ALIGN;
  if (c->ws_bytes < c->L.total) return TDP_ERR_BUFFER;
  return TDP_OK;
}

}  // namespace
}  // namespace tdp

using namespace tdp;

extern "C" tdp_status tdp_tile_attention_workspace(const tdp_attn_desc *desc, int32_t n_tiles,
                                                   int64_t n_rows, size_t *bytes) {
  if (!bytes) return TDP_ERR_NULL;
  Layout L;
  const tdp_status s = make_layout(desc, n_tiles, n_rows, &L);
  if (s != TDP_OK) return s;
  *bytes = L.total;
  return TDP_OK;
}

extern "C" tdp_status tdp_attn_prepare(const tdp_attn_desc *desc, int32_t n_tiles,
                                       const int64_t *tile_row_begin, int32_t max_tile_rows,
                                       int64_t n_rows, const void *wq, const void *wk,
                                       const void *wv, const void *wo, void *workspace,
                                       size_t workspace_bytes, void *hip_stream) {
  Call c{desc, n_tiles, tile_row_begin, max_tile_rows, n_rows, workspace, workspace_bytes, {}};
  tdp_status s = check_call(&c);
  if (s != TDP_OK) return s;
  if (!wq || !wk || !wv || !wo) return TDP_ERR_NULL;
  if (!aligned16(wq) || !aligned16(wk) || !aligned16(wv) || !aligned16(wo)) return TDP_ERR_ALIGN;
  const Layout &L = c.L;
  const hipStream_t stream = as_stream(hip_stream);
  const int64_t n_el = 4LL * L.hidden * kC;
  hipLaunchKernelGGL(transpose_weights_kernel, dim3(static_cast<uint32_t>(ceil_div(n_el, 256))),
                     dim3(256), 0, stream, static_cast<const bf16 *>(wq),
                     static_cast<const bf16 *>(wk), static_cast<const bf16 *>(wv),
                     static_cast<const bf16 *>(wo), L.hidden, ws_at<bf16>(workspace, L.off_wt),
                     ws_at<bf16>(workspace, L.off_wot));
  if ((s = launch_status()) != TDP_OK) return s;
  hipLaunchKernelGGL(block_table_kernel, dim3(1), dim3(1024), 0, stream, tile_row_begin, n_tiles,
                     n_rows, max_tile_rows, L.npb, ws_at<int32_t>(workspace, L.off_pad_begin),
                     ws_at<int32_t>(workspace, L.off_blk_tile),
                     ws_at<int32_t>(workspace, L.off_blk_q0),
                     ws_at<uint32_t>(workspace, L.off_kmax),
                     static_cast<int64_t>(desc->batch) * desc->heads * (n_tiles + 1) + 1);
  return launch_status();
}

namespace {

template <typename TX, int D>
void launch_qkv(const Call &c, const void *x_tiles, const float *row_pos, const void *x_audio,
                hipStream_t stream) {
  const Layout &L = c.L;
  QkvArgs a{};
  a.blk_tile = ws_at<int32_t>(c.ws, L.off_blk_tile);
  a.blk_q0 = ws_at<int32_t>(c.ws, L.off_blk_q0);
  a.pad_begin = ws_at<int32_t>(c.ws, L.off_pad_begin);
  a.trb = c.trb;
  a.n_rows = c.n_rows;
  a.max_rows = c.max_rows;
  a.row_pos = row_pos;
  a.wt = ws_at<bf16>(c.ws, L.off_wt);
  a.kmax2 = ws_at<uint32_t>(c.ws, L.off_kmax);
  a.n_tiles = c.n_tiles;
  a.heads = c.d->heads;
  a.hidden = L.hidden;
  a.log2_theta_step = -std::log2(static_cast<double>(c.d->rope_base)) / (D / 6);
  a.q_scale = static_cast<float>(1.4426950408889634 / std::sqrt(static_cast<double>(D)));
  const int n_chunks = 3 * c.d->heads;
  // A launch with fewer than kQkvTargetWgs / 2 workgroups (one per 128 rows)
  // splits its chunks over blockIdx.z until it has about kQkvTargetWgs
  // (measured: 0.17 -> 0.07 ms on a 4-tile 8x32x32 latent; the 16-tile
  // 16x64x64 step, 968 workgroups, runs fastest unsplit).
  auto split = [&](int64_t wgs) {
    const int64_t want =
        wgs * 2 >= kQkvTargetWgs
            ? 1
            : std::max<int64_t>(1, std::min<int64_t>(n_chunks, ceil_div(kQkvTargetWgs, wgs)));
    const int per = static_cast<int>(ceil_div(n_chunks, want));
    return std::make_pair(per, static_cast<uint32_t>(ceil_div(n_chunks, per)));
  };
  // tile rows
  a.x = x_tiles;
  a.x_rows = c.n_rows;
  a.n_pad = L.n_pad;
  a.vt_cols = L.vt_cols;
  a.vt_col0 = 0;
  a.q = ws_at<bf16>(c.ws, L.off_q);
  a.k = ws_at<bf16>(c.ws, L.off_k);
  a.vt = ws_at<bf16>(c.ws, L.off_vt);
  {
    const auto [per, nz] = split(L.npb * c.d->batch);
    a.chunks_per_wg = per;
    hipLaunchKernelGGL((qkv_rope_kernel<TX, D, false>),
                       dim3(static_cast<uint32_t>(L.npb), c.d->batch, nz), dim3(kThreads), 0, stream,
                       a);
  }
  if (c.d->n_audio > 0) {
    a.x = x_audio;
    a.x_rows = c.d->n_audio;
    a.n_pad = L.a_pad;
    a.vt_col0 = L.n_pad;
    a.q = ws_at<bf16>(c.ws, L.off_qa);
    a.k = ws_at<bf16>(c.ws, L.off_ka);
    const auto [per, nz] = split(L.a_pad / kBlk * c.d->batch);
    a.chunks_per_wg = per;
    hipLaunchKernelGGL((qkv_rope_kernel<TX, D, true>),
                       dim3(static_cast<uint32_t>(L.a_pad / kBlk), c.d->batch, nz), dim3(kThreads),
                       0, stream, a);
  }
}

template <int D>
void launch_core(const Call &c, hipStream_t stream, bool tile_keys = true,
                 bool audio_queries = true) {
  const Layout &L = c.L;
  CoreArgs a{};
  a.q = ws_at<bf16>(c.ws, L.off_q);
  a.k = ws_at<bf16>(c.ws, L.off_k);
  a.vt = ws_at<bf16>(c.ws, L.off_vt);
  a.qa = ws_at<bf16>(c.ws, L.off_qa);
  a.ka = ws_at<bf16>(c.ws, L.off_ka);
  a.o = ws_at<bf16>(c.ws, L.off_o);
  a.oa = ws_at<bf16>(c.ws, L.off_oa);
  a.blk_tile = ws_at<int32_t>(c.ws, L.off_blk_tile);
  a.blk_q0 = ws_at<int32_t>(c.ws, L.off_blk_q0);
  a.pad_begin = ws_at<int32_t>(c.ws, L.off_pad_begin);
  a.trb = c.trb;
  a.n_units = L.npb / (kUnit / kBlk);
  a.n_pad = L.n_pad;
  a.a_pad = L.a_pad;
  a.vt_cols = L.vt_cols;
  a.n_rows = c.n_rows;
  a.units_per_bh = a.n_units + (audio_queries ? static_cast<int64_t>(c.n_tiles) * L.n_aqb : 0);
  a.total_units = a.units_per_bh * c.d->batch * c.d->heads;
  a.T = c.n_tiles;
  a.heads = c.d->heads;
  a.batch = c.d->batch;
  a.A = c.d->n_audio;
  a.n_aqb = audio_queries ? L.n_aqb : 0;
  a.tile_keys = tile_keys ? 1 : 0;
  a.max_rows = c.max_rows;
  a.hidden = L.hidden;
  a.kmax2 = ws_at<uint32_t>(c.ws, L.off_kmax);
  const int64_t slots = a.total_units * (kUnit / CoreShape<D>::kRowsWG);
  // Cross-attention (second segment only) is never split: its keys are few.
  // Chosen parts: as the layout's, or fewer when the longest tile
  // (max_rows) is shorter than the layout's bound.
  int32_t S = tile_keys ? L.kv_splits : 1;
  if (S > 1 && c.d->kv_splits == 0) {
    constexpr int64_t bn = CoreShape<D>::kBN;
    const int64_t nkb = ceil_div(c.max_rows, bn) + ceil_div(c.d->n_audio, bn);
    S = min(S, auto_kv_splits(slots, nkb, core_resident(D)));
  }
  if (S == 1) {
    const int64_t grid = ceil_div(slots, 8) * 8;
    if constexpr (TDP_ATTN_NG2) {
      // one 256-query workgroup per unit: per_xcd units per XCD, then (for
      // launches of two rounds or more, with the launch shape left to the
      // library: kv_splits 0) a claimed tail of about 1/12 of the units, with
      // 1.5 times its even share of claiming workgroups per XCD
      const int64_t U = a.total_units;
      const int64_t resident = kCUs * (D == 128 ? 1 : 2);
      a.per_xcd = ceil_div(U, 8);
      int64_t claims = 0;
      if (c.d->kv_splits == 0 && U >= 2 * resident) {
        a.per_xcd = (U - U / 12) / 8;
        claims = ceil_div(3 * (U - 8 * a.per_xcd), 16);
      }
      a.pool_claims = static_cast<uint32_t>(8 * claims);
      a.pool_ctr = ws_at<uint32_t>(c.ws, L.off_pool);
      const int64_t grid2 = 8 * (a.per_xcd + claims);
      hipLaunchKernelGGL((attn_core2_kernel<D>), dim3(static_cast<uint32_t>(grid2)), dim3(256), 0,
                         stream, a);
      return;
    }
    hipLaunchKernelGGL((attn_core_kernel<D, false>), dim3(static_cast<uint32_t>(grid)),
                       dim3(64 * CoreShape<D>::kWaves), 0, stream, a);
    return;
  }
  a.kv_splits = S;
  a.op = ws_at<float>(c.ws, L.off_op);
  a.ml = ws_at<float2>(c.ws, L.off_ml);
  const int64_t grid = ceil_div(slots * S, 8) * 8;
  hipLaunchKernelGGL((attn_core_kernel<D, true>), dim3(static_cast<uint32_t>(grid)),
                     dim3(64 * CoreShape<D>::kWaves), 0, stream, a);
  constexpr int64_t kCombineWGs = CoreShape<D>::kRowsWG / (256 / (D / 4));   // per slot
  hipLaunchKernelGGL(attn_combine_kernel<D>, dim3(static_cast<uint32_t>(slots * kCombineWGs)),
                     dim3(256), 0, stream, a);
}

}  // namespace

extern "C" tdp_status tdp_attn_qkv_rope(const tdp_attn_desc *desc, int32_t n_tiles,
                                        const int64_t *tile_row_begin, int32_t max_tile_rows,
                                        int64_t n_rows, const void *x_tiles, const float *row_pos,
                                        const void *x_audio, void *workspace,
                                        size_t workspace_bytes, void *hip_stream) {
  Call c{desc, n_tiles, tile_row_begin, max_tile_rows, n_rows, workspace, workspace_bytes, {}};
  const tdp_status s = check_call(&c);
  if (s != TDP_OK) return s;
  if (!x_tiles || !row_pos || (desc->n_audio > 0 && !x_audio)) return TDP_ERR_NULL;
  if (!aligned16(x_tiles) || (desc->n_audio > 0 && !aligned16(x_audio))) return TDP_ERR_ALIGN;
  if (c.L.npb > INT32_MAX) return TDP_ERR_ARG;
  const hipStream_t stream = as_stream(hip_stream);
  const bool f32 = desc->x_dtype == TDP_F32;
  if (desc->head_dim == 64) {
    if (f32) launch_qkv<float, 64>(c, x_tiles, row_pos, x_audio, stream);
    else launch_qkv<bf16, 64>(c, x_tiles, row_pos, x_audio, stream);
  } else {
    if (f32) launch_qkv<float, 128>(c, x_tiles, row_pos, x_audio, stream);
    else launch_qkv<bf16, 128>(c, x_tiles, row_pos, x_audio, stream);
  }
  return launch_status();
}

extern "C" tdp_status tdp_attn_core(const tdp_attn_desc *desc, int32_t n_tiles,
                                    const int64_t *tile_row_begin, int32_t max_tile_rows,
                                    int64_t n_rows, void *workspace, size_t workspace_bytes,
                                    void *hip_stream) {
  Call c{desc, n_tiles, tile_row_begin, max_tile_rows, n_rows, workspace, workspace_bytes, {}};
  const tdp_status s = check_call(&c);
  if (s != TDP_OK) return s;
  const int64_t units = (c.L.npb / (kUnit / kBlk) + static_cast<int64_t>(n_tiles) * c.L.n_aqb) *
                        desc->batch * desc->heads;
  const int64_t rows_wg = desc->head_dim == 64 ? CoreShape<64>::kRowsWG : CoreShape<128>::kRowsWG;
  const int64_t slots = units * (kUnit / rows_wg);
  // grids: the core (slots x parts) and, split, the combine (<= 32 per slot)
  if (ceil_div(slots * c.L.kv_splits, 8) * 8 > INT32_MAX ||
      (c.L.kv_splits > 1 && slots * 32 > INT32_MAX))
    return TDP_ERR_ARG;
  const hipStream_t stream = as_stream(hip_stream);
  if (desc->head_dim == 64) launch_core<64>(c, stream);
  else launch_core<128>(c, stream);
  return launch_status();
}

extern "C" tdp_status tdp_attn_out_proj(const tdp_attn_desc *desc, int32_t n_tiles,
                                        const int64_t *tile_row_begin, int32_t max_tile_rows,
                                        int64_t n_rows, void *y_tiles, float *y_audio_tiles,
                                        void *workspace, size_t workspace_bytes,
                                        void *hip_stream) {
  Call c{desc, n_tiles, tile_row_begin, max_tile_rows, n_rows, workspace, workspace_bytes, {}};
  tdp_status s = check_call(&c);
  if (s != TDP_OK) return s;
  if (!y_tiles || (desc->n_audio > 0 && !y_audio_tiles)) return TDP_ERR_NULL;
  if (!aligned16(y_tiles) || (desc->n_audio > 0 && !aligned16(y_audio_tiles))) return TDP_ERR_ALIGN;
  const Layout &L = c.L;
  const hipStream_t stream = as_stream(hip_stream);
  const bf16 *wot = ws_at<bf16>(workspace, L.off_wot);
  const int64_t M = static_cast<int64_t>(desc->batch) * n_rows;
  const int64_t Ma = static_cast<int64_t>(n_tiles) * desc->batch * desc->n_audio;
  // Y = O Wo with O head-major (see the attention core's stores)
  GemmDesc g;
  g.a = ws_at<bf16>(workspace, L.off_o);
  g.a_seg_rows = n_rows;
  g.a_heads = desc->heads;
  g.a_head_dim = desc->head_dim;
  g.bt = wot;
  g.ldb = L.hidden;
  g.M = M;
  g.N = kC;
  g.K = L.hidden;
  g.c = y_tiles;
  g.ldc = kC;
  s = gemm(desc->y_dtype == TDP_F32 ? kEpiF32 : kEpiBf16, g, stream);
  if (s != TDP_OK || Ma == 0) return s;
  g.a = ws_at<bf16>(workspace, L.off_oa);
  g.a_seg_rows = desc->n_audio;
  g.M = Ma;
  g.c = y_audio_tiles;
  return gemm(kEpiF32, g, stream);
}

extern "C" tdp_status tdp_tile_attention(const tdp_attn_desc *desc, int32_t n_tiles,
                                         const int64_t *tile_row_begin, int32_t max_tile_rows,
                                         int64_t n_rows, const void *x_tiles,
                                         const float *row_pos, const void *wq, const void *wk,
                                         const void *wv, const void *wo, const void *x_audio,
                                         void *y_tiles, float *y_audio_tiles, void *workspace,
                                         size_t workspace_bytes, void *hip_stream) {
  // Validate every argument before the first launch.
  Call c{desc, n_tiles, tile_row_begin, max_tile_rows, n_rows, workspace, workspace_bytes, {}};
  tdp_status s = check_call(&c);
  if (s != TDP_OK) return s;
  if (!x_tiles || !row_pos || !wq || !wk || !wv || !wo || !y_tiles ||
      (desc->n_audio > 0 && (!x_audio || !y_audio_tiles)))
    return TDP_ERR_NULL;
  s = tdp_attn_prepare(desc, n_tiles, tile_row_begin, max_tile_rows, n_rows, wq, wk, wv, wo,
                       workspace, workspace_bytes, hip_stream);
  if (s != TDP_OK) return s;
  s = tdp_attn_qkv_rope(desc, n_tiles, tile_row_begin, max_tile_rows, n_rows, x_tiles, row_pos,
                        x_audio, workspace, workspace_bytes, hip_stream);
  if (s != TDP_OK) return s;
  s = tdp_attn_core(desc, n_tiles, tile_row_begin, max_tile_rows, n_rows, workspace,
                    workspace_bytes, hip_stream);
  if (s != TDP_OK) return s;
  return tdp_attn_out_proj(desc, n_tiles, tile_row_begin, max_tile_rows, n_rows, y_tiles,
                           y_audio_tiles, workspace, workspace_bytes, hip_stream);
}

// ---------------------------------------------------------------------------
// the attention layer without a caller workspace
// ---------------------------------------------------------------------------

// Device scratch of tdp_tile_attention_noalloc: its whole workspace (weights
// transposed, block table, K-norm maxima, Q/K/V^T, O, key-split partials).
// Each GPU the library runs on holds its own copy for the life of the
// process.  In host code `scratch` names a host-side stand-in, never the
// device memory: the device address comes from hipGetSymbolAddress, once per
// device, and only that address is handed to kernels.
static __device__ __align__(256) unsigned char scratch[TDP_NOALLOC_SCRATCH_BYTES];

namespace tdp {
namespace {

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void *g_scratch_dev[kMaxDevices] = {};

// Device address of the current device's copy of `scratch`.
tdp_status scratch_address(void **out) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return TDP_ERR_HIP;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_dev[dev]) {
    void *p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return TDP_ERR_HIP;
    g_scratch_dev[dev] = p;
  }
  *out = g_scratch_dev[dev];
  return TDP_OK;
}

}  // namespace
}  // namespace tdp

extern "C" tdp_status tdp_tile_attention_noalloc(const tdp_attn_desc *desc, int32_t n_tiles,
                                                 const int64_t *tile_row_begin,
                                                 int32_t max_tile_rows, int64_t n_rows,
                                                 const void *x_tiles, const float *row_pos,
                                                 const void *wq, const void *wk, const void *wv,
                                                 const void *wo, const void *x_audio,
                                                 void *y_tiles, float *y_audio_tiles,
                                                 void *hip_stream) {
  // sizes first: a call that does not fit fails before touching the device
  Layout L;
  tdp_status s = make_layout(desc, n_tiles, n_rows, &L);
  if (s != TDP_OK) return s;
  if (L.total > static_cast<size_t>(TDP_NOALLOC_SCRATCH_BYTES)) return TDP_ERR_BUFFER;
  void *ws = nullptr;
  if ((s = scratch_address(&ws)) != TDP_OK) return s;
  // every region of the workspace is rewritten by the call's own kernels
  // (the K-norm maxima are cleared by a kernel of the prepare stage)
  return tdp_tile_attention(desc, n_tiles, tile_row_begin, max_tile_rows, n_rows, x_tiles,
                            row_pos, wq, wk, wv, wo, x_audio, y_tiles, y_audio_tiles, ws,
                            static_cast<size_t>(TDP_NOALLOC_SCRATCH_BYTES), hip_stream);
}

// ---------------------------------------------------------------------------
// internal entry points for the per-tile transformer block
// ---------------------------------------------------------------------------

namespace tdp {

tdp_status attn_tables(const tdp_attn_desc *desc, int32_t n_tiles, const int64_t *trb,
                       int32_t max_rows, int64_t n_rows, void *ws, size_t ws_bytes,
                       hipStream_t stream) {
  Call c{desc, n_tiles, trb, max_rows, n_rows, ws, ws_bytes, {}};
  const tdp_status s = check_call(&c);
  if (s != TDP_OK) return s;
  const Layout &L = c.L;
  hipLaunchKernelGGL(block_table_kernel, dim3(1), dim3(1024), 0, stream, trb, n_tiles, n_rows,
                     max_rows, L.npb, ws_at<int32_t>(ws, L.off_pad_begin),
                     ws_at<int32_t>(ws, L.off_blk_tile), ws_at<int32_t>(ws, L.off_blk_q0),
                     ws_at<uint32_t>(ws, L.off_kmax),
                     static_cast<int64_t>(desc->batch) * desc->heads * (n_tiles + 1) + 1);
  return launch_status();
}

tdp_status attn_rows_to_heads(const tdp_attn_desc *desc, int32_t n_tiles, const int64_t *trb,
                              int32_t max_rows, int64_t n_rows, const bf16 *src, int64_t ld,
                              int32_t q_col, int32_t k_col, int32_t v_col, const float *row_pos,
                              bool text, const bf16 *text_src, int64_t text_ld, void *ws,
                              size_t ws_bytes, hipStream_t stream) {
  Call c{desc, n_tiles, trb, max_rows, n_rows, ws, ws_bytes, {}};
  const tdp_status s = check_call(&c);
  if (s != TDP_OK) return s;
  const Layout &L = c.L;
  const int D = desc->head_dim;
  HeadsArgs a{};
  a.src = text ? text_src : src;
  a.ld = text ? text_ld : ld;
  a.src_rows = text ? desc->n_audio : n_rows;
  if (!a.src || a.ld % 8 != 0 || (text && desc->n_audio < 1)) return TDP_ERR_ARG;
  a.q_col = q_col;
  a.k_col = k_col;
  a.v_col = v_col;
  a.row_pos = row_pos;
  a.rope = (!text && row_pos) ? 1 : 0;
  a.log2_theta_step = static_cast<float>(-std::log2(static_cast<double>(desc->rope_base)) / (D / 6));
  a.q_scale = static_cast<float>(1.4426950408889634 / std::sqrt(static_cast<double>(D)));
  a.q = ws_at<bf16>(ws, text ? L.off_qa : L.off_q);
  a.k = ws_at<bf16>(ws, text ? L.off_ka : L.off_k);
  a.vt = ws_at<bf16>(ws, L.off_vt);
  a.n_pad = text ? L.a_pad : L.n_pad;
  a.vt_cols = L.vt_cols;
  a.vt_col0 = text ? L.n_pad : 0;
  a.kmax2 = ws_at<uint32_t>(ws, L.off_kmax);
  a.n_tiles = n_tiles;
  a.heads = desc->heads;
  a.blk_tile = ws_at<int32_t>(ws, L.off_blk_tile);
  a.blk_q0 = ws_at<int32_t>(ws, L.off_blk_q0);
  a.pad_begin = ws_at<int32_t>(ws, L.off_pad_begin);
  a.trb = trb;
  a.n_rows = n_rows;
  a.max_rows = max_rows;
  // heads split over workgroups until about 4096 of them (4 per CU are
  // resident; each walks its heads one after another)
  const int64_t wgs = (text ? L.a_pad / kBlk : L.npb) * desc->batch;
  const int64_t groups = std::min<int64_t>(desc->heads, std::max<int64_t>(1, ceil_div(4096, wgs)));
  a.heads_per_wg = static_cast<int32_t>(ceil_div(desc->heads, groups));
  const dim3 grid(static_cast<uint32_t>(text ? L.a_pad / kBlk : L.npb), desc->batch,
                  static_cast<uint32_t>(ceil_div(desc->heads, a.heads_per_wg)));
  if (D == 128) {
    if (text) hipLaunchKernelGGL((rows_to_heads_kernel<128, true>), grid, dim3(256), 0, stream, a);
    else hipLaunchKernelGGL((rows_to_heads_kernel<128, false>), grid, dim3(256), 0, stream, a);
  } else {
    if (text) hipLaunchKernelGGL((rows_to_heads_kernel<64, true>), grid, dim3(256), 0, stream, a);
    else hipLaunchKernelGGL((rows_to_heads_kernel<64, false>), grid, dim3(256), 0, stream, a);
  }
  return launch_status();
}

tdp_status attn_core_run(const tdp_attn_desc *desc, int32_t n_tiles, const int64_t *trb,
                         int32_t max_rows, int64_t n_rows, void *ws, size_t ws_bytes,
                         bool tile_keys, hipStream_t stream) {
  Call c{desc, n_tiles, trb, max_rows, n_rows, ws, ws_bytes, {}};
  const tdp_status s = check_call(&c);
  if (s != TDP_OK) return s;
  if (desc->head_dim == 64) launch_core<64>(c, stream, tile_keys, tile_keys);
  else launch_core<128>(c, stream, tile_keys, tile_keys);
  return launch_status();
}

const bf16 *attn_output(const tdp_attn_desc *desc, int32_t n_tiles, int64_t n_rows, void *ws) {
  Layout L;
  if (make_layout(desc, n_tiles, n_rows, &L) != TDP_OK) return nullptr;
  return ws_at<bf16>(ws, L.off_o);
}

uint32_t *attn_tail_counter(const tdp_attn_desc *desc, int32_t n_tiles, int64_t n_rows, void *ws) {
  Layout L;
  if (make_layout(desc, n_tiles, n_rows, &L) != TDP_OK) return nullptr;
  return ws_at<uint32_t>(ws, L.off_pool);
}

}  // namespace tdp
