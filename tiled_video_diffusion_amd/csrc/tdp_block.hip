// The per-tile transformer block for gfx950: the whole denoising network each
// rank applies to its tiles (TDP page, "What it is"), built as L blocks of
//
//   h = rms(x) (1 + scale_a) + shift_a;  x += gate_a * SelfAttn(h)
//   h = rms(x);                          x += CrossAttn(h, text)
//   h = rms(x) (1 + scale_f) + shift_f;  x += gate_f * FFN(h)
//
// around x_0 = X W_in and y = rms(x_L) W_out.  The page does not describe the
// transformer; the layout above (one shared timestep modulation, text
// cross-attention, tanh-GELU FFN of width 4D) is the reading this library
// uses.  Every matrix product runs on gemm() (tdp_gemm.hip) with its
// epilogue fused (GELU, SiLU); self- and cross-attention run on the attention
// core; RMSNorm with the modulation is one row kernel, which also performs
// the residual add x += gate * branch of the branch that ran before it (the
// branch's GEMM stores its output in bf16), so no GEMM reads and rewrites the
// float32 residual stream.  The residual stream x is float32; GEMM operands
// are bf16.
#include <cmath>

#include "tdp_internal.h"

namespace tdp {
namespace {

constexpr int kRowsPerWg = 4;   // rows (one per wave) per RMSNorm workgroup
constexpr float kRmsEps = 1e-6f;
// 1: rows of 256, 1024, 2048 or 4096 features go through the register form.
#ifndef TDP_RMS_ROWS
#define TDP_RMS_ROWS 1
#endif

// One wave per row m (batch entry b = m / rows_per_batch):
//   with y: x[m][:] += g * y[m][:] first (the residual add of the branch that
//     produced y; g = ge[b][:] + gt[:], either term may be absent, g = 1 when
//     both are), written back to x;
//   h[m][:] = bf16(rms(x[m][:]) * (1 + scale) + shift), shift and scale =
//     e[b][row r of 6] + table[r] for r = shift_row, shift_row + 1 (both
//     absent: plain RMSNorm).
// VEC: D a multiple of 256, each lane moves 16-byte pieces (4 floats) of the
// row.  y and h may be the same buffer: a row's y is read in full before its
// h is written, by the same wave.
template <bool VEC>
__global__ __launch_bounds__(64 * kRowsPerWg) void rms_mod_kernel(
    float *__restrict__ x, int64_t M, int32_t D, int64_t rows_per_batch,
    const float *__restrict__ e, const float *__restrict__ table, int32_t shift_row,
    const bf16 *y, const float *__restrict__ ge, const float *__restrict__ gt, bf16 *h) {
  const int lane = threadIdx.x & 63;
  const int64_t m = static_cast<int64_t>(blockIdx.x) * kRowsPerWg + (threadIdx.x >> 6);
  if (m >= M) return;
  float *xr = x + m * D;
  const int64_t b = m / rows_per_batch;
  const float *es = e ? e + (b * 6 + shift_row) * D : nullptr;
  const float *ts = table ? table + static_cast<int64_t>(shift_row) * D : nullptr;
  const float *gs = ge ? ge + b * 6 * D : nullptr;
  const bf16 *yr = y ? y + m * D : nullptr;
  bf16 *hr = h + m * D;
  float ss = 0.f;
  if constexpr (VEC) {
    for (int j = 4 * lane; j < D; j += 256) {
      f32x4 v = *reinterpret_cast<const f32x4 *>(xr + j);
      if (yr) {
        const bf16x4 yv = *reinterpret_cast<const bf16x4 *>(yr + j);
        f32x4 g = {1.f, 1.f, 1.f, 1.f};
        if (gs || gt) {
          g = f32x4{0.f, 0.f, 0.f, 0.f};
          if (gs) g += *reinterpret_cast<const f32x4 *>(gs + j);
          if (gt) g += *reinterpret_cast<const f32x4 *>(gt + j);
        }
#pragma unroll
        for (int q = 0; q < 4; ++q) v[q] = fmaf(g[q], static_cast<float>(yv[q]), v[q]);
        *reinterpret_cast<f32x4 *>(xr + j) = v;
      }
      ss = fmaf(v[0], v[0], fmaf(v[1], v[1], fmaf(v[2], v[2], fmaf(v[3], v[3], ss))));
    }
  } else {
    for (int j = lane; j < D; j += 64) {
      float v = xr[j];
      if (yr) {
        const float g = (gs || gt) ? (gs ? gs[j] : 0.f) + (gt ? gt[j] : 0.f) : 1.f;
        v = fmaf(g, static_cast<float>(yr[j]), v);
        xr[j] = v;
      }
      ss = fmaf(v, v, ss);
    }
  }
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) ss += __shfl_xor(ss, off);
  const float rs = 1.0f / sqrtf(ss / static_cast<float>(D) + kRmsEps);
  if constexpr (VEC) {
    for (int j = 4 * lane; j < D; j += 256) {
      const f32x4 v = *reinterpret_cast<const f32x4 *>(xr + j);
      f32x4 shift = {0.f, 0.f, 0.f, 0.f}, scale = {0.f, 0.f, 0.f, 0.f};
      if (es) {
        shift += *reinterpret_cast<const f32x4 *>(es + j);
        scale += *reinterpret_cast<const f32x4 *>(es + D + j);
      }
      if (ts) {
        shift += *reinterpret_cast<const f32x4 *>(ts + j);
        scale += *reinterpret_cast<const f32x4 *>(ts + D + j);
      }
      bf16x4 o;
#pragma unroll
      for (int q = 0; q < 4; ++q) o[q] = static_cast<bf16>((v[q] * rs) * (1.0f + scale[q]) + shift[q]);
      *reinterpret_cast<bf16x4 *>(hr + j) = o;
    }
  } else {
    for (int j = lane; j < D; j += 64) {
      float v = xr[j] * rs;
      if (es || ts) {
        const float shift = (es ? es[j] : 0.f) + (ts ? ts[j] : 0.f);
        const float scale = (es ? es[D + j] : 0.f) + (ts ? ts[D + j] : 0.f);
        v = v * (1.0f + scale) + shift;
      }
      hr[j] = static_cast<bf16>(v);
    }
  }
}

// The same for D = 256 NC with the row held in registers: every load of x
// and y is issued before the first use, and the second pass reads no x
// again (the loop form above keeps one 16-byte load per lane in flight and
// re-reads the row).  Same arithmetic in the same order, so the results
// are bitwise those of rms_mod_kernel<true>.  NT: x is read and written and
// h written with non-temporal hints (for x larger than the 256 MB
// last-level cache, where keeping these streams out of it pays).
template <int NC, bool NT>
__global__ __launch_bounds__(64 * kRowsPerWg) void rms_mod_row_kernel(
    float *__restrict__ x, int64_t M, int64_t rows_per_batch, const float *__restrict__ e,
    const float *__restrict__ table, int32_t shift_row, const bf16 *y,
    const float *__restrict__ ge, const float *__restrict__ gt, bf16 *h) {
  constexpr int D = 256 * NC;
  const int lane = threadIdx.x & 63;
  const int64_t m = static_cast<int64_t>(blockIdx.x) * kRowsPerWg + (threadIdx.x >> 6);
  if (m >= M) return;
  float *xr = x + m * D;
  const int64_t b = m / rows_per_batch;
  const float *es = e ? e + (b * 6 + shift_row) * D : nullptr;
  const float *ts = table ? table + static_cast<int64_t>(shift_row) * D : nullptr;
  const float *gs = ge ? ge + b * 6 * D : nullptr;
  const bf16 *yr = y ? y + m * D : nullptr;
  bf16 *hr = h + m * D;
  f32x4 v[NC];
#pragma unroll
  for (int c = 0; c < NC; ++c) {
    const f32x4 *p = reinterpret_cast<const f32x4 *>(xr + 256 * c + 4 * lane);
    v[c] = NT ? __builtin_nontemporal_load(p) : *p;
  }
  float ss = 0.f;
  if (yr) {
    bf16x4 yv[NC];
#pragma unroll
    for (int c = 0; c < NC; ++c)
      yv[c] = *reinterpret_cast<const bf16x4 *>(yr + 256 * c + 4 * lane);
#pragma unroll
    for (int c = 0; c < NC; ++c) {
      const int j = 256 * c + 4 * lane;
      f32x4 g = {1.f, 1.f, 1.f, 1.f};
      if (gs || gt) {
        g = f32x4{0.f, 0.f, 0.f, 0.f};
        if (gs) g += *reinterpret_cast<const f32x4 *>(gs + j);
        if (gt) g += *reinterpret_cast<const f32x4 *>(gt + j);
      }
#pragma unroll
      for (int q = 0; q < 4; ++q) v[c][q] = fmaf(g[q], static_cast<float>(yv[c][q]), v[c][q]);
      f32x4 *p = reinterpret_cast<f32x4 *>(xr + j);
      if (NT) __builtin_nontemporal_store(v[c], p);
      else *p = v[c];
    }
  }
#pragma unroll
  for (int c = 0; c < NC; ++c)
    ss = fmaf(v[c][0], v[c][0], fmaf(v[c][1], v[c][1], fmaf(v[c][2], v[c][2], fmaf(v[c][3], v[c][3], ss))));
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) ss += __shfl_xor(ss, off);
  const float rs = 1.0f / sqrtf(ss / static_cast<float>(D) + kRmsEps);
#pragma unroll
  for (int c = 0; c < NC; ++c) {
    const int j = 256 * c + 4 * lane;
    f32x4 shift = {0.f, 0.f, 0.f, 0.f}, scale = {0.f, 0.f, 0.f, 0.f};
    if (es) {
      shift += *reinterpret_cast<const f32x4 *>(es + j);
      scale += *reinterpret_cast<const f32x4 *>(es + D + j);
    }
    if (ts) {
      shift += *reinterpret_cast<const f32x4 *>(ts + j);
      scale += *reinterpret_cast<const f32x4 *>(ts + D + j);
    }
    bf16x4 o;
#pragma unroll
    for (int q = 0; q < 4; ++q) o[q] = static_cast<bf16>((v[c][q] * rs) * (1.0f + scale[q]) + shift[q]);
    bf16x4 *p = reinterpret_cast<bf16x4 *>(hr + j);
    if (NT) __builtin_nontemporal_store(o, p);
    else *p = o;
  }
}


// emb[b][i] = cos(tau_b w_i), emb[b][half + i] = sin(tau_b w_i),
// w_i = 10000^(-i / half), rounded to bf16.
__global__ void time_embed_kernel(const float *__restrict__ tau, int32_t B, int32_t dim,
                                  bf16 *__restrict__ emb) {
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  const int half = dim / 2;
  if (i >= B * half) return;
  const int b = i / half, k = i - b * half;
  const float w = exp2f(-static_cast<float>(k) / static_cast<float>(half) * 13.287712379549449f);
  float s, c;
  sincosf(tau[b] * w, &s, &c);
  emb[b * dim + k] = static_cast<bf16>(c);
  emb[b * dim + half + k] = static_cast<bf16>(s);
}

__global__ void to_bf16_kernel(const float *__restrict__ src, int64_t n, bf16 *__restrict__ dst) {
  const int64_t i = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
  if (i < n) dst[i] = static_cast<bf16>(src[i]);
}

size_t a256(size_t x) { return (x + 255) & ~static_cast<size_t>(255); }

struct BlockLayout {
  tdp_attn_desc self{}, cross{};
  size_t off_self = 0, off_cross = 0, off_x = 0, off_h = 0, off_big = 0, off_xin = 0;
  size_t off_emb = 0, off_e1 = 0, off_e = 0, off_ckv = 0, total = 0;
  size_t self_bytes = 0, cross_bytes = 0;
  int64_t D = 0, M = 0;
};

tdp_status make_block_layout(const tdp_block_desc *d, int32_t n_tiles, int64_t n_rows,
                             BlockLayout *L) {
  if (!d) return TDP_ERR_NULL;
  if (d->batch < 1 || d->heads < 1 || d->n_text < 1 || d->layers < 0 || d->time_dim < 64 ||
      d->time_dim % 64 != 0 || n_rows < 1 || n_tiles < 1)
    return TDP_ERR_ARG;
  if (d->C != 128 || (d->head_dim != 64 && d->head_dim != 128)) return TDP_ERR_UNSUPPORTED;
  const int64_t D = static_cast<int64_t>(d->heads) * d->head_dim;
  if (D % 128 != 0 || D > (1 << 16)) return TDP_ERR_UNSUPPORTED;
  if ((d->x_dtype != TDP_F32 && d->x_dtype != TDP_BF16) ||
      (d->y_dtype != TDP_F32 && d->y_dtype != TDP_BF16))
    return TDP_ERR_UNSUPPORTED;
  L->D = D;
  L->M = static_cast<int64_t>(d->batch) * n_rows;
  L->self = tdp_attn_desc{d->batch, 128, d->heads, d->head_dim, 0, TDP_BF16, TDP_BF16,
                          d->rope_base};
  L->cross = L->self;
  L->cross.n_audio = d->n_text;
  tdp_status s = tdp_tile_attention_workspace(&L->self, n_tiles, n_rows, &L->self_bytes);
  if (s != TDP_OK) return s;
  s = tdp_tile_attention_workspace(&L->cross, n_tiles, n_rows, &L->cross_bytes);
  if (s != TDP_OK) return s;
  const size_t M = L->M, B = d->batch;
  size_t off = 0;
  auto take = [&off](size_t bytes) { const size_t o = off; off = a256(off + bytes); return o; };
  L->off_self = take(L->self_bytes);
  L->off_cross = take(L->cross_bytes);
  L->off_x = take(M * D * 4);
  L->off_h = take(M * D * 2);
  L->off_big = take(M * 4 * D * 2);
  L->off_xin = take(M * 128 * 2);
  L->off_emb = take(B * d->time_dim * 2);
  L->off_e1 = take(B * D * 2);
  L->off_e = take(B * 6 * D * 4);
  L->off_ckv = take(B * static_cast<size_t>(d->n_text) * 2 * D * 2);
  L->total = off;
  return TDP_OK;
}

template <typename T>
T *at(void *ws, size_t off) { return reinterpret_cast<T *>(static_cast<char *>(ws) + off); }

}  // namespace
}  // namespace tdp

using namespace tdp;

extern "C" tdp_status tdp_block_workspace(const tdp_block_desc *desc, int32_t n_tiles,
                                          int64_t n_rows, size_t *bytes) {
  if (!bytes) return TDP_ERR_NULL;
  BlockLayout L;
  const tdp_status s = make_block_layout(desc, n_tiles, n_rows, &L);
  if (s != TDP_OK) return s;
  *bytes = L.total;
  return TDP_OK;
}

extern "C" tdp_status tdp_block_forward(const tdp_block_desc *desc, int32_t n_tiles,
                                        const int64_t *tile_row_begin, int32_t max_tile_rows,
                                        int64_t n_rows, const void *x_tiles,
                                        const float *row_pos, const void *text, const float *tau,
                                        const tdp_block_weights *w, void *y_tiles,
                                        void *workspace, size_t workspace_bytes,
                                        void *hip_stream) {
  BlockLayout L;
  tdp_status s = make_block_layout(desc, n_tiles, n_rows, &L);
  if (s != TDP_OK) return s;
  if (!tile_row_begin || !x_tiles || !row_pos || !text || !tau || !w || !y_tiles || !workspace ||
      !w->w_in || !w->w_out || !w->wt1 || !w->wt2 || (desc->layers > 0 && !w->layers))
    return TDP_ERR_NULL;
  for (int l = 0; l < desc->layers; ++l) {
    const tdp_block_layer &y = w->layers[l];
    if (!y.wqkv || !y.wo || !y.cq || !y.ckv || !y.co || !y.w1 || !y.w2 || !y.table)
      return TDP_ERR_NULL;
    if (!aligned16(y.wqkv) || !aligned16(y.wo) || !aligned16(y.cq) || !aligned16(y.ckv) ||
        !aligned16(y.co) || !aligned16(y.w1) || !aligned16(y.w2) || !aligned16(y.table))
      return TDP_ERR_ALIGN;
  }
  if (!aligned16(w->w_in) || !aligned16(w->w_out) || !aligned16(w->wt1) || !aligned16(w->wt2))
    return TDP_ERR_ALIGN;
  if (max_tile_rows < 1 || max_tile_rows > n_rows) return TDP_ERR_ARG;
  if (workspace_bytes < L.total) return TDP_ERR_BUFFER;
  if (!aligned16(workspace) || !aligned16(x_tiles) || !aligned16(text) || !aligned16(y_tiles))
    return TDP_ERR_ALIGN;
  const hipStream_t stream = as_stream(hip_stream);
  const int64_t D = L.D, M = L.M, B = desc->batch, NT = desc->n_text;
  void *ws_self = at<char>(workspace, L.off_self);
  void *ws_cross = at<char>(workspace, L.off_cross);
  float *x = at<float>(workspace, L.off_x);
  bf16 *h = at<bf16>(workspace, L.off_h);
  bf16 *big = at<bf16>(workspace, L.off_big);
  bf16 *e1 = at<bf16>(workspace, L.off_e1);
  float *E = at<float>(workspace, L.off_e);
  bf16 *ckv = at<bf16>(workspace, L.off_ckv);
  // every launch below runs in stream order, so the large GEMMs share the
  // self-attention workspace's tail counter with its core (zeroed by
  // attn_tables before the first of them)
  uint32_t *tail_ctr = attn_tail_counter(&L.self, n_tiles, n_rows, ws_self);
  // h = RMSNorm of x with the modulation rows (shift_row, shift_row + 1) of
  // `table` (and E), after x += gate * y when y is given (y = the branch
  // output a GEMM just stored in h; gate rows of E and of the table by
  // pointer, both absent = 1).
  auto rms = [&](const float *table, int shift_row, const bf16 *y = nullptr,
                 const float *gate_e = nullptr, const float *gate_t = nullptr) {
    const dim3 grid(static_cast<uint32_t>((M + kRowsPerWg - 1) / kRowsPerWg));
    const float *ep = table ? E : nullptr;
    const bool nt = M * D * 4 >= (int64_t{256} << 20);   // x beyond the last-level cache
#define TDP_RMS_ROW(NC)                                                                        \
  if (D == 256 * NC) {                                                                         \
    if (nt)                                                                                    \
      hipLaunchKernelGGL((rms_mod_row_kernel<NC, true>), grid, dim3(64 * kRowsPerWg), 0,        \
                         stream, x, M, n_rows, ep, table, shift_row, y, gate_e, gate_t, h);    \
    else                                                                                       \
      hipLaunchKernelGGL((rms_mod_row_kernel<NC, false>), grid, dim3(64 * kRowsPerWg), 0,       \
                         stream, x, M, n_rows, ep, table, shift_row, y, gate_e, gate_t, h);    \
    return launch_status();                                                                    \
  }
    if (TDP_RMS_ROWS) {
      TDP_RMS_ROW(16)
      TDP_RMS_ROW(8)
      TDP_RMS_ROW(4)
      TDP_RMS_ROW(1)
    }
#undef TDP_RMS_ROW
    if (D % 256 == 0)
      hipLaunchKernelGGL(rms_mod_kernel<true>, grid, dim3(64 * kRowsPerWg), 0, stream, x, M,
                         static_cast<int32_t>(D), n_rows, table ? E : nullptr, table, shift_row,
                         y, gate_e, gate_t, h);
    else
      hipLaunchKernelGGL(rms_mod_kernel<false>, grid, dim3(64 * kRowsPerWg), 0, stream, x, M,
                         static_cast<int32_t>(D), n_rows, table ? E : nullptr, table, shift_row,
                         y, gate_e, gate_t, h);
    return launch_status();
  };
  auto mm = [&](int epi, const bf16 *a, int64_t lda, int64_t m, const void *bt, int32_t n,
                int32_t k, void *c, int64_t ldc, const float *g0 = nullptr,
                const float *g1 = nullptr) {
    GemmDesc g;
    g.a = a;
    g.lda = lda;
    g.bt = static_cast<const bf16 *>(bt);
    g.ldb = k;
    g.M = m;
    g.N = n;
    g.K = k;
    g.c = c;
    g.ldc = ldc;
    g.g0 = g0;
    g.g0_stride = 6 * D;
    g.g1 = g1;
    g.rows_per_batch = n_rows;
    g.tail_ctr = tail_ctr;
    return gemm(epi, g, stream);
  };
  auto proj_o = [&](const tdp_attn_desc *ad, void *aws, const void *wo) {
    GemmDesc g;
    g.a = attn_output(ad, n_tiles, n_rows, aws);
    g.a_seg_rows = n_rows;
    g.a_heads = desc->heads;
    g.a_head_dim = desc->head_dim;
    g.bt = static_cast<const bf16 *>(wo);
    g.ldb = D;
    g.M = M;
    g.N = static_cast<int32_t>(D);
    g.K = static_cast<int32_t>(D);
    g.c = h;
    g.ldc = D;
    g.tail_ctr = tail_ctr;
    return gemm(kEpiBf16, g, stream);
  };
#define TDP_TRY(expr)               \
  do {                              \
    const tdp_status st_ = (expr);  \
    if (st_ != TDP_OK) return st_;  \
  } while (0)

  TDP_TRY(attn_tables(&L.self, n_tiles, tile_row_begin, max_tile_rows, n_rows, ws_self,
                      L.self_bytes, stream));
  TDP_TRY(attn_tables(&L.cross, n_tiles, tile_row_begin, max_tile_rows, n_rows, ws_cross,
                      L.cross_bytes, stream));
  // x_0 = X W_in
  const bf16 *xin = static_cast<const bf16 *>(x_tiles);
  if (desc->x_dtype == TDP_F32) {
    bf16 *xb = at<bf16>(workspace, L.off_xin);
    const int64_t n = M * 128;
    hipLaunchKernelGGL(to_bf16_kernel, dim3(static_cast<uint32_t>((n + 255) / 256)), dim3(256), 0,
                       stream, static_cast<const float *>(x_tiles), n, xb);
    TDP_TRY(launch_status());
    xin = xb;
  }
  TDP_TRY(mm(kEpiF32, xin, 128, M, w->w_in, static_cast<int32_t>(D), 128, x, D));
  // timestep modulation E[b] = silu(emb(tau_b) Wt1) Wt2, shared by the layers
  bf16 *emb = at<bf16>(workspace, L.off_emb);
  hipLaunchKernelGGL(time_embed_kernel,
                     dim3(static_cast<uint32_t>((B * desc->time_dim / 2 + 255) / 256)), dim3(256),
                     0, stream, tau, static_cast<int32_t>(B), desc->time_dim, emb);
  TDP_TRY(launch_status());
  TDP_TRY(mm(kEpiSiluBf16, emb, desc->time_dim, B, w->wt1, static_cast<int32_t>(D), desc->time_dim,
             e1, D));
  TDP_TRY(mm(kEpiF32, e1, D, B, w->wt2, static_cast<int32_t>(6 * D), static_cast<int32_t>(D), E,
             6 * D));
  // Each branch's GEMM stores its output in h (bf16); the residual add
  // x += gate * branch happens in the RMSNorm kernel that reads x next.
  const bf16 *pend_y = nullptr;                 // branch output waiting in h
  const float *pend_ge = nullptr, *pend_gt = nullptr;
  for (int l = 0; l < desc->layers; ++l) {
    const tdp_block_layer &y = w->layers[l];
    // self-attention, gated
    TDP_TRY(rms(y.table, 0, pend_y, pend_ge, pend_gt));
    TDP_TRY(mm(kEpiBf16, h, D, M, y.wqkv, static_cast<int32_t>(3 * D), static_cast<int32_t>(D),
               big, 3 * D));
    TDP_TRY(attn_rows_to_heads(&L.self, n_tiles, tile_row_begin, max_tile_rows, n_rows, big,
                               3 * D, 0, static_cast<int32_t>(D), static_cast<int32_t>(2 * D),
                               row_pos, false, nullptr, 0, ws_self, L.self_bytes, stream));
    TDP_TRY(attn_core_run(&L.self, n_tiles, tile_row_begin, max_tile_rows, n_rows, ws_self,
                          L.self_bytes, true, stream));
    TDP_TRY(proj_o(&L.self, ws_self, y.wo));
    // cross-attention over the text tokens (after x += gate_a * attention)
    TDP_TRY(rms(nullptr, 0, h, E + 2 * D, y.table + 2 * D));
    TDP_TRY(mm(kEpiBf16, h, D, M, y.cq, static_cast<int32_t>(D), static_cast<int32_t>(D), big, D));
    TDP_TRY(attn_rows_to_heads(&L.cross, n_tiles, tile_row_begin, max_tile_rows, n_rows, big, D, 0,
                               -1, -1, nullptr, false, nullptr, 0, ws_cross, L.cross_bytes,
                               stream));
    TDP_TRY(mm(kEpiBf16, static_cast<const bf16 *>(text), D, B * NT, y.ckv,
               static_cast<int32_t>(2 * D), static_cast<int32_t>(D), ckv, 2 * D));
    TDP_TRY(attn_rows_to_heads(&L.cross, n_tiles, tile_row_begin, max_tile_rows, n_rows, nullptr,
                               0, -1, 0, static_cast<int32_t>(D), nullptr, true, ckv, 2 * D,
                               ws_cross, L.cross_bytes, stream));
    TDP_TRY(attn_core_run(&L.cross, n_tiles, tile_row_begin, max_tile_rows, n_rows, ws_cross,
                          L.cross_bytes, false, stream));
    TDP_TRY(proj_o(&L.cross, ws_cross, y.co));
    // FFN, gated (after x += cross-attention, ungated)
    TDP_TRY(rms(y.table, 3, h, nullptr, nullptr));
    TDP_TRY(mm(kEpiGeluBf16, h, D, M, y.w1, static_cast<int32_t>(4 * D), static_cast<int32_t>(D),
               big, 4 * D));
    TDP_TRY(mm(kEpiBf16, big, 4 * D, M, y.w2, static_cast<int32_t>(D),
               static_cast<int32_t>(4 * D), h, D));
    pend_y = h;
    pend_ge = E + 5 * D;
    pend_gt = y.table + 5 * D;
  }
  // y = rms(x_L) W_out (after x += gate_f * FFN of the last block)
  TDP_TRY(rms(nullptr, 0, pend_y, pend_ge, pend_gt));
  return mm(desc->y_dtype == TDP_F32 ? kEpiF32 : kEpiBf16, h, D, M, w->w_out, 128,
            static_cast<int32_t>(D), y_tiles, 128);
#undef TDP_TRY
}
