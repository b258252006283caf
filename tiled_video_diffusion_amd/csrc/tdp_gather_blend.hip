// Gather of tile rows, the weighted blend into the global latent, and the
// audio average: the HBM-bound ends of a TDP step on gfx950.
//
// "Tiled Data Parallelism (TDP)" page, "What it is": tiles are pieces of the
// latent; their mask-weighted outputs are summed into the result by one
// all_reduce, which on one GPU becomes the blend below; audio is averaged over
// tiles.  "Shared negative (reference) positions": conditioning rows weigh 1/k.
//
// Rows are 128-channel token rows (512 B in float32, 256 B in bf16).  Each
// thread moves 16-byte vectors; a block covers whole rows so every row is read
// and written by consecutive lanes in full 16-byte pieces.
#include "tdp_common.h"

namespace tdp {
namespace {

// Data touched exactly once (the blend's tile rows and result, the gather's
// written rows) goes with non-temporal hints when the stream is larger than
// the 256 MB last-level cache (NT = true).  Smaller streams keep ordinary
// accesses: the producer ran just before, so they hit in that cache (measured:
// a 122 MB blend runs at half speed with the hints, an 877 MB one 11% faster).
constexpr int64_t kStreamBytes = int64_t{256} << 20;

template <bool NT, typename V>
__device__ __forceinline__ V ld_once(const V *p) {
  if constexpr (NT) return __builtin_nontemporal_load(p);
  else return *p;
}
template <bool NT, typename V>
__device__ __forceinline__ void st_once(V *p, V v) {
  if constexpr (NT) __builtin_nontemporal_store(v, p);
  else *p = v;
}

constexpr int kGatherThreads = 256;
#ifndef TDP_GATHER_UNROLL
#define TDP_GATHER_UNROLL 4
#endif
constexpr int kGatherUnroll = TDP_GATHER_UNROLL;

// x_tiles[b][r] = x_global[b][row_src[r]] with `vpr` 16-byte vectors per row.
// Grid: (ceil(n_rows / rows_per_block), batch).  Rows whose source lies
// outside [0, n_src_rows) are written as zeros.
template <bool NT>
__global__ __launch_bounds__(kGatherThreads) void gather_rows_kernel(
    const uint4 *__restrict__ src, const int32_t *__restrict__ row_src, int64_t n_src_rows,
    int64_t n_rows, int32_t vpr, uint4 *__restrict__ dst) {
  const int32_t rows_per_pass = kGatherThreads / vpr;
  const int32_t lrow = threadIdx.x / vpr;
  const int32_t v = threadIdx.x - lrow * vpr;
  if (lrow >= rows_per_pass) return;
  const int64_t b = blockIdx.y;
  const int64_t r0 = static_cast<int64_t>(blockIdx.x) * rows_per_pass * kGatherUnroll + lrow;
  const uint4 *sb = src + b * n_src_rows * vpr;
  uint4 *db = dst + b * n_rows * vpr;
  uint4 val[kGatherUnroll];
#pragma unroll
  for (int u = 0; u < kGatherUnroll; ++u) {
    const int64_t r = r0 + static_cast<int64_t>(u) * rows_per_pass;
    val[u] = make_uint4(0, 0, 0, 0);
    if (r < n_rows) {
      const int32_t s = row_src[r];
      if (s >= 0 && s < n_src_rows) val[u] = sb[static_cast<int64_t>(s) * vpr + v];
    }
  }
#pragma unroll
  for (int u = 0; u < kGatherUnroll; ++u) {
    const int64_t r = r0 + static_cast<int64_t>(u) * rows_per_pass;
    if (r < n_rows) {
      typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
      st_once<NT>(reinterpret_cast<u32x4 *>(db + r * vpr + v),
              u32x4{val[u].x, val[u].y, val[u].z, val[u].w});
    }
  }
}

constexpr int kBlendThreads = 256;
// Destination rows per thread: their index, weight and data loads are all
// issued before any arithmetic (measured best: 1; 4 loses 2-25%).
#ifndef TDP_BLEND_ROWS
#define TDP_BLEND_ROWS 1
#endif
constexpr int kBlendRows = TDP_BLEND_ROWS;
template <bool NT, typename T>
struct Vec4Once;
template <bool NT>
struct Vec4Once<NT, float> {
  __device__ static f32x4 load(const float *p) { return ld_once<NT>(reinterpret_cast<const f32x4 *>(p)); }
};
template <bool NT>
struct Vec4Once<NT, bf16> {
  __device__ static f32x4 load(const bf16 *p) {
    const bf16x4 v = ld_once<NT>(reinterpret_cast<const bf16x4 *>(p));
    return f32x4{static_cast<float>(v[0]), static_cast<float>(v[1]), static_cast<float>(v[2]),
                 static_cast<float>(v[3])};
  }
};

// y_global[b][n][4q..4q+3] (+)= sum_k w[r_k] * y_tiles[b][r_k][4q..4q+3] over the
// rows r_k = dst_rows[k], k in [dst_row_begin[n], dst_row_begin[n+1]), in that
// order.  Each thread owns 4 output channels of kBlendRows tokens (rows
// n0 + i * rows_per_pass): no atomics.  The first four contributions of every
// row are loaded together; rows with more (three-dimensional overlaps) finish
// in a loop.  Row ids outside [0, n_rows) are skipped.
// Grid: (ceil(n_dst / (rows_per_pass * kBlendRows)), batch), qpr = C / 4
// threads per row.
template <typename T, bool NT>
__global__ __launch_bounds__(kBlendThreads) void blend_rows_kernel(
    const T *__restrict__ y_tiles, int64_t n_rows, int32_t C,
    const int64_t *__restrict__ dst_row_begin, const int32_t *__restrict__ dst_rows,
    const float *__restrict__ row_weight, int64_t n_dst, float *__restrict__ y_global,
    int32_t accumulate) {
  constexpr int R = kBlendRows;
  const int32_t qpr = C / 4;
  const int32_t rows_per_pass = kBlendThreads / qpr;
  const int32_t lrow = threadIdx.x / qpr;
  const int32_t q = threadIdx.x - lrow * qpr;
  if (lrow >= rows_per_pass) return;
  const int64_t n0 = static_cast<int64_t>(blockIdx.x) * rows_per_pass * R + lrow;
  const int64_t b = blockIdx.y;
  const T *yb = y_tiles + b * n_rows * C + 4 * q;
  float *ob = y_global + b * n_dst * C + 4 * q;
  int64_t kb[R], ke[R];
#pragma unroll
  for (int i = 0; i < R; ++i) {
    const int64_t n = n0 + static_cast<int64_t>(i) * rows_per_pass;
    kb[i] = 0;
    ke[i] = 0;
    if (n < n_dst) {
      kb[i] = max(dst_row_begin[n], static_cast<int64_t>(0));
      ke[i] = min(dst_row_begin[n + 1], n_rows);
    }
  }
  int32_t r[R][4];
#pragma unroll
  for (int i = 0; i < R; ++i)
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      r[i][u] = (kb[i] + u < ke[i]) ? dst_rows[kb[i] + u] : -1;
      if (r[i][u] >= n_rows) r[i][u] = -1;
    }
  float w[R][4];
  f32x4 y[R][4];
#pragma unroll
  for (int i = 0; i < R; ++i)
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      w[i][u] = r[i][u] >= 0 ? row_weight[r[i][u]] : 0.f;
      y[i][u] = r[i][u] >= 0 ? Vec4Once<NT, T>::load(yb + static_cast<int64_t>(r[i][u]) * C)
                             : f32x4{0.f, 0.f, 0.f, 0.f};
    }
#pragma unroll
  for (int i = 0; i < R; ++i) {
    const int64_t n = n0 + static_cast<int64_t>(i) * rows_per_pass;
    if (n >= n_dst) continue;
    float *out = ob + n * C;
    f32x4 acc = accumulate ? *reinterpret_cast<const f32x4 *>(out) : f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      if (r[i][u] >= 0) {
        acc[0] = fmaf(w[i][u], y[i][u][0], acc[0]);
        acc[1] = fmaf(w[i][u], y[i][u][1], acc[1]);
        acc[2] = fmaf(w[i][u], y[i][u][2], acc[2]);
        acc[3] = fmaf(w[i][u], y[i][u][3], acc[3]);
      }
    }
    for (int64_t k = kb[i] + 4; k < ke[i]; ++k) {
      const int32_t rr = dst_rows[k];
      if (rr < 0 || rr >= n_rows) continue;
      const float ww = row_weight[rr];
      const f32x4 yy = Vec4Once<NT, T>::load(yb + static_cast<int64_t>(rr) * C);
      acc[0] = fmaf(ww, yy[0], acc[0]);
      acc[1] = fmaf(ww, yy[1], acc[1]);
      acc[2] = fmaf(ww, yy[2], acc[2]);
      acc[3] = fmaf(ww, yy[3], acc[3]);
    }
    st_once<NT>(reinterpret_cast<f32x4 *>(out), acc);
  }
}

// y_audio[i] (+)= sum_t inv_t * y_audio_tiles[t][i] over 4-float vectors i.
__global__ __launch_bounds__(256) void audio_mean_kernel(const f32x4 *__restrict__ tiles,
                                                          int32_t n_tiles, int64_t n_vec,
                                                          float inv_t, f32x4 *__restrict__ out,
                                                          int32_t accumulate) {
  const int64_t i = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
  if (i >= n_vec) return;
  f32x4 acc = accumulate ? out[i] : f32x4{0.f, 0.f, 0.f, 0.f};
  for (int32_t t = 0; t < n_tiles; ++t) {
    const f32x4 y = tiles[static_cast<int64_t>(t) * n_vec + i];
    acc[0] = fmaf(inv_t, y[0], acc[0]);
    acc[1] = fmaf(inv_t, y[1], acc[1]);
    acc[2] = fmaf(inv_t, y[2], acc[2]);
    acc[3] = fmaf(inv_t, y[3], acc[3]);
  }
  out[i] = acc;
}

int esize_of(int32_t dtype) { return dtype == TDP_F32 ? 4 : (dtype == TDP_BF16 ? 2 : 0); }

}  // namespace
}  // namespace tdp

using namespace tdp;

extern "C" tdp_status tdp_gather_tiles(const void *x_global, int32_t dtype, int32_t batch,
                                       int64_t n_src_rows, int32_t C, const int32_t *row_src,
                                       int64_t n_rows, void *x_tiles, void *hip_stream) {
  const int es = esize_of(dtype);
  if (es == 0) return TDP_ERR_UNSUPPORTED;
  if (batch < 1 || batch > 65535 || n_src_rows < 1 || C < 8 || C % 8 != 0 || n_rows < 0)
    return TDP_ERR_ARG;
  if (n_rows == 0) return TDP_OK;
  if (!x_global || !row_src || !x_tiles) return TDP_ERR_NULL;
  if (!aligned16(x_global) || !aligned16(x_tiles)) return TDP_ERR_ALIGN;
  const int32_t vpr = C * es / 16;
  if (vpr > kGatherThreads) return TDP_ERR_UNSUPPORTED;
  const int64_t rows_per_block = static_cast<int64_t>(kGatherThreads / vpr) * kGatherUnroll;
  const int64_t nblk = (n_rows + rows_per_block - 1) / rows_per_block;
  if (nblk > INT32_MAX) return TDP_ERR_ARG;
  const bool nt = static_cast<int64_t>(batch) * n_rows * C * es > kStreamBytes;
  auto kernel = nt ? gather_rows_kernel<true> : gather_rows_kernel<false>;
  hipLaunchKernelGGL(kernel, dim3(static_cast<uint32_t>(nblk), batch), dim3(kGatherThreads), 0,
                     as_stream(hip_stream), static_cast<const uint4 *>(x_global), row_src,
                     n_src_rows, n_rows, vpr, static_cast<uint4 *>(x_tiles));
  return launch_status();
}

extern "C" tdp_status tdp_blend_accumulate(const void *y_tiles, int32_t dtype, int32_t batch,
                                           int64_t n_rows, int32_t C,
                                           const int64_t *dst_row_begin,
                                           const int32_t *dst_rows, const float *row_weight,
                                           int64_t n_dst_rows, float *y_global,
                                           int32_t accumulate, void *hip_stream) {
  if (esize_of(dtype) == 0) return TDP_ERR_UNSUPPORTED;
  if (batch < 1 || batch > 65535 || n_rows < 0 || C < 8 || C % 8 != 0 || n_dst_rows < 0 ||
      (accumulate != 0 && accumulate != 1))
    return TDP_ERR_ARG;
  if (C / 4 > kBlendThreads) return TDP_ERR_UNSUPPORTED;
  if (n_dst_rows == 0) return TDP_OK;
  if (!y_global || !dst_row_begin || (n_rows > 0 && (!y_tiles || !dst_rows || !row_weight)))
    return TDP_ERR_NULL;
  if ((n_rows > 0 && !aligned16(y_tiles)) || !aligned16(y_global)) return TDP_ERR_ALIGN;
  const int64_t rows_per_block = static_cast<int64_t>(kBlendThreads / (C / 4)) * kBlendRows;
  const int64_t nblk = (n_dst_rows + rows_per_block - 1) / rows_per_block;
  if (nblk > INT32_MAX) return TDP_ERR_ARG;
  const dim3 grid(static_cast<uint32_t>(nblk), batch);
  const bool nt = static_cast<int64_t>(batch) * n_rows * C * esize_of(dtype) > kStreamBytes;
  if (dtype == TDP_F32) {
    auto kernel = nt ? blend_rows_kernel<float, true> : blend_rows_kernel<float, false>;
    hipLaunchKernelGGL(kernel, grid, dim3(kBlendThreads), 0, as_stream(hip_stream),
                       static_cast<const float *>(y_tiles), n_rows, C, dst_row_begin, dst_rows,
                       row_weight, n_dst_rows, y_global, accumulate);
  } else {
    auto kernel = nt ? blend_rows_kernel<bf16, true> : blend_rows_kernel<bf16, false>;
    hipLaunchKernelGGL(kernel, grid, dim3(kBlendThreads), 0, as_stream(hip_stream),
                       static_cast<const bf16 *>(y_tiles), n_rows, C, dst_row_begin, dst_rows,
                       row_weight, n_dst_rows, y_global, accumulate);
  }
  return launch_status();
}

extern "C" tdp_status tdp_audio_accumulate(const float *y_audio_tiles, int32_t n_tiles_local,
                                           int32_t n_tiles_total, int32_t batch,
                                           int32_t n_audio, int32_t C, float *y_audio,
                                           int32_t accumulate, void *hip_stream) {
  if (n_tiles_local < 0 || n_tiles_total < 1 || n_tiles_local > n_tiles_total || batch < 1 ||
      n_audio < 0 || C < 8 || C % 8 != 0 || (accumulate != 0 && accumulate != 1))
    return TDP_ERR_ARG;
  if (n_audio == 0) return TDP_OK;
  if (!y_audio || (n_tiles_local > 0 && !y_audio_tiles)) return TDP_ERR_NULL;
  if (!aligned16(y_audio) || (n_tiles_local > 0 && !aligned16(y_audio_tiles)))
    return TDP_ERR_ALIGN;
  const int64_t n_vec = static_cast<int64_t>(batch) * n_audio * C / 4;
  const int64_t nblk = (n_vec + 255) / 256;
  if (nblk > INT32_MAX) return TDP_ERR_ARG;
  const float inv_t = 1.0f / static_cast<float>(n_tiles_total);
  hipLaunchKernelGGL(audio_mean_kernel, dim3(static_cast<uint32_t>(nblk)), dim3(256), 0,
                     as_stream(hip_stream), reinterpret_cast<const f32x4 *>(y_audio_tiles),
                     n_tiles_local, n_vec, inv_t, reinterpret_cast<f32x4 *>(y_audio), accumulate);
  return launch_status();
}
