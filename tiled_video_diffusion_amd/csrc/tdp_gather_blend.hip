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

constexpr int kGatherThreads = 256;
constexpr int kGatherUnroll = 4;

// x_tiles[b][r] = x_global[b][row_src[r]] with `vpr` 16-byte vectors per row.
// Grid: (ceil(n_rows / rows_per_block), batch).  Rows whose source lies
// outside [0, n_src_rows) are written as zeros.
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
    if (r < n_rows) db[r * vpr + v] = val[u];
  }
}

template <typename T>
struct Vec4Load;
template <>
struct Vec4Load<float> {
  __device__ static f32x4 load(const float *p) { return *reinterpret_cast<const f32x4 *>(p); }
};
template <>
struct Vec4Load<bf16> {
  __device__ static f32x4 load(const bf16 *p) {
    const bf16x4 v = *reinterpret_cast<const bf16x4 *>(p);
    return f32x4{static_cast<float>(v[0]), static_cast<float>(v[1]), static_cast<float>(v[2]),
                 static_cast<float>(v[3])};
  }
};

constexpr int kBlendThreads = 256;

// y_global[b][n][4q..4q+3] (+)= sum_k w[r_k] * y_tiles[b][r_k][4q..4q+3] over the
// rows r_k = dst_rows[k], k in [dst_row_begin[n], dst_row_begin[n+1]), in that
// order.  Each thread owns 4 output channels of one token: no atomics.
// Grid: (ceil(n_dst / rows_per_block), batch), qpr = C / 4 threads per row.
template <typename T>
__global__ __launch_bounds__(kBlendThreads) void blend_rows_kernel(
    const T *__restrict__ y_tiles, int64_t n_rows, int32_t C,
    const int64_t *__restrict__ dst_row_begin, const int32_t *__restrict__ dst_rows,
    const float *__restrict__ row_weight, int64_t n_dst, float *__restrict__ y_global,
    int32_t accumulate) {
  const int32_t qpr = C / 4;
  const int32_t rows_per_block = kBlendThreads / qpr;
  const int32_t lrow = threadIdx.x / qpr;
  const int32_t q = threadIdx.x - lrow * qpr;
  if (lrow >= rows_per_block) return;
  const int64_t n = static_cast<int64_t>(blockIdx.x) * rows_per_block + lrow;
  if (n >= n_dst) return;
  const int64_t b = blockIdx.y;
  const T *yb = y_tiles + b * n_rows * C + 4 * q;
  float *out = y_global + (b * n_dst + n) * C + 4 * q;
  f32x4 acc = accumulate ? *reinterpret_cast<const f32x4 *>(out) : f32x4{0.f, 0.f, 0.f, 0.f};
  int64_t k = max(dst_row_begin[n], static_cast<int64_t>(0));
  const int64_t k1 = min(dst_row_begin[n + 1], n_rows);
  // Four contributions in flight at a time; summed in list order.
  for (; k < k1; k += 4) {
    int32_t r[4];
    float w[4];
    f32x4 y[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      r[u] = (k + u < k1) ? dst_rows[k + u] : -1;
      if (r[u] >= n_rows) r[u] = -1;
    }
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      w[u] = r[u] >= 0 ? row_weight[r[u]] : 0.f;
      y[u] = r[u] >= 0 ? Vec4Load<T>::load(yb + static_cast<int64_t>(r[u]) * C)
                       : f32x4{0.f, 0.f, 0.f, 0.f};
    }
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      if (r[u] >= 0) {
        acc[0] = fmaf(w[u], y[u][0], acc[0]);
        acc[1] = fmaf(w[u], y[u][1], acc[1]);
        acc[2] = fmaf(w[u], y[u][2], acc[2]);
        acc[3] = fmaf(w[u], y[u][3], acc[3]);
      }
    }
  }
  *reinterpret_cast<f32x4 *>(out) = acc;
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
  hipLaunchKernelGGL(gather_rows_kernel, dim3(static_cast<uint32_t>(nblk), batch),
                     dim3(kGatherThreads), 0, as_stream(hip_stream),
                     static_cast<const uint4 *>(x_global), row_src, n_src_rows, n_rows, vpr,
                     static_cast<uint4 *>(x_tiles));
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
  const int64_t rows_per_block = kBlendThreads / (C / 4);
  const int64_t nblk = (n_dst_rows + rows_per_block - 1) / rows_per_block;
  if (nblk > INT32_MAX) return TDP_ERR_ARG;
  const dim3 grid(static_cast<uint32_t>(nblk), batch);
  if (dtype == TDP_F32) {
    hipLaunchKernelGGL(blend_rows_kernel<float>, grid, dim3(kBlendThreads), 0,
                       as_stream(hip_stream), static_cast<const float *>(y_tiles), n_rows, C,
                       dst_row_begin, dst_rows, row_weight, n_dst_rows, y_global, accumulate);
  } else {
    hipLaunchKernelGGL(blend_rows_kernel<bf16>, grid, dim3(kBlendThreads), 0,
                       as_stream(hip_stream), static_cast<const bf16 *>(y_tiles), n_rows, C,
                       dst_row_begin, dst_rows, row_weight, n_dst_rows, y_global, accumulate);
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
