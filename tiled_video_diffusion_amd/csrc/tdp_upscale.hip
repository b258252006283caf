// The TDP upscale loop on gfx950: re-noise, the blend fused with the Euler
// update and the tiles' seam spread, and the loop driver.
//
// "Tiled Data Parallelism (TDP)" page, "When to use it" (the note on stages):
// TDP is the upscale stage, run on a first stage's full-frame result; it
// re-injects noise up to its first sigma, and its tiles drift apart more as
// that sigma grows.  The page names no sampler.  This library's reading is the
// flow-matching form: a latent at noise level sigma is (1 - sigma) x0 +
// sigma eps, the blend of the tile outputs is the velocity, and each interval
// of the schedule is one explicit Euler step on the generated rows; the
// conditioning rows keep the clean stage-1 tokens.
//
// The loop's state is the global latent in float32, [B][N+M][C] with C = 128.
// One step is gather -> per-tile transformer -> blend_euler; blend_euler reads
// each generated token's tile rows once and updates the state in place, so
// the blended velocity never goes to memory.
#include <cmath>

#include "tdp_internal.h"

namespace tdp {
namespace {

constexpr int kThreads = 256;

// x[b][n] = (1 - s) x1[b][n] + s eps[b][n] on generated rows n < n_gen, x1[b][n]
// on the others.  One thread per 4-float vector; q4 = C / 4 vectors per row;
// total = B * n_dst * q4.  x may be x1.
__global__ __launch_bounds__(kThreads) void renoise_kernel(const f32x4 *x1, const f32x4 *eps,
                                                            int64_t n_gen, int64_t n_dst,
                                                            int32_t q4, float s, f32x4 *x,
                                                            int64_t total) {
  const int64_t i = static_cast<int64_t>(blockIdx.x) * kThreads + threadIdx.x;
  if (i >= total) return;
  const int64_t per_b = n_dst * q4;
  const int64_t b = i / per_b;
  const int64_t rem = i - b * per_b;     // n * q4 + q
  f32x4 v = x1[i];
  if (rem / q4 < n_gen) {
    const f32x4 e = eps[b * n_gen * q4 + rem];
    const float keep = 1.0f - s;
#pragma unroll
    for (int c = 0; c < 4; ++c) v[c] = fmaf(s, e[c], keep * v[c]);
  }
  x[i] = v;
}

// Tile rows and the latent are streamed with non-temporal hints when the tile
// rows are larger than the 256 MB last-level cache (NT = true); smaller ones
// were just written by the transformer and are read from that cache.
constexpr int64_t kStreamBytes = int64_t{256} << 20;

template <typename T, bool NT>
struct Load4;
template <bool NT>
struct Load4<float, NT> {
  __device__ static f32x4 at(const float *p) {
    const f32x4 *q = reinterpret_cast<const f32x4 *>(p);
    if constexpr (NT) return __builtin_nontemporal_load(q);
    else return *q;
  }
};
template <bool NT>
struct Load4<bf16, NT> {
  __device__ static f32x4 at(const bf16 *p) {
    const bf16x4 *q = reinterpret_cast<const bf16x4 *>(p);
    bf16x4 v;
    if constexpr (NT) v = __builtin_nontemporal_load(q);
    else v = *q;
    return f32x4{static_cast<float>(v[0]), static_cast<float>(v[1]), static_cast<float>(v[2]),
                 static_cast<float>(v[3])};
  }
};

__device__ __forceinline__ float sq_dist(f32x4 a, f32x4 b) {
  float t = 0.f;
#pragma unroll
  for (int c = 0; c < 4; ++c) {
    const float d = a[c] - b[c];
    t = fmaf(d, d, t);
  }
  return t;
}

// For every generated token n < n_gen of batch entry b = blockIdx.y:
//   v = sum_k w[r_k] y_tiles[b][r_k] over the token's rows r_k = dst_rows[k],
//       k in [dst_row_begin[n], dst_row_begin[n+1]), in that order (the blend);
//   x[b][n] += dsigma * v (Euler);
// and, with `partial`, the token's seam terms when two or more rows cover it:
//   s2 = sum_k w[r_k] |y_tiles[b][r_k] - v|^2, s0 = |v|^2,
// summed over the workgroup into partial[b * gridDim.x + blockIdx.x].
// Each thread owns 4 channels of one token (C / 4 threads per token); the
// first four rows of a token are loaded together, more (three-dimensional
// overlaps) in a loop.  Row ids outside [0, n_rows) are skipped.
template <typename T, bool NT>
__global__ __launch_bounds__(kThreads) void blend_euler_kernel(
    const T *__restrict__ y_tiles, int64_t n_rows, int32_t C,
    const int64_t *__restrict__ dst_row_begin, const int32_t *__restrict__ dst_rows,
    const float *__restrict__ row_weight, int64_t n_gen, int64_t n_dst, float *__restrict__ x,
    float dsigma, float2 *__restrict__ partial) {
  const int32_t qpr = C / 4;
  const int32_t rows_per_pass = kThreads / qpr;
  const int32_t lrow = threadIdx.x / qpr;
  const int32_t q = threadIdx.x - lrow * qpr;
  const int64_t n = static_cast<int64_t>(blockIdx.x) * rows_per_pass + lrow;
  const int64_t b = blockIdx.y;
  float s2 = 0.f, s0 = 0.f;
  if (lrow < rows_per_pass && n < n_gen) {
    const T *yb = y_tiles + b * n_rows * C + 4 * q;
    const int64_t kb = max(dst_row_begin[n], static_cast<int64_t>(0));
    const int64_t ke = min(dst_row_begin[n + 1], n_rows);
    int32_t r[4];
    float w[4];
    f32x4 y[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      r[u] = (kb + u < ke) ? dst_rows[kb + u] : -1;
      if (r[u] >= n_rows) r[u] = -1;
    }
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      w[u] = r[u] >= 0 ? row_weight[r[u]] : 0.f;
      y[u] = r[u] >= 0 ? Load4<T, NT>::at(yb + static_cast<int64_t>(r[u]) * C)
                       : f32x4{0.f, 0.f, 0.f, 0.f};
    }
    f32x4 v = {0.f, 0.f, 0.f, 0.f};
    int cnt = 0;
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      if (r[u] >= 0) {
#pragma unroll
        for (int c = 0; c < 4; ++c) v[c] = fmaf(w[u], y[u][c], v[c]);
        ++cnt;
      }
    }
    for (int64_t k = kb + 4; k < ke; ++k) {
      const int32_t rr = dst_rows[k];
      if (rr < 0 || rr >= n_rows) continue;
      const float ww = row_weight[rr];
      const f32x4 yy = Load4<T, NT>::at(yb + static_cast<int64_t>(rr) * C);
#pragma unroll
      for (int c = 0; c < 4; ++c) v[c] = fmaf(ww, yy[c], v[c]);
      ++cnt;
    }
    f32x4 *xp = reinterpret_cast<f32x4 *>(x + (b * n_dst + n) * C + 4 * q);
    f32x4 xv;
    if constexpr (NT) xv = __builtin_nontemporal_load(xp);
    else xv = *xp;
#pragma unroll
    for (int c = 0; c < 4; ++c) xv[c] = fmaf(dsigma, v[c], xv[c]);
    if constexpr (NT) __builtin_nontemporal_store(xv, xp);
    else *xp = xv;
    if (partial && cnt >= 2) {
#pragma unroll
      for (int c = 0; c < 4; ++c) s0 = fmaf(v[c], v[c], s0);
#pragma unroll
      for (int u = 0; u < 4; ++u)
        if (r[u] >= 0) s2 = fmaf(w[u], sq_dist(y[u], v), s2);
      for (int64_t k = kb + 4; k < ke; ++k) {
        const int32_t rr = dst_rows[k];
        if (rr < 0 || rr >= n_rows) continue;
        s2 = fmaf(row_weight[rr], sq_dist(Load4<T, NT>::at(yb + static_cast<int64_t>(rr) * C), v), s2);
      }
    }
  }
  if (partial) {   // uniform over the workgroup
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) {
      s2 += __shfl_xor(s2, off);
      s0 += __shfl_xor(s0, off);
    }
    __shared__ float red[2][kThreads / kWave];
    const int wave = threadIdx.x / kWave;
    if ((threadIdx.x & (kWave - 1)) == 0) {
      red[0][wave] = s2;
      red[1][wave] = s0;
    }
    __syncthreads();
    if (threadIdx.x == 0) {
      float a = 0.f, c = 0.f;
#pragma unroll
      for (int i = 0; i < kThreads / kWave; ++i) {
        a += red[0][i];
        c += red[1][i];
      }
      partial[b * gridDim.x + blockIdx.x] = make_float2(a, c);
    }
  }
}

// The seam sums in two fixed-order passes (the result does not depend on
// timing): pass 1, workgroup g adds the float2 partials [g * kSeamChunk,
// (g + 1) * kSeamChunk) in double; pass 2, one workgroup adds pass 1's sums and
// writes out = {S2, S0, sqrt(S2 / S0) or 0}.
constexpr int kSeamPerThread = 16;
constexpr int64_t kSeamChunk = static_cast<int64_t>(kThreads) * kSeamPerThread;

__device__ __forceinline__ void block_sum2(double &a, double &c) {
  __shared__ double red[2][kThreads];
  red[0][threadIdx.x] = a;
  red[1][threadIdx.x] = c;
  __syncthreads();
  for (int s = kThreads / 2; s > 0; s >>= 1) {
    if (static_cast<int>(threadIdx.x) < s) {
      red[0][threadIdx.x] += red[0][threadIdx.x + s];
      red[1][threadIdx.x] += red[1][threadIdx.x + s];
    }
    __syncthreads();
  }
  a = red[0][0];
  c = red[1][0];
}

__global__ __launch_bounds__(kThreads) void seam_pass1_kernel(const float2 *__restrict__ partial,
                                                               int64_t n,
                                                               double2 *__restrict__ sums) {
  const int64_t base = static_cast<int64_t>(blockIdx.x) * kSeamChunk + threadIdx.x;
  float2 v[kSeamPerThread];
#pragma unroll
  for (int j = 0; j < kSeamPerThread; ++j) {
    const int64_t i = base + static_cast<int64_t>(j) * kThreads;
    v[j] = i < n ? partial[i] : make_float2(0.f, 0.f);
  }
  double a = 0.0, c = 0.0;
#pragma unroll
  for (int j = 0; j < kSeamPerThread; ++j) {
    a += static_cast<double>(v[j].x);
    c += static_cast<double>(v[j].y);
  }
  block_sum2(a, c);
  if (threadIdx.x == 0) sums[blockIdx.x] = make_double2(a, c);
}

__global__ __launch_bounds__(kThreads) void seam_pass2_kernel(const double2 *__restrict__ sums,
                                                               int64_t n, double *__restrict__ out) {
  double a = 0.0, c = 0.0;
  for (int64_t i = threadIdx.x; i < n; i += kThreads) {
    a += sums[i].x;
    c += sums[i].y;
  }
  block_sum2(a, c);
  if (threadIdx.x == 0) {
    out[0] = a;
    out[1] = c;
    out[2] = c > 0.0 ? sqrt(a / c) : 0.0;
  }
}

__global__ void fill_kernel(float *__restrict__ p, int32_t n, float v) {
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) p[i] = v;
}

int esize_of(int32_t dtype) { return dtype == TDP_F32 ? 4 : (dtype == TDP_BF16 ? 2 : 0); }

int64_t blend_euler_blocks(int32_t C, int64_t n_gen) {
  const int64_t rows_per_block = kThreads / (C / 4);
  return (n_gen + rows_per_block - 1) / rows_per_block;
}

size_t a256(size_t v) { return (v + 255) & ~static_cast<size_t>(255); }

// Seam workspace: the workgroup partials, then pass 1's sums.
int64_t seam_partials(int32_t batch, int64_t n_gen, int32_t C) {
  return static_cast<int64_t>(batch) * blend_euler_blocks(C, n_gen);
}
int64_t seam_pass1_blocks(int64_t n_partials) {
  return (n_partials + kSeamChunk - 1) / kSeamChunk;
}
size_t partial_bytes(int32_t batch, int64_t n_gen, int32_t C) {
  const int64_t n = seam_partials(batch, n_gen, C);
  return a256(static_cast<size_t>(n) * sizeof(float2)) +
         a256(static_cast<size_t>(seam_pass1_blocks(n)) * sizeof(double2));
}

tdp_status check_blend_euler(int32_t dtype, int32_t batch, int64_t n_rows, int32_t C,
                             int64_t n_gen, int64_t n_dst) {
  if (esize_of(dtype) == 0) return TDP_ERR_UNSUPPORTED;
  if (batch < 1 || batch > 65535 || n_rows < 0 || C < 8 || C % 8 != 0 || n_gen < 0 ||
      n_dst < n_gen)
    return TDP_ERR_ARG;
  if (C / 4 > kThreads) return TDP_ERR_UNSUPPORTED;
  if (blend_euler_blocks(C, n_gen) > INT32_MAX) return TDP_ERR_ARG;
  return TDP_OK;
}

// Launch blend_euler (+ the seam reduction when seam is given); arguments
// already checked.
tdp_status launch_blend_euler(const void *y_tiles, int32_t dtype, int32_t batch, int64_t n_rows,
                              int32_t C, const int64_t *dst_row_begin, const int32_t *dst_rows,
                              const float *row_weight, int64_t n_gen, float *x, int64_t n_dst,
                              float dsigma, double *seam, void *seam_ws, hipStream_t stream) {
  const int64_t nblk = blend_euler_blocks(C, n_gen);
  const int64_t n_part = seam_partials(batch, n_gen, C);
  float2 *partial = seam ? static_cast<float2 *>(seam_ws) : nullptr;
  double2 *sums = seam ? reinterpret_cast<double2 *>(
                             static_cast<char *>(seam_ws) +
                             a256(static_cast<size_t>(n_part) * sizeof(float2)))
                       : nullptr;
  if (nblk > 0) {
    const dim3 grid(static_cast<uint32_t>(nblk), batch);
    const bool nt = static_cast<int64_t>(batch) * n_rows * C * esize_of(dtype) > kStreamBytes;
    if (dtype == TDP_F32) {
      auto k = nt ? blend_euler_kernel<float, true> : blend_euler_kernel<float, false>;
      hipLaunchKernelGGL(k, grid, dim3(kThreads), 0, stream, static_cast<const float *>(y_tiles),
                         n_rows, C, dst_row_begin, dst_rows, row_weight, n_gen, n_dst, x, dsigma,
                         partial);
    } else {
      auto k = nt ? blend_euler_kernel<bf16, true> : blend_euler_kernel<bf16, false>;
      hipLaunchKernelGGL(k, grid, dim3(kThreads), 0, stream, static_cast<const bf16 *>(y_tiles),
                         n_rows, C, dst_row_begin, dst_rows, row_weight, n_gen, n_dst, x, dsigma,
                         partial);
    }
    const tdp_status s = launch_status();
    if (s != TDP_OK) return s;
  }
  if (seam) {
    const int64_t g = seam_pass1_blocks(n_part);
    if (g > 0) {
      hipLaunchKernelGGL(seam_pass1_kernel, dim3(static_cast<uint32_t>(g)), dim3(kThreads), 0,
                         stream, partial, n_part, sums);
      const tdp_status s = launch_status();
      if (s != TDP_OK) return s;
    }
    hipLaunchKernelGGL(seam_pass2_kernel, dim3(1), dim3(kThreads), 0, stream, sums, g, seam);
    return launch_status();
  }
  return TDP_OK;
}

struct UpscaleLayout {
  size_t block_bytes = 0, off_block = 0, off_xt = 0, off_yt = 0, off_tau = 0, off_partial = 0;
  size_t total = 0;
};

tdp_status make_upscale_layout(const tdp_block_desc *d, const tdp_plan_dev *p,
                               UpscaleLayout *L) {
  if (!d || !p) return TDP_ERR_NULL;
  if (d->x_dtype != TDP_F32 || d->y_dtype != TDP_F32) return TDP_ERR_UNSUPPORTED;
  if (p->n_tiles < 1 || p->n_rows < 1 || p->n_gen < 1 || p->n_dst_rows < p->n_gen ||
      p->max_tile_rows < 1 || p->max_tile_rows > p->n_rows)
    return TDP_ERR_ARG;
  tdp_status s = tdp_block_workspace(d, p->n_tiles, p->n_rows, &L->block_bytes);
  if (s != TDP_OK) return s;
  s = check_blend_euler(TDP_F32, d->batch, p->n_rows, d->C, p->n_gen, p->n_dst_rows);
  if (s != TDP_OK) return s;
  const size_t tile_bytes = static_cast<size_t>(d->batch) * p->n_rows * d->C * sizeof(float);
  size_t off = 0;
  auto take = [&off](size_t bytes) { const size_t o = off; off = a256(off + bytes); return o; };
  L->off_block = take(L->block_bytes);
  L->off_xt = take(tile_bytes);
  L->off_yt = take(tile_bytes);
  L->off_tau = take(static_cast<size_t>(d->batch) * sizeof(float));
  L->off_partial = take(partial_bytes(d->batch, p->n_gen, d->C));
  L->total = off;
  return TDP_OK;
}

}  // namespace
}  // namespace tdp

using namespace tdp;

extern "C" tdp_status tdp_renoise(const float *x_stage1, const float *noise, int32_t batch,
                                  int64_t n_gen, int64_t n_dst_rows, int32_t C, float sigma0,
                                  float *x, void *hip_stream) {
  if (batch < 1 || n_gen < 0 || n_dst_rows < n_gen || C < 4 || C % 4 != 0 ||
      !(sigma0 >= 0.f && sigma0 <= 1.f))
    return TDP_ERR_ARG;
  if (n_dst_rows == 0) return TDP_OK;
  if (!x_stage1 || !x || (n_gen > 0 && !noise)) return TDP_ERR_NULL;
  if (!aligned16(x_stage1) || !aligned16(x) || (n_gen > 0 && !aligned16(noise)))
    return TDP_ERR_ALIGN;
  const int64_t total = static_cast<int64_t>(batch) * n_dst_rows * (C / 4);
  const int64_t nblk = (total + kThreads - 1) / kThreads;
  if (nblk > INT32_MAX) return TDP_ERR_ARG;
  hipLaunchKernelGGL(renoise_kernel, dim3(static_cast<uint32_t>(nblk)), dim3(kThreads), 0,
                     as_stream(hip_stream), reinterpret_cast<const f32x4 *>(x_stage1),
                     reinterpret_cast<const f32x4 *>(noise), n_gen, n_dst_rows, C / 4, sigma0,
                     reinterpret_cast<f32x4 *>(x), total);
  return launch_status();
}

extern "C" tdp_status tdp_blend_euler_workspace(int32_t batch, int64_t n_gen, int32_t C,
                                                size_t *bytes) {
  if (!bytes) return TDP_ERR_NULL;
  const tdp_status s = check_blend_euler(TDP_F32, batch, 0, C, n_gen, n_gen);
  if (s != TDP_OK) return s;
  *bytes = partial_bytes(batch, n_gen, C);
  return TDP_OK;
}

extern "C" tdp_status tdp_blend_euler(const void *y_tiles, int32_t dtype, int32_t batch,
                                      int64_t n_rows, int32_t C, const int64_t *dst_row_begin,
                                      const int32_t *dst_rows, const float *row_weight,
                                      int64_t n_gen, float *x, int64_t n_dst_rows, float sigma,
                                      float sigma_next, double *seam, void *workspace,
                                      size_t workspace_bytes, void *hip_stream) {
  tdp_status s = check_blend_euler(dtype, batch, n_rows, C, n_gen, n_dst_rows);
  if (s != TDP_OK) return s;
  if ((n_gen > 0 && (!x || !dst_row_begin)) ||
      (n_rows > 0 && n_gen > 0 && (!y_tiles || !dst_rows || !row_weight)))
    return TDP_ERR_NULL;
  if (seam) {
    if (!workspace) return TDP_ERR_NULL;
    if (workspace_bytes < partial_bytes(batch, n_gen, C)) return TDP_ERR_BUFFER;
    if (!aligned16(workspace) || (reinterpret_cast<uintptr_t>(seam) & 7u) != 0)
      return TDP_ERR_ALIGN;
  }
  if ((n_gen > 0 && !aligned16(x)) || (n_rows > 0 && n_gen > 0 && !aligned16(y_tiles)))
    return TDP_ERR_ALIGN;
  return launch_blend_euler(y_tiles, dtype, batch, n_rows, C, dst_row_begin, dst_rows,
                            row_weight, n_gen, x, n_dst_rows, sigma_next - sigma, seam, workspace,
                            as_stream(hip_stream));
}

extern "C" tdp_status tdp_upscale_workspace(const tdp_block_desc *desc,
                                            const tdp_plan_dev *plan, size_t *bytes) {
  if (!bytes) return TDP_ERR_NULL;
  UpscaleLayout L;
  const tdp_status s = make_upscale_layout(desc, plan, &L);
  if (s != TDP_OK) return s;
  *bytes = L.total;
  return TDP_OK;
}

extern "C" tdp_status tdp_upscale_loop(const tdp_block_desc *desc, const tdp_plan_dev *plan,
                                       const tdp_block_weights *weights, const void *text,
                                       const float *sigmas, int32_t n_steps, float *x,
                                       double *seam, void *workspace, size_t workspace_bytes,
                                       void *hip_stream) {
  UpscaleLayout L;
  tdp_status s = make_upscale_layout(desc, plan, &L);
  if (s != TDP_OK) return s;
  if (n_steps < 0) return TDP_ERR_ARG;
  if (!plan->tile_row_begin || !plan->row_src || !plan->row_weight || !plan->row_pos ||
      !plan->dst_row_begin || !plan->dst_rows || !weights || !text || !x || !workspace ||
      (n_steps > 0 && !sigmas))
    return TDP_ERR_NULL;
  if (workspace_bytes < L.total) return TDP_ERR_BUFFER;
  if (!aligned16(workspace) || !aligned16(x) || (seam && (reinterpret_cast<uintptr_t>(seam) & 7u)))
    return TDP_ERR_ALIGN;
  for (int32_t i = 0; i <= n_steps && n_steps > 0; ++i)
    if (!(sigmas[i] >= 0.f && sigmas[i] <= 1.f)) return TDP_ERR_ARG;
  const hipStream_t stream = as_stream(hip_stream);
  char *ws = static_cast<char *>(workspace);
  float *xt = reinterpret_cast<float *>(ws + L.off_xt);
  float *yt = reinterpret_cast<float *>(ws + L.off_yt);
  float *tau = reinterpret_cast<float *>(ws + L.off_tau);
  void *seam_ws = ws + L.off_partial;
  const int32_t B = desc->batch, Cc = desc->C;
  for (int32_t i = 0; i < n_steps; ++i) {
    // transformer timestep tau = 1000 sigma_i for every batch entry
    hipLaunchKernelGGL(fill_kernel, dim3((B + 255) / 256), dim3(256), 0, stream, tau, B,
                       1000.0f * sigmas[i]);
    if ((s = launch_status()) != TDP_OK) return s;
    if ((s = tdp_gather_tiles(x, TDP_F32, B, plan->n_dst_rows, Cc, plan->row_src, plan->n_rows,
                              xt, hip_stream)) != TDP_OK)
      return s;
    if ((s = tdp_block_forward(desc, plan->n_tiles, plan->tile_row_begin, plan->max_tile_rows,
                               plan->n_rows, xt, plan->row_pos, text, tau, weights, yt,
                               ws + L.off_block, L.block_bytes, hip_stream)) != TDP_OK)
      return s;
    if ((s = launch_blend_euler(yt, TDP_F32, B, plan->n_rows, Cc, plan->dst_row_begin,
                                plan->dst_rows, plan->row_weight, plan->n_gen, x,
                                plan->n_dst_rows, sigmas[i + 1] - sigmas[i],
                                seam ? seam + 3 * static_cast<int64_t>(i) : nullptr, seam_ws,
                                stream)) != TDP_OK)
      return s;
  }
  return TDP_OK;
}
