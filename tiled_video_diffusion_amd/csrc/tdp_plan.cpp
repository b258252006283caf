// Host-side tile plan of one TDP step: tile boxes, round-robin share, rows,
// trapezoid masks, normalized positions, conditioning keep rule and 1/k
// weights, and the inverse (token -> rows) map.
//
// Follows the "Tiled Data Parallelism (TDP)" design page: "What it is" (tiles,
// round-robin assignment, trapezoidal masks summing to one), "API / Tiling
// config" (tile counts and overlap in latent units), "Position normalization"
// and "Shared negative (reference) positions".  Float outputs are float32
// values produced by single IEEE operations (quotients of small integers,
// products of two floats, differences of integer-valued floats), so they do
// not depend on evaluation order or contraction; the file is built with
// -ffp-contract=off all the same.
#include <algorithm>
#include <climits>
#include <cmath>
#include <cstdint>
#include <cstring>
#include <vector>

#include "tdp.h"

namespace {

int32_t core_at(int32_t i, int32_t L, int32_t n) {
  return static_cast<int32_t>((static_cast<int64_t>(i) * L) / n);
}

// A dimension of length L split into n tiles overlapping by o (see tdp.h).
struct DimTiling {
  int32_t L = 1, n = 1, o = 0;

  tdp_status check() const {
    if (L < 1 || L > (1 << 24)) return TDP_ERR_ARG;  // positions must be exact floats
    if (n < 1 || n > L) return TDP_ERR_ARG;
    if (o < 0) return TDP_ERR_ARG;
    if (n == 1) return TDP_OK;
    int32_t min_core = INT32_MAX;
    for (int32_t i = 0; i < n; ++i)
      min_core = std::min(min_core, core_at(i + 1, L, n) - core_at(i, L, n));
    return o <= min_core ? TDP_OK : TDP_ERR_ARG;
  }
  void box(int32_t i, int32_t *a, int32_t *b) const {
    if (n == 1) { *a = 0; *b = L; return; }
    const int32_t lo = o / 2, hi = o - o / 2;
    *a = std::max(0, core_at(i, L, n) - lo);
    *b = std::min(L, core_at(i + 1, L, n) + hi);
  }
  // Trapezoid factor of tile i at grid position p (p inside the tile's box):
  // ramp up (2k+1)/(2o) across the overlap with tile i-1, ramp down
  // (2o-2k-1)/(2o) across the overlap with tile i+1, 1 elsewhere.
  float weight(int32_t i, int32_t p) const {
    if (n == 1 || o == 0) return 1.0f;
    const int32_t lo = o / 2;
    const float two_o = static_cast<float>(2 * o);
    if (i > 0) {
      const int32_t s = core_at(i, L, n) - lo;
      if (p >= s && p < s + o) return static_cast<float>(2 * (p - s) + 1) / two_o;
    }
    if (i < n - 1) {
      const int32_t s = core_at(i + 1, L, n) - lo;
      if (p >= s && p < s + o) return static_cast<float>(2 * o - 2 * (p - s) - 1) / two_o;
    }
    return 1.0f;
  }
};

struct Geometry {
  DimTiling dim[3];
  int32_t T = 1;
  int64_t N = 0;
  int32_t M = 0;

  void tile_coords(int32_t t, int32_t ii[3]) const {
    ii[2] = t % dim[2].n;
    ii[1] = (t / dim[2].n) % dim[1].n;
    ii[0] = t / (dim[2].n * dim[1].n);
  }
  void tile_box(int32_t t, int32_t a[3], int32_t b[3]) const {
    int32_t ii[3];
    tile_coords(t, ii);
    for (int d = 0; d < 3; ++d) dim[d].box(ii[d], &a[d], &b[d]);
  }
};

tdp_status make_geometry(const tdp_plan_desc *desc, Geometry *g) {
  if (!desc) return TDP_ERR_NULL;
  if (desc->n_cond < 0) return TDP_ERR_ARG;
  if (desc->n_cond > 0 && !desc->cond_pos) return TDP_ERR_NULL;
  if (desc->world_size < 1 || desc->rank < 0 || desc->rank >= desc->world_size)
    return TDP_ERR_ARG;
  if (desc->normalize_positions != 0 && desc->normalize_positions != 1) return TDP_ERR_ARG;
  if (desc->assignment != 0 && desc->assignment != 1) return TDP_ERR_ARG;
  int64_t T = 1, N = 1;
  for (int d = 0; d < 3; ++d) {
    g->dim[d].L = desc->grid[d];
    g->dim[d].n = desc->tiling[d].num_tiles;
    g->dim[d].o = desc->tiling[d].overlap;
    const tdp_status s = g->dim[d].check();
    if (s != TDP_OK) return s;
    T *= g->dim[d].n;
    N *= g->dim[d].L;
  }
  if (T > INT32_MAX || N + desc->n_cond > INT32_MAX) return TDP_ERR_ARG;
  for (int64_t k = 0; k < 6LL * desc->n_cond; ++k) {
    if (!std::isfinite(desc->cond_pos[k])) return TDP_ERR_ARG;
  }
  for (int32_t j = 0; j < desc->n_cond; ++j)
    for (int d = 0; d < 3; ++d)
      if (desc->cond_pos[6 * j + 2 * d + 1] < desc->cond_pos[6 * j + 2 * d]) return TDP_ERR_ARG;
  g->T = static_cast<int32_t>(T);
  g->N = N;
  g->M = desc->n_cond;
  return TDP_OK;
}

// Keep rule ("Shared negative (reference) positions"): a negative time start,
// or a strict half-open overlap with the tile's generated extent [a, b) in all
// three dims (global coordinates).
bool keeps(const float *cp, const int32_t a[3], const int32_t b[3]) {
  if (cp[0] < 0.0f) return true;
  for (int d = 0; d < 3; ++d) {
    const float s = cp[2 * d], e = cp[2 * d + 1];
    if (!(s < static_cast<float>(b[d]) && e > static_cast<float>(a[d]))) return false;
  }
  return true;
}

int64_t box_volume(const int32_t a[3], const int32_t b[3]) {
  return static_cast<int64_t>(b[0] - a[0]) * (b[1] - a[1]) * (b[2] - a[2]);
}

// Rows of tile t: its generated tokens plus the conditioning tokens it keeps.
int64_t tile_rows(const Geometry &g, const tdp_plan_desc *desc, int32_t t) {
  int32_t a[3], b[3];
  g.tile_box(t, a, b);
  int64_t rows = box_volume(a, b);
  for (int32_t j = 0; j < g.M; ++j) rows += keeps(desc->cond_pos + 6 * j, a, b) ? 1 : 0;
  return rows;
}

// The tiles of desc->rank, ascending.  Round robin: t mod world_size == rank
// ("What it is").  Longest first (a balancing alternative the page does not
// give): tiles by cost rows^2 descending, ties by index, each to the rank
// with the least accumulated cost, ties to the lower rank.
std::vector<int32_t> local_tiles(const Geometry &g, const tdp_plan_desc *desc) {
  std::vector<int32_t> mine;
  const int32_t W = desc->world_size;
  if (desc->assignment == 0) {
    for (int32_t t = desc->rank; t < g.T; t += W) mine.push_back(t);
    return mine;
  }
  std::vector<int64_t> cost(g.T);
  std::vector<int32_t> order(g.T);
  for (int32_t t = 0; t < g.T; ++t) {
    const int64_t r = tile_rows(g, desc, t);
    cost[t] = r * r;
    order[t] = t;
  }
  std::stable_sort(order.begin(), order.end(),
                   [&](int32_t x, int32_t y) { return cost[x] > cost[y]; });
  std::vector<int64_t> load(W, 0);
  for (const int32_t t : order) {
    int32_t best = 0;
    for (int32_t r = 1; r < W; ++r)
      if (load[r] < load[best]) best = r;
    load[best] += cost[t];
    if (best == desc->rank) mine.push_back(t);
  }
  std::sort(mine.begin(), mine.end());
  return mine;
}

}  // namespace

extern "C" {

const char *tdp_status_string(int32_t status) {
  switch (status) {
    case TDP_OK: return "ok";
    case TDP_ERR_NULL: return "a required pointer is NULL";
    case TDP_ERR_ARG: return "argument out of range";
    case TDP_ERR_SHAPE: return "sizes disagree";
    case TDP_ERR_UNSUPPORTED: return "unsupported shape or dtype";
    case TDP_ERR_BUFFER: return "buffer or workspace too small";
    case TDP_ERR_HIP: return "HIP runtime error";
    case TDP_ERR_ALIGN: return "device pointer not 16-byte aligned";
    default: return "unknown status";
  }
}

tdp_status tdp_plan_query(const tdp_plan_desc *desc, tdp_plan_sizes *sizes) {
  if (!desc || !sizes) return TDP_ERR_NULL;
  Geometry g;
  const tdp_status s = make_geometry(desc, &g);
  if (s != TDP_OK) return s;
  tdp_plan_sizes out{};
  out.n_tiles_total = g.T;
  out.n_gen_total = static_cast<int32_t>(g.N);
  out.n_dst_rows = g.N + g.M;
  for (const int32_t t : local_tiles(g, desc)) {
    const int64_t rows = tile_rows(g, desc, t);
    if (rows > INT32_MAX) return TDP_ERR_ARG;
    out.n_tiles_local += 1;
    out.max_tile_rows = std::max<int32_t>(out.max_tile_rows, static_cast<int32_t>(rows));
    out.n_rows += rows;
  }
  if (out.n_rows > INT32_MAX) return TDP_ERR_ARG;  // row ids are int32
  *sizes = out;
  return TDP_OK;
}

tdp_status tdp_plan(const tdp_plan_desc *desc, const tdp_plan_sizes *sizes,
                    tdp_plan_out *out) {
  if (!desc || !sizes || !out) return TDP_ERR_NULL;
  tdp_plan_sizes want{};
  const tdp_status s = tdp_plan_query(desc, &want);
  if (s != TDP_OK) return s;
  if (std::memcmp(&want, sizes, sizeof(want)) != 0) return TDP_ERR_SHAPE;
  if (!out->tile_id || !out->tile_box || !out->tile_offset || !out->tile_row_begin ||
      !out->tile_n_gen || !out->row_src || !out->row_weight || !out->row_pos ||
      !out->dst_row_begin || !out->dst_rows || (desc->n_cond > 0 && !out->cond_keep_count))
    return TDP_ERR_NULL;

  Geometry g;
  make_geometry(desc, &g);
  const int32_t F = desc->grid[0], H = desc->grid[1], W = desc->grid[2];
  const float *cp = desc->cond_pos;

  // k_j over every tile of every rank.
  for (int32_t j = 0; j < g.M; ++j) out->cond_keep_count[j] = 0;
  for (int32_t t = 0; t < g.T; ++t) {
    int32_t a[3], b[3];
    g.tile_box(t, a, b);
    for (int32_t j = 0; j < g.M; ++j)
      if (keeps(cp + 6 * j, a, b)) out->cond_keep_count[j] += 1;
  }
  (void)F;

  int64_t row = 0;
  int32_t li = 0;
  std::vector<float> wdim[3];
  for (const int32_t t : local_tiles(g, desc)) {
    int32_t ii[3], a[3], b[3];
    g.tile_coords(t, ii);
    g.tile_box(t, a, b);
    out->tile_id[li] = t;
    float off[3];
    for (int d = 0; d < 3; ++d) {
      out->tile_box[6 * li + 2 * d] = a[d];
      out->tile_box[6 * li + 2 * d + 1] = b[d];
      // smallest start over the tile's generated tokens = its box start
      off[d] = desc->normalize_positions ? static_cast<float>(a[d]) : 0.0f;
      out->tile_offset[3 * li + d] = off[d];
      wdim[d].resize(b[d] - a[d]);
      for (int32_t p = a[d]; p < b[d]; ++p) wdim[d][p - a[d]] = g.dim[d].weight(ii[d], p);
    }
    out->tile_row_begin[li] = row;
    for (int32_t f = a[0]; f < b[0]; ++f) {
      for (int32_t h = a[1]; h < b[1]; ++h) {
        const float wfh = wdim[0][f - a[0]] * wdim[1][h - a[1]];
        for (int32_t w = a[2]; w < b[2]; ++w, ++row) {
          out->row_src[row] = (f * H + h) * W + w;
          out->row_weight[row] = wfh * wdim[2][w - a[2]];
          const int32_t cell[3] = {f, h, w};
          for (int d = 0; d < 3; ++d) {
            const float st = static_cast<float>(cell[d]);
            const float en = st + 1.0f;
            out->row_pos[6 * row + 2 * d] = st - off[d];
            out->row_pos[6 * row + 2 * d + 1] = en - off[d];
          }
        }
      }
    }
    out->tile_n_gen[li] = static_cast<int32_t>(row - out->tile_row_begin[li]);
    for (int32_t j = 0; j < g.M; ++j) {
      if (!keeps(cp + 6 * j, a, b)) continue;
      out->row_src[row] = static_cast<int32_t>(g.N) + j;
      out->row_weight[row] = 1.0f / static_cast<float>(out->cond_keep_count[j]);
      for (int d = 0; d < 3; ++d) {
        out->row_pos[6 * row + 2 * d] = cp[6 * j + 2 * d] - off[d];
        out->row_pos[6 * row + 2 * d + 1] = cp[6 * j + 2 * d + 1] - off[d];
      }
      ++row;
    }
    ++li;
  }
  out->tile_row_begin[li] = row;

  // Inverse map by counting sort: rows of each token in ascending row order,
  // which is ascending tile order.
  const int64_t n_dst = g.N + g.M;
  for (int64_t n = 0; n <= n_dst; ++n) out->dst_row_begin[n] = 0;
  for (int64_t r = 0; r < row; ++r) out->dst_row_begin[out->row_src[r] + 1] += 1;
  for (int64_t n = 0; n < n_dst; ++n) out->dst_row_begin[n + 1] += out->dst_row_begin[n];
  std::vector<int64_t> fill(out->dst_row_begin, out->dst_row_begin + n_dst);
  for (int64_t r = 0; r < row; ++r)
    out->dst_rows[fill[out->row_src[r]]++] = static_cast<int32_t>(r);
  return TDP_OK;
}

tdp_status tdp_balanced_tile_split(int32_t n, int32_t *h_tiles, int32_t *w_tiles) {
  if (!h_tiles || !w_tiles) return TDP_ERR_NULL;
  if (n < 1) return TDP_ERR_ARG;
  // largest h with h * h <= n, then down to the first divisor
  int64_t h = 1;
  while ((h + 1) * (h + 1) <= n) ++h;
  while (n % h != 0) --h;
  *h_tiles = static_cast<int32_t>(h);
  *w_tiles = static_cast<int32_t>(n / h);
  return TDP_OK;
}

// The upscale loop's schedule (TDP page, "When to use it": the upscale stage
// starts from a first sigma; the page names no schedule): linear from sigma0
// to 0 in n_steps steps, each value computed in double and rounded once.
tdp_status tdp_linear_sigmas(float sigma0, int32_t n_steps, float *sigmas) {
  if (!sigmas) return TDP_ERR_NULL;
  if (n_steps < 0 || !(sigma0 >= 0.0f && sigma0 <= 1.0f)) return TDP_ERR_ARG;
  if (n_steps == 0) {
    sigmas[0] = sigma0;
    return TDP_OK;
  }
  const double s0 = sigma0;
  for (int32_t i = 0; i <= n_steps; ++i)
    sigmas[i] = static_cast<float>(s0 * (1.0 - static_cast<double>(i) / n_steps));
  return TDP_OK;
}

}  // extern "C"
