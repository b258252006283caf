// Host plan under AddressSanitizer and UndefinedBehaviorSanitizer: random
// valid and invalid descriptors through tdp_plan_query / tdp_plan (every
// output array sized exactly as the query says, so any write past an array
// is reported), the host helpers, and the plan's invariants:
//   - the row CSR starts at 0, never decreases, ends at n_rows;
//   - every row's source token is in range, and every row feeds exactly one
//     entry of the inverse map, which lists the token's rows;
//   - weights lie in (0, 1]; with one rank, the weights feeding every
//     generated token sum to 1 (the page's masks sum to one) and those of a
//     kept conditioning token sum to 1 (1/k over its k tiles);
//   - the sizes handed to tdp_plan must be the query's (TDP_ERR_SHAPE), and
//     every output array is required (TDP_ERR_NULL).
// Usage: plan_fuzz ITERATIONS SEED.  Prints "ok VALID INVALID", exit 0.
#include <algorithm>
#include <cmath>
#include <cstdio>
#include <cstdlib>
#include <random>
#include <vector>

#include "tdp.h"

namespace {

std::mt19937_64 rng;

int uni(int lo, int hi) { return std::uniform_int_distribution<int>(lo, hi)(rng); }
bool coin(double p) { return std::uniform_real_distribution<double>(0, 1)(rng) < p; }

int fail(const char *what, int it) {
  std::printf("FAIL iteration %d: %s\n", it, what);
  return 1;
}

// Every output array is a separate heap block of exactly the queried size
// (new T[n] is non-null and distinct even for n = 0, so a rank with no rows
// still passes real pointers, and any access past n is reported).
template <typename T>
struct Buf {
  T *p;
  explicit Buf(size_t n) : p(new T[n]()) {}
  ~Buf() { delete[] p; }
  Buf(const Buf &) = delete;
  Buf &operator=(const Buf &) = delete;
  T &operator[](size_t i) { return p[i]; }
};

struct Arrays {
  Buf<int32_t> tile_id, tile_box, tile_n_gen, row_src, cond_keep_count, dst_rows;
  Buf<float> tile_offset, row_weight, row_pos;
  Buf<int64_t> tile_row_begin, dst_row_begin;
  tdp_plan_out out{};
  Arrays(const tdp_plan_sizes &s, int32_t m)
      : tile_id(s.n_tiles_local), tile_box(6 * static_cast<size_t>(s.n_tiles_local)),
        tile_n_gen(s.n_tiles_local), row_src(s.n_rows), cond_keep_count(m > 0 ? m : 0),
        dst_rows(s.n_rows), tile_offset(3 * static_cast<size_t>(s.n_tiles_local)),
        row_weight(s.n_rows), row_pos(6 * static_cast<size_t>(s.n_rows)),
        tile_row_begin(static_cast<size_t>(s.n_tiles_local) + 1),
        dst_row_begin(static_cast<size_t>(s.n_dst_rows) + 1) {
    out = {tile_id.p, tile_box.p, tile_offset.p, tile_row_begin.p, tile_n_gen.p, row_src.p,
           row_weight.p, row_pos.p, cond_keep_count.p, dst_row_begin.p, dst_rows.p};
  }
};

}  // namespace

int main(int argc, char **argv) {
  const int iters = argc > 1 ? std::atoi(argv[1]) : 1000;
  rng.seed(argc > 2 ? std::strtoull(argv[2], nullptr, 10) : 1);
  int valid = 0, invalid = 0;
  for (int it = 0; it < iters; ++it) {
    tdp_plan_desc d{};
    for (int k = 0; k < 3; ++k) {
      const int L = uni(1, k == 0 ? 12 : 40);
      const int n = coin(0.03) ? L + 1 : uni(1, std::min(6, L));
      const int core = L / n;               // shortest core length (cores are floor/ceil)
      d.grid[k] = coin(0.03) ? uni(-2, 0) : L;
      d.tiling[k].num_tiles = coin(0.03) ? uni(-1, 0) : n;
      d.tiling[k].overlap = coin(0.05) ? uni(-3, -1)
                                       : (coin(0.1) ? core + uni(1, 4) : uni(0, core));
    }
    const int32_t m = coin(0.02) ? -1 : uni(0, 12);
    d.n_cond = m;
    std::vector<float> cond(m > 0 ? 6 * m : 0);
    for (int j = 0; j < m; ++j)
      for (int k = 0; k < 3; ++k) {
        const int L = d.grid[k] > 0 ? d.grid[k] : 4;
        float s = static_cast<float>(uni(k == 0 ? -4 : 0, L - 1)) + (coin(0.2) ? 0.5f : 0.f);
        float e = s + static_cast<float>(uni(0, 4));
        if (coin(0.01)) s = NAN;
        cond[6 * j + 2 * k] = s;
        cond[6 * j + 2 * k + 1] = e;
      }
    d.cond_pos = (m > 0 && !coin(0.02)) ? cond.data() : nullptr;
    d.normalize_positions = coin(0.02) ? 2 : uni(0, 1);
    d.world_size = coin(0.03) ? 0 : uni(1, 5);
    d.rank = coin(0.03) ? d.world_size : uni(0, d.world_size > 0 ? d.world_size - 1 : 0);
    d.assignment = coin(0.03) ? 2 : uni(0, 1);

    tdp_plan_sizes s{};
    if (tdp_plan_query(&d, &s) != TDP_OK) {
      ++invalid;
      continue;
    }
    ++valid;
    if (s.n_tiles_local < 0 || s.n_rows < 0 || s.n_dst_rows < s.n_gen_total)
      return fail("sizes", it);
    Arrays a(s, m);
    if (tdp_plan(&d, &s, &a.out) != TDP_OK) return fail("tdp_plan after a good query", it);
    // invariants
    const int64_t R = s.n_rows, nd = s.n_dst_rows;
    if (a.tile_row_begin[0] != 0 || a.tile_row_begin[s.n_tiles_local] != R)
      return fail("row CSR ends", it);
    for (int t = 0; t < s.n_tiles_local; ++t)
      if (a.tile_row_begin[t + 1] < a.tile_row_begin[t]) return fail("row CSR order", it);
    std::vector<int> seen(static_cast<size_t>(R), 0);
    if (a.dst_row_begin[0] != 0 || a.dst_row_begin[nd] != R) return fail("inverse CSR ends", it);
    for (int64_t n = 0; n < nd; ++n) {
      if (a.dst_row_begin[n + 1] < a.dst_row_begin[n]) return fail("inverse CSR order", it);
      double wsum = 0.0;
      for (int64_t k = a.dst_row_begin[n]; k < a.dst_row_begin[n + 1]; ++k) {
        const int32_t r = a.dst_rows[k];
        if (r < 0 || r >= R) return fail("inverse row id", it);
        if (a.row_src[r] != n) return fail("inverse map names the wrong token", it);
        ++seen[r];
        wsum += a.row_weight[r];
      }
      const bool covered = a.dst_row_begin[n + 1] > a.dst_row_begin[n];
      if (d.world_size == 1 && covered && std::fabs(wsum - 1.0) > 1e-5)
        return fail("weights of a token do not sum to 1", it);
      if (d.world_size == 1 && n < s.n_gen_total && !covered)
        return fail("a generated token no tile covers", it);
    }
    for (int64_t r = 0; r < R; ++r) {
      if (seen[r] != 1) return fail("a row not in the inverse map exactly once", it);
      if (!(a.row_weight[r] > 0.f && a.row_weight[r] <= 1.f)) return fail("weight range", it);
    }
    // sizes that are not the query's, and a missing array
    tdp_plan_sizes bad = s;
    bad.n_rows += 1;
    if (tdp_plan(&d, &bad, &a.out) != TDP_ERR_SHAPE) return fail("shape check", it);
    tdp_plan_out none = a.out;
    none.dst_rows = nullptr;
    if (tdp_plan(&d, &s, &none) != TDP_ERR_NULL) return fail("null check", it);
  }
  // host helpers
  for (int it = 0; it < iters; ++it) {
    int32_t h = 0, w = 0;
    const int32_t n = uni(-3, 5000);
    const tdp_status st = tdp_balanced_tile_split(n, &h, &w);
    if (n < 1 ? st != TDP_ERR_ARG : (st != TDP_OK || h * w != n || h > w))
      return fail("balanced split", it);
    const int32_t steps = uni(-2, 64);
    std::vector<float> sig(steps > 0 ? steps + 1 : 1);
    const float s0 = coin(0.1) ? 1.5f : static_cast<float>(uni(0, 100)) / 100.f;
    const tdp_status ss = tdp_linear_sigmas(s0, steps, sig.data());
    if ((steps < 0 || s0 > 1.f) ? ss != TDP_ERR_ARG : ss != TDP_OK) return fail("sigmas", it);
  }
  for (int c = -10; c <= 3; ++c)
    if (!tdp_status_string(c)) return fail("status string", c);
  if (valid == 0 || invalid == 0) return fail("fuzzer drew no valid or no invalid descriptor", 0);
  std::printf("ok %d %d\n", valid, invalid);
  return 0;
}
