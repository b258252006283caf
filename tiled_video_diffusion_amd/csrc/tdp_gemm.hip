// bf16 GEMM with fused epilogues for gfx950: C = A B, B given as B^T [N][K].
//
// Used by the attention's output projection (A = the head-major attention
// output) and by the per-tile transformer block (projections, FFN, timestep
// MLP).  One workgroup = 256 rows (8 waves x 32) and 128 columns; each wave
// owns 32 rows x 128 columns (four 32x32 MFMA tiles).  Each 64-wide k chunk
// of A (32 KB) and of B^T (16 KB) goes global -> LDS by direct loads, one
// 128-byte row segment per 8 lanes, into a 3-stage ring, so a chunk has two
// chunk-times to arrive while the MFMAs work on the one before.  LDS rows are
// 128 bytes, 16-byte piece p of row r at slot p ^ ((r / 2) % 8): the 16 lanes
// of a fragment read phase (16 consecutive rows, one piece) hit 16 distinct
// slots of a 256-byte bank window.
#include "tdp_internal.h"

namespace tdp {
namespace {

typedef __attribute__((address_space(1))) void gvoid_t;
typedef __attribute__((address_space(3))) void lvoid_t;

constexpr int kGWaves = 8;
constexpr int kGThreads = 64 * kGWaves;
constexpr int kGRows = 32 * kGWaves;   // rows per workgroup
constexpr int kGCols = 128;            // columns per workgroup
constexpr int kGK = 64;                // k per chunk
constexpr int kGALoads = kGRows * kGK * 2 / 1024 / kGWaves;   // 1 KB A loads per wave
constexpr int kGBLoads = kGCols * kGK * 2 / 1024 / kGWaves;   // 1 KB B^T loads per wave

__host__ __device__ inline int64_t cdiv(int64_t a, int64_t b) { return (a + b - 1) / b; }

__device__ __forceinline__ int g_slot(int r, int piece) { return piece ^ ((r >> 1) & 7); }

constexpr float kLog2e = 1.4426950408889634f;
// tanh-form GELU via 0.5 (1 + tanh z) = 1 / (1 + exp(-2 z)), z = sqrt(2/pi) (u + 0.044715 u^3).
__device__ __forceinline__ float gelu_tanh(float u) {
  const float z = 0.7978845608028654f * (u + 0.044715f * u * u * u);
  return u / (1.0f + __builtin_amdgcn_exp2f(-2.0f * kLog2e * z));
}
// u sigmoid(u)
__device__ __forceinline__ float silu(float u) {
  return u / (1.0f + __builtin_amdgcn_exp2f(-kLog2e * u));
}

struct GemmArgs {
  const bf16 *a;
  int64_t lda, a_seg_rows;
  int32_t a_heads;
  const bf16 *bt;
  int64_t ldb, M;
  int32_t N, K;
  void *c;
  int64_t ldc;
  const float *g0;
  int64_t g0_stride;
  const float *g1;
  int64_t rows_per_batch;
};

// HD = 0: row-major A; HD = 64 / 128: head-major A with that head size.
template <int EPI, int HD>
__global__ __launch_bounds__(kGThreads, 1) void gemm_kernel(GemmArgs g) {
  static_assert(HD % kGK == 0, "whole k chunks per head");
  __shared__ __attribute__((aligned(16))) bf16 sA0[kGRows * kGK], sA1[kGRows * kGK],
      sA2[kGRows * kGK];
  __shared__ __attribute__((aligned(16))) bf16 sB0[kGCols * kGK], sB1[kGCols * kGK],
      sB2[kGCols * kGK];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int l32 = lane & 31, hh = lane >> 5;
  const int uwave = __builtin_amdgcn_readfirstlane(wave);
  const int64_t row0 = static_cast<int64_t>(blockIdx.x) * kGRows;
  const int64_t col0 = static_cast<int64_t>(blockIdx.y) * kGCols;
  const int64_t M = g.M;

  // Per-lane byte offsets of the direct loads (k chunk 0); LDS position
  // (r, slot) holds piece slot ^ ((r / 2) % 8) of row r.  Rows past M re-read
  // row M - 1 (their results are not stored).
  uint64_t aoff[kGALoads];
  uint64_t boff[kGBLoads];
#pragma unroll
  for (int i = 0; i < kGALoads; ++i) {
    const int pos = (i * kGWaves + uwave) * 64 + lane;   // 16-byte position in the tile
    const int r = pos / 8, slot = pos % 8;
    const int64_t gr = min(row0 + r, M - 1);
    int64_t el;
    if constexpr (HD > 0) {
      const int64_t L = g.a_seg_rows;
      const int64_t seg = gr / L;
      el = (seg * g.a_heads * L + (gr - seg * L)) * HD;
    } else {
      el = gr * g.lda;
    }
    aoff[i] = static_cast<uint64_t>(el * 2 + 16 * g_slot(r, slot));
  }
#pragma unroll
  for (int i = 0; i < kGBLoads; ++i) {
    const int pos = (i * kGWaves + uwave) * 64 + lane;
    const int r = pos / 8, slot = pos % 8;
    boff[i] = static_cast<uint64_t>((col0 + r) * g.ldb * 2 + 16 * g_slot(r, slot));
  }
  const char *abase = reinterpret_cast<const char *>(g.a);
  const char *bbase = reinterpret_cast<const char *>(g.bt);
  auto load_chunk = [&](int c, bf16 *sa, bf16 *sb) __attribute__((always_inline)) {
    const int64_t kb = static_cast<int64_t>(c) * kGK * 2;   // B^T (and row-major A): k = 64 c
    int64_t ab = kb;
    if constexpr (HD > 0) {
      constexpr int kPerHead = HD / kGK;
      const int h = c / kPerHead;
      ab = (static_cast<int64_t>(h) * g.a_seg_rows * HD + (c - h * kPerHead) * kGK) * 2;
    }
#pragma unroll
    for (int i = 0; i < kGALoads; ++i)
      __builtin_amdgcn_global_load_lds((gvoid_t *)(abase + ab + aoff[i]),
                                       (lvoid_t *)(sa + (i * kGWaves + uwave) * 512), 16, 0, 0);
#pragma unroll
    for (int i = 0; i < kGBLoads; ++i)
      __builtin_amdgcn_global_load_lds((gvoid_t *)(bbase + kb + boff[i]),
                                       (lvoid_t *)(sb + (i * kGWaves + uwave) * 512), 16, 0, 0);
  };
  // fragment offsets (elements): A row wave*32 + l32, B^T row 32 ct + l32;
  // piece 2 ks + hh
  const int ar = wave * 32 + l32;
  int32_t afo[kGK / 16], bfo[4][kGK / 16];
#pragma unroll
  for (int ks = 0; ks < kGK / 16; ++ks) {
    afo[ks] = ar * kGK + 8 * g_slot(ar, 2 * ks + hh);
#pragma unroll
    for (int ct = 0; ct < 4; ++ct) {
      const int br = 32 * ct + l32;
      bfo[ct][ks] = br * kGK + 8 * g_slot(br, 2 * ks + hh);
    }
  }
  f32x16 acc[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) acc[i] = f32x16{};
  auto compute = [&](const bf16 *sa, const bf16 *sb) __attribute__((always_inline)) {
#pragma unroll
    for (int ks = 0; ks < kGK / 16; ++ks) {
      const bf16x8 af = *reinterpret_cast<const bf16x8 *>(sa + afo[ks]);
#pragma unroll
      for (int ct = 0; ct < 4; ++ct) {
        const bf16x8 bfr = *reinterpret_cast<const bf16x8 *>(sb + bfo[ct][ks]);
        acc[ct] = mfma32(af, bfr, acc[ct]);
      }
    }
  };
  constexpr int kPer = kGALoads + kGBLoads;   // loads per wave per chunk
  static_assert(kPer == 6, "vmcnt below counts 6 loads per chunk");
  const int nc = g.K / kGK;
  load_chunk(0, sA0, sB0);
  if (nc > 1) load_chunk(1, sA1, sB1);
  if (nc > 1) asm volatile("s_waitcnt vmcnt(6)" ::: "memory");
  else asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  __syncthreads();
  // Step c: load chunk c+2 into the ring slot of chunk c-1, compute chunk c,
  // wait for chunk c+1, barrier.  Loads past the last chunk re-read chunk
  // nc-1 (in range; never used) so every step waits on the same count.
  auto step = [&](int c, bf16 *ln_a, bf16 *ln_b, const bf16 *ca, const bf16 *cb)
      __attribute__((always_inline)) {
    load_chunk(min(c + 2, nc - 1), ln_a, ln_b);
    compute(ca, cb);
    asm volatile("s_waitcnt vmcnt(6)" ::: "memory");
    __syncthreads();
  };
  int c = 0;
  for (; c + 3 <= nc; c += 3) {
    step(c, sA2, sB2, sA0, sB0);
    step(c + 1, sA0, sB0, sA1, sB1);
    step(c + 2, sA1, sB1, sA2, sB2);
  }
  if (c < nc) step(c, sA2, sB2, sA0, sB0);
  if (c + 1 < nc) step(c + 1, sA0, sB0, sA1, sB1);
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");

  // acc[ct][v]: row 8 (v/4) + 4 hh + v%4 of the wave's 32, column 32 ct + l32
  const int64_t base = row0 + wave * 32;
#pragma unroll
  for (int v = 0; v < 16; ++v) {
    const int64_t r = base + 8 * (v / 4) + 4 * hh + (v % 4);
    if (r >= M) continue;
    float gb[4] = {0.f, 0.f, 0.f, 0.f};
    if constexpr (EPI == kEpiResidGate) {
      const int64_t b = r / g.rows_per_batch;
#pragma unroll
      for (int ct = 0; ct < 4; ++ct) {
        const int64_t n = col0 + 32 * ct + l32;
        gb[ct] = (g.g0 ? g.g0[b * g.g0_stride + n] : 0.f) + (g.g1 ? g.g1[n] : 0.f);
      }
    }
#pragma unroll
    for (int ct = 0; ct < 4; ++ct) {
      const int64_t idx = r * g.ldc + col0 + 32 * ct + l32;
      const float x = acc[ct][v];
      if constexpr (EPI == kEpiBf16) static_cast<bf16 *>(g.c)[idx] = static_cast<bf16>(x);
      if constexpr (EPI == kEpiF32) static_cast<float *>(g.c)[idx] = x;
      if constexpr (EPI == kEpiGeluBf16) static_cast<bf16 *>(g.c)[idx] = static_cast<bf16>(gelu_tanh(x));
      if constexpr (EPI == kEpiSiluBf16) static_cast<bf16 *>(g.c)[idx] = static_cast<bf16>(silu(x));
      if constexpr (EPI == kEpiResid) static_cast<float *>(g.c)[idx] += x;
      if constexpr (EPI == kEpiResidGate) static_cast<float *>(g.c)[idx] += gb[ct] * x;
    }
  }
}

// Wide form for large GEMMs: one workgroup = 256 rows x 256
// columns, 8 waves as 4 (rows) x 2 (columns), each wave 64 x 128 (2 x 4
// MFMA tiles).  A fragment read from LDS feeds 4 MFMAs and a B^T fragment 2
// (0.75 reads per MFMA against 1.25 above), and the operand bytes per MFMA
// drop by a third.  64-wide k chunks of A and B^T (32 KB each) in two LDS
// stages.
constexpr int kWRows = 256, kWCols = 256;
// Tile order of the wide form: consecutive workgroup ids go to the 8 XCDs in
// turn; the id is remapped so each XCD walks a contiguous range of tiles,
// taken TDP_GEMM_GROUP_M row blocks at a time down a column of tiles (the
// workgroups that run together on one XCD then share their A and B^T tiles
// in its L2).  0: the plain order, row blocks first.
#ifndef TDP_GEMM_GROUP_M
#define TDP_GEMM_GROUP_M 4
#endif
constexpr int kWALoads = kWRows * kGK * 2 / 1024 / kGWaves;   // 4
constexpr int kWBLoads = kWCols * kGK * 2 / 1024 / kGWaves;   // 4

template <int EPI, int HD>
__global__ __launch_bounds__(kGThreads, 1) void gemm_wide_kernel(GemmArgs g) {
  static_assert(HD % kGK == 0, "whole k chunks per head");
  __shared__ __attribute__((aligned(16))) bf16 sA0[kWRows * kGK], sA1[kWRows * kGK];
  __shared__ __attribute__((aligned(16))) bf16 sB0[kWCols * kGK], sB1[kWCols * kGK];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int l32 = lane & 31, hh = lane >> 5;
  const int uwave = __builtin_amdgcn_readfirstlane(wave);
  const int wm = wave & 3, wn = wave >> 2;
  const int64_t M = g.M;
  const int64_t nm = cdiv(M, kWRows), nn = g.N / kWCols;
  int64_t tm, tn;
  if constexpr (TDP_GEMM_GROUP_M > 0) {
    const int64_t G = gridDim.x;   // a multiple of 8, >= nm * nn
    const int64_t bid = blockIdx.x;
    const int64_t lid = (bid % 8) * (G / 8) + bid / 8;
    if (lid >= nm * nn) return;
    const int64_t per_group = static_cast<int64_t>(TDP_GEMM_GROUP_M) * nn;
    const int64_t grp = lid / per_group;
    const int64_t first_m = grp * TDP_GEMM_GROUP_M;
    const int64_t gm = min(static_cast<int64_t>(TDP_GEMM_GROUP_M), nm - first_m);
    const int64_t in = lid - grp * per_group;
    tm = first_m + in % gm;
    tn = in / gm;
  } else {
    tm = blockIdx.x;
    tn = blockIdx.y;
  }
  const int64_t row0 = tm * kWRows;
  const int64_t col0 = tn * kWCols;
  uint64_t aoff[kWALoads], boff[kWBLoads];
#pragma unroll
  for (int i = 0; i < kWALoads; ++i) {
    const int pos = (i * kGWaves + uwave) * 64 + lane;
    const int r = pos / 8, slot = pos % 8;
    const int64_t gr = min(row0 + r, M - 1);
    int64_t el;
    if constexpr (HD > 0) {
      const int64_t L = g.a_seg_rows;
      const int64_t seg = gr / L;
      el = (seg * g.a_heads * L + (gr - seg * L)) * HD;
    } else {
      el = gr * g.lda;
    }
    aoff[i] = static_cast<uint64_t>(el * 2 + 16 * g_slot(r, slot));
  }
#pragma unroll
  for (int i = 0; i < kWBLoads; ++i) {
    const int pos = (i * kGWaves + uwave) * 64 + lane;
    const int r = pos / 8, slot = pos % 8;
    boff[i] = static_cast<uint64_t>((col0 + r) * g.ldb * 2 + 16 * g_slot(r, slot));
  }
  const char *abase = reinterpret_cast<const char *>(g.a);
  const char *bbase = reinterpret_cast<const char *>(g.bt);
  auto load_chunk = [&](int c, bf16 *sa, bf16 *sb) __attribute__((always_inline)) {
    const int64_t kb = static_cast<int64_t>(c) * kGK * 2;
    int64_t ab = kb;
    if constexpr (HD > 0) {
      constexpr int kPerHead = HD / kGK;
      const int h = c / kPerHead;
      ab = (static_cast<int64_t>(h) * g.a_seg_rows * HD + (c - h * kPerHead) * kGK) * 2;
    }
#pragma unroll
    for (int i = 0; i < kWALoads; ++i)
      __builtin_amdgcn_global_load_lds((gvoid_t *)(abase + ab + aoff[i]),
                                       (lvoid_t *)(sa + (i * kGWaves + uwave) * 512), 16, 0, 0);
#pragma unroll
    for (int i = 0; i < kWBLoads; ++i)
      __builtin_amdgcn_global_load_lds((gvoid_t *)(bbase + kb + boff[i]),
                                       (lvoid_t *)(sb + (i * kGWaves + uwave) * 512), 16, 0, 0);
  };
  int32_t afo[2][kGK / 16], bfo[4][kGK / 16];
#pragma unroll
  for (int ks = 0; ks < kGK / 16; ++ks) {
#pragma unroll
    for (int mt = 0; mt < 2; ++mt) {
      const int ar = 64 * wm + 32 * mt + l32;
      afo[mt][ks] = ar * kGK + 8 * g_slot(ar, 2 * ks + hh);
    }
#pragma unroll
    for (int ct = 0; ct < 4; ++ct) {
      const int br = 128 * wn + 32 * ct + l32;
      bfo[ct][ks] = br * kGK + 8 * g_slot(br, 2 * ks + hh);
    }
  }
  f32x16 acc[2][4];
#pragma unroll
  for (int mt = 0; mt < 2; ++mt)
#pragma unroll
    for (int ct = 0; ct < 4; ++ct) acc[mt][ct] = f32x16{};
  auto compute = [&](const bf16 *sa, const bf16 *sb) __attribute__((always_inline)) {
#pragma unroll
    for (int ks = 0; ks < kGK / 16; ++ks) {
      const bf16x8 a0 = *reinterpret_cast<const bf16x8 *>(sa + afo[0][ks]);
      const bf16x8 a1 = *reinterpret_cast<const bf16x8 *>(sa + afo[1][ks]);
#pragma unroll
      for (int ct = 0; ct < 4; ++ct) {
        const bf16x8 bfr = *reinterpret_cast<const bf16x8 *>(sb + bfo[ct][ks]);
        acc[0][ct] = mfma32(a0, bfr, acc[0][ct]);
        acc[1][ct] = mfma32(a1, bfr, acc[1][ct]);
      }
    }
  };
  const int nc = g.K / kGK;
  load_chunk(0, sA0, sB0);
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  __syncthreads();
  // Step c: load chunk c+1 into the other stage (last read in step c-1),
  // compute chunk c, wait for the loads, barrier.
  int c = 0;
  for (; c + 2 <= nc; c += 2) {
    load_chunk(c + 1, sA1, sB1);
    compute(sA0, sB0);
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();
    if (c + 2 < nc) load_chunk(c + 2, sA0, sB0);
    compute(sA1, sB1);
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();
  }
  if (c < nc) compute(sA0, sB0);

  // acc[mt][ct][v]: row 64 wm + 32 mt + 8 (v/4) + 4 hh + v%4, column
  // 128 wn + 32 ct + l32
#pragma unroll
  for (int mt = 0; mt < 2; ++mt) {
    const int64_t base = row0 + 64 * wm + 32 * mt;
#pragma unroll
    for (int v = 0; v < 16; ++v) {
      const int64_t r = base + 8 * (v / 4) + 4 * hh + (v % 4);
      if (r >= M) continue;
      float gb[4] = {0.f, 0.f, 0.f, 0.f};
      if constexpr (EPI == kEpiResidGate) {
        const int64_t b = r / g.rows_per_batch;
#pragma unroll
        for (int ct = 0; ct < 4; ++ct) {
          const int64_t n = col0 + 128 * wn + 32 * ct + l32;
          gb[ct] = (g.g0 ? g.g0[b * g.g0_stride + n] : 0.f) + (g.g1 ? g.g1[n] : 0.f);
        }
      }
#pragma unroll
      for (int ct = 0; ct < 4; ++ct) {
        const int64_t idx = r * g.ldc + col0 + 128 * wn + 32 * ct + l32;
        const float x = acc[mt][ct][v];
        if constexpr (EPI == kEpiBf16) static_cast<bf16 *>(g.c)[idx] = static_cast<bf16>(x);
        if constexpr (EPI == kEpiF32) static_cast<float *>(g.c)[idx] = x;
        if constexpr (EPI == kEpiGeluBf16) static_cast<bf16 *>(g.c)[idx] = static_cast<bf16>(gelu_tanh(x));
        if constexpr (EPI == kEpiSiluBf16) static_cast<bf16 *>(g.c)[idx] = static_cast<bf16>(silu(x));
        if constexpr (EPI == kEpiResid) static_cast<float *>(g.c)[idx] += x;
        if constexpr (EPI == kEpiResidGate) static_cast<float *>(g.c)[idx] += gb[ct] * x;
      }
    }
  }
}

#ifndef TDP_GEMM_WIDE
#define TDP_GEMM_WIDE 1
#endif

template <int EPI>
tdp_status launch_epi(const GemmArgs &a, int hd, dim3 grid, hipStream_t stream) {
  // the wide form for a multiple of 256 columns and enough rows
  if (TDP_GEMM_WIDE && a.N % kWCols == 0 && a.M >= 8 * kWRows) {
    const int64_t nm = cdiv(a.M, kWRows), nn = a.N / kWCols;
    const dim3 wgrid = TDP_GEMM_GROUP_M > 0
                           ? dim3(static_cast<uint32_t>(cdiv(nm * nn, 8) * 8))
                           : dim3(static_cast<uint32_t>(nm), static_cast<uint32_t>(nn));
    if (hd == 0)
      hipLaunchKernelGGL((gemm_wide_kernel<EPI, 0>), wgrid, dim3(kGThreads), 0, stream, a);
    else if (hd == 64)
      hipLaunchKernelGGL((gemm_wide_kernel<EPI, 64>), wgrid, dim3(kGThreads), 0, stream, a);
    else
      hipLaunchKernelGGL((gemm_wide_kernel<EPI, 128>), wgrid, dim3(kGThreads), 0, stream, a);
    return launch_status();
  }
  if (hd == 0)
    hipLaunchKernelGGL((gemm_kernel<EPI, 0>), grid, dim3(kGThreads), 0, stream, a);
  else if (hd == 64)
    hipLaunchKernelGGL((gemm_kernel<EPI, 64>), grid, dim3(kGThreads), 0, stream, a);
  else
    hipLaunchKernelGGL((gemm_kernel<EPI, 128>), grid, dim3(kGThreads), 0, stream, a);
  return launch_status();
}

}  // namespace

tdp_status gemm(int epi, const GemmDesc &d, hipStream_t stream) {
  if (!d.a || !d.bt || !d.c) return TDP_ERR_NULL;
  if (d.M < 1 || d.N < kGCols || d.N % kGCols != 0 || d.K < kGK || d.K % kGK != 0)
    return TDP_ERR_UNSUPPORTED;
  if (d.a_head_dim != 0) {
    if ((d.a_head_dim != 64 && d.a_head_dim != 128) || d.a_seg_rows < 1 || d.a_heads < 1 ||
        static_cast<int64_t>(d.a_heads) * d.a_head_dim != d.K)
      return TDP_ERR_UNSUPPORTED;
  } else if (d.lda < d.K || d.lda % 8 != 0) {
    return TDP_ERR_UNSUPPORTED;
  }
  if (d.ldb < d.K || d.ldb % 8 != 0 || d.ldc < d.N) return TDP_ERR_UNSUPPORTED;
  if (epi == kEpiResidGate && d.rows_per_batch < 1) return TDP_ERR_ARG;
  if (cdiv(d.M, kGRows) > INT32_MAX) return TDP_ERR_UNSUPPORTED;
  GemmArgs a{d.a, d.lda, d.a_seg_rows, d.a_heads, d.bt, d.ldb, d.M, d.N, d.K, d.c, d.ldc,
             d.g0, d.g0_stride, d.g1, d.rows_per_batch};
  const dim3 grid(static_cast<uint32_t>(cdiv(d.M, kGRows)), static_cast<uint32_t>(d.N / kGCols));
  switch (epi) {
    case kEpiBf16: return launch_epi<kEpiBf16>(a, d.a_head_dim, grid, stream);
    case kEpiF32: return launch_epi<kEpiF32>(a, d.a_head_dim, grid, stream);
    case kEpiGeluBf16: return launch_epi<kEpiGeluBf16>(a, d.a_head_dim, grid, stream);
    case kEpiSiluBf16: return launch_epi<kEpiSiluBf16>(a, d.a_head_dim, grid, stream);
    case kEpiResid: return launch_epi<kEpiResid>(a, d.a_head_dim, grid, stream);
    case kEpiResidGate: return launch_epi<kEpiResidGate>(a, d.a_head_dim, grid, stream);
    default: return TDP_ERR_ARG;
  }
}

}  // namespace tdp
