// bf16 GEMM with fused epilogues for gfx950: C = A B, B given as B^T [N][K].
//
// Used by the attention's output projection (A = the head-major attention
// output) and by the per-tile transformer block (projections, FFN, timestep
// MLP).  Three forms: the narrow one below (N a multiple of 128, small M),
// the wide one, and the large one (the big products), further down.
//
// Narrow form: one workgroup = 256 rows (8 waves x 32) and 128 columns; each wave
// owns 32 rows x 128 columns (four 32x32 MFMA tiles).  Each 64-wide k chunk
// of A (32 KB) and of B^T (16 KB) goes global -> LDS by direct loads, one
// 128-byte row segment per 8 lanes, into a 3-stage ring, so a chunk has two
// chunk-times to arrive while the MFMAs work on the one before.  LDS rows are
// 128 bytes, 16-byte piece p of row r at slot p ^ ((r / 2) % 8): the 16 lanes
// of a fragment read phase (16 consecutive rows, one piece) hit 16 distinct
// slots of a 256-byte bank window.
#include "tdp_internal.h"

#include <algorithm>
#include <atomic>

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
// The exponent -2 z log2(e) is u (c0 + c1 u^2): a multiply, an fma and a
// multiply (written out literally it took five multiplies and an fma; FFN up
// 13.47 -> 13.28 ms).  The quotient uses the hardware reciprocal (about 1
// ulp, far below the bf16 rounding of the result); for very negative u,
// exp2 -> inf and the reciprocal -> 0.
__device__ __forceinline__ float gelu_tanh(float u) {
  constexpr float c0 = -2.0f * kLog2e * 0.7978845608028654f;
  constexpr float c1 = c0 * 0.044715f;
  const float y = u * fmaf(u * u, c1, c0);
  return u * __builtin_amdgcn_rcpf(1.0f + __builtin_amdgcn_exp2f(y));
}
// u sigmoid(u)
__device__ __forceinline__ float silu(float u) {
  return u * __builtin_amdgcn_rcpf(1.0f + __builtin_amdgcn_exp2f(-kLog2e * u));
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
  int32_t group_m;        // 64-wide large form: row blocks per tile-order group
  // 64-wide large form: tiles per XCD taken in order, then a tail of tiles
  // claimed from *tail_ctr (tail_claims claims per launch; 0: no tail)
  int64_t per_xcd;
  uint32_t *tail_ctr;
  uint32_t tail_claims;
};

// Workgroup barrier ordering LDS only (the direct loads are waited for with
// an explicit vmcnt before it; a plain __syncthreads would also wait for every
// load still in flight).
__device__ __forceinline__ void lds_barrier() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}


typedef int i32x4 __attribute__((ext_vector_type(4)));

// Buffer descriptor of `bytes` bytes at `base` (wave-uniform): raw, stride 0,
// the gfx9 data-format word.
__device__ __forceinline__ i32x4 buffer_rsrc(const void *base, uint32_t bytes) {
  const uint64_t a = reinterpret_cast<uint64_t>(base);
  i32x4 r;
  r[0] = __builtin_amdgcn_readfirstlane(static_cast<int>(a & 0xffffffffu));
  r[1] = __builtin_amdgcn_readfirstlane(static_cast<int>((a >> 32) & 0xffffu));
  r[2] = __builtin_amdgcn_readfirstlane(static_cast<int>(bytes));
  r[3] = 0x00020000;
  return r;
}

// 16 bytes per lane from descriptor offset voff + soff into LDS: the wave's
// 64 lanes fill the 1 KB at `lds` (wave-uniform) in lane order.
__device__ __forceinline__ void load_lds16(i32x4 rsrc, uint32_t voff, uint32_t soff,
                                           const bf16 *lds) {
  const uint32_t m0 = static_cast<uint32_t>(
      reinterpret_cast<uintptr_t>((__attribute__((address_space(3))) const bf16 *)lds));
  asm volatile("buffer_load_dwordx4 %0, %1, %2 offen lds"
               :
               : "v"(voff), "s"(rsrc), "s"(soff), "{m0}"(m0)
               : "memory");
}


// HD = 0: row-major A; HD = 64 / 128: head-major A with that head size.
// ASM: the direct loads are buffer loads into LDS written in inline assembly,
// which the compiler does not track; with the builtin (FLAT) form it waits
// for every direct load in flight, the ring's later chunks included, before
// the first fragment read of each step, so no load gets more than one step
// to land.  The launcher takes the builtin form only when a workgroup's A
// offsets do not fit the descriptors' 32 bits.
template <int EPI, int HD, bool ASM = true>
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
  // row M - 1 (their results are not stored).  With ASM they are relative to
  // the workgroup's first row (A) and first column (B^T), the bases of the
  // two descriptors, and a chunk's k offset is the scalar offset.
  auto a_elem = [&](int64_t gr) __attribute__((always_inline)) {
    if constexpr (HD > 0) {
      const int64_t L = g.a_seg_rows;
      const int64_t seg = gr / L;
      return (seg * g.a_heads * L + (gr - seg * L)) * HD;
    } else {
      return gr * g.lda;
    }
  };
  const int64_t ael0 = ASM ? a_elem(min(row0, M - 1)) : 0;
  const int64_t bel0 = ASM ? col0 * g.ldb : 0;
  uint64_t aoff[kGALoads];
  uint64_t boff[kGBLoads];
#pragma unroll
  for (int i = 0; i < kGALoads; ++i) {
    const int pos = (i * kGWaves + uwave) * 64 + lane;   // 16-byte position in the tile
    const int r = pos / 8, slot = pos % 8;
    const int64_t gr = min(row0 + r, M - 1);
    aoff[i] = static_cast<uint64_t>((a_elem(gr) - ael0) * 2 + 16 * g_slot(r, slot));
  }
#pragma unroll
  for (int i = 0; i < kGBLoads; ++i) {
    const int pos = (i * kGWaves + uwave) * 64 + lane;
    const int r = pos / 8, slot = pos % 8;
    boff[i] = static_cast<uint64_t>(((col0 + r) * g.ldb - bel0) * 2 + 16 * g_slot(r, slot));
  }
  const char *abase = reinterpret_cast<const char *>(g.a) + ael0 * 2;
  const char *bbase = reinterpret_cast<const char *>(g.bt) + bel0 * 2;
  // descriptors (ASM): A from the first row to the end of A, B^T from the
  // first column to the end of the workgroup's columns
  i32x4 arsrc, brsrc;
  if constexpr (ASM) {
    int64_t a_end;
    if constexpr (HD > 0) {
      const int64_t segs = cdiv(M, g.a_seg_rows);
      a_end = segs * g.a_heads * g.a_seg_rows * HD;
    } else {
      a_end = (M - 1) * g.lda + g.K;
    }
    arsrc = buffer_rsrc(abase, static_cast<uint32_t>(min<int64_t>((a_end - ael0) * 2, 0xffffffffLL)));
    brsrc = buffer_rsrc(bbase, static_cast<uint32_t>((static_cast<int64_t>(kGCols - 1) * g.ldb + g.K) * 2));
  }
  auto load_chunk = [&](int c, bf16 *sa, bf16 *sb) __attribute__((always_inline)) {
    const int64_t kb = static_cast<int64_t>(c) * kGK * 2;   // B^T (and row-major A): k = 64 c
    int64_t ab = kb;
    if constexpr (HD > 0) {
      constexpr int kPerHead = HD / kGK;
      const int h = c / kPerHead;
      ab = (static_cast<int64_t>(h) * g.a_seg_rows * HD + (c - h * kPerHead) * kGK) * 2;
    }
    if constexpr (ASM) {
      i32x4 ar, br;   // (wave-uniform: readfirstlane keeps them in scalar registers)
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        ar[k] = __builtin_amdgcn_readfirstlane(arsrc[k]);
        br[k] = __builtin_amdgcn_readfirstlane(brsrc[k]);
      }
      const uint32_t sa_off = __builtin_amdgcn_readfirstlane(static_cast<uint32_t>(ab));
      const uint32_t sb_off = __builtin_amdgcn_readfirstlane(static_cast<uint32_t>(kb));
#pragma unroll
      for (int i = 0; i < kGALoads; ++i)
        load_lds16(ar, static_cast<uint32_t>(aoff[i]), sa_off, sa + (i * kGWaves + uwave) * 512);
#pragma unroll
      for (int i = 0; i < kGBLoads; ++i)
        load_lds16(br, static_cast<uint32_t>(boff[i]), sb_off, sb + (i * kGWaves + uwave) * 512);
    } else {
#pragma unroll
      for (int i = 0; i < kGALoads; ++i)
        __builtin_amdgcn_global_load_lds((gvoid_t *)(abase + ab + aoff[i]),
                                         (lvoid_t *)(sa + (i * kGWaves + uwave) * 512), 16, 0, 0);
#pragma unroll
      for (int i = 0; i < kGBLoads; ++i)
        __builtin_amdgcn_global_load_lds((gvoid_t *)(bbase + kb + boff[i]),
                                         (lvoid_t *)(sb + (i * kGWaves + uwave) * 512), 16, 0, 0);
    }
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
  if constexpr (ASM) lds_barrier();
  else __syncthreads();
  // Step c: load chunk c+2 into the ring slot of chunk c-1, compute chunk c,
  // wait for chunk c+1, barrier.  Loads past the last chunk re-read chunk
  // nc-1 (in range; never used) so every step waits on the same count.
  auto step = [&](int c, bf16 *ln_a, bf16 *ln_b, const bf16 *ca, const bf16 *cb)
      __attribute__((always_inline)) {
    load_chunk(min(c + 2, nc - 1), ln_a, ln_b);
    compute(ca, cb);
    asm volatile("s_waitcnt vmcnt(6)" ::: "memory");
    if constexpr (ASM) lds_barrier();
    else __syncthreads();
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

// Large form for the big products: one workgroup = 256 x 256 like the wide
// form, but 4 waves as 2 x 2, each wave 128 x 128 (4 x 4 MFMA tiles, 256
// accumulator registers, one wave per SIMD).  Every A and B^T fragment read
// from LDS feeds 4 MFMAs (0.5 reads per MFMA, against 0.75 in the wide form).
// The k loop runs over 32-wide chunks (16 KB of A and 16 KB of B^T) in a
// ring of kBStages LDS stages (K a multiple of 32 kBStages), the direct loads
// running kBStages - 1 chunks ahead: with one wave per SIMD nothing else hides a load that misses the
// L2, and one chunk of lead (the two-stage forms) left the MFMAs waiting.
// LDS rows are 64 bytes, 16-byte piece p of row r at slot p ^ ((r / 4) % 4),
// so the 16 lanes of a fragment read phase (16 consecutive rows, one piece)
// cover all 64 banks.  The fragments of the next 16-wide k step are read
// while the MFMAs of the current one run.
#ifndef TDP_GEMM_STAGES
#define TDP_GEMM_STAGES 4
#endif
// MFMAs of a chunk's last k step issued before its barrier (the rest carry
// the next chunk's first fragment reads); at most 8.
#ifndef TDP_GEMM_PRE_BARRIER
#define TDP_GEMM_PRE_BARRIER 8
#endif
constexpr int kBPreBarrier = TDP_GEMM_PRE_BARRIER;
static_assert(kBPreBarrier >= 0 && kBPreBarrier <= 8, "8 reads after the barrier");
// 1: the chunk body interleaves MFMAs and memory instructions one by one;
// 0: grouped (reads, then MFMAs, fenced).
#ifndef TDP_GEMM_INTERLEAVE
#define TDP_GEMM_INTERLEAVE 1
#endif
constexpr int kBStages = TDP_GEMM_STAGES;
constexpr int kBK = 32;                      // k per chunk
constexpr int kBWaves = 4;
constexpr int kBThreads = 64 * kBWaves;
constexpr int kBLoadsA = kWRows * kBK * 2 / 1024 / kBWaves;   // 4 (1 KB each, per wave)
constexpr int kBLoadsB = kWCols * kBK * 2 / 1024 / kBWaves;   // 4
constexpr int kBLoads = kBLoadsA + kBLoadsB;
static_assert(kBStages >= 2 && kBStages <= 4, "2..4 stages of 32 KB");


// Wait until at most N chunks of direct loads (8 instructions each) are in
// flight.
template <int N>
__device__ __forceinline__ void wait_chunks() {
  static_assert(N >= 0 && N <= 2, "vmcnt of 0, 8 or 16");
  if constexpr (N == 0) asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  if constexpr (N == 1) asm volatile("s_waitcnt vmcnt(8)" ::: "memory");
  if constexpr (N == 2) asm volatile("s_waitcnt vmcnt(16)" ::: "memory");
}

__device__ __forceinline__ int b_slot(int r, int piece) { return piece ^ ((r >> 2) & 3); }

template <int EPI, int HD>
__global__ __launch_bounds__(kBThreads, 1) void gemm_big_kernel(GemmArgs g) {
  static_assert(HD % kBK == 0, "whole k chunks per head");
  __shared__ __attribute__((aligned(16))) bf16 sA[kBStages][kWRows * kBK];
  __shared__ __attribute__((aligned(16))) bf16 sB[kBStages][kWCols * kBK];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int l32 = lane & 31, hh = lane >> 5;
  const int uwave = __builtin_amdgcn_readfirstlane(wave);
  const int wm = wave & 1, wn = wave >> 1;
  const int64_t M = g.M;
  const int64_t nm = cdiv(M, kWRows), nn = g.N / kWCols;
  int64_t tm, tn;
  {
    const int64_t G = gridDim.x;   // a multiple of 8, >= nm * nn
    const int64_t bid = blockIdx.x;
    const int64_t lid = (bid % 8) * (G / 8) + bid / 8;
    if (lid >= nm * nn) return;
    constexpr int64_t kGroup = TDP_GEMM_GROUP_M > 0 ? TDP_GEMM_GROUP_M : 1;
    const int64_t per_group = kGroup * nn;
    const int64_t grp = lid / per_group;
    const int64_t first_m = grp * kGroup;
    const int64_t gm = min(kGroup, nm - first_m);
    const int64_t in = lid - grp * per_group;
    tm = first_m + in % gm;
    tn = in / gm;
  }
  // The tile indices come out of 64-bit divisions on the vector unit; make
  // them wave-uniform so the buffer descriptors below sit in scalar registers.
  const int64_t row0 = static_cast<int64_t>(__builtin_amdgcn_readfirstlane(static_cast<int>(tm))) *
                       kWRows;
  const int64_t col0 = static_cast<int64_t>(__builtin_amdgcn_readfirstlane(static_cast<int>(tn))) *
                       kWCols;
  // Direct loads: buffer_load ... lds written as inline assembly, through
  // buffer descriptors.  The compiler then tracks none of them, so it never
  // waits for a stage's loads before reading another stage (its alias
  // tracking of LDS direct loads loses track across a ring of stages and
  // waits for all of them); the waits are the explicit vmcnt counts before
  // each barrier.  Each descriptor covers exactly the bytes this workgroup may
  // read (a load outside it returns zeros instead of faulting); per-lane
  // offsets are 32-bit within it and a chunk's k offset is the scalar offset.
  // Rows past M re-read row M - 1 (their results are not stored).
  const int64_t rows_here = min(static_cast<int64_t>(kWRows), M - row0);
  const char *abase;
  uint32_t a_extent;
  if constexpr (HD > 0) {
    abase = reinterpret_cast<const char *>(g.a);
    a_extent = static_cast<uint32_t>(M * g.K * 2);   // host: < 2^32 bytes
  } else {
    abase = reinterpret_cast<const char *>(g.a + row0 * g.lda);
    a_extent = static_cast<uint32_t>(((rows_here - 1) * g.lda + g.K) * 2);
  }
  const char *bbase = reinterpret_cast<const char *>(g.bt + col0 * g.ldb);
  const uint32_t b_extent = static_cast<uint32_t>(((kWCols - 1) * g.ldb + g.K) * 2);
  const i32x4 arsrc = buffer_rsrc(abase, a_extent);
  const i32x4 brsrc = buffer_rsrc(bbase, b_extent);
  uint32_t aoff[kBLoadsA], boff[kBLoadsB];
#pragma unroll
  for (int i = 0; i < kBLoadsA; ++i) {
    const int pos = (i * kBWaves + uwave) * 64 + lane;   // 16-byte position in the stage
    const int r = pos / 4, slot = pos % 4;
    const int64_t gr = min(row0 + r, M - 1);
    int64_t el;
    if constexpr (HD > 0) {
      const int64_t L = g.a_seg_rows;
      const int64_t seg = gr / L;
      el = (seg * g.a_heads * L + (gr - seg * L)) * HD;
    } else {
      el = (gr - row0) * g.lda;
    }
    aoff[i] = static_cast<uint32_t>(el * 2 + 16 * b_slot(r, slot));
  }
#pragma unroll
  for (int i = 0; i < kBLoadsB; ++i) {
    const int pos = (i * kBWaves + uwave) * 64 + lane;
    const int r = pos / 4, slot = pos % 4;
    boff[i] = static_cast<uint32_t>(r * g.ldb * 2 + 16 * b_slot(r, slot));
  }
  // Scalar offsets of chunk c: {A, B^T}.
  auto chunk_soff = [&](int c) __attribute__((always_inline)) {
    const uint32_t kb = static_cast<uint32_t>(c) * kBK * 2;
    uint32_t ab = kb;
    if constexpr (HD > 0) {
      constexpr int kPerHead = HD / kBK;
      const int h = c / kPerHead;
      ab = static_cast<uint32_t>((static_cast<int64_t>(h) * g.a_seg_rows * HD +
                                  (c - h * kPerHead) * kBK) * 2);
    }
    return uint2{ab, kb};
  };
  // Load i (0..7: four of A, then four of B^T) of a chunk.
  auto load_one = [&](int i, uint2 so, bf16 *sa, bf16 *sb) __attribute__((always_inline)) {
    if (i < kBLoadsA) load_lds16(arsrc, aoff[i], so.x, sa + (i * kBWaves + uwave) * 512);
    else load_lds16(brsrc, boff[i - kBLoadsA], so.y, sb + ((i - kBLoadsA) * kBWaves + uwave) * 512);
  };
  auto load_chunk = [&](int c, bf16 *sa, bf16 *sb) __attribute__((always_inline)) {
    const uint2 so = chunk_soff(c);
#pragma unroll
    for (int i = 0; i < kBLoads; ++i) load_one(i, so, sa, sb);
  };
  // fragment offsets (elements): A row 128 wm + 32 t + l32, B^T row
  // 128 wn + 32 t + l32; piece 2 ks + hh
  int32_t afo[4][2], bfo[4][2];
#pragma unroll
  for (int ks = 0; ks < 2; ++ks) {
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      const int ar = 128 * wm + 32 * t + l32;
      afo[t][ks] = ar * kBK + 8 * b_slot(ar, 2 * ks + hh);
      const int br = 128 * wn + 32 * t + l32;
      bfo[t][ks] = br * kBK + 8 * b_slot(br, 2 * ks + hh);
    }
  }
  f32x16 acc[4][4];
#pragma unroll
  for (int mt = 0; mt < 4; ++mt)
#pragma unroll
    for (int ct = 0; ct < 4; ++ct) acc[mt][ct] = f32x16{};
  // Two fragment sets: k step ks of a chunk uses set ks.
  bf16x8 fa0[4], fb0[4], fa1[4], fb1[4];
  auto read = [&](const bf16 *sa, const bf16 *sb, int ks, bf16x8 (&fa)[4], bf16x8 (&fb)[4])
      __attribute__((always_inline)) {
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      fa[t] = *reinterpret_cast<const bf16x8 *>(sa + afo[t][ks]);
      fb[t] = *reinterpret_cast<const bf16x8 *>(sb + bfo[t][ks]);
    }
  };
  auto mfmas = [&](const bf16x8 (&fa)[4], const bf16x8 (&fb)[4], int mt0, int mt1)
      __attribute__((always_inline)) {
#pragma unroll
    for (int mt = mt0; mt < mt1; ++mt)
#pragma unroll
      for (int ct = 0; ct < 4; ++ct) acc[mt][ct] = mfma32(fa[mt], fb[ct], acc[mt][ct]);
  };
  const int nc = g.K / kBK;
#define TDP_FENCE() __builtin_amdgcn_sched_barrier(0)
  // Chunk c in stage (sa, sb); chunk c + kBStages - 1 goes to (la, lb), the
  // stage chunk c - 1 used; the next chunk is in (na, nb).  The loads go out
  // first; the reads of step 1 go out before the MFMAs of step 0; the wait for
  // the next chunk (the newer kBStages - 2 chunks may still be in flight), the
  // barrier and the next chunk's first reads sit between the two halves of
  // step 1's MFMAs.  Loads past the last chunk re-load chunk nc - 1 (in range,
  // never used), so every chunk leaves the same count of loads in flight.
  auto chunk = [&](int c, const bf16 *sa, const bf16 *sb, bf16 *la, bf16 *lb, const bf16 *na,
                   const bf16 *nb) __attribute__((always_inline)) {
#if TDP_GEMM_INTERLEAVE
    // One MFMA, then one memory instruction, in a fixed order: step 0's 16
    // MFMAs carry the 8 fragment reads of step 1 and the chunk's 8 direct
    // loads; step 1's second 8 MFMAs carry the next chunk's 8 first reads.
    const uint2 so = chunk_soff(min(c + kBStages - 1, nc - 1));
#pragma unroll
    for (int q = 0; q < 16; ++q) {
      acc[q / 4][q % 4] = mfma32(fa0[q / 4], fb0[q % 4], acc[q / 4][q % 4]);
      if (q < 4) fa1[q] = *reinterpret_cast<const bf16x8 *>(sa + afo[q][1]);
      else if (q < 8) fb1[q - 4] = *reinterpret_cast<const bf16x8 *>(sb + bfo[q - 4][1]);
      else load_one(q - 8, so, la, lb);
      TDP_FENCE();
    }
#pragma unroll
    for (int q = 0; q < kBPreBarrier; ++q) {
      acc[q / 4][q % 4] = mfma32(fa1[q / 4], fb1[q % 4], acc[q / 4][q % 4]);
      TDP_FENCE();
    }
    wait_chunks<kBStages - 2>();
    lds_barrier();
    TDP_FENCE();
    // the next chunk's step-0 fragments, in the order its first MFMAs use
    // them: A tile 0, B tiles 0..3, A tiles 1..3
#pragma unroll
    for (int q = kBPreBarrier; q < 16; ++q) {
      const int r = q - kBPreBarrier;
      if (r == 0) fa0[0] = *reinterpret_cast<const bf16x8 *>(na + afo[0][0]);
      else if (r < 5) fb0[r - 1] = *reinterpret_cast<const bf16x8 *>(nb + bfo[r - 1][0]);
      else if (r < 8) fa0[r - 4] = *reinterpret_cast<const bf16x8 *>(na + afo[r - 4][0]);
      acc[q / 4][q % 4] = mfma32(fa1[q / 4], fb1[q % 4], acc[q / 4][q % 4]);
      TDP_FENCE();
    }
    return;
#endif
    load_chunk(min(c + kBStages - 1, nc - 1), la, lb);
    TDP_FENCE();
    read(sa, sb, 1, fa1, fb1);
    TDP_FENCE();
    mfmas(fa0, fb0, 0, 4);
    TDP_FENCE();
    mfmas(fa1, fb1, 0, 2);
    TDP_FENCE();
    wait_chunks<kBStages - 2>();
    lds_barrier();
    read(na, nb, 0, fa0, fb0);
    TDP_FENCE();
    mfmas(fa1, fb1, 2, 4);
    TDP_FENCE();
  };
  static_assert(kBLoads == 8, "wait_chunks counts 8 loads per chunk");
  // Prologue: chunks 0 .. kBStages - 2 into stages 0 .. kBStages - 2, wait
  // for chunk 0, its first fragments.
  auto prologue = [&](bf16 *a0, bf16 *b0, bf16 *a1, bf16 *b1, bf16 *a2, bf16 *b2)
      __attribute__((always_inline)) {
    load_chunk(0, a0, b0);
    if constexpr (kBStages > 2) load_chunk(min(1, nc - 1), a1, b1);
    if constexpr (kBStages > 3) load_chunk(min(2, nc - 1), a2, b2);
    wait_chunks<kBStages - 2>();
    lds_barrier();
    read(a0, b0, 0, fa0, fb0);
  };
  prologue(sA[0], sB[0], sA[1 % kBStages], sB[1 % kBStages], sA[2 % kBStages],
           sB[2 % kBStages]);
  // nc is a multiple of kBStages (host check): every stage index below is a
  // constant.
  for (int c0 = 0; c0 < nc; c0 += kBStages) {
#pragma unroll
    for (int st = 0; st < kBStages; ++st)
      chunk(c0 + st, sA[st], sB[st], sA[(st + kBStages - 1) % kBStages],
            sB[(st + kBStages - 1) % kBStages], sA[(st + 1) % kBStages],
            sB[(st + 1) % kBStages]);
  }
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
#undef TDP_FENCE

  // acc[mt][ct][v]: row 128 wm + 32 mt + 8 (v/4) + 4 hh + v%4, column
  // 128 wn + 32 ct + l32.  The residual forms read all of a 32-row group's
  // old values before storing any (one wave per SIMD: nothing else hides the
  // load latency).
#pragma unroll
  for (int mt = 0; mt < 4; ++mt) {
    const int64_t base = row0 + 128 * wm + 32 * mt;
    if constexpr (EPI == kEpiResid || EPI == kEpiResidGate) {
      float old[16][4];
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        const int64_t r = base + 8 * (v / 4) + 4 * hh + (v % 4);
#pragma unroll
        for (int ct = 0; ct < 4; ++ct)
          old[v][ct] = r < M ? static_cast<const float *>(g.c)[r * g.ldc + col0 + 128 * wn +
                                                                 32 * ct + l32]
                             : 0.f;
      }
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        const int64_t r = base + 8 * (v / 4) + 4 * hh + (v % 4);
        if (r >= M) continue;
        const int64_t b = r / g.rows_per_batch;
#pragma unroll
        for (int ct = 0; ct < 4; ++ct) {
          const int64_t n = col0 + 128 * wn + 32 * ct + l32;
          float gt = 1.0f;
          if constexpr (EPI == kEpiResidGate)
            gt = (g.g0 ? g.g0[b * g.g0_stride + n] : 0.f) + (g.g1 ? g.g1[n] : 0.f);
          static_cast<float *>(g.c)[r * g.ldc + n] = fmaf(gt, acc[mt][ct][v], old[v][ct]);
        }
      }
    } else {
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        const int64_t r = base + 8 * (v / 4) + 4 * hh + (v % 4);
        if (r >= M) continue;
#pragma unroll
        for (int ct = 0; ct < 4; ++ct) {
          const int64_t idx = r * g.ldc + col0 + 128 * wn + 32 * ct + l32;
          const float x = acc[mt][ct][v];
          if constexpr (EPI == kEpiBf16) static_cast<bf16 *>(g.c)[idx] = static_cast<bf16>(x);
          if constexpr (EPI == kEpiF32) static_cast<float *>(g.c)[idx] = x;
          if constexpr (EPI == kEpiGeluBf16) static_cast<bf16 *>(g.c)[idx] = static_cast<bf16>(gelu_tanh(x));
          if constexpr (EPI == kEpiSiluBf16) static_cast<bf16 *>(g.c)[idx] = static_cast<bf16>(silu(x));
        }
      }
    }
  }
}

// Large form with 64-wide k chunks: 256 x 256 per tile, 4 waves of 128 x 128
// (one wave per SIMD), two LDS buffers.  Chunk c + 1 goes global -> LDS by
// direct loads into the buffer chunk c - 1 used while chunk c is computed
// (its loads spread over the first half of the chunk's MFMAs), so each chunk
// costs one barrier and its loads have half to all of a chunk to land.  One
// memory instruction after each MFMA, in a fixed order; the next chunk's
// first fragments are read after the barrier, under the last 8 MFMAs.
// Measured against the 4-stage ring of 32-wide chunks on the block's shapes:
// FFN up 14.30 -> 13.37 ms, FFN down 15.47 -> 13.83, QKV 9.87 -> 9.08;
// staging the loads through registers instead (two chunks ahead) gave 13.76
// / 13.67 / 9.8, its LDS writes and their waits costing more than the extra
// lead saved.
//
// Persistent: one workgroup per CU walks the tiles of its XCD (blockIdx % 8)
// in order; with a counter given, the last ~1/12 of the tiles are instead
// claimed one at a time by whichever workgroups get there first (the XCDs
// hold different shader clocks under load).  The last chunk of a tile loads
// the next tile's first chunk into the free buffer and reads its first
// fragments after the barrier, so the next tile's prologue runs under the
// previous tile's last MFMAs and its epilogue; the first k step of a tile
// starts its accumulators from zero in the MFMA itself.  Measured on the
// block's shapes against one workgroup per tile (same box): FFN up 13.2 ->
// 12.96 ms, QKV 9.27 -> 9.08, FFN down unchanged, results bitwise the same;
// the claimed tail then took the block step from 63.9 to 62.9 ms.
#ifndef TDP_GEMM_K64
#define TDP_GEMM_K64 1
#endif
constexpr int kRK = 64;                                 // k per chunk
constexpr int kRLoads = 256 * kRK * 2 / 1024 / 4;       // 1 KB per wave-load, per operand: 8
// LDS rows of 64 k (128 bytes, 8 pieces of 16 B); piece p of row r sits at
// p ^ ((r / 2) % 8).  Two rows share a 256-byte bank window, so a fragment
// read's 16 consecutive rows of one piece land in 16 distinct 16-byte bank
// groups, and a load's 8 whole rows fill each group four times.
__device__ __forceinline__ int rs_slot(int r, int p) { return p ^ ((r >> 1) & 7); }

// HD = 0: row-major A; HD = 64 / 128: head-major A with that head size.
// LEAD: chunk c + 2's A loads go out right after chunk c's barrier (its
// buffer is free from there) and chunk c + 1's B loads in chunk c's first
// step, instead of both in chunk c's first two steps: more time for each
// load to land.  Measured on the block's shapes: FFN down (K = 16384)
// 13.75 -> 13.00 ms; FFN up and QKV (K = 4096) 12.56 -> 12.76 and 8.82 ->
// 8.98 ms, so the launch takes it for K >= 8192 only (there K / 64 >= 128).
template <int EPI, int HD, bool LEAD = false>
__global__ __launch_bounds__(256, 1) void gemm_k64_kernel(GemmArgs g) {
  static_assert(HD % kRK == 0, "whole k chunks per head");
  __shared__ __attribute__((aligned(16))) bf16 sA[2][256 * kRK];
  __shared__ __attribute__((aligned(16))) bf16 sB[2][256 * kRK];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int l32 = lane & 31, hh = lane >> 5;
  const int uwave = __builtin_amdgcn_readfirstlane(wave);
  const int wm = wave & 1, wn = wave >> 1;
  const int64_t M = g.M;
  const int64_t nm = cdiv(M, kWRows), nn = g.N / kWCols;
  const int64_t T = nm * nn;
  // XCD x takes tiles [x S8, (x + 1) S8); its G / 8 workgroups one tile each
  // at a time, in order (gridDim.x is a multiple of 8).  Tiles from 8 S8 on
  // (with a tail) are claimed: a claim returns the next of them; every
  // workgroup claims until a claim returns no tile, so a launch makes
  // exactly tail_claims = tail + G claims, and the last one puts the counter
  // back to zero.  A tile's claim for its successor goes out as the tile
  // starts; its result reaches the other waves through LDS at chunk 0's
  // barrier.
  const int64_t G = gridDim.x, bid = blockIdx.x;
  const int64_t S8 = g.per_xcd;
  const int64_t lid_end = min((bid % 8) * S8 + S8, T);
  const int64_t lstep = G / 8;
  const bool tail = g.tail_claims != 0;
  __shared__ int64_t s_claim;
  auto claim = [&]() __attribute__((always_inline)) {
    const uint32_t tk = atomicAdd(g.tail_ctr, 1u);
    if (tk == g.tail_claims - 1u) atomicExch(g.tail_ctr, 0u);
    return 8 * S8 + static_cast<int64_t>(tk);
  };
  int64_t lid = (bid % 8) * S8 + bid / 8;
  if (lid >= lid_end) {
    if (!tail) return;
    if (threadIdx.x == 0) s_claim = claim();
    __syncthreads();
    lid = s_claim;
    if (lid >= T) return;
  }
  // Tile order within the XCD's range: groups of group_m row blocks walk
  // down a column of tiles.
  auto tile_of = [&](int64_t l, int64_t &row0, int64_t &col0) __attribute__((always_inline)) {
    const int64_t group = g.group_m;
    const int64_t per_group = group * nn;
    const int64_t grp = l / per_group;
    const int64_t first_m = grp * group;
    const int64_t gm = min(group, nm - first_m);
    const int64_t in = l - grp * per_group;
    row0 = (first_m + in % gm) * kWRows;
    col0 = (in / gm) * kWCols;
  };
  int64_t row0, col0;
  tile_of(lid, row0, col0);
  // Direct load i of an operand's chunk: LDS 16-byte position (i * 4 +
  // wave) * 64 + lane = row * 8 + slot takes the row's piece slot ^ key(row)
  // (the swizzle is its own inverse).  Each descriptor covers exactly the
  // bytes this tile may read (none once there is no next tile: those loads
  // touch no memory); rows past M re-read row M - 1 (their results are not
  // stored).
  i32x4 arsrc, brsrc;
  uint32_t aoff[kRLoads], boff[kRLoads];
  auto set_a = [&](int64_t r0, bool live) __attribute__((always_inline)) {
    const int rows_here = static_cast<int>(min(static_cast<int64_t>(kWRows), M - r0));
    if constexpr (HD > 0) {
      arsrc = buffer_rsrc(g.a, live ? static_cast<uint32_t>(M * g.K * 2) : 0u);   // host: < 2^32 bytes
    } else {
      arsrc = buffer_rsrc(g.a + r0 * g.lda,
                          live ? static_cast<uint32_t>(((rows_here - 1) * g.lda + g.K) * 2) : 0u);
    }
#pragma unroll
    for (int i = 0; i < kRLoads; ++i) {
      const int pos = (i * 4 + uwave) * 64 + lane;
      const int r = pos / 8, p = rs_slot(r, pos % 8);
      const int ra = min(r, rows_here - 1);
      if constexpr (HD > 0) {
        // head-major A: row gr of segment seg (a_seg_rows rows each) is row
        // gr - seg L of every head's slab; a chunk's head offset is scalar
        const uint32_t L = static_cast<uint32_t>(g.a_seg_rows);
        const uint32_t gr = static_cast<uint32_t>(r0 + ra);
        const uint32_t seg = gr / L;
        aoff[i] = ((seg * static_cast<uint32_t>(g.a_heads) * L + (gr - seg * L)) * HD + 8 * p) * 2;
      } else {
        aoff[i] = static_cast<uint32_t>((static_cast<int64_t>(ra) * g.lda + 8 * p) * 2);
      }
    }
  };
  auto set_b = [&](int64_t c0, bool live) __attribute__((always_inline)) {
    brsrc = buffer_rsrc(g.bt + c0 * g.ldb,
                        live ? static_cast<uint32_t>(((kWCols - 1) * g.ldb + g.K) * 2) : 0u);
  };
#pragma unroll
  for (int i = 0; i < kRLoads; ++i) {
    const int pos = (i * 4 + uwave) * 64 + lane;
    const int r = pos / 8, p = rs_slot(r, pos % 8);
    boff[i] = static_cast<uint32_t>((static_cast<int64_t>(r) * g.ldb + 8 * p) * 2);
  }
  set_a(row0, true);
  set_b(col0, true);
  // Fragment offsets: A row 128 wm + 32 t + l32, B^T row 128 wn + 32 t + l32,
  // piece 2 s + hh of k step s; the swizzle key of the row depends on l32
  // only, so tile t adds 32 t rows.
  int32_t fao[4], fbo[4];
#pragma unroll
  for (int s = 0; s < 4; ++s) {
    const int x = 8 * rs_slot(l32, 2 * s + hh);
    fao[s] = (128 * wm + l32) * kRK + x;
    fbo[s] = (128 * wn + l32) * kRK + x;
  }
  f32x16 acc[4][4];
  bf16x8 fa[2][4], fb[2][4];            // fragments of k step s (set s % 2)
  const int nc = g.K / kRK;
#define TDP_FENCE() __builtin_amdgcn_sched_barrier(0)
  // chunk c's load i into buffer buf, with the current descriptors
  auto dload = [&](int buf, int c, int i) __attribute__((always_inline)) {
    const uint32_t so = static_cast<uint32_t>(c) * kRK * 2;
    uint32_t sa = so;
    if constexpr (HD > 0) {
      constexpr int kPerHead = HD / kRK;
      const int h = c / kPerHead;
      sa = static_cast<uint32_t>((static_cast<int64_t>(h) * g.a_seg_rows * HD +
                                  (c - h * kPerHead) * kRK) * 2);
    }
    if (i < kRLoads) load_lds16(arsrc, aoff[i], sa, &sA[buf][(i * 4 + uwave) * 512]);
    else load_lds16(brsrc, boff[i - kRLoads], so, &sB[buf][((i - kRLoads) * 4 + uwave) * 512]);
  };
  // fragment read q of k step s: A tile 0, B tiles 0..3, A tiles 1..3 (the
  // order step s's MFMAs use them)
  auto fread = [&](int buf, int s, int q) __attribute__((always_inline)) {
    if (q == 0) fa[s & 1][0] = *reinterpret_cast<const bf16x8 *>(&sA[buf][fao[s]]);
    else if (q < 5) fb[s & 1][q - 1] = *reinterpret_cast<const bf16x8 *>(&sB[buf][fbo[s] + 32 * (q - 1) * kRK]);
    else fa[s & 1][q - 4] = *reinterpret_cast<const bf16x8 *>(&sA[buf][fao[s] + 32 * (q - 4) * kRK]);
  };
  // the first tile's chunk 0 (and, LEAD, chunk 1's A)
#pragma unroll
  for (int i = 0; i < 2 * kRLoads; ++i) dload(0, 0, i);
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  lds_barrier();
  if constexpr (LEAD) {
#pragma unroll
    for (int i = 0; i < kRLoads; ++i) dload(1, 1, i);
  }
#pragma unroll
  for (int q = 0; q < 8; ++q) fread(0, 0, q);
  int64_t nrow0 = row0, ncol0 = col0;
  bool has_next = false;
  int64_t claimed = 0;           // thread 0: this tile's claim for its successor
  bool claiming = false;         // the successor comes from a claim
  // Chunk c in buffer c % 2: step s's MFMAs carry step s + 1's reads (even
  // slots) and chunk c + 1's 16 direct loads (odd slots of steps 0 and 1;
  // LEAD: the B loads in step 0, chunk c + 2's A loads after the barrier);
  // after 8 of step 3's MFMAs the wait for those loads and the barrier, then
  // chunk c + 1's step-0 reads.  MODE 0: the loads are of this tile; 1 (LEAD,
  // chunk nc - 2): the A loads after the barrier are of the next tile's
  // chunk 0; 2 (chunk nc - 1): the loads are of the next tile's chunk 0
  // (LEAD: its B, then chunk 1's A).  Z: step 0 starts the accumulators.
  auto chunk = [&](int c, auto par, auto zero, auto mode) __attribute__((always_inline)) {
    constexpr int P = decltype(par)::value;
    constexpr bool Z = decltype(zero)::value;
    constexpr int MODE = decltype(mode)::value;
    if constexpr (MODE == 2) {
      if constexpr (!LEAD) set_a(nrow0, has_next);
      set_b(ncol0, has_next);
    }
#pragma unroll
    for (int s = 0; s < 4; ++s) {
#pragma unroll
      for (int q = 0; q < 16; ++q) {
        const int am = q / 4, bn = q % 4;
        if (s == 3 && q == 8) {
          asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
          if constexpr (Z) {
            if (claiming && threadIdx.x == 0) s_claim = claimed;
          }
          lds_barrier();
          TDP_FENCE();
          if constexpr (LEAD && MODE == 1) set_a(nrow0, has_next);
        }
        if (Z && s == 0) acc[am][bn] = mfma32(fa[0][am], fb[0][bn], f32x16{});
        else acc[am][bn] = mfma32(fa[s & 1][am], fb[s & 1][bn], acc[am][bn]);
        const int cb = MODE == 2 ? 0 : c + 1;   // chunk of the B loads (and of A without LEAD)
        if constexpr (LEAD) {
          const int ca = MODE == 0 ? c + 2 : (MODE == 1 ? 0 : 1);
          if (s < 3 && q % 2 == 0) fread(P, s + 1, q / 2);
          else if (s == 0) dload(1 - P, cb, kRLoads + q / 2);
          else if (s == 3 && q >= 8) {
            fread(1 - P, 0, q - 8);
            dload(P, ca, q - 8);
          }
        } else {
          if (s < 3 && q % 2 == 0) fread(P, s + 1, q / 2);
          else if (s < 2) dload(1 - P, cb, 8 * s + q / 2);
          else if (s == 3 && q >= 8) fread(1 - P, 0, q - 8);
        }
        TDP_FENCE();
      }
    }
  };
  using P0 = std::integral_constant<int, 0>;
  using P1 = std::integral_constant<int, 1>;
  using M0 = std::integral_constant<int, 0>;
  using M1 = std::integral_constant<int, 1>;
  using M2 = std::integral_constant<int, 2>;
  for (;;) {
    int64_t nlid = lid + lstep;
    claiming = tail && !(nlid < lid_end);
    if (claiming) {
      if (threadIdx.x == 0) claimed = claim();
    } else {
      has_next = nlid < lid_end;
      if (has_next) tile_of(nlid, nrow0, ncol0);
    }
    // K is a multiple of 128 and at least 256: the first pair, the middle
    // pairs, the last pair
    chunk(0, P0{}, std::true_type{}, M0{});
    if (claiming) {
      nlid = s_claim;
      has_next = nlid < T;
      if (has_next) tile_of(nlid, nrow0, ncol0);
    }
    chunk(1, P1{}, std::false_type{}, M0{});
    for (int c = 2; c < nc - 2; c += 2) {
      chunk(c, P0{}, std::false_type{}, M0{});
      chunk(c + 1, P1{}, std::false_type{}, M0{});
    }
    if constexpr (LEAD) chunk(nc - 2, P0{}, std::false_type{}, M1{});
    else chunk(nc - 2, P0{}, std::false_type{}, M0{});
    chunk(nc - 1, P1{}, std::false_type{}, M2{});
    // acc[mt][ct][v]: row 128 wm + 32 mt + 8 (v/4) + 4 hh + v%4, column
    // 128 wn + 32 ct + l32
#pragma unroll
    for (int mt = 0; mt < 4; ++mt) {
      const int64_t base = row0 + 128 * wm + 32 * mt;
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        const int64_t r = base + 8 * (v / 4) + 4 * hh + (v % 4);
        if (r >= M) continue;
#pragma unroll
        for (int ct = 0; ct < 4; ++ct) {
          const int64_t idx = r * g.ldc + col0 + 128 * wn + 32 * ct + l32;
          const float x = acc[mt][ct][v];
          if constexpr (EPI == kEpiBf16) static_cast<bf16 *>(g.c)[idx] = static_cast<bf16>(x);
          if constexpr (EPI == kEpiF32) static_cast<float *>(g.c)[idx] = x;
          if constexpr (EPI == kEpiGeluBf16) static_cast<bf16 *>(g.c)[idx] = static_cast<bf16>(gelu_tanh(x));
          if constexpr (EPI == kEpiSiluBf16) static_cast<bf16 *>(g.c)[idx] = static_cast<bf16>(silu(x));
        }
      }
    }
    if (!has_next) break;
    lid = nlid;
    row0 = nrow0;
    col0 = ncol0;
  }
  // the last tile's loads of "the next tile" touched no memory but still
  // write LDS: wait for them before the workgroup ends
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
#undef TDP_FENCE
}


// Which form serves the large products: 2 = the large form above, 1 = the
// wide form.
#ifndef TDP_GEMM_BIG
#define TDP_GEMM_BIG 2
#endif

#ifndef TDP_GEMM_WIDE
#define TDP_GEMM_WIDE 1
#endif

// Workgroups of the persistent large form: one per CU, rounded down to a
// multiple of 8 (the XCD count), per device; 0 if HIP cannot say.
int persistent_slots() {
  static std::atomic<int> slots[64];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 0;
  int n = slots[dev].load(std::memory_order_relaxed);
  if (n == 0) {
    int cus = 0;
    if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
      return 0;
    n = cus >= 8 ? cus / 8 * 8 : 8;
    slots[dev].store(n, std::memory_order_relaxed);
  }
  return n;
}

template <int EPI>
tdp_status launch_epi(const GemmArgs &a, int hd, dim3 grid, hipStream_t stream) {
  // the wide form for a multiple of 256 columns and enough rows
  if (TDP_GEMM_WIDE && a.N % kWCols == 0 && a.M >= 8 * kWRows) {
    const int64_t nm = cdiv(a.M, kWRows), nn = a.N / kWCols;
    const dim3 wgrid = TDP_GEMM_GROUP_M > 0
                           ? dim3(static_cast<uint32_t>(cdiv(nm * nn, 8) * 8))
                           : dim3(static_cast<uint32_t>(nm), static_cast<uint32_t>(nn));
    // the large form, except for the read-modify-write epilogues (with one
    // wave per SIMD their load latency shows; measured slower than the wide
    // form there)
    // (its buffer descriptors cover a workgroup's rows of A and B^T, or all of
    // a head-major A, in 32-bit byte ranges)
    constexpr int64_t k4G = int64_t{1} << 32;
    const bool fits = (static_cast<int64_t>(kWRows) * a.lda + a.K) * 2 < k4G &&
                      (static_cast<int64_t>(kWCols) * a.ldb + a.K) * 2 < k4G &&
                      (hd == 0 || a.M * a.K * 2 < k4G);
    if (TDP_GEMM_BIG == 2 && EPI != kEpiResid && EPI != kEpiResidGate &&
        a.K % (kBK * kBStages) == 0 && fits) {
      const dim3 bgrid(static_cast<uint32_t>(cdiv(nm * nn, 8) * 8));
      if (TDP_GEMM_K64 && a.K % (2 * kRK) == 0 && a.K >= 4 * kRK) {
        // Tile order: groups of 4 row blocks walk down a column of tiles,
        // groups of 2 for outputs of 16384 or more columns (measured on the
        // block's shapes: FFN up, 16384 columns, 13.33 -> 12.95 ms with 2;
        // FFN down and QKV, 4096 and 12288 columns, 13.79 -> 15.03 and 9.07
        // -> 9.33 ms with 2; 8 slower for all three; 1 for FFN up 15.1
        // against 13.3 ms)
        GemmArgs b = a;
        b.group_m = a.N >= 16384 ? 2 : 4;
        const int slots = persistent_slots();
        if (slots == 0) return TDP_ERR_HIP;
        const int64_t T = nm * nn;
        const dim3 pgrid(static_cast<uint32_t>(std::min<int64_t>(cdiv(T, 8) * 8, slots)));
        // tiles per XCD in order; with a counter and at least 16 tiles per
        // workgroup, about 1/12 of the tiles are left to a claimed tail
        b.per_xcd = cdiv(T, 8);
        b.tail_claims = 0;
        if (a.tail_ctr && T >= 16 * static_cast<int64_t>(pgrid.x)) {
          b.per_xcd = (T - T / 12) / 8;
          b.tail_claims = static_cast<uint32_t>(T - 8 * b.per_xcd + pgrid.x);
        }
        if (hd == 0 && a.K >= 8192)
          hipLaunchKernelGGL((gemm_k64_kernel<EPI, 0, true>), pgrid, dim3(256), 0, stream, b);
        else if (hd == 0)
          hipLaunchKernelGGL((gemm_k64_kernel<EPI, 0>), pgrid, dim3(256), 0, stream, b);
        else if (hd == 64)
          hipLaunchKernelGGL((gemm_k64_kernel<EPI, 64>), pgrid, dim3(256), 0, stream, b);
        else
          hipLaunchKernelGGL((gemm_k64_kernel<EPI, 128>), pgrid, dim3(256), 0, stream, b);
      } else if (hd == 0)
        hipLaunchKernelGGL((gemm_big_kernel<EPI, 0>), bgrid, dim3(kBThreads), 0, stream, a);
      else if (hd == 64)
        hipLaunchKernelGGL((gemm_big_kernel<EPI, 64>), bgrid, dim3(kBThreads), 0, stream, a);
      else
        hipLaunchKernelGGL((gemm_big_kernel<EPI, 128>), bgrid, dim3(kBThreads), 0, stream, a);
      return launch_status();
    }
    if (hd == 0)
      hipLaunchKernelGGL((gemm_wide_kernel<EPI, 0>), wgrid, dim3(kGThreads), 0, stream, a);
    else if (hd == 64)
      hipLaunchKernelGGL((gemm_wide_kernel<EPI, 64>), wgrid, dim3(kGThreads), 0, stream, a);
    else
      hipLaunchKernelGGL((gemm_wide_kernel<EPI, 128>), wgrid, dim3(kGThreads), 0, stream, a);
    return launch_status();
  }
  // buffer-descriptor offsets of the inline-assembly loads: a workgroup's A
  // rows (one segment boundary at most in head-major A) plus a chunk's k
  // offset, and B^T's 128 rows plus k, all below 2^32
  constexpr int64_t k4G = int64_t{1} << 32;
  const int64_t a_span = hd > 0 ? 2 * (a.a_seg_rows * a.K * 2) + int64_t{kGRows} * hd * 2
                                : int64_t{kGRows} * a.lda * 2 + int64_t{a.K} * 2;
  const int64_t b_span = int64_t{kGCols} * a.ldb * 2 + int64_t{a.K} * 2;
  const bool asm_fits = a_span + 256 < k4G && b_span + 256 < k4G;
  if (asm_fits) {
    if (hd == 0)
      hipLaunchKernelGGL((gemm_kernel<EPI, 0>), grid, dim3(kGThreads), 0, stream, a);
    else if (hd == 64)
      hipLaunchKernelGGL((gemm_kernel<EPI, 64>), grid, dim3(kGThreads), 0, stream, a);
    else
      hipLaunchKernelGGL((gemm_kernel<EPI, 128>), grid, dim3(kGThreads), 0, stream, a);
  } else {
    if (hd == 0)
      hipLaunchKernelGGL((gemm_kernel<EPI, 0, false>), grid, dim3(kGThreads), 0, stream, a);
    else if (hd == 64)
      hipLaunchKernelGGL((gemm_kernel<EPI, 64, false>), grid, dim3(kGThreads), 0, stream, a);
    else
      hipLaunchKernelGGL((gemm_kernel<EPI, 128, false>), grid, dim3(kGThreads), 0, stream, a);
  }
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
             d.g0, d.g0_stride, d.g1, d.rows_per_batch, 4, 0, d.tail_ctr, 0};
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
