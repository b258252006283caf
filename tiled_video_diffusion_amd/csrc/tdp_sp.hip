// The head exchange of sequence parallelism (SP) on gfx950: a rank's token
// slice of Q, K or V (all heads) goes to every rank's buffer of all tokens x
// its heads, and the inverse for the attention output.
//
// LTX-2 sequence-parallel guide (the section on how a denoising step is
// split, and the one on the all2all kernel): tokens are split evenly over
// the W ranks; before self-attention an all2all gives every rank all tokens
// of H/W heads, and a second one returns each token slice's outputs for all
// heads; the kernel writes straight into the destination GPU's buffer and
// assigns its compute units to destination ranks in turn.  Here the
// destinations are plain device pointers: buffers of this GPU (the one-GPU
// build and its tests) or peer buffers mapped into this process, which the
// same kernel writes over the GPU links.  The guide's cross-GPU completion
// counters are not part of this file (one GPU).
//
// Layouts (row-major): a rank's slice [t_loc][H][d]; a rank's head buffer
// [W t_loc][H/W][d], token t of rank r at row r t_loc + t.  A token's H/W
// heads are one contiguous segment of H/W * d elements on both sides, so the
// exchange is a copy of whole segments in 16-byte pieces.
#include "tdp_internal.h"

namespace tdp {
namespace {

constexpr int kSpThreads = 256;
constexpr int kSpTokens = 16;          // tokens per workgroup
constexpr int kSpMaxWorld = 16;

struct SpPtrs {
  char *p[kSpMaxWorld];
};

// Workgroup b: peer s = b % world, tokens [(b / world) kSpTokens, +kSpTokens)
// of this rank's slice (consecutive workgroups serve different peers).
// send: dst[s] row (rank t_loc + t) <- src row t, heads of s;
// gather: dst row t, heads of s <- src[s] row (rank t_loc + t).
template <bool SEND>
__global__ __launch_bounds__(kSpThreads) void sp_exchange_kernel(
    const char *__restrict__ local_src, char *__restrict__ local_dst, SpPtrs peers,
    int64_t t_loc, int32_t world, int32_t rank, int64_t seg_bytes) {
  const int32_t s = static_cast<int32_t>(blockIdx.x % static_cast<uint32_t>(world));
  const int64_t t0 = static_cast<int64_t>(blockIdx.x / static_cast<uint32_t>(world)) * kSpTokens;
  const int64_t vpt = seg_bytes / 16;               // 16-byte pieces per segment
  const int64_t row_bytes = seg_bytes * world;      // one token of the slice
  const int64_t n = min(static_cast<int64_t>(kSpTokens), t_loc - t0) * vpt;
  for (int64_t i = threadIdx.x; i < n; i += kSpThreads) {
    const int64_t t = t0 + i / vpt, v = i - (i / vpt) * vpt;
    const int64_t slice_off = t * row_bytes + s * seg_bytes + 16 * v;
    const int64_t peer_off = (static_cast<int64_t>(rank) * t_loc + t) * seg_bytes + 16 * v;
    if constexpr (SEND) {
      const uint4 x = *reinterpret_cast<const uint4 *>(local_src + slice_off);
      *reinterpret_cast<uint4 *>(peers.p[s] + peer_off) = x;
    } else {
      const uint4 x = *reinterpret_cast<const uint4 *>(peers.p[s] + peer_off);
      *reinterpret_cast<uint4 *>(local_dst + slice_off) = x;
    }
  }
}

int esize_of(int32_t dtype) { return dtype == TDP_F32 ? 4 : (dtype == TDP_BF16 ? 2 : 0); }

tdp_status check(int32_t dtype, int64_t t_loc, int32_t heads, int32_t head_dim, int32_t world,
                 int32_t rank, int64_t *seg_bytes) {
  const int es = esize_of(dtype);
  if (es == 0) return TDP_ERR_UNSUPPORTED;
  if (t_loc < 0 || heads < 1 || head_dim < 1 || world < 1 || rank < 0 || rank >= world)
    return TDP_ERR_ARG;
  if (world > kSpMaxWorld || heads % world != 0) return TDP_ERR_UNSUPPORTED;
  *seg_bytes = static_cast<int64_t>(heads / world) * head_dim * es;
  if (*seg_bytes % 16 != 0) return TDP_ERR_UNSUPPORTED;
  const int64_t nblk = (t_loc + kSpTokens - 1) / kSpTokens * world;
  if (nblk > INT32_MAX) return TDP_ERR_ARG;
  return TDP_OK;
}

template <bool SEND>
tdp_status launch(const void *local_src, void *local_dst, const void *const *peers, int64_t t_loc,
                  int32_t world, int32_t rank, int64_t seg_bytes, void *hip_stream) {
  SpPtrs pp{};
  for (int32_t s = 0; s < world; ++s) {
    if (!peers[s]) return TDP_ERR_NULL;
    if (!aligned16(peers[s])) return TDP_ERR_ALIGN;
    pp.p[s] = static_cast<char *>(const_cast<void *>(peers[s]));
  }
  if (t_loc == 0) return TDP_OK;
  const int64_t nblk = (t_loc + kSpTokens - 1) / kSpTokens * world;
  hipLaunchKernelGGL(sp_exchange_kernel<SEND>, dim3(static_cast<uint32_t>(nblk)),
                     dim3(kSpThreads), 0, as_stream(hip_stream),
                     static_cast<const char *>(local_src), static_cast<char *>(local_dst), pp,
                     t_loc, world, rank, seg_bytes);
  return launch_status();
}

}  // namespace
}  // namespace tdp

using namespace tdp;

extern "C" tdp_status tdp_sp_send_heads(const void *src, int32_t dtype, int64_t t_loc,
                                        int32_t heads, int32_t head_dim, int32_t world,
                                        int32_t rank, void *const *dst, void *hip_stream) {
  int64_t seg = 0;
  const tdp_status s = check(dtype, t_loc, heads, head_dim, world, rank, &seg);
  if (s != TDP_OK) return s;
  if (!dst || (t_loc > 0 && !src)) return TDP_ERR_NULL;
  if (t_loc > 0 && !aligned16(src)) return TDP_ERR_ALIGN;
  return launch<true>(src, nullptr, dst, t_loc, world, rank, seg, hip_stream);
}

extern "C" tdp_status tdp_sp_gather_heads(const void *const *src, int32_t dtype, int64_t t_loc,
                                          int32_t heads, int32_t head_dim, int32_t world,
                                          int32_t rank, void *dst, void *hip_stream) {
  int64_t seg = 0;
  const tdp_status s = check(dtype, t_loc, heads, head_dim, world, rank, &seg);
  if (s != TDP_OK) return s;
  if (!src || (t_loc > 0 && !dst)) return TDP_ERR_NULL;
  if (t_loc > 0 && !aligned16(dst)) return TDP_ERR_ALIGN;
  return launch<false>(nullptr, dst, src, t_loc, world, rank, seg, hip_stream);
}
