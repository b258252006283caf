// Shared device/host helpers of the gfx950 kernels (internal header).
#pragma once

#include <hip/hip_runtime.h>

#include <cstddef>
#include <cstdint>

#include "tdp.h"

namespace tdp {

typedef __bf16 bf16;
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

constexpr int kWave = 64;

inline bool aligned16(const void *p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

inline tdp_status launch_status() {
  return hipGetLastError() == hipSuccess ? TDP_OK : TDP_ERR_HIP;
}

inline hipStream_t as_stream(void *s) { return reinterpret_cast<hipStream_t>(s); }

// v_mfma_f32_32x32x16_bf16: D[32][32] += A[32][16] * B[16][32].
// Lane l supplies A[l%32][8*(l/32) + 0..7] and B[8*(l/32) + 0..7][l%32]; it
// receives D[8*(v/4) + 4*(l/32) + v%4][l%32] in element v (0..15).
__device__ __forceinline__ f32x16 mfma32(bf16x8 a, bf16x8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

}  // namespace tdp
