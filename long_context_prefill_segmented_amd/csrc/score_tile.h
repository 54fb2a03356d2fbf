// One 32x32 tile of chunk scores qbar . kbar^T on fp32 MFMA
// (v_mfma_f32_32x32x2f32), used by the chunk-score kernel.
//
// The contraction over the 128 dimensions is split by lane half: lanes 0-31
// feed d in [0,64), lanes 32-63 feed d in [64,128); the chain order is
// fixed, so scores are reproducible run to run.  The caller passes the
// lane's 64 floats of its query row (qv) and key row (kv) for its half.
// Result layout: lane -> key column (lane & 31); register r -> query row
// 8*(r/4) + 4*(lane/32) + r%4 of the tile.
#pragma once

#include "dhsa_internal.h"

namespace dhsa {

typedef float f32x16_t __attribute__((ext_vector_type(16)));

__device__ __forceinline__ f32x16_t score_tile(const float4* qv, const float4* kv) {
  f32x16_t acc;
#pragma unroll
  for (int r = 0; r < 16; ++r) acc[r] = 0.f;
#pragma unroll
  for (int u = 0; u < 16; ++u) {
    acc = __builtin_amdgcn_mfma_f32_32x32x2f32(qv[u].x, kv[u].x, acc, 0, 0, 0);
    acc = __builtin_amdgcn_mfma_f32_32x32x2f32(qv[u].y, kv[u].y, acc, 0, 0, 0);
    acc = __builtin_amdgcn_mfma_f32_32x32x2f32(qv[u].z, kv[u].z, acc, 0, 0, 0);
    acc = __builtin_amdgcn_mfma_f32_32x32x2f32(qv[u].w, kv[u].w, acc, 0, 0, 0);
  }
  return acc;
}

}  // namespace dhsa
