// Chunk-by-chunk similarity: S[b,h,i,j] = qbar[b,h,i] . kbar[b,h/G,j], j <= i
// (gist.science Technical Summary, Methodology, Step 1: a chunk-level
// similarity matrix estimates the importance of chunk interactions).
//
// One wave computes one 32x32 tile of the lower triangle with fp32 MFMA
// (v_mfma_f32_32x32x2f32), accumulating over the 128 dimensions in a fixed
// order, so scores are reproducible run to run.  The contraction index is
// split by lane half: lanes 0-31 feed d in [0,64), lanes 32-63 feed d in
// [64,128).
//
// In that operand layout each lane owns one row, so loading it straight from
// memory makes every 64-lane load touch 64 cache lines.  The 32 key rows and
// the 32 query rows are instead read row-contiguously (each load instruction
// covers two whole 512-byte rows) into an LDS block padded by 16 bytes per
// row, and each lane takes its half row from there.
//
// The query heads of one KV head share the key block, so a wave computes the
// tile for hpw consecutive query heads of a group in turn, staging the key
// block once.  The host picks hpw (a divisor of the group size) so that the
// grid keeps at least one and a half waves per SIMD; each head's tile is
// computed exactly as with hpw = 1.  At 128K (hpw = 2) the 1,680 waves fit
// the GPU at once, where 3,360 single-head waves needed a second round
// (25.6 -> 20.2 us).  Loading the next head's query rows during the current
// head's MFMA chain holds 64 more registers (one wave per SIMD) and measured
// slower (23.5 us).
#include "score_tile.h"

namespace dhsa {
namespace {

struct ScoreGrid {
  int32_t stbase[kMaxBatch + 1];  // first tile of each sequence
};

constexpr int kStageStride = kHeadDim / 4 + 1;  // float4 per staged row (one of padding)
constexpr int64_t kScoreMinWaves = 1536;       // waves the grid should keep at least

// Rows r0 .. r0+31 of a [*, 128] fp32 matrix (rows >= nrows read as zero),
// row-contiguous: load u of a lane holds row 2u + lane/32, floats
// 4 * (lane & 31) .., so each load instruction covers two whole rows.
__device__ __forceinline__ void load_rows(const float* base, int r0, int nrows, int lane,
                                          float4* t) {
  const float4* src = reinterpret_cast<const float4*>(base);
#pragma unroll
  for (int u = 0; u < 16; ++u) {
    const int r = 2 * u + (lane >> 5);
    t[u] = r0 + r < nrows ? src[(size_t)(r0 + r) * (kHeadDim / 4) + (lane & 31)]
                          : make_float4(0.f, 0.f, 0.f, 0.f);
  }
}

// The rows held by load_rows into this lane's operand half row v[0..15] (row
// lane & 31, floats 64 * (lane >> 5) ..), through the LDS block stage.
__device__ __forceinline__ void to_operand(const float4* t, int lane, float4* stage, float4* v) {
  __syncthreads();  // the previous block's reads are done
#pragma unroll
  for (int u = 0; u < 16; ++u) stage[(2 * u + (lane >> 5)) * kStageStride + (lane & 31)] = t[u];
  __syncthreads();
#pragma unroll
  for (int u = 0; u < 16; ++u) v[u] = stage[(lane & 31) * kStageStride + 16 * (lane >> 5) + u];
}

__global__ __launch_bounds__(64) void scores_kernel(const float* __restrict__ qbar,
                                                    const float* __restrict__ kbar,
                                                    float* __restrict__ scores, int32_t hq,
                                                    int32_t hkv, SeqTable st, ScoreGrid sg,
                                                    int32_t hpw) {
  const int x = blockIdx.x;
  const int b = find_seq(sg.stbase, st.batch, x);
  const int C = st.num_chunks[b];
  const int T = (C + 31) / 32;
  const int per_head = T * (T + 1) / 2;
  const int local = x - sg.stbase[b];
  const int hb = local / per_head;  // query heads hb*hpw .. hb*hpw + hpw - 1
  const int tri = local - hb * per_head;
  int ti = (int)((sqrtf(8.f * (float)tri + 1.f) - 1.f) * 0.5f);
  while (ti * (ti + 1) / 2 > tri) --ti;
  while ((ti + 1) * (ti + 2) / 2 <= tri) ++ti;
  const int tj = tri - ti * (ti + 1) / 2;
  const int i0 = ti * 32, j0 = tj * 32;
  const int G = hq / hkv;
  const int h0 = hb * hpw;

  const int lane = threadIdx.x;
  const int row = lane & 31;
  const int half = lane >> 5;
  const float* qbase = qbar + (size_t)hq * st.cbase[b] * kHeadDim;
  const float* kp = kbar + ((size_t)hkv * st.cbase[b] + (size_t)(h0 / G) * C) * kHeadDim;

  __shared__ float4 stage[32 * kStageStride];
  float4 t[16], qv[16], kv[16];
  load_rows(kp, j0, C, lane, t);
  to_operand(t, lane, stage, kv);
  for (int e = 0; e < hpw; ++e) {
    const int h = h0 + e;
    load_rows(qbase + (size_t)h * C * kHeadDim, i0, C, lane, t);
    to_operand(t, lane, stage, qv);
    const f32x16_t acc = score_tile(qv, kv);
    // accumulator layout: lane -> column j0 + (lane & 31); register r -> row
    // i0 + 8*(r/4) + 4*(lane/32) + r%4
    float* sp = scores + st.sbase[b] + (size_t)h * C * C;
    const int j = j0 + row;
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int i = i0 + 8 * (r >> 2) + 4 * half + (r & 3);
      if (i < C && j <= i) sp[(size_t)i * C + j] = acc[r];
    }
  }
}

}  // namespace

hipError_t launch_scores(const float* qbar, const float* kbar, float* scores,
                         int32_t hq, int32_t hkv, const SeqTable& st,
                         int64_t total_tiles, hipStream_t stream) {
  int64_t per_head_total = 0;
  for (int b = 0; b < st.batch; ++b) {
    const int64_t T = (st.num_chunks[b] + 31) / 32;
    per_head_total += T * (T + 1) / 2;
  }
  if ((int64_t)hq * per_head_total != total_tiles) return hipErrorInvalidValue;
  if (total_tiles <= 0) return hipSuccess;
  // heads per wave: the largest divisor of the group size that still leaves
  // one and a half waves of work per SIMD (256 CUs x 4 SIMDs)
  const int G = hq / hkv;
  int hpw = 1;
  for (int d = G; d > 1; --d) {
    if (G % d == 0 && (int64_t)(hq / d) * per_head_total >= kScoreMinWaves) {
      hpw = d;
      break;
    }
  }
  ScoreGrid sg;
  int64_t acc = 0;
  for (int b = 0; b < st.batch; ++b) {
    sg.stbase[b] = (int32_t)acc;
    const int64_t T = (st.num_chunks[b] + 31) / 32;
    acc += (int64_t)(hq / hpw) * T * (T + 1) / 2;
  }
  sg.stbase[st.batch] = (int32_t)acc;
  hipLaunchKernelGGL(scores_kernel, dim3((unsigned)acc), dim3(64), 0, stream, qbar, kbar,
                     scores, hq, hkv, st, sg, hpw);
  return hipGetLastError();
}

}  // namespace dhsa
