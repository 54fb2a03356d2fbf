// Chunk-by-chunk similarity: S[b,h,i,j] = qbar[b,h,i] . kbar[b,h/G,j], j <= i
// (gist.science Technical Summary, Methodology, Step 1: a chunk-level
// similarity matrix estimates the importance of chunk interactions).
//
// One wave computes one 32x32 tile of the lower triangle with fp32 MFMA
// (v_mfma_f32_32x32x2f32), accumulating over the 128 dimensions in a fixed
// order, so scores are reproducible run to run.  The contraction index is
// split by lane half: lanes 0-31 feed d in [0,64), lanes 32-63 feed d in
// [64,128), so each lane streams one contiguous 256-byte half row.
#include "score_tile.h"

namespace dhsa {
namespace {

struct ScoreGrid {
  int32_t stbase[kMaxBatch + 1];  // first tile of each sequence
};

__global__ __launch_bounds__(64) void scores_kernel(const float* __restrict__ qbar,
                                                    const float* __restrict__ kbar,
                                                    float* __restrict__ scores, int32_t hq,
                                                    int32_t hkv, SeqTable st, ScoreGrid sg) {
  const int x = blockIdx.x;
  const int b = find_seq(sg.stbase, st.batch, x);
  const int C = st.num_chunks[b];
  const int T = (C + 31) / 32;
  const int per_head = T * (T + 1) / 2;
  const int local = x - sg.stbase[b];
  const int h = local / per_head;
  const int tri = local - h * per_head;
  int ti = (int)((sqrtf(8.f * (float)tri + 1.f) - 1.f) * 0.5f);
  while (ti * (ti + 1) / 2 > tri) --ti;
  while ((ti + 1) * (ti + 2) / 2 <= tri) ++ti;
  const int tj = tri - ti * (ti + 1) / 2;
  const int i0 = ti * 32, j0 = tj * 32;
  const int G = hq / hkv;

  const int lane = threadIdx.x;
  const int row = lane & 31;
  const int half = lane >> 5;
  const bool qok = i0 + row < C;
  const bool kok = j0 + row < C;
  const float* qp = qbar + ((size_t)hq * st.cbase[b] + (size_t)h * C + (i0 + row)) * kHeadDim + 64 * half;
  const float* kp = kbar + ((size_t)hkv * st.cbase[b] + (size_t)(h / G) * C + (j0 + row)) * kHeadDim + 64 * half;

  float4 qv[16], kv[16];
  load_half_row(qp, qok, qv);
  load_half_row(kp, kok, kv);
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

}  // namespace

hipError_t launch_scores(const float* qbar, const float* kbar, float* scores,
                         int32_t hq, int32_t hkv, const SeqTable& st,
                         int64_t total_tiles, hipStream_t stream) {
  ScoreGrid sg;
  int64_t acc = 0;
  for (int b = 0; b < st.batch; ++b) {
    sg.stbase[b] = (int32_t)acc;
    const int64_t T = (st.num_chunks[b] + 31) / 32;
    acc += (int64_t)hq * T * (T + 1) / 2;
  }
  sg.stbase[st.batch] = (int32_t)acc;
  if (acc != total_tiles || acc <= 0) return acc <= 0 ? hipSuccess : hipErrorInvalidValue;
  hipLaunchKernelGGL(scores_kernel, dim3((unsigned)acc), dim3(64), 0, stream, qbar, kbar,
                     scores, hq, hkv, st, sg);
  return hipGetLastError();
}

}  // namespace dhsa
