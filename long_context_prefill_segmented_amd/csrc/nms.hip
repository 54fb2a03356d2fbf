// Boundary finalisation: greedy non-maximum suppression of per-token
// boundary scores into chunk offsets (gist.science Technical Summary,
// Methodology, "Dynamic Boundary Detection": the boundary predictor's output
// is finalised with NMS so that boundaries are well separated and robust to
// noise).
//
// Rule: token t (min_gap <= t <= L - min_gap) is a candidate when
// p[t] >= threshold.  Candidates are taken by score descending, then token
// ascending, and kept when every kept boundary -- the sequence ends 0 and L
// included -- is at least min_gap tokens away.
//
// The greedy order is sequential by definition; this kernel computes the same
// set in rounds.  In a round every live candidate that ranks above all other
// live or kept candidates closer than min_gap is kept, then every live
// candidate closer than min_gap to a kept one dies.  A candidate is decided
// exactly when every higher-ranked candidate near it is decided, and then as
// the greedy pass decides it, so the rounds end with the greedy set; each
// round keeps at least the highest-ranked live candidate, so they end.
// A round costs O(live candidates + kept * min_gap); the number of rounds is
// the longest chain of ever-higher candidates spaced under min_gap apart
// (a few for noisy peaks, up to L / min_gap for a monotone ramp).
//
// One workgroup per sequence.  The per-token state (0 none or dead, 1 live,
// 2 kept) and two live-candidate lists sit in the workspace; lists are
// compacted per wave with a ballot and one LDS atomic, since their order does
// not matter; the final pass compacts kept tokens in token order.
#include "dhsa_internal.h"

namespace dhsa {
namespace {

constexpr int kNmsThreads = 1024;
constexpr int kNmsWaves = kNmsThreads / 64;

__device__ __forceinline__ bool ranks_above(float pa, int a, float pb, int b) {
  return pa > pb || (pa == pb && a < b);
}

__device__ __forceinline__ uint64_t lanes_below(int lane) {
  return lane ? ((~0ull) >> (64 - lane)) : 0ull;
}

__global__ __launch_bounds__(kNmsThreads) void nms_kernel(
    const float* __restrict__ scores, int32_t seq_len, int32_t min_gap, float threshold,
    int32_t* __restrict__ offsets_out, int32_t stride, int32_t* __restrict__ num_chunks_out,
    uint8_t* state_ws, int32_t* list_ws, int64_t state_stride) {
  __shared__ int s_count;
  __shared__ int s_wsum[kNmsWaves];
  const int b = blockIdx.x;
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const int L = seq_len, g = min_gap;
  const float* p = scores + (size_t)b * L;
  uint8_t* st = state_ws + (size_t)b * state_stride;
  int32_t* la = list_ws + (size_t)b * 2 * L;
  int32_t* lb = la + L;

  // ---- candidates
  if (tid == 0) s_count = 0;
  __syncthreads();
  for (int t0 = 0; t0 < L; t0 += kNmsThreads) {
    const int t = t0 + tid;
    bool cand = false;
    if (t < L) {
      cand = t >= g && t <= L - g && p[t] >= threshold;
      st[t] = cand ? 1 : 0;
    }
    const uint64_t m = __ballot(cand);
    int base = 0;
    if (lane == 0 && m) base = atomicAdd(&s_count, __popcll(m));
    base = __shfl(base, 0);
    if (cand) la[base + __popcll(m & lanes_below(lane))] = t;
  }
  __syncthreads();
  int n = s_count;
  __syncthreads();

  // ---- rounds
  while (n > 0) {
    // keep every live candidate that no live or kept neighbour outranks
    for (int idx = tid; idx < n; idx += kNmsThreads) {
      const int t = la[idx];
      const float pt = p[t];
      const int lo = t - g + 1 > 0 ? t - g + 1 : 0;
      const int hi = t + g - 1 < L - 1 ? t + g - 1 : L - 1;
      bool top = true;
      for (int u = lo; u <= hi; ++u) {
        if (u != t && st[u] != 0 && ranks_above(p[u], u, pt, t)) {
          top = false;
          break;
        }
      }
      if (top) st[t] = 2;
    }
    __syncthreads();
    // each candidate kept in this round retires the live ones near it (two
    // kept candidates may share such a neighbour: both write the same 0)
    for (int idx = tid; idx < n; idx += kNmsThreads) {
      const int t = la[idx];
      if (st[t] != 2) continue;
      const int lo = t - g + 1 > 0 ? t - g + 1 : 0;
      const int hi = t + g - 1 < L - 1 ? t + g - 1 : L - 1;
      for (int u = lo; u <= hi; ++u)
        if (st[u] == 1) st[u] = 0;
    }
    if (tid == 0) s_count = 0;
    __syncthreads();
    // the still-live candidates go to the next round
    for (int i0 = 0; i0 < n; i0 += kNmsThreads) {
      const int idx = i0 + tid;
      int t = 0;
      bool live = false;
      if (idx < n) {
        t = la[idx];
        live = st[t] == 1;
      }
      const uint64_t m = __ballot(live);
      int base = 0;
      if (lane == 0 && m) base = atomicAdd(&s_count, __popcll(m));
      base = __shfl(base, 0);
      if (live) lb[base + __popcll(m & lanes_below(lane))] = t;
    }
    __syncthreads();
    n = s_count;
    int32_t* tmp = la;
    la = lb;
    lb = tmp;
    __syncthreads();
  }

  // ---- kept tokens in token order -> offsets 0, kept..., L
  int32_t* out = offsets_out + (size_t)b * stride;
  int carry = 1;  // out[0] = 0
  for (int t0 = 0; t0 < L; t0 += kNmsThreads) {
    const int t = t0 + tid;
    const bool kept = t < L && st[t] == 2;
    const uint64_t m = __ballot(kept);
    if (lane == 0) s_wsum[wv] = __popcll(m);
    __syncthreads();
    int before = carry, total = carry;
    for (int w = 0; w < kNmsWaves; ++w) {
      before += w < wv ? s_wsum[w] : 0;
      total += s_wsum[w];
    }
    if (kept) out[before + __popcll(m & lanes_below(lane))] = t;
    carry = total;
    __syncthreads();
  }
  if (tid == 0) {
    out[0] = 0;
    out[carry] = L;
    num_chunks_out[b] = carry;
  }
}

}  // namespace

hipError_t launch_nms(const float* scores, int32_t batch, int32_t seq_len, int32_t min_gap,
                      float threshold, int32_t* offsets_out, int32_t stride,
                      int32_t* num_chunks_out, void* workspace, int64_t state_stride,
                      hipStream_t stream) {
  uint8_t* state = static_cast<uint8_t*>(workspace);
  int32_t* lists = reinterpret_cast<int32_t*>(state + (size_t)batch * state_stride);
  hipLaunchKernelGGL(nms_kernel, dim3(batch), dim3(kNmsThreads), 0, stream, scores, seq_len,
                     min_gap, threshold, offsets_out, stride, num_chunks_out, state, lists,
                     state_stride);
  return hipGetLastError();
}

}  // namespace dhsa
