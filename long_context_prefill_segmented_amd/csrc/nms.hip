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
// A round costs O(live candidates * min_gap / 16); the number of rounds is
// the longest chain of ever-higher candidates spaced under min_gap apart
// (a few for noisy peaks, up to L / min_gap for a monotone ramp).
//
// One workgroup per sequence.  Every token's state (0 none or dead, 1 live,
// 2 kept) is a 2-bit field in LDS, 16 tokens to a 32-bit word, so a
// neighbourhood of 2 min_gap - 1 tokens is a handful of word reads and the
// live candidates near a token are found with bit operations; a transition
// is one LDS atomic on its word.  The live-candidate lists sit in the
// workspace (their order does not matter: waves append with one LDS atomic);
// the final pass emits kept tokens in token order with a block-wide scan.
#include "dhsa_internal.h"

namespace dhsa {
namespace {

constexpr int kNmsThreads = 1024;
constexpr int kNmsWaves = kNmsThreads / 64;
constexpr int kNmsWords = kNmsMaxLen / 16;  // 2 bits per token

__device__ __forceinline__ bool ranks_above(float pa, int a, float pb, int b) {
  return pa > pb || (pa == pb && a < b);
}

__device__ __forceinline__ uint64_t lanes_below(int lane) {
  return lane ? ((~0ull) >> (64 - lane)) : 0ull;
}

// exclusive prefix sum across the wave, and the wave's total
__device__ __forceinline__ int wave_excl_scan(int v, int lane, int* total) {
  int incl = v;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const int y = __shfl_up(incl, off, 64);
    if (lane >= off) incl += y;
  }
  *total = __shfl(incl, 63, 64);
  return incl - v;
}

// both bits of the 2-bit fields of word wd whose tokens lie in [lo, hi]
__device__ __forceinline__ uint32_t range_fields(int wd, int lo, int hi) {
  const int f0 = lo > 16 * wd ? lo - 16 * wd : 0;
  const int f1 = hi < 16 * wd + 15 ? hi - 16 * wd : 15;
  const uint32_t upto = f1 == 15 ? 0xffffffffu : ((1u << (2 * f1 + 2)) - 1u);
  const uint32_t below = (1u << (2 * f0)) - 1u;
  return upto & ~below;
}

__device__ __forceinline__ uint32_t field_of(const uint32_t* sw, int t) {
  return (sw[t >> 4] >> (2 * (t & 15))) & 3u;
}

__global__ __launch_bounds__(kNmsThreads) void nms_kernel(
    const float* __restrict__ scores, int32_t seq_len, int32_t min_gap, float threshold,
    int32_t* __restrict__ offsets_out, int32_t stride, int32_t* __restrict__ num_chunks_out,
    int32_t* list_ws) {
  __shared__ uint32_t sw[kNmsWords];
  __shared__ int s_count;
  __shared__ int s_wsum[kNmsWaves];
  const int b = blockIdx.x;
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const int L = seq_len, g = min_gap;
  const int nw = (L + 15) / 16;
  const float* p = scores + (size_t)b * L;
  int32_t* la = list_ws + (size_t)b * 2 * L;
  int32_t* lb = la + L;

  // ---- candidates: kWordsPerStep state words (16 tokens each) per thread
  // and step, their score loads all issued before any is used
  if (tid == 0) s_count = 0;
  __syncthreads();
  const bool vec_ok = (reinterpret_cast<uintptr_t>(p) & 15) == 0;
  constexpr int kWordsPerStep = 4;
  for (int w0 = 0; w0 < nw; w0 += kWordsPerStep * kNmsThreads) {
    float x[kWordsPerStep][16];
#pragma unroll
    for (int j = 0; j < kWordsPerStep; ++j) {
      const int w = w0 + j * kNmsThreads + tid;
      const int t0 = 16 * w;
      if (w < nw && vec_ok && t0 + 16 <= L) {
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const float4 f = *reinterpret_cast<const float4*>(p + t0 + 4 * e);
          x[j][4 * e] = f.x;
          x[j][4 * e + 1] = f.y;
          x[j][4 * e + 2] = f.z;
          x[j][4 * e + 3] = f.w;
        }
      } else {
#pragma unroll
        for (int e = 0; e < 16; ++e) x[j][e] = (w < nw && t0 + e < L) ? p[t0 + e] : 0.f;
      }
    }
#pragma unroll
    for (int j = 0; j < kWordsPerStep; ++j) {
      const int w = w0 + j * kNmsThreads + tid;
      const int t0 = 16 * w;
      uint32_t word = 0;
      int cnt = 0;
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        const int t = t0 + e;
        const bool cand = w < nw && t >= g && t <= L - g && x[j][e] >= threshold;
        word |= cand ? (1u << (2 * e)) : 0u;
        cnt += cand ? 1 : 0;
      }
      if (w < nw) sw[w] = word;
      int wtotal;
      const int ex = wave_excl_scan(cnt, lane, &wtotal);
      int base = 0;
      if (lane == 0 && wtotal) base = atomicAdd(&s_count, wtotal);
      base = __shfl(base, 0, 64) + ex;
      while (word) {
        la[base++] = t0 + (__builtin_ctz(word) >> 1);
        word &= word - 1;
      }
    }
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
      for (int wd = lo >> 4; wd <= (hi >> 4) && top; ++wd) {
        uint32_t x = sw[wd] & range_fields(wd, lo, hi);
        if (wd == (t >> 4)) x &= ~(3u << (2 * (t & 15)));
        uint32_t nz = (x | (x >> 1)) & 0x55555555u;  // live or kept fields
        while (nz) {
          const int u = 16 * wd + (__builtin_ctz(nz) >> 1);
          if (ranks_above(p[u], u, pt, t)) {
            top = false;
            break;
          }
          nz &= nz - 1;
        }
      }
      if (top) atomicXor(&sw[t >> 4], 3u << (2 * (t & 15)));  // live -> kept
    }
    __syncthreads();
    // each candidate kept in this round retires the live ones near it
    for (int idx = tid; idx < n; idx += kNmsThreads) {
      const int t = la[idx];
      if (field_of(sw, t) != 2u) continue;
      const int lo = t - g + 1 > 0 ? t - g + 1 : 0;
      const int hi = t + g - 1 < L - 1 ? t + g - 1 : L - 1;
      for (int wd = lo >> 4; wd <= (hi >> 4); ++wd) {
        const uint32_t x = sw[wd];
        const uint32_t live = x & ~(x >> 1) & 0x55555555u & range_fields(wd, lo, hi);
        if (live) atomicAnd(&sw[wd], ~(live | (live << 1)));
      }
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
        live = field_of(sw, t) == 1u;
      }
      const uint64_t m = __ballot(live);
      int base = 0;
      if (lane == 0 && m) base = atomicAdd(&s_count, __popcll(m));
      base = __shfl(base, 0, 64);
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
  for (int w0 = 0; w0 < nw; w0 += kNmsThreads) {
    const int w = w0 + tid;
    uint32_t kept = w < nw ? (sw[w] >> 1) & 0x55555555u : 0u;
    int wtotal;
    const int ex = wave_excl_scan(__popc(kept), lane, &wtotal);
    if (lane == 0) s_wsum[wv] = wtotal;
    __syncthreads();
    int before = carry, total = carry;
    for (int x = 0; x < kNmsWaves; ++x) {
      before += x < wv ? s_wsum[x] : 0;
      total += s_wsum[x];
    }
    int pos = before + ex;
    while (kept) {
      out[pos++] = 16 * w + (__builtin_ctz(kept) >> 1);
      kept &= kept - 1;
    }
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
                      int32_t* num_chunks_out, void* workspace, hipStream_t stream) {
  hipLaunchKernelGGL(nms_kernel, dim3(batch), dim3(kNmsThreads), 0, stream, scores, seq_len,
                     min_gap, threshold, offsets_out, stride, num_chunks_out,
                     static_cast<int32_t*>(workspace));
  return hipGetLastError();
}

}  // namespace dhsa
