// Per-row causal chunk selection (device side) for the top-k kernel.
//
// Row (b,h,i) with budget k and recent window w keeps chunk i, the w chunks
// just before it, and the k-1 highest-scoring chunks among the older ones
// (j < i - w); when i + 1 <= k + w it keeps every chunk 0..i.  With w = 0
// this is the fixed-budget rule: the diagonal plus the k-1 best earlier
// chunks (gist.science Technical Summary, Methodology, Step 2: each query
// chunk is routed to its highest-scoring chunks under the causal constraint;
// DHSA README, "Predictor Checkpoints": fixed and query-dependent row
// budgets; the codewithpapers record of the repository names a recent-block
// keep OR'ed with a scattered top-k by row budget).  The order is total:
// score descending, then chunk index ascending; -0 and +0 are equal; NaN
// ranks below every number.
//
// One wavefront owns one row.  Candidate j sits in lane j % 64, slot j / 64,
// as an order-preserving 32-bit key of its score.  The k-1 winners are found
// by a threshold search rather than k-1 arg-max rounds: a binary search over
// the key bits, from the top, keeps the largest threshold T with at least
// k-1 candidates >= T (each count a ballot and popcount per slot).  It stops
// as soon as exactly k-1 candidates are >= T; otherwise T ends as the
// (k-1)-th largest key, every candidate above T is kept and the remaining
// places go to the candidates equal to T with the lowest chunk indices.
// Either way the kept set is the first k-1 in the order score descending,
// index ascending.  The winners are emitted in ascending index order by a
// ballot and prefix popcount per slot; the window chunks i-w..i follow them.
#pragma once

#include "dhsa_internal.h"

namespace dhsa {

__device__ __forceinline__ uint32_t order_key(float s) {
  s = s + 0.0f;  // -0 -> +0
  const uint32_t u = __float_as_uint(s);
  if (s != s) return 1u;  // NaN: below every number, above empty slots
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

// entries in rows 0..i-1 of one head when every row keeps min(k, i'+1):
// sum_{i' < i} min(k, i'+1)  (k = budget + recent window)
__device__ __forceinline__ int64_t entries_before(int64_t i, int64_t k) {
  return i <= k ? i * (i + 1) / 2 : k * (k + 1) / 2 + (i - k) * k;
}

// Writes the kept chunks of row i (ascending) to out[0 .. min(k+w, i+1)-1];
// srow[j] is the score of key chunk j (j < i - w are read).  All 64 lanes
// of the wave call it together; k >= 1, w >= 0.
template <int NS>
__device__ __forceinline__ void select_row(const float* srow, int i, int k, int w, int lane,
                                           int32_t* out) {
  if (i + 1 <= k + w) {
    for (int j = lane; j <= i; j += 64) out[j] = j;
    return;
  }
  const int older = i - w;  // candidates j < older; older >= k >= 1
  uint32_t key[NS];
#pragma unroll
  for (int s = 0; s < NS; ++s) {
    const int j = lane + 64 * s;
    key[s] = j < older ? order_key(srow[j]) : 0u;  // 0: empty slot
  }
  // candidates with key >= y, across the wave (wave-uniform)
  auto count_ge = [&](uint32_t y) {
    int c = 0;
#pragma unroll
    for (int s = 0; s < NS; ++s) c += __popcll(__ballot(key[s] >= y));
    return c;
  };
  const int need = k - 1;  // older >= k real candidates (keys >= 1) exist
  uint32_t thr = 0;
  int cthr = 64 * NS;      // count_ge(thr)
  for (int bit = 31; bit >= 0 && need > 0; --bit) {
    const uint32_t y = thr | (1u << bit);
    const int c = count_ge(y);
    if (c >= need) {
      thr = y;
      cthr = c;
      if (c == need) break;
    }
  }
  uint32_t taken = 0;
  if (need > 0) {
    if (cthr == need) {
#pragma unroll
      for (int s = 0; s < NS; ++s) taken |= (key[s] >= thr ? 1u : 0u) << s;
    } else {
      // thr is the need-th largest key: keep the keys above it, then the
      // lowest-index keys equal to it (slot-major order is index order)
      int rem = need - count_ge(thr + 1u);
#pragma unroll
      for (int s = 0; s < NS; ++s) {
        const bool eq = key[s] == thr;
        const uint64_t m = __ballot(eq);
        const uint64_t below = lane ? (m & ((~0ull) >> (64 - lane))) : 0ull;
        const bool sel = (key[s] > thr) || (eq && (int)__popcll(below) < rem);
        taken |= (sel ? 1u : 0u) << s;
        const int pm = __popcll(m);
        rem -= pm < rem ? pm : rem;
      }
    }
  }
  // emit ascending: slot-major is index order
  int base = 0;
#pragma unroll
  for (int s = 0; s < NS; ++s) {
    const bool sel = (taken >> s) & 1u;
    const uint64_t m = __ballot(sel);
    if (sel) {
      const uint64_t below = lane ? (m & ((~0ull) >> (64 - lane))) : 0ull;
      out[base + __popcll(below)] = lane + 64 * s;
    }
    base += __popcll(m);
  }
  // the recent window and the diagonal: chunks older..i
  for (int t = lane; t <= w; t += 64) out[k - 1 + t] = older + t;
}

}  // namespace dhsa
