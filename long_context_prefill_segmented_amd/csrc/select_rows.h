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
// as an order-preserving 32-bit key of its score.  Each of the k-1 rounds
// takes every lane's best untaken candidate, reduces the keys across the
// wave with DPP moves, and picks the holder of the maximum (the lowest chunk
// index when several lanes hold it).  The winners are emitted in ascending
// index order by a ballot and prefix popcount per slot; the window chunks
// i-w..i follow them.
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

// Wave-wide max / min of a 32-bit value with DPP lane moves (no LDS round
// trip): quad swaps, half-row and row mirrors, then row broadcasts carry the
// result to lane 63, which is read back as a uniform value.
__device__ __forceinline__ uint32_t wave_max_u32(uint32_t v) {
  uint32_t t;
  t = (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0xB1, 0xF, 0xF, false);   // quad [1,0,3,2]
  v = v > t ? v : t;
  t = (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x4E, 0xF, 0xF, false);   // quad [2,3,0,1]
  v = v > t ? v : t;
  t = (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x141, 0xF, 0xF, false);  // row half mirror
  v = v > t ? v : t;
  t = (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x140, 0xF, 0xF, false);  // row mirror
  v = v > t ? v : t;
  t = (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x142, 0xA, 0xF, false);  // row bcast 15
  v = v > t ? v : t;
  t = (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x143, 0xC, 0xF, false);  // row bcast 31
  v = v > t ? v : t;
  return (uint32_t)__builtin_amdgcn_readlane((int)v, 63);
}

__device__ __forceinline__ uint32_t wave_min_u32(uint32_t v) {
  uint32_t t;
  t = (uint32_t)__builtin_amdgcn_update_dpp(-1, (int)v, 0xB1, 0xF, 0xF, false);
  v = v < t ? v : t;
  t = (uint32_t)__builtin_amdgcn_update_dpp(-1, (int)v, 0x4E, 0xF, 0xF, false);
  v = v < t ? v : t;
  t = (uint32_t)__builtin_amdgcn_update_dpp(-1, (int)v, 0x141, 0xF, 0xF, false);
  v = v < t ? v : t;
  t = (uint32_t)__builtin_amdgcn_update_dpp(-1, (int)v, 0x140, 0xF, 0xF, false);
  v = v < t ? v : t;
  t = (uint32_t)__builtin_amdgcn_update_dpp(-1, (int)v, 0x142, 0xA, 0xF, false);
  v = v < t ? v : t;
  t = (uint32_t)__builtin_amdgcn_update_dpp(-1, (int)v, 0x143, 0xC, 0xF, false);
  v = v < t ? v : t;
  return (uint32_t)__builtin_amdgcn_readlane((int)v, 63);
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
  uint32_t taken = 0;
  for (int round = 0; round < k - 1; ++round) {
    // this lane's best untaken candidate (the lowest slot among equal keys)
    uint32_t best = 0;
    int bslot = 0;
#pragma unroll
    for (int s = 0; s < NS; ++s) {
      const uint32_t kv = ((taken >> s) & 1u) ? 0u : key[s];
      if (kv > best) {
        best = kv;
        bslot = s;
      }
    }
    const uint32_t top = wave_max_u32(best);
    const uint64_t holders = __ballot(best == top);
    int wl;
    if (__popcll(holders) == 1) {
      wl = __ffsll((long long)holders) - 1;
    } else {  // equal keys in several lanes: the lowest chunk index wins
      const uint32_t j = best == top ? (uint32_t)(64 * bslot + lane) : 0xffffffffu;
      wl = (int)(wave_min_u32(j) & 63u);
    }
    if (lane == wl) taken |= 1u << bslot;
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
