// Causal per-query-chunk top-k selection, written as CSR.
//
// Row (b,h,i) keeps its diagonal chunk i plus the topk-1 earlier chunks with
// the highest scores; when i + 1 <= topk it keeps every chunk 0..i
// (gist.science Technical Summary, Methodology, Step 2: each query chunk is
// routed to its highest-scoring chunks under the causal constraint; DHSA
// README, "Predictor Checkpoints": a fixed row budget).  The order is total:
// score descending, then chunk index ascending; -0 and +0 are equal; NaN
// ranks below every number.
//
// One wavefront owns one row.  Candidate j < i sits in lane j % 64, slot
// j / 64, as a 64-bit key (order-preserving score bits, then the complement
// of j), so each round is a register max followed by a 6-step butterfly max
// across the wave.  The winners are emitted in ascending index order by a
// ballot and prefix popcount per slot, and the diagonal goes last.
// row_ptr is closed form: row i holds min(topk, i + 1) entries.
#include "dhsa_internal.h"

namespace dhsa {
namespace {

__device__ __forceinline__ uint32_t order_key(float s) {
  s = s + 0.0f;  // -0 -> +0
  uint32_t u = __float_as_uint(s);
  if (s != s) return 1u;  // NaN: below every number, above empty slots
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

// entries in rows 0..i-1 of one head: sum_{i' < i} min(k, i'+1)
__device__ __forceinline__ int64_t entries_before(int64_t i, int64_t k) {
  return i <= k ? i * (i + 1) / 2 : k * (k + 1) / 2 + (i - k) * k;
}

__device__ __forceinline__ uint64_t wave_max_u64(uint64_t v) {
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) {
    const uint32_t lo = __shfl_xor((uint32_t)v, m, 64);
    const uint32_t hi = __shfl_xor((uint32_t)(v >> 32), m, 64);
    const uint64_t o = ((uint64_t)hi << 32) | lo;
    v = o > v ? o : v;
  }
  return v;
}

template <int NS>
__global__ __launch_bounds__(256) void topk_kernel(const float* __restrict__ scores,
                                                   SeqTable st, int32_t hq, int32_t total_rows,
                                                   int32_t topk, int32_t* __restrict__ row_ptr,
                                                   int32_t* __restrict__ col_idx) {
  const int wave = threadIdx.x >> 6;
  const int lane = threadIdx.x & 63;
  const int r = blockIdx.x * 4 + wave;
  if (r >= total_rows) return;  // no block-level synchronisation below

  int b = 0;
  while (b + 1 < st.batch && (int64_t)hq * st.cbase[b + 1] <= r) ++b;
  const int C = st.num_chunks[b];
  const int rl = r - hq * st.cbase[b];
  const int h = rl / C;
  const int i = rl - h * C;
  const int64_t k = topk;
  const int64_t per_head = entries_before(C, k);
  const int64_t rp = st.nbase[b] + (int64_t)h * per_head + entries_before(i, k);
  if (lane == 0) {
    row_ptr[r] = (int32_t)rp;
    if (r == total_rows - 1) row_ptr[total_rows] = (int32_t)(rp + (i + 1 <= k ? i + 1 : k));
  }
  int32_t* out = col_idx + rp;
  if (i + 1 <= k) {
    for (int j = lane; j <= i; j += 64) out[j] = j;
    return;
  }
  const float* srow = scores + st.sbase[b] + ((size_t)h * C + i) * C;
  uint32_t key[NS];
#pragma unroll
  for (int s = 0; s < NS; ++s) {
    const int j = lane + 64 * s;
    key[s] = j < i ? order_key(srow[j]) : 0u;  // 0: empty slot
  }
  uint32_t taken = 0;
  for (int round = 0; round < (int)k - 1; ++round) {
    uint64_t best = 0;
#pragma unroll
    for (int s = 0; s < NS; ++s) {
      const uint64_t cand = ((taken >> s) & 1u)
                                ? 0ull
                                : (((uint64_t)key[s] << 32) |
                                   (uint32_t)(0xffffffffu - (uint32_t)(lane + 64 * s)));
      best = cand > best ? cand : best;
    }
    best = wave_max_u64(best);
    const uint32_t jwin = 0xffffffffu - (uint32_t)best;
    if ((int)(jwin & 63u) == lane) taken |= 1u << (jwin >> 6);
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
  if (lane == 0) out[k - 1] = i;
}

template <int NS>
void launch_ns(const float* scores, const SeqTable& st, int32_t hq, int32_t total_rows,
               int32_t topk, int32_t* row_ptr, int32_t* col_idx, hipStream_t stream) {
  const unsigned grid = (unsigned)((total_rows + 3) / 4);
  hipLaunchKernelGGL(topk_kernel<NS>, dim3(grid), dim3(256), 0, stream, scores, st, hq,
                     total_rows, topk, row_ptr, col_idx);
}

}  // namespace

hipError_t launch_topk(const float* scores, const SeqTable& st, int32_t hq,
                       int32_t total_rows, int32_t topk, int32_t max_chunks,
                       int32_t* row_ptr, int32_t* col_idx, hipStream_t stream) {
  if (total_rows <= 0) return hipSuccess;
  const int slots = (max_chunks + 63) / 64;
  if (slots <= 1) launch_ns<1>(scores, st, hq, total_rows, topk, row_ptr, col_idx, stream);
  else if (slots <= 2) launch_ns<2>(scores, st, hq, total_rows, topk, row_ptr, col_idx, stream);
  else if (slots <= 4) launch_ns<4>(scores, st, hq, total_rows, topk, row_ptr, col_idx, stream);
  else if (slots <= 8) launch_ns<8>(scores, st, hq, total_rows, topk, row_ptr, col_idx, stream);
  else if (slots <= 16) launch_ns<16>(scores, st, hq, total_rows, topk, row_ptr, col_idx, stream);
  else if (slots <= 32) launch_ns<32>(scores, st, hq, total_rows, topk, row_ptr, col_idx, stream);
  else return hipErrorInvalidValue;
  return hipGetLastError();
}

}  // namespace dhsa
