// Stand-alone causal top-k: given fp32 chunk scores, one wavefront per CSR
// row selects the kept chunks (select_rows.h) and writes them in ascending
// order; row_ptr is closed form (row i holds min(topk, i + 1) entries).
#include "select_rows.h"

namespace dhsa {
namespace {

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
  const float* srow = scores + st.sbase[b] + ((size_t)h * C + i) * C;
  select_row<NS>(srow, i, k, lane, col_idx + rp);
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
  // candidate slots per lane: one per 64 chunks, rounded up to a built size
  const int slots = (max_chunks + 63) / 64;
#define DHSA_TOPK_CASE(N)                                                           \
  if (slots <= N) {                                                                 \
    launch_ns<N>(scores, st, hq, total_rows, topk, row_ptr, col_idx, stream);       \
    return hipGetLastError();                                                       \
  }
  DHSA_TOPK_CASE(1) DHSA_TOPK_CASE(2) DHSA_TOPK_CASE(3) DHSA_TOPK_CASE(4)
  DHSA_TOPK_CASE(5) DHSA_TOPK_CASE(6) DHSA_TOPK_CASE(8) DHSA_TOPK_CASE(10)
  DHSA_TOPK_CASE(12) DHSA_TOPK_CASE(16) DHSA_TOPK_CASE(24) DHSA_TOPK_CASE(32)
#undef DHSA_TOPK_CASE
  return hipErrorInvalidValue;
}

}  // namespace dhsa
