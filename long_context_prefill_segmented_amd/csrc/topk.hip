// Causal chunk selection from fp32 chunk scores: one wavefront per CSR row
// selects the kept chunks (select_rows.h) and writes them in ascending order.
//
// With one budget for every row, row_ptr is closed form (row i holds
// min(budget + recent, i + 1) entries).  With a budget per row (DHSA README,
// "Predictor Checkpoints": query-dependent row budgets) the row lengths
// differ, so a single-workgroup scan first turns the per-row counts into
// row_ptr on the device, and the selection kernel reads its row's offset.
#include "select_rows.h"

namespace dhsa {
namespace {

// CSR row r -> (sequence b, head h, query chunk i)
struct RowId {
  int b, h, i;
};

__device__ __forceinline__ RowId row_id(const SeqTable& st, int32_t hq, int r) {
  int b = 0;
  while (b + 1 < st.batch && (int64_t)hq * st.cbase[b + 1] <= r) ++b;
  const int C = st.num_chunks[b];
  const int rl = r - hq * st.cbase[b];
  const int h = rl / C;
  return RowId{b, h, rl - h * C};
}

__device__ __forceinline__ int clamp_budget(int32_t v, int32_t cap) {
  return v < 1 ? 1 : (v > cap ? cap : v);
}

template <int NS>
__global__ __launch_bounds__(256) void topk_kernel(const float* __restrict__ scores,
                                                   SeqTable st, int32_t hq, int32_t total_rows,
                                                   int32_t topk, int32_t recent,
                                                   const int32_t* __restrict__ budgets,
                                                   int32_t* __restrict__ row_ptr,
                                                   int32_t* __restrict__ col_idx) {
  const int wave = threadIdx.x >> 6;
  const int lane = threadIdx.x & 63;
  const int r = blockIdx.x * 4 + wave;
  if (r >= total_rows) return;  // no block-level synchronisation below

  const RowId id = row_id(st, hq, r);
  const int C = st.num_chunks[id.b];
  int k;
  int64_t rp;
  if (budgets) {
    k = clamp_budget(budgets[r], topk);
    rp = row_ptr[r];  // written by the scan kernel earlier on the stream
  } else {
    k = topk;
    const int64_t m = (int64_t)topk + recent;
    rp = st.nbase[id.b] + (int64_t)id.h * entries_before(C, m) + entries_before(id.i, m);
    if (lane == 0) {
      row_ptr[r] = (int32_t)rp;
      if (r == total_rows - 1)
        row_ptr[total_rows] = (int32_t)(rp + (id.i + 1 <= m ? id.i + 1 : m));
    }
  }
  const float* srow = scores + st.sbase[id.b] + ((size_t)id.h * C + id.i) * C;
  select_row<NS>(srow, id.i, k, recent, lane, col_idx + rp);
}

// row_ptr from per-row budgets: count_r = min(i + 1, clamp(budget_r) + recent).
// One workgroup of 1024 threads walks the rows in blocks of 4096 (four
// consecutive rows per thread), scans each block (in-thread, then across the
// wave with DPP row shifts and broadcasts, then across the 16 waves through
// LDS) and carries the running total from block to block.
constexpr int kScanThreads = 1024;
constexpr int kScanWaves = kScanThreads / 64;

__device__ __forceinline__ int32_t wave_inclusive_scan(int32_t v) {
  int32_t t;
  t = __builtin_amdgcn_update_dpp(0, v, 0x111, 0xF, 0xF, false);  // row_shr:1
  v += t;
  t = __builtin_amdgcn_update_dpp(0, v, 0x112, 0xF, 0xF, false);  // row_shr:2
  v += t;
  t = __builtin_amdgcn_update_dpp(0, v, 0x114, 0xF, 0xF, false);  // row_shr:4
  v += t;
  t = __builtin_amdgcn_update_dpp(0, v, 0x118, 0xF, 0xF, false);  // row_shr:8
  v += t;
  t = __builtin_amdgcn_update_dpp(0, v, 0x142, 0xA, 0xF, false);  // row_bcast:15
  v += t;
  t = __builtin_amdgcn_update_dpp(0, v, 0x143, 0xC, 0xF, false);  // row_bcast:31
  v += t;
  return v;
}

__global__ __launch_bounds__(kScanThreads) void budget_scan_kernel(
    const int32_t* __restrict__ budgets, SeqTable st, int32_t hq, int32_t total_rows,
    int32_t topk, int32_t recent, int32_t* __restrict__ row_ptr) {
  __shared__ int32_t wsum[kScanWaves];
  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  int32_t carry = 0;
  for (int base = 0; base < total_rows; base += 4 * kScanThreads) {
    const int r0 = base + 4 * tid;
    int32_t cnt[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int r = r0 + u;
      cnt[u] = 0;
      if (r < total_rows) {
        const RowId id = row_id(st, hq, r);
        const int m = clamp_budget(budgets[r], topk) + recent;
        cnt[u] = id.i + 1 <= m ? id.i + 1 : m;
      }
    }
    const int32_t own = cnt[0] + cnt[1] + cnt[2] + cnt[3];
    const int32_t incl = wave_inclusive_scan(own);
    if (lane == 63) wsum[wave] = incl;
    __syncthreads();
    int32_t before = carry;
    for (int w = 0; w < wave; ++w) before += wsum[w];
    int32_t total = carry;
    for (int w = 0; w < kScanWaves; ++w) total += wsum[w];
    int32_t run = before + incl - own;
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      if (r0 + u < total_rows) row_ptr[r0 + u] = run;
      run += cnt[u];
    }
    if (base + 4 * kScanThreads >= total_rows && tid == 0) row_ptr[total_rows] = total;
    carry = total;
    __syncthreads();  // wsum is rewritten by the next block
  }
}

template <int NS>
void launch_ns(const float* scores, const SeqTable& st, int32_t hq, int32_t total_rows,
               int32_t topk, int32_t recent, const int32_t* budgets, int32_t* row_ptr,
               int32_t* col_idx, hipStream_t stream) {
  const unsigned grid = (unsigned)((total_rows + 3) / 4);
  hipLaunchKernelGGL(topk_kernel<NS>, dim3(grid), dim3(256), 0, stream, scores, st, hq,
                     total_rows, topk, recent, budgets, row_ptr, col_idx);
}

}  // namespace

hipError_t launch_topk(const float* scores, const SeqTable& st, int32_t hq,
                       int32_t total_rows, int32_t topk, int32_t recent,
                       const int32_t* budgets, int32_t max_chunks, int32_t* row_ptr,
                       int32_t* col_idx, hipStream_t stream) {
  if (total_rows <= 0) return hipSuccess;
  if (budgets) {
    hipLaunchKernelGGL(budget_scan_kernel, dim3(1), dim3(kScanThreads), 0, stream, budgets, st,
                       hq, total_rows, topk, recent, row_ptr);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  // candidate slots per lane: one per 64 chunks, rounded up to a built size
  const int slots = (max_chunks + 63) / 64;
#define DHSA_TOPK_CASE(N)                                                                   \
  if (slots <= N) {                                                                         \
    launch_ns<N>(scores, st, hq, total_rows, topk, recent, budgets, row_ptr, col_idx,       \
                 stream);                                                                   \
    return hipGetLastError();                                                               \
  }
  DHSA_TOPK_CASE(1) DHSA_TOPK_CASE(2) DHSA_TOPK_CASE(3) DHSA_TOPK_CASE(4)
  DHSA_TOPK_CASE(5) DHSA_TOPK_CASE(6) DHSA_TOPK_CASE(7) DHSA_TOPK_CASE(8) DHSA_TOPK_CASE(10)
  DHSA_TOPK_CASE(12) DHSA_TOPK_CASE(16) DHSA_TOPK_CASE(24) DHSA_TOPK_CASE(32)
#undef DHSA_TOPK_CASE
  return hipErrorInvalidValue;
}

}  // namespace dhsa
