// Host side of the C ABI: argument validation, sizes, launch planning.
// Every check runs before any HIP call; on an error nothing is enqueued.
#include <stdarg.h>
#include <stdlib.h>
#include <stdio.h>
#include <string.h>

#include <cmath>
#include <mutex>

#include "dhsa_internal.h"

namespace dhsa {

thread_local char g_err[512] = "";

int fail(int status, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_err, sizeof(g_err), fmt, ap);
  va_end(ap);
  return status;
}

int ok() {
  g_err[0] = '\0';
  return DHSA_OK;
}

namespace {

int hip_fail(hipError_t e, const char* what) {
  return fail(DHSA_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
}

constexpr size_t kAlign = 256;
size_t align_up(size_t x) { return (x + kAlign - 1) / kAlign * kAlign; }

int check_batch_chunks(int32_t batch, const int32_t* num_chunks) {
  if (num_chunks == nullptr) return fail(DHSA_ERR_NULL_POINTER, "num_chunks is NULL");
  if (batch < 1 || batch > kMaxBatch)
    return fail(DHSA_ERR_SHAPE, "batch %d outside [1, %d]", batch, kMaxBatch);
  int64_t total = 0;
  for (int b = 0; b < batch; ++b) {
    if (num_chunks[b] < 1)
      return fail(DHSA_ERR_OFFSETS, "sequence %d has %d chunks", b, num_chunks[b]);
    total += num_chunks[b];
  }
  if (total > INT32_MAX / 4) return fail(DHSA_ERR_UNSUPPORTED, "too many chunks (%lld)", (long long)total);
  return DHSA_OK;
}

int check_heads(int32_t hq, int32_t hkv, int32_t head_dim) {
  if (head_dim != kHeadDim) return fail(DHSA_ERR_SHAPE, "head_dim %d != %d", head_dim, kHeadDim);
  if (hq < 1 || hkv < 1) return fail(DHSA_ERR_SHAPE, "head counts must be >= 1 (%d, %d)", hq, hkv);
  if (hq % hkv) return fail(DHSA_ERR_SHAPE, "num_q_heads %d not a multiple of num_kv_heads %d", hq, hkv);
  return DHSA_OK;
}

int check_offsets(int32_t batch, int32_t seq_len, const int32_t* num_chunks,
                  const int32_t* offs) {
  if (offs == nullptr) return fail(DHSA_ERR_NULL_POINTER, "chunk_offsets is NULL");
  if (seq_len < 1) return fail(DHSA_ERR_SHAPE, "seq_len %d < 1", seq_len);
  size_t o = 0;
  for (int b = 0; b < batch; ++b) {
    const int C = num_chunks[b];
    if (C > seq_len) return fail(DHSA_ERR_OFFSETS, "sequence %d: %d chunks > seq_len", b, C);
    if (offs[o] != 0) return fail(DHSA_ERR_OFFSETS, "sequence %d: offsets must start at 0", b);
    for (int c = 0; c < C; ++c) {
      if (offs[o + c + 1] <= offs[o + c])
        return fail(DHSA_ERR_OFFSETS, "sequence %d: offsets not strictly increasing at %d", b, c);
    }
    if (offs[o + C] != seq_len)
      return fail(DHSA_ERR_OFFSETS, "sequence %d: offsets end at %d, not seq_len %d", b, offs[o + C],
                  seq_len);
    o += C + 1;
  }
  return DHSA_OK;
}

int64_t entries_per_head(int64_t C, int64_t k) {
  return C <= k ? C * (C + 1) / 2 : k * (k + 1) / 2 + (C - k) * k;
}

// per_row: entries a row i keeps at most (budget + recent window), 0 when the
// table is not used for CSR offsets
void fill_table(SeqTable& st, int32_t batch, const int32_t* num_chunks, int32_t hq,
                int64_t per_row) {
  memset(&st, 0, sizeof(st));
  st.batch = batch;
  int64_t cb = 0, sb = 0, nb = 0;
  for (int b = 0; b < batch; ++b) {
    const int64_t C = num_chunks[b];
    st.num_chunks[b] = (int32_t)C;
    st.cbase[b] = (int32_t)cb;
    st.sbase[b] = sb;
    st.nbase[b] = nb;
    cb += C;
    sb += (int64_t)hq * C * C;
    if (per_row > 0) nb += (int64_t)hq * entries_per_head(C, per_row);
  }
}

int64_t total_chunks(int32_t batch, const int32_t* num_chunks) {
  int64_t t = 0;
  for (int b = 0; b < batch; ++b) t += num_chunks[b];
  return t;
}

int64_t score_elems(int32_t batch, const int32_t* num_chunks, int32_t hq) {
  int64_t t = 0;
  for (int b = 0; b < batch; ++b) t += (int64_t)hq * num_chunks[b] * num_chunks[b];
  return t;
}

int64_t score_tiles(int32_t batch, const int32_t* num_chunks, int32_t hq) {
  int64_t t = 0;
  for (int b = 0; b < batch; ++b) {
    const int64_t T = (num_chunks[b] + 31) / 32;
    t += hq * T * (T + 1) / 2;
  }
  return t;
}

// Query tiles of one height: per chunk floor(n / block_m) full tiles plus
// one for a remainder; with narrow != nullptr a remainder of at most
// kNarrowRows rows is counted in *narrow instead (and its per-sequence base
// written to nbase).
int64_t query_tiles(int32_t batch, const int32_t* num_chunks, const int32_t* offs,
                    int32_t block_m, int32_t* tbase, int64_t* narrow = nullptr,
                    int32_t* nbase = nullptr) {
  int64_t t = 0, nt = 0;
  size_t o = 0;
  for (int b = 0; b < batch; ++b) {
    if (tbase) tbase[b] = (int32_t)t;
    if (nbase) nbase[b] = (int32_t)nt;
    for (int c = 0; c < num_chunks[b]; ++c) {
      const int32_t n = offs[o + c + 1] - offs[o + c];
      const int32_t full = n / block_m, rem = n - full * block_m;
      if (narrow && rem > 0 && rem <= kNarrowRows) {
        t += full;
        nt += 1;
      } else {
        t += full + (rem > 0 ? 1 : 0);
      }
    }
    o += num_chunks[b] + 1;
  }
  if (narrow) *narrow = nt;
  return t;
}

// Query tile height for the attention kernel.  A 256-row tile (8 waves, one
// workgroup per CU) streams each kept K/V sub-tile for twice as many rows as
// a 128-row tile, while a chunk of at most 128 rows leaves half of its waves
// idle.  The large tile is taken when at least half of the tiled query rows
// (remainders of at most kNarrowRows rows go to the narrow tiles either way)
// lie in chunks longer than 128 rows.  Measured on 32K layers with uniform
// chunk-length laws: U[33,128] and U[40,160] (0 % and 38 % of the rows in
// longer chunks) run faster with 128-row tiles, U[64,192] (62 %), U[96,256],
// U[128,384] and U[33,512] with 256-row tiles, as do the 16K, 32K, 128K and
// ragged layers of the bench.
// DHSA_ATTN_BLOCK_M=128|256 in the environment forces one of them.
int32_t choose_block_m(int32_t batch, const int32_t* num_chunks, const int32_t* offs) {
  if (const char* env = getenv("DHSA_ATTN_BLOCK_M")) {
    const int v = atoi(env);
    if (v == kBlockMSmall || v == kBlockMLarge) return v;
  }
  int64_t rows = 0, long_rows = 0;
  size_t o = 0;
  for (int b = 0; b < batch; ++b) {
    for (int c = 0; c < num_chunks[b]; ++c) {
      const int64_t n = offs[o + c + 1] - offs[o + c];
      const int64_t full = n / kBlockMLarge, rem = n - full * kBlockMLarge;
      const int64_t wide_rows = rem <= kNarrowRows ? full * kBlockMLarge : n;
      rows += wide_rows;
      if (n > kBlockMSmall) long_rows += wide_rows;
    }
    o += num_chunks[b] + 1;
  }
  return 2 * long_rows >= rows ? kBlockMLarge : kBlockMSmall;
}

int check_nms_sizes(int32_t batch, int32_t seq_len, int32_t min_gap) {
  if (batch < 1 || batch > kMaxBatch)
    return fail(DHSA_ERR_SHAPE, "batch %d outside [1, %d]", batch, kMaxBatch);
  if (seq_len < 1) return fail(DHSA_ERR_SHAPE, "seq_len %d < 1", seq_len);
  if (seq_len > kNmsMaxLen)
    return fail(DHSA_ERR_UNSUPPORTED, "seq_len %d > %d for boundary NMS", seq_len, kNmsMaxLen);
  if (min_gap < 1) return fail(DHSA_ERR_SHAPE, "min_gap %d < 1", min_gap);
  return DHSA_OK;
}

int max_chunks(int32_t batch, const int32_t* num_chunks) {
  int m = 0;
  for (int b = 0; b < batch; ++b) m = num_chunks[b] > m ? num_chunks[b] : m;
  return m;
}

}  // namespace
}  // namespace dhsa

using namespace dhsa;

extern "C" {

const char* dhsa_status_string(int status) {
  switch (status) {
    case DHSA_OK: return "DHSA_OK";
    case DHSA_ERR_NULL_POINTER: return "DHSA_ERR_NULL_POINTER";
    case DHSA_ERR_SHAPE: return "DHSA_ERR_SHAPE";
    case DHSA_ERR_OFFSETS: return "DHSA_ERR_OFFSETS";
    case DHSA_ERR_TOPK: return "DHSA_ERR_TOPK";
    case DHSA_ERR_CAPACITY: return "DHSA_ERR_CAPACITY";
    case DHSA_ERR_CSR: return "DHSA_ERR_CSR";
    case DHSA_ERR_UNSUPPORTED: return "DHSA_ERR_UNSUPPORTED";
    case DHSA_ERR_HIP: return "DHSA_ERR_HIP";
    default: return "DHSA_ERR_UNKNOWN";
  }
}

const char* dhsa_last_error(void) { return dhsa::g_err; }

int dhsa_version(void) { return 102; }

int dhsa_csr_capacity(int32_t batch, const int32_t* num_chunks, int32_t num_q_heads,
                      int32_t topk, int32_t recent, int32_t* num_rows, int64_t* nnz) {
  if (num_rows == nullptr || nnz == nullptr) return fail(DHSA_ERR_NULL_POINTER, "output pointer is NULL");
  int s = check_batch_chunks(batch, num_chunks);
  if (s) return s;
  if (num_q_heads < 1) return fail(DHSA_ERR_SHAPE, "num_q_heads %d < 1", num_q_heads);
  if (topk < 1) return fail(DHSA_ERR_TOPK, "topk %d < 1", topk);
  if (recent < 0) return fail(DHSA_ERR_TOPK, "recent %d < 0", recent);
  const int64_t m = (int64_t)topk + recent;
  int64_t R = 0, N = 0;
  for (int b = 0; b < batch; ++b) {
    R += (int64_t)num_q_heads * num_chunks[b];
    N += (int64_t)num_q_heads * entries_per_head(num_chunks[b], m);
  }
  if (R > INT32_MAX - 1 || N > INT32_MAX)
    return fail(DHSA_ERR_UNSUPPORTED, "CSR too large for int32 indices");
  *num_rows = (int32_t)R;
  *nnz = N;
  return ok();
}

int dhsa_csr_size(int32_t batch, const int32_t* num_chunks, int32_t num_q_heads, int32_t topk,
                  int32_t* num_rows, int64_t* nnz) {
  return dhsa_csr_capacity(batch, num_chunks, num_q_heads, topk, 0, num_rows, nnz);
}

int dhsa_mask_workspace_size(int32_t batch, const int32_t* num_chunks, int32_t num_q_heads,
                             int32_t num_kv_heads, int32_t head_dim, size_t* bytes) {
  if (bytes == nullptr) return fail(DHSA_ERR_NULL_POINTER, "bytes is NULL");
  int s = check_batch_chunks(batch, num_chunks);
  if (s) return s;
  s = check_heads(num_q_heads, num_kv_heads, head_dim);
  if (s) return s;
  const int64_t tc = total_chunks(batch, num_chunks);
  size_t n = align_up((size_t)num_q_heads * tc * kHeadDim * sizeof(float));
  n += align_up((size_t)num_kv_heads * tc * kHeadDim * sizeof(float));
  n += align_up((size_t)score_elems(batch, num_chunks, num_q_heads) * sizeof(float));
  n += align_up((size_t)tc * sizeof(int32_t));  // pooling order, longest chunk first
  *bytes = n;
  return ok();
}

int dhsa_prefill_workspace_size(int32_t batch, int32_t seq_len, const int32_t* num_chunks,
                                const int32_t* chunk_offsets, size_t* bytes) {
  if (bytes == nullptr) return fail(DHSA_ERR_NULL_POINTER, "bytes is NULL");
  int s = check_batch_chunks(batch, num_chunks);
  if (s) return s;
  s = check_offsets(batch, seq_len, num_chunks, chunk_offsets);
  if (s) return s;
  // sized for the smaller tile height (the larger needs fewer tiles)
  *bytes = align_up((size_t)query_tiles(batch, num_chunks, chunk_offsets, kBlockMSmall, nullptr) *
                    sizeof(int4));
  return ok();
}

int dhsa_nms_offsets_stride(int32_t seq_len, int32_t min_gap, int32_t* stride) {
  if (stride == nullptr) return fail(DHSA_ERR_NULL_POINTER, "stride is NULL");
  int s = check_nms_sizes(1, seq_len, min_gap);
  if (s) return s;
  const int32_t c = seq_len / min_gap;
  *stride = (c > 1 ? c : 1) + 1;
  return ok();
}

int dhsa_nms_workspace_size(int32_t batch, int32_t seq_len, int32_t min_gap, size_t* bytes) {
  if (bytes == nullptr) return fail(DHSA_ERR_NULL_POINTER, "bytes is NULL");
  int s = check_nms_sizes(batch, seq_len, min_gap);
  if (s) return s;
  *bytes = align_up((size_t)batch * 2 * seq_len * sizeof(int32_t));
  return ok();
}

int dhsa_nms_boundaries(const float* scores, int32_t batch, int32_t seq_len, int32_t min_gap,
                        float threshold, int32_t* offsets_out, int32_t offsets_stride,
                        int32_t* num_chunks_out, void* workspace, size_t workspace_bytes,
                        void* stream) {
  if (!scores || !offsets_out || !num_chunks_out || !workspace)
    return fail(DHSA_ERR_NULL_POINTER, "NULL device pointer");
  int s = check_nms_sizes(batch, seq_len, min_gap);
  if (s) return s;
  if (!(threshold == threshold)) return fail(DHSA_ERR_SHAPE, "threshold is NaN");
  int32_t need_stride;
  s = dhsa_nms_offsets_stride(seq_len, min_gap, &need_stride);
  if (s) return s;
  if (offsets_stride < need_stride)
    return fail(DHSA_ERR_CAPACITY, "offsets_stride %d < %d", offsets_stride, need_stride);
  size_t need;
  s = dhsa_nms_workspace_size(batch, seq_len, min_gap, &need);
  if (s) return s;
  if (workspace_bytes < need)
    return fail(DHSA_ERR_CAPACITY, "workspace %zu < %zu bytes", workspace_bytes, need);
  if (reinterpret_cast<uintptr_t>(workspace) % kAlign)
    return fail(DHSA_ERR_CAPACITY, "workspace not %zu-byte aligned", kAlign);
  hipError_t e = launch_nms(scores, batch, seq_len, min_gap, threshold, offsets_out,
                            offsets_stride, num_chunks_out, workspace,
                            static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return hip_fail(e, "boundary NMS launch");
  return ok();
}

int dhsa_pool(const void* x, int32_t batch, int32_t seq_len, int32_t num_heads, int32_t head_dim,
              const int32_t* num_chunks, const int32_t* chunk_offsets,
              const int32_t* chunk_offsets_dev, float* pooled, void* stream) {
  if (!x || !pooled || !chunk_offsets_dev) return fail(DHSA_ERR_NULL_POINTER, "NULL device pointer");
  int s = check_batch_chunks(batch, num_chunks);
  if (s) return s;
  s = check_heads(num_heads, 1, head_dim);
  if (s) return s;
  s = check_offsets(batch, seq_len, num_chunks, chunk_offsets);
  if (s) return s;
  SeqTable st;
  fill_table(st, batch, num_chunks, num_heads, 0);
  hipError_t e = launch_pool(static_cast<const uint16_t*>(x), pooled, num_heads, nullptr, nullptr, 0,
                             (int32_t)total_chunks(batch, num_chunks), chunk_offsets_dev, nullptr,
                             st, seq_len, nullptr, static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return hip_fail(e, "pool launch");
  return ok();
}

int dhsa_chunk_scores(const float* qbar, const float* kbar, int32_t batch, int32_t num_q_heads,
                      int32_t num_kv_heads, int32_t head_dim, const int32_t* num_chunks,
                      float* scores, void* stream) {
  if (!qbar || !kbar || !scores) return fail(DHSA_ERR_NULL_POINTER, "NULL device pointer");
  int s = check_batch_chunks(batch, num_chunks);
  if (s) return s;
  s = check_heads(num_q_heads, num_kv_heads, head_dim);
  if (s) return s;
  SeqTable st;
  fill_table(st, batch, num_chunks, num_q_heads, 0);
  const int64_t tiles = score_tiles(batch, num_chunks, num_q_heads);
  if (tiles > INT32_MAX) return fail(DHSA_ERR_UNSUPPORTED, "too many score tiles");
  hipError_t e = launch_scores(qbar, kbar, scores, num_q_heads, num_kv_heads, st, tiles,
                               static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return hip_fail(e, "chunk score launch");
  return ok();
}

int dhsa_topk_csr_ex(const float* scores, int32_t batch, int32_t num_q_heads,
                     const int32_t* num_chunks, int32_t topk, const int32_t* row_budgets,
                     int32_t recent, int32_t* row_ptr, int32_t* col_idx, int64_t col_capacity,
                     void* stream) {
  if (!scores || !row_ptr || !col_idx) return fail(DHSA_ERR_NULL_POINTER, "NULL device pointer");
  int32_t R;
  int64_t nnz;
  int s = dhsa_csr_capacity(batch, num_chunks, num_q_heads, topk, recent, &R, &nnz);
  if (s) return s;
  const int cmax = max_chunks(batch, num_chunks);
  if (cmax > kMaxChunks)
    return fail(DHSA_ERR_UNSUPPORTED, "more than %d chunks in a sequence", kMaxChunks);
  if (col_capacity < nnz)
    return fail(DHSA_ERR_CAPACITY, "col_capacity %lld < nnz %lld", (long long)col_capacity,
                (long long)nnz);
  // a budget or window beyond the longest sequence keeps the same chunks as
  // one equal to it, so both are clamped there (keeps device sums in int32)
  const int32_t k_dev = topk < cmax ? topk : cmax;
  const int32_t w_dev = recent < cmax ? recent : cmax;
  SeqTable st;
  fill_table(st, batch, num_chunks, num_q_heads, (int64_t)k_dev + w_dev);
  hipError_t e = launch_topk(scores, st, num_q_heads, R, k_dev, w_dev, row_budgets, cmax,
                             row_ptr, col_idx, static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return hip_fail(e, "top-k launch");
  return ok();
}

int dhsa_topk_csr(const float* scores, int32_t batch, int32_t num_q_heads,
                  const int32_t* num_chunks, int32_t topk, int32_t* row_ptr, int32_t* col_idx,
                  int64_t col_capacity, void* stream) {
  return dhsa_topk_csr_ex(scores, batch, num_q_heads, num_chunks, topk, nullptr, 0, row_ptr,
                          col_idx, col_capacity, stream);
}

int dhsa_build_mask_ex(const void* q, const void* k, int32_t batch, int32_t seq_len,
                       int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim,
                       const int32_t* num_chunks, const int32_t* chunk_offsets,
                       const int32_t* chunk_offsets_dev, int32_t topk,
                       const int32_t* row_budgets, int32_t recent, int32_t* row_ptr,
                       int32_t* col_idx, int64_t col_capacity, float* scores_out,
                       void* workspace, size_t workspace_bytes, void* stream) {
  if (!q || !k || !chunk_offsets_dev || !row_ptr || !col_idx || !workspace)
    return fail(DHSA_ERR_NULL_POINTER, "NULL device pointer");
  int s = check_batch_chunks(batch, num_chunks);
  if (s) return s;
  s = check_heads(num_q_heads, num_kv_heads, head_dim);
  if (s) return s;
  s = check_offsets(batch, seq_len, num_chunks, chunk_offsets);
  if (s) return s;
  int32_t R;
  int64_t nnz;
  s = dhsa_csr_capacity(batch, num_chunks, num_q_heads, topk, recent, &R, &nnz);
  if (s) return s;
  const int cmax = max_chunks(batch, num_chunks);
  if (cmax > kMaxChunks)
    return fail(DHSA_ERR_UNSUPPORTED, "more than %d chunks in a sequence", kMaxChunks);
  if (col_capacity < nnz)
    return fail(DHSA_ERR_CAPACITY, "col_capacity %lld < nnz %lld", (long long)col_capacity,
                (long long)nnz);
  size_t need;
  s = dhsa_mask_workspace_size(batch, num_chunks, num_q_heads, num_kv_heads, head_dim, &need);
  if (s) return s;
  if (workspace_bytes < need)
    return fail(DHSA_ERR_CAPACITY, "workspace %zu < %zu bytes", workspace_bytes, need);
  if (reinterpret_cast<uintptr_t>(workspace) % kAlign)
    return fail(DHSA_ERR_CAPACITY, "workspace not %zu-byte aligned", kAlign);

  const int64_t tc = total_chunks(batch, num_chunks);
  char* ws = static_cast<char*>(workspace);
  float* qbar = reinterpret_cast<float*>(ws);
  ws += align_up((size_t)num_q_heads * tc * kHeadDim * sizeof(float));
  float* kbar = reinterpret_cast<float*>(ws);
  ws += align_up((size_t)num_kv_heads * tc * kHeadDim * sizeof(float));
  float* scores = scores_out ? scores_out : reinterpret_cast<float*>(ws);
  ws += align_up((size_t)score_elems(batch, num_chunks, num_q_heads) * sizeof(float));
  int32_t* order = reinterpret_cast<int32_t*>(ws);

  const int32_t k_dev = topk < cmax ? topk : cmax;
  const int32_t w_dev = recent < cmax ? recent : cmax;
  SeqTable st;
  fill_table(st, batch, num_chunks, num_q_heads, (int64_t)k_dev + w_dev);
  hipStream_t strm = static_cast<hipStream_t>(stream);
  hipError_t e = launch_pool(static_cast<const uint16_t*>(q), qbar, num_q_heads,
                             static_cast<const uint16_t*>(k), kbar, num_kv_heads, (int32_t)tc,
                             chunk_offsets_dev, chunk_offsets, st, seq_len, order, strm);
  if (e != hipSuccess) return hip_fail(e, "pool launch");
  e = launch_scores(qbar, kbar, scores, num_q_heads, num_kv_heads, st,
                    score_tiles(batch, num_chunks, num_q_heads), strm);
  if (e != hipSuccess) return hip_fail(e, "chunk score launch");
  e = launch_topk(scores, st, num_q_heads, R, k_dev, w_dev, row_budgets, cmax, row_ptr, col_idx,
                  strm);
  if (e != hipSuccess) return hip_fail(e, "top-k launch");
  return ok();
}

int dhsa_build_mask(const void* q, const void* k, int32_t batch, int32_t seq_len,
                    int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim,
                    const int32_t* num_chunks, const int32_t* chunk_offsets,
                    const int32_t* chunk_offsets_dev, int32_t topk, int32_t* row_ptr,
                    int32_t* col_idx, int64_t col_capacity, float* scores_out, void* workspace,
                    size_t workspace_bytes, void* stream) {
  return dhsa_build_mask_ex(q, k, batch, seq_len, num_q_heads, num_kv_heads, head_dim,
                            num_chunks, chunk_offsets, chunk_offsets_dev, topk, nullptr, 0,
                            row_ptr, col_idx, col_capacity, scores_out, workspace,
                            workspace_bytes, stream);
}

}  // extern "C"

namespace dhsa {
namespace {

// The query-tile list of dhsa_sparse_prefill_noalloc lives here instead of a
// caller workspace.  Each GPU holds its own copy; its device address comes
// from hipGetSymbolAddress on the first call on that device.
__device__ __attribute__((aligned(256))) int4 scratch[DHSA_NOALLOC_MAX_TILES];
constexpr size_t kScratchBytes = sizeof(int4) * DHSA_NOALLOC_MAX_TILES;
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

// Device address of `scratch` on the current device (looked up once per
// device, with that device current); nullptr and a message on failure.
void* scratch_address(int* status) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) {
    *status = hip_fail(e, "hipGetDevice");
    return nullptr;
  }
  if (dev < 0 || dev >= kMaxDevices) {
    *status = fail(DHSA_ERR_UNSUPPORTED, "device %d beyond the %d the library tracks", dev,
                   kMaxDevices);
    return nullptr;
  }
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (g_scratch_ptr[dev] == nullptr) {
    void* ptr = nullptr;
    e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    if (e != hipSuccess || ptr == nullptr) {
      *status = hip_fail(e != hipSuccess ? e : hipErrorInvalidSymbol, "hipGetSymbolAddress(scratch)");
      return nullptr;
    }
    g_scratch_ptr[dev] = ptr;
  }
  return g_scratch_ptr[dev];
}

// dhsa_sparse_prefill; with use_scratch the tile list goes to this device's
// static scratch array (workspace and workspace_bytes are ignored).
int sparse_prefill_impl(const void* q, const void* k, const void* v, int32_t batch,
                        int32_t seq_len, int32_t num_q_heads, int32_t num_kv_heads,
                        int32_t head_dim, const int32_t* num_chunks, const int32_t* chunk_offsets,
                        const int32_t* chunk_offsets_dev, const int32_t* row_ptr,
                        const int32_t* col_idx, int64_t nnz, float softmax_scale, void* out,
                        float* lse, void* workspace, size_t workspace_bytes, void* stream,
                        bool use_scratch) {
  if (!q || !k || !v || !chunk_offsets_dev || !row_ptr || !out || (!use_scratch && !workspace))
    return fail(DHSA_ERR_NULL_POINTER, "NULL device pointer");
  if (nnz > 0 && !col_idx) return fail(DHSA_ERR_NULL_POINTER, "col_idx is NULL");
  if (nnz < 0 || nnz > INT32_MAX) return fail(DHSA_ERR_CSR, "nnz %lld out of range", (long long)nnz);
  int s = check_batch_chunks(batch, num_chunks);
  if (s) return s;
  s = check_heads(num_q_heads, num_kv_heads, head_dim);
  if (s) return s;
  s = check_offsets(batch, seq_len, num_chunks, chunk_offsets);
  if (s) return s;
  if (!(softmax_scale == softmax_scale) || std::isinf(softmax_scale))
    return fail(DHSA_ERR_SHAPE, "softmax_scale is not finite");
  // the attention kernel addresses a sequence's K/V rows with 32-bit offsets
  if ((uint64_t)seq_len * num_kv_heads * kHeadDim * 2 > UINT32_MAX)
    return fail(DHSA_ERR_UNSUPPORTED, "seq_len * num_kv_heads * %d bytes exceeds 4 GiB",
                kHeadDim * 2);
  const int32_t ntiles_max = INT32_MAX / num_q_heads;
  int32_t tbase[kMaxBatch], nbase[kMaxBatch];
  const int32_t block_m = choose_block_m(batch, num_chunks, chunk_offsets);
  int64_t nnarrow = 0;
  const int64_t ntiles =
      query_tiles(batch, num_chunks, chunk_offsets, block_m, tbase, &nnarrow, nbase);
  if (ntiles > ntiles_max || nnarrow > ntiles_max)
    return fail(DHSA_ERR_UNSUPPORTED, "too many query tiles");
  // the workspace bound (tiles of the smaller height) also covers the two lists
  const size_t need = align_up((size_t)(ntiles + nnarrow) * sizeof(int4));
  if (use_scratch) {
    if (need > kScratchBytes)
      return fail(DHSA_ERR_CAPACITY,
                  "%lld query tiles exceed the static scratch of %d tiles (DHSA_NOALLOC_MAX_TILES)",
                  (long long)(ntiles + nnarrow), DHSA_NOALLOC_MAX_TILES);
    int st_fail = DHSA_OK;
    workspace = scratch_address(&st_fail);
    if (workspace == nullptr) return st_fail;
    workspace_bytes = kScratchBytes;
  }
  if (workspace_bytes < need)
    return fail(DHSA_ERR_CAPACITY, "workspace %zu < %zu bytes", workspace_bytes, need);
  if (reinterpret_cast<uintptr_t>(workspace) % kAlign)
    return fail(DHSA_ERR_CAPACITY, "workspace not %zu-byte aligned", kAlign);

  SeqTable st;
  fill_table(st, batch, num_chunks, num_q_heads, 0);
  for (int b = 0; b < batch; ++b) {
    st.tbase[b] = tbase[b];
    st.ntbase[b] = nbase[b];
  }
  hipStream_t strm = static_cast<hipStream_t>(stream);
  int4* tiles = static_cast<int4*>(workspace);
  int4* narrow = tiles + ntiles;
  hipError_t e = launch_plan_tiles(chunk_offsets_dev, st, tiles, narrow, block_m, strm);
  if (e != hipSuccess) return hip_fail(e, "tile plan launch");

  AttnParams p;
  p.q = static_cast<const uint16_t*>(q);
  p.k = static_cast<const uint16_t*>(k);
  p.v = static_cast<const uint16_t*>(v);
  p.o = static_cast<uint16_t*>(out);
  p.lse = lse;
  p.tiles = tiles;
  p.narrow = narrow;
  p.offs = chunk_offsets_dev;
  p.row_ptr = row_ptr;
  p.col_idx = col_idx;
  p.nnz = nnz;
  p.num_tiles = (int32_t)ntiles;
  p.num_narrow = (int32_t)nnarrow;
  p.seq_len = seq_len;
  p.hq = num_q_heads;
  p.hkv = num_kv_heads;
  p.block_m = block_m;
  const float scale = softmax_scale > 0.f ? softmax_scale : 1.0f / sqrtf((float)kHeadDim);
  p.scale_log2 = scale * 1.4426950408889634f;
  e = launch_attention(p, st, strm);
  if (e != hipSuccess) return hip_fail(e, "attention launch");
  return ok();
}

}  // namespace
}  // namespace dhsa

extern "C" {

int dhsa_sparse_prefill(const void* q, const void* k, const void* v, int32_t batch,
                        int32_t seq_len, int32_t num_q_heads, int32_t num_kv_heads,
                        int32_t head_dim, const int32_t* num_chunks, const int32_t* chunk_offsets,
                        const int32_t* chunk_offsets_dev, const int32_t* row_ptr,
                        const int32_t* col_idx, int64_t nnz, float softmax_scale, void* out,
                        float* lse, void* workspace, size_t workspace_bytes, void* stream) {
  return dhsa::sparse_prefill_impl(q, k, v, batch, seq_len, num_q_heads, num_kv_heads, head_dim,
                                   num_chunks, chunk_offsets, chunk_offsets_dev, row_ptr, col_idx,
                                   nnz, softmax_scale, out, lse, workspace, workspace_bytes, stream,
                                   false);
}

int dhsa_sparse_prefill_noalloc(const void* q, const void* k, const void* v, int32_t batch,
                                int32_t seq_len, int32_t num_q_heads, int32_t num_kv_heads,
                                int32_t head_dim, const int32_t* num_chunks,
                                const int32_t* chunk_offsets, const int32_t* chunk_offsets_dev,
                                const int32_t* row_ptr, const int32_t* col_idx, int64_t nnz,
                                float softmax_scale, void* out, float* lse, void* stream) {
  return dhsa::sparse_prefill_impl(q, k, v, batch, seq_len, num_q_heads, num_kv_heads, head_dim,
                                   num_chunks, chunk_offsets, chunk_offsets_dev, row_ptr, col_idx,
                                   nnz, softmax_scale, out, lse, nullptr, 0, stream, true);
}

}  // extern "C"
