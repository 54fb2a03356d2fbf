// One attention layer (mask construction + block-sparse attention) over a
// batch of sequences, processed in groups of consecutive sequences that fit
// a caller-given workspace.  A budget that holds one sequence's buffers gives
// the sequential per-sequence loop (gist.science Technical Summary, Experimental Results,
// Efficiency, "Batching": in memory-constrained settings the batch is processed one
// sequence after another in a plain loop instead of one batched call);
// a budget that holds every sequence gives one pass over the whole batch.
// Host code only: each group is two calls of the C ABI on the caller's
// stream, which orders the reuse of the workspace between groups.
#include <cmath>

#include "dhsa_internal.h"

namespace dhsa {
namespace {

constexpr size_t kLayerAlign = 256;
size_t al(size_t x) { return (x + kLayerAlign - 1) / kLayerAlign * kLayerAlign; }

struct GroupLayout {
  size_t mask, row_ptr, col_idx, prefill;  // bytes of each part
  int32_t rows;
  int64_t nnz_cap;
  size_t total() const { return mask + row_ptr + col_idx + prefill; }
};

// buffers for sequences [b0, b1); offs points at sequence b0's offsets
int group_layout(int32_t b0, int32_t b1, int32_t seq_len, int32_t hq, int32_t hkv,
                 const int32_t* num_chunks, const int32_t* offs, int32_t topk, int32_t recent,
                 GroupLayout* g) {
  const int32_t n = b1 - b0;
  size_t mask = 0, pre = 0;
  int s = dhsa_mask_workspace_size(n, num_chunks + b0, hq, hkv, kHeadDim, &mask);
  if (s) return s;
  s = dhsa_prefill_workspace_size(n, seq_len, num_chunks + b0, offs, &pre);
  if (s) return s;
  s = dhsa_csr_capacity(n, num_chunks + b0, hq, topk, recent, &g->rows, &g->nnz_cap);
  if (s) return s;
  g->mask = al(mask);
  g->row_ptr = al(sizeof(int32_t) * ((size_t)g->rows + 1));
  g->col_idx = al(sizeof(int32_t) * (size_t)(g->nnz_cap > 0 ? g->nnz_cap : 1));
  g->prefill = al(pre);
  return DHSA_OK;
}

}  // namespace
}  // namespace dhsa

using namespace dhsa;

extern "C" {

int dhsa_layer_workspace_size(int32_t batch, int32_t seq_len, int32_t num_q_heads,
                              int32_t num_kv_heads, int32_t head_dim, const int32_t* num_chunks,
                              const int32_t* chunk_offsets, int32_t topk, int32_t recent,
                              int32_t max_group, size_t* bytes) {
  if (bytes == nullptr) return fail(DHSA_ERR_NULL_POINTER, "bytes is NULL");
  if (head_dim != kHeadDim) return fail(DHSA_ERR_SHAPE, "head_dim %d != %d", head_dim, kHeadDim);
  if (max_group < 1) return fail(DHSA_ERR_SHAPE, "max_group %d < 1", max_group);
  // validates batch, chunk counts, offsets, heads, topk and recent once
  GroupLayout whole;
  int s = group_layout(0, batch, seq_len, num_q_heads, num_kv_heads, num_chunks, chunk_offsets,
                       topk, recent, &whole);
  if (s) return s;
  const int32_t m = max_group < batch ? max_group : batch;
  size_t worst = 0;
  size_t o = 0;  // offsets index of sequence b0
  for (int32_t b0 = 0; b0 + m <= batch; ++b0) {
    GroupLayout g;
    s = group_layout(b0, b0 + m, seq_len, num_q_heads, num_kv_heads, num_chunks,
                     chunk_offsets + o, topk, recent, &g);
    if (s) return s;
    worst = g.total() > worst ? g.total() : worst;
    o += num_chunks[b0] + 1;
  }
  *bytes = worst;
  return ok();
}

int dhsa_layer_forward(const void* q, const void* k, const void* v, int32_t batch,
                       int32_t seq_len, int32_t num_q_heads, int32_t num_kv_heads,
                       int32_t head_dim, const int32_t* num_chunks, const int32_t* chunk_offsets,
                       const int32_t* chunk_offsets_dev, int32_t topk,
                       const int32_t* row_budgets, int32_t recent, float softmax_scale,
                       void* out, float* lse, void* workspace, size_t workspace_bytes,
                       int32_t* num_groups, void* stream) {
  if (!q || !k || !v || !chunk_offsets_dev || !out || !workspace)
    return fail(DHSA_ERR_NULL_POINTER, "NULL device pointer");
  if (head_dim != kHeadDim) return fail(DHSA_ERR_SHAPE, "head_dim %d != %d", head_dim, kHeadDim);
  if (!std::isfinite(softmax_scale))
    return fail(DHSA_ERR_SHAPE, "softmax_scale is not finite");
  if (reinterpret_cast<uintptr_t>(workspace) % kLayerAlign)
    return fail(DHSA_ERR_CAPACITY, "workspace not %zu-byte aligned", kLayerAlign);
  GroupLayout whole;
  int s = group_layout(0, batch, seq_len, num_q_heads, num_kv_heads, num_chunks, chunk_offsets,
                       topk, recent, &whole);
  if (s) return s;
  int cmax = 0;
  for (int b = 0; b < batch; ++b) cmax = num_chunks[b] > cmax ? num_chunks[b] : cmax;
  if (cmax > kMaxChunks)
    return fail(DHSA_ERR_UNSUPPORTED, "more than %d chunks in a sequence", kMaxChunks);

  // plan: greedy groups of consecutive sequences within the budget (the
  // bytes a group needs grow with every sequence added)
  int32_t starts[kMaxBatch + 1];
  size_t ostart[kMaxBatch + 1];
  size_t o = 0;
  for (int b = 0; b < batch; ++b) {
    ostart[b] = o;
    o += num_chunks[b] + 1;
  }
  ostart[batch] = o;
  int32_t ng = 0;
  for (int32_t b0 = 0; b0 < batch;) {
    int32_t b1 = b0;
    while (b1 < batch) {
      GroupLayout g;
      s = group_layout(b0, b1 + 1, seq_len, num_q_heads, num_kv_heads, num_chunks,
                       chunk_offsets + ostart[b0], topk, recent, &g);
      if (s) return s;
      if (g.total() > workspace_bytes) break;
      ++b1;
    }
    if (b1 == b0) {
      GroupLayout g;
      group_layout(b0, b0 + 1, seq_len, num_q_heads, num_kv_heads, num_chunks,
                   chunk_offsets + ostart[b0], topk, recent, &g);
      return fail(DHSA_ERR_CAPACITY, "workspace %zu < %zu bytes needed by sequence %d alone",
                  workspace_bytes, g.total(), b0);
    }
    starts[ng++] = b0;
    b0 = b1;
  }
  starts[ng] = batch;

  // run the groups in order on the stream
  const size_t qs = (size_t)seq_len * num_q_heads * kHeadDim;   // elements per sequence
  const size_t kvs = (size_t)seq_len * num_kv_heads * kHeadDim;
  int64_t rows_before = 0;
  for (int32_t gi = 0; gi < ng; ++gi) {
    const int32_t b0 = starts[gi], b1 = starts[gi + 1], n = b1 - b0;
    GroupLayout g;
    s = group_layout(b0, b1, seq_len, num_q_heads, num_kv_heads, num_chunks,
                     chunk_offsets + ostart[b0], topk, recent, &g);
    if (s) return s;
    char* ws = static_cast<char*>(workspace);
    void* mask_ws = ws;
    int32_t* row_ptr = reinterpret_cast<int32_t*>(ws + g.mask);
    int32_t* col_idx = reinterpret_cast<int32_t*>(ws + g.mask + g.row_ptr);
    void* pre_ws = ws + g.mask + g.row_ptr + g.col_idx;
    const uint16_t* qg = static_cast<const uint16_t*>(q) + (size_t)b0 * qs;
    const uint16_t* kg = static_cast<const uint16_t*>(k) + (size_t)b0 * kvs;
    const uint16_t* vg = static_cast<const uint16_t*>(v) + (size_t)b0 * kvs;
    uint16_t* og = static_cast<uint16_t*>(out) + (size_t)b0 * qs;
    float* lg = lse ? lse + (size_t)b0 * num_q_heads * seq_len : nullptr;
    const int32_t* bg = row_budgets ? row_budgets + rows_before : nullptr;
    s = dhsa_build_mask_ex(qg, kg, n, seq_len, num_q_heads, num_kv_heads, head_dim,
                           num_chunks + b0, chunk_offsets + ostart[b0],
                           chunk_offsets_dev + ostart[b0], topk, bg, recent, row_ptr, col_idx,
                           g.nnz_cap, nullptr, mask_ws, g.mask, stream);
    if (s) return s;
    s = dhsa_sparse_prefill(qg, kg, vg, n, seq_len, num_q_heads, num_kv_heads, head_dim,
                            num_chunks + b0, chunk_offsets + ostart[b0],
                            chunk_offsets_dev + ostart[b0], row_ptr, col_idx, g.nnz_cap,
                            softmax_scale, og, lg, pre_ws, g.prefill, stream);
    if (s) return s;
    rows_before += (int64_t)g.rows;
  }
  if (num_groups) *num_groups = ng;
  return ok();
}

}  // extern "C"
