/*
 * dhsa.h -- C ABI of the DHSA (Dynamic Hierarchical Sparse Attention) prefill
 * path for one causal attention layer on an AMD Instinct MI355X (gfx950).
 *
 * The layer is the prefill of one decoder attention layer: BF16, causal,
 * forward only, head dimension 128, grouped-query attention (DHSA README,
 * "Installation": the sparse kernel is BF16, causal, forward-only and needs
 * head dimension 128; "Overview": DHSA handles prompt prefill only).  The
 * method sits between the query/key projections and the attention backend
 * (gist.science Technical Summary, "Key Contributions": drop-in module).
 *
 * Two calls make the path:
 *   dhsa_build_mask     q, k, chunk offsets, top-k  ->  CSR block list
 *   dhsa_sparse_prefill q, k, v, CSR                ->  out (and optional LSE)
 * and three stage calls expose its steps one by one (pool, chunk scores,
 * top-k) for stage-wise checking.  dhsa_build_mask_ex and dhsa_topk_csr_ex
 * widen the selection rule with per-row budgets and a recent-chunk window.
 * dhsa_nms_boundaries, the step before the path, turns per-token boundary
 * scores into chunk offsets.  dhsa_sparse_prefill_noalloc is
 * dhsa_sparse_prefill for callers that cannot allocate a workspace.
 *
 * Conventions shared by every call
 * --------------------------------
 * Tensors are dense, contiguous, row-major and live in device memory:
 *   q    bf16 [B][L][Hq][128]      k, v  bf16 [B][L][Hkv][128]
 *   out  bf16 [B][L][Hq][128]      lse   f32  [B][Hq][L]   (natural log)
 * bf16 values are passed as raw 16-bit patterns (uint16) through void*.
 * Query head h reads KV head h / (Hq / Hkv).
 *
 * Chunks.  Sequence b is cut into C_b chunks by offsets o_0 = 0 < o_1 < ... <
 * o_{C_b} = L (chunk c holds tokens [o_c, o_{c+1})).  The offsets of all
 * sequences are concatenated, C_b + 1 entries per sequence.  Every call that
 * needs them takes BOTH a host copy (chunk_offsets, used to validate and to
 * size launches) and a device copy with the same values (chunk_offsets_dev,
 * read by the kernels); the library never copies between them.
 *
 * Rows.  A CSR row is one (sequence b, query head h, query chunk i), numbered
 * r = Hq * cbase_b + h * C_b + i with cbase_b = C_0 + ... + C_{b-1}.
 * row_ptr has R + 1 entries (R = Hq * sum_b C_b), col_idx holds chunk
 * indices local to the sequence, ascending within a row.
 *
 * Ownership.  The caller allocates and frees every buffer (inputs, outputs,
 * workspaces).  The library allocates nothing and keeps no state besides a
 * thread-local error string, and, for dhsa_sparse_prefill_noalloc only, one
 * static 1 MiB device array per GPU and its per-device address.
 *
 * Asynchrony.  Work is enqueued on `stream` (a hipStream_t; NULL = the null
 * stream) and the calls never synchronise.  Host-side inputs may be released
 * as soon as a call returns.
 *
 * Errors.  Arguments are checked on the host before anything is enqueued;
 * on an error the call returns a negative status, enqueues nothing and
 * writes nothing.  DHSA_ERR_HIP reports a failed launch.  dhsa_last_error()
 * returns the calling thread's last message.  No C++ exception crosses the
 * ABI.
 *
 * Limits: 1 <= B <= DHSA_MAX_BATCH, head_dim == 128, Hq % Hkv == 0,
 * 1 <= C_b <= DHSA_MAX_CHUNKS for calls that select (the top-k keeps one
 * candidate set of a row in registers).
 */
#ifndef DHSA_H
#define DHSA_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define DHSA_HEAD_DIM 128
#define DHSA_MAX_BATCH 64
#define DHSA_MAX_CHUNKS 2048
#define DHSA_NMS_MAX_LEN 524288
#define DHSA_NOALLOC_MAX_TILES 65536

typedef enum dhsa_status {
  DHSA_OK = 0,
  DHSA_ERR_NULL_POINTER = -1,   /* a required pointer is NULL               */
  DHSA_ERR_SHAPE = -2,          /* batch/heads/head_dim/seq_len not allowed */
  DHSA_ERR_OFFSETS = -3,        /* offsets not 0 < ... < L, or C_b invalid  */
  DHSA_ERR_TOPK = -4,           /* topk < 1 or recent < 0                   */
  DHSA_ERR_CAPACITY = -5,       /* output or workspace buffer too small     */
  DHSA_ERR_CSR = -6,            /* CSR size arguments inconsistent          */
  DHSA_ERR_UNSUPPORTED = -7,    /* beyond a documented limit                */
  DHSA_ERR_HIP = -8             /* a HIP launch failed                      */
} dhsa_status;

/* Status name, e.g. "DHSA_ERR_OFFSETS".  Never NULL. */
const char* dhsa_status_string(int status);

/* Last error message of the calling thread ("" if none).  Never NULL. */
const char* dhsa_last_error(void);

/* ABI version of this library (major * 100 + minor). */
int dhsa_version(void);

/* ------------------------------------------------------------------------
 * Sizes (host only; no device access)
 * ---------------------------------------------------------------------- */

/* CSR sizes for a fixed row budget: row i of a sequence keeps min(topk, i+1)
 * chunks, so R = Hq * sum_b C_b and nnz = Hq * sum_b sum_i min(topk, i+1).
 * (DHSA README, "Predictor Checkpoints": static predictors use a fixed row
 * budget.)  num_chunks: host [batch].  Outputs may not be NULL. */
int dhsa_csr_size(int32_t batch, const int32_t* num_chunks, int32_t num_q_heads,
                  int32_t topk, int32_t* num_rows, int64_t* nnz);

/* CSR sizes when each row keeps at most min(topk + recent, i + 1) chunks:
 * nnz = Hq * sum_b sum_i min(topk + recent, i + 1).  Exact for one budget
 * per layer (row_budgets NULL in the _ex calls); with per-row budgets (each
 * capped at topk) it is the capacity col_idx needs, and the exact count is
 * row_ptr[R] on the device.  recent >= 0; dhsa_csr_size is recent = 0. */
int dhsa_csr_capacity(int32_t batch, const int32_t* num_chunks, int32_t num_q_heads,
                      int32_t topk, int32_t recent, int32_t* num_rows, int64_t* nnz);

/* Bytes of device workspace dhsa_build_mask needs: pooled Q and K (fp32),
 * the chunk-score matrices (fp32) and the pooling order (one int32 per
 * chunk: the pooling grid runs the chunks longest first), each 256-byte
 * aligned. */
int dhsa_mask_workspace_size(int32_t batch, const int32_t* num_chunks,
                             int32_t num_q_heads, int32_t num_kv_heads,
                             int32_t head_dim, size_t* bytes);

/* Bytes of device workspace dhsa_sparse_prefill needs (its query-tile list);
 * depends on the chunk lengths, hence the host offsets. */
int dhsa_prefill_workspace_size(int32_t batch, int32_t seq_len,
                                const int32_t* num_chunks,
                                const int32_t* chunk_offsets, size_t* bytes);

/* ------------------------------------------------------------------------
 * The two calls of the path
 * ---------------------------------------------------------------------- */

/* Mask construction: length-normalised pooling of Q and K per chunk, chunk
 * scores, and a causal top-k per query chunk, written as CSR.
 *   - pooling: qbar[b,h,c] = (sum of q over chunk c) / n_c * sqrt(n_c)
 *     (OpenReview abstract "...for On-Device LLMs": the averaged embeddings
 *     are scaled by the square root of the chunk size; gist.science
 *     Technical Summary, "Robust Chunk Representation");
 *   - scores: S[b,h,i,j] = qbar[b,h,i] . kbar[b,h/G,j] for j <= i, fp32,
 *     no 1/sqrt(d) (Technical Summary, Methodology, Step 1);
 *   - selection: row (b,h,i) keeps chunk i and the topk-1 earlier chunks
 *     with the highest scores, ties to the lower index, -0 == +0; all of
 *     0..i when i + 1 <= topk (Methodology, Step 2: causal selection; the
 *     kept chunks expand to their tokens, which dhsa_sparse_prefill does).
 * Inputs:  q, k (device bf16, see conventions), sizes, offsets (host and
 *          device copies), topk >= 1.
 * Outputs: row_ptr device int32 [R+1]; col_idx device int32 [col_capacity],
 *          col_capacity >= nnz of dhsa_csr_size; scores_out (nullable)
 *          device fp32, per sequence [Hq][C_b][C_b] concatenated, entries
 *          with j > i are not written.
 * workspace: device, >= dhsa_mask_workspace_size bytes, 256-byte aligned.
 * Errors: NULL pointers, shapes, offsets, topk, capacity, C_b >
 *         DHSA_MAX_CHUNKS. */
int dhsa_build_mask(const void* q, const void* k,
                    int32_t batch, int32_t seq_len, int32_t num_q_heads,
                    int32_t num_kv_heads, int32_t head_dim,
                    const int32_t* num_chunks, const int32_t* chunk_offsets,
                    const int32_t* chunk_offsets_dev, int32_t topk,
                    int32_t* row_ptr, int32_t* col_idx, int64_t col_capacity,
                    float* scores_out, void* workspace, size_t workspace_bytes,
                    void* stream);

/* dhsa_build_mask with a wider selection rule (DHSA README, "Predictor
 * Checkpoints": static predictors use a fixed row budget, dynamic ones a
 * query-dependent budget per row; the codewithpapers record of the DHSA
 * repository names a recent-key-block keep OR'ed with a scattered top-k by
 * row budget, without a formula).  Row (b,h,i) with budget k_r keeps:
 *   - chunk i and the `recent` chunks just before it (i-recent .. i-1),
 *   - the k_r - 1 highest-scoring chunks among j < i - recent (order and
 *     ties as in dhsa_build_mask),
 *   - every chunk 0..i when i + 1 <= k_r + recent.
 * row_budgets: NULL -> k_r = topk for every row; else device int32 [R] in
 *   CSR row order, read on the device, each value clamped to [1, topk]
 *   (so a predictor's output needs no host round trip), and row_ptr is
 *   built by a device prefix sum.
 * recent >= 0 (0 with NULL budgets is exactly dhsa_build_mask).
 * col_capacity >= nnz of dhsa_csr_capacity(topk, recent).  Other arguments,
 * outputs and errors as dhsa_build_mask. */
int dhsa_build_mask_ex(const void* q, const void* k,
                       int32_t batch, int32_t seq_len, int32_t num_q_heads,
                       int32_t num_kv_heads, int32_t head_dim,
                       const int32_t* num_chunks, const int32_t* chunk_offsets,
                       const int32_t* chunk_offsets_dev, int32_t topk,
                       const int32_t* row_budgets, int32_t recent,
                       int32_t* row_ptr, int32_t* col_idx, int64_t col_capacity,
                       float* scores_out, void* workspace, size_t workspace_bytes,
                       void* stream);

/* Block-sparse causal attention forward over the kept chunk tiles.
 * For query token t of chunk i, head h: out = softmax(scale * q_t k_s^T) v_s
 * over the tokens s of the kept chunks of row (b,h,i) with s <= t (token-
 * causal inside the diagonal chunk), computed tile by tile with an online
 * softmax so no score matrix is stored (gist.science Technical Summary,
 * "Hardware-Agnostic Backends": tiled online-softmax backend; DHSA README,
 * "Overview": block-sparse attention with variable-sized query and key
 * blocks).  Accumulation is fp32; out is rounded to bf16.
 * Inputs:  q, k, v device bf16; CSR row_ptr/col_idx (device, nnz entries)
 *          from dhsa_build_mask or any source whose rows are strictly
 *          ascending with entries in [0, i]; softmax_scale <= 0 selects
 *          1/sqrt(128).
 * Outputs: out device bf16 [B][L][Hq][128]; lse (nullable) device fp32
 *          [B][Hq][L].  A query with no visible key gets out = 0 and
 *          lse = -inf.
 * workspace: device, >= dhsa_prefill_workspace_size bytes.
 * Limit: seq_len * num_kv_heads * 256 bytes (one sequence's K, or V) must
 * stay below 4 GiB (DHSA_ERR_UNSUPPORTED otherwise).
 * Query tiles are 256 rows when at least half of the tiled query rows lie in
 * chunks longer than 128 rows, else 128; chunk remainders of at most 32 rows
 * run in one-wave tiles.
 * The environment variable DHSA_ATTN_BLOCK_M=128 or 256 forces the height.
 * Results of the two heights agree to rounding: a row whose tile changes
 * between a wide kernel and the one-wave kernel sees 32-key instead of
 * 64-key key blocks, so its running softmax maximum is refreshed at other
 * points.
 * The kernels bound-check CSR entries (entries outside [0, i] and row_ptr
 * values outside [0, nnz] are ignored), so a malformed CSR gives wrong
 * values but no out-of-bounds access.
 * Non-finite inputs: keys are processed in blocks of the row's gathered key
 * stream; a block's padding past the stream's end loads the stream's first
 * token, which every query row of the chunk sees.  A NaN or inf in K or V
 * therefore reaches the rows that see it and, through the causal mask's
 * exact-zero weights (0 * inf = NaN), the earlier query rows of its own
 * diagonal chunk; no other row reads it. */
int dhsa_sparse_prefill(const void* q, const void* k, const void* v,
                        int32_t batch, int32_t seq_len, int32_t num_q_heads,
                        int32_t num_kv_heads, int32_t head_dim,
                        const int32_t* num_chunks, const int32_t* chunk_offsets,
                        const int32_t* chunk_offsets_dev,
                        const int32_t* row_ptr, const int32_t* col_idx, int64_t nnz,
                        float softmax_scale, void* out, float* lse,
                        void* workspace, size_t workspace_bytes, void* stream);

/* dhsa_sparse_prefill without a workspace argument, for callers that cannot
 * allocate device memory around the call: code under HIP graph capture,
 * tight serving loops, harnesses that forbid allocation.  The query-tile
 * list lives in a static device array of the library (DHSA_NOALLOC_MAX_TILES
 * int4 entries, 1 MiB, one copy per GPU, held until the process ends); the
 * call allocates nothing.  Arguments, outputs and results are those of
 * dhsa_sparse_prefill (bit-identical: the same kernels run on the same
 * tiles).  Errors: those of dhsa_sparse_prefill, and DHSA_ERR_CAPACITY
 * when the problem needs more query tiles than the array holds (a tile is
 * at most 128 query rows of one chunk, so sum_b sum_c ceil(n_c / 128) <=
 * DHSA_NOALLOC_MAX_TILES always fits); the first call on a device looks up
 * the array's address (DHSA_ERR_HIP if that fails).  Every call on one GPU
 * shares its array: calls that overlap in time on one GPU (two streams, or
 * two host threads) race on it and give undefined results; serialise them. */
int dhsa_sparse_prefill_noalloc(const void* q, const void* k, const void* v,
                                int32_t batch, int32_t seq_len, int32_t num_q_heads,
                                int32_t num_kv_heads, int32_t head_dim,
                                const int32_t* num_chunks, const int32_t* chunk_offsets,
                                const int32_t* chunk_offsets_dev,
                                const int32_t* row_ptr, const int32_t* col_idx, int64_t nnz,
                                float softmax_scale, void* out, float* lse, void* stream);

/* ------------------------------------------------------------------------
 * Stage calls (the steps of dhsa_build_mask one at a time)
 * ---------------------------------------------------------------------- */

/* Pooling of one tensor x (device bf16 [B][L][H][128]) into pooled (device
 * fp32 [sum_b H*C_b][128], row H*cbase_b + h*C_b + c).  Citation as for the
 * pooling step of dhsa_build_mask. */
int dhsa_pool(const void* x, int32_t batch, int32_t seq_len, int32_t num_heads,
              int32_t head_dim, const int32_t* num_chunks,
              const int32_t* chunk_offsets, const int32_t* chunk_offsets_dev,
              float* pooled, void* stream);

/* Chunk scores from pooled Q (fp32 rows as dhsa_pool with H = Hq) and
 * pooled K (H = Hkv) into scores (device fp32, per sequence [Hq][C_b][C_b]
 * concatenated; j > i not written). */
int dhsa_chunk_scores(const float* qbar, const float* kbar, int32_t batch,
                      int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim,
                      const int32_t* num_chunks, float* scores, void* stream);

/* Causal top-k of given fp32 chunk scores (layout of dhsa_chunk_scores) into
 * CSR, with the selection rule of dhsa_build_mask.  NaN scores rank below
 * every number. */
int dhsa_topk_csr(const float* scores, int32_t batch, int32_t num_q_heads,
                  const int32_t* num_chunks, int32_t topk, int32_t* row_ptr,
                  int32_t* col_idx, int64_t col_capacity, void* stream);

/* dhsa_topk_csr with the selection rule of dhsa_build_mask_ex (row_budgets
 * nullable device int32 [R], clamped to [1, topk]; recent >= 0;
 * col_capacity >= nnz of dhsa_csr_capacity). */
int dhsa_topk_csr_ex(const float* scores, int32_t batch, int32_t num_q_heads,
                     const int32_t* num_chunks, int32_t topk,
                     const int32_t* row_budgets, int32_t recent, int32_t* row_ptr,
                     int32_t* col_idx, int64_t col_capacity, void* stream);

/* ------------------------------------------------------------------------
 * A whole layer over a batch, within a workspace budget
 * ---------------------------------------------------------------------- */

/* Bytes of device workspace dhsa_layer_forward needs to process any
 * max_group consecutive sequences in one pass (mask workspace, CSR buffers
 * and attention workspace of the largest such group, 256-byte aligned
 * parts).  max_group = 1 sizes the sequential per-sequence loop;
 * max_group >= batch sizes one pass over the whole batch.  recent as in
 * dhsa_build_mask_ex. */
int dhsa_layer_workspace_size(int32_t batch, int32_t seq_len, int32_t num_q_heads,
                              int32_t num_kv_heads, int32_t head_dim,
                              const int32_t* num_chunks, const int32_t* chunk_offsets,
                              int32_t topk, int32_t recent, int32_t max_group,
                              size_t* bytes);

/* One attention layer: dhsa_build_mask_ex then dhsa_sparse_prefill, run over
 * groups of consecutive sequences, each group as large as the workspace
 * allows (gist.science Technical Summary, Experimental Results, Efficiency,
 * "Batching": under a memory limit
 * the batch is processed sequence by sequence in a plain loop rather than
 * in one batched call).  Groups run in order on `stream` and reuse the one
 * workspace; results equal those of one pass over the whole batch.
 * Inputs, outputs and selection arguments as dhsa_build_mask_ex and
 * dhsa_sparse_prefill (row_budgets nullable, in CSR row order of the whole
 * batch).  num_groups (host, nullable) receives the number of groups.
 * workspace: device, 256-byte aligned; workspace_bytes must hold at least
 * the largest single sequence (dhsa_layer_workspace_size with max_group 1).
 * Errors: as the two calls, checked for the whole batch before anything is
 * enqueued; DHSA_ERR_CAPACITY when one sequence alone does not fit.  A
 * DHSA_ERR_HIP from a later group leaves the earlier groups enqueued. */
int dhsa_layer_forward(const void* q, const void* k, const void* v,
                       int32_t batch, int32_t seq_len, int32_t num_q_heads,
                       int32_t num_kv_heads, int32_t head_dim,
                       const int32_t* num_chunks, const int32_t* chunk_offsets,
                       const int32_t* chunk_offsets_dev, int32_t topk,
                       const int32_t* row_budgets, int32_t recent,
                       float softmax_scale, void* out, float* lse,
                       void* workspace, size_t workspace_bytes,
                       int32_t* num_groups, void* stream);

/* ------------------------------------------------------------------------
 * Boundary finalisation (the step that produces the chunk offsets)
 * ---------------------------------------------------------------------- */

/* Entries per sequence that dhsa_nms_boundaries' offsets_out needs:
 * max(seq_len / min_gap, 1) + 1 (every chunk holds >= min_gap tokens). */
int dhsa_nms_offsets_stride(int32_t seq_len, int32_t min_gap, int32_t* stride);

/* Bytes of device workspace dhsa_nms_boundaries needs: two int32 candidate
 * lists per sequence, seq_len entries each. */
int dhsa_nms_workspace_size(int32_t batch, int32_t seq_len, int32_t min_gap,
                            size_t* bytes);

/* Non-maximum suppression of per-token boundary scores into chunk offsets
 * (gist.science Technical Summary, Methodology, "Dynamic Boundary
 * Detection": the boundary predictor finalises boundaries with NMS so that
 * they are well separated and robust to noise; the window and threshold
 * are not given there, so both are arguments).
 *   scores[b][t] (device fp32 [B][L]) scores "a chunk starts at token t".
 *   Token t with min_gap <= t <= L - min_gap and scores >= threshold is a
 *   candidate (NaN never is); candidates are taken by score descending,
 *   then token ascending, and kept when every kept boundary, the ends 0 and
 *   L included, is >= min_gap tokens away.
 * Outputs: offsets_out device int32 [B][offsets_stride]: row b holds
 *          0, kept tokens ascending, L (C_b + 1 entries; the rest of the
 *          row is not written); num_chunks_out device int32 [B] = C_b.
 *          Every chunk holds >= min_gap tokens (or L < 2 min_gap and
 *          C_b = 1).  The offsets feed dhsa_build_mask after a copy to the
 *          host (the path sizes its launches from host offsets).
 * workspace: device, >= dhsa_nms_workspace_size bytes, 256-byte aligned.
 * Errors: NULL pointers; batch outside [1, DHSA_MAX_BATCH], seq_len < 1,
 *         min_gap < 1 or a NaN threshold (DHSA_ERR_SHAPE); seq_len >
 *         DHSA_NMS_MAX_LEN (DHSA_ERR_UNSUPPORTED: the per-token state of a
 *         sequence lives in one workgroup's LDS, 2 bits per token);
 *         offsets_stride or workspace too small (DHSA_ERR_CAPACITY). */
int dhsa_nms_boundaries(const float* scores, int32_t batch, int32_t seq_len,
                        int32_t min_gap, float threshold, int32_t* offsets_out,
                        int32_t offsets_stride, int32_t* num_chunks_out,
                        void* workspace, size_t workspace_bytes, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* DHSA_H */
