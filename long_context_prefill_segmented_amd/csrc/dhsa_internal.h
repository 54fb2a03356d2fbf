// Internal declarations shared by the host entry points and the kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "dhsa.h"

namespace dhsa {

constexpr int kHeadDim = DHSA_HEAD_DIM;
constexpr int kMaxBatch = DHSA_MAX_BATCH;
constexpr int kMaxChunks = DHSA_MAX_CHUNKS;

// Attention tiling: a workgroup of NW waves owns 32 * NW query rows (the
// query tile) of one query chunk and one query head, and streams the
// gathered kept keys kBlockN at a time.  Two tile heights are built: 128 rows
// (4 waves, two workgroups per CU) and 256 rows (8 waves, one per CU; every
// K/V sub-tile serves twice the rows).
constexpr int kBlockMSmall = 128;
constexpr int kBlockMLarge = 256;
constexpr int kBlockN = 64;

// Per-sequence bookkeeping passed by value in kernel arguments (host
// computed, so no upload is needed).
struct SeqTable {
  int32_t batch;
  int32_t num_chunks[kMaxBatch];
  int32_t cbase[kMaxBatch];    // sum of C over earlier sequences
  int32_t tbase[kMaxBatch];    // first query tile of the sequence
  int32_t ntbase[kMaxBatch];   // first narrow query tile of the sequence
  int64_t sbase[kMaxBatch];    // first score element of the sequence
  int64_t nbase[kMaxBatch];    // first CSR entry of the sequence
};

// Finds the sequence that owns global index x given per-sequence starts
// (starts[0] == 0, nondecreasing).
template <typename T>
__device__ __forceinline__ int find_seq(const T* starts, int batch, T x) {
  int b = 0;
  while (b + 1 < batch && starts[b + 1] <= x) ++b;
  return b;
}

// kernels' launchers (each returns hipGetLastError() of its launch)
// order (nullable, total_chunks int32 of device scratch): the pooling grid
// then runs the chunks longest first, used up to kPoolOrderMaxChunks chunks
// in all.  Up to kPoolOrderArgChunks chunks the host computes the order from
// offs_host (the concatenated host offsets) and passes it in the kernel's
// arguments; beyond that a one-workgroup device sort fills order.
constexpr int kPoolOrderMaxChunks = 16384;
constexpr int kPoolOrderArgChunks = 512;
hipError_t launch_pool(const uint16_t* x0, float* out0, int32_t h0,
                       const uint16_t* x1, float* out1, int32_t h1,
                       int32_t total_chunks, const int32_t* offs_dev,
                       const int32_t* offs_host, const SeqTable& st, int32_t seq_len,
                       int32_t* order, hipStream_t stream);

hipError_t launch_scores(const float* qbar, const float* kbar, float* scores,
                         int32_t hq, int32_t hkv, const SeqTable& st,
                         int64_t total_tiles, hipStream_t stream);

// topk: the uniform row budget, or the cap of the per-row budgets when
// budgets (device int32, one per CSR row) is not NULL; recent: window width.
hipError_t launch_topk(const float* scores, const SeqTable& st, int32_t hq,
                       int32_t total_rows, int32_t topk, int32_t recent,
                       const int32_t* budgets, int32_t max_chunks, int32_t* row_ptr,
                       int32_t* col_idx, hipStream_t stream);

// Longest sequence the boundary NMS takes: its per-token 2-bit states fill
// 128 KB of LDS.  workspace: batch * 2 * seq_len int32 candidate lists.
constexpr int kNmsMaxLen = DHSA_NMS_MAX_LEN;
hipError_t launch_nms(const float* scores, int32_t batch, int32_t seq_len, int32_t min_gap,
                      float threshold, int32_t* offsets_out, int32_t stride,
                      int32_t* num_chunks_out, void* workspace, hipStream_t stream);

// host side: set the calling thread's error message and return status
int fail(int status, const char* fmt, ...);
int ok();

// query-tile remainders of at most this many rows go to the narrow list
constexpr int kNarrowRows = 32;

hipError_t launch_plan_tiles(const int32_t* offs_dev, const SeqTable& st,
                             int4* tiles, int4* narrow, int32_t block_m, hipStream_t stream);

struct AttnParams {
  const uint16_t* q;
  const uint16_t* k;
  const uint16_t* v;
  uint16_t* o;
  float* lse;
  const int4* tiles;
  const int4* narrow;  // tiles of at most kNarrowRows rows (one wave each)
  const int32_t* offs;
  const int32_t* row_ptr;
  const int32_t* col_idx;
  int64_t nnz;
  int32_t num_tiles;
  int32_t num_narrow;
  int32_t seq_len;
  int32_t hq;
  int32_t hkv;
  int32_t block_m;  // query tile height: kBlockMSmall or kBlockMLarge
  float scale_log2;
};

hipError_t launch_attention(const AttnParams& p, const SeqTable& st,
                            hipStream_t stream);

}  // namespace dhsa
