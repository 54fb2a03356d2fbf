// Length-normalised chunk pooling (segmented column sums over [L, H*128]).
//
// pooled[b,h,c,:] = (sum over tokens t of chunk c of x[b,t,h,:]) / sqrt(n_c),
// i.e. the chunk mean scaled by sqrt(n_c) (OpenReview abstract "...for
// On-Device LLMs"; gist.science Technical Summary, "Robust Chunk
// Representation").
//
// In BSHD a chunk of x is one contiguous slab of n_c rows of H*128 bf16, so
// pooling is a segmented column sum.  A workgroup owns one chunk and a slab
// of 512 columns (4 heads): each of its 4 waves reads whole 1 KB row
// segments (64 lanes x 16 B, fully coalesced) of every 4th row, keeping 8
// independent row accumulators in flight per lane; the waves are then
// combined in LDS in a fixed order, so the result is deterministic.
#include "dhsa_internal.h"

namespace dhsa {
namespace {

constexpr int kCols = 512;      // columns per workgroup
constexpr int kUnroll = 8;      // rows in flight per wave

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

struct PoolJob {
  const uint16_t* x;
  float* out;
  int32_t heads;
  int32_t nblk;  // column blocks of kCols
};

__device__ __forceinline__ void add_bf16x8(float* acc, const u32x4& v) {
  const uint32_t w[4] = {v[0], v[1], v[2], v[3]};
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    acc[2 * e] += __uint_as_float(w[e] << 16);
    acc[2 * e + 1] += __uint_as_float(w[e] & 0xffff0000u);
  }
}

__global__ __launch_bounds__(256) void pool_kernel(PoolJob j0, PoolJob j1,
                                                   int32_t total_chunks,
                                                   const int32_t* __restrict__ offs,
                                                   SeqTable st, int32_t seq_len) {
  __shared__ float red[4][kCols];
  const int per0 = total_chunks * j0.nblk;
  const bool first = (int)blockIdx.x < per0;
  const PoolJob J = first ? j0 : j1;
  const int local = first ? (int)blockIdx.x : (int)blockIdx.x - per0;
  const int cg = local / J.nblk;
  const int blk = local - cg * J.nblk;
  const int b = find_seq(st.cbase, st.batch, cg);
  const int c = cg - st.cbase[b];
  const int C = st.num_chunks[b];
  const int obase = st.cbase[b] + b;
  const int t0 = offs[obase + c];
  const int n = offs[obase + c + 1] - t0;

  const int wave = threadIdx.x >> 6;
  const int lane = threadIdx.x & 63;
  const int ncols = J.heads * kHeadDim;
  const int col = blk * kCols + lane * 8;
  const bool active = col < ncols;

  float acc[kUnroll][8];
#pragma unroll
  for (int u = 0; u < kUnroll; ++u)
#pragma unroll
    for (int e = 0; e < 8; ++e) acc[u][e] = 0.f;

  if (active) {
    const size_t rs = (size_t)ncols;
    const uint16_t* base = J.x + ((size_t)b * seq_len + t0) * rs + col;
    int t = wave;
    for (; t + 4 * (kUnroll - 1) < n; t += 4 * kUnroll) {
      u32x4 v[kUnroll];
#pragma unroll
      for (int u = 0; u < kUnroll; ++u)
        v[u] = __builtin_nontemporal_load(
            reinterpret_cast<const u32x4*>(base + (size_t)(t + 4 * u) * rs));
#pragma unroll
      for (int u = 0; u < kUnroll; ++u) add_bf16x8(acc[u], v[u]);
    }
    // fewer than kUnroll rows of this wave remain
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
      if (t + 4 * u < n) {
        const u32x4 v = *reinterpret_cast<const u32x4*>(base + (size_t)(t + 4 * u) * rs);
        add_bf16x8(acc[u], v);
      }
    }
  }
  // fixed-order combine: accumulators, then waves
  float s[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    float a = 0.f;
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) a += acc[u][e];
    s[e] = a;
  }
#pragma unroll
  for (int e = 0; e < 8; ++e) red[wave][lane * 8 + e] = s[e];
  __syncthreads();
  const float inv = 1.0f / sqrtf((float)n);
  for (int idx = threadIdx.x; idx < kCols; idx += 256) {
    const int cc = blk * kCols + idx;
    if (cc >= ncols) continue;
    const float tot = ((red[0][idx] + red[1][idx]) + red[2][idx]) + red[3][idx];
    const int h = cc / kHeadDim;
    const int d = cc - h * kHeadDim;
    const size_t row = (size_t)J.heads * st.cbase[b] + (size_t)h * C + c;
    J.out[row * kHeadDim + d] = tot * inv;
  }
}

}  // namespace

hipError_t launch_pool(const uint16_t* x0, float* out0, int32_t h0,
                       const uint16_t* x1, float* out1, int32_t h1,
                       int32_t total_chunks, const int32_t* offs_dev,
                       const SeqTable& st, int32_t seq_len, hipStream_t stream) {
  PoolJob j0{x0, out0, h0, (h0 * kHeadDim + kCols - 1) / kCols};
  PoolJob j1{x1, out1, h1, x1 ? (h1 * kHeadDim + kCols - 1) / kCols : 0};
  const int64_t grid = (int64_t)total_chunks * (j0.nblk + j1.nblk);
  if (grid <= 0) return hipSuccess;
  hipLaunchKernelGGL(pool_kernel, dim3((unsigned)grid), dim3(256), 0, stream, j0, j1,
                     total_chunks, offs_dev, st, seq_len);
  return hipGetLastError();
}

}  // namespace dhsa
