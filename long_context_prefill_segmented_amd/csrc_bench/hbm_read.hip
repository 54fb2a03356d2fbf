// Streaming-read reference for bench.py: how fast this GPU's HBM delivers a
// large buffer to a kernel that only reads it, with the pooling kernel's
// access form (16-byte non-temporal loads, eight in flight per lane).  It is
// a measuring aid, not part of the DHSA library: bench.py reports the
// pooling and mask bandwidth against it next to the 8 TB/s nominal peak.
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
constexpr int kThreads = 256;
constexpr int kInFlight = 8;

// Each thread reads 16-byte words w = gid + u * stride (u < kInFlight) per
// round, rounds advancing by kInFlight * stride, and folds them into one
// value so that no load is dead; one 32-bit result per workgroup.
__global__ __launch_bounds__(kThreads) void hbm_read_kernel(const u32x4* __restrict__ src,
                                                            int64_t words,
                                                            uint32_t* __restrict__ out) {
  const int64_t stride = (int64_t)gridDim.x * kThreads;
  const int64_t gid = (int64_t)blockIdx.x * kThreads + threadIdx.x;
  uint32_t acc = 0;
  int64_t w = gid;
  for (; w + (kInFlight - 1) * stride < words; w += kInFlight * stride) {
    u32x4 v[kInFlight];
#pragma unroll
    for (int u = 0; u < kInFlight; ++u) v[u] = __builtin_nontemporal_load(src + w + u * stride);
#pragma unroll
    for (int u = 0; u < kInFlight; ++u) acc ^= v[u][0] ^ v[u][1] ^ v[u][2] ^ v[u][3];
  }
  for (; w < words; w += stride) {
    const u32x4 v = src[w];
    acc ^= v[0] ^ v[1] ^ v[2] ^ v[3];
  }
  __shared__ uint32_t red[kThreads];
  red[threadIdx.x] = acc;
  __syncthreads();
  if (threadIdx.x == 0) {
    uint32_t a = 0;
    for (int t = 0; t < kThreads; ++t) a ^= red[t];
    out[blockIdx.x] = a;
  }
}

}  // namespace

extern "C" {

// Reads bytes (a multiple of 16) from the device buffer src with grid
// workgroups of 256 threads; out: device uint32 [grid].  Returns 0, or the
// hipError_t of the launch.
int dhsa_bench_hbm_read(const void* src, int64_t bytes, uint32_t* out, int32_t grid,
                        void* stream) {
  if (src == nullptr || out == nullptr || bytes <= 0 || bytes % 16 != 0 || grid <= 0) return -1;
  hipLaunchKernelGGL(hbm_read_kernel, dim3((unsigned)grid), dim3(kThreads), 0,
                     static_cast<hipStream_t>(stream), static_cast<const u32x4*>(src),
                     bytes / 16, out);
  return (int)hipGetLastError();
}

}  // extern "C"
