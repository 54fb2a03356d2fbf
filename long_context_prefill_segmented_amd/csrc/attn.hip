// Variable-block-size block-sparse causal attention forward (bf16 MFMA,
// fp32 online softmax) over the kept chunk tiles of a CSR block list.
//
// For query token t of chunk i and head h the kernel computes
//   out[t,h] = sum_s softmax_s(scale * q_t . k_s) v_s
// over the tokens s of the kept chunks of row (b,h,i) with s <= t, the
// kept chunk list expanded to tokens (gist.science Technical Summary,
// Methodology, Step 2; OpenReview abstract: chunk scores upsampled to token
// level) and evaluated tile by tile with a streaming softmax that never
// stores the score matrix (Technical Summary, "Hardware-Agnostic Backends":
// tiled online-softmax backend; DHSA README, "Overview": block-sparse
// attention with variable-sized query and key blocks).
//
// Work decomposition (gfx950, wave64):
//  * a workgroup = 4 waves = 128 query rows of ONE query chunk and ONE query
//    head; each wave owns 32 rows;
//  * the kept chunks of the row are concatenated into one gathered key
//    stream (a prefix table in LDS maps stream positions to tokens), cut
//    into 64-key sub-tiles that may cross chunk boundaries, so short chunks
//    waste no MFMA work on padding;
//  * per sub-tile: S^T = K Q^T with v_mfma_f32_32x32x16_bf16 (K from LDS as
//    the A operand, Q held in registers as the B operand), so each lane owns
//    the scores of one query; the running max / sum live per lane; P^T is
//    rounded to bf16 in registers and feeds O^T += V^T P^T directly as the
//    B operand.  V is stored transposed in LDS with the key order permuted
//    (bits 2 and 3 of the key index swapped) so that each A-operand read is
//    one 16-byte LDS load;
//  * only the diagonal chunk needs the token-causal test (every earlier
//    kept chunk lies entirely before the query chunk), and its key range is
//    cut at the tile's last query row.
//  * workgroups are renumbered so that each XCD (own L2) works on a
//    contiguous range of (KV head, query tile) pairs, keeping one KV head's
//    K/V hot in that XCD's L2.
#include <float.h>

#include "dhsa_internal.h"

namespace dhsa {
namespace {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

constexpr int kKStride = kHeadDim + 8;  // bf16 per K row in LDS (272 B)
constexpr int kVStride = kBlockN + 8;   // bf16 per V^T row in LDS (144 B)
constexpr int kTable = 512;             // kept chunks per table window
constexpr int kNumXcd = 8;

__device__ __forceinline__ int xcd_remap(int w, int W) {
  const int q = W / kNumXcd, r = W % kNumXcd;
  const int x = w % kNumXcd, idx = w / kNumXcd;
  return x < r ? x * (q + 1) + idx : r * (q + 1) + (x - r) * q + idx;
}

__device__ __forceinline__ uint16_t f32_to_bf16_bits(float x) {
  return __builtin_bit_cast(uint16_t, (__bf16)x);
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

__global__ __launch_bounds__(256) void attn_fwd_kernel(AttnParams p, SeqTable st) {
  __shared__ __attribute__((aligned(16))) uint16_t Ks[kBlockN * kKStride];
  __shared__ __attribute__((aligned(16))) uint16_t Vt[kHeadDim * kVStride];
  __shared__ int tbl_start[kTable];
  __shared__ int tbl_pref[kTable + 1];
  __shared__ int wsum[4];
  __shared__ int s_diag[2];

  const int tid = threadIdx.x;
  const int wv = tid >> 6;
  const int lane = tid & 63;
  const int l32 = lane & 31;
  const int hl = lane >> 5;

  // ---- which (KV head, query tile, query head) this workgroup owns
  const int G = p.hq / p.hkv;
  const int W = p.num_tiles * p.hq;
  const int w = xcd_remap((int)blockIdx.x, W);
  const int hg = w % G;
  const int rest = w / G;
  const int tile = rest % p.num_tiles;
  const int g = rest / p.num_tiles;
  const int h = g * G + hg;
  const int4 te = p.tiles[tile];
  const int b = te.x, i = te.y, q0 = te.z;
  const int C = st.num_chunks[b];
  const int obase = st.cbase[b] + b;
  const int o_i = p.offs[obase + i];
  const int n_i = p.offs[obase + i + 1] - o_i;
  const int rows = min(kBlockM, n_i - q0);
  const int r = p.hq * st.cbase[b] + h * C + i;
  int64_t e0 = p.row_ptr[r], e1 = p.row_ptr[r + 1];
  e0 = e0 < 0 ? 0 : (e0 > p.nnz ? p.nnz : e0);
  e1 = e1 < e0 ? e0 : (e1 > p.nnz ? p.nnz : e1);

  // ---- Q fragment (B operand of S^T): lane -> query row, 8 dims per step
  const int qloc = wv * 32 + l32;       // row within the tile
  const int qrow = q0 + qloc;           // row within the chunk
  const bool qvalid = qloc < rows;
  const bool wave_active = wv * 32 < rows;
  bf16x8_t qf[8];
  {
    const uint16_t* qp = p.q + (((size_t)b * p.seq_len + o_i + qrow) * p.hq + h) * kHeadDim + hl * 8;
#pragma unroll
    for (int ds = 0; ds < 8; ++ds) {
      if (qvalid) {
        qf[ds] = *reinterpret_cast<const bf16x8_t*>(qp + ds * 16);
      } else {
#pragma unroll
        for (int e = 0; e < 8; ++e) qf[ds][e] = (__bf16)0.0f;
      }
    }
  }

  f32x16 oacc[4];
#pragma unroll
  for (int db = 0; db < 4; ++db)
#pragma unroll
    for (int rr = 0; rr < 16; ++rr) oacc[db][rr] = 0.f;
  float m_run = -INFINITY;
  float l_run = 0.f;

  const size_t kv_rs = (size_t)p.hkv * kHeadDim;
  const uint16_t* kbase = p.k + (size_t)b * p.seq_len * kv_rs + (size_t)g * kHeadDim;
  const uint16_t* vbase = p.v + (size_t)b * p.seq_len * kv_rs + (size_t)g * kHeadDim;

  // loader role: 4 consecutive keys x 8 dims per thread
  const int kg = tid >> 4;
  const int dc = tid & 15;
  const int key0 = 4 * kg;
  const int vpos0 = (key0 & ~12) | ((key0 & 4) << 1) | ((key0 & 8) >> 1);

  for (int64_t wb = e0; wb < e1; wb += kTable) {
    const int nent = (int)((e1 - wb) < kTable ? (e1 - wb) : kTable);
    __syncthreads();  // the previous window's table is no longer read
    int len2[2], beg2[2];
    int diag_u = -1;
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      const int idx = 2 * tid + u;
      len2[u] = 0;
      beg2[u] = 0;
      if (idx < nent) {
        const int j = p.col_idx[wb + idx];
        if (j >= 0 && j <= i) {
          beg2[u] = p.offs[obase + j];
          len2[u] = p.offs[obase + j + 1] - beg2[u];
          if (j == i) {
            len2[u] = min(len2[u], q0 + rows);
            diag_u = u;
          }
        }
      }
    }
    const int loc = len2[0] + len2[1];
    int incl = loc;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
      const int y = __shfl_up(incl, off, 64);
      if (lane >= off) incl += y;
    }
    if (lane == 63) wsum[wv] = incl;
    if (tid == 0) {
      s_diag[0] = INT_MAX;
      s_diag[1] = INT_MAX;
    }
    __syncthreads();
    int wpre = 0;
    for (int x = 0; x < wv; ++x) wpre += wsum[x];
    const int total = wsum[0] + wsum[1] + wsum[2] + wsum[3];
    const int excl = wpre + incl - loc;
    if (2 * tid < nent) {
      tbl_start[2 * tid] = beg2[0];
      tbl_pref[2 * tid] = excl;
    }
    if (2 * tid + 1 < nent) {
      tbl_start[2 * tid + 1] = beg2[1];
      tbl_pref[2 * tid + 1] = excl + len2[0];
    }
    if (diag_u >= 0) {
      const int gs = excl + (diag_u ? len2[0] : 0);
      s_diag[0] = gs;
      s_diag[1] = gs + len2[diag_u];
    }
    if (tid == 0) tbl_pref[nent] = total;
    __syncthreads();
    const int Gtot = total;
    const int Gd0 = s_diag[0];
    const int Gd1 = s_diag[1];

    int cur = 0;
    for (int p0 = 0; p0 < Gtot; p0 += kBlockN) {
      // ---- gather K/V rows of stream positions p0 + 4kg + u
      uint4 kr[4], vr[4];
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const int pos = p0 + key0 + u;
        if (pos < Gtot) {
          while (tbl_pref[cur + 1] <= pos) ++cur;
          const int s = tbl_start[cur] + (pos - tbl_pref[cur]);
          kr[u] = *reinterpret_cast<const uint4*>(kbase + (size_t)s * kv_rs + 8 * dc);
          vr[u] = *reinterpret_cast<const uint4*>(vbase + (size_t)s * kv_rs + 8 * dc);
        } else {
          kr[u] = make_uint4(0, 0, 0, 0);
          vr[u] = make_uint4(0, 0, 0, 0);
        }
      }
      __syncthreads();  // the previous sub-tile's LDS reads are done
#pragma unroll
      for (int u = 0; u < 4; ++u)
        *reinterpret_cast<uint4*>(&Ks[(key0 + u) * kKStride + 8 * dc]) = kr[u];
      {
        const uint32_t w0[4] = {vr[0].x, vr[0].y, vr[0].z, vr[0].w};
        const uint32_t w1[4] = {vr[1].x, vr[1].y, vr[1].z, vr[1].w};
        const uint32_t w2[4] = {vr[2].x, vr[2].y, vr[2].z, vr[2].w};
        const uint32_t w3[4] = {vr[3].x, vr[3].y, vr[3].z, vr[3].w};
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          // dims 2e (low halves) and 2e+1 (high halves) of keys key0..key0+3
          const uint32_t lo01 = (w0[e] & 0xffffu) | (w1[e] << 16);
          const uint32_t lo23 = (w2[e] & 0xffffu) | (w3[e] << 16);
          const uint32_t hi01 = (w0[e] >> 16) | (w1[e] & 0xffff0000u);
          const uint32_t hi23 = (w2[e] >> 16) | (w3[e] & 0xffff0000u);
          *reinterpret_cast<uint2*>(&Vt[(8 * dc + 2 * e) * kVStride + vpos0]) = make_uint2(lo01, lo23);
          *reinterpret_cast<uint2*>(&Vt[(8 * dc + 2 * e + 1) * kVStride + vpos0]) = make_uint2(hi01, hi23);
        }
      }
      __syncthreads();

      // a wave skips a sub-tile that lies inside the diagonal chunk beyond
      // all of its query rows
      const bool skip = (p0 >= Gd0) && (p0 + kBlockN <= Gd1) && (p0 - Gd0 > q0 + wv * 32 + 31);
      if (wave_active && !skip) {
        f32x16 sacc[2];
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
          for (int rr = 0; rr < 16; ++rr) sacc[kb][rr] = 0.f;
#pragma unroll
        for (int ds = 0; ds < 8; ++ds) {
#pragma unroll
          for (int kb = 0; kb < 2; ++kb) {
            const bf16x8_t a =
                *reinterpret_cast<const bf16x8_t*>(&Ks[(kb * 32 + l32) * kKStride + ds * 16 + hl * 8]);
            sacc[kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, qf[ds], sacc[kb], 0, 0, 0);
          }
        }
        // scale, mask, running max (accumulator: lane -> query, register rr
        // -> key 8*(rr/4) + 4*(lane/32) + rr%4 of the 32-key block)
        const bool need_mask = (p0 + kBlockN > Gtot) || (p0 + kBlockN > Gd0 && p0 < Gd1);
        float mx = -INFINITY;
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) {
#pragma unroll
          for (int rr = 0; rr < 16; ++rr) {
            float sv = sacc[kb][rr] * p.scale_log2;
            if (need_mask) {
              const int pos = p0 + kb * 32 + 8 * (rr >> 2) + 4 * hl + (rr & 3);
              const bool vis = pos < Gtot && (pos < Gd0 || pos >= Gd1 || pos - Gd0 <= qrow);
              sv = vis ? sv : -INFINITY;
            }
            sacc[kb][rr] = sv;
            mx = fmaxf(mx, sv);
          }
        }
        mx = fmaxf(mx, __shfl_xor(mx, 32, 64));
        const float m_new = fmaxf(m_run, mx);
        const float m_use = m_new == -INFINITY ? 0.f : m_new;
        const float alpha = fast_exp2(m_run - m_use);
        m_run = m_new;
        float lsum = 0.f;
        bf16x8_t pk[2][2];
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) {
#pragma unroll
          for (int rr = 0; rr < 16; ++rr) {
            const float pv = fast_exp2(sacc[kb][rr] - m_use);
            lsum += pv;
            pk[kb][rr >> 3][rr & 7] = (__bf16)pv;
          }
        }
        l_run = l_run * alpha + lsum;
#pragma unroll
        for (int db = 0; db < 4; ++db)
#pragma unroll
          for (int rr = 0; rr < 16; ++rr) oacc[db][rr] *= alpha;
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) {
#pragma unroll
          for (int hh = 0; hh < 2; ++hh) {
#pragma unroll
            for (int db = 0; db < 4; ++db) {
              const bf16x8_t a = *reinterpret_cast<const bf16x8_t*>(
                  &Vt[(db * 32 + l32) * kVStride + kb * 32 + 16 * hh + 8 * hl]);
              oacc[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, pk[kb][hh], oacc[db], 0, 0, 0);
            }
          }
        }
      }
    }
  }

  // ---- epilogue: O^T accumulator: lane -> query, register rr of block db
  // -> dim db*32 + 8*(rr/4) + 4*(lane/32) + rr%4
  const float l_tot = l_run + __shfl_xor(l_run, 32, 64);
  const float inv = l_tot > 0.f ? 1.0f / l_tot : 0.f;
  if (qvalid) {
    const size_t t = (size_t)b * p.seq_len + o_i + qrow;
    uint16_t* op = p.o + (t * p.hq + h) * kHeadDim;
#pragma unroll
    for (int db = 0; db < 4; ++db) {
#pragma unroll
      for (int q4 = 0; q4 < 4; ++q4) {
        const int d = db * 32 + 8 * q4 + 4 * hl;
        const uint32_t a0 = f32_to_bf16_bits(oacc[db][4 * q4 + 0] * inv);
        const uint32_t a1 = f32_to_bf16_bits(oacc[db][4 * q4 + 1] * inv);
        const uint32_t a2 = f32_to_bf16_bits(oacc[db][4 * q4 + 2] * inv);
        const uint32_t a3 = f32_to_bf16_bits(oacc[db][4 * q4 + 3] * inv);
        *reinterpret_cast<uint2*>(op + d) = make_uint2(a0 | (a1 << 16), a2 | (a3 << 16));
      }
    }
    if (p.lse != nullptr && hl == 0) {
      p.lse[((size_t)b * p.hq + h) * p.seq_len + o_i + qrow] =
          l_tot > 0.f ? (m_run + __log2f(l_tot)) * 0.69314718055994531f : -INFINITY;
    }
  }
}

// One workgroup per sequence: expand chunk lengths into the query-tile list
// (b, chunk, first row) with a block-wide exclusive scan.
__global__ __launch_bounds__(256) void plan_tiles_kernel(const int32_t* __restrict__ offs,
                                                         SeqTable st, int4* __restrict__ tiles) {
  __shared__ int wsum[4];
  const int b = blockIdx.x;
  const int C = st.num_chunks[b];
  const int obase = st.cbase[b] + b;
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  int base = st.tbase[b];
  for (int c0 = 0; c0 < C; c0 += 256) {
    const int c = c0 + tid;
    const int nt = c < C ? (offs[obase + c + 1] - offs[obase + c] + kBlockM - 1) / kBlockM : 0;
    int incl = nt;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
      const int y = __shfl_up(incl, off, 64);
      if (lane >= off) incl += y;
    }
    if (lane == 63) wsum[wv] = incl;
    __syncthreads();
    int pre = 0;
    for (int x = 0; x < wv; ++x) pre += wsum[x];
    const int tot = wsum[0] + wsum[1] + wsum[2] + wsum[3];
    const int ex = base + pre + incl - nt;
    for (int t = 0; t < nt; ++t) tiles[ex + t] = make_int4(b, c, t * kBlockM, 0);
    base += tot;
    __syncthreads();
  }
}

}  // namespace

hipError_t launch_plan_tiles(const int32_t* offs_dev, const SeqTable& st, int4* tiles,
                             hipStream_t stream) {
  hipLaunchKernelGGL(plan_tiles_kernel, dim3(st.batch), dim3(256), 0, stream, offs_dev, st,
                     tiles);
  return hipGetLastError();
}

hipError_t launch_attention(const AttnParams& p, const SeqTable& st, hipStream_t stream) {
  const int64_t grid = (int64_t)p.num_tiles * p.hq;
  if (grid <= 0) return hipSuccess;
  hipLaunchKernelGGL(attn_fwd_kernel, dim3((unsigned)grid), dim3(256), 0, stream, p, st);
  return hipGetLastError();
}

}  // namespace dhsa
