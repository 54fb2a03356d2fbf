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
//  * a workgroup = NW waves = 32*NW query rows of ONE query chunk and ONE
//    query head; each wave owns 32 rows.  Chunks are cut into tiles of 256
//    rows (8 waves, one workgroup per CU) or 128 rows (4 waves, two per CU);
//    a chunk's remainder of at most 32 rows goes to a second launch of one
//    wave per workgroup with 32-key sub-tiles (four workgroups per CU);
//  * the kept chunks of the row are concatenated into one gathered key
//    stream (a prefix table in LDS maps stream positions to tokens), cut
//    into 64-key sub-tiles that may cross chunk boundaries, so short chunks
//    waste no MFMA work on padding;
//  * K and V sub-tiles go straight from global memory into LDS
//    (buffer_load_dwordx4 ... lds, 16 bytes per lane, no staging registers), double
//    buffered: the loads of sub-tile j+1 are in flight while sub-tile j is
//    computed, with one barrier per sub-tile.  Both tiles are row-major
//    [64 keys][128 dims] with the 16-byte chunks of each row XOR-swizzled so
//    that the MFMA operand reads hit distinct LDS banks;
//  * per sub-tile: S^T = K Q^T with v_mfma_f32_32x32x16_bf16 (K rows from LDS
//    as the A operand, Q held in registers as the B operand), so each lane
//    owns the scores of one query and the running max / sum live per lane;
//    P^T is rounded to bf16 in registers and feeds O^T += V^T P^T directly as
//    the B operand; the V^T operand is read with the LDS transpose read
//    (ds_read_b64_tr_b16) from the row-major V tile;
//  * the running max is updated lazily: the output is rescaled only when the
//    max grows by more than 2^8, which keeps every p <= 256 and leaves the
//    normalised result unchanged;
//  * only the diagonal chunk needs the token-causal test (every earlier
//    kept chunk lies entirely before the query chunk), and its key range is
//    cut at the tile's last query row;
//  * workgroups are renumbered in runs of 32 consecutive (KV head, query
//    tile, query head) items per XCD: a run keeps the query heads and tiles
//    of one query chunk on one L2, and the eight XCDs advance through the
//    list together, so they stream the K/V of the same KV head at a time.
#include <float.h>

#include "dhsa_internal.h"

namespace dhsa {
namespace {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4_t __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
#define DHSA_GLOBAL __attribute__((address_space(1)))
#define DHSA_LDS __attribute__((address_space(3)))

constexpr int kTileElems = kBlockN * kHeadDim;  // one K or V sub-tile (bf16)
constexpr int kTable = 512;                      // kept chunks per table window
constexpr int kNumXcd = 8;
constexpr float kLazyRescale = 8.0f;             // log2 of the largest p allowed

// blocks of kXcdRun consecutive work items stay on one XCD (its L2 sees the
// query heads and tiles of one query chunk together), and the XCDs advance
// through the work list side by side, so at any time they all stream the K/V
// of the same KV head (which then stays resident in the shared last-level
// cache)
constexpr int kXcdRun = 32;
__device__ __forceinline__ int xcd_interleave(int w, int W) {
  const int x = w % kNumXcd, k = w / kNumXcd;  // XCD and its k-th block
  const int full = W / (kNumXcd * kXcdRun);    // complete rounds of runs
  const int round = k / kXcdRun;
  if (round < full) return (round * kNumXcd + x) * kXcdRun + (k % kXcdRun);
  return w;  // the ragged last round keeps the dispatch order
}

__device__ __forceinline__ uint16_t f32_to_bf16_bits(float x) {
  return __builtin_bit_cast(uint16_t, (__bf16)x);
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// LDS tile layout: element (row, d) of a [64][128] bf16 tile sits at
//   row * 128 + 8 * (chunk ^ swz(row)) + d % 8,   chunk = d / 8,
// with swz_k(row) = row & 15 for K and swz_v(row) = (row & 3) << 2 for V.
// word 3 of a raw buffer descriptor (no swizzle, no index stride, 32-bit
// data format) for the buffer loads below
constexpr int kRsrcWord3 = 0x00020000;

__device__ __forceinline__ int swz_k(int row) { return row & 15; }
__device__ __forceinline__ int swz_v(int row) { return (row & 3) << 2; }

// Position -> token walk over the LDS prefix table (positions only grow).
struct Cursor {
  int cur, beg, pref, end;
};

__device__ __forceinline__ int cursor_token(Cursor& c, int pos, const int* tbl_start,
                                            const int* tbl_pref) {
  while (pos >= c.end) {
    ++c.cur;
    c.beg = tbl_start[c.cur];
    c.pref = tbl_pref[c.cur];
    c.end = tbl_pref[c.cur + 1];
  }
  return c.beg + (pos - c.pref);
}

// vmcnt(n) with the other counters left alone (gfx9 s_waitcnt encoding:
// vmcnt bits [3:0] and [15:14], expcnt [6:4], lgkmcnt [11:8])
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt");
  __builtin_amdgcn_s_waitcnt(0x0F70 | (N & 15) | ((N >> 4) << 14));
}

// PD: how many 16-dim steps ahead of its MFMA each K operand read is issued.
// Occupancy: the wide tiles run two waves per SIMD (8 waves of 256 registers
// per CU, or two 4-wave workgroups); the one-wave remainder kernel's 36.9 KB
// of LDS (two K and two V 32-key sub-tiles plus the table) fits four
// workgroups per CU, one wave per SIMD, so it is built for that occupancy.
// A single-buffered remainder kernel (17 KB, two waves per SIMD) was
// measured slower on the ragged layer: 9.46 against 8.98 ms.
template <int NW, int KB, int PD>
__global__ __launch_bounds__(64 * NW, NW == 1 ? 1 : 2) void attn_fwd_kernel(AttnParams p,
                                                                             SeqTable st) {
  constexpr int kBlockM = 32 * NW;               // query rows per workgroup
  constexpr int kBN = 32 * KB;                   // keys per sub-tile
  constexpr int kTileE = kBN * kHeadDim;         // one K or V sub-tile (bf16)
  constexpr int kRowsPerWave = kBN / NW;         // tile rows each wave loads
  constexpr int kLoadsPerMat = kRowsPerWave / 4; // 1 KB direct loads per wave per matrix
  constexpr int kEntPerThread = kTable / (64 * NW);
  static_assert(kLoadsPerMat >= 1 && kEntPerThread >= 1, "shape");
  // two K and two V buffers as distinct LDS objects; the sub-tile loop is
  // unrolled by two, so every access names its buffer statically and the
  // compiler can tell the in-flight direct loads into the other pair from
  // the reads of the current one (it does not wait for them)
  __shared__ __attribute__((aligned(16))) uint16_t K0[kTileE];
  __shared__ __attribute__((aligned(16))) uint16_t K1[kTileE];
  __shared__ __attribute__((aligned(16))) uint16_t V0[kTileE];
  __shared__ __attribute__((aligned(16))) uint16_t V1[kTileE];
  __shared__ int tbl_start[kTable];
  __shared__ int tbl_pref[kTable + 1];
  __shared__ int wsum[NW];
  __shared__ int s_diag[2];

  const int tid = threadIdx.x;
  const int wv = tid >> 6;
  const int lane = tid & 63;
  const int l32 = lane & 31;
  const int hl = lane >> 5;

  // ---- which (KV head, query tile, query head) this workgroup owns
  const int G = p.hq / p.hkv;
  const int W = p.num_tiles * p.hq;
  const int w = xcd_interleave((int)blockIdx.x, W);
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
  float m_run = -INFINITY;  // running max of scale*log2(e)*s, per query
  float l_run = 0.f;        // this lane's share of the running sum
  const float c2 = p.scale_log2;

  // K/V of KV head g: row t starts at byte t * rowbytes from these bases
  const uint32_t rowbytes = (uint32_t)p.hkv * kHeadDim * 2;
  const size_t kv_rs = (size_t)p.hkv * kHeadDim;
  const char* kbytes = reinterpret_cast<const char*>(p.k + (size_t)b * p.seq_len * kv_rs + (size_t)g * kHeadDim);
  const char* vbytes = reinterpret_cast<const char*>(p.v + (size_t)b * p.seq_len * kv_rs + (size_t)g * kHeadDim);
  // buffer descriptors over this sequence's rows (the host keeps
  // seq_len * rowbytes below 2^32).  The K/V tiles are staged with the
  // buffer form of the direct-to-LDS load: while a global-form one is in
  // flight the compiler can only wait for all LDS reads at once, which would
  // serialise every K operand read below with its MFMA
  const uint32_t nrec = (uint32_t)p.seq_len * rowbytes;
  const __amdgpu_buffer_rsrc_t krsrc =
      __builtin_amdgcn_make_buffer_rsrc(const_cast<char*>(kbytes), 0, (int)nrec, kRsrcWord3);
  const __amdgpu_buffer_rsrc_t vrsrc =
      __builtin_amdgcn_make_buffer_rsrc(const_cast<char*>(vbytes), 0, (int)nrec, kRsrcWord3);

  // loader role: direct load u of wave wv fills tile rows
  // kRowsPerWave*wv + 4*u + lane/16, lane & 15 being the physical 16-byte
  // chunk; lane & (kRowsPerWave-1) walks the token of stream row
  // kRowsPerWave*wv + that and hands it to the lanes that load the row
  const int lsub = lane & 15;
  const int lgrp = lane >> 4;
  const int lwalk = lane & (kRowsPerWave - 1);
  uint32_t kchunk[kLoadsPerMat];
#pragma unroll
  for (int u = 0; u < kLoadsPerMat; ++u)
    kchunk[u] = 16u * (uint32_t)(lsub ^ swz_k(kRowsPerWave * wv + 4 * u + lgrp));
  const uint32_t vchunk = 16u * (uint32_t)(lsub ^ swz_v(lgrp));

  // V^T operand reads: lane 16*G + s of transpose read a covers 4 dims of key
  //   kb*32 + 16*hh + 8*a + 4*(G/2) + s/4, dims db*32 + 16*(G%2) + 4*(s%4)
  const int vkey_off = 4 * (lgrp >> 1) + (lsub >> 2);
  const int vd_off = 16 * (lgrp & 1) + 4 * (lsub & 3);
  const int qmin = q0 + wv * 32;  // first query row (chunk-local) of this wave
  constexpr int kNoDiag = 0x3fffffff;

  bf16x2_t pp[KB][8];  // P^T of the current sub-tile, bf16 pairs
  // ---- O^T += V^T P^T over the sub-tile whose V sits in Vs
  auto pv = [&](const uint16_t* Vs) {
#pragma unroll
    for (int kb = 0; kb < KB; ++kb) {
#pragma unroll
      for (int hh = 0; hh < 2; ++hh) {
        const bf16x8_t pk = __builtin_shufflevector(
            __builtin_shufflevector(pp[kb][4 * hh], pp[kb][4 * hh + 1], 0, 1, 2, 3),
            __builtin_shufflevector(pp[kb][4 * hh + 2], pp[kb][4 * hh + 3], 0, 1, 2, 3),
            0, 1, 2, 3, 4, 5, 6, 7);
#pragma unroll
        for (int db = 0; db < 4; ++db) {
          bf16x4_t part[2];
#pragma unroll
          for (int a = 0; a < 2; ++a) {
            const int key = kb * 32 + 16 * hh + 8 * a + vkey_off;
            const int d = db * 32 + vd_off;
            const int idx = key * kHeadDim + 8 * ((d >> 3) ^ swz_v(key)) + (d & 7);
            part[a] = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((DHSA_LDS bf16x4_t*)(&Vs[idx]));
          }
          const bf16x8_t va = __builtin_shufflevector(part[0], part[1], 0, 1, 2, 3, 4, 5, 6, 7);
          oacc[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(va, pk, oacc[db], 0, 0, 0);
        }
      }
    }
  };

  for (int64_t wb = e0; wb < e1; wb += kTable) {
    const int nent = (int)((e1 - wb) < kTable ? (e1 - wb) : kTable);
    __syncthreads();  // the previous window's table and tiles are no longer read
    int lenv[kEntPerThread], begv[kEntPerThread];
    int diag_u = -1;
    int loc = 0;
#pragma unroll
    for (int u = 0; u < kEntPerThread; ++u) {
      const int idx = kEntPerThread * tid + u;
      lenv[u] = 0;
      begv[u] = 0;
      if (idx < nent) {
        const int j = p.col_idx[wb + idx];
        if (j >= 0 && j <= i) {
          begv[u] = p.offs[obase + j];
          lenv[u] = p.offs[obase + j + 1] - begv[u];
          if (j == i) {
            lenv[u] = min(lenv[u], q0 + rows);
            diag_u = u;
          }
        }
      }
      loc += lenv[u];
    }
    int incl = loc;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
      const int y = __shfl_up(incl, off, 64);
      if (lane >= off) incl += y;
    }
    if (lane == 63) wsum[wv] = incl;
    if (tid == 0) {
      s_diag[0] = kNoDiag;
      s_diag[1] = kNoDiag;
    }
    __syncthreads();
    int wpre = 0, total = 0;
#pragma unroll
    for (int x = 0; x < NW; ++x) {
      wpre += x < wv ? wsum[x] : 0;
      total += wsum[x];
    }
    int run = wpre + incl - loc;
#pragma unroll
    for (int u = 0; u < kEntPerThread; ++u) {
      const int idx = kEntPerThread * tid + u;
      if (idx < nent) {
        tbl_start[idx] = begv[u];
        tbl_pref[idx] = run;
      }
      if (u == diag_u) {
        s_diag[0] = run;
        s_diag[1] = run + lenv[u];
      }
      run += lenv[u];
    }
    if (tid == 0) tbl_pref[nent] = total;
    __syncthreads();
    const int Gtot = total;
    const int Gd0 = s_diag[0];
    const int Gd1 = s_diag[1];
    if (Gtot == 0) continue;
    const int nsub = (Gtot + kBN - 1) / kBN;
    // stream positions past Gtot (the last sub-tile's padding) load the
    // first token of the stream: it lies in the row's first non-empty kept
    // chunk, an earlier chunk or the diagonal chunk's first token, so every
    // query row of the tile sees it, and a non-finite value there reaches
    // no row that could not see it anyway (the padding's weight is exactly
    // 0, and 0 * inf would otherwise leak NaN into rows that never see the
    // loaded key)
    int tok_pad;
    {
      Cursor c0{-1, 0, 0, 0};
      tok_pad = cursor_token(c0, 0, tbl_start, tbl_pref);
    }

    Cursor cur{-1, 0, 0, 0};
    // direct-to-LDS loads of sub-tile js into (Kd, Vd)
    auto issue = [&](int js, uint16_t* Kd, uint16_t* Vd) {
      const int pos = js * kBN + kRowsPerWave * wv + lwalk;
      const int tok = pos < Gtot ? cursor_token(cur, pos, tbl_start, tbl_pref) : tok_pad;
#pragma unroll
      for (int u = 0; u < kLoadsPerMat; ++u) {
        const uint32_t tk = (uint32_t)__shfl(tok, 4 * u + lgrp, 64);
        const uint32_t rb = tk * rowbytes;
        uint16_t* kd = Kd + (kRowsPerWave * wv + 4 * u) * kHeadDim;
        uint16_t* vd = Vd + (kRowsPerWave * wv + 4 * u) * kHeadDim;
        __builtin_amdgcn_raw_ptr_buffer_load_lds(krsrc, (DHSA_LDS void*)kd, 16, (int)(rb + kchunk[u]),
                                                 0, 0, 0);
        __builtin_amdgcn_raw_ptr_buffer_load_lds(vrsrc, (DHSA_LDS void*)vd, 16, (int)(rb + vchunk), 0,
                                                 0, 0);
      }
    };

    // one sub-tile js: compute on (Kt, Vt) while sub-tile js+1 streams into
    // (Kn, Vn), the buffers of sub-tile js-1
    auto subtile = [&](int js, const uint16_t* Kt, const uint16_t* Vt, uint16_t* Kn, uint16_t* Vn) {
      const int p0 = js * kBN;
      if (js + 1 < nsub) issue(js + 1, Kn, Vn);
      // a wave skips a sub-tile that lies inside the diagonal chunk beyond
      // all of its query rows
      const bool skip = (p0 >= Gd0) && (p0 + kBN <= Gd1 || Gd1 >= Gtot) &&
                        (p0 - Gd0 > qmin + 31);
      if (wave_active && !skip) {
        // ---- S^T = K Q^T, K operand reads one step ahead of the MFMAs
        f32x16 sacc[KB];
#pragma unroll
        for (int kb = 0; kb < KB; ++kb)
#pragma unroll
          for (int rr = 0; rr < 16; ++rr) sacc[kb][rr] = 0.f;
        // operand ring: step ds lives in slot ds % PD, read PD steps ahead
        bf16x8_t kr[PD][KB];
        auto ld = [&](int ds, int slot) {
#pragma unroll
          for (int kb = 0; kb < KB; ++kb) {
            const int row = kb * 32 + l32;
            kr[slot][kb] = *reinterpret_cast<const bf16x8_t*>(
                &Kt[row * kHeadDim + 8 * ((2 * ds + hl) ^ swz_k(row))]);
          }
        };
#pragma unroll
        for (int ds = 0; ds < PD; ++ds) ld(ds, ds);
#pragma unroll
        for (int ds = 0; ds < 8; ++ds) {
          const int slot = ds % PD;
          // keep the ring as written: the scheduler would otherwise pull each
          // read down to just before its MFMA
          if (PD > 2) __builtin_amdgcn_sched_barrier(0);
#pragma unroll
          for (int kb = 0; kb < KB; ++kb)
            sacc[kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kr[slot][kb], qf[ds], sacc[kb], 0, 0,
                                                               0);
          if (ds + PD < 8) ld(ds + PD, slot);
        }
        if (PD > 2) __builtin_amdgcn_sched_barrier(0);

        // ---- mask: only the tail of the stream and the part of the diagonal
        // chunk past this wave's first query row can hold hidden keys
        // (accumulator: lane -> query, register rr -> key
        //  8*(rr/4) + 4*(lane/32) + rr%4 of the 32-key block)
        const bool need_mask =
            (p0 + kBN > Gtot) || (p0 + kBN > Gd0 + qmin + 1 && p0 < Gd1);
        if (need_mask) {
          const int rel_tot = Gtot - p0;
          const int rel_lo = Gd0 + qrow - p0;
          const int rel_hi = Gd1 - p0;
#pragma unroll
          for (int kb = 0; kb < KB; ++kb) {
#pragma unroll
            for (int rr = 0; rr < 16; ++rr) {
              const int rel = kb * 32 + 8 * (rr >> 2) + 4 * hl + (rr & 3);
              const bool hidden = (rel >= rel_tot) | ((rel > rel_lo) & (rel < rel_hi));
              sacc[kb][rr] = hidden ? -INFINITY : sacc[kb][rr];
            }
          }
        }
        float mx = -INFINITY;
#pragma unroll
        for (int kb = 0; kb < KB; ++kb)
#pragma unroll
          for (int rr = 0; rr < 16; ++rr) mx = fmaxf(mx, sacc[kb][rr]);
        mx = fmaxf(mx, __shfl_xor(mx, 32, 64));
        const float mxs = mx * c2;
        const bool upd = mxs > m_run + kLazyRescale;
        if (__ballot(upd)) {
          const float alpha = upd ? fast_exp2(m_run - mxs) : 1.0f;
          m_run = upd ? mxs : m_run;
          l_run *= alpha;
#pragma unroll
          for (int db = 0; db < 4; ++db)
#pragma unroll
            for (int rr = 0; rr < 16; ++rr) oacc[db][rr] *= alpha;
        }
        // ---- P^T = exp2(c2 * s - m) in bf16; the row sum adds the rounded
        // values (the weights the PV product actually uses) two at a time
        const float mneg = m_run == -INFINITY ? 0.f : -m_run;
        const bf16x2_t ones = {(__bf16)1.0f, (__bf16)1.0f};
#pragma unroll
        for (int kb = 0; kb < KB; ++kb) {
#pragma unroll
          for (int e = 0; e < 8; ++e) {
            const float p0v = fast_exp2(__builtin_fmaf(sacc[kb][2 * e], c2, mneg));
            const float p1v = fast_exp2(__builtin_fmaf(sacc[kb][2 * e + 1], c2, mneg));
            pp[kb][e] = bf16x2_t{(__bf16)p0v, (__bf16)p1v};
            l_run = __builtin_amdgcn_fdot2_f32_bf16(pp[kb][e], ones, l_run, false);
          }
        }
        pv(Vt);
      }
      wait_vmcnt<0>();  // this wave's loads of sub-tile js+1 have landed
      __syncthreads();
    };

    issue(0, K0, V0);
    wait_vmcnt<0>();
    __syncthreads();
    for (int js = 0; js < nsub; js += 2) {
      subtile(js, K0, V0, K1, V1);
      if (js + 1 < nsub) subtile(js + 1, K1, V1, K0, V0);
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

// One workgroup per sequence: expand chunk lengths into the query-tile lists
// with block-wide exclusive scans.  A chunk gives floor(n / block_m) full
// tiles of block_m rows; a remainder of more than kNarrowRows rows gives one
// more tile of that list, a remainder of 1..kNarrowRows rows one tile of the
// narrow list (32 rows, one wave).  Entries: (sequence, chunk, first row).
__global__ __launch_bounds__(256) void plan_tiles_kernel(const int32_t* __restrict__ offs,
                                                         SeqTable st, int4* __restrict__ tiles,
                                                         int4* __restrict__ narrow,
                                                         int32_t block_m) {
  __shared__ int wsum[2][4];
  const int b = blockIdx.x;
  const int C = st.num_chunks[b];
  const int obase = st.cbase[b] + b;
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  int base = st.tbase[b], nbase = st.ntbase[b];
  for (int c0 = 0; c0 < C; c0 += 256) {
    const int c = c0 + tid;
    const int n = c < C ? offs[obase + c + 1] - offs[obase + c] : 0;
    const int full = n / block_m, rem = n - full * block_m;
    const int nt = full + (rem > kNarrowRows ? 1 : 0);
    const int nn = (rem > 0 && rem <= kNarrowRows) ? 1 : 0;
    int incl = nt, incn = nn;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
      const int y = __shfl_up(incl, off, 64);
      const int z = __shfl_up(incn, off, 64);
      if (lane >= off) {
        incl += y;
        incn += z;
      }
    }
    if (lane == 63) {
      wsum[0][wv] = incl;
      wsum[1][wv] = incn;
    }
    __syncthreads();
    int pre = 0, pren = 0;
    for (int x = 0; x < wv; ++x) {
      pre += wsum[0][x];
      pren += wsum[1][x];
    }
    const int tot = wsum[0][0] + wsum[0][1] + wsum[0][2] + wsum[0][3];
    const int totn = wsum[1][0] + wsum[1][1] + wsum[1][2] + wsum[1][3];
    const int ex = base + pre + incl - nt;
    for (int t = 0; t < nt; ++t) tiles[ex + t] = make_int4(b, c, t * block_m, 0);
    if (nn) narrow[nbase + pren + incn - nn] = make_int4(b, c, full * block_m, 0);
    base += tot;
    nbase += totn;
    __syncthreads();
  }
}

}  // namespace

hipError_t launch_plan_tiles(const int32_t* offs_dev, const SeqTable& st, int4* tiles,
                             int4* narrow, int32_t block_m, hipStream_t stream) {
  hipLaunchKernelGGL(plan_tiles_kernel, dim3(st.batch), dim3(256), 0, stream, offs_dev, st,
                     tiles, narrow, block_m);
  return hipGetLastError();
}

hipError_t launch_attention(const AttnParams& p, const SeqTable& st, hipStream_t stream) {
  const int64_t grid = (int64_t)p.num_tiles * p.hq;
  if (grid > 0) {
    if (p.block_m == kBlockMLarge) {
      hipLaunchKernelGGL((attn_fwd_kernel<8, 2, 3>), dim3((unsigned)grid), dim3(512), 0, stream, p,
                         st);
    } else {
      hipLaunchKernelGGL((attn_fwd_kernel<4, 2, 3>), dim3((unsigned)grid), dim3(256), 0,
                         stream, p, st);
    }
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  // remainders of at most 32 rows: one wave per workgroup, 32-key sub-tiles
  // (36 KB of LDS, so four such workgroups share a CU)
  const int64_t ngrid = (int64_t)p.num_narrow * p.hq;
  if (ngrid > 0) {
    AttnParams q = p;
    q.tiles = p.narrow;
    q.num_tiles = p.num_narrow;
    hipLaunchKernelGGL((attn_fwd_kernel<1, 1, 2>), dim3((unsigned)ngrid), dim3(64), 0,
                       stream, q, st);
    return hipGetLastError();
  }
  return hipSuccess;
}

}  // namespace dhsa
