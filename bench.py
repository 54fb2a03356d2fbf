#!/usr/bin/env python3
"""Benchmark of the DHSA sparse prefill path on one MI355X.

One step = one attention layer's whole hot path on the Llama-3.1-8B layer
shape at 128K context: dhsa_build_mask (pool + chunk scores + causal top-k)
then dhsa_sparse_prefill (block-sparse causal attention), inputs resident in
HBM.  Prints ONE JSON line:
  value        kept-tile TFLOP/s over the whole layer (mask + attention)
  ms_per_step  ms per layer
  roofline     the attention kernel against the bf16 MFMA peak
  mask_stages  pooling, chunk scores and top-k timed one by one (stage calls),
               with the HBM GB/s of pooling and top-k
  layers       the other layer shapes (Qwen2.5-3B at 16K, Llama-3.1-8B at
               32K) and the same 128K layer with every causal chunk kept
               (dense causal, the sparse-vs-dense context), each as ms per
               layer, kept-tile TFLOP/s and mask GB/s against the roofline
  cpu_baseline the CPU oracle on a bounded sample of the same layer
Latencies are also given as the median of 5 timed runs after 2 warmups (the
DHSA README's kernel-latency protocol) next to the mean over --steps runs.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import statistics
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2500.0   # MI355X dense bf16 MFMA
PEAK_HBM_GBPS = 8000.0      # MI355X HBM3E
ATTN_SOURCES = ["long_context_prefill_segmented_amd/csrc/attn.hip"]
PMC_FILE = os.path.join(ROOT, "profiles", "attn_fwd_llama31_8b_128k_pmc.json")


def log(msg):
    print(msg, file=sys.stderr, flush=True)


def kept_tile_flops(offsets, row_ptr, col_idx, hq, d=128):
    """Algorithmic FLOPs of the kept tiles: 4*d per visible (query, key) pair;
    the diagonal chunk counts its causal half n(n+1)/2."""
    total = 0
    r = 0
    for o in offsets:
        n = np.diff(np.asarray(o, dtype=np.int64))
        C = n.size
        for _h in range(hq):
            for i in range(C):
                cols = col_idx[row_ptr[r]:row_ptr[r + 1]]
                r += 1
                off = cols[cols < i]
                total += int(n[i]) * int(n[off].sum())
                if np.any(cols == i):
                    total += int(n[i]) * (int(n[i]) + 1) // 2
    return 4 * d * total


def source_hash(paths):
    h = hashlib.sha256()
    for p in paths:
        with open(os.path.join(ROOT, p), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def host_cpu_model() -> str:
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:  # pragma: no cover
        pass
    return "unknown"


def cpu_baseline(x, hq, hkv, budget_rows=1500, seed=0):
    """The oracle, untuned, on a bounded sample of the layer: full-layer mask
    construction plus attention for a seeded sample of (head, query chunk)
    rows, scaled to kept-tile TFLOP/s.  Runs on every core this process may
    use (its CPU affinity set), with the BLAS thread pools pinned to that
    count."""
    from oracle import dhsa_oracle as orc
    cores = len(os.sched_getaffinity(0))
    try:
        from threadpoolctl import threadpool_info, threadpool_limits
        limiter = threadpool_limits(limits=cores)
    except Exception:  # pragma: no cover
        threadpool_info, limiter = None, None
    try:
        blas = sorted({i.get("num_threads", 1) for i in threadpool_info()}) if threadpool_info \
            else []
        b = 0
        t0 = time.perf_counter()
        q = orc.widen_bf16(x.q[b])
        k = orc.widen_bf16(x.k[b])
        _, _, _, _, rows = orc.build_mask(q, k, x.offsets[b], x.topk)
        t_mask = time.perf_counter() - t0
        v = orc.widen_bf16(x.v[b])
        rng = np.random.default_rng(seed)
        o = np.asarray(x.offsets[b], dtype=np.int64)
        C = o.size - 1
        n = np.diff(o)
        G = hq // hkv
        picks = [(int(rng.integers(0, hq)), int(rng.integers(0, C))) for _ in range(budget_rows)]
        flops = 0
        t1 = time.perf_counter()
        for (h, i) in picks:
            orc.chunk_attention(q, k, v, o, rows[h][i], i, h, h // G, 1.0 / math.sqrt(128))
            cols = np.asarray(rows[h][i])
            flops += 4 * 128 * (int(n[i]) * int(n[cols[cols < i]].sum())
                                + int(n[i]) * (int(n[i]) + 1) // 2)
        t_att = time.perf_counter() - t1
    finally:
        if limiter is not None:
            limiter.restore_original_limits()
    rows_total = hq * C * x.workload.batch
    frac = budget_rows / rows_total
    t_layer_share = t_att + t_mask * frac
    return {
        "value": flops / t_layer_share / 1e12,
        "unit": "TFLOP/s (kept tiles)",
        "cores": int(cores),
        "kind": "oracle",
        "cpu_model": host_cpu_model(),
        "blas_threads": blas,
        "sample": (f"oracle (NumPy float64) mask construction of the whole layer ({t_mask:.1f} s, "
                   f"prorated by {frac:.2e}) + attention of {budget_rows} seeded (head, query "
                   f"chunk) rows ({t_att:.1f} s, {flops / 1e9:.1f} GFLOP kept); cores = the "
                   f"process's CPU affinity set, BLAS pools limited to it"),
    }


def mask_bytes_of(w, hq, hkv, rp_size, nnz):
    """Algorithmic bytes of mask construction: Q and K read once, the CSR
    written once (pooled vectors and scores stay in the L2-sized workspace
    and are not counted)."""
    return 2 * w.batch * w.seq_len * (hq + hkv) * 128 + 4 * (rp_size + nnz)


def timed_runs(torch, stream, fns, steps):
    """Runs the callables in order `steps` times, with HIP events recorded on
    `stream` around each; returns per-callable lists of ms."""
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(len(fns) + 1)]
          for _ in range(steps)]
    for s in range(steps):
        ev[s][0].record(stream)
        for j, f in enumerate(fns):
            f()
            ev[s][j + 1].record(stream)
    torch.cuda.synchronize()
    return [[ev[s][j].elapsed_time(ev[s][j + 1]) for s in range(steps)]
            for j in range(len(fns))]


def pages_protocol(torch, stream, fns, warmup=2, timed=5):
    """The DHSA README's kernel-latency protocol: `warmup` untimed runs, then
    the median of `timed` runs (per callable, ms)."""
    for _ in range(warmup):
        for f in fns:
            f()
    torch.cuda.synchronize()
    return [statistics.median(t) for t in timed_runs(torch, stream, fns, timed)]


def time_layer(dhsa, synth, torch, dev, name, steps, topk=None, label=None, x=None):
    """One whole layer (mask + attention) of workload `name`, inputs resident:
    mean over `steps` runs and the median of 5 after 2 warmups.  topk
    overrides the workload's (topk >= the chunk count keeps every causal
    chunk: dense causal attention through the same kernels)."""
    w = synth.WORKLOADS[name]
    if x is None:
        x = synth.generate(w)
    hq, hkv = w.num_q_heads, w.num_kv_heads
    k_used = x.topk if topk is None else topk
    offs = dhsa.ChunkOffsets.from_list(x.offsets, w.seq_len, device=dev)
    q, k, v = (dhsa.bf16_from_bits(a, dev) for a in (x.q, x.k, x.v))
    mb = dhsa.MaskBuilder(offs, hq, hkv, k_used, device=dev)
    pf = dhsa.Prefill(offs, hq, hkv, device=dev)
    stream = torch.cuda.current_stream()
    state = {}

    def mask():
        state["csr"] = mb(q, k)

    def attn():
        pf(q, k, v, state["csr"])

    p_mask, p_attn = pages_protocol(torch, stream, [mask, attn])
    rp = state["csr"].row_ptr.cpu().numpy()
    ci = state["csr"].col_idx.cpu().numpy()[:state["csr"].nnz]
    flops = kept_tile_flops(x.offsets, rp, ci, hq)
    t_mask, t_attn = timed_runs(torch, stream, [mask, attn], steps)
    m_avg, a_avg = statistics.mean(t_mask), statistics.mean(t_attn)
    mbytes = mask_bytes_of(w, hq, hkv, rp.size, ci.size)
    res = {
        "workload": label or name, "batch": w.batch, "seq_len": w.seq_len,
        "num_q_heads": hq, "num_kv_heads": hkv, "topk": k_used,
        "num_chunks": [len(o) - 1 for o in x.offsets], "nnz": int(ci.size),
        "chunk_pair_density": float(ci.size / (hq * sum((len(o) - 1) * len(o) // 2
                                                          for o in x.offsets))),
        "steps": steps, "ms_per_layer": m_avg + a_avg, "mask_ms": m_avg, "attention_ms": a_avg,
        "ms_per_layer_median5": p_mask + p_attn, "mask_ms_median5": p_mask,
        "attention_ms_median5": p_attn,
        "kept_tile_TFLOP": flops / 1e12,
        "TFLOP_per_s": flops / ((m_avg + a_avg) * 1e-3) / 1e12,
        "attention_TFLOP_per_s": flops / (a_avg * 1e-3) / 1e12,
        "attention_frac_of_peak": flops / (a_avg * 1e-3) / 1e12 / PEAK_BF16_TFLOPS,
        "mask_GBps": mbytes / (m_avg * 1e-3) / 1e9,
        "mask_frac_of_hbm": mbytes / (m_avg * 1e-3) / 1e9 / PEAK_HBM_GBPS,
    }
    log(f"[bench] layer {res['workload']}: mask {m_avg:.3f} ms  attention {a_avg:.3f} ms  "
        f"({res['attention_TFLOP_per_s']:.0f} TFLOP/s, mask {res['mask_GBps']:.0f} GB/s)")
    del q, k, v, mb, pf, state
    torch.cuda.empty_cache()
    return res


def time_mask_stages(dhsa, torch, x, offs, q, k, hq, hkv, steps):
    """The mask's steps one at a time through the stage calls, into
    preallocated buffers: pooling of Q and of K (dhsa_pool), chunk scores
    (dhsa_chunk_scores), causal top-k to CSR (dhsa_topk_csr).  GB/s are
    algorithmic bytes: pooling reads the tensor once and writes the pooled
    fp32 rows; top-k reads the causal half of the fp32 scores and writes the
    CSR."""
    w = x.workload
    tc = int(offs.num_chunks.sum())
    qbar = torch.empty((hq * tc, 128), dtype=torch.float32, device=q.device)
    kbar = torch.empty((hkv * tc, 128), dtype=torch.float32, device=q.device)
    sc = torch.zeros(dhsa.scores_numel(offs, hq), dtype=torch.float32, device=q.device)
    R, nnz = dhsa.csr_size(offs, hq, x.topk)
    csr = dhsa.CSR(torch.empty(R + 1, dtype=torch.int32, device=q.device),
                   torch.empty(max(nnz, 1), dtype=torch.int32, device=q.device), nnz)
    fns = [lambda: dhsa.pool(q, offs, out=qbar), lambda: dhsa.pool(k, offs, out=kbar),
           lambda: dhsa.chunk_scores(qbar, kbar, offs, hq, hkv, out=sc),
           lambda: dhsa.topk_csr(sc, offs, hq, x.topk, out=csr)]
    stream = torch.cuda.current_stream()
    for f in fns:
        f()
    torch.cuda.synchronize()
    t = [statistics.mean(ts) for ts in timed_runs(torch, stream, fns, steps)]
    L = w.batch * w.seq_len
    bq = 2 * L * hq * 128 + 4 * hq * tc * 128
    bk = 2 * L * hkv * 128 + 4 * hkv * tc * 128
    causal = sum(hq * c * (c + 1) // 2 for c in offs.num_chunks.tolist())
    btop = 4 * causal + 4 * (R + 1 + nnz)
    res = {"steps": steps,
           "pool_q_ms": t[0], "pool_q_GBps": bq / (t[0] * 1e-3) / 1e9,
           "pool_k_ms": t[1], "pool_k_GBps": bk / (t[1] * 1e-3) / 1e9,
           "pool_GBps": (bq + bk) / ((t[0] + t[1]) * 1e-3) / 1e9,
           "pool_frac_of_hbm": (bq + bk) / ((t[0] + t[1]) * 1e-3) / 1e9 / PEAK_HBM_GBPS,
           "scores_ms": t[2],
           "scores_GFLOP_per_s": 2 * 128 * causal / (t[2] * 1e-3) / 1e9,
           "topk_ms": t[3], "topk_GBps": btop / (t[3] * 1e-3) / 1e9,
           "topk_frac_of_hbm": btop / (t[3] * 1e-3) / 1e9 / PEAK_HBM_GBPS,
           "how": "stage calls into preallocated buffers, HIP events around each; pooling "
                  "counts the bf16 tensor read once and the fp32 pooled rows written; top-k "
                  "counts the causal half of the fp32 scores read and the CSR written"}
    log(f"[bench] mask stages: pool Q {t[0] * 1e3:.1f} us + K {t[1] * 1e3:.1f} us "
        f"({res['pool_GBps']:.0f} GB/s), scores {t[2] * 1e3:.1f} us, top-k {t[3] * 1e3:.1f} us "
        f"({res['topk_GBps']:.0f} GB/s)")
    return res


def time_variant(dhsa, synth, torch, x, offs, q, k, v, pf, hq, hkv, recent, steps, dev):
    """The same layer with the widened selection rule: synthetic per-row
    budgets (uniform in [1, 2 topk - 1], mean topk) capped at 2 topk - 1,
    plus a window of `recent` chunks before the diagonal
    (dhsa_build_mask_ex: device prefix sum for row_ptr)."""
    cap = 2 * x.topk - 1
    bud = torch.from_numpy(synth.row_budgets(offs.num_chunks, hq, x.topk, seed=x.workload.seed)
                           ).to(dev)
    mb = dhsa.MaskBuilder(offs, hq, hkv, cap, device=dev, recent=recent)
    stream = torch.cuda.current_stream()
    for _ in range(2):
        pf(q, k, v, mb(q, k, row_budgets=bud))
    torch.cuda.synchronize()
    csr = mb(q, k, row_budgets=bud)
    torch.cuda.synchronize()
    rp = csr.row_ptr.cpu().numpy()
    ci = csr.col_idx.cpu().numpy()[:int(rp[-1])]
    flops = kept_tile_flops(x.offsets, rp, ci, hq)
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(steps)]
    for s in range(steps):
        ev[s][0].record(stream)
        csr = mb(q, k, row_budgets=bud)
        ev[s][1].record(stream)
        pf(q, k, v, csr)
        ev[s][2].record(stream)
    torch.cuda.synchronize()
    mask_avg = statistics.mean(a.elapsed_time(b) for a, b, _ in ev)
    attn_avg = statistics.mean(b.elapsed_time(c) for _, b, c in ev)
    log(f"[bench] variant budgets+recent{recent}: mask {mask_avg:.3f} ms  attention "
        f"{attn_avg:.3f} ms")
    mask_bytes = 2 * x.q.shape[0] * x.q.shape[1] * (hq + hkv) * 128 + 4 * (rp.size + ci.size) \
        + 4 * int(bud.numel())
    return {"selection": f"per-row budgets in [1, {cap}] (mean {x.topk}), recent {recent}",
            "steps": steps, "nnz": int(ci.size), "mask_ms": mask_avg, "attention_ms": attn_avg,
            "kept_tile_TFLOP": flops / 1e12,
            "TFLOP_per_s": flops / ((mask_avg + attn_avg) * 1e-3) / 1e12,
            "attention_TFLOP_per_s": flops / (attn_avg * 1e-3) / 1e12,
            "mask_GBps": mask_bytes / (mask_avg * 1e-3) / 1e9}


def time_nms(dhsa, synth, torch, x, dev, min_gap=32, threshold=0.5, steps=20):
    """Boundary finalisation on synthetic predictor scores for the same
    sequences (peaks at the layer's chunk starts, shoulders, spurious
    spikes): dhsa_nms_boundaries, one workgroup per sequence."""
    w = x.workload
    p = torch.from_numpy(synth.boundary_scores(x.offsets, w.seq_len, seed=w.seed)).to(dev)
    nms = dhsa.BoundaryNMS(w.batch, w.seq_len, min_gap, threshold, device=dev)
    stream = torch.cuda.current_stream()
    for _ in range(2):
        nms(p)
    torch.cuda.synchronize()
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(2)] for _ in range(steps)]
    for s in range(steps):
        ev[s][0].record(stream)
        nms(p)
        ev[s][1].record(stream)
    torch.cuda.synchronize()
    ms = statistics.mean(a.elapsed_time(b) for a, b in ev)
    nc = [int(c) for c in nms.num_chunks.cpu().numpy()]
    log(f"[bench] boundary NMS: {ms * 1e3:.1f} us  chunks {nc}")
    nbytes = 4 * w.batch * w.seq_len + 4 * sum(c + 1 for c in nc)
    return {"min_gap": min_gap, "threshold": threshold, "steps": steps, "ms": ms,
            "num_chunks": nc, "GBps": nbytes / (ms * 1e-3) / 1e9}


def time_batched_loop(dhsa, synth, torch, dev, name="ragged_2x64k", steps=5):
    """The batched workload through dhsa_layer_forward twice: as the
    sequential per-sequence loop (workspace for one sequence) and as one pass
    over the batch; per-step time and the peak device memory above the
    resident inputs (torch's allocator holds every device buffer)."""
    w = synth.WORKLOADS[name]
    x = synth.generate(w)
    offs = dhsa.ChunkOffsets.from_list(x.offsets, w.seq_len, device=dev)
    q, k, v = (dhsa.bf16_from_bits(a, dev) for a in (x.q, x.k, x.v))
    stream = torch.cuda.current_stream()
    res = {"workload": name, "batch": w.batch, "seq_len": w.seq_len, "topk": x.topk}
    for label, g in (("sequential", 1), ("one_pass", w.batch)):
        torch.cuda.synchronize()
        base = torch.cuda.memory_allocated()
        torch.cuda.reset_peak_memory_stats()
        layer = dhsa.Layer(offs, w.num_q_heads, w.num_kv_heads, x.topk, max_group=g, device=dev)
        layer(q, k, v)
        torch.cuda.synchronize()
        ev = [[torch.cuda.Event(enable_timing=True) for _ in range(2)] for _ in range(steps)]
        for s in range(steps):
            ev[s][0].record(stream)
            layer(q, k, v)
            ev[s][1].record(stream)
        torch.cuda.synchronize()
        ms = statistics.mean(a.elapsed_time(b) for a, b in ev)
        peak = torch.cuda.max_memory_allocated() - base
        log(f"[bench] batched {label}: {ms:.3f} ms/layer, {layer.num_groups} groups, "
            f"peak {peak / 2**20:.1f} MiB above inputs")
        res[label] = {"ms": ms, "groups": layer.num_groups,
                      "workspace_MiB": layer.ws.numel() / 2**20, "peak_MiB": peak / 2**20}
        del layer
    res["inputs_MiB"] = (q.numel() + k.numel() + v.numel()) * 2 / 2**20
    return res


def hip_stream_read(torch, buf, timed):
    """Best read bandwidth (GB/s) of the streaming-read reference kernel over
    the device buffer buf, and the grid that reached it; None when the
    reference library is not built."""
    import ctypes
    path = os.path.join(ROOT, "long_context_prefill_segmented_amd", "libdhsa_bench.so")
    if not os.path.exists(path):
        return None
    lib = ctypes.CDLL(path)
    lib.dhsa_bench_hbm_read.restype = ctypes.c_int
    lib.dhsa_bench_hbm_read.argtypes = [ctypes.c_void_p, ctypes.c_int64, ctypes.c_void_p,
                                        ctypes.c_int32, ctypes.c_void_p]
    nbytes = buf.numel() * buf.element_size()
    best = None
    stream = torch.cuda.current_stream().cuda_stream
    for grid in (4096, 16384, 32768, 65536, 131072):
        out = torch.empty(grid, dtype=torch.int32, device=buf.device)

        def run():
            rc = lib.dhsa_bench_hbm_read(ctypes.c_void_p(buf.data_ptr()), nbytes,
                                         ctypes.c_void_p(out.data_ptr()), grid,
                                         ctypes.c_void_p(stream))
            if rc != 0:
                raise RuntimeError(f"dhsa_bench_hbm_read returned {rc}")
        gbps = nbytes / (timed(run) * 1e-3) / 1e9
        if best is None or gbps > best[0]:
            best = (gbps, grid)
    return best


def measure_ceilings(torch, dev, reps=10):
    """On-box references, timed outside the layer's timed region with torch as
    a measuring tool: bf16 GEMMs of 8192^3 and 16384^3 (torch.matmul on
    contiguous 2-D operands, the faster reported) as the reachable MFMA
    rate, plus torch's 2 GiB device copy (read + write bytes) and its sum
    over 4 GiB of fp32 (read bytes) as memory references."""
    def timed(fn):
        fn()
        torch.cuda.synchronize()
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(reps):
            fn()
        e1.record()
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / reps  # ms

    n = 2 << 30
    a = torch.empty(n, dtype=torch.uint8, device=dev)
    b = torch.empty_like(a)
    copy_ms = timed(lambda: b.copy_(a))
    del a, b
    f = torch.ones(n // 2, dtype=torch.float32, device=dev)  # 4 GiB
    read_ms = timed(lambda: f.sum())
    hip_read = hip_stream_read(torch, f, timed)
    del f
    g = torch.Generator(device=dev)
    g.manual_seed(0)
    gemm = {}
    for m in (8192, 16384):
        x = torch.randn(m, m, dtype=torch.bfloat16, device=dev, generator=g)
        y = torch.randn(m, m, dtype=torch.bfloat16, device=dev, generator=g)
        gemm[m] = 2 * m ** 3 / (timed(lambda: torch.matmul(x, y)) * 1e-3) / 1e12
        del x, y
    torch.cuda.empty_cache()
    return {"torch_copy_GBps": 2 * n / (copy_ms * 1e-3) / 1e9,
            "torch_sum_read_GBps": 2 * n / (read_ms * 1e-3) / 1e9,
            "hip_stream_read_GBps": hip_read[0] if hip_read else None,
            "hip_stream_read_grid": hip_read[1] if hip_read else None,
            "bf16_gemm_TFLOPs": max(gemm.values()),
            "bf16_gemm_TFLOPs_by_size": {str(m): v for m, v in gemm.items()},
            "how": "2 GiB device copy (read + write bytes), sum of 4 GiB fp32 (read bytes), "
                   "a HIP kernel streaming the same 4 GiB with 16-byte non-temporal loads "
                   "(libdhsa_bench.so, best of five grid sizes), "
                   f"8192^3 and 16384^3 bf16 matmuls; {reps} repetitions each, outside the "
                   "timed region"}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=2)
    ap.add_argument("--workload", default="llama31_8b_128k")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-variants", action="store_true",
                    help="skip the widened-selection, NMS and batched-loop legs and the "
                         "reference ceilings (for profiling runs)")
    ap.add_argument("--no-layers", action="store_true",
                    help="skip the other layer shapes and the dense-causal 128K leg")
    ap.add_argument("--calib-copy", action="store_true",
                    help="also run one 1 GiB device copy (counter calibration)")
    args = ap.parse_args()

    if args.gpus != 1:
        print(f"bench.py measures one GPU only (asked for --gpus {args.gpus}); the path is "
              "single-GPU by design", file=sys.stderr)
        sys.exit(2)

    import torch
    from long_context_prefill_segmented_amd import dhsa, synth

    w = synth.WORKLOADS[args.workload]
    log(f"[bench] generating {w.name} (seed {w.seed})")
    x = synth.generate(w)
    hq, hkv = w.num_q_heads, w.num_kv_heads
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    offs = dhsa.ChunkOffsets.from_list(x.offsets, w.seq_len, device=dev)
    q = dhsa.bf16_from_bits(x.q, dev)
    k = dhsa.bf16_from_bits(x.k, dev)
    v = dhsa.bf16_from_bits(x.v, dev)
    mb = dhsa.MaskBuilder(offs, hq, hkv, x.topk, device=dev)
    pf = dhsa.Prefill(offs, hq, hkv, device=dev)
    stream = torch.cuda.current_stream()

    if args.calib_copy:
        a = torch.empty(1 << 30, dtype=torch.uint8, device=dev)
        bb = torch.empty_like(a)
        bb.copy_(a)
        torch.cuda.synchronize()
        del a, bb

    log(f"[bench] warmup {args.warmup}")
    for _ in range(args.warmup):
        csr = mb(q, k)
        pf(q, k, v, csr)
    torch.cuda.synchronize()
    csr = mb(q, k)
    torch.cuda.synchronize()
    rp = csr.row_ptr.cpu().numpy()
    ci = csr.col_idx.cpu().numpy()[:csr.nnz]
    flops = kept_tile_flops(x.offsets, rp, ci, hq)
    total_pairs = sum(len(o) - 1 for o in x.offsets)
    mask_bytes = 2 * w.batch * w.seq_len * (hq + hkv) * 128 + 4 * (rp.size + ci.size)

    log(f"[bench] timing {args.steps} steps")
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True),
           torch.cuda.Event(enable_timing=True)) for _ in range(args.steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for s in range(args.steps):
        ev[s][0].record(stream)
        csr = mb(q, k)
        ev[s][1].record(stream)
        pf(q, k, v, csr)
        ev[s][2].record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    mask_ms = [a.elapsed_time(b) for a, b, _ in ev]
    attn_ms = [b.elapsed_time(c) for _, b, c in ev]
    ms_per_step = wall * 1e3 / args.steps
    attn_avg = statistics.mean(attn_ms)
    mask_avg = statistics.mean(mask_ms)
    log(f"[bench] mask {mask_avg:.3f} ms  attention {attn_avg:.3f} ms  wall/step {ms_per_step:.3f} ms")
    state = {}

    def run_mask():
        state["csr"] = mb(q, k)

    def run_attn():
        pf(q, k, v, state["csr"])

    p_mask, p_attn = pages_protocol(torch, stream, [run_mask, run_attn])
    log(f"[bench] median of 5 after 2 warmups: mask {p_mask:.3f} ms  attention {p_attn:.3f} ms")

    achieved = flops / (attn_avg * 1e-3) / 1e12
    traffic = None
    if os.path.exists(PMC_FILE):
        try:
            pm = json.load(open(PMC_FILE))
            if pm.get("source_hash") == source_hash(ATTN_SOURCES) and pm.get("workload") == w.name:
                traffic = pm.get("hbm_bytes_per_launch")
        except Exception:
            traffic = None

    stages = time_mask_stages(dhsa, torch, x, offs, q, k, hq, hkv, steps=args.steps)

    layers = {}
    if not args.no_layers:
        for name in ("qwen25_3b_16k", "llama31_8b_32k"):
            if name != w.name:
                layers[name] = time_layer(dhsa, synth, torch, dev, name, steps=args.steps)
        C = max(len(o) - 1 for o in x.offsets)
        layers["dense_causal_" + w.name] = time_layer(
            dhsa, synth, torch, dev, w.name, steps=3, topk=C, label="dense_causal_" + w.name, x=x)
        d = layers["dense_causal_" + w.name]
        d["sparse_speedup"] = d["ms_per_layer_median5"] / (p_mask + p_attn)
        d["note"] = ("same layer and kernels with topk >= chunk count: every causal chunk kept; "
                     "sparse_speedup = this median latency / the sparse layer's")

    variants = {}
    if not args.no_variants:
        variants["row_budgets_recent2"] = time_variant(
            dhsa, synth, torch, x, offs, q, k, v, pf, hq, hkv, recent=2,
            steps=max(2, args.steps // 2), dev=dev)
        variants["boundary_nms"] = time_nms(dhsa, synth, torch, x, dev)
        variants["batched_loop"] = time_batched_loop(dhsa, synth, torch, dev)

    ceilings = None
    if not args.no_variants:
        log("[bench] reference ceilings (copy, bf16 GEMM)")
        ceilings = measure_ceilings(torch, dev)
        # torch's copy and reduction are references, not the HBM limit (the
        # pooling kernel streams faster than either)
        ceilings["mask_vs_torch_copy"] = (mask_bytes / (mask_avg * 1e-3) / 1e9) / \
            ceilings["torch_copy_GBps"]
        sr = ceilings.get("hip_stream_read_GBps")
        if sr:
            # the measured streaming-read rate: the realistic HBM limit of
            # the read-dominated mask, next to the nominal 8 TB/s
            ceilings["mask_vs_stream_read"] = (mask_bytes / (mask_avg * 1e-3) / 1e9) / sr
            ceilings["pool_q_vs_stream_read"] = stages["pool_q_GBps"] / sr
        ceilings["attention_frac_of_gemm"] = achieved / ceilings["bf16_gemm_TFLOPs"]

    cpu = None
    if not args.no_cpu_baseline:
        log("[bench] cpu baseline (oracle on a bounded sample)")
        cpu = cpu_baseline(x, hq, hkv)

    line = {
        "metric": "sparse prefill ms/layer + kept-tile TFLOP/s, Llama-3.1-8B layer shape @128K",
        "value": flops / (ms_per_step * 1e-3) / 1e12,
        "unit": "TFLOP/s (kept tiles, whole layer incl. mask construction)",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_per_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic (seeded; chunk offsets and values drawn per the workload recipe)",
        "config": {"workload": w.name, "batch": w.batch, "seq_len": w.seq_len,
                   "num_q_heads": hq, "num_kv_heads": hkv, "head_dim": 128, "topk": x.topk,
                   "num_chunks": [len(o) - 1 for o in x.offsets], "nnz": int(ci.size)},
        "mask_ms": mask_avg,
        "attention_ms": attn_avg,
        "mask_ms_median": statistics.median(mask_ms),
        "attention_ms_median": statistics.median(attn_ms),
        "ms_per_layer_median5": p_mask + p_attn,
        "mask_ms_median5": p_mask,
        "attention_ms_median5": p_attn,
        "mask_GBps": mask_bytes / (mask_avg * 1e-3) / 1e9,
        "mask_hbm_frac": mask_bytes / (mask_avg * 1e-3) / 1e9 / PEAK_HBM_GBPS,
        "mask_stages": stages,
        "kept_tile_TFLOP": flops / 1e12,
        "chunk_pairs": total_pairs,
        "roofline": {"bound": "mfma", "kernel": "attn_fwd_kernel", "achieved": achieved,
                     "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s", "frac": achieved / PEAK_BF16_TFLOPS,
                     "traffic": traffic},
        "ceilings": ceilings,
        "layers": layers,
        "variants": variants,
        "cpu_baseline": cpu,
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
