"""GPU parity at the full workload sizes, in the launch configuration bench.py
times: the whole GPU path runs on the full layer; the oracle recomputes the
mask for the whole layer (pooling, scores and selection are cheap in
float64) and the attention output for a seeded sample of (sequence, head,
query chunk) rows plus the edge rows (first and last chunk, the longest
chunk, every needle row).  Same bars as the small cases."""
import sys

import numpy as np
import pytest

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

if not torch.cuda.is_available():  # pragma: no cover
    pytest.skip("needs a GPU", allow_module_level=True)

from long_context_prefill_segmented_amd import dhsa, synth  # noqa: E402
from oracle import dhsa_oracle as orc  # noqa: E402

ATOL = RTOL = 1e-2
SAMPLES = 10


def say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def to_np_bf16(t):
    return t.view(torch.int16).cpu().numpy().view(np.uint16)


@pytest.mark.parametrize("name", ["qwen25_3b_16k", "llama31_8b_32k", "llama31_8b_128k",
                                  "ragged_2x64k"])
def test_full_size_layer(name):
    w = synth.WORKLOADS[name]
    say(f"[full] {name}: generating")
    x = synth.generate(w)
    hq, hkv, G = w.num_q_heads, w.num_kv_heads, w.num_q_heads // w.num_kv_heads
    offs = dhsa.ChunkOffsets.from_list(x.offsets, w.seq_len)
    q, k, v = (dhsa.bf16_from_bits(a) for a in (x.q, x.k, x.v))
    say(f"[full] {name}: GPU mask + attention (topk {x.topk})")
    mb = dhsa.MaskBuilder(offs, hq, hkv, x.topk, keep_scores=True)
    pf = dhsa.Prefill(offs, hq, hkv, with_lse=True)
    csr = mb(q, k)
    out, lse = pf(q, k, v, csr)
    torch.cuda.synchronize()
    rp = csr.row_ptr.cpu().numpy()
    ci = csr.col_idx.cpu().numpy()[:csr.nnz]
    gpu_rows = orc.csr_to_rows(rp, ci, offs.num_chunks, hq)
    scores = mb.scores.cpu().numpy()
    out_np = to_np_bf16(out)
    lse_np = lse.cpu().numpy()

    rng = np.random.default_rng(7)
    spos = 0
    ref_rows_all = []
    for b in range(w.batch):
        o = x.offsets[b]
        C = len(o) - 1
        say(f"[full] {name}: oracle mask, sequence {b} ({C} chunks)")
        qf = orc.widen_bf16(x.q[b])
        kf = orc.widen_bf16(x.k[b])
        qbar, kbar, s64, s32, rows = orc.build_mask(qf, kf, o, x.topk)
        ref_rows_all.append(rows)
        # scores within the normwise bound
        gs = scores[spos:spos + hq * C * C].reshape(hq, C, C)
        spos += hq * C * C
        qn = np.linalg.norm(qbar, axis=2)
        kn = np.linalg.norm(kbar, axis=2)
        low = np.tril(np.ones((C, C), dtype=bool))
        for h in range(hq):
            bound = 1e-5 * qn[h][:, None] * kn[h // G][None, :]
            err = np.abs(gs[h] - s64[h])
            assert np.all(err[low] <= bound[low]), (name, b, h, float(err[low].max()))
        # the fixed rule on the GPU's own fp32 scores: bit-exact
        assert orc.select_topk(gs.astype(np.float64), x.topk) == gpu_rows[b], (name, b)
        # mask: equal, or a near-tie within the score bound
        near = 0
        for h in range(hq):
            for i in range(C):
                got, want = gpu_rows[b][h][i], rows[h][i]
                if got == want:
                    continue
                tol = 2e-5 * qn[h, i] * kn[h // G].max()
                lo = min(s64[h, i, j] for j in set(want) - set(got))
                assert all(s64[h, i, j] >= lo - tol for j in set(got) - set(want)), (b, h, i)
                near += 1
        say(f"[full] {name}: sequence {b}: {near} near-tie rows of {hq * C}")
        assert near <= max(1, hq * C // 1000)
        # needles
        for (nb, ni, nj, ng) in x.needles:
            if nb == b:
                for h in range(ng * G, (ng + 1) * G):
                    assert nj in gpu_rows[b][h][ni], (ni, nj, h)
        # sampled attention rows on the GPU's own mask (where it equals the oracle's)
        vf = orc.widen_bf16(x.v[b])
        n = np.diff(o)
        picks = {(int(rng.integers(0, hq)), int(rng.integers(0, C))) for _ in range(SAMPLES)}
        picks |= {(0, 0), (hq - 1, C - 1), (hq // 2, int(np.argmax(n)))}
        picks |= {(ng * G, ni) for (nb, ni, nj, ng) in x.needles if nb == b}
        for (h, i) in sorted(picks):
            if gpu_rows[b][h][i] != rows[h][i]:
                continue
            ref, lref = orc.chunk_attention(qf, kf, vf, o, rows[h][i], i, h, h // G,
                                            1.0 / np.sqrt(128))
            got = orc.widen_bf16(out_np[b, o[i]:o[i + 1], h])
            err = np.abs(got - ref)
            assert np.all(err <= ATOL + RTOL * np.abs(ref)), (name, b, h, i, float(err.max()))
            lg = lse_np[b, h, o[i]:o[i + 1]].astype(np.float64)
            assert np.all(np.abs(lg - lref) <= 2e-3 * (1 + np.abs(lref))), (name, b, h, i)
        del qf, kf, vf

    # attention on the oracle's mask: the same sampled rows, selection decoupled
    rp_ref, ci_ref = orc.rows_to_csr(ref_rows_all)
    out2 = pf(q, k, v, dhsa.csr_from_host(rp_ref, ci_ref))[0]
    torch.cuda.synchronize()
    out2_np = to_np_bf16(out2)
    for b in range(w.batch):
        o = x.offsets[b]
        C = len(o) - 1
        qf = orc.widen_bf16(x.q[b])
        kf = orc.widen_bf16(x.k[b])
        vf = orc.widen_bf16(x.v[b])
        rows = ref_rows_all[b]
        # every query chunk of two heads (the first and the last; the last
        # head's KV group differs from the first's)
        for h in sorted({0, hq - 1}):
            for i in range(C):
                ref, _ = orc.chunk_attention(qf, kf, vf, o, rows[h][i], i, h, h // G,
                                             1.0 / np.sqrt(128))
                got = orc.widen_bf16(out2_np[b, o[i]:o[i + 1], h])
                err = np.abs(got - ref)
                assert np.all(err <= ATOL + RTOL * np.abs(ref)), (name, b, h, i, float(err.max()))
        say(f"[full] {name}: sequence {b}: all {C} query chunks of heads 0 and {hq - 1} "
            f"on the oracle mask within the bar")
        del qf, kf, vf
    say(f"[full] {name}: ok")


@pytest.mark.parametrize("name", ["llama31_8b_128k", "ragged_2x64k"])
def test_full_size_budgets_and_recent(name):
    """The widened selection rule at full size (per-row budgets with mean
    topk, capped at 2 topk - 1, and a 2-chunk recent window, as bench.py's
    variant leg): the GPU selection equals the oracle's on the GPU's own
    fp32 scores bit for bit, and the oracle's float64 selection up to
    near-ties; sampled attention rows within the attention bar."""
    w = synth.WORKLOADS[name]
    say(f"[full-ex] {name}: generating")
    x = synth.generate(w)
    hq, hkv, G = w.num_q_heads, w.num_kv_heads, w.num_q_heads // w.num_kv_heads
    offs = dhsa.ChunkOffsets.from_list(x.offsets, w.seq_len)
    q, k, v = (dhsa.bf16_from_bits(a) for a in (x.q, x.k, x.v))
    cap, recent = 2 * x.topk - 1, 2
    bud_np = synth.row_budgets(offs.num_chunks, hq, x.topk, seed=w.seed)
    mb = dhsa.MaskBuilder(offs, hq, hkv, cap, keep_scores=True, recent=recent)
    pf = dhsa.Prefill(offs, hq, hkv)
    csr = mb(q, k, row_budgets=torch.from_numpy(bud_np).cuda())
    out = pf(q, k, v, csr)
    torch.cuda.synchronize()
    rp = csr.row_ptr.cpu().numpy()
    assert rp[-1] <= csr.nnz
    gpu_rows = orc.csr_to_rows(rp, csr.col_idx.cpu().numpy()[:rp[-1]], offs.num_chunks, hq)
    scores = mb.scores.cpu().numpy()
    out_np = to_np_bf16(out)
    rng = np.random.default_rng(8)
    spos = bpos = 0
    for b in range(w.batch):
        o = x.offsets[b]
        C = len(o) - 1
        bud = np.clip(bud_np[bpos:bpos + hq * C].reshape(hq, C), 1, cap)
        bpos += hq * C
        gs = scores[spos:spos + hq * C * C].reshape(hq, C, C).astype(np.float64)
        spos += hq * C * C
        say(f"[full-ex] {name}: oracle selection on the GPU scores, sequence {b}")
        assert orc.select_topk_ex(gs, bud, recent) == gpu_rows[b]
        qf = orc.widen_bf16(x.q[b])
        kf = orc.widen_bf16(x.k[b])
        qbar, kbar, s64, _s32, _rows = orc.build_mask(qf, kf, o, x.topk)
        rows = orc.select_topk_ex(s64, bud, recent)
        qn = np.linalg.norm(qbar, axis=2)
        kn = np.linalg.norm(kbar, axis=2)
        near = 0
        for h in range(hq):
            for i in range(C):
                got, want = gpu_rows[b][h][i], rows[h][i]
                if got == want:
                    continue
                tol = 2e-5 * qn[h, i] * kn[h // G].max()
                lo = min(s64[h, i, j] for j in set(want) - set(got))
                assert all(s64[h, i, j] >= lo - tol for j in set(got) - set(want)), (b, h, i)
                near += 1
        say(f"[full-ex] {name}: sequence {b}: {near} near-tie rows of {hq * C}")
        assert near <= max(1, hq * C // 1000)
        vf = orc.widen_bf16(x.v[b])
        picks = {(int(rng.integers(0, hq)), int(rng.integers(0, C))) for _ in range(SAMPLES)}
        picks |= {(0, C - 1), (hq - 1, min(C - 1, recent + 1))}
        for (h, i) in sorted(picks):
            if gpu_rows[b][h][i] != rows[h][i]:
                continue
            ref, _ = orc.chunk_attention(qf, kf, vf, o, rows[h][i], i, h, h // G,
                                         1.0 / np.sqrt(128))
            got = orc.widen_bf16(out_np[b, o[i]:o[i + 1], h])
            err = np.abs(got - ref)
            assert np.all(err <= ATOL + RTOL * np.abs(ref)), (name, b, h, i, float(err.max()))
        del qf, kf, vf
    say(f"[full-ex] {name}: ok")
