"""GPU parity of boundary finalisation (dhsa_nms_boundaries) against the
oracle's greedy NMS: offsets bit-exact (the kernel and the oracle compare the
same float32 scores), on synthetic predictor outputs, exact ties, NaNs,
all-candidate inputs, monotone ramps (the longest chains of rounds), and the
degenerate cases; then at full size, feeding the offsets to the mask and
attention path."""
import sys

import numpy as np
import pytest

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

if not torch.cuda.is_available():  # pragma: no cover
    pytest.skip("needs a GPU", allow_module_level=True)

from long_context_prefill_segmented_amd import dhsa, synth  # noqa: E402
from oracle import dhsa_oracle as orc  # noqa: E402


def say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def run_and_compare(p, g, tau, what):
    p = np.ascontiguousarray(p, dtype=np.float32)
    B, L = p.shape
    say(f"  nms {what}: B={B} L={L} min_gap={g} threshold={tau}")
    offs, nc = dhsa.nms_boundaries(torch.from_numpy(p).cuda(), g, tau)
    torch.cuda.synchronize()
    offs = offs.cpu().numpy()
    nc = nc.cpu().numpy()
    out = []
    for b in range(B):
        want = orc.nms_boundaries(p[b].astype(np.float64), g, tau)
        got = offs[b, :int(nc[b]) + 1]
        np.testing.assert_array_equal(got, want, err_msg=f"{what} b{b}")
        out.append(got)
    return out


def test_nms_on_synthetic_predictor_scores():
    for name, g in (("tiny_1k", 8), ("qwen25_3b_16k", 16)):
        w = synth.WORKLOADS[name]
        x = synth.generate(w)
        p = synth.boundary_scores(x.offsets, w.seq_len, seed=w.seed)
        run_and_compare(p, g, 0.5, name)


def test_nms_batch_of_ragged_sequences():
    rng = np.random.default_rng(3)
    offsets = [synth.draw_chunk_lengths(rng, 6000, ((0.7, 8, 32), (0.3, 64, 256)))
               for _ in range(3)]
    p = synth.boundary_scores(offsets, 6000, seed=9, spurious_per_token=1 / 300)
    run_and_compare(p, 6, 0.5, "ragged batch")


def test_nms_ties_nans_and_all_candidates():
    rng = np.random.default_rng(4)
    p = (rng.integers(0, 4, size=(2, 3000)) / 4.0).astype(np.float32)   # exact ties
    run_and_compare(p, 5, 0.5, "ties")
    p[0, rng.integers(0, 3000, size=200)] = np.nan
    run_and_compare(p, 5, 0.25, "nans")
    p = rng.random((1, 5000), dtype=np.float32)
    run_and_compare(p, 16, 0.0, "all candidates")
    run_and_compare(p, 1, 0.0, "min_gap 1")


def test_nms_monotone_ramps_and_degenerate_cases():
    L = 4096
    up = (np.arange(L, dtype=np.float32) / L)[None]
    run_and_compare(up, 32, 0.0, "increasing ramp")     # L / min_gap rounds
    run_and_compare(up[:, ::-1].copy(), 32, 0.0, "decreasing ramp")
    flat = np.full((1, 1000), 0.7, dtype=np.float32)
    run_and_compare(flat, 10, 0.5, "flat")              # ties everywhere
    run_and_compare(np.zeros((1, 1000), np.float32), 10, 0.5, "no candidate")
    run_and_compare(np.ones((1, 15), np.float32), 8, 0.5, "shorter than 2 min_gap")
    run_and_compare(np.ones((1, 1), np.float32), 1, 0.5, "one token")


def test_nms_at_the_maximum_length():
    # DHSA_NMS_MAX_LEN tokens: every 2-bit token state of the sequence in LDS
    L = dhsa.NMS_MAX_LEN
    offsets = [synth.draw_chunk_lengths(np.random.default_rng(6), L, ((1.0, 64, 512),))]
    p = synth.boundary_scores(offsets, L, seed=10)
    out = run_and_compare(p, 32, 0.5, "maximum length")
    assert len(out[0]) > 1000
    # dense candidates at that length (one in four tokens above threshold)
    p = np.random.default_rng(7).random((1, L), dtype=np.float32)
    run_and_compare(p, 8, 0.75, "maximum length, dense")


def test_nms_reuse_and_smaller_batch():
    # one BoundaryNMS object, two different inputs: no state leaks between calls
    rng = np.random.default_rng(5)
    nms = dhsa.BoundaryNMS(2, 2048, 12, 0.5)
    for trial in range(2):
        p = rng.random((2, 2048), dtype=np.float32)
        offs, nc = nms(torch.from_numpy(p).cuda())
        torch.cuda.synchronize()
        for b in range(2):
            want = orc.nms_boundaries(p[b].astype(np.float64), 12, 0.5)
            np.testing.assert_array_equal(offs.cpu().numpy()[b, :int(nc[b]) + 1], want)


@pytest.mark.parametrize("name", ["llama31_8b_128k", "ragged_2x64k"])
def test_nms_full_size_feeds_the_path(name):
    w = synth.WORKLOADS[name]
    x = synth.generate(w)
    p = synth.boundary_scores(x.offsets, w.seq_len, seed=w.seed)
    g = 32 if name == "llama31_8b_128k" else 6
    nms = dhsa.BoundaryNMS(w.batch, w.seq_len, g, 0.5)
    nms(torch.from_numpy(p).cuda())
    co = nms.to_chunk_offsets()
    starts = np.concatenate([[0], np.cumsum(co.num_chunks.astype(np.int64) + 1)])
    for b in range(w.batch):
        want = orc.nms_boundaries(p[b].astype(np.float64), g, 0.5)
        np.testing.assert_array_equal(co.host[starts[b]:starts[b + 1]], want)
        say(f"  {name} b{b}: {len(want) - 1} chunks from NMS, {len(x.offsets[b]) - 1} drawn")
    # the NMS offsets drive the mask and the attention: the selection equals
    # the oracle's on the GPU's own fp32 scores, and sampled attention rows
    # (first, last, longest chunk and seeded picks) equal the oracle's
    assert int(co.num_chunks.max()) <= 2048
    q, k, v = (dhsa.bf16_from_bits(a) for a in (x.q, x.k, x.v))
    hq, G = w.num_q_heads, w.num_q_heads // w.num_kv_heads
    csr, flat = dhsa.build_mask(q, k, co, x.topk, return_scores=True)
    out = dhsa.sparse_prefill(q, k, v, co, csr)
    torch.cuda.synchronize()
    rows = orc.csr_to_rows(csr.row_ptr.cpu().numpy(), csr.col_idx.cpu().numpy()[:csr.nnz],
                           co.num_chunks, hq)
    scores = flat.cpu().numpy()
    got_all = orc.widen_bf16(out.view(torch.int16).cpu().numpy().view(np.uint16))
    rng = np.random.default_rng(11)
    spos = 0
    for b in range(w.batch):
        o = co.host[starts[b]:starts[b + 1]].astype(np.int64)
        C = len(o) - 1
        gs = scores[spos:spos + hq * C * C].reshape(hq, C, C).astype(np.float64)
        spos += hq * C * C
        assert orc.select_topk(gs, x.topk) == rows[b]
        qf, kf, vf = (orc.widen_bf16(a[b]) for a in (x.q, x.k, x.v))
        n = np.diff(o)
        picks = {(0, 0), (hq - 1, C - 1), (hq // 2, int(np.argmax(n)))}
        picks |= {(int(rng.integers(0, hq)), int(rng.integers(0, C))) for _ in range(8)}
        for (h, i) in sorted(picks):
            ref, _ = orc.chunk_attention(qf, kf, vf, o, rows[b][h][i], i, h, h // G,
                                         1.0 / np.sqrt(128))
            got = got_all[b, o[i]:o[i + 1], h]
            err = np.abs(got - ref)
            assert np.all(err <= 1e-2 + 1e-2 * np.abs(ref)), (name, b, h, i, float(err.max()))
        say(f"  {name} b{b}: selection bit-exact, {len(picks)} attention rows within the bar")
