"""The seeded input generators: determinism, valid boundaries, the recipe."""
import numpy as np
import torch

from long_context_prefill_segmented_amd import synth


def test_bf16_rounding_matches_torch():
    rng = np.random.default_rng(0)
    x = np.concatenate([rng.standard_normal(100000).astype(np.float32),
                        np.array([0.0, -0.0, 1.0, -1.5, 3.0e38, 1e-40], dtype=np.float32)])
    ours = synth.f32_to_bf16_bits(x)
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    np.testing.assert_array_equal(ours, ref)
    back = synth.bf16_bits_to_f32(ours)
    np.testing.assert_array_equal(back, torch.from_numpy(x).to(torch.bfloat16).float().numpy())


def test_generation_is_deterministic_and_seed_dependent():
    w = synth.WORKLOADS["tiny_1k"]
    a = synth.generate(w)
    b = synth.generate(w)
    c = synth.generate(w, seed=99)
    np.testing.assert_array_equal(a.q, b.q)
    np.testing.assert_array_equal(a.offsets_concat, b.offsets_concat)
    assert not np.array_equal(a.q, c.q)


def test_offsets_follow_the_law_and_end_at_L():
    for name in ("tiny_1k", "qwen25_3b_16k"):
        w = synth.WORKLOADS[name]
        x = synth.generate(w) if name == "tiny_1k" else None
        rng = np.random.Generator(np.random.PCG64(w.seed))
        o = synth.draw_chunk_lengths(rng, w.seq_len, w.chunk_law)
        assert o[0] == 0 and o[-1] == w.seq_len
        n = np.diff(o)
        _, lo, hi = w.chunk_law[0]
        assert np.all(n[:-1] >= lo) and np.all(n <= hi) and n[-1] >= 1
        if x is not None:
            np.testing.assert_array_equal(x.offsets[0], o)


def test_ragged_mix_components():
    w = synth.WORKLOADS["ragged_2x64k"]
    rng = np.random.Generator(np.random.PCG64(w.seed))
    n = np.diff(synth.draw_chunk_lengths(rng, w.seq_len, w.chunk_law))[:-1]
    small = np.mean((n >= 8) & (n <= 32))
    mid = np.mean((n >= 64) & (n <= 256))
    big = np.mean((n >= 1024) & (n <= 2048))
    assert abs(small - 0.70) < 0.08 and abs(mid - 0.25) < 0.08 and 0.01 < big < 0.1
    assert np.all(((n >= 8) & (n <= 32)) | ((n >= 64) & (n <= 256)) | ((n >= 1024) & (n <= 2048)))


def test_density_rule():
    # k=1 keeps only the diagonal: density 2/(C+1); k=C keeps every pair
    assert abs(synth.causal_pair_density(10, 1) - 10 / 55) < 1e-12
    assert synth.causal_pair_density(10, 10) == 1.0
    k = synth.choose_topk([438], 0.05)
    d = synth.causal_pair_density(438, k)
    assert abs(d - 0.05) <= abs(synth.causal_pair_density(438, k + 1) - 0.05)
    assert abs(d - 0.05) <= abs(synth.causal_pair_density(438, k - 1) - 0.05)


def test_structured_values_and_needles():
    w = synth.small_workload("s", 1, 4096, 4, 2, (64, 128), "qkv_centroid", topk=3,
                             seed=7, needles=3)
    x = synth.generate(w)
    assert x.q.dtype == np.uint16 and x.q.shape == (1, 4096, 4, 128)
    assert len(x.needles) == 3 * 2
    C = len(x.offsets[0]) - 1
    pairs = {(i, j) for (_b, i, j, _g) in x.needles}
    assert len(pairs) == 3
    for (i, j) in pairs:
        assert C // 2 <= i < C and 0 <= j <= i - 2
    # tokens of one chunk cluster around their centroid: within-chunk spread
    # is the 0.5 noise, far below the unit spread between centroids
    k = synth.bf16_bits_to_f32(x.k[0, :, 0])
    o = x.offsets[0]
    c = 3
    seg = k[o[c]:o[c + 1]]
    assert 0.4 < seg.std(axis=0).mean() < 0.6
