"""Seeded synthetic inputs for the DHSA prefill path.

This module only *draws* inputs: chunk boundaries, bf16 Q/K/V values and the
planted "needle" pairs.  It holds none of the method's arithmetic (no pooling,
no scores, no selection, no attention), so both the GPU path and the CPU
oracle can consume what it produces without sharing any computation.

Workload shapes follow the DHSA pages: Llama-3.1-8B and Qwen2.5-3B attention
layer shapes (32/8 and 16/2 heads, head dim 128), BF16, causal prefill
(DHSA README, "Installation": the sparse kernel is BF16, causal, forward-only,
head dim 128).  Chunk boundaries stand in for the learned boundary predictor
(gist.science technical summary, "Methodology" step 1: variable-length chunks)
and are drawn from a seed.  The needle pairs are a synthetic stand-in for the
retrieval structure of a needle-in-a-haystack test; no benchmark item is used.

Recipe (all draws from ``numpy.random.Generator(PCG64(seed))``, in this order):

1. chunk lengths, sequence by sequence: integers drawn uniformly (inclusive
   bounds) from the workload's law until the running sum reaches L; the last
   chunk is truncated so that the offsets end exactly at L;
2. per-(chunk, head) centroids mu ~ N(0, 1)^128 for each structured tensor
   (in the order Q, K, V), then token values mu + 0.5 * z with z ~ N(0, 1);
   iid tensors are plain N(0, 1);
3. needles (if any): pairs (i, j) with i in the last half of the chunks and
   j in [0, i - 2]; for each KV head g a vector nu ~ N(0,1)^128; every query
   head of group g gets nu + 0.5 z on chunk i and KV head g gets
   4 nu + 0.5 z on chunk j.

Values are drawn in float32 and rounded once to bfloat16 with
round-to-nearest-even; the result is kept as raw uint16 bit patterns so that
every consumer reads identical bits.
"""
from __future__ import annotations

import dataclasses
from typing import List, Optional, Sequence, Tuple

import numpy as np

HEAD_DIM = 128


@dataclasses.dataclass(frozen=True)
class Workload:
    """Shape and input recipe of one synthetic attention layer."""

    name: str
    batch: int
    seq_len: int
    num_q_heads: int
    num_kv_heads: int
    # chunk-length law: a tuple of (probability, lo, hi) components
    chunk_law: Tuple[Tuple[float, int, int], ...]
    # "iid", "kv_centroid" (K and V structured) or "qkv_centroid"
    structure: str
    topk: Optional[int] = None           # fixed top-k, or
    target_density: Optional[float] = None  # chosen per the density rule
    needles: int = 0
    seed: int = 0
    head_dim: int = HEAD_DIM

    def with_seed(self, seed: int) -> "Workload":
        return dataclasses.replace(self, seed=seed)


WORKLOADS = {
    # small single layer the oracle finishes in seconds
    "tiny_1k": Workload("tiny_1k", 1, 1024, 2, 1, ((1.0, 16, 64),), "iid",
                        topk=4, seed=1),
    "qwen25_3b_16k": Workload("qwen25_3b_16k", 1, 16384, 16, 2,
                              ((1.0, 32, 256),), "kv_centroid",
                              target_density=0.20, seed=2),
    "llama31_8b_32k": Workload("llama31_8b_32k", 1, 32768, 32, 8,
                               ((1.0, 64, 512),), "qkv_centroid",
                               target_density=0.10, seed=3),
    # the headline layer: Llama-3.1-8B shape at 128K context
    "llama31_8b_128k": Workload("llama31_8b_128k", 1, 131072, 32, 8,
                                ((1.0, 64, 512),), "qkv_centroid",
                                target_density=0.05, needles=8, seed=4),
    "ragged_2x64k": Workload("ragged_2x64k", 2, 65536, 32, 8,
                             ((0.70, 8, 32), (0.25, 64, 256), (0.05, 1024, 2048)),
                             "iid", topk=16, seed=5),
}
HEADLINE = "llama31_8b_128k"


@dataclasses.dataclass
class Inputs:
    """One drawn layer: bf16 bit patterns plus chunk boundaries."""

    workload: Workload
    q: np.ndarray            # uint16 [B, L, Hq, D] (bf16 bits)
    k: np.ndarray            # uint16 [B, L, Hkv, D]
    v: np.ndarray            # uint16 [B, L, Hkv, D]
    offsets: List[np.ndarray]  # per sequence int32 [C_b + 1], 0 ... L
    topk: int
    needles: List[Tuple[int, int, int, int]]  # (b, i, j, kv_head)

    @property
    def num_chunks(self) -> np.ndarray:
        return np.array([len(o) - 1 for o in self.offsets], dtype=np.int32)

    @property
    def offsets_concat(self) -> np.ndarray:
        return np.concatenate(self.offsets).astype(np.int32)


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 to bfloat16 (nearest, ties to even); returns uint16 bits."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    u = x.view(np.uint32)
    out = np.empty(u.shape, dtype=np.uint16)
    # process in slabs to bound temporary memory
    flat_u = u.reshape(-1)
    flat_o = out.reshape(-1)
    step = 1 << 26
    for s in range(0, flat_u.size, step):
        a = flat_u[s:s + step]
        r = (a + np.uint32(0x7FFF) + ((a >> np.uint32(16)) & np.uint32(1))) >> np.uint32(16)
        flat_o[s:s + step] = r.astype(np.uint16)
    return out


def bf16_bits_to_f32(bits: np.ndarray) -> np.ndarray:
    """Exact widening of bf16 bit patterns to float32."""
    return (bits.astype(np.uint32) << np.uint32(16)).view(np.float32)


def draw_chunk_lengths(rng: np.random.Generator, seq_len: int,
                       law: Sequence[Tuple[float, int, int]]) -> np.ndarray:
    """Chunk offsets for one sequence: lengths drawn until the sum reaches L."""
    probs = np.array([p for p, _, _ in law], dtype=np.float64)
    cum = np.cumsum(probs)
    cum[-1] = 1.0
    lengths: List[int] = []
    total = 0
    while total < seq_len:
        block = 1024
        if len(law) == 1:
            _, lo, hi = law[0]
            lens = rng.integers(lo, hi + 1, size=block)
        else:
            u = rng.random(block)
            comp = np.searchsorted(cum, u, side="right")
            comp = np.minimum(comp, len(law) - 1)
            lens = np.empty(block, dtype=np.int64)
            draws = [rng.integers(lo, hi + 1, size=block) for _, lo, hi in law]
            for c in range(len(law)):
                sel = comp == c
                lens[sel] = draws[c][sel]
        for n in lens.tolist():
            if total >= seq_len:
                break
            n = min(int(n), seq_len - total)
            lengths.append(n)
            total += n
    offs = np.zeros(len(lengths) + 1, dtype=np.int32)
    offs[1:] = np.cumsum(lengths)
    return offs


def causal_pair_density(num_chunks: int, k: int) -> float:
    """Fraction of causal chunk pairs kept when every row keeps min(k, i+1)."""
    c = num_chunks
    kept = sum(min(k, i + 1) for i in range(c))
    return kept / (c * (c + 1) / 2)


def choose_topk(num_chunks: Sequence[int], target: float) -> int:
    """Smallest k whose causal chunk-pair density is closest to ``target``.

    The density is pooled over all sequences of the layer; ties go to the
    smaller k.
    """
    best_k, best_err = 1, None
    cmax = max(num_chunks)
    for k in range(1, cmax + 1):
        kept = sum(sum(min(k, i + 1) for i in range(c)) for c in num_chunks)
        pairs = sum(c * (c + 1) / 2 for c in num_chunks)
        err = abs(kept / pairs - target)
        if best_err is None or err < best_err - 1e-15:
            best_k, best_err = k, err
    return best_k


def _structured(rng, offsets: np.ndarray, heads: int, d: int) -> np.ndarray:
    c = len(offsets) - 1
    lens = np.diff(offsets)
    mu = rng.standard_normal((c, heads, d), dtype=np.float32)
    x = np.repeat(mu, lens, axis=0)
    x += np.float32(0.5) * rng.standard_normal(x.shape, dtype=np.float32)
    return x


def generate(w: Workload, seed: Optional[int] = None) -> Inputs:
    """Draw one layer's inputs for workload ``w`` (seed defaults to w.seed)."""
    if seed is None:
        seed = w.seed
    rng = np.random.Generator(np.random.PCG64(seed))
    B, L, Hq, Hkv, D = w.batch, w.seq_len, w.num_q_heads, w.num_kv_heads, w.head_dim
    offsets = [draw_chunk_lengths(rng, L, w.chunk_law) for _ in range(B)]

    q = np.empty((B, L, Hq, D), dtype=np.uint16)
    k = np.empty((B, L, Hkv, D), dtype=np.uint16)
    v = np.empty((B, L, Hkv, D), dtype=np.uint16)
    qf_keep = []
    kf_keep = []
    for b in range(B):
        o = offsets[b]
        if w.structure == "qkv_centroid":
            qf = _structured(rng, o, Hq, D)
        else:
            qf = rng.standard_normal((L, Hq, D), dtype=np.float32)
        if w.structure in ("qkv_centroid", "kv_centroid"):
            kf = _structured(rng, o, Hkv, D)
            vf = _structured(rng, o, Hkv, D)
        else:
            kf = rng.standard_normal((L, Hkv, D), dtype=np.float32)
            vf = rng.standard_normal((L, Hkv, D), dtype=np.float32)
        v[b] = f32_to_bf16_bits(vf)
        del vf
        qf_keep.append(qf)
        kf_keep.append(kf)

    needles: List[Tuple[int, int, int, int]] = []
    if w.needles:
        G = Hq // Hkv
        for b in range(B):
            o = offsets[b]
            c = len(o) - 1
            used = set()
            pairs = []
            while len(pairs) < w.needles:
                i = int(rng.integers(c // 2, c))
                if i < 2:
                    continue
                j = int(rng.integers(0, i - 1))  # j in [0, i-2]
                if i in used or j in used:
                    continue
                used.update((i, j))
                pairs.append((i, j))
            for (i, j) in pairs:
                ni = int(o[i + 1] - o[i])
                nj = int(o[j + 1] - o[j])
                for g in range(Hkv):
                    nu = rng.standard_normal(D, dtype=np.float32)
                    qf_keep[b][o[i]:o[i + 1], g * G:(g + 1) * G, :] = (
                        nu + np.float32(0.5) * rng.standard_normal((ni, G, D), dtype=np.float32))
                    kf_keep[b][o[j]:o[j + 1], g, :] = (
                        np.float32(4.0) * nu
                        + np.float32(0.5) * rng.standard_normal((nj, D), dtype=np.float32))
                    needles.append((b, i, j, g))

    for b in range(B):
        q[b] = f32_to_bf16_bits(qf_keep[b])
        k[b] = f32_to_bf16_bits(kf_keep[b])
    del qf_keep, kf_keep

    if w.topk is not None:
        topk = int(w.topk)
    else:
        topk = choose_topk([len(o) - 1 for o in offsets], float(w.target_density))
    return Inputs(w, q, k, v, offsets, topk, needles)


def small_workload(name: str, batch: int, seq_len: int, hq: int, hkv: int,
                   law, structure: str = "iid", topk: int = 4, seed: int = 0,
                   needles: int = 0) -> Workload:
    """A parity-test sized workload with the same recipe as the full ones."""
    if isinstance(law, tuple) and len(law) == 2 and isinstance(law[0], int):
        law = ((1.0, law[0], law[1]),)
    return Workload(name, batch, seq_len, hq, hkv, tuple(law), structure,
                    topk=topk, needles=needles, seed=seed)


def row_budgets(num_chunks: Sequence[int], hq: int, topk: int, seed: int,
                lo: int = 1, hi: Optional[int] = None) -> np.ndarray:
    """Synthetic query-dependent row budgets, one per CSR row (sequence b,
    query head h, query chunk i in that order), drawn uniformly from
    [lo, hi] (default [1, 2 * topk - 1], mean topk).  They stand in for the
    output of a trained budget predictor, whose weights are not available."""
    if hi is None:
        hi = 2 * topk - 1
    rng = np.random.Generator(np.random.PCG64([seed, 0xB0D6]))
    total = int(hq * sum(int(c) for c in num_chunks))
    return rng.integers(lo, hi + 1, size=total, dtype=np.int64).astype(np.int32)


def boundary_scores(offsets: Sequence[np.ndarray], seq_len: int, seed: int,
                    spurious_per_token: float = 1.0 / 4000) -> np.ndarray:
    """Synthetic per-token boundary scores [B, L] float32 in [0, 1), standing in
    for a trained boundary predictor's output (no weights are available).

    Background tokens draw U(0, 0.45).  At every chunk start s of `offsets`
    (s > 0) the score peaks at U(0.85, 1.0), and its two neighbours s - 1 and
    s + 1 form shoulders U(0.5, 0.8): above a 0.5 threshold, below the peak.
    Isolated spurious spikes U(0.5, 1.0) appear at `spurious_per_token`."""
    rng = np.random.Generator(np.random.PCG64([seed, 0xB0B]))
    B = len(offsets)
    p = rng.uniform(0.0, 0.45, size=(B, seq_len)).astype(np.float32)
    for b, o in enumerate(offsets):
        starts = np.asarray(o[1:-1], dtype=np.int64)
        for d in (-1, 1):
            nb = starts + d
            nb = nb[(nb > 0) & (nb < seq_len)]
            p[b, nb] = rng.uniform(0.5, 0.8, size=nb.size)
        p[b, starts] = rng.uniform(0.85, 1.0, size=starts.size)
        n_sp = rng.binomial(seq_len, spurious_per_token)
        sp = rng.integers(1, seq_len, size=n_sp)
        p[b, sp] = rng.uniform(0.5, 1.0, size=n_sp)
    return p
