"""CPU oracle for the DHSA prefill path -- TEST INFRASTRUCTURE ONLY.

Only ``tests/``, ``__graft_entry__.smoke()`` and ``bench.py``'s cpu_baseline
leg may import or run anything in this package.  The product path never
calls it and shares no code with it: the only thing both sides consume is the
seeded input generator, which holds none of the method's arithmetic.

Everything here is the plain definition, in NumPy float64, with no blocking,
fusion or reordering beyond what the definition states:

* pooling      -- chunk mean scaled by sqrt(chunk length)
                  (OpenReview abstract "...for On-Device LLMs": length-normalised
                  aggregation scales the averaged embeddings by the square root
                  of the chunk size; gist.science Technical Summary,
                  Methodology, "Robust Chunk Representation": prefix sums of
                  embeddings divided by the actual chunk length, then length
                  normalisation);
* chunk scores -- dot products of pooled query and key chunks
                  (Technical Summary, Methodology, Step 1: chunk-level
                  similarity matrix);
* selection    -- per query chunk, the highest-scoring key chunks under the
                  causal constraint, expanded to their tokens (Technical
                  Summary, Methodology, Step 2; OpenReview abstract:
                  chunk scores upsampled to token level; DHSA README,
                  "Predictor Checkpoints": a fixed row budget);
* boundaries   -- greedy non-maximum suppression of per-token boundary
                  scores into well-separated chunk offsets (Technical
                  Summary, Methodology, "Dynamic Boundary Detection": the
                  predictor finalises boundaries with NMS so that they are
                  well separated and robust to noise);
* attention    -- dense softmax attention restricted to the token mask
                  (Technical Summary, "Hardware-Agnostic Backends": the SDPA
                  backend is dense masked attention; the tiled backend is its
                  streaming form).

Readings where the pages are silent (each also listed with the design notes):
pooling is sum / sqrt(n) (= mean * sqrt(n)); scores carry no 1/sqrt(d); the
mask is per query head with K taken from KV head h // (Hq / Hkv); a row keeps
min(k, i + 1) chunks: the diagonal chunk plus the k - 1 best earlier ones;
ties go to the lowest chunk index and -0 == +0; inside the diagonal chunk the
mask is token-causal (s <= t); the softmax scale defaults to 1/sqrt(128).

Parity status: every function here is pinned by tests under ``tests/``
(closed forms, brute force, library dense attention, invariants); none is
"parity unpinned".
"""
from __future__ import annotations

import math
from typing import List, Optional, Sequence, Tuple

import numpy as np

# --------------------------------------------------------------------------
# inputs
# --------------------------------------------------------------------------


def widen_bf16(bits: np.ndarray) -> np.ndarray:
    """bf16 bit patterns (uint16) -> float64, exactly."""
    return (bits.astype(np.uint32) << np.uint32(16)).view(np.float32).astype(np.float64)


def check_offsets(offsets: Sequence[int], seq_len: int) -> np.ndarray:
    """Chunk offsets must start at 0, increase strictly and end at L."""
    o = np.asarray(offsets, dtype=np.int64)
    if o.ndim != 1 or o.size < 2:
        raise ValueError("offsets need at least two entries")
    if o[0] != 0 or o[-1] != seq_len:
        raise ValueError("offsets must start at 0 and end at seq_len")
    if np.any(np.diff(o) <= 0):
        raise ValueError("offsets must increase strictly (no empty chunk)")
    return o


def chunk_of_token(offsets: np.ndarray) -> np.ndarray:
    """Index of the chunk that holds each token."""
    o = np.asarray(offsets, dtype=np.int64)
    return np.repeat(np.arange(o.size - 1), np.diff(o))


# --------------------------------------------------------------------------
# stage 1: length-normalised pooling
# --------------------------------------------------------------------------


def pool_chunks(x: np.ndarray, offsets: Sequence[int]) -> np.ndarray:
    """Pooled chunk representation: mean of the chunk's tokens times sqrt(n).

    x: [L, H, D] float64 (one sequence).  Returns [H, C, D] float64.
    """
    o = check_offsets(offsets, x.shape[0])
    C = o.size - 1
    out = np.empty((x.shape[1], C, x.shape[2]), dtype=np.float64)
    for c in range(C):
        n = int(o[c + 1] - o[c])
        mean = x[o[c]:o[c + 1]].sum(axis=0) / n
        out[:, c, :] = mean * math.sqrt(n)
    return out


def pool_chunks_prefix(x: np.ndarray, offsets: Sequence[int]) -> np.ndarray:
    """The same pooling written as the explainer describes it: prefix sums of
    the embeddings, differenced at the chunk boundaries, divided by the actual
    chunk length, then scaled by sqrt(length)."""
    o = check_offsets(offsets, x.shape[0])
    P = np.zeros((x.shape[0] + 1,) + x.shape[1:], dtype=np.float64)
    np.cumsum(x, axis=0, out=P[1:])
    n = np.diff(o).astype(np.float64)
    seg = P[o[1:]] - P[o[:-1]]                     # [C, H, D]
    pooled = seg / n[:, None, None] * np.sqrt(n)[:, None, None]
    return np.transpose(pooled, (1, 0, 2)).copy()


# --------------------------------------------------------------------------
# stage 2: chunk-by-chunk similarity
# --------------------------------------------------------------------------


def chunk_scores(qbar: np.ndarray, kbar: np.ndarray) -> np.ndarray:
    """S[h, i, j] = qbar[h, i] . kbar[h // G, j] for j <= i; NaN above.

    qbar: [Hq, C, D], kbar: [Hkv, C, D].  Returns [Hq, C, C] float64.
    """
    Hq, C, _ = qbar.shape
    Hkv = kbar.shape[0]
    if Hq % Hkv:
        raise ValueError("Hq must be a multiple of Hkv")
    G = Hq // Hkv
    S = np.full((Hq, C, C), np.nan, dtype=np.float64)
    lower = np.tril(np.ones((C, C), dtype=bool))
    for h in range(Hq):
        full = qbar[h] @ kbar[h // G].T
        S[h][lower] = full[lower]
    return S


# --------------------------------------------------------------------------
# stage 3: causal top-k per query chunk
# --------------------------------------------------------------------------


def select_row(scores_row: np.ndarray, i: int, k: int) -> List[int]:
    """Kept key chunks of query chunk i, ascending.

    Keeps every chunk 0..i when i + 1 <= k; otherwise the diagonal chunk i
    plus the k - 1 earlier chunks that come first under the order
    "score descending, then index ascending" (-0 and +0 compare equal).
    """
    if k < 1:
        raise ValueError("topk must be >= 1")
    if i + 1 <= k:
        return list(range(i + 1))
    cand = np.asarray(scores_row[:i], dtype=np.float64)
    if not np.all(np.isfinite(cand)):
        raise ValueError("scores must be finite")
    j = np.arange(i)
    order = np.lexsort((j, -cand))   # primary: -score, secondary: j
    keep = sorted(int(x) for x in order[:k - 1])
    return keep + [i]


def select_row_ex(scores_row: np.ndarray, i: int, budget: int, recent: int) -> List[int]:
    """Kept chunks of query chunk i with a row budget and a recent window.

    The row keeps chunk i, the `recent` chunks just before it and the
    budget - 1 best-scoring chunks among the older ones (j < i - recent),
    under the same order as select_row; when i + 1 <= budget + recent it
    keeps every chunk 0..i.  Readings of the pages: the README's dynamic
    predictors use query-dependent row budgets ("Predictor Checkpoints"), and
    the codewithpapers record names a recent-key-block keep OR'ed with a
    scattered top-k by row budget; the pages give no formula, so this is the
    plainest rule consistent with both.  With recent = 0 it is select_row.
    """
    if budget < 1 or recent < 0:
        raise ValueError("budget must be >= 1 and recent >= 0")
    if i + 1 <= budget + recent:
        return list(range(i + 1))
    older = i - recent  # candidates j < older
    cand = np.asarray(scores_row[:older], dtype=np.float64)
    if not np.all(np.isfinite(cand)):
        raise ValueError("scores must be finite")
    j = np.arange(older)
    order = np.lexsort((j, -cand))
    keep = sorted(int(x) for x in order[:budget - 1])
    return keep + list(range(older, i + 1))


def select_topk(scores: np.ndarray, k: int) -> List[List[List[int]]]:
    """rows[h][i] for one sequence; scores [Hq, C, C] (lower triangle read)."""
    Hq, C, _ = scores.shape
    return [[select_row(scores[h, i], i, k) for i in range(C)] for h in range(Hq)]


def select_topk_ex(scores: np.ndarray, budgets: np.ndarray, recent: int
                   ) -> List[List[List[int]]]:
    """rows[h][i] with a budget per row (budgets [Hq, C]) and a recent window."""
    Hq, C, _ = scores.shape
    return [[select_row_ex(scores[h, i], i, int(budgets[h, i]), recent) for i in range(C)]
            for h in range(Hq)]


def rows_to_csr(rows_per_seq: Sequence[Sequence[Sequence[Sequence[int]]]]
                ) -> Tuple[np.ndarray, np.ndarray]:
    """CSR over rows r = rowbase_b + h * C_b + i (row order: b, h, i)."""
    counts: List[int] = []
    cols: List[int] = []
    for rows in rows_per_seq:
        for per_head in rows:
            for row in per_head:
                counts.append(len(row))
                cols.extend(row)
    row_ptr = np.zeros(len(counts) + 1, dtype=np.int64)
    row_ptr[1:] = np.cumsum(counts)
    return row_ptr.astype(np.int32), np.asarray(cols, dtype=np.int32)


def csr_to_rows(row_ptr: np.ndarray, col_idx: np.ndarray, num_chunks: Sequence[int],
                num_q_heads: int) -> List[List[List[List[int]]]]:
    """Inverse of rows_to_csr."""
    out = []
    r = 0
    for C in num_chunks:
        seq = []
        for _h in range(num_q_heads):
            per_head = []
            for _i in range(C):
                per_head.append([int(x) for x in col_idx[row_ptr[r]:row_ptr[r + 1]]])
                r += 1
            seq.append(per_head)
        out.append(seq)
    return out


# --------------------------------------------------------------------------
# token-level mask and attention
# --------------------------------------------------------------------------


def token_mask(offsets: Sequence[int], rows_h: Sequence[Sequence[int]]) -> np.ndarray:
    """Token t may attend token s iff chunk(s) is kept for chunk(t) and s <= t."""
    o = np.asarray(offsets, dtype=np.int64)
    L = int(o[-1])
    cid = chunk_of_token(o)
    C = o.size - 1
    keep = np.zeros((C, C), dtype=bool)
    for i, row in enumerate(rows_h):
        keep[i, list(row)] = True
    M = keep[cid[:, None], cid[None, :]]
    M &= np.tril(np.ones((L, L), dtype=bool))
    return M


def dense_masked_attention(q: np.ndarray, k: np.ndarray, v: np.ndarray,
                           mask: np.ndarray, scale: float
                           ) -> Tuple[np.ndarray, np.ndarray]:
    """Literal softmax(scale * q k^T over the mask) v in float64.

    q, k, v: [L, D]; mask: [L, L] bool.  Rows with no visible key give 0 and
    log-sum-exp -inf.
    """
    z = scale * (q @ k.T)
    z = np.where(mask, z, -np.inf)
    m = z.max(axis=1, keepdims=True)
    safe_m = np.where(np.isfinite(m), m, 0.0)
    w = np.exp(z - safe_m)
    l = w.sum(axis=1, keepdims=True)
    with np.errstate(invalid="ignore", divide="ignore"):
        o = np.where(l > 0, (w @ v) / np.where(l > 0, l, 1.0), 0.0)
        lse = np.where(l[:, 0] > 0, safe_m[:, 0] + np.log(l[:, 0]), -np.inf)
    return o, lse


def chunk_attention(q: np.ndarray, k: np.ndarray, v: np.ndarray,
                    offsets: Sequence[int], row: Sequence[int], i: int,
                    h: int, g: int, scale: float
                    ) -> Tuple[np.ndarray, np.ndarray]:
    """Attention of the query tokens of chunk i (head h) over the kept keys.

    Gathers the tokens of the kept chunks of KV head g; masked pairs are
    exactly the ones outside this gather or with s > t, whose softmax weight
    is exp(-inf) = 0, so this equals the dense masked form.
    q: [L, Hq, D]; k, v: [L, Hkv, D] (float64).  Returns ([n_i, D], [n_i]).
    """
    o = np.asarray(offsets, dtype=np.int64)
    t = np.arange(o[i], o[i + 1])
    s = np.concatenate([np.arange(o[j], o[j + 1]) for j in row]) if len(row) else \
        np.zeros(0, dtype=np.int64)
    mask = s[None, :] <= t[:, None]
    if s.size == 0:
        return np.zeros((t.size, q.shape[2])), np.full(t.size, -np.inf)
    return dense_masked_attention(q[t, h], k[s, g], v[s, g], mask, scale)


def sparse_prefill(q: np.ndarray, k: np.ndarray, v: np.ndarray,
                   offsets: Sequence[int], rows: Sequence[Sequence[Sequence[int]]],
                   scale: Optional[float] = None,
                   heads: Optional[Sequence[int]] = None,
                   chunks: Optional[Sequence[int]] = None
                   ) -> Tuple[np.ndarray, np.ndarray]:
    """Masked attention for one sequence; q [L,Hq,D], k/v [L,Hkv,D] float64.

    Returns O [L, Hq, D] and lse [Hq, L]; entries of heads/chunks not asked
    for are NaN.
    """
    L, Hq, D = q.shape
    G = Hq // k.shape[1]
    if scale is None:
        scale = 1.0 / math.sqrt(D)
    o = np.asarray(offsets, dtype=np.int64)
    C = o.size - 1
    O = np.full((L, Hq, D), np.nan)
    lse = np.full((Hq, L), np.nan)
    for h in (range(Hq) if heads is None else heads):
        for i in (range(C) if chunks is None else chunks):
            oi, li = chunk_attention(q, k, v, o, rows[h][i], i, h, h // G, scale)
            O[o[i]:o[i + 1], h] = oi
            lse[h, o[i]:o[i + 1]] = li
    return O, lse


# --------------------------------------------------------------------------
# the whole path for one layer
# --------------------------------------------------------------------------


def build_mask(q: np.ndarray, k: np.ndarray, offsets: Sequence[int], topk: int):
    """Pool, score and select for one sequence (float64 inputs).

    Returns (qbar, kbar, scores64, scores32, rows): the selection runs on the
    scores rounded to float32, the precision the GPU path selects in.
    """
    qbar = pool_chunks(q, offsets)
    kbar = pool_chunks(k, offsets)
    s64 = chunk_scores(qbar, kbar)
    s32 = s64.astype(np.float32)
    rows = select_topk(s32, topk)
    return qbar, kbar, s64, s32, rows


# --------------------------------------------------------------------------
# stage 0: boundary finalisation (NMS)
# --------------------------------------------------------------------------


def nms_boundaries(p: np.ndarray, min_gap: int, threshold: float) -> np.ndarray:
    """Chunk offsets of one sequence from per-token boundary scores.

    p[t] scores "a new chunk starts at token t" (t = 0 .. L-1).  Readings
    where the pages are silent: the sequence ends 0 and L are boundaries
    that are always kept; a candidate is a token t with p[t] >= threshold
    (NaN never is); candidates are visited by score descending, then token
    ascending, and one is kept when every kept boundary, the two ends
    included, lies at least min_gap tokens away.  Every chunk then holds at
    least min_gap tokens.  Returns int64 [0, kept ascending..., L].
    """
    p = np.asarray(p, dtype=np.float64)
    L = p.size
    if min_gap < 1:
        raise ValueError("min_gap must be >= 1")
    if L < 1:
        raise ValueError("empty sequence")
    t = np.arange(L)
    cand = t[(p >= threshold) & (t >= min_gap) & (t <= L - min_gap)]
    order = cand[np.lexsort((cand, -p[cand]))]
    kept = [0, L]
    taken = np.zeros(L + 1, dtype=bool)
    taken[0] = taken[L] = True
    for c in order:
        lo, hi = max(0, c - min_gap + 1), min(L, c + min_gap - 1)
        if not taken[lo:hi + 1].any():
            taken[c] = True
            kept.append(int(c))
    return np.array(sorted(kept), dtype=np.int64)
