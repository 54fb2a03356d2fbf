"""The Python binding checks every tensor against the chunk offsets before a
call reaches the library: the kernels take the sequence length, the batch
and every row count from the offsets, so a smaller tensor or a CSR built for
another shape would be read past its end.  Each mismatch must raise
ValueError on the host; these tests build CPU tensors and never reach a
library call that touches a device."""
import numpy as np
import pytest

torch = pytest.importorskip("torch")
dhsa = pytest.importorskip("long_context_prefill_segmented_amd.dhsa",
                           reason="libdhsa.so not built")

B, L, HQ, HKV, D = 2, 96, 4, 2, 128
OFFS = [np.array([0, 40, 96], dtype=np.int32), np.array([0, 10, 50, 96], dtype=np.int32)]


def offsets():
    return dhsa.ChunkOffsets.from_list(OFFS, L, device="cpu")


def bf16(*shape):
    return torch.zeros(shape, dtype=torch.bfloat16)


def qkv():
    return bf16(B, L, HQ, D), bf16(B, L, HKV, D), bf16(B, L, HKV, D)


def csr_for(o, hq=HQ, topk=2):
    R, nnz = dhsa.csr_size(o, hq, topk)
    return dhsa.CSR(torch.zeros(R + 1, dtype=torch.int32), torch.zeros(nnz, dtype=torch.int32),
                    nnz)


BAD_QKV = {
    "q short sequence": lambda q, k, v: (bf16(B, L - 1, HQ, D), k, v),
    "q batch": lambda q, k, v: (bf16(B - 1, L, HQ, D), k, v),
    "q heads": lambda q, k, v: (bf16(B, L, HQ + 1, D), k, v),
    "q head dim": lambda q, k, v: (bf16(B, L, HQ, 64), k, v),
    "k heads": lambda q, k, v: (q, bf16(B, L, HKV + 1, D), v),
    "k sequence": lambda q, k, v: (q, bf16(B, L // 2, HKV, D), v),
    "v shape": lambda q, k, v: (q, k, bf16(B, L, HKV, 64)),
    "q dtype": lambda q, k, v: (q.float(), k, v),
    "v dtype": lambda q, k, v: (q, k, v.to(torch.float16)),
    "k not contiguous": lambda q, k, v: (q, bf16(B, HKV, L, D).transpose(1, 2), v),
}


@pytest.mark.parametrize("case", sorted(BAD_QKV))
def test_prefill_rejects(case):
    o = offsets()
    pf = dhsa.Prefill(o, HQ, HKV, device="cpu")
    q, k, v = BAD_QKV[case](*qkv())
    with pytest.raises(ValueError):
        pf(q, k, v, csr_for(o))


@pytest.mark.parametrize("case", sorted(k for k in BAD_QKV if not k.startswith("v")))
def test_mask_builder_rejects(case):
    o = offsets()
    mb = dhsa.MaskBuilder(o, HQ, HKV, 2, device="cpu")
    q, k, _v = BAD_QKV[case](*qkv())
    with pytest.raises(ValueError):
        mb(q, k)


@pytest.mark.parametrize("case", sorted(BAD_QKV))
def test_layer_rejects(case):
    o = offsets()
    layer = dhsa.Layer(o, HQ, HKV, 2, device="cpu")
    q, k, v = BAD_QKV[case](*qkv())
    with pytest.raises(ValueError):
        layer(q, k, v)


def test_prefill_rejects_csr_of_another_shape():
    o = offsets()
    pf = dhsa.Prefill(o, HQ, HKV, device="cpu")
    q, k, v = qkv()
    # row_ptr sized for fewer query heads
    with pytest.raises(ValueError, match="row_ptr"):
        pf(q, k, v, csr_for(o, hq=HQ // 2))
    # col_idx shorter than nnz
    c = csr_for(o)
    short = dhsa.CSR(c.row_ptr, c.col_idx[:-1], c.nnz)
    with pytest.raises(ValueError, match="col_idx"):
        pf(q, k, v, short)
    # row_ptr of the wrong dtype
    bad = dhsa.CSR(c.row_ptr.long(), c.col_idx, c.nnz)
    with pytest.raises(ValueError, match="row_ptr"):
        pf(q, k, v, bad)
    # negative nnz
    with pytest.raises(ValueError):
        pf(q, k, v, dhsa.CSR(c.row_ptr, c.col_idx, -1))


def test_heads_must_divide():
    o = offsets()
    pf = dhsa.Prefill(o, 3, 2, device="cpu")
    with pytest.raises(ValueError, match="multiple"):
        pf(bf16(B, L, 3, D), bf16(B, L, 2, D), bf16(B, L, 2, D), csr_for(o, hq=3))


def test_stage_calls_reject():
    o = offsets()
    # pool: the tensor's batch must be the offsets' batch (host code reads
    # num_chunks[b] for every b < batch)
    with pytest.raises(ValueError, match="shape"):
        dhsa.pool(bf16(B + 1, L, HQ, D), o)
    with pytest.raises(ValueError, match="shape"):
        dhsa.pool(bf16(B, L + 8, HQ, D), o)
    tc = int(o.num_chunks.sum())
    qbar = torch.zeros(HQ * tc, D)
    kbar = torch.zeros(HKV * tc, D)
    with pytest.raises(ValueError, match="qbar"):
        dhsa.chunk_scores(qbar[:-1], kbar, o, HQ, HKV)
    with pytest.raises(ValueError, match="kbar"):
        dhsa.chunk_scores(qbar, kbar[:-1], o, HQ, HKV)
    with pytest.raises(ValueError, match="scores"):
        dhsa.topk_csr(torch.zeros(dhsa.scores_numel(o, HQ) - 1), o, HQ, 2)


def test_tensor_on_another_device_is_rejected():
    """A tensor whose device differs from the offsets' is refused (checked
    here with offsets on the meta device and tensors on the CPU)."""
    o = offsets()
    o_meta = dhsa.ChunkOffsets(o.host, o.num_chunks, o.seq_len,
                               torch.empty(o.host.size, dtype=torch.int32, device="meta"))
    pf = dhsa.Prefill(o, HQ, HKV, device="cpu")
    pf.offsets = o_meta
    q, k, v = qkv()
    with pytest.raises(ValueError, match="device|expected"):
        pf(q, k, v, csr_for(o))
