"""dhsa_sparse_prefill_noalloc through the C ABI: its output and LSE equal
dhsa_sparse_prefill's bit for bit on two calls in a row, the second with a
smaller problem (the static tile array keeps the first call's contents; the
second call must not read them), for both query-tile heights."""
import ctypes
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


def _inputs(w):
    x = synth.generate(w)
    offs = dhsa.ChunkOffsets.from_list(x.offsets, w.seq_len)
    q, k, v = (dhsa.bf16_from_bits(a) for a in (x.q, x.k, x.v))
    csr = dhsa.build_mask(q, k, offs, x.topk)
    return x, offs, q, k, v, csr


def _noalloc_call(w, offs, q, k, v, csr, out, lse):
    """The C entry point itself (ctypes), no binding logic in between."""
    st = dhsa.lib.dhsa_sparse_prefill_noalloc(
        q.data_ptr(), k.data_ptr(), v.data_ptr(), w.batch, w.seq_len, w.num_q_heads,
        w.num_kv_heads, 128, offs.num_chunks.ctypes.data, offs.host.ctypes.data,
        offs.device.data_ptr(), csr.row_ptr.data_ptr(), csr.col_idx.data_ptr(), csr.nnz,
        ctypes.c_float(0.0), out.data_ptr(), lse.data_ptr(),
        torch.cuda.current_stream().cuda_stream)
    assert st == 0, dhsa.lib.dhsa_last_error()


@pytest.mark.parametrize("block_m", ["256", "128"])
def test_noalloc_equals_workspace_call_twice(block_m, monkeypatch):
    monkeypatch.setenv("DHSA_ATTN_BLOCK_M", block_m)
    big = synth.small_workload("noalloc_big", 2, 6144, 8, 2,
                               ((0.6, 8, 40), (0.3, 64, 300), (0.1, 400, 900)), "iid", topk=6,
                               seed=51)
    small = synth.WORKLOADS["tiny_1k"]
    for trial, w in enumerate((big, small)):
        say(f"[noalloc] call {trial + 1}: {w.name} B={w.batch} L={w.seq_len} Hq={w.num_q_heads}")
        x, offs, q, k, v, csr = _inputs(w)
        ref_out, ref_lse = dhsa.sparse_prefill(q, k, v, offs, csr, return_lse=True)
        out = torch.full_like(ref_out, float("nan"))
        lse = torch.full_like(ref_lse, float("nan"))
        _noalloc_call(w, offs, q, k, v, csr, out, lse)
        torch.cuda.synchronize()
        assert torch.equal(out.view(torch.int16), ref_out.view(torch.int16))
        assert torch.equal(lse.view(torch.int32), ref_lse.view(torch.int32))
        # and within the attention bar of the oracle (first sequence)
        qf, kf, vf = (orc.widen_bf16(a[0]) for a in (x.q, x.k, x.v))
        rows = orc.csr_to_rows(csr.row_ptr.cpu().numpy(), csr.col_idx.cpu().numpy()[:csr.nnz],
                               offs.num_chunks, w.num_q_heads)[0]
        O_ref, _ = orc.sparse_prefill(qf, kf, vf, x.offsets[0], rows)
        got = orc.widen_bf16(out.view(torch.int16).cpu().numpy().view(np.uint16))[0]
        assert np.all(np.abs(got - O_ref) <= 1e-2 + 1e-2 * np.abs(O_ref))


def test_noalloc_binding_wrapper():
    w = synth.WORKLOADS["tiny_1k"]
    x, offs, q, k, v, csr = _inputs(w)
    ref = dhsa.sparse_prefill(q, k, v, offs, csr)
    out = torch.empty_like(ref)
    dhsa.sparse_prefill_noalloc(q, k, v, offs, csr, out)
    torch.cuda.synchronize()
    assert torch.equal(out.view(torch.int16), ref.view(torch.int16))
