"""Concurrent use of the library: two host threads drive two independent
layers (mask construction + sparse attention) on two HIP streams at once.
The library keeps no state between calls besides a thread-local error
message, so every output must equal, bit for bit, the same layer run alone
on the default stream."""
import sys
import threading

import numpy as np
import pytest

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

if not torch.cuda.is_available():  # pragma: no cover
    pytest.skip("needs a GPU", allow_module_level=True)

from long_context_prefill_segmented_amd import dhsa, synth  # noqa: E402


def say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def make_layer(seed):
    w = synth.small_workload(f"streams_{seed}", 2, 8192, 8, 2, (64, 512), "iid", topk=6,
                             seed=seed)
    x = synth.generate(w)
    offs = dhsa.ChunkOffsets.from_list(x.offsets, w.seq_len)
    q, k, v = (dhsa.bf16_from_bits(a) for a in (x.q, x.k, x.v))
    return dict(offs=offs, q=q, k=k, v=v, hq=w.num_q_heads, hkv=w.num_kv_heads, topk=x.topk)


def run_layer(L, stream, reps):
    mb = dhsa.MaskBuilder(L["offs"], L["hq"], L["hkv"], L["topk"], device="cuda")
    pf = dhsa.Prefill(L["offs"], L["hq"], L["hkv"], device="cuda", with_lse=True)
    torch.cuda.synchronize()  # buffers exist before another stream uses them
    for _ in range(reps):
        csr = mb(L["q"], L["k"], stream=stream)
        out, lse = pf(L["q"], L["k"], L["v"], csr, stream=stream)
    return csr, out, lse


def test_two_threads_two_streams_match_sequential_runs():
    layers = [make_layer(41), make_layer(42)]
    torch.cuda.synchronize()
    say("  sequential reference runs")
    ref = []
    for L in layers:
        csr, out, lse = run_layer(L, None, 1)
        torch.cuda.synchronize()
        ref.append((csr.row_ptr.clone(), csr.col_idx.clone(), out.clone(), lse.clone()))
    streams = [torch.cuda.Stream(), torch.cuda.Stream()]  # default priority
    results = [None, None]
    errors = []

    def worker(i):
        try:
            results[i] = run_layer(layers[i], streams[i], 4)
        except Exception as e:  # pragma: no cover - reported below
            errors.append(repr(e))

    say("  two threads, two streams, four layers each")
    threads = [threading.Thread(target=worker, args=(i,)) for i in range(2)]
    for t in threads:
        t.start()
    for t in threads:
        t.join(timeout=120)
    torch.cuda.synchronize()
    assert not errors, errors
    for i in range(2):
        csr, out, lse = results[i]
        rp, ci, o_ref, l_ref = ref[i]
        assert torch.equal(csr.row_ptr, rp)
        n = int(rp[-1])
        assert torch.equal(csr.col_idx[:n], ci[:n])
        assert torch.equal(out, o_ref)
        assert torch.equal(torch.nan_to_num(lse, neginf=-1e30), torch.nan_to_num(l_ref, neginf=-1e30))
    assert not torch.equal(ref[0][2][:, :1000], ref[1][2][:, :1000])  # the two layers differ
