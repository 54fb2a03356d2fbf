"""Property tests of the host-only size queries of the C ABI (no GPU): for
random batches of chunk layouts, heads, budgets and windows, each query
either returns DHSA_OK with the closed-form size, or the documented error
when an argument breaks a documented rule."""
import ctypes

import numpy as np
import pytest

hypothesis = pytest.importorskip("hypothesis")
from hypothesis import given, settings, strategies as stg  # noqa: E402

dhsa = pytest.importorskip("long_context_prefill_segmented_amd.dhsa",
                           reason="libdhsa.so not built")
lib = dhsa.lib

OK, ESHAPE, EOFF, ETOPK, EUNSUP = 0, -2, -3, -4, -7


def arr(x):
    return np.ascontiguousarray(np.asarray(x, dtype=np.int32))


def align(x):
    return (x + 255) // 256 * 256


layouts = stg.lists(stg.lists(stg.integers(1, 700), min_size=1, max_size=40),
                    min_size=1, max_size=6)


@settings(max_examples=300, deadline=None)
@given(layouts, stg.integers(-1, 40), stg.integers(-2, 30), stg.integers(-1, 64))
def test_csr_capacity(lens, topk, recent, hq):
    nc = arr([len(x) for x in lens])
    R, N = ctypes.c_int32(), ctypes.c_int64()
    st = lib.dhsa_csr_capacity(nc.size, nc.ctypes.data, hq, topk, recent, ctypes.byref(R),
                               ctypes.byref(N))
    if hq < 1:
        assert st == ESHAPE
    elif topk < 1 or recent < 0:
        assert st == ETOPK
    else:
        assert st == OK
        assert R.value == hq * int(nc.sum())
        assert N.value == hq * sum(sum(min(topk + recent, i + 1) for i in range(c)) for c in nc)


@settings(max_examples=300, deadline=None)
@given(layouts, stg.integers(0, 3))
def test_prefill_workspace_and_offset_validation(lens, corrupt):
    # per sequence: offsets 0, cumulative lengths; all sequences padded to a
    # common seq_len by lengthening their last chunk
    L = max(sum(x) for x in lens)
    offs, nc = [], []
    for x in lens:
        x = list(x)
        x[-1] += L - sum(x)
        offs += [0] + list(np.cumsum(x))
        nc.append(len(x))
    tiles = sum((n + 127) // 128 for x in lens for n in (list(x[:-1]) + [x[-1] + L - sum(x)]))
    if corrupt == 1:       # a repeated offset: not strictly increasing
        if len(offs) > 2:
            offs[1] = offs[0]
    elif corrupt == 2:     # the last offset of a sequence misses seq_len
        offs[-1] -= 1 if offs[-1] - 1 > offs[-2] else -1
    o, c = arr(offs), arr(nc)
    n = ctypes.c_size_t()
    st = lib.dhsa_prefill_workspace_size(c.size, L, c.ctypes.data, o.ctypes.data, ctypes.byref(n))
    bad = (corrupt == 1 and len(offs) > 2) or corrupt == 2
    if bad:
        assert st == EOFF
    else:
        assert st == OK
        assert n.value == align(16 * tiles)


@settings(max_examples=200, deadline=None)
@given(layouts, stg.sampled_from([(8, 2), (4, 4), (2, 1), (32, 8)]))
def test_mask_workspace(lens, heads):
    hq, hkv = heads
    nc = arr([len(x) for x in lens])
    n = ctypes.c_size_t()
    assert lib.dhsa_mask_workspace_size(nc.size, nc.ctypes.data, hq, hkv, 128,
                                        ctypes.byref(n)) == OK
    tc = int(nc.sum())
    want = (align(hq * tc * 512) + align(hkv * tc * 512)
            + align(4 * hq * int((nc.astype(np.int64) ** 2).sum())) + align(4 * tc))
    assert n.value == want
    assert lib.dhsa_mask_workspace_size(nc.size, nc.ctypes.data, hq, hkv, 64,
                                        ctypes.byref(n)) == ESHAPE
    assert lib.dhsa_mask_workspace_size(nc.size, nc.ctypes.data, hq + 1, hkv, 128,
                                        ctypes.byref(n)) == (OK if (hq + 1) % hkv == 0 else ESHAPE)


@settings(max_examples=300, deadline=None)
@given(stg.integers(-3, 600000), stg.integers(-2, 5000))
def test_nms_stride(L, g):
    s = ctypes.c_int32()
    st = lib.dhsa_nms_offsets_stride(L, g, ctypes.byref(s))
    # checked in this order: length, length limit, window
    if L < 1:
        assert st == ESHAPE
    elif L > dhsa.NMS_MAX_LEN:
        assert st == EUNSUP
    elif g < 1:
        assert st == ESHAPE
    else:
        assert st == OK
        assert s.value == max(L // g, 1) + 1
