"""Thin Python binding over libdhsa.so (argument marshalling only).

Every step of the path runs in the library's HIP kernels; this module only
turns torch tensors into device pointers and sizes, allocates outputs and
workspaces with torch (device memory and streams are all torch is used for),
and raises on a non-zero status.  There is no fallback: importing it raises
if the library has not been built.
"""
from __future__ import annotations

import ctypes
import dataclasses
import os
from typing import Optional, Sequence

import numpy as np

# torch ships its own HIP runtime under the same soname as the system one
# (libamdhip64.so.7); loading torch first makes libdhsa.so bind to that
# already-loaded runtime, so the process holds ONE HIP runtime and torch's
# device memory and streams are valid in the library's calls.
import torch  # noqa: E402,F401  (must precede the CDLL below)

# DHSA_LIBRARY may name another build of the same library (e.g. a debug build)
LIB_PATH = os.environ.get("DHSA_LIBRARY") or os.path.join(
    os.path.dirname(os.path.abspath(__file__)), "libdhsa.so")

if not os.path.exists(LIB_PATH):
    raise ImportError(
        f"{LIB_PATH} is not built; run `python -m long_context_prefill_segmented_amd.build_lib`")

# limits of include/dhsa.h (the same #defines; a CPU test keeps them equal)
HEAD_DIM = 128
MAX_BATCH = 64
MAX_CHUNKS = 2048
NMS_MAX_LEN = 524288
NOALLOC_MAX_TILES = 65536

_i32 = ctypes.c_int32
_i64 = ctypes.c_int64
_sz = ctypes.c_size_t
_vp = ctypes.c_void_p
_f32 = ctypes.c_float
_pi32 = ctypes.POINTER(ctypes.c_int32)
_pi64 = ctypes.POINTER(ctypes.c_int64)
_psz = ctypes.POINTER(ctypes.c_size_t)

lib = ctypes.CDLL(LIB_PATH)

_SIGNATURES = {
    "dhsa_status_string": (ctypes.c_char_p, [ctypes.c_int]),
    "dhsa_last_error": (ctypes.c_char_p, []),
    "dhsa_version": (ctypes.c_int, []),
    "dhsa_csr_size": (ctypes.c_int, [_i32, _vp, _i32, _i32, _pi32, _pi64]),
    "dhsa_csr_capacity": (ctypes.c_int, [_i32, _vp, _i32, _i32, _i32, _pi32, _pi64]),
    "dhsa_mask_workspace_size": (ctypes.c_int, [_i32, _vp, _i32, _i32, _i32, _psz]),
    "dhsa_prefill_workspace_size": (ctypes.c_int, [_i32, _i32, _vp, _vp, _psz]),
    "dhsa_build_mask": (ctypes.c_int, [_vp, _vp, _i32, _i32, _i32, _i32, _i32, _vp, _vp, _vp,
                                       _i32, _vp, _vp, _i64, _vp, _vp, _sz, _vp]),
    "dhsa_build_mask_ex": (ctypes.c_int, [_vp, _vp, _i32, _i32, _i32, _i32, _i32, _vp, _vp,
                                          _vp, _i32, _vp, _i32, _vp, _vp, _i64, _vp, _vp, _sz,
                                          _vp]),
    "dhsa_sparse_prefill": (ctypes.c_int, [_vp, _vp, _vp, _i32, _i32, _i32, _i32, _i32, _vp,
                                           _vp, _vp, _vp, _vp, _i64, _f32, _vp, _vp, _vp, _sz,
                                           _vp]),
    "dhsa_sparse_prefill_noalloc": (ctypes.c_int, [_vp, _vp, _vp, _i32, _i32, _i32, _i32, _i32,
                                                   _vp, _vp, _vp, _vp, _vp, _i64, _f32, _vp, _vp,
                                                   _vp]),
    "dhsa_pool": (ctypes.c_int, [_vp, _i32, _i32, _i32, _i32, _vp, _vp, _vp, _vp, _vp]),
    "dhsa_chunk_scores": (ctypes.c_int, [_vp, _vp, _i32, _i32, _i32, _i32, _vp, _vp, _vp]),
    "dhsa_topk_csr": (ctypes.c_int, [_vp, _i32, _i32, _vp, _i32, _vp, _vp, _i64, _vp]),
    "dhsa_topk_csr_ex": (ctypes.c_int, [_vp, _i32, _i32, _vp, _i32, _vp, _i32, _vp, _vp, _i64,
                                        _vp]),
    "dhsa_layer_workspace_size": (ctypes.c_int, [_i32, _i32, _i32, _i32, _i32, _vp, _vp, _i32,
                                                 _i32, _i32, _psz]),
    "dhsa_layer_forward": (ctypes.c_int, [_vp, _vp, _vp, _i32, _i32, _i32, _i32, _i32, _vp, _vp,
                                          _vp, _i32, _vp, _i32, _f32, _vp, _vp, _vp, _sz, _pi32,
                                          _vp]),
    "dhsa_nms_offsets_stride": (ctypes.c_int, [_i32, _i32, _pi32]),
    "dhsa_nms_workspace_size": (ctypes.c_int, [_i32, _i32, _i32, _psz]),
    "dhsa_nms_boundaries": (ctypes.c_int, [_vp, _i32, _i32, _i32, _f32, _vp, _i32, _vp, _vp, _sz,
                                           _vp]),
}
for _name, (_res, _args) in _SIGNATURES.items():
    _fn = getattr(lib, _name)
    _fn.restype = _res
    _fn.argtypes = _args

EXPORTED = tuple(_SIGNATURES)
HEAD_DIM = 128
ALIGN = 256


class DhsaError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(f"{lib.dhsa_status_string(status).decode()}: {message}")
        self.status = status


def check(status: int) -> None:
    if status != 0:
        raise DhsaError(status, lib.dhsa_last_error().decode())


def _np_ptr(a: np.ndarray) -> int:
    return a.ctypes.data


# --------------------------------------------------------------------------
# torch side: device memory and streams
# --------------------------------------------------------------------------


def _torch():
    import torch
    return torch


def _stream_ptr(stream) -> Optional[int]:
    torch = _torch()
    s = stream if stream is not None else torch.cuda.current_stream()
    return s.cuda_stream


def _dptr(t) -> int:
    return t.data_ptr()


@dataclasses.dataclass
class ChunkOffsets:
    """Concatenated chunk offsets: host copy (validation, launch sizes) and a
    device copy with the same values (read by the kernels)."""

    host: np.ndarray          # int32 [sum_b (C_b + 1)]
    num_chunks: np.ndarray    # int32 [B]
    seq_len: int
    device: object            # torch int32 tensor, same values

    @classmethod
    def from_list(cls, offsets: Sequence[np.ndarray], seq_len: int, device="cuda"):
        torch = _torch()
        host = np.ascontiguousarray(np.concatenate([np.asarray(o) for o in offsets]).astype(np.int32))
        nc = np.ascontiguousarray(np.array([len(o) - 1 for o in offsets], dtype=np.int32))
        dev = torch.from_numpy(host.copy()).to(device)
        return cls(host, nc, int(seq_len), dev)

    @property
    def batch(self) -> int:
        return int(self.num_chunks.size)


@dataclasses.dataclass
class CSR:
    row_ptr: object   # torch int32 [R + 1]
    col_idx: object   # torch int32 [nnz]
    nnz: int

    @property
    def num_rows(self) -> int:
        return int(self.row_ptr.numel()) - 1


def csr_size(offsets: ChunkOffsets, num_q_heads: int, topk: int):
    R = _i32()
    nnz = _i64()
    check(lib.dhsa_csr_size(offsets.batch, _np_ptr(offsets.num_chunks), num_q_heads, topk,
                            ctypes.byref(R), ctypes.byref(nnz)))
    return R.value, nnz.value


def csr_capacity(offsets: ChunkOffsets, num_q_heads: int, topk: int, recent: int = 0):
    """(R, nnz bound) when rows keep at most min(topk + recent, i + 1) chunks."""
    R = _i32()
    nnz = _i64()
    check(lib.dhsa_csr_capacity(offsets.batch, _np_ptr(offsets.num_chunks), num_q_heads, topk,
                                recent, ctypes.byref(R), ctypes.byref(nnz)))
    return R.value, nnz.value


def _budgets_ptr(row_budgets, num_rows: int):
    if row_budgets is None:
        return None
    torch = _torch()
    if (row_budgets.dtype != torch.int32 or not row_budgets.is_contiguous()
            or not row_budgets.is_cuda or row_budgets.numel() != num_rows):
        raise ValueError(f"row_budgets must be a contiguous CUDA int32 tensor of {num_rows} rows")
    return _dptr(row_budgets)


def mask_workspace_size(offsets: ChunkOffsets, hq: int, hkv: int) -> int:
    n = _sz()
    check(lib.dhsa_mask_workspace_size(offsets.batch, _np_ptr(offsets.num_chunks), hq, hkv,
                                       HEAD_DIM, ctypes.byref(n)))
    return n.value


def prefill_workspace_size(offsets: ChunkOffsets) -> int:
    n = _sz()
    check(lib.dhsa_prefill_workspace_size(offsets.batch, offsets.seq_len,
                                          _np_ptr(offsets.num_chunks), _np_ptr(offsets.host),
                                          ctypes.byref(n)))
    return n.value


def _workspace(nbytes: int, device):
    torch = _torch()
    return torch.empty(max(nbytes, ALIGN), dtype=torch.uint8, device=device)


def _check_tensor(name, t, shape, dtype, device):
    """Raises ValueError unless t is a contiguous tensor of exactly this
    shape and dtype on this device.  The shape is checked first, so a wrong
    shape is reported whatever device the tensor is on."""
    torch = _torch()
    if not isinstance(t, torch.Tensor):
        raise ValueError(f"{name} must be a torch tensor")
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {tuple(shape)}")
    if t.dtype != dtype:
        raise ValueError(f"{name} has dtype {t.dtype}, expected {dtype}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if t.device != torch.device(device):
        raise ValueError(f"{name} is on {t.device}, expected {device} (the offsets' device)")


def _check_heads(hq: int, hkv: int):
    if hq < 1 or hkv < 1 or hq % hkv != 0:
        raise ValueError(f"num_q_heads {hq} must be a positive multiple of num_kv_heads {hkv}")


def _check_qkv(offsets: "ChunkOffsets", hq: int, hkv: int, q, k, v=None):
    """q [B, L, hq, 128], k and v [B, L, hkv, 128], bf16, contiguous, on the
    offsets' device, B and L those of the offsets: the kernels take the
    sequence length and every row count from the offsets, so a smaller
    tensor would be read past its end."""
    torch = _torch()
    _check_heads(hq, hkv)
    B, L = offsets.batch, offsets.seq_len
    _check_tensor("q", q, (B, L, hq, HEAD_DIM), torch.bfloat16, offsets.device.device)
    _check_tensor("k", k, (B, L, hkv, HEAD_DIM), torch.bfloat16, offsets.device.device)
    if v is not None:
        _check_tensor("v", v, (B, L, hkv, HEAD_DIM), torch.bfloat16, offsets.device.device)


def _check_csr(offsets: "ChunkOffsets", hq: int, csr: "CSR"):
    """row_ptr holds R + 1 entries (R = hq * sum_b C_b), col_idx at least
    max(nnz, 1), both int32 on the offsets' device."""
    torch = _torch()
    R = hq * int(offsets.num_chunks.sum())
    _check_tensor("csr.row_ptr", csr.row_ptr, (R + 1,), torch.int32, offsets.device.device)
    if csr.nnz < 0:
        raise ValueError(f"csr.nnz {csr.nnz} < 0")
    ci = csr.col_idx
    if not isinstance(ci, torch.Tensor) or ci.dim() != 1 or ci.numel() < max(csr.nnz, 1):
        raise ValueError(f"csr.col_idx must be a 1-D tensor of at least {max(csr.nnz, 1)} entries")
    _check_tensor("csr.col_idx", ci, (ci.numel(),), torch.int32, offsets.device.device)


def scores_numel(offsets: ChunkOffsets, num_q_heads: int) -> int:
    return int(sum(num_q_heads * int(c) * int(c) for c in offsets.num_chunks))


class MaskBuilder:
    """Preallocated buffers for repeated mask builds on one shape.

    topk is the row budget (the cap of per-row budgets when row_budgets is
    given to a call); recent is the window of chunks before the diagonal
    that every row keeps.  With recent = 0 and no row budgets this is
    dhsa_build_mask, otherwise dhsa_build_mask_ex.  csr.nnz is the col_idx
    capacity (exact for a single budget; row_ptr[-1] is the exact count)."""

    def __init__(self, offsets: ChunkOffsets, hq: int, hkv: int, topk: int, device="cuda",
                 keep_scores: bool = False, recent: int = 0):
        torch = _torch()
        self.offsets, self.hq, self.hkv, self.topk, self.recent = offsets, hq, hkv, topk, recent
        R, nnz = csr_capacity(offsets, hq, topk, recent)
        self.csr = CSR(torch.empty(R + 1, dtype=torch.int32, device=device),
                       torch.empty(max(nnz, 1), dtype=torch.int32, device=device), nnz)
        self.ws = _workspace(mask_workspace_size(offsets, hq, hkv), device)
        self.scores = (torch.empty(scores_numel(offsets, hq), dtype=torch.float32, device=device)
                       if keep_scores else None)

    def __call__(self, q, k, stream=None, row_budgets=None) -> CSR:
        o = self.offsets
        _check_qkv(o, self.hq, self.hkv, q, k)
        scores = _dptr(self.scores) if self.scores is not None else None
        if row_budgets is None and self.recent == 0:
            check(lib.dhsa_build_mask(
                _dptr(q), _dptr(k), o.batch, o.seq_len, self.hq, self.hkv, HEAD_DIM,
                _np_ptr(o.num_chunks), _np_ptr(o.host), _dptr(o.device), self.topk,
                _dptr(self.csr.row_ptr), _dptr(self.csr.col_idx), self.csr.col_idx.numel(),
                scores, _dptr(self.ws), self.ws.numel(), _stream_ptr(stream)))
        else:
            check(lib.dhsa_build_mask_ex(
                _dptr(q), _dptr(k), o.batch, o.seq_len, self.hq, self.hkv, HEAD_DIM,
                _np_ptr(o.num_chunks), _np_ptr(o.host), _dptr(o.device), self.topk,
                _budgets_ptr(row_budgets, self.csr.num_rows), self.recent,
                _dptr(self.csr.row_ptr), _dptr(self.csr.col_idx), self.csr.col_idx.numel(),
                scores, _dptr(self.ws), self.ws.numel(), _stream_ptr(stream)))
        return self.csr


def build_mask(q, k, offsets: ChunkOffsets, topk: int, return_scores: bool = False,
               stream=None, row_budgets=None, recent: int = 0):
    """dhsa_build_mask(_ex): pooled chunk scores -> causal chunk selection as CSR."""
    if q.dim() != 4 or k.dim() != 4:
        raise ValueError("q and k must be [B, L, H, 128] tensors")
    hq, hkv = int(q.shape[2]), int(k.shape[2])
    mb = MaskBuilder(offsets, hq, hkv, topk, device=q.device, keep_scores=return_scores,
                     recent=recent)
    csr = mb(q, k, stream, row_budgets=row_budgets)
    return (csr, mb.scores) if return_scores else csr


class Prefill:
    """Preallocated buffers for repeated dhsa_sparse_prefill calls on one shape."""

    def __init__(self, offsets: ChunkOffsets, hq: int, hkv: int, device="cuda",
                 with_lse: bool = False, softmax_scale: float = 0.0):
        torch = _torch()
        self.offsets, self.hq, self.hkv = offsets, hq, hkv
        self.scale = float(softmax_scale)
        B, L = offsets.batch, offsets.seq_len
        self.out = torch.empty((B, L, hq, HEAD_DIM), dtype=torch.bfloat16, device=device)
        self.lse = torch.empty((B, hq, L), dtype=torch.float32, device=device) if with_lse else None
        self.ws = _workspace(prefill_workspace_size(offsets), device)

    def __call__(self, q, k, v, csr: CSR, stream=None):
        o = self.offsets
        _check_qkv(o, self.hq, self.hkv, q, k, v)
        _check_csr(o, self.hq, csr)
        check(lib.dhsa_sparse_prefill(
            _dptr(q), _dptr(k), _dptr(v), o.batch, o.seq_len, self.hq, self.hkv, HEAD_DIM,
            _np_ptr(o.num_chunks), _np_ptr(o.host), _dptr(o.device), _dptr(csr.row_ptr),
            _dptr(csr.col_idx), csr.nnz, self.scale, _dptr(self.out),
            _dptr(self.lse) if self.lse is not None else None,
            _dptr(self.ws), self.ws.numel(), _stream_ptr(stream)))
        return (self.out, self.lse) if self.lse is not None else self.out


def sparse_prefill(q, k, v, offsets: ChunkOffsets, csr: CSR, softmax_scale: float = 0.0,
                   return_lse: bool = False, stream=None):
    """dhsa_sparse_prefill: block-sparse causal attention over the kept tiles."""
    if q.dim() != 4 or k.dim() != 4:
        raise ValueError("q, k and v must be [B, L, H, 128] tensors")
    pf = Prefill(offsets, q.shape[2], k.shape[2], device=q.device, with_lse=return_lse,
                 softmax_scale=softmax_scale)
    return pf(q, k, v, csr, stream)


def sparse_prefill_noalloc(q, k, v, offsets: ChunkOffsets, csr: CSR, out, lse=None,
                           softmax_scale: float = 0.0, stream=None):
    """dhsa_sparse_prefill_noalloc into caller-provided out (bf16 [B, L, Hq,
    128]) and optional lse (fp32 [B, Hq, L]): the library's static tile
    array replaces the workspace, so the call allocates nothing."""
    torch = _torch()
    hq, hkv = int(q.shape[2]), int(k.shape[2])
    _check_qkv(offsets, hq, hkv, q, k, v)
    _check_csr(offsets, hq, csr)
    B, L = offsets.batch, offsets.seq_len
    _check_tensor("out", out, (B, L, hq, HEAD_DIM), torch.bfloat16, offsets.device.device)
    if lse is not None:
        _check_tensor("lse", lse, (B, hq, L), torch.float32, offsets.device.device)
    check(lib.dhsa_sparse_prefill_noalloc(
        _dptr(q), _dptr(k), _dptr(v), B, L, hq, hkv, HEAD_DIM, _np_ptr(offsets.num_chunks),
        _np_ptr(offsets.host), _dptr(offsets.device), _dptr(csr.row_ptr), _dptr(csr.col_idx),
        csr.nnz, float(softmax_scale), _dptr(out), _dptr(lse) if lse is not None else None,
        _stream_ptr(stream)))
    return out


def pool(x, offsets: ChunkOffsets, stream=None, out=None):
    """dhsa_pool: fp32 [sum_b H*C_b, 128] pooled chunk representations
    (written into `out` when given)."""
    torch = _torch()
    if x.dim() != 4:
        raise ValueError("x must be a [B, L, H, 128] tensor")
    B, L, H = offsets.batch, offsets.seq_len, int(x.shape[2])
    _check_tensor("x", x, (B, L, H, HEAD_DIM), torch.bfloat16, offsets.device.device)
    shape = (H * int(offsets.num_chunks.sum()), HEAD_DIM)
    if out is None:
        out = torch.empty(shape, dtype=torch.float32, device=x.device)
    _check_tensor("out", out, shape, torch.float32, offsets.device.device)
    check(lib.dhsa_pool(_dptr(x), B, L, H, HEAD_DIM, _np_ptr(offsets.num_chunks),
                        _np_ptr(offsets.host), _dptr(offsets.device), _dptr(out),
                        _stream_ptr(stream)))
    return out


def chunk_scores(qbar, kbar, offsets: ChunkOffsets, hq: int, hkv: int, stream=None, out=None):
    """dhsa_chunk_scores: fp32 per sequence [Hq, C_b, C_b] (j > i untouched: NaN
    in a freshly allocated output; `out`, when given, keeps its values there)."""
    torch = _torch()
    _check_heads(hq, hkv)
    tc = int(offsets.num_chunks.sum())
    _check_tensor("qbar", qbar, (hq * tc, HEAD_DIM), torch.float32, offsets.device.device)
    _check_tensor("kbar", kbar, (hkv * tc, HEAD_DIM), torch.float32, offsets.device.device)
    if out is None:
        out = torch.full((scores_numel(offsets, hq),), float("nan"), dtype=torch.float32,
                         device=qbar.device)
    _check_tensor("out", out, (scores_numel(offsets, hq),), torch.float32,
                  offsets.device.device)
    check(lib.dhsa_chunk_scores(_dptr(qbar), _dptr(kbar), offsets.batch, hq, hkv, HEAD_DIM,
                                _np_ptr(offsets.num_chunks), _dptr(out), _stream_ptr(stream)))
    return out


def topk_csr(scores, offsets: ChunkOffsets, hq: int, topk: int, stream=None,
             row_budgets=None, recent: int = 0, out: Optional[CSR] = None) -> CSR:
    """dhsa_topk_csr(_ex): CSR from given fp32 chunk scores (into `out`, a CSR
    of dhsa_csr_capacity's sizes, when given)."""
    torch = _torch()
    _check_tensor("scores", scores, (scores_numel(offsets, hq),), torch.float32,
                  offsets.device.device)
    R, nnz = csr_capacity(offsets, hq, topk, recent)
    if out is None:
        out = CSR(torch.empty(R + 1, dtype=torch.int32, device=scores.device),
                  torch.empty(max(nnz, 1), dtype=torch.int32, device=scores.device), nnz)
    _check_csr(offsets, hq, out)
    if out.col_idx.numel() < max(nnz, 1):
        raise ValueError(f"out.col_idx holds {out.col_idx.numel()} entries, {nnz} needed")
    csr = out
    if row_budgets is None and recent == 0:
        check(lib.dhsa_topk_csr(_dptr(scores), offsets.batch, hq, _np_ptr(offsets.num_chunks),
                                topk, _dptr(csr.row_ptr), _dptr(csr.col_idx),
                                csr.col_idx.numel(), _stream_ptr(stream)))
    else:
        check(lib.dhsa_topk_csr_ex(_dptr(scores), offsets.batch, hq, _np_ptr(offsets.num_chunks),
                                   topk, _budgets_ptr(row_budgets, R), recent,
                                   _dptr(csr.row_ptr), _dptr(csr.col_idx), csr.col_idx.numel(),
                                   _stream_ptr(stream)))
    return csr


def layer_workspace_size(offsets: ChunkOffsets, hq: int, hkv: int, topk: int, recent: int = 0,
                         max_group: int = 1) -> int:
    n = _sz()
    check(lib.dhsa_layer_workspace_size(offsets.batch, offsets.seq_len, hq, hkv, HEAD_DIM,
                                        _np_ptr(offsets.num_chunks), _np_ptr(offsets.host), topk,
                                        recent, max_group, ctypes.byref(n)))
    return n.value


class Layer:
    """dhsa_layer_forward with a fixed workspace: the whole layer (mask and
    attention) over the batch, in groups of consecutive sequences that fit
    the workspace.  max_group = 1 sizes it for the sequential per-sequence
    loop, max_group = batch for one pass; workspace_bytes overrides both."""

    def __init__(self, offsets: ChunkOffsets, hq: int, hkv: int, topk: int, recent: int = 0,
                 max_group: int = 1, workspace_bytes: Optional[int] = None, device="cuda",
                 with_lse: bool = False, softmax_scale: float = 0.0):
        torch = _torch()
        self.offsets, self.hq, self.hkv, self.topk, self.recent = offsets, hq, hkv, topk, recent
        self.scale = float(softmax_scale)
        if workspace_bytes is None:
            workspace_bytes = layer_workspace_size(offsets, hq, hkv, topk, recent, max_group)
        self.ws = _workspace(workspace_bytes, device)
        B, L = offsets.batch, offsets.seq_len
        self.out = torch.empty((B, L, hq, HEAD_DIM), dtype=torch.bfloat16, device=device)
        self.lse = torch.empty((B, hq, L), dtype=torch.float32, device=device) if with_lse else None
        self.num_groups = 0

    def __call__(self, q, k, v, row_budgets=None, stream=None):
        o = self.offsets
        _check_qkv(o, self.hq, self.hkv, q, k, v)
        R = self.hq * int(o.num_chunks.sum())
        ng = _i32()
        check(lib.dhsa_layer_forward(
            _dptr(q), _dptr(k), _dptr(v), o.batch, o.seq_len, self.hq, self.hkv, HEAD_DIM,
            _np_ptr(o.num_chunks), _np_ptr(o.host), _dptr(o.device), self.topk,
            _budgets_ptr(row_budgets, R), self.recent, self.scale, _dptr(self.out),
            _dptr(self.lse) if self.lse is not None else None, _dptr(self.ws), self.ws.numel(),
            ctypes.byref(ng), _stream_ptr(stream)))
        self.num_groups = ng.value
        return (self.out, self.lse) if self.lse is not None else self.out


class BoundaryNMS:
    """Preallocated buffers for repeated dhsa_nms_boundaries calls on one
    shape: per-token boundary scores [B, L] -> chunk offsets."""

    def __init__(self, batch: int, seq_len: int, min_gap: int, threshold: float, device="cuda"):
        torch = _torch()
        self.batch, self.seq_len, self.min_gap = batch, seq_len, min_gap
        self.threshold = float(threshold)
        st = _i32()
        check(lib.dhsa_nms_offsets_stride(seq_len, min_gap, ctypes.byref(st)))
        self.stride = st.value
        n = _sz()
        check(lib.dhsa_nms_workspace_size(batch, seq_len, min_gap, ctypes.byref(n)))
        self.ws = _workspace(n.value, device)
        self.offsets = torch.empty((batch, self.stride), dtype=torch.int32, device=device)
        self.num_chunks = torch.empty(batch, dtype=torch.int32, device=device)

    def __call__(self, scores, stream=None):
        torch = _torch()
        if (scores.dtype != torch.float32 or not scores.is_contiguous() or not scores.is_cuda
                or tuple(scores.shape) != (self.batch, self.seq_len)):
            raise ValueError(f"scores must be contiguous CUDA float32 [{self.batch}, {self.seq_len}]")
        check(lib.dhsa_nms_boundaries(_dptr(scores), self.batch, self.seq_len, self.min_gap,
                                      self.threshold, _dptr(self.offsets), self.stride,
                                      _dptr(self.num_chunks), _dptr(self.ws), self.ws.numel(),
                                      _stream_ptr(stream)))
        return self.offsets, self.num_chunks

    def to_chunk_offsets(self, device="cuda") -> "ChunkOffsets":
        """Copies the last result to the host (synchronising) as ChunkOffsets."""
        nc = self.num_chunks.cpu().numpy()
        offs = self.offsets.cpu().numpy()
        return ChunkOffsets.from_list([offs[b, :int(nc[b]) + 1] for b in range(self.batch)],
                                      self.seq_len, device=device)


def nms_boundaries(scores, min_gap: int, threshold: float, stream=None):
    """dhsa_nms_boundaries: returns (offsets [B, stride], num_chunks [B]) on the device."""
    B, L = scores.shape
    return BoundaryNMS(B, L, min_gap, threshold, device=scores.device)(scores, stream)


def csr_from_host(row_ptr: np.ndarray, col_idx: np.ndarray, device="cuda") -> CSR:
    """Uploads a CSR built elsewhere (e.g. a reference mask) for dhsa_sparse_prefill."""
    torch = _torch()
    rp = torch.from_numpy(np.ascontiguousarray(row_ptr, dtype=np.int32)).to(device)
    ci = torch.from_numpy(np.ascontiguousarray(col_idx, dtype=np.int32))
    nnz = int(ci.numel())
    if nnz == 0:
        ci = torch.zeros(1, dtype=torch.int32)
    return CSR(rp, ci.to(device), nnz)


def bf16_from_bits(bits: np.ndarray, device="cuda"):
    """uint16 bf16 bit patterns -> CUDA bfloat16 tensor (same bits)."""
    torch = _torch()
    t = torch.from_numpy(np.ascontiguousarray(bits).view(np.int16))
    return t.to(device).view(torch.bfloat16)
