"""Python binding of libisa, the MI355X IndexShare sparse-attention library.

Argument marshalling only: every step of the computation runs in the HIP
kernels behind the C ABI declared in include/isa.h.  PyTorch provides device
memory and the current stream.  The names mirror the C entry points.

If libisa.so has not been built, every call raises: there is no fallback.
Build it with ``python -m long_context_sparse_indexshare_amd.build``.
"""
from __future__ import annotations

import ctypes
import os
from typing import List, Optional, Sequence, Tuple

import torch

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libisa.so")
ISA_ABI_VERSION = 3
ISA_MAX_TOPK = 2048

ISA_OK = 0
ISA_ERR_INVALID_ARG = -1
ISA_ERR_UNSUPPORTED = -2
ISA_ERR_WORKSPACE = -3
ISA_ERR_HIP = -4

EXPORTED_SYMBOLS = (
    "isa_abi_version", "isa_last_error", "isa_indexer_scores", "isa_topk_workspace_bytes",
    "isa_topk_select", "isa_attend_workspace_bytes", "isa_sparse_mla_attend",
    "isa_attend_fp8_workspace_bytes", "isa_sparse_mla_attend_fp8", "isa_index_histogram",
    "isa_indexer_scores_paged", "isa_sparse_mla_attend_paged",
    "isa_group_workspace_bytes", "isa_group_forward",
    "isa_group_noalloc_max_bytes", "isa_group_forward_noalloc",
)


class IsaError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(f"isa status {status}: {message}")
        self.status = status


_P = ctypes.c_void_p
_I = ctypes.c_int
_F = ctypes.c_float
_Z = ctypes.c_size_t


class GroupArgs(ctypes.Structure):
    """Mirror of isa_group_args."""
    _fields_ = [
        ("B", _I), ("Tq", _I), ("L_cap", _I),
        ("H_I", _I), ("D_I", _I), ("k", _I),
        ("H", _I), ("D", _I), ("D_v", _I),
        ("n_layers", _I), ("sm_scale", _F),
        ("qI", _P), ("w", _P), ("kI", _P), ("kv_len", _P),
        ("Q", _P), ("C", _P), ("out", _P), ("lse", _P),
        ("idx", _P), ("reuse_idx", _I), ("per_layer_indexer", _I),
        ("ws", _P), ("ws_bytes", _Z),
        ("kv_fp8", _I), ("C8", _P), ("Ce", _P), ("Cr", _P),
        ("paged", _I), ("block_table", _P), ("max_blocks", _I), ("block_size", _I),
        ("n_pages", _I),
    ]


_lib = None


def load_library():
    """Loads libisa.so; raises if it is missing or its ABI does not match."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(f"{LIB_PATH} is missing; build it with "
                           "`python -m long_context_sparse_indexshare_amd.build`")
    lib = ctypes.CDLL(LIB_PATH)
    lib.isa_abi_version.restype = _I
    lib.isa_abi_version.argtypes = []
    lib.isa_last_error.restype = ctypes.c_char_p
    lib.isa_last_error.argtypes = []
    lib.isa_indexer_scores.restype = _I
    lib.isa_indexer_scores.argtypes = [_P, _P, _P, _P, _I, _I, _I, _I, _I, _P, _P]
    lib.isa_topk_workspace_bytes.restype = _Z
    lib.isa_topk_workspace_bytes.argtypes = [_I, _I, _I, _I]
    lib.isa_topk_select.restype = _I
    lib.isa_topk_select.argtypes = [_P, _P, _I, _I, _I, _I, _P, _P, _Z, _P]
    lib.isa_attend_workspace_bytes.restype = _Z
    lib.isa_attend_workspace_bytes.argtypes = [_I, _I, _I, _I, _I, _I]
    lib.isa_sparse_mla_attend.restype = _I
    lib.isa_sparse_mla_attend.argtypes = [_P, _P, _P, _I, _I, _I, _I, _I, _I, _I, _F, _P, _P,
                                          _P, _Z, _P]
    lib.isa_attend_fp8_workspace_bytes.restype = _Z
    lib.isa_attend_fp8_workspace_bytes.argtypes = [_I, _I, _I, _I, _I, _I]
    lib.isa_sparse_mla_attend_fp8.restype = _I
    lib.isa_sparse_mla_attend_fp8.argtypes = [_P, _P, _P, _P, _P, _I, _I, _I, _I, _I, _I, _I, _F,
                                              _P, _P, _P, _Z, _P]
    lib.isa_indexer_scores_paged.restype = _I
    lib.isa_indexer_scores_paged.argtypes = [_P, _P, _P, _P, _I, _I, _I, _P, _I, _I, _I, _I, _P,
                                             _P]
    lib.isa_sparse_mla_attend_paged.restype = _I
    lib.isa_sparse_mla_attend_paged.argtypes = [_P, _P, _P, _I, _I, _I, _P, _I, _I, _I, _I, _I,
                                                _I, _F, _P, _P, _P, _Z, _P]
    lib.isa_index_histogram.restype = _I
    lib.isa_index_histogram.argtypes = [_P, _I, _I, _I, _I, _P, _P]
    lib.isa_group_workspace_bytes.restype = _Z
    lib.isa_group_workspace_bytes.argtypes = [ctypes.POINTER(GroupArgs)]
    lib.isa_group_forward.restype = _I
    lib.isa_group_forward.argtypes = [ctypes.POINTER(GroupArgs), _P]
    lib.isa_group_noalloc_max_bytes.restype = _Z
    lib.isa_group_noalloc_max_bytes.argtypes = []
    lib.isa_group_forward_noalloc.restype = _I
    lib.isa_group_forward_noalloc.argtypes = [ctypes.POINTER(GroupArgs), _P]
    if lib.isa_abi_version() != ISA_ABI_VERSION:
        raise RuntimeError(f"libisa ABI {lib.isa_abi_version()} != {ISA_ABI_VERSION}")
    _lib = lib
    return lib


def isa_abi_version() -> int:
    return load_library().isa_abi_version()


def isa_last_error() -> str:
    return load_library().isa_last_error().decode()


def _check(status: int):
    if status != ISA_OK:
        raise IsaError(status, isa_last_error())


def _ptr(t: Optional[torch.Tensor]) -> Optional[int]:
    return None if t is None else t.data_ptr()


def _stream_ptr(stream) -> int:
    return _stream_of(stream).cuda_stream


def _dev(t: torch.Tensor, dtype, name: str) -> torch.Tensor:
    if not isinstance(t, torch.Tensor) or t.device.type != "cuda":
        raise TypeError(f"{name} must be a device tensor")
    if t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    return t


# ------------------------------------------------------------- workspaces ----

class Workspace:
    """A device byte buffer reused across calls (one call at a time).

    The library clears whatever counters it needs at the start of each call,
    so the buffer needs no initialisation and may be shared by different
    entry points that run one after another on one stream.  Calls that may
    overlap (different streams) need different workspaces; the default
    workspace of the entry points is kept per device and stream.
    """

    def __init__(self, device=None):
        self.device = torch.device("cuda" if device is None else device)
        self.buf: Optional[torch.Tensor] = None
        self._streams = {}        # streams the current buffer was used on

    def get(self, nbytes: int, stream=None) -> torch.Tensor:
        if nbytes <= 0:
            nbytes = 256
        if self.buf is None or self.buf.numel() < nbytes:
            if self.buf is not None:
                # work already queued on those streams may still use the old
                # buffer: the allocator must not hand it out before it ends
                for st in self._streams.values():
                    self.buf.record_stream(st)
            self.buf = torch.empty(nbytes, dtype=torch.uint8, device=self.device)
            self._streams = {}
        if stream is not None:
            self._streams[stream.cuda_stream] = stream
        return self.buf


_default_ws = {}


def _stream_of(stream):
    return torch.cuda.current_stream() if stream is None else stream


def _workspace(ws: Optional[Workspace], device, st) -> Workspace:
    """ws, or the default workspace of (device, st); st is a resolved stream."""
    if ws is not None:
        return ws
    key = (str(device), st.cuda_stream)
    if key not in _default_ws:
        _default_ws[key] = Workspace(device)
    return _default_ws[key]


def _on_stream(stream, *tensors):
    """Marks tensors allocated on the current stream as used by `stream` too
    (an explicitly given stream), so that the caching allocator does not
    reuse them while work queued there may still touch them."""
    if stream is None or stream == torch.cuda.current_stream():
        return
    for t in tensors:
        if t is not None:
            t.record_stream(stream)


# -------------------------------------------------------------- entry points ----

def isa_indexer_scores(qI, w, kI, kv_len, S=None, stream=None) -> torch.Tensor:
    """S [B,Tq,L_cap] fp32 = sum_h w * ReLU(qI_h . kI_s) on visible keys, -inf elsewhere."""
    _dev(qI, torch.int8, "qI"); _dev(w, torch.float32, "w"); _dev(kI, torch.int8, "kI")
    _dev(kv_len, torch.int32, "kv_len")
    B, Tq, H_I, D_I = qI.shape
    L_cap = kI.shape[1]
    if S is None:
        S = torch.empty((B, Tq, L_cap), dtype=torch.float32, device=qI.device)
    _dev(S, torch.float32, "S")
    _on_stream(stream, S)
    _check(load_library().isa_indexer_scores(_ptr(qI), _ptr(w), _ptr(kI), _ptr(kv_len), B, Tq, H_I,
                                             D_I, L_cap, _ptr(S), _stream_ptr(stream)))
    return S


def isa_topk_workspace_bytes(B: int, Tq: int, L_cap: int, k: int) -> int:
    return int(load_library().isa_topk_workspace_bytes(B, Tq, L_cap, k))


def isa_topk_select(S, kv_len, k: int, idx=None, ws: Optional[Workspace] = None,
                    stream=None) -> torch.Tensor:
    """idx [B,Tq,k] int32: best min(k, pos+1) positions in ascending order, -1 padded."""
    _dev(S, torch.float32, "S"); _dev(kv_len, torch.int32, "kv_len")
    B, Tq, L_cap = S.shape
    if idx is None:
        idx = torch.empty((B, Tq, k), dtype=torch.int32, device=S.device)
    _dev(idx, torch.int32, "idx")
    nbytes = isa_topk_workspace_bytes(B, Tq, L_cap, k)
    st = _stream_of(stream)
    buf = _workspace(ws, S.device, st).get(nbytes, st)
    _on_stream(stream, idx, buf)
    _check(load_library().isa_topk_select(_ptr(S), _ptr(kv_len), B, Tq, L_cap, int(k), _ptr(idx),
                                          _ptr(buf), buf.numel(), st.cuda_stream))
    return idx


def isa_attend_workspace_bytes(B: int, Tq: int, H: int, D: int, D_v: int, k: int) -> int:
    return int(load_library().isa_attend_workspace_bytes(B, Tq, H, D, D_v, k))


def isa_sparse_mla_attend(Q, C, idx, D_v: int, sm_scale: float, out=None, lse=None,
                          want_lse: bool = False, ws: Optional[Workspace] = None,
                          stream=None) -> Tuple[torch.Tensor, Optional[torch.Tensor]]:
    """(out [B,Tq,H,D_v] bf16, lse [B,Tq,H] fp32 or None) of sparse latent attention."""
    _dev(Q, torch.bfloat16, "Q"); _dev(C, torch.bfloat16, "C"); _dev(idx, torch.int32, "idx")
    B, Tq, H, D = Q.shape
    L_cap = C.shape[1]
    k = idx.shape[2]
    if out is None:
        out = torch.empty((B, Tq, H, D_v), dtype=torch.bfloat16, device=Q.device)
    _dev(out, torch.bfloat16, "out")
    if lse is None and want_lse:
        lse = torch.empty((B, Tq, H), dtype=torch.float32, device=Q.device)
    if lse is not None:
        _dev(lse, torch.float32, "lse")
    nbytes = isa_attend_workspace_bytes(B, Tq, H, D, D_v, k)
    st = _stream_of(stream)
    buf = _workspace(ws, Q.device, st).get(nbytes, st)
    _on_stream(stream, out, lse, buf)
    _check(load_library().isa_sparse_mla_attend(
        _ptr(Q), _ptr(C), _ptr(idx), B, Tq, H, D, int(D_v), L_cap, k, float(sm_scale), _ptr(out),
        _ptr(lse), _ptr(buf), buf.numel(), st.cuda_stream))
    return out, lse


def isa_attend_fp8_workspace_bytes(B: int, Tq: int, H: int, D_c: int, D_r: int, k: int) -> int:
    return int(load_library().isa_attend_fp8_workspace_bytes(B, Tq, H, D_c, D_r, k))


def isa_sparse_mla_attend_fp8(Q, C8, Ce, Cr, idx, sm_scale: float, out=None, lse=None,
                              want_lse: bool = False, ws: Optional[Workspace] = None,
                              stream=None) -> Tuple[torch.Tensor, Optional[torch.Tensor]]:
    """Sparse latent attention over an FP8 cache: C8 [B,L_cap,D_c] E4M3 codes
    (uint8), Ce [B,L_cap] exponent bytes (uint8, scale 2^(e-127)), Cr
    [B,L_cap,D_r] bf16 RoPE dims.  Returns (out [B,Tq,H,D_c] bf16, lse or None)."""
    _dev(Q, torch.bfloat16, "Q"); _dev(C8, torch.uint8, "C8"); _dev(Ce, torch.uint8, "Ce")
    _dev(Cr, torch.bfloat16, "Cr"); _dev(idx, torch.int32, "idx")
    B, Tq, H, D = Q.shape
    L_cap, D_c = C8.shape[1], C8.shape[2]
    D_r = Cr.shape[2]
    k = idx.shape[2]
    if out is None:
        out = torch.empty((B, Tq, H, D_c), dtype=torch.bfloat16, device=Q.device)
    _dev(out, torch.bfloat16, "out")
    if lse is None and want_lse:
        lse = torch.empty((B, Tq, H), dtype=torch.float32, device=Q.device)
    if lse is not None:
        _dev(lse, torch.float32, "lse")
    nbytes = isa_attend_fp8_workspace_bytes(B, Tq, H, D_c, D_r, k)
    st = _stream_of(stream)
    buf = _workspace(ws, Q.device, st).get(nbytes, st)
    _on_stream(stream, out, lse, buf)
    _check(load_library().isa_sparse_mla_attend_fp8(
        _ptr(Q), _ptr(C8), _ptr(Ce), _ptr(Cr), _ptr(idx), B, Tq, H, D_c, D_r, L_cap, k,
        float(sm_scale), _ptr(out), _ptr(lse), _ptr(buf), buf.numel(), st.cuda_stream))
    return out, lse


def isa_indexer_scores_paged(qI, w, kI_pages, block_table, kv_len, S=None,
                             stream=None) -> torch.Tensor:
    """Indexer scores over a paged key cache: kI_pages [n_pages, block_size,
    D_I] int8, block_table [B, max_blocks] int32.  S [B,Tq,max_blocks*block_size]."""
    _dev(qI, torch.int8, "qI"); _dev(w, torch.float32, "w"); _dev(kI_pages, torch.int8, "kI_pages")
    _dev(block_table, torch.int32, "block_table"); _dev(kv_len, torch.int32, "kv_len")
    B, Tq, H_I, D_I = qI.shape
    n_pages, bs = kI_pages.shape[0], kI_pages.shape[1]
    max_blocks = block_table.shape[1]
    if S is None:
        S = torch.empty((B, Tq, max_blocks * bs), dtype=torch.float32, device=qI.device)
    _dev(S, torch.float32, "S")
    _on_stream(stream, S)
    _check(load_library().isa_indexer_scores_paged(
        _ptr(qI), _ptr(w), _ptr(kI_pages), _ptr(block_table), max_blocks, bs, n_pages,
        _ptr(kv_len), B, Tq, H_I, D_I, _ptr(S), _stream_ptr(stream)))
    return S


def isa_sparse_mla_attend_paged(Q, C_pages, block_table, idx, D_v: int, sm_scale: float,
                                out=None, lse=None, want_lse: bool = False,
                                ws: Optional[Workspace] = None, stream=None):
    """Sparse latent attention over a paged cache: C_pages [n_pages, block_size,
    D] bf16, block_table [B, max_blocks] int32; idx holds logical positions."""
    _dev(Q, torch.bfloat16, "Q"); _dev(C_pages, torch.bfloat16, "C_pages")
    _dev(block_table, torch.int32, "block_table"); _dev(idx, torch.int32, "idx")
    B, Tq, H, D = Q.shape
    n_pages, bs = C_pages.shape[0], C_pages.shape[1]
    max_blocks = block_table.shape[1]
    k = idx.shape[2]
    if out is None:
        out = torch.empty((B, Tq, H, D_v), dtype=torch.bfloat16, device=Q.device)
    _dev(out, torch.bfloat16, "out")
    if lse is None and want_lse:
        lse = torch.empty((B, Tq, H), dtype=torch.float32, device=Q.device)
    if lse is not None:
        _dev(lse, torch.float32, "lse")
    nbytes = isa_attend_workspace_bytes(B, Tq, H, D, D_v, k)
    st = _stream_of(stream)
    buf = _workspace(ws, Q.device, st).get(nbytes, st)
    _on_stream(stream, out, lse, buf)
    _check(load_library().isa_sparse_mla_attend_paged(
        _ptr(Q), _ptr(C_pages), _ptr(block_table), max_blocks, bs, n_pages, _ptr(idx), B, Tq, H,
        D, int(D_v), k, float(sm_scale), _ptr(out), _ptr(lse), _ptr(buf), buf.numel(),
        st.cuda_stream))
    return out, lse


def isa_index_histogram(idx, L_cap: int, counts=None, stream=None) -> torch.Tensor:
    """counts [B,L_cap] int32 (read as uint32) += the occurrences of every
    position in idx [B,Tq,k]; a zeroed tensor is made when counts is None."""
    _dev(idx, torch.int32, "idx")
    B, Tq, k = idx.shape
    if counts is None:
        counts = torch.zeros((B, L_cap), dtype=torch.int32, device=idx.device)
    _dev(counts, torch.int32, "counts")
    if tuple(counts.shape) != (B, L_cap):
        raise ValueError(f"counts must be [{B}, {L_cap}]")
    _on_stream(stream, counts)
    _check(load_library().isa_index_histogram(_ptr(idx), B, Tq, k, int(L_cap), _ptr(counts),
                                              _stream_ptr(stream)))
    return counts


class GroupCall:
    """Marshals one isa_group_forward call and keeps its ctypes arrays alive.
    With kv8 = (C8, Ce, Cr), three per-layer lists, the layers' caches are FP8
    (as in isa_sparse_mla_attend_fp8) and C is ignored.  With block_table
    [B, max_blocks] int32, kI and the layers' caches are page pools
    [n_pages, block_size, row] sharing that table."""

    def __init__(self, qI: Sequence, w: Sequence, kI: Sequence, kv_len, Q: Sequence,
                 C: Optional[Sequence], k: int, D_v: int, sm_scale: float, idx=None,
                 reuse_idx: bool = False, per_layer_indexer: bool = False,
                 out: Optional[Sequence] = None, lse: Optional[Sequence] = None,
                 ws: Optional[Workspace] = None, kv8: Optional[Tuple[Sequence, Sequence, Sequence]] = None,
                 block_table: Optional[torch.Tensor] = None, noalloc: bool = False):
        n = len(Q)
        dev = Q[0].device
        for i, x in enumerate(Q):
            _dev(x, torch.bfloat16, f"Q[{i}]")
        if kv8 is not None:
            C8, Ce, Cr = (list(x) for x in kv8)
            if not (len(C8) == len(Ce) == len(Cr) == n):
                raise ValueError("kv8 needs one (C8, Ce, Cr) entry per layer")
            for i in range(n):
                _dev(C8[i], torch.uint8, f"C8[{i}]"); _dev(Ce[i], torch.uint8, f"Ce[{i}]")
                _dev(Cr[i], torch.bfloat16, f"Cr[{i}]")
            C = []
            L_cap = C8[0].shape[1]
        else:
            C8 = Ce = Cr = []
            for i, x in enumerate(C):
                _dev(x, torch.bfloat16, f"C[{i}]")
            L_cap = C[0].shape[1]
        _dev(kv_len, torch.int32, "kv_len")
        B, Tq, H, D = Q[0].shape
        pool = (C8[0] if kv8 is not None else C[0])
        if block_table is not None:
            _dev(block_table, torch.int32, "block_table")
            n_pages, bs = pool.shape[0], pool.shape[1]
            L_cap = block_table.shape[1] * bs
        n_ix = n if per_layer_indexer else (0 if reuse_idx else 1)
        qI = list(qI or [])[: max(n_ix, 0)]
        w = list(w or [])[: max(n_ix, 0)]
        kI = list(kI or [])[: max(n_ix, 0)]
        for i in range(n_ix):
            _dev(qI[i], torch.int8, f"qI[{i}]"); _dev(w[i], torch.float32, f"w[{i}]")
            _dev(kI[i], torch.int8, f"kI[{i}]")
        H_I, D_I = (qI[0].shape[2], qI[0].shape[3]) if n_ix else (64, 128)
        if idx is None:
            if reuse_idx:
                raise ValueError("reuse_idx needs idx")
            idx = torch.empty((B, Tq, k), dtype=torch.int32, device=dev)
        _dev(idx, torch.int32, "idx")
        if out is None:
            out = [torch.empty((B, Tq, H, D_v), dtype=torch.bfloat16, device=dev) for _ in range(n)]
        self.idx, self.out, self.lse = idx, list(out), (list(lse) if lse is not None else None)
        self._keep = [qI, w, kI, Q, C, self.out, self.lse, C8, Ce, Cr, block_table]

        def arr(ts):
            return (_P * len(ts))(*[_ptr(t) for t in ts]) if ts else None

        self._arrays = [arr(qI), arr(w), arr(kI), arr(list(Q)), arr(list(C)), arr(self.out),
                        arr(self.lse) if self.lse is not None else None,
                        arr(C8), arr(Ce), arr(Cr)]
        a = GroupArgs()
        a.B, a.Tq, a.L_cap, a.H_I, a.D_I, a.k = B, Tq, L_cap, H_I, D_I, int(k)
        a.H, a.D, a.D_v, a.n_layers, a.sm_scale = H, D, int(D_v), n, float(sm_scale)
        a.qI = ctypes.cast(self._arrays[0], _P) if self._arrays[0] else None
        a.w = ctypes.cast(self._arrays[1], _P) if self._arrays[1] else None
        a.kI = ctypes.cast(self._arrays[2], _P) if self._arrays[2] else None
        a.kv_len = _ptr(kv_len)
        a.Q = ctypes.cast(self._arrays[3], _P)
        a.C = ctypes.cast(self._arrays[4], _P) if self._arrays[4] else None
        a.out = ctypes.cast(self._arrays[5], _P)
        a.lse = ctypes.cast(self._arrays[6], _P) if self._arrays[6] is not None else None
        a.idx = _ptr(idx)
        a.reuse_idx = int(bool(reuse_idx))
        a.per_layer_indexer = int(bool(per_layer_indexer))
        a.kv_fp8 = int(kv8 is not None)
        if block_table is not None:
            a.paged, a.block_table = 1, _ptr(block_table)
            a.max_blocks, a.block_size, a.n_pages = block_table.shape[1], bs, n_pages
        if kv8 is not None:
            a.C8 = ctypes.cast(self._arrays[7], _P)
            a.Ce = ctypes.cast(self._arrays[8], _P)
            a.Cr = ctypes.cast(self._arrays[9], _P)
        self.args = a
        self._nbytes = int(load_library().isa_group_workspace_bytes(ctypes.byref(a)))
        self._ws, self._dev = ws, dev
        self._noalloc = bool(noalloc)

    def __call__(self, stream=None):
        if self._noalloc:
            # the library's own fixed scratch memory (isa_group_forward_noalloc)
            st = _stream_of(stream)
            self.args.ws, self.args.ws_bytes = None, 0
            _on_stream(stream, self.idx, *self.out, *(self.lse or []))
            _check(load_library().isa_group_forward_noalloc(ctypes.byref(self.args), st.cuda_stream))
            return self.idx, self.out, self.lse
        # the workspace is taken at call time (the given one, or the default
        # one of this device and stream), so calls on different streams never
        # share scratch memory and a workspace grown by another call is seen
        st = _stream_of(stream)
        buf = _workspace(self._ws, self._dev, st).get(self._nbytes, st)
        self.args.ws = _ptr(buf)
        self.args.ws_bytes = buf.numel()
        _on_stream(stream, buf, self.idx, *self.out, *(self.lse or []))
        _check(load_library().isa_group_forward(ctypes.byref(self.args), st.cuda_stream))
        return self.idx, self.out, self.lse


def isa_group_workspace_bytes(call: GroupCall) -> int:
    return int(load_library().isa_group_workspace_bytes(ctypes.byref(call.args)))


def isa_group_forward(qI: Sequence, w: Sequence, kI: Sequence, kv_len, Q: Sequence,
                      C: Optional[Sequence], k: int, D_v: int, sm_scale: float, idx=None,
                      reuse_idx: bool = False, per_layer_indexer: bool = False, out=None, lse=None,
                      ws: Optional[Workspace] = None, stream=None, kv8=None, block_table=None):
    """One IndexShare layer group: (idx, [out_l], [lse_l] or None)."""
    call = GroupCall(qI, w, kI, kv_len, Q, C, k, D_v, sm_scale, idx=idx, reuse_idx=reuse_idx,
                     per_layer_indexer=per_layer_indexer, out=out, lse=lse, ws=ws, kv8=kv8,
                     block_table=block_table)
    return call(stream)


def isa_group_noalloc_max_bytes() -> int:
    return int(load_library().isa_group_noalloc_max_bytes())


def isa_group_forward_noalloc(qI: Sequence, w: Sequence, kI: Sequence, kv_len, Q: Sequence,
                              C: Optional[Sequence], k: int, D_v: int, sm_scale: float, idx=None,
                              reuse_idx: bool = False, per_layer_indexer: bool = False, out=None,
                              lse=None, stream=None, kv8=None, block_table=None):
    """isa_group_forward on the library's fixed scratch memory (no workspace
    is allocated): (idx, [out_l], [lse_l] or None).  Calls that may overlap on
    one GPU share that memory and must not be issued concurrently."""
    call = GroupCall(qI, w, kI, kv_len, Q, C, k, D_v, sm_scale, idx=idx, reuse_idx=reuse_idx,
                     per_layer_indexer=per_layer_indexer, out=out, lse=lse, kv8=kv8,
                     block_table=block_table, noalloc=True)
    return call(stream)
