"""CPU oracle for one IndexShare layer group (ctypes front end of oracle.c).

TEST INFRASTRUCTURE ONLY: the test suite, the smoke check and the
benchmark's CPU-baseline leg are the only callers.  The GPU library never
imports, links or calls anything here, and nothing here imports the GPU
package.

Inputs are numpy arrays or CPU torch tensors; bf16 tensors may be passed as
torch.bfloat16 or as uint16 bit patterns.  Every function is a thin
marshalling layer over the plain C loops in oracle.c, which state the
definitions and cite the pages they follow.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from typing import Sequence

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(_HERE, "liboracle.so")
_lib = None


def build() -> str:
    """Compile oracle.c into liboracle.so beside it (gcc, -O2, no fp contraction)."""
    subprocess.run(["sh", os.path.join(_HERE, "build.sh")], check=True)
    return _LIB_PATH


def _load():
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_LIB_PATH):
        build()
    lib = ctypes.CDLL(_LIB_PATH)
    P = ctypes.c_void_p
    I = ctypes.c_int
    lib.oracle_indexer_scores.argtypes = [P, P, P, P, I, I, I, I, I, P]
    lib.oracle_indexer_scores.restype = None
    lib.oracle_topk_select.argtypes = [P, P, I, I, I, I, P]
    lib.oracle_topk_select.restype = None
    lib.oracle_sparse_mla_attend.argtypes = [P, P, P, I, I, I, I, I, I, I, ctypes.c_float, P, P]
    lib.oracle_sparse_mla_attend.restype = None
    lib.oracle_group_forward.argtypes = [I, I, I, I, I, I, I, I, I, I, ctypes.c_float,
                                         P, P, P, P, P, P, P, P, P, I, I, P]
    lib.oracle_group_forward.restype = None
    lib.oracle_indexer_scores_paged.argtypes = [P, P, P, P, I, I, I, P, I, I, I, I, P]
    lib.oracle_indexer_scores_paged.restype = None
    lib.oracle_sparse_mla_attend_paged.argtypes = [P, P, P, I, I, I, P, I, I, I, I, I, I,
                                                   ctypes.c_float, P, P]
    lib.oracle_sparse_mla_attend_paged.restype = None
    lib.oracle_index_histogram.argtypes = [P, I, I, I, I, P]
    lib.oracle_index_histogram.restype = None
    lib.oracle_e4m3_to_double.argtypes = [ctypes.c_uint8]
    lib.oracle_e4m3_to_double.restype = ctypes.c_double
    lib.oracle_sparse_mla_attend_fp8.argtypes = [P, P, P, P, P, I, I, I, I, I, I, I,
                                                 ctypes.c_float, P, P]
    lib.oracle_sparse_mla_attend_fp8.restype = None
    _lib = lib
    return lib


def _np(x, dtype) -> np.ndarray:
    """Contiguous numpy view/copy with the given dtype (bf16 torch -> uint16 bits)."""
    try:
        import torch
        if isinstance(x, torch.Tensor):
            x = x.detach()
            if x.device.type != "cpu":
                raise ValueError("oracle inputs must live in host memory")
            if x.dtype == torch.bfloat16:
                x = x.view(torch.int16)
            x = x.contiguous().numpy()
    except ImportError:  # pragma: no cover - torch is always present here
        pass
    a = np.ascontiguousarray(x)
    if dtype == np.uint16 and a.dtype == np.int16:
        a = a.view(np.uint16)
    if a.dtype != dtype:
        raise TypeError(f"expected {np.dtype(dtype)}, got {a.dtype}")
    return a


def _ptr(a: np.ndarray) -> int:
    return a.ctypes.data


def indexer_scores(qI, w, kI, kv_len) -> np.ndarray:
    """S [B,Tq,L_cap] float32: sum_h w*ReLU(qI_h . kI_s) for visible s, -inf elsewhere."""
    qI = _np(qI, np.int8)
    w = _np(w, np.float32)
    kI = _np(kI, np.int8)
    kv_len = _np(kv_len, np.int32)
    B, Tq, H_I, D_I = qI.shape
    L_cap = kI.shape[1]
    assert w.shape == (B, Tq, H_I) and kI.shape == (B, L_cap, D_I) and kv_len.shape == (B,)
    S = np.empty((B, Tq, L_cap), dtype=np.float32)
    _load().oracle_indexer_scores(_ptr(qI), _ptr(w), _ptr(kI), _ptr(kv_len), B, Tq, H_I, D_I,
                                  L_cap, _ptr(S))
    return S


def topk_select(S, kv_len, k: int) -> np.ndarray:
    """idx [B,Tq,k] int32: the best min(k, pos+1) positions, ascending, -1 padded."""
    S = _np(S, np.float32)
    kv_len = _np(kv_len, np.int32)
    B, Tq, L_cap = S.shape
    idx = np.empty((B, Tq, k), dtype=np.int32)
    _load().oracle_topk_select(_ptr(S), _ptr(kv_len), B, Tq, L_cap, int(k), _ptr(idx))
    return idx


def sparse_mla_attend(Q, C, idx, D_v: int, sm_scale: float):
    """(out [B,Tq,H,D_v] float64, lse [B,Tq,H] float64) of sparse softmax attention."""
    Q = _np(Q, np.uint16)
    C = _np(C, np.uint16)
    idx = _np(idx, np.int32)
    B, Tq, H, D = Q.shape
    L_cap = C.shape[1]
    k = idx.shape[2]
    assert C.shape == (B, L_cap, D) and idx.shape == (B, Tq, k)
    out = np.empty((B, Tq, H, D_v), dtype=np.float64)
    lse = np.empty((B, Tq, H), dtype=np.float64)
    _load().oracle_sparse_mla_attend(_ptr(Q), _ptr(C), _ptr(idx), B, Tq, H, D, int(D_v), L_cap,
                                     k, ctypes.c_float(sm_scale), _ptr(out), _ptr(lse))
    return out, lse


def indexer_scores_paged(qI, w, kI_pages, table, kv_len) -> np.ndarray:
    """S [B,Tq,max_blocks*block_size] float32 over a paged key cache
    (kI_pages [n_pages, block_size, D_I] int8, table [B, max_blocks] int32)."""
    qI = _np(qI, np.int8)
    w = _np(w, np.float32)
    kI_pages = _np(kI_pages, np.int8)
    table = _np(table, np.int32)
    kv_len = _np(kv_len, np.int32)
    B, Tq, H_I, D_I = qI.shape
    n_pages, bs, _ = kI_pages.shape
    max_blocks = table.shape[1]
    S = np.empty((B, Tq, max_blocks * bs), dtype=np.float32)
    _load().oracle_indexer_scores_paged(_ptr(qI), _ptr(w), _ptr(kI_pages), _ptr(table), max_blocks,
                                        bs, n_pages, _ptr(kv_len), B, Tq, H_I, D_I, _ptr(S))
    return S


def sparse_mla_attend_paged(Q, C_pages, table, idx, D_v: int, sm_scale: float):
    """(out, lse) of sparse attention over a paged latent cache
    (C_pages [n_pages, block_size, D] bf16, table [B, max_blocks] int32)."""
    Q = _np(Q, np.uint16)
    C_pages = _np(C_pages, np.uint16)
    table = _np(table, np.int32)
    idx = _np(idx, np.int32)
    B, Tq, H, D = Q.shape
    n_pages, bs, _ = C_pages.shape
    max_blocks = table.shape[1]
    k = idx.shape[2]
    out = np.empty((B, Tq, H, D_v), dtype=np.float64)
    lse = np.empty((B, Tq, H), dtype=np.float64)
    _load().oracle_sparse_mla_attend_paged(_ptr(Q), _ptr(C_pages), _ptr(table), max_blocks, bs,
                                           n_pages, _ptr(idx), B, Tq, H, D, int(D_v), k,
                                           ctypes.c_float(sm_scale), _ptr(out), _ptr(lse))
    return out, lse


def index_histogram(idx, L_cap: int, counts=None) -> np.ndarray:
    """counts [B,L_cap] uint32 += occurrences of each position in idx [B,Tq,k]."""
    idx = _np(idx, np.int32)
    B, Tq, k = idx.shape
    if counts is None:
        counts = np.zeros((B, L_cap), dtype=np.uint32)
    counts = np.ascontiguousarray(counts, dtype=np.uint32)
    _load().oracle_index_histogram(_ptr(idx), B, Tq, k, int(L_cap), _ptr(counts))
    return counts


def e4m3_to_double(code: int) -> float:
    """Value of one OCP FP8 E4M3 code."""
    return float(_load().oracle_e4m3_to_double(int(code) & 0xFF))


def sparse_mla_attend_fp8(Q, C8, Ce, Cr, idx, sm_scale: float):
    """(out [B,Tq,H,D_c] float64, lse [B,Tq,H] float64) of sparse attention over
    an FP8 latent cache (C8 codes, Ce exponent bytes, Cr bf16 RoPE dims)."""
    Q = _np(Q, np.uint16)
    C8 = _np(C8, np.uint8)
    Ce = _np(Ce, np.uint8)
    Cr = _np(Cr, np.uint16)
    idx = _np(idx, np.int32)
    B, Tq, H, D = Q.shape
    L_cap, D_c = C8.shape[1], C8.shape[2]
    D_r = Cr.shape[2]
    k = idx.shape[2]
    assert D == D_c + D_r and Ce.shape == (B, L_cap) and Cr.shape == (B, L_cap, D_r)
    out = np.empty((B, Tq, H, D_c), dtype=np.float64)
    lse = np.empty((B, Tq, H), dtype=np.float64)
    _load().oracle_sparse_mla_attend_fp8(_ptr(Q), _ptr(C8), _ptr(Ce), _ptr(Cr), _ptr(idx), B, Tq,
                                         H, D_c, D_r, L_cap, k, ctypes.c_float(sm_scale),
                                         _ptr(out), _ptr(lse))
    return out, lse


def group_forward(qI: Sequence, w: Sequence, kI: Sequence, kv_len, Q: Sequence, C: Sequence,
                  k: int, D_v: int, sm_scale: float, idx=None,
                  reuse_idx: bool = False, per_layer_indexer: bool = False):
    """One layer group via oracle_group_forward: (idx, [out_l], [lse_l]).

    The index set is computed once from the first indexer entry and shared by
    every layer; ``reuse_idx`` takes ``idx`` as given (later MTP draft steps);
    ``per_layer_indexer`` recomputes it per layer from that layer's entry (the
    ablation baseline) and leaves the last layer's set in idx.
    """
    n_layers = len(Q)
    n_ix = n_layers if per_layer_indexer else (0 if reuse_idx else 1)
    qI = [_np(x, np.int8) for x in list(qI or [])[:n_ix]]
    w = [_np(x, np.float32) for x in list(w or [])[:n_ix]]
    kI = [_np(x, np.int8) for x in list(kI or [])[:n_ix]]
    kv_len = _np(kv_len, np.int32)
    Q = [_np(x, np.uint16) for x in Q]
    C = [_np(x, np.uint16) for x in C]
    B, Tq, H, D = Q[0].shape
    L_cap = C[0].shape[1]
    H_I, D_I = (qI[0].shape[2], qI[0].shape[3]) if n_ix else (1, 1)
    if reuse_idx:
        if idx is None:
            raise ValueError("reuse_idx needs idx")
        idx_out = _np(idx, np.int32).copy()
    else:
        idx_out = np.empty((B, Tq, k), dtype=np.int32)
    outs = [np.empty((B, Tq, H, D_v), dtype=np.float64) for _ in range(n_layers)]
    lses = [np.empty((B, Tq, H), dtype=np.float64) for _ in range(n_layers)]
    S = np.empty((B, Tq, L_cap) if n_ix else (1,), dtype=np.float32)

    def parr(arrs):
        return (ctypes.c_void_p * len(arrs))(*[_ptr(a) for a in arrs])

    lib = _load()
    lib.oracle_group_forward(
        B, Tq, L_cap, H_I, D_I, int(k), H, D, int(D_v), n_layers, ctypes.c_float(sm_scale),
        parr(qI), parr(w), parr(kI), _ptr(kv_len), parr(Q), parr(C), parr(outs), parr(lses),
        _ptr(idx_out), int(bool(reuse_idx)), int(bool(per_layer_indexer)), _ptr(S))
    return idx_out, outs, lses
