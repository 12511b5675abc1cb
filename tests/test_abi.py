"""The C-ABI library loads, exports every declared symbol, and rejects bad
arguments on the host before any GPU work (runs without a GPU)."""
import ctypes
import os
import re

import pytest

import long_context_sparse_indexshare_amd as isa

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "isa.h")

# fake, never-dereferenced addresses: every call below fails its host checks first
A16 = 1 << 20          # 16-byte aligned
A4 = (1 << 20) + 4     # 4-byte aligned only


def _declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(isa_[a-z0-9_]+)\s*\(", text)))


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(isa.LIB_PATH):
        import long_context_sparse_indexshare_amd.build as b
        b.build()
    return isa.load_library()


def test_exports_every_declared_symbol(lib):
    declared = _declared_functions()
    assert set(declared) == set(isa.EXPORTED_SYMBOLS)
    for name in declared:
        assert hasattr(lib, name), name


def test_abi_version(lib):
    assert lib.isa_abi_version() == isa.ISA_ABI_VERSION
    assert isa.isa_abi_version() == 3


def _status(lib, fn, *args):
    st = getattr(lib, fn)(*args)
    # every call here must stop at the host checks: a call that passed them
    # would have launched a kernel on the fake addresses
    assert st not in (isa.ISA_OK, isa.ISA_ERR_HIP), f"{fn} passed the host checks"
    return st, lib.isa_last_error().decode()


def test_indexer_rejects_bad_arguments(lib):
    good = (A16, A4, A16, A4, 2, 1, 64, 128, 4096, A4, None)
    st, _ = _status(lib, "isa_indexer_scores", None, *good[1:])
    assert st == isa.ISA_ERR_INVALID_ARG
    for pos, bad in ((4, 0), (5, -1), (6, 0), (7, 0), (8, 0)):
        args = list(good)
        args[pos] = bad
        assert _status(lib, "isa_indexer_scores", *args)[0] == isa.ISA_ERR_INVALID_ARG
    args = list(good)
    args[8] = (1 << 21) + 1
    assert _status(lib, "isa_indexer_scores", *args)[0] == isa.ISA_ERR_INVALID_ARG
    for H_I, D_I in ((3, 128), (64, 96), (128, 128), (64, 256)):
        args = list(good)
        args[6], args[7] = H_I, D_I
        st, msg = _status(lib, "isa_indexer_scores", *args)
        assert st == isa.ISA_ERR_UNSUPPORTED and "not compiled" in msg
    args = list(good)
    args[0] = A4          # qI must be 16-byte aligned
    assert _status(lib, "isa_indexer_scores", *args)[0] == isa.ISA_ERR_INVALID_ARG


def test_topk_rejects_bad_arguments(lib):
    need = lib.isa_topk_workspace_bytes(2, 1, 4096, 2048)
    assert need > 0
    good = [A4, A4, 2, 1, 4096, 2048, A4, A16 << 8, need, None]
    for k in (0, -5, 2049):
        args = list(good)
        args[5] = k
        st, msg = _status(lib, "isa_topk_select", *args)
        assert st == isa.ISA_ERR_INVALID_ARG and "k=" in msg
    args = list(good)
    args[8] = need - 1
    assert _status(lib, "isa_topk_select", *args)[0] == isa.ISA_ERR_WORKSPACE
    args = list(good)
    args[7] = None
    assert _status(lib, "isa_topk_select", *args)[0] == isa.ISA_ERR_WORKSPACE
    args = list(good)
    args[7] = (A16 << 8) + 16   # workspace must be 256-byte aligned
    assert _status(lib, "isa_topk_select", *args)[0] == isa.ISA_ERR_WORKSPACE
    args = list(good)
    args[0] = None
    assert _status(lib, "isa_topk_select", *args)[0] == isa.ISA_ERR_INVALID_ARG


def test_attend_rejects_bad_arguments(lib):
    f = ctypes.c_float
    need = lib.isa_attend_workspace_bytes(8, 1, 64, 576, 512, 2048)
    assert need > 0       # decode splits the k slots, so it needs partials
    assert lib.isa_attend_workspace_bytes(1, 4096, 64, 576, 512, 2048) == 0
    good = [A16, A16, A4, 8, 1, 64, 576, 512, 4096, 2048, f(1 / 24), A16, None, A16 << 8, need,
            None]
    for H, D, D_v in ((64, 512, 512), (65, 576, 512), (65, 160, 128), (16, 192, 128)):
        args = list(good)
        args[5], args[6], args[7] = H, D, D_v
        assert _status(lib, "isa_sparse_mla_attend", *args)[0] == isa.ISA_ERR_UNSUPPORTED
    for bad_scale in (float("inf"), float("nan"), 0.0, -0.5):
        args = list(good)
        args[10] = f(bad_scale)
        assert _status(lib, "isa_sparse_mla_attend", *args)[0] == isa.ISA_ERR_INVALID_ARG
    args = list(good)
    args[9] = 4096
    assert _status(lib, "isa_sparse_mla_attend", *args)[0] == isa.ISA_ERR_INVALID_ARG
    args = list(good)
    args[14] = 100
    assert _status(lib, "isa_sparse_mla_attend", *args)[0] == isa.ISA_ERR_WORKSPACE
    args = list(good)
    args[1] = A4
    assert _status(lib, "isa_sparse_mla_attend", *args)[0] == isa.ISA_ERR_INVALID_ARG


def test_attend_fp8_rejects_bad_arguments(lib):
    f = ctypes.c_float
    need = lib.isa_attend_fp8_workspace_bytes(8, 1, 64, 512, 64, 2048)
    assert need == lib.isa_attend_workspace_bytes(8, 1, 64, 576, 512, 2048) > 0
    # Q, C8, Ce, Cr, idx, B, Tq, H, D_c, D_r, L_cap, k, scale, out, lse, ws, ws_bytes, stream
    good = [A16, A16, A4, A16, A4, 8, 1, 64, 512, 64, 4096, 2048, f(1 / 24), A16, None, A16 << 8,
            need, None]
    for D_c, D_r in ((512, 32), (256, 64), (128, 64)):
        args = list(good)
        args[8], args[9] = D_c, D_r
        assert _status(lib, "isa_sparse_mla_attend_fp8", *args)[0] == isa.ISA_ERR_UNSUPPORTED
    for i in (1, 2, 3):                                   # each FP8 cache array
        args = list(good)
        args[i] = None
        assert _status(lib, "isa_sparse_mla_attend_fp8", *args)[0] == isa.ISA_ERR_INVALID_ARG
    for i in (1, 3):                                      # codes and RoPE need 16-byte rows
        args = list(good)
        args[i] = A4
        assert _status(lib, "isa_sparse_mla_attend_fp8", *args)[0] == isa.ISA_ERR_INVALID_ARG
    args = list(good)
    args[12] = f(float("nan"))
    assert _status(lib, "isa_sparse_mla_attend_fp8", *args)[0] == isa.ISA_ERR_INVALID_ARG
    args = list(good)
    args[16] = 100
    assert _status(lib, "isa_sparse_mla_attend_fp8", *args)[0] == isa.ISA_ERR_WORKSPACE


def test_histogram_rejects_bad_arguments(lib):
    good = [A16, 2, 1, 2048, 4096, A4, None]
    assert _status(lib, "isa_index_histogram", None, *good[1:])[0] == isa.ISA_ERR_INVALID_ARG
    for i, bad in ((1, 0), (3, 0), (3, 4096), (4, (1 << 21) + 1)):
        args = list(good)
        args[i] = bad
        assert _status(lib, "isa_index_histogram", *args)[0] == isa.ISA_ERR_INVALID_ARG
    args = list(good)
    args[0] = A4                                          # idx rows are read 16 bytes at a time
    assert _status(lib, "isa_index_histogram", *args)[0] == isa.ISA_ERR_INVALID_ARG


def test_paged_calls_reject_bad_page_geometry(lib):
    f = ctypes.c_float
    # qI, w, kI_pages, table, max_blocks, block_size, n_pages, kv_len, B, Tq, H_I, D_I, S, stream
    good = [A16, A4, A16, A4, 64, 64, 600, A4, 8, 1, 64, 128, A4, None]
    for i, bad in ((3, None), (4, 0), (6, 0), (5, 48), (5, 16), (5, 1 << 17), (6, 1 << 26),
                   (4, (1 << 21) // 64 + 1)):
        args = list(good)
        args[i] = bad
        assert _status(lib, "isa_indexer_scores_paged", *args)[0] == isa.ISA_ERR_INVALID_ARG, (i, bad)
    need = lib.isa_attend_workspace_bytes(8, 1, 64, 576, 512, 2048)
    # Q, C_pages, table, max_blocks, block_size, n_pages, idx, B, Tq, H, D, D_v, k, scale, out,
    # lse, ws, ws_bytes, stream
    gooda = [A16, A16, A4, 64, 64, 600, A4, 8, 1, 64, 576, 512, 2048, f(1 / 24), A16, None,
             A16 << 8, need, None]
    for i, bad in ((2, A4 + 1), (4, 100), (5, -1)):
        args = list(gooda)
        args[i] = bad
        assert _status(lib, "isa_sparse_mla_attend_paged", *args)[0] == isa.ISA_ERR_INVALID_ARG
    args = list(gooda)
    args[10] = 512
    assert _status(lib, "isa_sparse_mla_attend_paged", *args)[0] == isa.ISA_ERR_UNSUPPORTED


def test_group_rejects_bad_arguments(lib):
    P = ctypes.c_void_p
    arr1 = (P * 1)(A16)
    arr4 = (P * 4)(A16, A16, A16, A16)
    a = isa.GroupArgs()
    a.B, a.Tq, a.L_cap, a.H_I, a.D_I, a.k = 8, 1, 4096, 64, 128, 2048
    a.H, a.D, a.D_v, a.n_layers, a.sm_scale = 64, 576, 512, 4, 1 / 24
    a.qI = ctypes.cast(arr1, P); a.w = ctypes.cast((P * 1)(A4), P); a.kI = ctypes.cast(arr1, P)
    a.kv_len = A4
    a.Q = ctypes.cast(arr4, P); a.C = ctypes.cast(arr4, P); a.out = ctypes.cast(arr4, P)
    a.lse = None
    a.idx = A4
    need = lib.isa_group_workspace_bytes(ctypes.byref(a))
    assert need > lib.isa_topk_workspace_bytes(8, 1, 4096, 2048)
    a.ws, a.ws_bytes = A16 << 8, need - 1
    assert lib.isa_group_forward(ctypes.byref(a), None) == isa.ISA_ERR_WORKSPACE
    a.ws_bytes = need
    a.n_layers = 0
    assert lib.isa_group_forward(ctypes.byref(a), None) == isa.ISA_ERR_INVALID_ARG
    a.n_layers = 4
    a.k = 0
    assert lib.isa_group_forward(ctypes.byref(a), None) == isa.ISA_ERR_INVALID_ARG
    a.k = 2048
    a.per_layer_indexer = 1          # needs 4 indexer entries; the 1-entry arrays are too short,
    a.qI = None                      # so pass none at all and expect the NULL check
    assert lib.isa_group_forward(ctypes.byref(a), None) == isa.ISA_ERR_INVALID_ARG
    assert "indexer" in lib.isa_last_error().decode()
    # reuse_idx needs no indexer inputs and no score buffer
    a.per_layer_indexer = 0
    a.reuse_idx = 1
    assert lib.isa_group_workspace_bytes(ctypes.byref(a)) < need
    assert lib.isa_group_forward(None, None) == isa.ISA_ERR_INVALID_ARG
    # FP8 caches: the three arrays are required, C is not; shapes as for the call
    a.kv_fp8 = 1
    a.C = None
    assert lib.isa_group_forward(ctypes.byref(a), None) == isa.ISA_ERR_INVALID_ARG
    a.C8 = ctypes.cast(arr4, P); a.Ce = ctypes.cast((P * 4)(A4, A4, A4, A4), P)
    a.Cr = ctypes.cast(arr4, P)
    a.D_v = 448
    assert lib.isa_group_forward(ctypes.byref(a), None) == isa.ISA_ERR_UNSUPPORTED
    a.D_v = 512
    a.Cr = ctypes.cast((P * 4)(A16, A4, A16, A16), P)       # layer 1's RoPE slice misaligned
    assert lib.isa_group_forward(ctypes.byref(a), None) == isa.ISA_ERR_INVALID_ARG
    assert "fp8" in lib.isa_last_error().decode()
    # paged caches: the logical capacity must be max_blocks * block_size
    a.Cr = ctypes.cast(arr4, P)
    a.paged, a.block_table, a.max_blocks, a.block_size, a.n_pages = 1, A4, 32, 64, 600
    assert lib.isa_group_forward(ctypes.byref(a), None) == isa.ISA_ERR_INVALID_ARG
    assert "L_cap" in lib.isa_last_error().decode()
    a.block_size = 96
    assert lib.isa_group_forward(ctypes.byref(a), None) == isa.ISA_ERR_INVALID_ARG


def test_group_noalloc_rejects_calls_beyond_its_scratch(lib):
    # the 4096-query prefill's score buffer alone is 2.2 GB: far above the
    # fixed scratch, so the call stops at the host check (nothing launched)
    P = ctypes.c_void_p
    arr1 = (P * 1)(A16)
    arr4 = (P * 4)(A16, A16, A16, A16)
    a = isa.GroupArgs()
    a.B, a.Tq, a.L_cap, a.H_I, a.D_I, a.k = 1, 4096, 135168, 64, 128, 2048
    a.H, a.D, a.D_v, a.n_layers, a.sm_scale = 64, 576, 512, 4, 1 / 24
    a.qI = ctypes.cast(arr1, P); a.w = ctypes.cast((P * 1)(A4), P); a.kI = ctypes.cast(arr1, P)
    a.kv_len = A4
    a.Q = ctypes.cast(arr4, P); a.C = ctypes.cast(arr4, P); a.out = ctypes.cast(arr4, P)
    a.idx = A4
    assert lib.isa_group_noalloc_max_bytes() == 64 << 20
    assert lib.isa_group_workspace_bytes(ctypes.byref(a)) > lib.isa_group_noalloc_max_bytes()
    st, msg = _status(lib, "isa_group_forward_noalloc", ctypes.byref(a), None)
    assert st == isa.ISA_ERR_WORKSPACE and "scratch" in msg
    # argument errors are reported before the size check, as for isa_group_forward
    a.k = 0
    st, _ = _status(lib, "isa_group_forward_noalloc", ctypes.byref(a), None)
    assert st == isa.ISA_ERR_INVALID_ARG


def test_binding_fails_loudly_without_device():
    import torch
    x = torch.zeros(4, dtype=torch.int8)
    with pytest.raises(TypeError):
        isa.isa_indexer_scores(x, x, x, x)
