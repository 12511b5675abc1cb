"""isa_group_forward_noalloc (the group call on the library's fixed scratch
memory, for callers that cannot allocate) against isa_group_forward on the
same inputs: two calls in a row, the second with a smaller input, each
compared bit for bit (the same kernels run on the same data), which is within
the parity bar (indices exact, outputs within the attention tolerance)."""
import pytest
import torch

import long_context_sparse_indexshare_amd as isa
import synth

pytestmark = pytest.mark.gpu


def _print_case(*a):
    print("CASE", *a, flush=True)


CASES = [
    # a 128K-context decode group of 8 sequences, then a smaller 8K one
    synth.WORKLOADS["C2_128K"],
    synth.WORKLOADS["C2"].scaled(name="C2-8K-small", B=3, kv_len=8000, L_cap=8192),
]


def _inputs(wl):
    d = synth.group_inputs(wl, device="cuda")
    torch.cuda.synchronize()
    return d


def _group(fn, wl, d, **kw):
    return fn([d["qI"]], [d["w"]], [d["kI"]], d["kv_len"], d["Q"], d["C"], wl.k, wl.D_v,
              wl.sm_scale, **kw)


def test_noalloc_group_equals_workspace_group_on_two_calls():
    assert isa.isa_group_noalloc_max_bytes() == 64 << 20
    for wl in CASES:
        d = _inputs(wl)
        _print_case("noalloc group", wl.name)
        lse_n = [torch.empty(wl.B, wl.Tq, wl.H, device="cuda") for _ in range(wl.n_layers)]
        idx_n, outs_n, _ = _group(isa.isa_group_forward_noalloc, wl, d, lse=lse_n)
        torch.cuda.synchronize()
        _print_case("workspace group", wl.name)
        lse_w = [torch.empty(wl.B, wl.Tq, wl.H, device="cuda") for _ in range(wl.n_layers)]
        idx_w, outs_w, _ = _group(isa.isa_group_forward, wl, d, lse=lse_w)
        torch.cuda.synchronize()
        assert torch.equal(idx_n, idx_w), f"{wl.name}: index sets differ"
        for l in range(wl.n_layers):
            assert torch.equal(outs_n[l], outs_w[l]), f"{wl.name}: layer {l} output differs"
            assert torch.equal(lse_n[l], lse_w[l]), f"{wl.name}: layer {l} lse differs"


def test_noalloc_reuse_idx_step():
    # a later MTP draft step on the fixed scratch (attention only, reused set)
    wl = CASES[1]
    d = _inputs(wl)
    idx, _, _ = _group(isa.isa_group_forward, wl, d)
    Q2 = synth.mtp_queries(wl.scaled(mtp_steps=2), 2, device="cuda")
    _print_case("noalloc reuse step", wl.name)
    _, outs_n, _ = isa.isa_group_forward_noalloc(None, None, None, d["kv_len"], Q2, d["C"], wl.k,
                                                 wl.D_v, wl.sm_scale, idx=idx, reuse_idx=True)
    _, outs_w, _ = isa.isa_group_forward(None, None, None, d["kv_len"], Q2, d["C"], wl.k, wl.D_v,
                                         wl.sm_scale, idx=idx, reuse_idx=True)
    torch.cuda.synchronize()
    for l in range(wl.n_layers):
        assert torch.equal(outs_n[l], outs_w[l]), f"reuse step layer {l} differs"
