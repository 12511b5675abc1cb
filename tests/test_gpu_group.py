"""GPU parity of the IndexShare group entry point against the oracle, and the
group's invariants: one index set shared by every layer, each layer equal to
a standalone sparse layer fed that set, later MTP steps reusing the step-1
set, the per-layer-indexer baseline, and run-to-run determinism."""
import numpy as np
import pytest
import torch

import long_context_sparse_indexshare_amd as isa
import oracle
import synth
from _parity import assert_attn_close, assert_idx_equal, assert_lse_close, dev, guarded, host

pytestmark = pytest.mark.gpu


def _print_case(*a):
    print("CASE", *a, flush=True)


def _to_dev(inp):
    return {k: ([dev(x) for x in v] if isinstance(v, list) else dev(v)) for k, v in inp.items()}


SMALL = {
    "C1": synth.WORKLOADS["C1"],
    "C2-8K": synth.WORKLOADS["C2"].scaled(name="C2-8K", kv_len=8000, L_cap=8192),
    "decode-B3-Tq2": synth.WORKLOADS["C2"].scaled(name="decode-B3-Tq2", B=3, Tq=2, kv_len=6000,
                                                  L_cap=6100),
    "prefill-96": synth.WORKLOADS["C3"].scaled(name="prefill-96", Tq=96, kv_len=5000, L_cap=5000),
    # multi-query decode: 8 queries per sequence share each streamed key block
    "mq-decode-B2-Tq8": synth.WORKLOADS["C2_128K_MQ8"].scaled(name="mq-decode-B2-Tq8", B=2,
                                                             kv_len=7000, L_cap=7200),
}


@pytest.mark.parametrize("name", list(SMALL))
def test_group_matches_oracle(name):
    wl = SMALL[name]
    _print_case("group", wl)
    inp = synth.group_inputs(wl)
    idx_ref, outs_ref, lses_ref = oracle.group_forward([inp["qI"]], [inp["w"]], [inp["kI"]],
                                                       inp["kv_len"], inp["Q"], inp["C"], wl.k,
                                                       wl.D_v, wl.sm_scale)
    d = _to_dev(inp)
    # every output between canary pads
    idx_g, g_idx = guarded((wl.B, wl.Tq, wl.k), torch.int32)
    outs_g = [guarded((wl.B, wl.Tq, wl.H, wl.D_v), torch.bfloat16) for _ in range(wl.n_layers)]
    lse_g = [guarded((wl.B, wl.Tq, wl.H), torch.float32) for _ in range(wl.n_layers)]
    lse = [t for t, _ in lse_g]
    idx, outs, _ = isa.isa_group_forward([d["qI"]], [d["w"]], [d["kI"]], d["kv_len"], d["Q"],
                                         d["C"], wl.k, wl.D_v, wl.sm_scale, idx=idx_g,
                                         out=[t for t, _ in outs_g], lse=lse)
    torch.cuda.synchronize()
    g_idx.check(f"{name} idx")
    for l in range(wl.n_layers):
        outs_g[l][1].check(f"{name} out {l}")
        lse_g[l][1].check(f"{name} lse {l}")
    assert_idx_equal(idx, idx_ref, name)
    for l in range(wl.n_layers):
        assert_attn_close(outs[l], outs_ref[l], f"{name} layer {l}")
        assert_lse_close(lse[l], lses_ref[l], f"{name} layer {l}")

    # each layer equals a standalone sparse layer fed the same index set, bit for bit
    for l in range(wl.n_layers):
        o, _ = isa.isa_sparse_mla_attend(d["Q"][l], d["C"][l], idx, wl.D_v, wl.sm_scale)
        assert torch.equal(o, outs[l]), f"layer {l} differs from standalone"
    # and a second run gives identical bits (deterministic reductions)
    idx2, outs2, _ = isa.isa_group_forward([d["qI"]], [d["w"]], [d["kI"]], d["kv_len"], d["Q"],
                                           d["C"], wl.k, wl.D_v, wl.sm_scale)
    assert torch.equal(idx2, idx)
    for l in range(wl.n_layers):
        assert torch.equal(outs2[l], outs[l])


@pytest.mark.parametrize("name", ["C1", "C2-8K", "prefill-96"])
def test_group_fp8_cache_matches_oracle(name):
    # the layers' latent caches in FP8 (E4M3 codes, a power-of-two scale per
    # row, bf16 RoPE dims); the index set is computed and shared as before
    wl = SMALL[name]
    _print_case("group fp8", wl)
    inp = synth.group_inputs(wl, kv8=True)
    S = oracle.indexer_scores(inp["qI"], inp["w"], inp["kI"], inp["kv_len"])
    idx_ref = oracle.topk_select(S, inp["kv_len"], wl.k)
    d = _to_dev({k: v for k, v in inp.items() if v is not None})
    kv8 = (d["C8"], d["Ce"], d["Cr"])
    idx, outs, _ = isa.isa_group_forward([d["qI"]], [d["w"]], [d["kI"]], d["kv_len"], d["Q"], None,
                                         wl.k, wl.D_v, wl.sm_scale, kv8=kv8)
    torch.cuda.synchronize()
    assert_idx_equal(idx, idx_ref, name)
    for l in range(wl.n_layers):
        out_ref, _ = oracle.sparse_mla_attend_fp8(inp["Q"][l], inp["C8"][l], inp["Ce"][l],
                                                  inp["Cr"][l], idx_ref, wl.sm_scale)
        assert_attn_close(outs[l], out_ref, f"{name} fp8 layer {l}")
        o, _ = isa.isa_sparse_mla_attend_fp8(d["Q"][l], d["C8"][l], d["Ce"][l], d["Cr"][l], idx,
                                             wl.sm_scale)
        assert torch.equal(o, outs[l]), f"fp8 layer {l} differs from standalone"


@pytest.mark.parametrize("kv8", [False, True])
def test_group_paged_caches_equal_contiguous(kv8):
    # kI and every layer's cache in page pools (random page order, one table):
    # the same index set and the same outputs, bit for bit, as the contiguous
    # group on the logical caches
    wl = SMALL["C2-8K"]
    bs = 64
    _print_case("group paged", wl, bs, kv8)
    d = _to_dev({k: v for k, v in synth.group_inputs(wl, kv8=kv8).items() if v is not None})
    g = torch.Generator(device="cuda").manual_seed(77)
    table = synth.page_layout(wl.B, wl.L_cap, bs, g, "cuda", extra_pages=9)
    n_pages = wl.B * (wl.L_cap // bs) + 9
    pg = lambda x: synth.to_pages(x, table, bs, n_pages)
    kv = (d["C8"], d["Ce"], d["Cr"]) if kv8 else None
    kv_p = tuple([pg(x) for x in arr] for arr in kv) if kv8 else None
    idx_c, outs_c, _ = isa.isa_group_forward([d["qI"]], [d["w"]], [d["kI"]], d["kv_len"], d["Q"],
                                             None if kv8 else d["C"], wl.k, wl.D_v, wl.sm_scale,
                                             kv8=kv)
    idx_p, outs_p, _ = isa.isa_group_forward([d["qI"]], [d["w"]], [pg(d["kI"])], d["kv_len"],
                                             d["Q"], None if kv8 else [pg(x) for x in d["C"]],
                                             wl.k, wl.D_v, wl.sm_scale, kv8=kv_p,
                                             block_table=table)
    torch.cuda.synchronize()
    assert torch.equal(idx_p, idx_c)
    for l in range(wl.n_layers):
        assert torch.equal(outs_p[l], outs_c[l]), f"layer {l}"


def test_group_dense_causal_when_context_fits_k():
    # context <= k: every query keeps its whole causal prefix (dense attention)
    wl = synth.WORKLOADS["C1"].scaled(Tq=60, kv_len=60, L_cap=64)
    inp = synth.group_inputs(wl, layers=1)
    d = _to_dev(inp)
    idx, outs, _ = isa.isa_group_forward([d["qI"]], [d["w"]], [d["kI"]], d["kv_len"], d["Q"],
                                         d["C"], wl.k, wl.D_v, wl.sm_scale)
    want = np.full((1, wl.Tq, wl.k), -1, dtype=np.int32)
    for t in range(wl.Tq):
        want[0, t, : t + 1] = np.arange(t + 1)
    assert_idx_equal(idx, want, "dense")
    _, outs_ref, _ = oracle.group_forward([inp["qI"]], [inp["w"]], [inp["kI"]], inp["kv_len"],
                                          inp["Q"], inp["C"], wl.k, wl.D_v, wl.sm_scale)
    assert_attn_close(outs[0], outs_ref[0], "dense")


def test_mtp_steps_reuse_step1_index_set():
    wl = synth.WORKLOADS["C5"].scaled(B=4, kv_len=9000, L_cap=9000, mtp_steps=3)
    _print_case("mtp", wl)
    inp = synth.group_inputs(wl)
    d = _to_dev(inp)
    idx = None
    step_idx = []
    for step in range(1, wl.mtp_steps + 1):
        Qs = synth.mtp_queries(wl, step)
        Qd = [dev(x) for x in Qs]
        if step == 1:
            idx, outs, _ = isa.isa_group_forward([d["qI"]], [d["w"]], [d["kI"]], d["kv_len"], Qd,
                                                 d["C"], wl.k, wl.D_v, wl.sm_scale)
            idx_ref, outs_ref, _ = oracle.group_forward([inp["qI"]], [inp["w"]], [inp["kI"]],
                                                        inp["kv_len"], Qs, inp["C"], wl.k, wl.D_v,
                                                        wl.sm_scale)
            assert_idx_equal(idx, idx_ref, "mtp step 1")
        else:
            before = idx.clone()
            _, outs, _ = isa.isa_group_forward(None, None, None, d["kv_len"], Qd, d["C"], wl.k,
                                               wl.D_v, wl.sm_scale, idx=idx, reuse_idx=True)
            assert torch.equal(idx, before), "reuse must not touch idx"
            _, outs_ref, _ = oracle.group_forward(None, None, None, inp["kv_len"], Qs, inp["C"],
                                                  wl.k, wl.D_v, wl.sm_scale, idx=host(idx).numpy(),
                                                  reuse_idx=True)
        step_idx.append(host(idx).clone())
        for l in range(wl.n_layers):
            assert_attn_close(outs[l], outs_ref[l], f"mtp step {step} layer {l}")
    for s in step_idx[1:]:
        assert torch.equal(s, step_idx[0])


def test_per_layer_indexer_ablation():
    wl = synth.WORKLOADS["C4"].scaled(kv_len=7000, L_cap=7000)
    _print_case("ablation", wl)
    inp = synth.group_inputs(wl)
    ix = [synth.indexer_inputs(wl, seed=s) for s in wl.ablation_seeds]
    qI, w, kI = [x["qI"] for x in ix], [x["w"] for x in ix], [x["kI"] for x in ix]
    d = _to_dev(inp)
    idx, outs, _ = isa.isa_group_forward([dev(x) for x in qI], [dev(x) for x in w],
                                         [dev(x) for x in kI], d["kv_len"], d["Q"], d["C"], wl.k,
                                         wl.D_v, wl.sm_scale, per_layer_indexer=True)
    idx_ref, outs_ref, _ = oracle.group_forward(qI, w, kI, inp["kv_len"], inp["Q"], inp["C"],
                                                wl.k, wl.D_v, wl.sm_scale, per_layer_indexer=True)
    assert_idx_equal(idx, idx_ref, "ablation last layer")
    for l in range(wl.n_layers):
        assert_attn_close(outs[l], outs_ref[l], f"ablation layer {l}")
    # identical indexer inputs in every layer reproduce the shared group exactly
    n = wl.n_layers
    idx_a, outs_a, _ = isa.isa_group_forward([d["qI"]] * n, [d["w"]] * n, [d["kI"]] * n,
                                             d["kv_len"], d["Q"], d["C"], wl.k, wl.D_v,
                                             wl.sm_scale, per_layer_indexer=True)
    idx_s, outs_s, _ = isa.isa_group_forward([d["qI"]], [d["w"]], [d["kI"]], d["kv_len"], d["Q"],
                                             d["C"], wl.k, wl.D_v, wl.sm_scale)
    assert torch.equal(idx_a, idx_s)
    for l in range(n):
        assert torch.equal(outs_a[l], outs_s[l])


def test_groups_on_two_streams_use_separate_workspaces():
    # two groups launched at the same time on two streams with the default
    # workspaces (one per stream), against the same groups run one after the
    # other on the current stream: the bits must be equal
    wls = [SMALL["C2-8K"], SMALL["decode-B3-Tq2"]]
    ds = [_to_dev(synth.group_inputs(wl)) for wl in wls]

    def run(i, stream=None):
        wl, d = wls[i], ds[i]
        return isa.isa_group_forward([d["qI"]], [d["w"]], [d["kI"]], d["kv_len"], d["Q"], d["C"],
                                     wl.k, wl.D_v, wl.sm_scale, stream=stream)

    ref = [run(0), run(1)]
    torch.cuda.synchronize()
    ref = [(i.clone(), [o.clone() for o in outs]) for i, outs, _ in ref]
    streams = [torch.cuda.Stream(), torch.cuda.Stream()]
    for st in streams:
        st.wait_stream(torch.cuda.current_stream())
    for rep in range(3):
        got = [run(0, streams[0]), run(1, streams[1])]
        torch.cuda.synchronize()
        for (ri, ro), (gi, go, _) in zip(ref, got):
            assert torch.equal(ri, gi), f"rep {rep}: idx differs"
            for l in range(len(ro)):
                assert torch.equal(ro[l], go[l]), f"rep {rep}: layer {l} differs"


@pytest.mark.parametrize("name,wl,lens", [
    # decode: an empty sequence, one visible position, exactly k, a long one
    ("decode-mixed-lengths", synth.WORKLOADS["C2"].scaled(name="decode-mixed-lengths", B=4,
                                                         kv_len=5000, L_cap=5120),
     [0, 1, 2048, 5000]),
    # several queries per sequence: empty, shorter than the query count (the
    # first queries see nothing), dense within k, and past L_cap (clamped)
    ("multi-query-mixed-lengths", synth.WORKLOADS["C3"].scaled(name="multi-query-mixed-lengths", B=4,
                                                              Tq=16, kv_len=2990, L_cap=3000),
     [0, 10, 1500, 3500]),
])
def test_group_degenerate_lengths(name, wl, lens):
    """One group call over sequences of very different lengths (the edge cases
    of the causal visibility rule) against the oracle, every output guarded."""
    _print_case("group", name, lens)
    inp = synth.group_inputs(wl)
    inp["kv_len"] = torch.tensor(lens, dtype=torch.int32)
    idx_ref, outs_ref, lses_ref = oracle.group_forward([inp["qI"]], [inp["w"]], [inp["kI"]],
                                                       inp["kv_len"], inp["Q"], inp["C"], wl.k,
                                                       wl.D_v, wl.sm_scale)
    d = _to_dev(inp)
    idx_g, g_idx = guarded((wl.B, wl.Tq, wl.k), torch.int32)
    outs_g = [guarded((wl.B, wl.Tq, wl.H, wl.D_v), torch.bfloat16) for _ in range(wl.n_layers)]
    lse_g = [guarded((wl.B, wl.Tq, wl.H), torch.float32) for _ in range(wl.n_layers)]
    lse = [t for t, _ in lse_g]
    idx, outs, _ = isa.isa_group_forward([d["qI"]], [d["w"]], [d["kI"]], d["kv_len"], d["Q"],
                                         d["C"], wl.k, wl.D_v, wl.sm_scale, idx=idx_g,
                                         out=[t for t, _ in outs_g], lse=lse)
    torch.cuda.synchronize()
    g_idx.check(f"{name} idx")
    assert_idx_equal(idx, idx_ref, name)
    for l in range(wl.n_layers):
        outs_g[l][1].check(f"{name} out {l}")
        lse_g[l][1].check(f"{name} lse {l}")
        assert_attn_close(outs[l], outs_ref[l], f"{name} layer {l}")
        assert_lse_close(lse[l], lses_ref[l], f"{name} layer {l}")
