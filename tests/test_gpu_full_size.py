"""GPU parity at the workloads' full sizes, in the launch configuration the
benchmark times (one isa_group_forward call per group), against the oracle
on sampled sequences / query rows it can compute one by one in seconds.

Inputs are generated on the GPU by the seeded generators; the oracle gets host
copies of the sampled slices.  Indices are compared bit for bit, outputs to
the attention tolerance.  Covered: the 32K and 128K decode groups, sampled
rows of the 4096-query causal prefill, the 1M-context decode group with the
shared index set and with per-layer indexers (the ablation), the 7-step MTP
run that reuses the step-1 index set, and the 128K decode group with FP8
caches and with paged caches."""
import os

import pytest
import torch

import long_context_sparse_indexshare_amd as isa
import oracle
import synth
from _parity import assert_attn_close, assert_idx_equal, assert_scores_bitwise

pytestmark = pytest.mark.gpu


def _print_case(*a):
    print("CASE", *a, flush=True)


def _slice_b(inp, bs):
    """Host copies of sequences bs (a slice) of every input tensor."""
    out = {}
    for key, v in inp.items():
        if isinstance(v, list):
            out[key] = [x[bs].cpu() for x in v]
        else:
            out[key] = v[bs].cpu()
    return out


def _run_group(wl, d, **kw):
    _print_case("gpu group", wl.name, kw.get("per_layer_indexer", False))
    idx, outs, _ = isa.isa_group_forward([d["qI"]], [d["w"]], [d["kI"]], d["kv_len"], d["Q"],
                                         d["C"], wl.k, wl.D_v, wl.sm_scale, **kw)
    torch.cuda.synchronize()
    return idx, outs


def _parallel(fn, items):
    """fn over items in host threads (the oracle's C loops run outside the
    interpreter lock); results in item order."""
    from concurrent.futures import ThreadPoolExecutor
    with ThreadPoolExecutor(max_workers=max(1, min(16, os.cpu_count() or 1, len(items)))) as ex:
        return list(ex.map(fn, items))


def _check_sequences(wl, d, idx, outs, seqs):
    hs = {b: _slice_b(d, slice(b, b + 1)) for b in seqs}
    _print_case("oracle", wl.name, "sequences", seqs)
    refs = _parallel(lambda b: oracle.group_forward(
        [hs[b]["qI"]], [hs[b]["w"]], [hs[b]["kI"]], hs[b]["kv_len"], hs[b]["Q"], hs[b]["C"], wl.k,
        wl.D_v, wl.sm_scale), seqs)
    for b, (idx_ref, outs_ref, _) in zip(seqs, refs):
        assert_idx_equal(idx[b:b + 1], idx_ref, f"{wl.name} seq {b}")
        for l in range(wl.n_layers):
            assert_attn_close(outs[l][b:b + 1], outs_ref[l], f"{wl.name} seq {b} layer {l}")


@pytest.mark.parametrize("name,seqs", [("C2", list(range(8))), ("C2_128K", [0, 7])])
def test_decode_group_full_size(name, seqs):
    wl = synth.WORKLOADS[name]
    d = synth.group_inputs(wl, device="cuda")
    idx, outs = _run_group(wl, d)
    _check_sequences(wl, d, idx, outs, seqs)


def test_multi_query_decode_group_full_size():
    # 8 sequences x 8 queries at 128K: the indexer streams each key block once
    # for all 8 queries of a sequence
    wl = synth.WORKLOADS["C2_128K_MQ8"]
    d = synth.group_inputs(wl, device="cuda")
    idx, outs = _run_group(wl, d)
    _check_sequences(wl, d, idx, outs, [0, 7])


# rows of the 4096-query chunk checked against the oracle: 0, every 65th
# and 4095 (64 rows spread over the causal ramp)
C3_ROWS = sorted(set(range(0, 4096, 65)) | {4095})


def _oracle_rows(wl, d, rows, C):
    """Oracle group results of single query rows of sequence 0 (each over the
    keys it sees), computed in parallel host threads (the oracle's C loops run
    outside the interpreter lock)."""
    kI = d["kI"][0:1].cpu()
    inputs = {t: (torch.tensor([wl.kv_len - wl.Tq + t + 1], dtype=torch.int32),
                  d["qI"][0:1, t:t + 1].cpu(), d["w"][0:1, t:t + 1].cpu(),
                  [x[0:1, t:t + 1].cpu() for x in d["Q"]]) for t in rows}

    def one(t):
        kv, qI, w, Q = inputs[t]
        return t, oracle.group_forward([qI], [w], [kI], kv, Q, C, wl.k, wl.D_v, wl.sm_scale)

    return dict(_parallel(one, rows))


def test_prefill_group_full_size_sampled_rows():
    wl = synth.WORKLOADS["C3"]
    d = synth.group_inputs(wl, device="cuda")
    idx, outs = _run_group(wl, d)
    C = [x[0:1].cpu() for x in d["C"]]
    assert len(C3_ROWS) == 64
    _print_case("oracle C3 rows", C3_ROWS[:4], "...", len(C3_ROWS))
    refs = _oracle_rows(wl, d, C3_ROWS, C)
    for t in C3_ROWS:
        idx_ref, outs_ref, _ = refs[t]
        assert_idx_equal(idx[0:1, t:t + 1], idx_ref, f"C3 row {t}")
        for l in range(wl.n_layers):
            assert_attn_close(outs[l][0:1, t:t + 1], outs_ref[l], f"C3 row {t} layer {l}")


def test_prefill_scores_full_size_whole_rows_bitwise():
    # the indexer alone at the full prefill size (the launch the group call
    # makes): whole score rows, the -inf tail included, bit for bit
    wl = synth.WORKLOADS["C3"]
    d = synth.indexer_inputs(wl, device="cuda")
    _print_case("gpu indexer C3 full size")
    S = isa.isa_indexer_scores(d["qI"], d["w"], d["kI"], d["kv_len"])
    torch.cuda.synchronize()
    kI = d["kI"].cpu()
    for t in (0, 2047, 4095):
        _print_case("oracle C3 scores row", t)
        # as a single query over the full-length buffer: same position, same row
        kv = torch.tensor([wl.kv_len - wl.Tq + t + 1], dtype=torch.int32)
        ref = oracle.indexer_scores(d["qI"][:, t:t + 1].cpu(), d["w"][:, t:t + 1].cpu(), kI, kv)
        assert_scores_bitwise(S[:, t:t + 1], ref, f"C3 scores row {t}")


def test_1m_decode_shared_and_per_layer_indexer():
    wl = synth.WORKLOADS["C4"]
    d = synth.group_inputs(wl, device="cuda")
    idx, outs = _run_group(wl, d)
    _check_sequences(wl, d, idx, outs, [0, 1])
    # ablation: every layer its own indexer inputs; layer l attends over its own set
    abl = synth.ablation_indexers(wl, device="cuda")
    _print_case("gpu group C4 per-layer indexers")
    idx_pl, outs_pl, _ = isa.isa_group_forward([a["qI"] for a in abl], [a["w"] for a in abl],
                                               [a["kI"] for a in abl], d["kv_len"], d["Q"], d["C"],
                                               wl.k, wl.D_v, wl.sm_scale, per_layer_indexer=True)
    torch.cuda.synchronize()
    _print_case("oracle C4 per-layer indexers, sequences 0 and 1")

    host_in = {b: (_slice_b(d, slice(b, b + 1)), [_slice_b(a, slice(b, b + 1)) for a in abl])
               for b in (0, 1)}

    def per_layer_ref(b):
        h, ha = host_in[b]
        return oracle.group_forward([a["qI"] for a in ha], [a["w"] for a in ha],
                                    [a["kI"] for a in ha], h["kv_len"], h["Q"], h["C"], wl.k,
                                    wl.D_v, wl.sm_scale, per_layer_indexer=True)

    for b, (idx_ref, outs_ref, _) in zip((0, 1), _parallel(per_layer_ref, [0, 1])):
        assert_idx_equal(idx_pl[b:b + 1], idx_ref, f"C4 per-layer seq {b}: last layer's set")
        for l in range(wl.n_layers):
            assert_attn_close(outs_pl[l][b:b + 1], outs_ref[l], f"C4 per-layer seq {b} layer {l}")
    # the shared set differs from the last per-layer set (independent indexers)
    assert not torch.equal(idx_pl, idx)


def test_mtp_seven_steps_full_size():
    wl = synth.WORKLOADS["C5"]
    d = synth.group_inputs(wl, device="cuda")
    seqs = [0, wl.B - 1]
    hs = {b: _slice_b(d, slice(b, b + 1)) for b in seqs}   # host copies of the sampled sequences
    idx = None
    idx_ref = {}
    for step in range(1, wl.mtp_steps + 1):
        Qd = synth.mtp_queries(wl, step, device="cuda")
        _print_case("gpu mtp step", step)
        if step == 1:
            idx, outs, _ = isa.isa_group_forward([d["qI"]], [d["w"]], [d["kI"]], d["kv_len"], Qd,
                                                 d["C"], wl.k, wl.D_v, wl.sm_scale)
        else:
            before = idx.clone()
            _, outs, _ = isa.isa_group_forward(None, None, None, d["kv_len"], Qd, d["C"], wl.k,
                                               wl.D_v, wl.sm_scale, idx=idx, reuse_idx=True)
            torch.cuda.synchronize()
            assert torch.equal(idx, before), "reuse must not touch idx"
        torch.cuda.synchronize()
        for b in seqs:
            _print_case("oracle mtp step", step, "sequence", b)
            h = hs[b]
            Qh = [x[b:b + 1].cpu() for x in Qd]
            if step == 1:
                ir, outs_ref, _ = oracle.group_forward([h["qI"]], [h["w"]], [h["kI"]], h["kv_len"],
                                                       Qh, h["C"], wl.k, wl.D_v, wl.sm_scale)
                idx_ref[b] = ir
                assert_idx_equal(idx[b:b + 1], ir, f"mtp step 1 seq {b}")
            else:
                _, outs_ref, _ = oracle.group_forward(None, None, None, h["kv_len"], Qh, h["C"],
                                                      wl.k, wl.D_v, wl.sm_scale, idx=idx_ref[b],
                                                      reuse_idx=True)
            for l in range(wl.n_layers):
                assert_attn_close(outs[l][b:b + 1], outs_ref[l], f"mtp step {step} seq {b} layer {l}")


def test_fp8_cache_decode_group_full_size():
    # the 128K decode group with FP8 latent caches (as bench.py times it),
    # sampled sequences against the oracle's indexer, top-k and FP8 attention
    wl = synth.WORKLOADS["C2_128K"]
    d = synth.group_inputs(wl, device="cuda", kv8=True)
    _print_case("gpu group fp8", wl.name)
    idx, outs, _ = isa.isa_group_forward([d["qI"]], [d["w"]], [d["kI"]], d["kv_len"], d["Q"],
                                         None, wl.k, wl.D_v, wl.sm_scale,
                                         kv8=(d["C8"], d["Ce"], d["Cr"]))
    torch.cuda.synchronize()
    for b in (0, wl.B - 1):
        _print_case("oracle fp8", wl.name, "sequence", b)
        sl = slice(b, b + 1)
        S = oracle.indexer_scores(d["qI"][sl].cpu(), d["w"][sl].cpu(), d["kI"][sl].cpu(),
                                  d["kv_len"][sl].cpu())
        idx_ref = oracle.topk_select(S, d["kv_len"][sl].cpu(), wl.k)
        assert_idx_equal(idx[sl], idx_ref, f"fp8 seq {b}")
        for l in range(wl.n_layers):
            out_ref, _ = oracle.sparse_mla_attend_fp8(
                d["Q"][l][sl].cpu(), d["C8"][l][sl].cpu(), d["Ce"][l][sl].cpu(),
                d["Cr"][l][sl].cpu(), idx_ref, wl.sm_scale)
            assert_attn_close(outs[l][sl], out_ref, f"fp8 seq {b} layer {l}")


def test_paged_decode_group_full_size_equals_contiguous():
    # the 128K decode group over 64-token pages in a random order (as bench.py
    # times it) gives the contiguous group's bits; the contiguous group is
    # pinned to the oracle by test_decode_group_full_size
    wl = synth.WORKLOADS["C2_128K"]
    bs = 64
    d = synth.group_inputs(wl, device="cuda")
    idx, outs = _run_group(wl, d)
    g = torch.Generator(device="cuda").manual_seed(900)
    table = synth.page_layout(wl.B, wl.L_cap, bs, g, "cuda", extra_pages=64)
    n_pages = wl.B * (wl.L_cap // bs) + 64
    kI = synth.to_pages(d["kI"], table, bs, n_pages)
    C = [synth.to_pages(x, table, bs, n_pages) for x in d["C"]]
    _print_case("gpu group paged", wl.name, bs)
    idx_p, outs_p, _ = isa.isa_group_forward([d["qI"]], [d["w"]], [kI], d["kv_len"], d["Q"], C,
                                             wl.k, wl.D_v, wl.sm_scale, block_table=table)
    torch.cuda.synchronize()
    assert torch.equal(idx_p, idx), "paged index set differs"
    for l in range(wl.n_layers):
        assert torch.equal(outs_p[l], outs[l]), f"paged layer {l} differs"
