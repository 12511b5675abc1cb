"""The group call inside a HIP graph: a decode server captures its step once
and replays it.  The library allocates nothing and clears its counters with
a fill kernel (no memset node), so a captured group call must give, on every
replay, the bits of the same call run eagerly; replays are interleaved with
eager calls and synchronisations, and the outputs are overwritten before the
replays so that each replay has to rewrite them."""
import pytest
import torch

import long_context_sparse_indexshare_amd as isa
import synth
from _parity import dev

pytestmark = pytest.mark.gpu


def _calls(wl, n_inst, ws, reuse_from=None):
    calls = []
    for i in range(n_inst):
        inp = synth.group_inputs(wl.scaled(seed=wl.seed + 100 * i))
        d = {k: ([dev(x) for x in v] if isinstance(v, list) else dev(v)) for k, v in inp.items()}
        calls.append((d, isa.GroupCall([d["qI"]], [d["w"]], [d["kI"]], d["kv_len"], d["Q"], d["C"],
                                       wl.k, wl.D_v, wl.sm_scale, ws=ws)))
    return calls


@pytest.mark.parametrize("name,wl", [
    ("C2-8K", synth.WORKLOADS["C2"].scaled(name="C2-8K", kv_len=8000, L_cap=8192)),
    ("mq-B2-Tq8", synth.WORKLOADS["C2_128K_MQ8"].scaled(name="mq-B2-Tq8", B=2, kv_len=7000,
                                                         L_cap=7200)),
])
def test_group_replays_match_eager(name, wl):
    print("CASE graph", name, flush=True)
    ws = isa.Workspace()
    pairs = _calls(wl, 2, ws)
    calls = [c for _, c in pairs]
    # MTP-style follow-up on instance 0: new queries, the index set reused
    d0 = pairs[0][0]
    Q2 = [dev(q) for q in synth.group_inputs(wl.scaled(seed=wl.seed + 7))["Q"]]
    reuse = isa.GroupCall(None, None, None, d0["kv_len"], Q2, d0["C"], wl.k, wl.D_v, wl.sm_scale,
                          idx=calls[0].idx, reuse_idx=True, ws=ws)
    everything = calls + [reuse]
    for c in everything:
        c()
    torch.cuda.synchronize()
    ref = [(c.idx.clone(), [o.clone() for o in c.out]) for c in everything]

    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for c in everything:
            c()
    for r in range(3):
        for c in everything:
            c.idx.fill_(-7)
            for o in c.out:
                o.fill_(3.0)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for (ri, ro), c in zip(ref, everything):
            assert torch.equal(ri, c.idx), f"{name}: replay {r} index set differs"
            for l, (a, b) in enumerate(zip(ro, c.out)):
                assert torch.equal(a, b), f"{name}: replay {r} layer {l} differs"
        calls[r % 2]()                      # eager work between replays
        torch.cuda.synchronize()
