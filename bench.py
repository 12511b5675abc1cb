#!/usr/bin/env python3
"""IndexShare group benchmark on one MI355X.

A step is one IndexShare layer group: lightning indexer + top-k once, then
sparse latent attention in each of the 4 layers that share the index set.
The headline workload is the 128K-context decode group (batch 8, one query
token per sequence, 131072 cached tokens, 64x128 int8 indexer, top-2048,
4 layers of 64-head 576-wide bf16 latent attention).  The 4096-token
prefill chunk over a 131072-token cache (MFMA-bound) is measured as well and
reported under "prefill" (--no-prefill skips it).

Inputs are synthetic (synth/), generated on the GPU; decode steps rotate over
several independent input instances so the 256 MiB MALL cannot hold the
working set between steps.  Timing: W untimed warm-up steps, then exactly K
steps between two synchronised HIP events on the stream the library launches
on.  Each stage (indexer, top-k, one attention layer) is also timed alone,
back to back with HIP events and taking the input instances in turn, for its
roofline entry, and the headline groups are also captured once in a HIP
graph and replayed ("hip_graph"); "roofline" is the stage
that takes the largest share of a step (attention, four launches per group),
and the CPU oracle is timed on one group of the same workload on the host.

Prints one JSON line.
"""
from __future__ import annotations

import argparse
import json
import os
import platform
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = ("IndexShare group tokens/s (indexer+top-k+4 sparse MLA) at 128K ctx; "
          "% HBM/MFMA peak")
PEAK_HBM = 8.0e12          # bytes/s
PEAK_BF16 = 2.5e15         # dense bf16 MFMA, FLOP/s
PEAK_INT8 = 5.0e15         # dense int8 MFMA, OP/s


def visible_counts(wl):
    """Per query row: visible keys n = pos + 1 and selected rows min(k, n)."""
    rows = []
    for b in range(wl.B):
        for t in range(wl.Tq):
            n = max(min(wl.kv_len, wl.L_cap) - wl.Tq + t + 1, 0)
            rows.append(n)
    return rows


def algorithmic(wl, n_layers=None):
    """Bytes and ops the method must move/do per group (score and partial-output
    traffic excluded): kI, qI, w, Q, the selected latent rows, out, idx."""
    L = wl.n_layers if n_layers is None else n_layers
    ns = visible_counts(wl)
    rows = len(ns)
    pairs = sum(ns)
    sel = sum(min(wl.k, n) for n in ns)
    keys_read = wl.B * min(wl.kv_len, wl.L_cap)
    ix_bytes = keys_read * wl.D_I + rows * wl.H_I * (wl.D_I + 4)
    ix_ops = 2 * wl.H_I * wl.D_I * pairs
    topk_bytes = rows * wl.k * 4
    topk_read_bytes = sum(ns) * 4 + topk_bytes      # the scores once, the index sets
    at_bytes = sel * wl.D * 2 + rows * wl.H * (wl.D + wl.D_v) * 2
    # the same with every cache row read at most once (rows shared by several
    # queries' index sets counted once: at most the whole cache)
    at_bytes_once = (min(sel, keys_read) * wl.D * 2 + rows * wl.H * (wl.D + wl.D_v) * 2)
    at_flops = sel * wl.H * 2 * (wl.D + wl.D_v)
    t_ix = max(ix_ops / PEAK_INT8, ix_bytes / PEAK_HBM)
    t_at = max(at_flops / PEAK_BF16, at_bytes / PEAK_HBM)
    t_at_once = max(at_flops / PEAK_BF16, at_bytes_once / PEAK_HBM)
    t_ideal = t_ix + topk_bytes / PEAK_HBM + L * t_at
    t_ideal_once = t_ix + topk_bytes / PEAK_HBM + L * t_at_once
    return {"ix_bytes": ix_bytes, "ix_ops": ix_ops, "topk_bytes": topk_bytes,
            "topk_read_bytes": topk_read_bytes,
            "at_bytes_per_layer": at_bytes, "at_flops_per_layer": at_flops,
            "group_bytes": ix_bytes + topk_bytes + L * at_bytes,
            "t_ideal_s": t_ideal, "t_ix_s": t_ix, "t_at_s": t_at,
            "at_bytes_once_per_layer": at_bytes_once, "t_ideal_once_s": t_ideal_once,
            "ix_bound": "mfma" if ix_ops / PEAK_INT8 > ix_bytes / PEAK_HBM else "hbm",
            "at_bound": "mfma" if at_flops / PEAK_BF16 > at_bytes / PEAK_HBM else "hbm"}


def host_info():
    cpu = platform.processor()
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    cpu = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    ram_gib = None
    try:
        with open("/proc/meminfo") as f:
            for line in f:
                if line.startswith("MemTotal:"):
                    ram_gib = round(int(line.split()[1]) / (1 << 20), 1)
                    break
    except OSError:
        pass
    return cpu, os.cpu_count(), ram_gib


def make_instances(wl, n_inst, device):
    import synth
    insts = []
    for i in range(n_inst):
        inst = synth.group_inputs(wl.scaled(seed=wl.seed + 1000 * i), device=device)
        insts.append(inst)
    return insts


def time_group(isa, calls, steps, warmup, torch):
    for i in range(warmup):
        calls[i % len(calls)]()
    torch.cuda.synchronize()
    start = torch.cuda.Event(enable_timing=True)
    stop = torch.cuda.Event(enable_timing=True)
    start.record()
    for i in range(steps):
        calls[i % len(calls)]()
    stop.record()
    torch.cuda.synchronize()
    return start.elapsed_time(stop) / 1e3 / steps


def time_group_graph(calls, reps, torch):
    """The same groups captured once in a HIP graph (one replay runs every
    call in turn) and replayed reps times: time per group, and whether the
    replays rewrite the eager results bit for bit."""
    for c in calls:
        c()
    torch.cuda.synchronize()
    ref = [(c.idx.clone(), [o.clone() for o in c.out]) for c in calls]
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for c in calls:
            c()
    for c in calls:
        c.idx.fill_(-7)
    g.replay()
    torch.cuda.synchronize()
    equal = all(torch.equal(ri, c.idx) and all(torch.equal(a, b) for a, b in zip(ro, c.out))
                for (ri, ro), c in zip(ref, calls))
    a = torch.cuda.Event(enable_timing=True)
    b = torch.cuda.Event(enable_timing=True)
    a.record()
    for _ in range(reps):
        g.replay()
    b.record()
    torch.cuda.synchronize()
    del g
    return a.elapsed_time(b) / 1e3 / (reps * len(calls)), equal


def time_per_launch(fn, n, torch):
    """Average device duration of fn's launches: n launches back to back on the
    launch stream between one pair of HIP events (the events' own overhead is
    spread over the n launches).  fn may be a list of callables, taken in turn
    (independent input instances, so that caches do not carry one launch's
    inputs to the next)."""
    fns = fn if isinstance(fn, (list, tuple)) else [fn]
    for f in fns:
        f()
    torch.cuda.synchronize()
    a = torch.cuda.Event(enable_timing=True)
    b = torch.cuda.Event(enable_timing=True)
    a.record()
    for i in range(n):
        fns[i % len(fns)]()
    b.record()
    torch.cuda.synchronize()
    return a.elapsed_time(b) / 1e3 / n


def _raw(lib_fn, *args):
    """A prepared C-ABI call: the arguments are marshalled once, so the timed
    launches cost the host a few microseconds each and the host stays ahead of
    the GPU even for kernels of a few microseconds (the binding's per-call
    checks would otherwise be timed along with short launches)."""
    def call():
        st = lib_fn(*args)
        if st != 0:
            raise RuntimeError(f"isa call failed with status {st}")
    return call


def stage_times(isa, insts, wl, torch, reps=20):
    """Per-stage device time of one group, each stage timed alone, launches
    taking the input instances in turn (as the group steps do)."""
    S = [torch.empty((wl.B, wl.Tq, wl.L_cap), dtype=torch.float32, device="cuda")
         for _ in insts]
    idx = [torch.empty((wl.B, wl.Tq, wl.k), dtype=torch.int32, device="cuda") for _ in insts]
    lib = isa.load_library()
    stream = torch.cuda.current_stream().cuda_stream
    B, Tq, L_cap, k = wl.B, wl.Tq, wl.L_cap, wl.k
    tk_ws = torch.empty(max(isa.isa_topk_workspace_bytes(B, Tq, L_cap, k), 256), dtype=torch.uint8,
                        device="cuda")
    at_ws = torch.empty(max(isa.isa_attend_workspace_bytes(B, Tq, wl.H, wl.D, wl.D_v, k), 256),
                        dtype=torch.uint8, device="cuda")
    out = torch.empty((B, Tq, wl.H, wl.D_v), dtype=torch.bfloat16, device="cuda")

    def ix(i):
        d = insts[i]
        return _raw(lib.isa_indexer_scores, d["qI"].data_ptr(), d["w"].data_ptr(),
                    d["kI"].data_ptr(), d["kv_len"].data_ptr(), B, Tq, wl.H_I, wl.D_I, L_cap,
                    S[i].data_ptr(), stream)

    def tk(i):
        return _raw(lib.isa_topk_select, S[i].data_ptr(), insts[i]["kv_len"].data_ptr(), B, Tq,
                    L_cap, k, idx[i].data_ptr(), tk_ws.data_ptr(), tk_ws.numel(), stream)

    def at(i):
        d = insts[i]
        return _raw(lib.isa_sparse_mla_attend, d["Q"][0].data_ptr(), d["C"][0].data_ptr(),
                    idx[i].data_ptr(), B, Tq, wl.H, wl.D, wl.D_v, L_cap, k, float(wl.sm_scale),
                    out.data_ptr(), None, at_ws.data_ptr(), at_ws.numel(), stream)

    n = range(len(insts))
    t_ix = time_per_launch([ix(i) for i in n], reps, torch)    # also fills S
    t_tk = time_per_launch([tk(i) for i in n], reps, torch)    # also fills idx
    t_at = time_per_launch([at(i) for i in n], reps, torch)
    # access counts of the index set (the HiSparse input; not part of the step)
    counts = torch.zeros((B, L_cap), dtype=torch.int32, device="cuda")
    t_h = time_per_launch(_raw(lib.isa_index_histogram, idx[0].data_ptr(), B, Tq, k, L_cap,
                               counts.data_ptr(), stream), reps, torch)
    return t_ix, t_tk, t_at, t_h


def pin_one_core():
    """Pins the calling thread (the one that runs the single-threaded oracle)
    to one host core, as taskset -c would; returns (core, previous mask)."""
    prev = os.sched_getaffinity(0)
    core = max(prev)
    os.sched_setaffinity(0, {core})
    return core, prev


def unpin(core):
    os.sched_setaffinity(0, core[1])


def oracle_baseline(wl, inst, n_seq, torch, q_rows=None):
    """Times the CPU oracle on one group over a bounded sample of the workload."""
    import numpy as np

    import oracle
    sub = {}
    bs = slice(0, n_seq)
    if q_rows is None:
        sub["qI"] = inst["qI"][bs].cpu()
        sub["w"] = inst["w"][bs].cpu()
        sub["kv_len"] = inst["kv_len"][bs].cpu()
        sub["Q"] = [x[bs].cpu() for x in inst["Q"]]
        tokens = n_seq * wl.Tq
    else:
        # prefill sample: query rows q_rows of sequence 0, each with its own
        # visible length so that it sees exactly what it sees in the full chunk
        sub["qI"] = None
        tokens = len(q_rows)
    sub["kI"] = inst["kI"][bs].cpu()
    sub["C"] = [x[bs].cpu() for x in inst["C"]]
    if q_rows is not None:
        # host copies of the sampled rows' inputs, made before the timed region
        rows_in = [(torch.tensor([wl.kv_len - wl.Tq + t + 1], dtype=torch.int32),
                    inst["qI"][0:1, t:t + 1].cpu(), inst["w"][0:1, t:t + 1].cpu(),
                    [x[0:1, t:t + 1].cpu() for x in inst["Q"]]) for t in q_rows]
    core = pin_one_core()
    t0 = time.perf_counter()
    if q_rows is None:
        idx, outs, _ = oracle.group_forward([sub["qI"]], [sub["w"]], [sub["kI"]], sub["kv_len"],
                                            sub["Q"], sub["C"], wl.k, wl.D_v, wl.sm_scale)
        results = (idx, outs)
    else:
        results = []
        for kv, qI, w, Q in rows_in:
            results.append(oracle.group_forward([qI], [w], [sub["kI"]], kv, Q, sub["C"], wl.k,
                                                wl.D_v, wl.sm_scale))
    dt = time.perf_counter() - t0
    unpin(core)
    return tokens, dt, results, core[0]


# committed counter summaries: stage -> (summary file, kernel source it was taken on;
# the digest covers that file followed by the header every kernel source includes)
TRAFFIC = {
    "indexer": ("indexer_scores_C2_128K_traffic.txt", "indexer.hip"),
    "attend": ("sparse_attend_C2_128K_traffic.txt", "attend.hip"),
    "topk": ("topk_C2_128K_traffic.txt", "topk.hip"),
}


SHARED_HEADER = "isa_internal.h"


def source_digest(path):
    """sha256 of a kernel source followed by the shared internal header."""
    import hashlib
    h = hashlib.sha256()
    for p in (path, os.path.join(os.path.dirname(path), SHARED_HEADER)):
        with open(p, "rb") as f:
            h.update(f.read())
    return h.hexdigest()


def measured_traffic(stage):
    """HBM bytes per launch of a stage from its committed counter summary, or
    None when there is none or the kernel source changed since it was taken."""
    if stage not in TRAFFIC:
        return None
    fname, srcname = TRAFFIC[stage]
    try:
        with open(os.path.join(ROOT, "profiles", fname)) as f:
            kv = dict(line.split(":", 1) for line in f if ":" in line and not line.startswith("#"))
    except OSError:
        return None
    src = os.path.join(ROOT, "long_context_sparse_indexshare_amd", "csrc", srcname)
    if kv.get("source_sha256", "").strip() != source_digest(src):
        return None
    return float(kv["traffic_bytes_per_launch"])


def mtp_calls(isa, wl, d, Qs, ws):
    """The 7-step MTP run: step 1 a whole group (indexer, top-k, 4 layers),
    steps 2-7 the 4 layers alone on the same index set."""
    first = isa.GroupCall([d["qI"]], [d["w"]], [d["kI"]], d["kv_len"], Qs[0], d["C"], wl.k,
                          wl.D_v, wl.sm_scale, ws=ws)
    later = [isa.GroupCall(None, None, None, d["kv_len"], Qs[s], d["C"], wl.k, wl.D_v,
                           wl.sm_scale, idx=first.idx, reuse_idx=True, ws=ws)
             for s in range(1, wl.mtp_steps)]

    def run():
        first()
        for c in later:
            c()
    return run


def mtp_roofline(wl):
    """(algorithmic bytes, ideal seconds) of the 7-step MTP run: one indexer +
    top-k, then 7 x 4 attention layers on the same index set.  Rows that stay
    in the 256 MB MALL between steps can make the measured fraction exceed 1."""
    a = algorithmic(wl)
    later_layers = (wl.mtp_steps - 1) * wl.n_layers
    return (a["group_bytes"] + later_layers * a["at_bytes_per_layer"],
            a["t_ideal_s"] + later_layers * a["t_at_s"])


def calibration_copy(torch):
    """A 1 GiB device copy: its counters calibrate the traffic figures."""
    src = torch.empty(1 << 30, dtype=torch.uint8, device="cuda")
    dst = torch.empty_like(src)
    dst.copy_(src)
    torch.cuda.synchronize()
    del src, dst


def run_stage(isa, wl, stage, reps, torch):
    """One stage alone on one input instance, for profiler runs (one JSON line).
    "mtp" runs the whole 7-step sequence of the C5 workload (one warm-up run,
    then reps timed runs)."""
    import synth
    d = synth.group_inputs(wl, device="cuda")
    if stage == "mtp":
        Qs = [synth.mtp_queries(wl, s, device="cuda") for s in range(1, wl.mtp_steps + 1)]
        run = mtp_calls(isa, wl, d, Qs, isa.Workspace())
        calibration_copy(torch)
        run()
        torch.cuda.synchronize()
        t = time_per_launch(run, reps, torch)
        print(json.dumps({"stage": stage, "workload": wl.name, "reps": reps,
                          "avg_us_per_7_steps": t * 1e6}), flush=True)
        return
    S = torch.empty((wl.B, wl.Tq, wl.L_cap), dtype=torch.float32, device="cuda")
    idx = torch.empty((wl.B, wl.Tq, wl.k), dtype=torch.int32, device="cuda")
    out = torch.empty((wl.B, wl.Tq, wl.H, wl.D_v), dtype=torch.bfloat16, device="cuda")
    ws = isa.Workspace()
    if stage in ("indexer", "attend", "topk"):
        calibration_copy(torch)
    isa.isa_indexer_scores(d["qI"], d["w"], d["kI"], d["kv_len"], S=S)
    isa.isa_topk_select(S, d["kv_len"], wl.k, idx=idx, ws=ws)
    torch.cuda.synchronize()
    fns = {
        "indexer": lambda: isa.isa_indexer_scores(d["qI"], d["w"], d["kI"], d["kv_len"], S=S),
        "topk": lambda: isa.isa_topk_select(S, d["kv_len"], wl.k, idx=idx, ws=ws),
        "attend": lambda: isa.isa_sparse_mla_attend(d["Q"][0], d["C"][0], idx, wl.D_v,
                                                    wl.sm_scale, out=out, ws=ws),
    }
    if stage == "group":
        call = isa.GroupCall([d["qI"]], [d["w"]], [d["kI"]], d["kv_len"], d["Q"], d["C"], wl.k,
                             wl.D_v, wl.sm_scale, ws=ws)
        fn = call
    else:
        fn = fns[stage]
    t = time_per_launch(fn, reps, torch)
    print(json.dumps({"stage": stage, "workload": wl.name, "reps": reps, "avg_us": t * 1e6}),
          flush=True)


def run_ablation(isa, torch, steps, warmup):
    """C4 (2 x 1M context): the shared index set vs an indexer + top-k per layer
    (the IndexShare saving), each timed over whole groups."""
    import synth
    wl = synth.WORKLOADS["C4"]
    log("C4: generating inputs (shared and per-layer indexers)")
    d = synth.group_inputs(wl, device="cuda")
    abl = synth.ablation_indexers(wl, device="cuda")
    ws = isa.Workspace()
    shared = isa.GroupCall([d["qI"]], [d["w"]], [d["kI"]], d["kv_len"], d["Q"], d["C"], wl.k,
                           wl.D_v, wl.sm_scale, ws=ws)
    per_layer = isa.GroupCall([a["qI"] for a in abl], [a["w"] for a in abl], [a["kI"] for a in abl],
                              d["kv_len"], d["Q"], d["C"], wl.k, wl.D_v, wl.sm_scale,
                              per_layer_indexer=True, ws=ws)
    t_sh = time_group(isa, [shared], steps, warmup, torch)
    t_pl = time_group(isa, [per_layer], steps, warmup, torch)
    a = algorithmic(wl)
    ix_topk_bytes = a["ix_bytes"] + a["topk_bytes"]
    bytes_sh = a["group_bytes"]
    bytes_pl = bytes_sh + (wl.n_layers - 1) * ix_topk_bytes
    # per-token FLOPs of the group, indexer (16384 per key) vs attention
    F_I = 2 * wl.H_I * wl.D_I * wl.kv_len
    F_A = a["at_flops_per_layer"] / wl.B
    # ideal times: the shared group's, and the same with an indexer + top-k per layer
    t_ideal_sh = a["t_ideal_s"]
    t_ideal_pl = t_ideal_sh + (wl.n_layers - 1) * (a["t_ix_s"] + a["topk_bytes"] / PEAK_HBM)
    del shared, per_layer, d, abl
    torch.cuda.empty_cache()
    return {"workload": "C4: 2 sequences x 1 query, context 1048576, 4 layers",
            "shared_us_per_group": t_sh * 1e6, "per_layer_us_per_group": t_pl * 1e6,
            "t_ideal_us_shared": t_ideal_sh * 1e6, "frac_of_roofline_shared": t_ideal_sh / t_sh,
            "t_ideal_us_per_layer": t_ideal_pl * 1e6, "frac_of_roofline_per_layer": t_ideal_pl / t_pl,
            "measured_ratio": t_pl / t_sh,
            "algorithmic_bytes_ratio": bytes_pl / bytes_sh,
            "group_flops_ratio": (4 * F_I + 4 * F_A) / (F_I + 4 * F_A),
            "pages_claim": "2.9x lower compute overhead (whole model, 1M context, no hardware "
                           "stated; context, not a target)"}


def run_mtp(isa, torch, reps):
    """C5: 7 sequential MTP draft steps on 16 x 262144 contexts; the index set
    is computed at step 1 and reused by steps 2-7 (every step attends in 4
    layers with its own queries), compared with recomputing it every step."""
    import synth
    wl = synth.WORKLOADS["C5"]
    log("C5: generating inputs")
    d = synth.group_inputs(wl, device="cuda")
    Qs = [synth.mtp_queries(wl, s, device="cuda") for s in range(1, wl.mtp_steps + 1)]
    ws = isa.Workspace()
    run_reuse = mtp_calls(isa, wl, d, Qs, ws)
    again = [isa.GroupCall([d["qI"]], [d["w"]], [d["kI"]], d["kv_len"], Qs[s], d["C"], wl.k,
                           wl.D_v, wl.sm_scale, ws=ws) for s in range(wl.mtp_steps)]

    def run_recompute():
        for c in again:
            c()

    t_reuse = time_group(isa, [run_reuse], reps, 2, torch)
    t_recompute = time_group(isa, [run_recompute], reps, 2, torch)
    tokens = wl.B * wl.mtp_steps
    del run_reuse, again, d, Qs
    torch.cuda.empty_cache()
    alg_bytes, t_ideal = mtp_roofline(wl)
    return {"workload": "C5: 16 sequences x 262144 context, 7 draft steps, 4 layers",
            "tokens_per_s": tokens / t_reuse, "ms_per_7_steps": t_reuse * 1e3,
            "ms_per_7_steps_recomputing_index": t_recompute * 1e3,
            "reuse_speedup": t_recompute / t_reuse,
            "algorithmic_bytes_per_7_steps": alg_bytes, "t_ideal_us": t_ideal * 1e6,
            "frac_of_roofline": t_ideal / t_reuse}


def run_fp8_kv(isa, torch, steps, warmup, n_inst):
    """The C2_128K decode group with FP8 latent caches (E4M3 codes, one
    power-of-two scale byte per row, bf16 RoPE dims): whole groups and one
    attention layer alone, against that layer's algorithmic bytes."""
    import synth
    wl = synth.WORKLOADS["C2_128K"]
    log("C2_128K fp8: generating inputs")
    insts = [synth.group_inputs(wl.scaled(seed=wl.seed + 1000 * i), device="cuda", kv8=True)
             for i in range(n_inst)]
    torch.cuda.synchronize()
    ws = isa.Workspace()
    calls = [isa.GroupCall([d["qI"]], [d["w"]], [d["kI"]], d["kv_len"], d["Q"], None, wl.k,
                           wl.D_v, wl.sm_scale, ws=ws, kv8=(d["C8"], d["Ce"], d["Cr"]))
             for d in insts]
    t = time_group(isa, calls, steps, warmup, torch)
    out = torch.empty((wl.B, wl.Tq, wl.H, wl.D_v), dtype=torch.bfloat16, device="cuda")

    def at(d, c):
        return lambda: isa.isa_sparse_mla_attend_fp8(d["Q"][0], d["C8"][0], d["Ce"][0], d["Cr"][0],
                                                     c.idx, wl.sm_scale, out=out, ws=ws)

    t_at = time_per_launch([at(d, c) for d, c in zip(insts, calls)], 20, torch)
    a = algorithmic(wl)
    row_bytes = wl.D_v + 1 + (wl.D - wl.D_v) * 2          # codes, scale byte, RoPE dims
    sel = wl.B * wl.Tq * min(wl.k, wl.kv_len)
    at_bytes = sel * row_bytes + wl.B * wl.Tq * wl.H * (wl.D + wl.D_v) * 2
    t_ideal = a["t_ix_s"] + a["topk_bytes"] / PEAK_HBM + wl.n_layers * at_bytes / PEAK_HBM
    del calls, insts
    torch.cuda.empty_cache()
    return {"workload": "C2_128K decode group with FP8 latent caches (E4M3 + per-row "
                        "power-of-two scale, bf16 RoPE)",
            "tokens_per_s": wl.tokens_per_group / t, "ms_per_step": t * 1e3,
            "attend_us_per_layer": t_at * 1e6, "attend_algorithmic_bytes": at_bytes,
            "attend_frac_hbm": at_bytes / t_at / PEAK_HBM,
            "group_frac_of_roofline": t_ideal / t}


def run_paged(isa, torch, steps, warmup, n_inst, block_size=64):
    """The C2_128K decode group over paged caches: kI and every layer's
    latent cache in pools of block_size-token pages, placed in a random
    order through one block table per instance."""
    import synth
    wl = synth.WORKLOADS["C2_128K"]
    log(f"C2_128K paged ({block_size}-token pages): generating inputs")
    calls, keep = [], []
    ws = isa.Workspace()
    for i in range(n_inst):
        d = synth.group_inputs(wl.scaled(seed=wl.seed + 1000 * i), device="cuda")
        g = torch.Generator(device="cuda").manual_seed(900 + i)
        table = synth.page_layout(wl.B, wl.L_cap, block_size, g, "cuda", extra_pages=64)
        n_pages = wl.B * (wl.L_cap // block_size) + 64
        kI = synth.to_pages(d["kI"], table, block_size, n_pages)
        C = [synth.to_pages(x, table, block_size, n_pages) for x in d["C"]]
        del d["kI"], d["C"]
        keep.append((d, kI, C, table))
        calls.append(isa.GroupCall([d["qI"]], [d["w"]], [kI], d["kv_len"], d["Q"], C, wl.k,
                                   wl.D_v, wl.sm_scale, ws=ws, block_table=table))
    torch.cuda.synchronize()
    t = time_group(isa, calls, steps, warmup, torch)
    a = algorithmic(wl)
    del calls, keep
    torch.cuda.empty_cache()
    return {"workload": f"C2_128K decode group, caches in {block_size}-token pages placed in a "
                        "random order",
            "tokens_per_s": wl.tokens_per_group / t, "ms_per_step": t * 1e3,
            "frac_of_roofline": a["t_ideal_s"] / t}


def run_prefill(isa, torch, args, cpu_name, ncpu):
    """C3: 4096 queries appended to a 131072-token cache (causal), 64x128 int8
    indexer, top-2048, 4 layers.  The bound is MFMA: T_ideal counts the
    indexer's int8 ops at the int8 peak and the attention's bf16 FLOP at the
    bf16 peak, each cache row read once (a layer's 156 MB cache is gathered
    about 62 times over by the 4096 queries and stays in the 256 MB MALL);
    the same with every query's gathered rows charged to HBM is reported
    too."""
    import synth
    wp = synth.WORKLOADS["C3"]
    # stratified sample of the chunk's rows for the oracle: first, last and
    # evenly spaced ones (bounded to keep the CPU leg near 20 s)
    q_rows = None if args.no_cpu_baseline else [0, 4095] + list(range(455, 4095, 455))
    pre = run_workload(isa, wp, max(2, min(args.steps, 5)), 2, 1, torch, q_rows=q_rows)
    a = pre["alg"]
    tp = pre["t_step"]
    st = pre["stages_us"]
    t_ix, t_tk, t_at = st["indexer"] * 1e-6, st["topk"] * 1e-6, st["attend_per_layer"] * 1e-6
    # per-stage MFMA fractions against the dense peaks
    ix_frac = a["ix_ops"] / t_ix / PEAK_INT8
    at_frac = a["at_flops_per_layer"] / t_at / PEAK_BF16
    t_ideal_mfma = a["ix_ops"] / PEAK_INT8 + wp.n_layers * a["at_flops_per_layer"] / PEAK_BF16
    res = {
        "workload": "C3 prefill group: 4096 queries over a 135168-token cache (causal), "
                    "64x128 int8 indexer, top-2048, 4 layers x 64 heads x 576 bf16 latent",
        "tokens_per_s": wp.tokens_per_group / tp, "ms_per_step": tp * 1e3,
        # primary: MFMA-bound, each cache row counted once
        "t_ideal_ms": a["t_ideal_once_s"] * 1e3, "frac_of_roofline": a["t_ideal_once_s"] / tp,
        "t_ideal_mfma_only_ms": t_ideal_mfma * 1e3,
        "roofline": {"bound": "mfma", "achieved": (a["ix_ops"] + wp.n_layers *
                                                   a["at_flops_per_layer"]) / tp / 1e12,
                     "unit": "TOP/s (int8 + bf16)",
                     "note": "frac = T_ideal / T_measured, T_ideal = int8 ops / 5.0 POP/s + "
                             "top-k index bytes / 8 TB/s + 4 x bf16 FLOP / 2.5 PFLOP/s"},
        # secondary: every query's gathered rows charged to HBM
        "t_ideal_ms_rows_per_query": a["t_ideal_s"] * 1e3,
        "frac_of_roofline_rows_per_query": a["t_ideal_s"] / tp,
        "stages_us": st,
        "stage_rooflines": {
            "indexer": {"bound": "mfma", "dtype": "int8", "launch_us": st["indexer"],
                        "ops": a["ix_ops"], "achieved_TOPS": a["ix_ops"] / t_ix / 1e12,
                        "peak_TOPS": PEAK_INT8 / 1e12, "frac": ix_frac},
            "topk": {"bound": "hbm", "launch_us": st["topk"],
                     "algorithmic_bytes": a["topk_read_bytes"],
                     "achieved_GBps": a["topk_read_bytes"] / t_tk / 1e9,
                     "frac": a["topk_read_bytes"] / t_tk / PEAK_HBM},
            "attend": {"bound": "mfma", "dtype": "bf16", "launch_us": st["attend_per_layer"],
                       "flops": a["at_flops_per_layer"],
                       "achieved_TFLOPS": a["at_flops_per_layer"] / t_at / 1e12,
                       "peak_TFLOPS": PEAK_BF16 / 1e12, "frac": at_frac,
                       "gathered_bytes": a["at_bytes_per_layer"],
                       "gathered_GBps": a["at_bytes_per_layer"] / t_at / 1e9},
        },
        "index_histogram_us": pre["index_histogram_us"],
    }
    if "oracle" in pre:
        o = pre["oracle"]
        res["cpu_baseline"] = {
            "value": o["tokens"] / o["seconds"], "unit": "tokens/s", "cores": 1,
            "kind": "oracle",
            "sample": f"{len(q_rows)} query rows of the chunk (0, 4095 and every 455th), each "
                      f"over the keys it sees, on one host core (core {o['core']}, pinned) of "
                      f"{cpu_name} ({ncpu} cpus)",
            "seconds": o["seconds"], "idx_exact": o["idx_exact"],
            "max_abs_err_vs_gpu": o["max_abs_err"]}
    return res


def measured_peaks(torch):
    """Attainable rates on this GPU from the probe kernels of
    long_context_sparse_indexshare_amd/peaks/peaks.hip (dense MFMA loops,
    an LDS read loop, a streaming HBM read), each timed with HIP events on
    the launch stream after one warm-up launch.  Context for the roofline
    fractions, which use the published peaks."""
    import ctypes
    path = os.path.join(ROOT, "long_context_sparse_indexshare_amd", "peaks", "libisa_peaks.so")
    if not os.path.exists(path):
        return None
    lib = ctypes.CDLL(path)
    P, I, Z = ctypes.c_void_p, ctypes.c_int, ctypes.c_size_t
    for name in ("peaks_mfma_bf16", "peaks_mfma_fp8", "peaks_mfma_i8", "peaks_lds_read"):
        getattr(lib, name).argtypes = [P, I, I, P]
        getattr(lib, name).restype = I
    lib.peaks_hbm_read.argtypes = [P, Z, P, I, P]
    lib.peaks_hbm_read.restype = I
    grid = 1024
    sink = torch.empty(grid * 1024, dtype=torch.float32, device="cuda")
    stream = torch.cuda.current_stream().cuda_stream

    def timed(fn):
        fn()
        torch.cuda.synchronize()
        return time_per_launch(fn, 3, torch)

    out = {}
    # (probe, iterations, work per (wave, iteration, chain) MFMA)
    for name, iters, per in (("bf16", 2000, 32768), ("fp8", 1000, 131072), ("int8", 2000, 65536)):
        fn = getattr(lib, f"peaks_mfma_{name if name != 'int8' else 'i8'}")
        t = timed(lambda: fn(sink.data_ptr(), grid, iters, stream))
        out[f"mfma_{name}_TFLOPS"] = grid * 8 * iters * 4 * per / t / 1e12
    t = timed(lambda: lib.peaks_lds_read(sink.data_ptr(), grid, 2000, stream))
    lds = grid * 1024 * 2000 * 8 * 16 / t
    out["lds_read_TBps"] = lds / 1e12
    out["lds_read_bytes_per_clk_per_cu"] = lds / 256 / 2.4e9
    buf = torch.empty(1 << 31, dtype=torch.uint8, device="cuda")
    t = timed(lambda: lib.peaks_hbm_read(buf.data_ptr(), buf.numel() // 16, sink.data_ptr(),
                                         256 * 8, stream))
    out["hbm_read_GBps"] = buf.numel() / t / 1e9
    del buf, sink
    torch.cuda.empty_cache()
    out["note"] = ("probe kernels in long_context_sparse_indexshare_amd/peaks/peaks.hip; "
                   "2.4 GHz and 256 CUs assumed for the per-CU LDS figure")
    return out


def log(*a):
    print("[bench]", *a, file=sys.stderr, flush=True)


def run_workload(isa, wl, steps, warmup, n_inst, torch, baseline_seq=None, q_rows=None,
                 graph=False):
    import numpy as np
    log(f"{wl.name}: generating {n_inst} input instance(s) on the GPU")
    insts = make_instances(wl, n_inst, "cuda")
    torch.cuda.synchronize()
    log(f"{wl.name}: timing {warmup} warm-up + {steps} steps")
    ws = isa.Workspace()
    calls = [isa.GroupCall([d["qI"]], [d["w"]], [d["kI"]], d["kv_len"], d["Q"], d["C"], wl.k,
                           wl.D_v, wl.sm_scale, ws=ws) for d in insts]
    t_step = time_group(isa, calls, steps, warmup, torch)
    # the same groups reusing each instance's index set (attention layers
    # only): the difference is what the indexer and the top-k take inside the
    # group (the indexer's epilogue writing the summary, the top-k reading it)
    reuse = [isa.GroupCall([], [], [], d["kv_len"], d["Q"], d["C"], wl.k, wl.D_v, wl.sm_scale,
                           idx=c.idx, reuse_idx=True, ws=ws) for c, d in zip(calls, insts)]
    t_reuse = time_group(isa, reuse, steps, warmup, torch)
    t_graph, graph_equal = (time_group_graph(calls, max(1, steps // len(calls)), torch)
                            if graph else (None, None))
    alg = algorithmic(wl)
    log(f"{wl.name}: {t_step * 1e6:.1f} us/step; timing stages")
    t_ix, t_tk, t_at, t_h = stage_times(isa, insts, wl, torch)
    res = {
        "t_step": t_step, "alg": alg, "t_graph": t_graph, "graph_equal": graph_equal,
        "stages_us": {"indexer": t_ix * 1e6, "topk": t_tk * 1e6, "attend_per_layer": t_at * 1e6},
        "group_index_us": (t_step - t_reuse) * 1e6,
        "index_histogram_us": t_h * 1e6,
    }
    # CPU oracle on a bounded sample of the same workload, plus a parity spot check
    if baseline_seq or q_rows:
        calls[0]()
        torch.cuda.synchronize()
        gidx = calls[0].idx.cpu().numpy()
        gout = [o.double().cpu().numpy() for o in calls[0].out]
        log(f"{wl.name}: timing the CPU oracle on a sample")
        tokens, dt, results, core = oracle_baseline(wl, insts[0], baseline_seq or 1, torch, q_rows)
        log(f"{wl.name}: oracle {dt:.1f} s for {tokens} token(s) on core {core}")
        if q_rows is None:
            idx, outs = results
            exact = bool(np.array_equal(gidx[: baseline_seq], idx))
            errs = [float(np.abs(gout[l][: baseline_seq] - outs[l]).max()) for l in range(len(outs))]
        else:
            exact = all(np.array_equal(gidx[0, t], r[0][0, 0]) for t, r in zip(q_rows, results))
            errs = [max(float(np.abs(gout[l][0, t] - r[1][l][0, 0]).max())
                        for t, r in zip(q_rows, results)) for l in range(wl.n_layers)]
        res["oracle"] = {"tokens": tokens, "seconds": dt, "idx_exact": exact,
                         "max_abs_err": max(errs), "core": core}
    del calls, insts
    torch.cuda.empty_cache()
    return res


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=100)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--instances", type=int, default=4)
    ap.add_argument("--no-prefill", action="store_true",
                    help="skip the 4K x 128K prefill group (measured by default)")
    ap.add_argument("--no-extra", action="store_true",
                    help="skip the 1M-context ablation, the 7-step MTP, the FP8-cache, the "
                         "paged-cache, the 32K-context decode and the multi-query measurements")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--stage", choices=["indexer", "topk", "attend", "group", "mtp"],
                    help="profiling mode: run one stage of --workload --reps times and print "
                         "its average launch time instead of the benchmark line (mtp: the "
                         "7-step run of C5)")
    ap.add_argument("--workload", default="C2_128K")
    ap.add_argument("--reps", type=int, default=5)
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU: this build has no multi-GPU path "
              "(only the one-GPU share of the work is built)", file=sys.stderr)
        sys.exit(2)

    import torch

    import long_context_sparse_indexshare_amd as isa
    import synth
    if not os.path.exists(isa.LIB_PATH):
        import __graft_entry__
        __graft_entry__.build()
    isa.load_library()
    torch.cuda.set_device(0)
    if args.stage:
        name = "C5" if args.stage == "mtp" else args.workload
        run_stage(isa, synth.WORKLOADS[name], args.stage, args.reps, torch)
        return

    # reference: what a plain device copy reaches on this machine (context for the
    # roofline fractions, which use the published 8 TB/s)
    src = torch.empty(1 << 30, dtype=torch.uint8, device="cuda")
    dst = torch.empty_like(src)
    for _ in range(3):
        dst.copy_(src)
    t_copy = time_per_launch(lambda: dst.copy_(src), 10, torch)
    copy_GBps = 2 * src.numel() / t_copy / 1e9
    del src, dst

    peaks = measured_peaks(torch)

    wl = synth.WORKLOADS["C2_128K"]
    dec = run_workload(isa, wl, args.steps, args.warmup, args.instances, torch,
                       baseline_seq=None if args.no_cpu_baseline else wl.B, graph=True)
    alg = dec["alg"]
    t = dec["t_step"]
    tokens = wl.tokens_per_group
    st = dec["stages_us"]
    # per stage: launches per group, algorithmic bytes per launch, kernels
    stages = {
        "indexer": (1, alg["ix_bytes"], "indexer_scores_kernel<64, 128>"),
        "topk": (1, alg["topk_read_bytes"],
                 "topk_summary_kernel + topk_direct_kernel<4> (stand-alone call; in the group "
                 "the indexer's epilogue writes the summary)"),
        "attend": (wl.n_layers, alg["at_bytes_per_layer"],
                   "sparse_attend_kernel<1, 1, 576, 512, 2, false> + merge_splits_kernel (one layer)"),
    }
    stage_us = {"indexer": st["indexer"], "topk": st["topk"], "attend": st["attend_per_layer"]}
    rooflines = {}
    for name, (per_group, nbytes, kernels) in stages.items():
        t_launch = stage_us[name] * 1e-6
        rooflines[name] = {"kernel": kernels, "bound": "hbm", "launches_per_group": per_group,
                           "launch_us": stage_us[name], "algorithmic_bytes": nbytes,
                           "achieved": nbytes / t_launch / 1e9, "peak": PEAK_HBM / 1e9,
                           "unit": "GB/s", "frac": nbytes / t_launch / PEAK_HBM,
                           "traffic": measured_traffic(name),
                           "share_of_step": per_group * t_launch / t}
    dominant = max(rooflines, key=lambda n: rooflines[n]["share_of_step"])
    cpu_name, ncpu, ram_gib = host_info()
    line = {
        "metric": METRIC,
        "value": tokens / t,
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": t * 1e3,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "int8+bf16",
        "data": "synthetic",
        "config": {"workload": "C2_128K decode group: B=8 x 1 query, context 131072, indexer "
                               "64x128 int8, top-2048, 4 layers x 64 heads x 576 bf16 latent",
                   "input_instances": args.instances},
        "roofline": dict(rooflines[dominant], stage=dominant),
        "stage_rooflines": rooflines,
        "group_roofline": {"t_ideal_us": alg["t_ideal_s"] * 1e6, "t_measured_us": t * 1e6,
                           "frac": alg["t_ideal_s"] / t,
                           "algorithmic_bytes": alg["group_bytes"],
                           "achieved_GBps": alg["group_bytes"] / t / 1e9},
        "stages_us": dec["stages_us"],
        "group_index_us": {"value": dec["group_index_us"],
                           "note": "indexer + top-k inside the group: the group's time minus "
                                   "the same groups reusing their index sets, so it also holds "
                                   "what the attention layers lose by following the indexer's "
                                   "134 MB stream (the stand-alone top-k stage runs its own "
                                   "summary kernel; in the group the indexer writes it)"},
        "index_histogram_us": dec["index_histogram_us"],
        "hip_graph": {"us_per_group": dec["t_graph"] * 1e6,
                      "replay_equals_eager": dec["graph_equal"],
                      "note": "the same groups captured once and replayed; value uses eager "
                              "launches"},
        "copy_GBps_measured": copy_GBps,
        "measured_peaks": peaks,
    }
    if "oracle" in dec:
        o = dec["oracle"]
        line["cpu_baseline"] = {"value": o["tokens"] / o["seconds"], "unit": "tokens/s",
                                "cores": 1, "kind": "oracle",
                                "sample": f"one whole C2_128K group ({o['tokens']} tokens) on one "
                                          f"host core (core {o['core']}, pinned) of {cpu_name} "
                                          f"({ncpu} cpus)",
                                "seconds": o["seconds"], "idx_exact": o["idx_exact"],
                                "max_abs_err_vs_gpu": o["max_abs_err"],
                                "host": {"cpu": cpu_name, "nproc": ncpu, "ram_GiB": ram_gib}}
    if not args.no_extra:
        line["ablation"] = run_ablation(isa, torch, steps=10, warmup=3)
        line["mtp"] = run_mtp(isa, torch, reps=5)
        line["fp8_kv"] = run_fp8_kv(isa, torch, steps=50, warmup=10, n_inst=args.instances)
        line["paged"] = run_paged(isa, torch, steps=50, warmup=10, n_inst=args.instances)
        w32 = synth.WORKLOADS["C2"]
        d32 = run_workload(isa, w32, 50, 10, args.instances, torch)
        line["decode_32k"] = {
            "workload": "C2 decode group: 8 sequences x 1 query over 32768 cached tokens, 4 layers",
            "tokens_per_s": w32.tokens_per_group / d32["t_step"], "ms_per_step": d32["t_step"] * 1e3,
            "stages_us": d32["stages_us"], "t_ideal_us": d32["alg"]["t_ideal_s"] * 1e6,
            "frac_of_roofline": d32["alg"]["t_ideal_s"] / d32["t_step"]}
        wm = synth.WORKLOADS["C2_128K_MQ8"]
        mq = run_workload(isa, wm, 30, 5, 2, torch)
        am = mq["alg"]
        line["multi_query"] = {
            "workload": "C2_128K_MQ8 decode group: 8 sequences x 8 queries (causal among them) "
                        "over 131072 cached tokens, one index set per query, 4 layers",
            "tokens_per_s": wm.tokens_per_group / mq["t_step"], "ms_per_step": mq["t_step"] * 1e3,
            "stages_us": mq["stages_us"],
            "t_ideal_us": am["t_ideal_s"] * 1e6, "frac_of_roofline": am["t_ideal_s"] / mq["t_step"],
            "indexer_int8_TOPS": am["ix_ops"] / (mq["stages_us"]["indexer"] * 1e-6) / 1e12}
    if not args.no_prefill:
        line["prefill"] = run_prefill(isa, torch, args, cpu_name, ncpu)
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
