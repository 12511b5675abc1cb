"""Host-side logic of bench.py (no GPU): the one-GPU guard, the algorithmic
byte and op counts its roofline fractions divide by, and the rule that a
counter summary only counts for the kernel source it was taken on."""
import os
import subprocess
import sys

import bench
import synth

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, cwd=ROOT)
    assert r.returncode == 2
    assert "one GPU" in r.stderr
    assert r.stdout == ""


def test_algorithmic_counts_decode_128k():
    wl = synth.WORKLOADS["C2_128K"]
    a = bench.algorithmic(wl)
    # indexer: every cached int8 key row once, plus each query's qI and w
    assert a["ix_bytes"] == 8 * 131072 * 128 + 8 * 64 * (128 + 4)
    assert a["ix_ops"] == 2 * 64 * 128 * 8 * 131072
    # top-k: the scores once and the index sets
    assert a["topk_read_bytes"] == 8 * 131072 * 4 + 8 * 2048 * 4
    # attention per layer: the selected latent rows, Q and the output
    assert a["at_bytes_per_layer"] == 8 * 2048 * 576 * 2 + 8 * 64 * (576 + 512) * 2
    assert a["at_flops_per_layer"] == 8 * 2048 * 64 * 2 * (576 + 512)
    assert a["ix_bound"] == "hbm" and a["at_bound"] == "hbm"


def test_algorithmic_counts_causal_prefill():
    wl = synth.WORKLOADS["C3"]
    a = bench.algorithmic(wl)
    n0 = wl.kv_len - wl.Tq + 1                     # keys the first query sees
    pairs = sum(n0 + t for t in range(wl.Tq))
    assert a["ix_ops"] == 2 * 64 * 128 * pairs
    assert a["ix_bound"] == "mfma"
    # every prefill query sees more than k keys: 2048 rows each
    assert a["at_bytes_per_layer"] == 4096 * 2048 * 1152 + 4096 * 64 * 1088 * 2
    # counting each cache row once: at most the 135168-row cache
    assert a["at_bytes_once_per_layer"] == 135168 * 1152 + 4096 * 64 * 1088 * 2
    # then the layer is bound by its bf16 MFMA work and the group's ideal time
    # is the indexer's int8 ops plus four such layers (plus the index sets)
    t_at = a["at_flops_per_layer"] / bench.PEAK_BF16
    assert abs(a["t_ideal_once_s"] - (a["t_ix_s"] + a["topk_bytes"] / bench.PEAK_HBM + 4 * t_at)) < 1e-12


def test_mtp_seven_step_roofline():
    wl = synth.WORKLOADS["C5"]
    nbytes, t_ideal = bench.mtp_roofline(wl)
    ix = 16 * 262144 * 128 + 16 * 64 * (128 + 4)       # keys once, qI and w of step 1
    at = 16 * 2048 * 576 * 2 + 16 * 64 * (576 + 512) * 2  # one layer of one step
    assert nbytes == ix + 16 * 2048 * 4 + 7 * 4 * at
    # every stage of C5 is bound by HBM bytes at 8 TB/s
    assert abs(t_ideal - nbytes / bench.PEAK_HBM) < 1e-12
    assert abs(t_ideal * 1e6 - 207.06) < 0.01


def test_traffic_is_null_for_another_kernel_source(tmp_path, monkeypatch):
    # a tree of its own: ROOT/profiles/<summary>, ROOT/<package>/csrc/{attend.hip,
    # the shared header}
    src = os.path.join(ROOT, "long_context_sparse_indexshare_amd", "csrc", "attend.hip")
    hdr = os.path.join(ROOT, "long_context_sparse_indexshare_amd", "csrc", bench.SHARED_HEADER)
    csrc = tmp_path / "long_context_sparse_indexshare_amd" / "csrc"
    csrc.mkdir(parents=True)
    (csrc / "attend.hip").write_bytes(open(src, "rb").read())
    (csrc / bench.SHARED_HEADER).write_bytes(open(hdr, "rb").read())
    prof = tmp_path / "profiles"
    prof.mkdir()
    (prof / "good.txt").write_text("# comment: with a colon\ntraffic_bytes_per_launch: 1234\n"
                                   f"source_sha256: {bench.source_digest(src)}\n")
    (prof / "stale.txt").write_text("traffic_bytes_per_launch: 1234\nsource_sha256: " + "0" * 64 + "\n")
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    monkeypatch.setattr(bench, "TRAFFIC", {"attend": ("good.txt", "attend.hip")})
    assert bench.measured_traffic("attend") == 1234.0
    monkeypatch.setattr(bench, "TRAFFIC", {"attend": ("stale.txt", "attend.hip")})
    assert bench.measured_traffic("attend") is None
    assert bench.measured_traffic("topk") is None          # no summary for this stage
    # a change to the shared header also makes the summary stale
    monkeypatch.setattr(bench, "TRAFFIC", {"attend": ("good.txt", "attend.hip")})
    (csrc / bench.SHARED_HEADER).write_bytes(open(hdr, "rb").read() + b"\n")
    assert bench.measured_traffic("attend") is None
