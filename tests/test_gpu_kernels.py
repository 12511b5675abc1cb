"""GPU parity of each C-ABI entry point against the CPU oracle, at sizes the
oracle finishes in seconds that still span several tiles and ragged tails,
plus the degenerate cases of the method (empty and short contexts, ties,
invalid slots)."""
import math
import zlib

import numpy as np
import pytest
import torch

import long_context_sparse_indexshare_amd as isa
import oracle
import synth
from _parity import (assert_attn_close, assert_idx_equal, assert_lse_close, assert_scores_bitwise,
                     dev, guarded, host)

pytestmark = pytest.mark.gpu


def _print_case(*a):
    print("CASE", *a, flush=True)


# ------------------------------------------------------------------ indexer ----

INDEXER_CASES = [
    # (name, B, Tq, kv_len list, L_cap, H_I, D_I)
    ("C1-full", 1, 1024, [1024], 1024, 4, 32),
    ("decode-ragged", 3, 1, [5000, 1, 3333], 5000, 64, 128),
    ("decode-Tq3", 2, 3, [2049, 700], 2100, 64, 128),
    ("prefill-64h", 1, 70, [1500], 1531, 64, 128),
    ("h8-d64", 2, 9, [400, 37], 410, 8, 64),
    ("h16-d128", 1, 5, [3], 64, 16, 128),
    ("h32-d32", 2, 4, [129, 0], 130, 32, 32),
    ("short-ctx", 2, 6, [2, 9], 33, 64, 128),
    # >= 64 queries per sequence take the prefill kernel (two queries per wave)
    ("prefill-kv<Tq", 2, 65, [40, 1000], 1100, 64, 128),
    ("prefill-d64", 1, 101, [3000], 3000, 64, 64),
    ("prefill-d32", 2, 64, [64, 333], 350, 64, 32),
    # multi-query decode: few queries, the keys split across workgroups
    ("mq-Tq8-split", 2, 8, [20000, 9000], 20100, 64, 128),
    ("mq-Tq5-split", 3, 5, [4097, 1, 70000], 70000, 64, 128),
]


@pytest.mark.parametrize("case", INDEXER_CASES, ids=[c[0] for c in INDEXER_CASES])
def test_indexer_scores_bitwise(case):
    name, B, Tq, lens, L_cap, H_I, D_I = case
    _print_case("indexer", case)
    g = torch.Generator().manual_seed(zlib.crc32(name.encode()) & 0xFFFF)
    qI = synth.int8_uniform((B, Tq, H_I, D_I), g, "cpu")
    w = synth.pow2_weights((B, Tq, H_I), g, "cpu")
    kI = synth.int8_uniform((B, L_cap, D_I), g, "cpu")
    kv_len = torch.tensor(lens, dtype=torch.int32)
    ref = oracle.indexer_scores(qI, w, kI, kv_len)
    S, guard = guarded((B, Tq, L_cap), torch.float32)
    isa.isa_indexer_scores(dev(qI), dev(w), dev(kI), dev(kv_len), S=S)
    guard.check(name)
    assert_scores_bitwise(S, ref, name)


def test_indexer_full_int8_range_is_exact():
    # |q.k| <= 128*128*128 stays exact in int32; weights 1 keep the fp32 head sum exact
    B, Tq, L_cap, H_I, D_I = 1, 2, 2000, 64, 128
    g = torch.Generator().manual_seed(9)
    qI = torch.randint(-128, 128, (B, Tq, H_I, D_I), generator=g, dtype=torch.int8)
    kI = torch.randint(-128, 128, (B, L_cap, D_I), generator=g, dtype=torch.int8)
    w = torch.ones(B, Tq, H_I) * 0.5
    kv_len = torch.tensor([L_cap], dtype=torch.int32)
    ref = oracle.indexer_scores(qI, w, kI, kv_len)
    S = isa.isa_indexer_scores(dev(qI), dev(w), dev(kI), dev(kv_len))
    assert_scores_bitwise(S, ref, "full-range")


@pytest.mark.parametrize("Tq", [2, 70], ids=["decode", "prefill"])
def test_indexer_full_int8_range_prefill_fallback_is_exact(Tq):
    # bytes beyond [-64, 63] with weight 1/2 cannot be folded into the int8
    # operand, so the prefill kernel takes its fp32 epilogue: still exact here
    B, L_cap, H_I, D_I = 1, 1500, 64, 128
    g = torch.Generator().manual_seed(19 + Tq)
    qI = torch.randint(-128, 128, (B, Tq, H_I, D_I), generator=g, dtype=torch.int8)
    kI = torch.randint(-128, 128, (B, L_cap, D_I), generator=g, dtype=torch.int8)
    w = torch.ones(B, Tq, H_I) * 0.5
    kv_len = torch.tensor([L_cap], dtype=torch.int32)
    _print_case("indexer full range", Tq)
    ref = oracle.indexer_scores(qI, w, kI, kv_len)
    S = isa.isa_indexer_scores(dev(qI), dev(w), dev(kI), dev(kv_len))
    assert_scores_bitwise(S, ref, f"full-range Tq={Tq}")


@pytest.mark.parametrize("Tq", [3, 96], ids=["decode", "prefill"])
def test_indexer_general_weights_within_fp32_bound(Tq):
    # Weights that are not powers of two (and of either sign) make the head sum
    # inexact in fp32.  Every product w*ReLU(dot) is rounded once and the H_I
    # terms are added in fp32, so against the exactly rounded oracle score the
    # error is at most (H_I + 2) * 2^-24 * sum_h |w_h| ReLU(dot_h), which is the
    # oracle's score for the weights |w|.
    B, L_cap, H_I, D_I = 2, 3000, 64, 128
    g = torch.Generator().manual_seed(31 + Tq)
    qI = synth.int8_uniform((B, Tq, H_I, D_I), g, "cpu")
    kI = synth.int8_uniform((B, L_cap, D_I), g, "cpu")
    w = torch.rand(B, Tq, H_I, generator=g) * 2.0 - 0.7
    kv_len = torch.tensor([L_cap, 1777], dtype=torch.int32)
    _print_case("indexer general weights", Tq)
    ref = oracle.indexer_scores(qI, w, kI, kv_len).astype(np.float64)
    mag = oracle.indexer_scores(qI, w.abs(), kI, kv_len).astype(np.float64)
    S = host(isa.isa_indexer_scores(dev(qI), dev(w), dev(kI), dev(kv_len))).numpy().astype(np.float64)
    vis = np.isfinite(ref)
    assert np.array_equal(vis, np.isfinite(S))
    bound = (H_I + 2) * 2.0 ** -24 * mag[vis] + 1e-30
    err = np.abs(S[vis] - ref[vis])
    assert np.all(err <= bound), f"max err/bound {float((err / bound).max()):.3g}"


# -------------------------------------------------------------------- top-k ----

def _topk_check(S, kv_len, k, name):
    _print_case("topk", name, tuple(S.shape), k)
    ref = oracle.topk_select(S, kv_len, k)
    idx, guard = guarded(tuple(S.shape[:2]) + (k,), torch.int32)
    isa.isa_topk_select(dev(torch.from_numpy(np.ascontiguousarray(S))), dev(kv_len), k, idx=idx)
    guard.check(name)
    assert_idx_equal(idx, ref, name)


@pytest.mark.parametrize("n,k", [(10000, 2048), (4097, 2048), (2048, 2048), (2047, 2048),
                                 (20000, 64), (70000, 1), (9000, 2047)])
def test_topk_random_scores(n, k):
    r = np.random.default_rng(n + k)
    B, Tq = 2, 3
    L_cap = n + 5
    S = (r.integers(0, 5000, size=(B, Tq, L_cap)) * 0.25).astype(np.float32)  # many ties
    kv_len = torch.tensor([n, max(n // 2, 1)], dtype=torch.int32)
    _topk_check(S, kv_len, k, f"random n={n} k={k}")


def test_topk_crafted_ties():
    L_cap, k = 9000, 2048
    kv_len = torch.tensor([L_cap] * 6, dtype=torch.int32)
    S = np.zeros((6, 1, L_cap), dtype=np.float32)
    S[1] = 3.5                                  # all equal
    S[2, 0, ::2] = -0.0                         # -0.0 and +0.0 tie
    S[3, 0, :] = np.arange(L_cap) % 7           # duplicates straddle the cut
    S[4, 0, :] = -np.inf                        # every score -inf
    S[4, 0, 5000:5003] = 1.0
    S[5, 0, :] = np.linspace(-1e30, 1e30, L_cap).astype(np.float32)[::-1]
    _topk_check(S, kv_len, k, "crafted")


def test_topk_crafted_ties_long_rows():
    # rows longer than 131072 positions take the histogram / classify path
    L_cap, k = 140000, 2048
    kv_len = torch.tensor([L_cap] * 5, dtype=torch.int32)
    S = np.random.default_rng(21).standard_normal((5, 1, L_cap)).astype(np.float32)
    S[1] = 3.5                                  # all equal
    S[2, 0, ::2] = -0.0                         # -0.0 and +0.0 tie
    S[3, 0, :] = np.arange(L_cap) % 7           # duplicates straddle the cut
    S[4, 0, :] = -np.inf
    S[4, 0, 70000:70003] = 1.0
    _topk_check(S, kv_len, k, "crafted long")


def test_topk_short_and_empty_runs_across_chunks():
    # Rows of 2^21 positions (512 chunks of 4096) whose candidates are a few
    # spikes per chunk, so most runs are shorter than the 8 consecutive
    # entries a finishing thread compacts (its range crosses two or more run
    # boundaries), or are packed into three chunks with every other run empty.
    L_cap, k = 1 << 21, 2048
    r = np.random.default_rng(23)
    S = (r.standard_normal((3, 1, L_cap)) * 0.01).astype(np.float32)
    spread = np.linspace(0, L_cap - 1, 2100).astype(np.int64)            # ~4 per chunk
    S[0, 0, spread] = 100.0 + r.integers(0, 40, size=spread.size) * 0.25  # ties at the cut
    packed = np.concatenate([c * 4096 + r.choice(4096, 800, replace=False) for c in (5, 200, 511)])
    S[1, 0, packed] = 50.0 + r.integers(0, 64, size=packed.size) * 0.5
    varied = np.concatenate([c * 4096 + r.choice(4096, int(n), replace=False)
                             for c, n in enumerate(r.integers(2, 8, size=512))])
    S[2, 0, varied] = 7.0 + r.integers(0, 16, size=varied.size) * 0.125
    kv_len = torch.tensor([L_cap] * 3, dtype=torch.int32)
    _topk_check(S, kv_len, k, "short runs")


def test_topk_all_in_one_bin_overflows_candidates():
    # every key in the first-digit bin: the candidate list overflows and the
    # last workgroup re-reads the row
    L_cap = 300000
    r = np.random.default_rng(3)
    S = (1000.0 + r.integers(0, 3, size=(1, 2, L_cap)) * 0.25).astype(np.float32)
    kv_len = torch.tensor([L_cap], dtype=torch.int32)
    _topk_check(S, kv_len, 2048, "overflow")


def test_topk_short_and_empty_rows():
    L_cap, k = 3000, 64
    S = np.random.default_rng(4).standard_normal((3, 4, L_cap)).astype(np.float32)
    kv_len = torch.tensor([2, 0, 70], dtype=torch.int32)   # pos < 0 rows see nothing
    _topk_check(S, kv_len, k, "short")


def test_topk_reuses_workspace_across_calls():
    ws = isa.Workspace()
    r = np.random.default_rng(5)
    for it in range(3):
        S = r.standard_normal((4, 1, 50000)).astype(np.float32)
        kv_len = torch.tensor([50000, 30000, 49999, 4097], dtype=torch.int32)
        ref = oracle.topk_select(S, kv_len, 2048)
        idx = isa.isa_topk_select(dev(torch.from_numpy(S)), dev(kv_len), 2048, ws=ws)
        assert_idx_equal(idx, ref, f"call {it}")


# Decode rows of 32768 positions (the C2 shape): their summary would hold
# fewer than 2k keys, so they take the filter / finish pair.

def test_topk_32k_rows():
    r = np.random.default_rng(77)
    L = 32768
    S = r.standard_normal((8, 1, L)).astype(np.float32)
    S[3, 0, 100:3000] += 6.0                         # a clustered block of high scores
    S[5] = (r.integers(0, 300, size=L) * 0.5).astype(np.float32)   # heavy ties at the cut
    kv_len = torch.tensor([L, L - 1, 20000, L, 2049, L, 31, L], dtype=torch.int32)
    _topk_check(S, kv_len, 2048, "32K rows")
    # several causal queries per sequence, the last seeing all 32768 positions
    S2 = (r.integers(0, 4000, size=(2, 6, L)) * 0.25).astype(np.float32)
    _topk_check(S2, torch.tensor([L, 9000], dtype=torch.int32), 2048, "32K causal rows")


# Few rows of 64K-256K positions take the direct path: one workgroup per row
# selects from the summary (the M largest keys of every 256-position wave
# chunk, with their positions) and reads again only the chunks whose summary
# may miss a candidate ("saturated"), staging their candidates in LDS or, past
# 8192 of them, reading them in every pass.

def _direct_case(name):
    r = np.random.default_rng(sum(map(ord, name)))
    L = 131072
    if name == "normal":
        S = r.standard_normal((2, 1, L)).astype(np.float32)
        return S, [L, L - 777]
    if name == "ties":
        S = (r.integers(0, 5000, size=(2, 1, L)) * 0.25).astype(np.float32)
        return S, [L, 100000]
    if name == "clustered":
        # high scores packed into runs: a few saturated chunks (staged), then
        # more candidates than the stage holds (read in every pass)
        S = r.standard_normal((3, 1, L)).astype(np.float32)
        S[0, 0, 5000:8000] += 10.0
        S[1, 0, 1000:9000] += 10.0
        S[2, 0, 20000:30000] += 10.0
        S[2, 0, 20000:30000:3] = 12.0                  # ties inside the run
        return S, [L, L, L - 5]
    if name == "short":
        # few visible positions: the summary holds fewer than k keys
        S = r.standard_normal((6, 1, L)).astype(np.float32)
        return S, [3000, 30000, 2049, 2048, 1, 0]
    if name == "crafted":
        S = r.standard_normal((6, 1, L)).astype(np.float32)
        S[1] = 3.5                                      # all equal
        S[2, 0, ::2] = -0.0                             # -0.0 and +0.0 tie
        S[3, 0, :] = np.arange(L) % 7                   # duplicates straddle the cut
        S[4, 0, :] = -np.inf
        S[4, 0, 5000:5003] = 1.0
        S[5, 0, :] = np.linspace(-1e30, 1e30, L).astype(np.float32)[::-1]
        return S, [L - 333] * 6
    if name == "256K":
        # 8 summary keys per chunk, 8 bitmap words per thread; the third row's
        # heavy ties saturate every chunk (more candidates than the stage holds)
        L = 262144
        S = r.standard_normal((3, 1, L)).astype(np.float32)
        S[1, 0, 100000:101500] += 8.0
        S[2, 0, :] = (np.arange(L) % 3).astype(np.float32)
        return S, [L, L - 1000, L - 77]
    if name == "64K":
        L = 65536
        S = (r.integers(0, 20000, size=(2, 1, L)) * 0.125).astype(np.float32)
        return S, [L, 40000]
    raise ValueError(name)


@pytest.mark.parametrize("name", ["normal", "ties", "clustered", "short", "crafted", "256K", "64K"])
def test_topk_direct_path(name):
    S, kv = _direct_case(name)
    _topk_check(S, torch.tensor(kv, dtype=torch.int32), 2048, f"direct {name}")


def test_topk_direct_path_multi_query_rows():
    # several queries per sequence (each row sees one position more) and a
    # smaller k
    r = np.random.default_rng(41)
    L = 131072
    S = (r.integers(0, 100000, size=(2, 4, L)) * 0.5).astype(np.float32)
    S[1, :, 7000:7400] = 1e6
    kv_len = torch.tensor([L - 3, 90001], dtype=torch.int32)
    _topk_check(S, kv_len, 1024, "direct multi-query")


# Many rows (a prefill chunk) take the one-workgroup-per-row path.

def test_topk_many_rows_causal_ragged():
    # rows see 1801..2100 positions: some padded (n <= k), the rest selected
    r = np.random.default_rng(11)
    B, Tq, L_cap = 2, 300, 2100
    S = (r.integers(0, 3000, size=(B, Tq, L_cap)) * 0.5).astype(np.float32)
    kv_len = torch.tensor([2100, 2090], dtype=torch.int32)
    _topk_check(S, kv_len, 2048, "many rows ragged")


def test_topk_many_rows_long_with_ties():
    r = np.random.default_rng(12)
    B, Tq, L_cap = 1, 260, 40000
    S = (r.integers(0, 20000, size=(B, Tq, L_cap)) * 0.125).astype(np.float32)
    S[0, 7] = 2.0                                # every score equal
    S[0, 8, ::3] = -0.0
    S[0, 9] = -np.inf
    S[0, 9, 12345:12350] = 4.0
    kv_len = torch.tensor([L_cap - 3], dtype=torch.int32)
    _topk_check(S, kv_len, 2048, "many rows long")


def test_topk_many_rows_entry_overflow():
    # the threshold bin holds every score: the LDS entry list overflows and
    # the row is read again
    r = np.random.default_rng(13)
    S = (1000.0 + r.integers(0, 3, size=(1, 256, 20000)) * 0.25).astype(np.float32)
    kv_len = torch.tensor([20000], dtype=torch.int32)
    _topk_check(S, kv_len, 2048, "many rows overflow")


@pytest.mark.parametrize("L_cap", [262144, 262145])
def test_topk_many_rows_size_limit(L_cap):
    # the largest row the one-workgroup path takes, and one past it
    r = np.random.default_rng(L_cap)
    S = r.standard_normal((1, 256, L_cap), dtype=np.float32)
    kv_len = torch.tensor([L_cap], dtype=torch.int32)
    _topk_check(S, kv_len, 2048, f"many rows L_cap={L_cap}")


# ---------------------------------------------------------------- attention ----

def _attend_case(B, Tq, H, D, D_v, L_cap, k, idx_np, seed, name, want_lse=True):
    _print_case("attend", name, B, Tq, H, D, D_v, L_cap, k)
    g = torch.Generator().manual_seed(seed)
    Q = synth.normal_bf16((B, Tq, H, D), g, "cpu")
    C = synth.normal_bf16((B, L_cap, D), g, "cpu")
    scale = 1.0 / math.sqrt(D)
    idx = torch.from_numpy(idx_np.astype(np.int32))
    ref_out, ref_lse = oracle.sparse_mla_attend(Q, C, idx, D_v, scale)
    out, gout = guarded((B, Tq, H, D_v), torch.bfloat16)
    lse, glse = guarded((B, Tq, H), torch.float32) if want_lse else (None, None)
    isa.isa_sparse_mla_attend(dev(Q), dev(C), dev(idx), D_v, scale, out=out, lse=lse)
    gout.check(name + " out")
    if want_lse:
        glse.check(name + " lse")
    assert_attn_close(out, ref_out, name)
    if want_lse:
        assert_lse_close(lse, ref_lse, name)
    return Q, C, idx, out


def _random_sets(B, Tq, L_cap, k, fill, r):
    idx = np.full((B, Tq, k), -1, dtype=np.int64)
    for b in range(B):
        for t in range(Tq):
            m = min(fill, L_cap, k)
            idx[b, t, :m] = np.sort(r.choice(L_cap, size=m, replace=False))
    return idx


@pytest.mark.parametrize("B,Tq,fill", [(8, 1, 2048), (2, 3, 1000), (1, 40, 2048), (3, 2, 77)])
def test_attend_576(B, Tq, fill):
    r = np.random.default_rng(B * 100 + Tq)
    L_cap, k = 20000, 2048
    idx = _random_sets(B, Tq, L_cap, k, fill, r)
    _attend_case(B, Tq, 64, 576, 512, L_cap, k, idx, seed=B + Tq, name=f"576 B{B} Tq{Tq} fill{fill}")


def test_attend_576_many_queries():
    # >= 256 queries: one workgroup per query holds all 64 heads and columns
    r = np.random.default_rng(12)
    idx = _random_sets(2, 130, 9000, 128, 128, r)
    idx[1, 5, 40:] = -1
    _attend_case(2, 130, 64, 576, 512, 9000, 128, idx, seed=13, name="576 wide")


def test_attend_576_many_queries_ragged_k():
    # the per-query kernel over a k that is not a whole number of tiles, with
    # sets of every fill, an empty set and invalid slots mid-tile
    r = np.random.default_rng(16)
    B, Tq, L_cap, k = 1, 260, 12000, 700
    idx = np.full((B, Tq, k), -1, dtype=np.int64)
    for t in range(Tq):
        m = int(r.integers(0, k + 1)) if t % 3 else k
        idx[0, t, :m] = np.sort(r.choice(L_cap, size=m, replace=False))
    idx[0, 7, :] = -1
    idx[0, 9, 33] = -5
    idx[0, 9, 34] = L_cap
    _attend_case(B, Tq, 64, 576, 512, L_cap, k, idx, seed=17, name="576 wide ragged")


def test_attend_576_many_queries_late_large_score():
    # the per-query kernel fixes a head's softmax reference at its first tile;
    # a later row that scores far above it (P about 2^95 times the first
    # tile's largest, head 17 of query 5) makes the kernel run the query again
    # with per-tile references.  Query 6 (the same head-17 query) has that row
    # in its first tile.  The score comes from the row's RoPE columns (keys
    # only), so the value columns, and the outputs, keep their usual size.
    r = np.random.default_rng(21)
    B, Tq, L_cap, k = 1, 256, 3000, 384
    idx = _random_sets(B, Tq, L_cap, k, k, r)
    g = torch.Generator().manual_seed(22)
    Q = synth.normal_bf16((B, Tq, 64, 576), g, "cpu")
    C = synth.normal_bf16((B, L_cap, 576), g, "cpu")
    big = int(idx[0, 5, 300])                   # tile 9 of query 5
    C[0, big, 512:] = (32.0 * Q[0, 5, 17, 512:].float()).to(torch.bfloat16)
    Q[0, 6, 17] = Q[0, 5, 17]
    idx[0, 6, 1:] = np.sort(r.choice(np.setdiff1d(np.arange(L_cap), [big]), size=k - 1,
                                     replace=False))
    idx[0, 6, 0] = big
    idx_t = torch.from_numpy(idx.astype(np.int32))
    scale = 1.0 / math.sqrt(576)
    ref_out, ref_lse = oracle.sparse_mla_attend(Q, C, idx_t, 512, scale)
    out, gout = guarded((B, Tq, 64, 512), torch.bfloat16)
    lse, glse = guarded((B, Tq, 64), torch.float32)
    isa.isa_sparse_mla_attend(dev(Q), dev(C), dev(idx_t), 512, scale, out=out, lse=lse)
    gout.check("late large out")
    glse.check("late large lse")
    assert_attn_close(out, ref_out, "late large")
    assert_lse_close(lse, ref_lse, "late large")
    # head 17 of queries 5 and 6 is that row's value part
    for t in (5, 6):
        np.testing.assert_allclose(host(out)[0, t, 17].float().numpy(),
                                   C[0, big, :512].float().numpy(), rtol=0, atol=1e-2)


def test_attend_576_decode_late_large_score():
    # the decode kernel moves a head's reference only when a row exceeds it by
    # more than its slack; a row far above it in a group's second tile (slot
    # 100 of the first split: tile 3, the second tile of group 1) makes the
    # workgroup run its split again with exact references, and the merge then
    # weights that split alone.  Sequence 1 has such a row in its first tile.
    # The other heads of both queries get no RoPE part, so that row scores
    # like any other for them (a row that dominates a head gives outputs of
    # up to about 4, where the bf16 roundings of the split partial and of the
    # output alone exceed the tolerance's absolute bound).
    r = np.random.default_rng(23)
    B, Tq, L_cap, k = 2, 1, 5000, 2048
    idx = _random_sets(B, Tq, L_cap, k, k, r)
    g = torch.Generator().manual_seed(24)
    Q = synth.normal_bf16((B, Tq, 64, 576), g, "cpu")
    C = synth.normal_bf16((B, L_cap, 576), g, "cpu")
    bigs = (int(idx[0, 0, 100]), int(idx[1, 0, 0]))
    for b, big in enumerate(bigs):
        C[b, big, 512:] = (32.0 * Q[b, 0, 17, 512:].float()).to(torch.bfloat16)
        Q[b, 0, :17, 512:] = 0
        Q[b, 0, 18:, 512:] = 0
    idx_t = torch.from_numpy(idx.astype(np.int32))
    scale = 1.0 / math.sqrt(576)
    ref_out, ref_lse = oracle.sparse_mla_attend(Q, C, idx_t, 512, scale)
    out, gout = guarded((B, Tq, 64, 512), torch.bfloat16)
    lse, glse = guarded((B, Tq, 64), torch.float32)
    isa.isa_sparse_mla_attend(dev(Q), dev(C), dev(idx_t), 512, scale, out=out, lse=lse)
    gout.check("decode late large out")
    glse.check("decode late large lse")
    assert_attn_close(out, ref_out, "decode late large")
    assert_lse_close(lse, ref_lse, "decode late large")
    for b, big in enumerate(bigs):
        np.testing.assert_allclose(host(out)[b, 0, 17].float().numpy(),
                                   C[b, big, :512].float().numpy(), rtol=0, atol=1e-2)


def test_attend_576_unsplit_two_groups():
    # 160 queries: the 32-head, two-group variant with enough workgroups that
    # the k slots are not split (each group writes its half of the columns)
    r = np.random.default_rng(14)
    idx = _random_sets(2, 80, 5000, 256, 256, r)
    idx[0, 3, 100:] = -1
    _attend_case(2, 80, 64, 576, 512, 5000, 256, idx, seed=15, name="576 unsplit")


@pytest.mark.parametrize("B,Tq,k", [(2, 20, 2048), (1, 64, 700), (1, 33, 2048)])
def test_attend_576_split_sets_of_mixed_fill(B, Tq, k):
    # tens of queries, the k slots split over workgroups and merged: full
    # sets, short sets that leave later splits empty, empty sets, invalid
    # slots and a ragged k
    r = np.random.default_rng(B * 1000 + Tq)
    L_cap = 9000
    idx = np.full((B, Tq, k), -1, dtype=np.int64)
    for b in range(B):
        for t in range(Tq):
            m = [k, 77, 0, int(r.integers(1, k + 1))][(b * Tq + t) % 4]
            idx[b, t, :m] = np.sort(r.choice(L_cap, size=m, replace=False))
    idx[0, 1, 5] = -9
    idx[0, 1, 6] = L_cap + 1
    _attend_case(B, Tq, 64, 576, 512, L_cap, k, idx, seed=B + Tq + k,
                 name=f"576 split mixed fill B{B} Tq{Tq} k{k}")


def test_attend_160_16_heads():
    r = np.random.default_rng(7)
    idx = _random_sets(1, 50, 1024, 64, 64, r)
    idx[0, :5, 3:] = -1
    _attend_case(1, 50, 16, 160, 128, 1024, 64, idx, seed=3, name="160x16")


def test_attend_invalid_and_empty_slots():
    r = np.random.default_rng(8)
    B, Tq, L_cap, k = 2, 3, 5000, 2048
    idx = _random_sets(B, Tq, L_cap, k, 1500, r)
    idx[0, 0, :] = -1                 # empty set: zeros, lse = -inf
    idx[0, 1, 7] = L_cap + 3          # out of range: skipped
    idx[0, 1, 9] = -77
    idx[1, 2, 1:] = -1                # one valid slot: exactly that row
    r.shuffle(idx[1, 0])              # slot order does not matter
    _, C, idx_t, out = _attend_case(B, Tq, 64, 576, 512, L_cap, k, idx, seed=11, name="invalid")
    o = host(out)
    assert torch.all(o[0, 0] == 0)
    np.testing.assert_array_equal(o[1, 2].float().numpy(),
                                  C[1, int(idx[1, 2, 0]), :512].float().expand(64, 512).numpy())


def test_attend_fewer_heads_than_block():
    r = np.random.default_rng(9)
    idx = _random_sets(2, 1, 3000, 2048, 2048, r)
    _attend_case(2, 1, 40, 576, 512, 3000, 2048, idx, seed=5, name="H40")


def test_attend_small_k():
    r = np.random.default_rng(10)
    idx = _random_sets(4, 2, 3000, 100, 100, r)
    _attend_case(4, 2, 64, 576, 512, 3000, 100, idx, seed=6, name="k100")


# ------------------------------------------------------- FP8 latent cache ----

def _attend_fp8_case(B, Tq, H, D_c, D_r, L_cap, k, idx_np, seed, name):
    _print_case("attend fp8", name, B, Tq, H, D_c, D_r, L_cap, k)
    g = torch.Generator().manual_seed(seed)
    C8, Ce, Cr = synth.fp8_cache(B, L_cap, D_c, D_r, g, "cpu")
    Q = synth.normal_bf16((B, Tq, H, D_c + D_r), g, "cpu")
    scale = 1.0 / math.sqrt(D_c + D_r)
    idx = torch.from_numpy(idx_np.astype(np.int32))
    ref_out, ref_lse = oracle.sparse_mla_attend_fp8(Q, C8, Ce, Cr, idx, scale)
    out, gout = guarded((B, Tq, H, D_c), torch.bfloat16)
    lse, glse = guarded((B, Tq, H), torch.float32)
    isa.isa_sparse_mla_attend_fp8(dev(Q), dev(C8), dev(Ce), dev(Cr), dev(idx), scale, out=out,
                                  lse=lse)
    gout.check(name + " out")
    glse.check(name + " lse")
    assert_attn_close(out, ref_out, name)
    assert_lse_close(lse, ref_lse, name)
    return Q, (C8, Ce, Cr), idx, out, lse


@pytest.mark.parametrize("B,Tq,fill", [(8, 1, 2048), (2, 3, 1000), (3, 2, 77)])
def test_attend_fp8_decode(B, Tq, fill):
    # few queries: the 32-head two-group variant with the k slots split
    r = np.random.default_rng(40 + fill)
    idx = _random_sets(B, Tq, 5000, 2048, fill, r)
    _attend_fp8_case(B, Tq, 64, 512, 64, 5000, 2048, idx, seed=41, name=f"fp8 decode fill={fill}")


def test_attend_fp8_wide_and_unsplit():
    r = np.random.default_rng(42)
    idx = _random_sets(2, 130, 9000, 128, 128, r)          # >= 256 queries: 64-head variant
    _attend_fp8_case(2, 130, 64, 512, 64, 9000, 128, idx, seed=43, name="fp8 wide")
    idx = _random_sets(2, 80, 5000, 256, 256, r)           # 160 queries: two groups, no split
    _attend_fp8_case(2, 80, 64, 512, 64, 5000, 256, idx, seed=44, name="fp8 unsplit")


def test_attend_fp8_160_16_heads():
    r = np.random.default_rng(45)
    idx = _random_sets(1, 40, 1024, 64, 64, r)
    _attend_fp8_case(1, 40, 16, 128, 32, 1024, 64, idx, seed=46, name="fp8 160")


def test_attend_fp8_invalid_and_empty_slots():
    r = np.random.default_rng(47)
    B, Tq, L_cap, k = 2, 3, 5000, 2048
    idx = _random_sets(B, Tq, L_cap, k, 1500, r)
    idx[0, 0, :] = -1
    idx[0, 1, 7] = L_cap + 3
    idx[0, 1, 9] = -77
    idx[1, 2, 1:] = -1
    _, _, _, out, lse = _attend_fp8_case(B, Tq, 64, 512, 64, L_cap, k, idx, seed=48,
                                         name="fp8 invalid")
    assert torch.all(host(out)[0, 0] == 0) and torch.all(host(lse)[0, 0] == -math.inf)


def test_attend_fp8_equals_bf16_kernel_on_dequantized_cache():
    # power-of-two row scales make the dequantized rows bf16 numbers: the FP8
    # kernel's LDS tiles then hold the bf16 kernel's, and the outputs agree bit
    # for bit (decode and wide variants)
    for (B, Tq, L_cap, k, seed) in ((8, 1, 4000, 2048, 50), (2, 130, 3000, 96, 51)):
        r = np.random.default_rng(seed)
        idx = _random_sets(B, Tq, L_cap, k, k, r)
        Q, (C8, Ce, Cr), idx_t, out8, lse8 = _attend_fp8_case(B, Tq, 64, 512, 64, L_cap, k, idx,
                                                              seed=seed, name=f"fp8 vs bf16 {B}x{Tq}")
        lat = C8.view(torch.float8_e4m3fn).double() * torch.exp2(Ce.double() - 127)[..., None]
        C = torch.cat([lat, Cr.double()], dim=-1).to(torch.bfloat16)
        outb, lseb = isa.isa_sparse_mla_attend(dev(Q), dev(C), dev(idx_t), 512, 1.0 / 24,
                                               want_lse=True)
        torch.cuda.synchronize()
        assert torch.equal(host(out8), host(outb))
        assert torch.equal(host(lse8), host(lseb))


# ------------------------------------------------------ index access counts ----

@pytest.mark.parametrize("B,Tq,k,L_cap", [(2, 300, 2048, 9000), (3, 5, 17, 60), (1, 1, 2048, 2048)])
def test_index_histogram_bitwise(B, Tq, k, L_cap):
    _print_case("histogram", B, Tq, k, L_cap)
    r = np.random.default_rng(B * 1000 + k)
    idx = r.integers(-2, L_cap + 2, size=(B, Tq, k)).astype(np.int32)
    idx[0, 0, : min(k, 40)] = 7                    # a hot position
    start = r.integers(0, 5, size=(B, L_cap)).astype(np.uint32)
    ref = oracle.index_histogram(idx, L_cap, counts=start.copy())
    counts, guard = guarded((B, L_cap), torch.int32)
    counts.copy_(torch.from_numpy(start.view(np.int32).copy()))
    isa.isa_index_histogram(dev(torch.from_numpy(idx)), L_cap, counts=counts)
    guard.check("histogram")
    np.testing.assert_array_equal(host(counts).numpy().view(np.uint32), ref)


# ------------------------------------------------------------ paged caches ----

def _pages(cache, bs, seed, extra=5):
    g = torch.Generator().manual_seed(seed)
    B, L = cache.shape[0], cache.shape[1]
    table = synth.page_layout(B, L, bs, g, "cpu", extra_pages=extra)
    return synth.to_pages(cache, table, bs, B * (L // bs) + extra), table


@pytest.mark.parametrize("Tq,bs", [(1, 64), (8, 32), (70, 256)])
def test_indexer_paged_bitwise(Tq, bs):
    # decode kernel (Tq 1) and the key-split kernel (Tq 8, 70); one block unallocated
    _print_case("indexer paged", Tq, bs)
    B, L = 2, 4096
    g = torch.Generator().manual_seed(Tq * 100 + bs)
    qI = synth.int8_uniform((B, Tq, 64, 128), g, "cpu")
    w = synth.pow2_weights((B, Tq, 64), g, "cpu")
    kI = synth.int8_uniform((B, L, 128), g, "cpu")
    kv_len = torch.tensor([L, 3000], dtype=torch.int32)
    pool, table = _pages(kI, bs, Tq + bs)
    table[1, 2] = -1
    ref = oracle.indexer_scores_paged(qI, w, pool, table, kv_len)
    S = isa.isa_indexer_scores_paged(dev(qI), dev(w), dev(pool), dev(table), dev(kv_len))
    torch.cuda.synchronize()
    assert_scores_bitwise(S, ref, f"paged Tq={Tq} bs={bs}")
    # the contiguous kernel on the logical cache gives the same bits where allocated
    Sc = isa.isa_indexer_scores(dev(qI), dev(w), dev(kI), dev(kv_len))
    torch.cuda.synchronize()
    live = torch.ones(L, dtype=torch.bool)
    live[2 * bs:3 * bs] = False
    assert torch.equal(host(S)[0], host(Sc)[0])
    assert torch.equal(host(S)[1][:, live], host(Sc)[1][:, live])


@pytest.mark.parametrize("B,Tq,bs", [(8, 1, 64), (2, 130, 128)])
def test_attend_paged(B, Tq, bs):
    _print_case("attend paged", B, Tq, bs)
    r = np.random.default_rng(B + Tq + bs)
    L, k = 4096, (2048 if Tq == 1 else 128)
    g = torch.Generator().manual_seed(60 + B)
    Q = synth.normal_bf16((B, Tq, 64, 576), g, "cpu")
    C = synth.normal_bf16((B, L, 576), g, "cpu")
    idx = torch.from_numpy(_random_sets(B, Tq, L, k, k, r).astype(np.int32))
    pool, table = _pages(C, bs, B * 7 + bs)
    table[0, 3] = -1                                  # its slots are skipped
    ref_out, ref_lse = oracle.sparse_mla_attend_paged(Q, pool, table, idx, 512, 1.0 / 24)
    out, lse = isa.isa_sparse_mla_attend_paged(dev(Q), dev(pool), dev(table), dev(idx), 512,
                                               1.0 / 24, want_lse=True)
    torch.cuda.synchronize()
    assert_attn_close(out, ref_out, "paged")
    assert_lse_close(lse, ref_lse, "paged")
    # with every block allocated, the paged and contiguous kernels agree bit for bit
    pool, table = _pages(C, bs, B * 11 + bs)
    out_p, _ = isa.isa_sparse_mla_attend_paged(dev(Q), dev(pool), dev(table), dev(idx), 512,
                                               1.0 / 24)
    out_c, _ = isa.isa_sparse_mla_attend(dev(Q), dev(C), dev(idx), 512, 1.0 / 24)
    torch.cuda.synchronize()
    assert torch.equal(host(out_p), host(out_c))
