"""Pins of the CPU oracle against facts that do not come from the oracle itself.

Each test ties one oracle function to something independent: exact rational
brute force, exhaustive subset enumeration, a library routine the definition
reduces to (torch scaled_dot_product_attention, logsumexp), closed forms, or
an invariant of the method.  The score, selection and attention definitions
follow "GLM-5.2 Explained: 1M Token Context AI Agent Model", section 2.1
(lightning-indexer relevance score, top-K positions, attention over the
selected positions only), with the readings stated in oracle.c.
"""
import itertools
import math
import random
from fractions import Fraction

import numpy as np
import pytest
import torch

import oracle
import synth


def _rng(seed):
    return np.random.default_rng(seed)


def _positions(kv_len, L_cap, Tq, b, t):
    ln = min(max(int(kv_len[b]), 0), L_cap)
    return ln - Tq + t


# ---------------------------------------------------------------- scores ----

def _exact_score(q, w, key):
    """sum_h w_h * ReLU(q_h . key) as an exact rational, rounded once to float32."""
    total = Fraction(0)
    for h in range(q.shape[0]):
        dot = sum(int(a) * int(b) for a, b in zip(q[h], key))
        total += Fraction(float(w[h])) * max(dot, 0)
    return np.float32(float(total))


@pytest.mark.parametrize("seed", range(40))
def test_scores_match_exact_rational_bruteforce(seed):
    r = _rng(seed)
    B, Tq, L_cap = int(r.integers(1, 3)), int(r.integers(1, 4)), int(r.integers(1, 9))
    H_I, D_I = int(r.integers(1, 5)), int(r.integers(1, 7))
    qI = r.integers(-128, 128, size=(B, Tq, H_I, D_I), dtype=np.int8)
    kI = r.integers(-128, 128, size=(B, L_cap, D_I), dtype=np.int8)
    # general fp32 weights of either sign, exponents kept close so every
    # double partial sum is exact and the only rounding is the final one
    mant = r.integers(-(1 << 23), 1 << 23, size=(B, Tq, H_I))
    expo = r.integers(-3, 3, size=(B, Tq, H_I))
    w = (mant * np.exp2(expo - 23.0)).astype(np.float32)
    kv_len = r.integers(-1, L_cap + 3, size=(B,), dtype=np.int32)
    S = oracle.indexer_scores(qI, w, kI, kv_len)
    for b in range(B):
        for t in range(Tq):
            pos = _positions(kv_len, L_cap, Tq, b, t)
            for s in range(L_cap):
                if s > pos:
                    assert S[b, t, s] == -np.inf
                else:
                    want = _exact_score(qI[b, t], w[b, t], kI[b, s])
                    assert S[b, t, s].tobytes() == want.tobytes(), (b, t, s)


@pytest.mark.parametrize("a,c", [(3, 2), (-3, 2), (7, -8), (-8, -8), (0, 5)])
def test_scores_closed_form_constant_inputs(a, c):
    # qI == a, kI == c  =>  S = D_I * max(a*c, 0) * sum_h w_h on visible keys
    B, Tq, L_cap, H_I, D_I = 2, 3, 11, 5, 16
    qI = np.full((B, Tq, H_I, D_I), a, dtype=np.int8)
    kI = np.full((B, L_cap, D_I), c, dtype=np.int8)
    w = np.array(synth.W_TABLE, dtype=np.float32)[_rng(7).integers(0, 4, size=(B, Tq, H_I))]
    kv_len = np.array([L_cap, 6], dtype=np.int32)
    S = oracle.indexer_scores(qI, w, kI, kv_len)
    for b in range(B):
        for t in range(Tq):
            pos = _positions(kv_len, L_cap, Tq, b, t)
            want = np.float32(D_I * max(a * c, 0) * float(np.sum(w[b, t].astype(np.float64))))
            for s in range(L_cap):
                assert S[b, t, s] == (want if s <= pos else -np.inf)


def _golden(name):
    import json
    import os
    with open(os.path.join(os.path.dirname(__file__), "golden", name)) as f:
        return json.load(f)


def test_scores_hand_worked_example():
    # tests/golden/indexer_hand_worked.json: a two-head example worked by hand
    # from the definition, with a tie at 0.0 between s2 and s3 for query 1.
    # The per-head dot products the fixture lists are first checked against
    # the inputs (plain integer arithmetic here), then the stated sums.
    g = _golden("indexer_hand_worked.json")
    qI = np.array(g["qI"], dtype=np.int8)
    w = np.array(g["w"], dtype=np.float32)
    kI = np.array(g["kI"], dtype=np.int8)
    kv_len = np.array(g["kv_len"], dtype=np.int32)
    for t, key in ((0, "t0"), (1, "t1")):
        for s, dots in enumerate(g["dots"][key]):
            assert dots == [int(np.dot(qI[0, t, h].astype(int), kI[0, s].astype(int)))
                            for h in range(2)]
    want = np.array([[[-np.inf if v == "-inf" else v for v in row] for row in b]
                     for b in g["S"]], dtype=np.float32)
    S = oracle.indexer_scores(qI, w, kI, kv_len)
    np.testing.assert_array_equal(S, want)
    for k, idx in g["topk"].items():
        np.testing.assert_array_equal(oracle.topk_select(S, kv_len, int(k)), idx)


def test_scores_zero_weights_closed_form():
    # w == 0 gives 0.0 (not -0.0) on every visible key whatever q and k are,
    # so the set is the first min(k, pos+1) positions (all scores tie)
    r = _rng(11)
    B, Tq, L_cap, H_I, D_I, k = 2, 5, 40, 6, 16, 7
    qI = r.integers(-128, 128, size=(B, Tq, H_I, D_I), dtype=np.int8)
    kI = r.integers(-128, 128, size=(B, L_cap, D_I), dtype=np.int8)
    w = np.zeros((B, Tq, H_I), dtype=np.float32)
    kv_len = np.array([L_cap, 3], dtype=np.int32)
    S = oracle.indexer_scores(qI, w, kI, kv_len)
    idx = oracle.topk_select(S, kv_len, k)
    for b in range(B):
        for t in range(Tq):
            pos = _positions(kv_len, L_cap, Tq, b, t)
            vis = S[b, t, : max(pos + 1, 0)]
            assert np.all(vis.view(np.uint32) == 0)
            assert np.all(S[b, t, max(pos + 1, 0):] == -np.inf)
            n = max(min(k, pos + 1), 0)
            assert idx[b, t].tolist() == list(range(n)) + [-1] * (k - n)


def test_power_of_two_weights_make_every_fp32_order_exact():
    # With int8 in [-8,7] (|q.k| <= 2^13 for D_I=128) and w in {1/4,..,2}, every
    # partial head sum is a multiple of 1/4 below 2^22, so any fp32 summation
    # order gives the same bits.  This is what lets a GPU kernel that sums heads
    # in its own order agree with the oracle bit for bit.
    wl = synth.WORKLOADS["C2"].scaled(B=1, L_cap=64, kv_len=64)
    inp = synth.indexer_inputs(wl)
    S = oracle.indexer_scores(inp["qI"], inp["w"], inp["kI"], inp["kv_len"])
    q = inp["qI"][0, 0].numpy().astype(np.int64)
    kk = inp["kI"][0].numpy().astype(np.int64)
    relu = np.maximum(kk @ q.T, 0).astype(np.float32)       # [L, H_I], exact
    wt = inp["w"][0, 0].numpy()
    perm = np.random.default_rng(1).permutation(wl.H_I)
    acc = np.zeros(64, dtype=np.float32)
    for h in perm:                                           # scrambled fp32 order
        acc = (acc + wt[h] * relu[:, h]).astype(np.float32)
    assert acc.tobytes() == S[0, 0].tobytes()
    assert np.all(np.abs(S[0, 0]) < 2.0 ** 22)


# ----------------------------------------------------------------- top-k ----

def _order_key(v, s):
    # total order of the selection: higher score first, then lower position;
    # -0.0 and +0.0 are the same score
    return (-float(v) + 0.0, s)


def _bruteforce_topk(row, n, k):
    m = min(k, n)
    winners = []
    for subset in itertools.combinations(range(n), m):
        rest = [u for u in range(n) if u not in subset]
        if all(_order_key(row[s], s) < _order_key(row[u], u) for s in subset for u in rest):
            winners.append(subset)
    assert len(winners) == 1          # exactly one subset dominates the others
    return list(winners[0]) + [-1] * (k - m)


@pytest.mark.parametrize("seed", range(60))
def test_topk_matches_subset_enumeration(seed):
    r = _rng(100 + seed)
    B, Tq, L_cap = int(r.integers(1, 3)), int(r.integers(1, 4)), int(r.integers(1, 10))
    k = int(r.integers(1, 12))
    palette = np.array([-np.inf, -2.5, -0.0, 0.0, 1.0, 1.0, 3.25, 7.0], dtype=np.float32)
    S = palette[r.integers(0, len(palette), size=(B, Tq, L_cap))]
    kv_len = r.integers(0, L_cap + 2, size=(B,), dtype=np.int32)
    idx = oracle.topk_select(S, kv_len, k)
    for b in range(B):
        for t in range(Tq):
            n = max(_positions(kv_len, L_cap, Tq, b, t) + 1, 0)
            assert idx[b, t].tolist() == _bruteforce_topk(S[b, t], n, k), (b, t)


def test_topk_special_cases():
    r = _rng(5)
    L_cap, Tq = 300, 4
    kv_len = np.array([L_cap], dtype=np.int32)
    S = r.standard_normal((1, Tq, L_cap)).astype(np.float32)
    # k >= visible count: the whole causal prefix, then -1
    idx = oracle.topk_select(S, kv_len, 400)
    for t in range(Tq):
        pos = L_cap - Tq + t
        assert idx[0, t, : pos + 1].tolist() == list(range(pos + 1))
        assert np.all(idx[0, t, pos + 1:] == -1)
    # all scores equal: the k lowest positions
    idx = oracle.topk_select(np.full_like(S, 2.0), kv_len, 17)
    assert np.all(idx[0] == np.arange(17))
    # distinct scores: the same set as a library top-k
    k = 37
    idx = oracle.topk_select(S, kv_len, k)
    for t in range(Tq):
        pos = L_cap - Tq + t
        lib = torch.topk(torch.from_numpy(S[0, t, : pos + 1].copy()), k).indices.numpy()
        assert idx[0, t].tolist() == sorted(lib.tolist())


# ------------------------------------------------------------- attention ----

def _bf16(shape, g):
    return torch.randn(shape, generator=g, dtype=torch.float32).to(torch.bfloat16)


def _sdpa_reference(Q, C, idx, D_v, scale):
    """torch SDPA in float64 with a boolean mask that keeps only the selected positions."""
    B, Tq, H, D = Q.shape
    L_cap = C.shape[1]
    out = torch.zeros(B, Tq, H, D_v, dtype=torch.float64)
    lse = torch.full((B, Tq, H), -math.inf, dtype=torch.float64)
    for b in range(B):
        for t in range(Tq):
            sel = [int(s) for s in idx[b, t] if 0 <= int(s) < L_cap]
            if not sel:
                continue
            mask = torch.zeros(1, L_cap, dtype=torch.bool)
            mask[0, sel] = True
            q = Q[b, t].double().unsqueeze(1)                    # [H, 1, D]
            kmat = C[b].double().unsqueeze(0).expand(H, L_cap, D)
            v = C[b, :, :D_v].double().unsqueeze(0).expand(H, L_cap, D_v)
            o = torch.nn.functional.scaled_dot_product_attention(q, kmat, v, attn_mask=mask,
                                                                 scale=scale)
            out[b, t] = o[:, 0]
            logits = (q[:, 0] @ C[b].double().T) * scale       # [H, L_cap]
            lse[b, t] = torch.logsumexp(logits[:, sel], dim=-1)
    return out, lse


@pytest.mark.parametrize("seed", range(12))
def test_attend_matches_masked_sdpa(seed):
    g = torch.Generator().manual_seed(seed)
    r = _rng(200 + seed)
    B, Tq, H = int(r.integers(1, 3)), int(r.integers(1, 3)), int(r.integers(1, 5))
    D_v = int(r.integers(1, 9))
    D = D_v + int(r.integers(0, 5))
    L_cap, k = int(r.integers(1, 40)), int(r.integers(1, 12))
    Q, C = _bf16((B, Tq, H, D), g), _bf16((B, L_cap, D), g)
    idx = np.full((B, Tq, k), -1, dtype=np.int32)
    for b in range(B):
        for t in range(Tq):
            m = int(r.integers(0, min(k, L_cap) + 1))
            idx[b, t, :m] = r.choice(L_cap, size=m, replace=False)
            r.shuffle(idx[b, t])
            if r.random() < 0.3:
                idx[b, t, r.integers(0, k)] = L_cap + 5       # out of range: skipped
    scale = float(np.float32(1.0 / math.sqrt(D)))
    out, lse = oracle.sparse_mla_attend(Q, C, idx, D_v, scale)
    ref_out, ref_lse = _sdpa_reference(Q, C, idx, D_v, scale)
    np.testing.assert_allclose(out, ref_out.numpy(), rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(lse, ref_lse.numpy(), rtol=1e-12, atol=1e-12)


def test_attend_high_precision_bruteforce():
    mpmath = pytest.importorskip("mpmath")
    mpmath.mp.dps = 40
    g = torch.Generator().manual_seed(3)
    H, D, D_v, L_cap = 2, 5, 3, 7
    Q, C = _bf16((1, 1, H, D), g), _bf16((1, L_cap, D), g)
    idx = np.array([[[4, -1, 0, 6, 2]]], dtype=np.int32)
    scale = 0.37
    out, lse = oracle.sparse_mla_attend(Q, C, idx, D_v, scale)
    sel = [4, 0, 6, 2]
    sc = mpmath.mpf(float(np.float32(scale)))
    for h in range(H):
        z = [sc * mpmath.fsum(mpmath.mpf(float(Q[0, 0, h, d])) * mpmath.mpf(float(C[0, s, d]))
                              for d in range(D)) for s in sel]
        Z = mpmath.fsum(mpmath.exp(x) for x in z)
        for v in range(D_v):
            want = mpmath.fsum(mpmath.exp(x) * mpmath.mpf(float(C[0, s, v]))
                               for x, s in zip(z, sel)) / Z
            assert abs(out[0, 0, h, v] - float(want)) < 1e-14
        assert abs(lse[0, 0, h] - float(mpmath.log(Z))) < 1e-14


def test_attend_closed_forms():
    g = torch.Generator().manual_seed(11)
    H, D, D_v, L_cap, k = 3, 12, 8, 20, 6
    C = _bf16((1, L_cap, D), g)
    Cd = C.double().numpy()
    idx = np.array([[[3, 17, -1, 8, 0, -1]]], dtype=np.int32)
    sel = [3, 17, 8, 0]
    # Q = 0: uniform weights, the mean of the selected value rows; lse = log n
    out, lse = oracle.sparse_mla_attend(torch.zeros(1, 1, H, D, dtype=torch.bfloat16), C, idx,
                                        D_v, 0.25)
    for h in range(H):
        np.testing.assert_allclose(out[0, 0, h], Cd[0, sel, :D_v].mean(axis=0), rtol=0,
                                   atol=1e-15)
        assert abs(lse[0, 0, h] - math.log(len(sel))) < 1e-15
    Q = _bf16((1, 1, H, D), g)
    # one valid slot: exactly that row; lse = its logit
    one = np.array([[[-1, -1, 9, -1, -1, -1]]], dtype=np.int32)
    out, lse = oracle.sparse_mla_attend(Q, C, one, D_v, 0.25)
    for h in range(H):
        np.testing.assert_array_equal(out[0, 0, h], Cd[0, 9, :D_v])
        want = 0.25 * float(np.dot(Q[0, 0, h].double().numpy(), Cd[0, 9]))
        assert abs(lse[0, 0, h] - want) < 1e-12
    # a value column that is constant over the selected rows stays that constant
    C2 = C.clone()
    C2[0, :, 2] = 1.5
    out, _ = oracle.sparse_mla_attend(Q, C2, idx, D_v, 0.25)
    np.testing.assert_allclose(out[0, 0, :, 2], 1.5, rtol=0, atol=1e-15)
    # no valid slot: zeros and lse = -inf
    none = np.full((1, 1, k), -1, dtype=np.int32)
    out, lse = oracle.sparse_mla_attend(Q, C, none, D_v, 0.25)
    assert np.all(out == 0) and np.all(lse == -np.inf)
    # the order of the slots does not matter
    out_a, lse_a = oracle.sparse_mla_attend(Q, C, idx, D_v, 0.25)
    out_b, lse_b = oracle.sparse_mla_attend(Q, C, idx[:, :, ::-1].copy(), D_v, 0.25)
    np.testing.assert_allclose(out_a, out_b, rtol=1e-14, atol=1e-15)
    np.testing.assert_allclose(lse_a, lse_b, rtol=1e-14, atol=1e-15)


# --------------------------------------------------------- FP8 latent cache ----

def test_e4m3_decoder_matches_torch_for_every_code():
    # the oracle decodes E4M3 from its bit definition; torch's float8_e4m3fn is
    # an independent implementation of the same OCP format
    ref = torch.arange(256, dtype=torch.int32).to(torch.uint8).view(torch.float8_e4m3fn).double()
    got = np.array([oracle.e4m3_to_double(c) for c in range(256)])
    nan = np.isnan(ref.numpy())
    assert list(np.flatnonzero(nan)) == [0x7F, 0xFF]
    np.testing.assert_array_equal(np.isnan(got), nan)
    np.testing.assert_array_equal(got[~nan], ref.numpy()[~nan])
    # closed forms: largest finite, smallest subnormal, smallest normal, signed zero
    assert oracle.e4m3_to_double(0x7E) == 448.0
    assert oracle.e4m3_to_double(0x01) == 2.0 ** -9
    assert oracle.e4m3_to_double(0x08) == 2.0 ** -6
    assert oracle.e4m3_to_double(0xC0) == -2.0
    assert math.copysign(1.0, oracle.e4m3_to_double(0x80)) == -1.0


def _fp8_case(seed, B, Tq, H, D_c, D_r, L_cap, k):
    g = torch.Generator().manual_seed(seed)
    r = _rng(seed)
    C8, Ce, Cr = synth.fp8_cache(B, L_cap, D_c, D_r, g, "cpu")
    Q = _bf16((B, Tq, H, D_c + D_r), g)
    idx = np.full((B, Tq, k), -1, dtype=np.int32)
    for b in range(B):
        for t in range(Tq):
            m = int(r.integers(1, min(k, L_cap) + 1))
            idx[b, t, :m] = r.choice(L_cap, size=m, replace=False)
    # the cache each row stands for, dequantized by torch in float64
    lat = C8.view(torch.float8_e4m3fn).double() * torch.exp2(Ce.double() - 127)[..., None]
    C = torch.cat([lat, Cr.double()], dim=-1)
    return Q, C8, Ce, Cr, idx, C


@pytest.mark.parametrize("seed", range(4))
def test_fp8_attend_matches_sdpa_on_the_dequantized_cache(seed):
    Q, C8, Ce, Cr, idx, C = _fp8_case(300 + seed, 2, 2, 3, 16, 4, 30, 9)
    scale = float(np.float32(1.0 / math.sqrt(20)))
    out, lse = oracle.sparse_mla_attend_fp8(Q, C8, Ce, Cr, idx, scale)
    ref_out, ref_lse = _sdpa_reference(Q, C, idx, 16, scale)
    np.testing.assert_allclose(out, ref_out.numpy(), rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(lse, ref_lse.numpy(), rtol=1e-12, atol=1e-12)


def test_fp8_attend_equals_bf16_attend_when_dequantization_is_exact():
    # with power-of-two row scales every dequantized value is a bf16 number, so
    # attention over the FP8 cache is attention over that bf16 cache, bit for bit
    Q, C8, Ce, Cr, idx, C = _fp8_case(7, 2, 3, 4, 32, 8, 50, 12)
    Cb = C.to(torch.bfloat16)
    assert torch.equal(Cb.double(), C)
    out8, lse8 = oracle.sparse_mla_attend_fp8(Q, C8, Ce, Cr, idx, 0.2)
    outb, lseb = oracle.sparse_mla_attend(Q, Cb, idx, 32, 0.2)
    np.testing.assert_array_equal(out8, outb)
    np.testing.assert_array_equal(lse8, lseb)


# ------------------------------------------------------------ paged caches ----

def _paged(cache, bs, seed, extra=3):
    g = torch.Generator().manual_seed(seed)
    B, L = cache.shape[0], cache.shape[1]
    table = synth.page_layout(B, L, bs, g, "cpu", extra_pages=extra)
    n_pages = B * (L // bs) + extra
    return synth.to_pages(cache, table, bs, n_pages), table


@pytest.mark.parametrize("bs", [32, 64])
def test_paged_oracle_is_the_contiguous_one_under_any_page_placement(bs):
    # pages placed in a random order (plus unused pages) give the results of
    # the logical, contiguous cache
    r = _rng(600 + bs)
    B, Tq, H_I, D_I, L = 2, 3, 4, 32, 256
    g = torch.Generator().manual_seed(bs)
    qI = synth.int8_uniform((B, Tq, H_I, D_I), g, "cpu")
    w = synth.pow2_weights((B, Tq, H_I), g, "cpu")
    kI = synth.int8_uniform((B, L, D_I), g, "cpu")
    kv_len = torch.tensor([L, 150], dtype=torch.int32)
    pool, table = _paged(kI, bs, bs)
    np.testing.assert_array_equal(oracle.indexer_scores_paged(qI, w, pool, table, kv_len),
                                  oracle.indexer_scores(qI, w, kI, kv_len))
    H, D, D_v, k = 2, 20, 16, 9
    Q, C = _bf16((B, Tq, H, D), g), _bf16((B, L, D), g)
    idx = r.integers(-1, L, size=(B, Tq, k)).astype(np.int32)
    cpool, ctable = _paged(C, bs, bs + 1)
    o1, l1 = oracle.sparse_mla_attend_paged(Q, cpool, ctable, idx, D_v, 0.3)
    o2, l2 = oracle.sparse_mla_attend(Q, C, idx, D_v, 0.3)
    np.testing.assert_array_equal(o1, o2)
    np.testing.assert_array_equal(l1, l2)


def test_paged_oracle_unallocated_blocks():
    # an unallocated block (-1, or a page id past the pool) scores -inf and
    # its slots are skipped: attention equals dropping those slots
    bs, B, Tq, L = 32, 1, 2, 128
    g = torch.Generator().manual_seed(5)
    qI = synth.int8_uniform((B, Tq, 4, 32), g, "cpu")
    w = synth.pow2_weights((B, Tq, 4), g, "cpu")
    kI = synth.int8_uniform((B, L, 32), g, "cpu")
    kv_len = torch.tensor([L], dtype=torch.int32)
    pool, table = _paged(kI, bs, 9, extra=0)
    table[0, 1] = -1
    table[0, 3] = 1000
    S = oracle.indexer_scores_paged(qI, w, pool, table, kv_len)
    ref = oracle.indexer_scores(qI, w, kI, kv_len)
    dead = np.zeros(L, dtype=bool)
    dead[32:64] = dead[96:128] = True
    assert np.all(np.isneginf(S[:, :, dead]))
    np.testing.assert_array_equal(S[:, :, ~dead], ref[:, :, ~dead])
    Q, C = _bf16((B, Tq, 2, 12), g), _bf16((B, L, 12), g)
    cpool, _ = _paged(C, bs, 9, extra=0)          # same seed: same placement as the keys
    idx = np.array([[[0, 40, 70, 100, -1], [33, 34, 35, 5, 64]]], dtype=np.int32)
    out, lse = oracle.sparse_mla_attend_paged(Q, cpool, table, idx, 8, 0.5)
    idx_live = np.where(dead[np.clip(idx, 0, L - 1)] | (idx < 0), -1, idx).astype(np.int32)
    out2, lse2 = oracle.sparse_mla_attend(Q, C, idx_live, 8, 0.5)
    np.testing.assert_array_equal(out, out2)
    np.testing.assert_array_equal(lse, lse2)


# ------------------------------------------------------ index access counts ----

@pytest.mark.parametrize("seed", range(3))
def test_index_histogram_matches_bincount(seed):
    r = _rng(500 + seed)
    B, Tq, k, L_cap = 3, 5, 17, 60
    idx = r.integers(-3, L_cap + 4, size=(B, Tq, k)).astype(np.int32)   # invalid values too
    counts = oracle.index_histogram(idx, L_cap)
    for b in range(B):
        v = idx[b].ravel()
        v = v[(v >= 0) & (v < L_cap)]
        np.testing.assert_array_equal(counts[b], np.bincount(v, minlength=L_cap))
    assert int(counts.sum()) == int(((idx >= 0) & (idx < L_cap)).sum())
    # counts accumulate: a second call adds the same counts again
    twice = oracle.index_histogram(idx, L_cap, counts=counts.copy())
    np.testing.assert_array_equal(twice, 2 * counts)


def test_dense_causal_when_context_fits_k():
    # When every query sees at most k keys, the sparse layer is plain causal
    # attention; checked against torch SDPA(is_causal) on a scaled-down C1.
    wl = synth.WORKLOADS["C1"].scaled(Tq=48, kv_len=48, L_cap=48, k=64)
    inp = synth.group_inputs(wl, layers=1)
    idx, outs, lses = oracle.group_forward([inp["qI"]], [inp["w"]], [inp["kI"]], inp["kv_len"],
                                           inp["Q"], inp["C"], wl.k, wl.D_v, wl.sm_scale)
    for t in range(wl.Tq):
        assert idx[0, t].tolist() == list(range(t + 1)) + [-1] * (wl.k - t - 1)
    Q = inp["Q"][0][0].double().transpose(0, 1)                # [H, Tq, D]
    C = inp["C"][0][0].double()
    K = C.unsqueeze(0).expand(wl.H, -1, -1)
    V = C[:, : wl.D_v].unsqueeze(0).expand(wl.H, -1, -1)
    ref = torch.nn.functional.scaled_dot_product_attention(Q, K, V, is_causal=True,
                                                           scale=float(np.float32(wl.sm_scale)))
    np.testing.assert_allclose(outs[0][0], ref.transpose(0, 1).numpy(), rtol=1e-11, atol=1e-12)


# ----------------------------------------------------------------- group ----

def test_group_shares_one_index_set_and_composes():
    wl = synth.WORKLOADS["C1"].scaled(Tq=96, kv_len=200, L_cap=224, k=16)
    inp = synth.group_inputs(wl)
    idx, outs, lses = oracle.group_forward([inp["qI"]], [inp["w"]], [inp["kI"]], inp["kv_len"],
                                           inp["Q"], inp["C"], wl.k, wl.D_v, wl.sm_scale)
    S = oracle.indexer_scores(inp["qI"], inp["w"], inp["kI"], inp["kv_len"])
    idx_one = oracle.topk_select(S, inp["kv_len"], wl.k)
    np.testing.assert_array_equal(idx, idx_one)
    for l in range(wl.n_layers):
        o, s = oracle.sparse_mla_attend(inp["Q"][l], inp["C"][l], idx_one, wl.D_v, wl.sm_scale)
        np.testing.assert_array_equal(outs[l], o)
        np.testing.assert_array_equal(lses[l], s)
    # later MTP steps: the given set is used as is, by every layer
    rng = random.Random(0)
    given = idx.copy()
    for row in given.reshape(-1, wl.k):
        rng.shuffle(row)
    idx2, outs2, _ = oracle.group_forward([inp["qI"]], [inp["w"]], [inp["kI"]], inp["kv_len"],
                                          inp["Q"], inp["C"], wl.k, wl.D_v, wl.sm_scale,
                                          idx=given, reuse_idx=True)
    np.testing.assert_array_equal(idx2, given)
    for l in range(wl.n_layers):
        np.testing.assert_allclose(outs2[l], outs[l], rtol=1e-13, atol=1e-15)
    # per-layer indexers fed identical inputs reproduce the shared group
    n = wl.n_layers
    idx3, outs3, _ = oracle.group_forward([inp["qI"]] * n, [inp["w"]] * n, [inp["kI"]] * n,
                                          inp["kv_len"], inp["Q"], inp["C"], wl.k, wl.D_v,
                                          wl.sm_scale, per_layer_indexer=True)
    np.testing.assert_array_equal(idx3, idx)
    for l in range(n):
        np.testing.assert_array_equal(outs3[l], outs[l])


def _numpy_scores(qI, w, kI, kv_len):
    """S by exact int64 dot products, ReLU, the weighted head sum in float64
    rounded once to float32; -inf past each query's position (numpy only)."""
    B, Tq, H_I, D_I = qI.shape
    L_cap = kI.shape[1]
    S = np.full((B, Tq, L_cap), -np.inf, dtype=np.float32)
    for b in range(B):
        dots = qI[b].astype(np.int64).reshape(Tq * H_I, D_I) @ kI[b].astype(np.int64).T
        relu = np.maximum(dots, 0).reshape(Tq, H_I, L_cap).astype(np.float64)
        tot = np.einsum("th,thl->tl", w[b].astype(np.float64), relu)
        for t in range(Tq):
            pos = _positions(kv_len, L_cap, Tq, b, t)
            if pos >= 0:
                S[b, t, : pos + 1] = tot[t, : pos + 1].astype(np.float32)
    return S


def _numpy_topk(S, kv_len, k):
    """Ascending positions of the best min(k, pos+1) keys under (score desc,
    position asc), -1 padded (numpy lexsort)."""
    B, Tq, L_cap = S.shape
    idx = np.full((B, Tq, k), -1, dtype=np.int32)
    for b in range(B):
        for t in range(Tq):
            n = max(_positions(kv_len, L_cap, Tq, b, t) + 1, 0)
            if n == 0:
                continue
            v = S[b, t, :n].astype(np.float64) + 0.0          # -0.0 ranks as +0.0
            order = np.lexsort((np.arange(n), -v))
            sel = np.sort(order[: min(k, n)])
            idx[b, t, : len(sel)] = sel
    return idx


def _sdpa_selected(Q, C, idx, D_v, sm_scale):
    """out [B,Tq,H,D_v] float64: torch float64 SDPA of each query over its
    selected rows (V = the first D_v columns)."""
    Qd = Q.double()
    Cd = C.double()
    B, Tq, H, D = Q.shape
    out = np.zeros((B, Tq, H, D_v))
    for b in range(B):
        for t in range(Tq):
            sel = [int(s) for s in idx[b, t] if s >= 0]
            if not sel:
                continue
            rows = Cd[b, sel]                                   # [n, D]
            q = Qd[b, t].unsqueeze(1)                           # [H, 1, D]
            K = rows.unsqueeze(0).expand(H, -1, -1)
            V = rows[:, :D_v].unsqueeze(0).expand(H, -1, -1)
            o = torch.nn.functional.scaled_dot_product_attention(
                q, K, V, scale=float(np.float32(sm_scale)))
            out[b, t] = o[:, 0].numpy()
    return out


def test_group_per_layer_indexer_distinct_inputs():
    # The ablation without sharing ("GLM-5.2核心技术解析", the per-layer vs
    # shared-indexer comparison table): layer l runs its own indexer + top-k
    # from its own (qI, w, kI).  Expected values come from numpy integer
    # scores, a lexsort top-k and float64 SDPA per layer, and also from the
    # single-layer oracle calls composed by hand.  The per-layer inputs are
    # drawn so that every layer's index set differs from every other layer's,
    # so reading layer 0's indexer inputs for every layer cannot pass.
    wl = synth.WORKLOADS["C1"].scaled(B=2, Tq=24, kv_len=90, L_cap=100, k=12,
                                      ablation_seeds=(40, 41, 42, 43))
    inp = synth.group_inputs(wl)
    abl = synth.ablation_indexers(wl)
    n = wl.n_layers
    idx, outs, lses = oracle.group_forward([a["qI"] for a in abl], [a["w"] for a in abl],
                                           [a["kI"] for a in abl], inp["kv_len"], inp["Q"],
                                           inp["C"], wl.k, wl.D_v, wl.sm_scale,
                                           per_layer_indexer=True)
    kv = inp["kv_len"].numpy()
    sets = []
    for l in range(n):
        a = abl[l]
        S_np = _numpy_scores(a["qI"].numpy(), a["w"].numpy(), a["kI"].numpy(), kv)
        idx_np = _numpy_topk(S_np, kv, wl.k)
        sets.append(idx_np)
        out_np = _sdpa_selected(inp["Q"][l], inp["C"][l], idx_np, wl.D_v, wl.sm_scale)
        np.testing.assert_allclose(outs[l], out_np, rtol=1e-10, atol=1e-12)
        # the same composed from the single-layer oracle calls
        S_o = oracle.indexer_scores(a["qI"], a["w"], a["kI"], inp["kv_len"])
        assert S_o.tobytes() == S_np.tobytes()
        idx_o = oracle.topk_select(S_o, inp["kv_len"], wl.k)
        np.testing.assert_array_equal(idx_o, idx_np)
        o_o, l_o = oracle.sparse_mla_attend(inp["Q"][l], inp["C"][l], idx_o, wl.D_v, wl.sm_scale)
        np.testing.assert_array_equal(outs[l], o_o)
        np.testing.assert_array_equal(lses[l], l_o)
    # idx ends holding the last layer's set
    np.testing.assert_array_equal(idx, sets[-1])
    for i in range(n):
        for j in range(i + 1, n):
            assert not np.array_equal(sets[i], sets[j]), (i, j)
