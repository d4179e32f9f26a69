"""Pins for the float64 oracle against what the pages and the mathematics fix.

Each test checks the oracle against something other than itself: values
the pages print (tests/golden/*.json, each with its source), closed forms,
invariants, high-precision brute force on tiny inputs, a library routine for
the special case it covers, and finite differences for the backward.
"""

import itertools
import json
import math
import os
from decimal import Decimal, getcontext

import numpy as np
import pytest

import oracle

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def golden(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


def rand_qkv(B, H, N, d, seed, Nk=None):
    rng = np.random.default_rng(seed)
    Nk = N if Nk is None else Nk
    return (rng.standard_normal((B, H, N, d)), rng.standard_normal((B, H, Nk, d)),
            rng.standard_normal((B, H, Nk, d)))


# ---------------------------------------------------------------------------
# Printed worked examples
# ---------------------------------------------------------------------------

def test_six_scores_running_state_matches_page():
    g = golden("six_scores.json")
    s = np.array(g["scores"])
    vals = np.zeros((6, 1))
    _, trace = oracle.online_row(s, vals, tile=g["tile"], return_state=True)
    assert len(trace) == 2
    m1, a1, l1, _ = trace[0]
    m2, a2, l2, _ = trace[1]
    nd = g["printed_decimals"]
    assert m1 == g["after_block_1"]["m"]
    assert round(l1, nd) == g["after_block_1"]["l"]
    assert m2 == g["after_block_2"]["m"]
    assert a2 == pytest.approx(math.exp(g["after_block_2"]["alpha_exponent"]), rel=1e-15)
    assert round(l2, nd) == g["after_block_2"]["l"]
    # the final running sum equals the whole-row sum relative to the final max
    whole = sum(math.exp(x - 4.0) for x in g["scores"])
    assert l2 == pytest.approx(whole, rel=1e-15)


def test_six_scores_with_values_matches_full_softmax():
    g = golden("six_scores.json")
    s = np.array(g["scores"])
    rng = np.random.default_rng(7)
    vals = rng.standard_normal((6, 5))          # values are not printed on the page
    out = oracle.online_row(s, vals, tile=3)
    w = np.exp(s - s.max())
    full = (w @ vals) / w.sum()
    # page: largest difference about 5.6e-17, i.e. rounding
    assert np.max(np.abs(out - full)) <= 1e-15


def test_toy_two_tiles_matches_page():
    g = golden("toy_two_tiles.json")
    ln2 = math.log(2.0)
    s = np.array([0.0, ln2])
    vals = np.array(g["values"])
    out, trace = oracle.online_row(s, vals, tile=g["tile"], return_state=True)
    (m1, _, l1, o1), (m2, a2, l2, o2) = trace
    assert (m1, l1) == (g["after_tile_1"]["m"], g["after_tile_1"]["l"])
    assert o1.tolist() == g["after_tile_1"]["o"]
    assert m2 == pytest.approx(ln2, rel=1e-15)
    assert a2 == pytest.approx(g["after_tile_2"]["alpha"], rel=1e-15)
    assert l2 == pytest.approx(g["after_tile_2"]["l"], rel=1e-15)
    assert o2[0] == pytest.approx(g["after_tile_2"]["o"][0], rel=1e-15)
    expect = g["output"]["numerator"] / g["output"]["denominator"]
    assert out[0] == pytest.approx(expect, rel=1e-15)
    # route A on the same toy (as a one-query, two-key head with d = 1)
    q = np.array([[[[1.0]]]])
    k = np.array([[[[0.0], [ln2]]]])
    v = np.array(vals)[None, None]
    o, lse = oracle.attention_materialised(q, k, v, 1.0)
    assert o[0, 0, 0, 0] == pytest.approx(expect, rel=1e-15)
    assert lse[0, 0, 0] == pytest.approx(math.log(3.0), rel=1e-15)


def test_tiled_run_bound_256x16_blocks_of_64():
    g = golden("exactness_bounds.json")["tiled_run"]
    q, k, v = rand_qkv(1, 1, g["tokens"], g["head_dim"], seed=11)
    scale = 1.0 / math.sqrt(g["head_dim"])
    oa, la = oracle.attention_materialised(q, k, v, scale)
    ob, lb = oracle.attention_online(q, k, v, scale, tile=g["block_rows"])
    # page: at most about 5.6e-16
    assert np.max(np.abs(oa - ob)) <= 1e-14
    assert np.max(np.abs(la - lb)) <= 1e-13
    # scores held: the whole matrix versus one block
    assert g["tokens"] ** 2 == g["standard_scores_held"]
    assert g["block_rows"] ** 2 == g["tiled_scores_held_max"]


# ---------------------------------------------------------------------------
# Tile-size invariance and the two classic breakages
# ---------------------------------------------------------------------------

def _fp32_equal_except_ties(a, b):
    """float32 rounding of a and b agree everywhere, except where the float64
    value sits within a few float64 ulps of a float32 rounding boundary."""
    fa = a.astype(np.float32)
    fb = b.astype(np.float32)
    diff = fa != fb
    if not diff.any():
        return True
    # a disagreement is acceptable only right at a float32 midpoint
    x = a[diff]
    lo = x.astype(np.float32).astype(np.float64)
    ulp = np.spacing(np.abs(x).astype(np.float32)).astype(np.float64)
    dist = np.minimum(np.abs(np.abs(x - lo) - ulp / 2), np.abs(x - lo))
    return bool(np.all(dist <= 1e-12 * np.maximum(np.abs(x), 1e-300)))


@pytest.mark.parametrize("causal,length", [(False, None), (True, None), (True, 70), (False, 33)])
def test_tile_size_invariance(causal, length):
    N, d = 100, 8
    q, k, v = rand_qkv(1, 2, N, d, seed=3)
    lengths = None if length is None else np.array([length])
    oa, la = oracle.attention_materialised(q, k, v, 0.35, causal, lengths)
    for T in (1, 2, 3, 5, 7, 16, 64, 100, N):
        ob, lb = oracle.attention_online(q, k, v, 0.35, causal, lengths, tile=T)
        assert np.max(np.abs(oa - ob)) <= 1e-14, T
        fin = np.isfinite(la)
        assert np.array_equal(fin, np.isfinite(lb))
        assert np.max(np.abs(la[fin] - lb[fin])) <= 1e-13
        assert _fp32_equal_except_ties(oa, ob), T


def test_missing_rescale_is_caught():
    s = np.array(golden("six_scores.json")["scores"])
    vals = np.random.default_rng(5).standard_normal((6, 3))
    good = oracle.online_row(s, vals, tile=3)
    bad = oracle.online_row(s, vals, tile=3, rescale=False)
    assert np.max(np.abs(good - bad)) > 1e-2


def test_missing_max_subtraction_overflows_fp32_at_x30():
    # scores at x30 magnitude: the largest is 90, exp(90) ~ 1.2e39 > fp32 max
    rng = np.random.default_rng(9)
    s = np.concatenate([rng.uniform(-3, 3, 63), [3.0]]) * 30.0
    vals = rng.standard_normal((64, 4))
    assert math.exp(90.0) > float(np.finfo(np.float32).max)
    good32 = oracle.online_row(s, vals, tile=8, dtype=np.float32)
    bad32 = oracle.online_row(s, vals, tile=8, dtype=np.float32, subtract_max=False)
    assert np.all(np.isfinite(good32))
    assert not np.all(np.isfinite(bad32))
    # at x6 the subtraction is algebraically a no-op and both agree
    s6 = s / 5.0
    a = oracle.online_row(s6, vals, tile=8, dtype=np.float32)
    b = oracle.online_row(s6, vals, tile=8, dtype=np.float32, subtract_max=False)
    assert np.max(np.abs(a - b)) <= 1e-5


def test_route_a_and_b_finite_with_x30_queries():
    q, k, v = rand_qkv(1, 1, 64, 16, seed=4)
    q = q * 30.0
    oa, la = oracle.attention_materialised(q, k, v, 0.25, causal=True)
    ob, lb = oracle.attention_online(q, k, v, 0.25, causal=True, tile=16)
    assert np.all(np.isfinite(oa)) and np.all(np.isfinite(la))
    assert np.max(np.abs(oa - ob)) <= 1e-13
    assert np.max(np.abs(la)) > 60.0          # scores really are large


# ---------------------------------------------------------------------------
# Empty-row policy and input validation
# ---------------------------------------------------------------------------

def test_empty_rows_return_zeros_and_neg_inf_lse():
    q, k, v = rand_qkv(2, 1, 16, 4, seed=8)
    lengths = np.array([0, 5])
    for causal in (False, True):
        oa, la = oracle.attention_materialised(q, k, v, 0.5, causal, lengths)
        ob, lb = oracle.attention_online(q, k, v, 0.5, causal, lengths, tile=3)
        assert np.all(oa[0] == 0.0) and np.all(np.isneginf(la[0]))
        assert np.all(ob[0] == 0.0) and np.all(np.isneginf(lb[0]))
        assert np.all(np.isfinite(la[1]))


def test_online_row_skips_leading_masked_chunk():
    s = np.array([-np.inf, -np.inf, -np.inf, 1.0, 2.0, -np.inf])
    vals = np.arange(12, dtype=float).reshape(6, 2)
    with np.errstate(invalid="raise"):
        out = oracle.online_row(s, vals, tile=3)
    w = np.exp(np.array([1.0, 2.0]) - 2.0)
    assert np.allclose(out, (w @ vals[3:5]) / w.sum(), rtol=0, atol=1e-15)
    assert np.all(oracle.online_row(np.full(4, -np.inf), vals[:4], tile=2) == 0.0)
    assert np.all(oracle.online_row(np.zeros(0), np.zeros((0, 3)), tile=2) == 0.0)


@pytest.mark.parametrize("scores,values,tile", [
    (np.zeros(3), np.zeros((4, 2)), 2),              # one score per value row
    (np.zeros((3, 1)), np.zeros((3, 2)), 2),         # scores must be 1-D
    (np.zeros(3), np.zeros(3), 2),                   # values must be 2-D
    (np.zeros(3), np.zeros((3, 2)), 0),              # positive tile
    (np.zeros(3), np.zeros((3, 2)), -1),
    (np.zeros(3), np.zeros((3, 2)), 2.0),            # int tile
    (np.zeros(3), np.zeros((3, 2)), True),
    (np.array([0.0, np.nan, 1.0]), np.zeros((3, 2)), 2),
    (np.array([0.0, np.inf, 1.0]), np.zeros((3, 2)), 2),
    (np.zeros(3), np.array([[0.0, np.inf]] * 3), 2),
    (np.zeros(3), np.array([[0.0, np.nan]] * 3), 2),
])
def test_online_row_validation(scores, values, tile):
    with pytest.raises(ValueError):
        oracle.online_row(scores, values, tile=tile)


def test_attention_online_rejects_bad_tile():
    q, k, v = rand_qkv(1, 1, 4, 2, seed=0)
    for t in (0, -3, 2.5, True):
        with pytest.raises(ValueError):
            oracle.attention_online(q, k, v, 1.0, tile=t)


# ---------------------------------------------------------------------------
# Closed forms and invariances
# ---------------------------------------------------------------------------

def test_single_visible_key_closed_form():
    q, k, v = rand_qkv(1, 2, 12, 5, seed=12)
    scale = 0.7
    # causal row 0 sees only key 0
    o, lse = oracle.attention_materialised(q, k, v, scale, causal=True)
    assert np.allclose(o[0, :, 0], v[0, :, 0], rtol=0, atol=1e-15)
    s00 = scale * np.einsum("hd,hd->h", q[0, :, 0], k[0, :, 0])
    assert np.allclose(lse[0, :, 0], s00, rtol=0, atol=1e-14)
    # key length 1: every row sees only key 0
    o, lse = oracle.attention_materialised(q, k, v, scale, causal=False, lengths=np.array([1]))
    assert np.allclose(o[0], np.broadcast_to(v[0, :, :1], o[0].shape), rtol=0, atol=1e-15)
    s_i0 = scale * np.einsum("hnd,hd->hn", q[0], k[0, :, 0])
    assert np.allclose(lse[0], s_i0, rtol=0, atol=1e-14)


@pytest.mark.parametrize("causal,length", [(False, None), (True, None), (True, 9), (False, 4)])
def test_zero_queries_give_mean_of_visible_values(causal, length):
    _, k, v = rand_qkv(1, 1, 13, 6, seed=21)
    q = np.zeros_like(k)
    lengths = None if length is None else np.array([length])
    for route in ("A", "B"):
        if route == "A":
            o, lse = oracle.attention_materialised(q, k, v, 1.3, causal, lengths)
        else:
            o, lse = oracle.attention_online(q, k, v, 1.3, causal, lengths, tile=4)
        L = 13 if length is None else length
        for i in range(13):
            n_vis = min(i + 1, L) if causal else L
            assert np.allclose(o[0, 0, i], v[0, 0, :n_vis].mean(axis=0), rtol=0, atol=1e-14)
            assert lse[0, 0, i] == pytest.approx(math.log(n_vis), abs=1e-14)


def test_constant_values_give_that_constant():
    q, k, _ = rand_qkv(1, 2, 17, 3, seed=2)
    c = np.array([1.5, -2.0, 0.25])
    v = np.broadcast_to(c, k.shape).copy()
    o, _ = oracle.attention_materialised(q, k, v, 0.9, causal=True)
    assert np.allclose(o, np.broadcast_to(c, o.shape), rtol=0, atol=1e-14)


def test_key_shift_and_value_shift_invariances():
    q, k, v = rand_qkv(1, 1, 20, 4, seed=31)
    scale = 0.6
    c = np.array([0.3, -1.1, 2.0, 0.5])
    lengths = np.array([15])
    o, lse = oracle.attention_materialised(q, k, v, scale, True, lengths)
    o2, lse2 = oracle.attention_materialised(q, k + c, v, scale, True, lengths)
    assert np.allclose(o2, o, rtol=0, atol=1e-13)
    assert np.allclose(lse2, lse + scale * (q @ c), rtol=0, atol=1e-13)
    o3, _ = oracle.attention_materialised(q, k, v + c, scale, True, lengths)
    assert np.allclose(o3, o + c, rtol=0, atol=1e-13)


def test_key_value_permutation_invariance_unmasked():
    q, k, v = rand_qkv(1, 1, 24, 4, seed=17)
    perm = np.random.default_rng(1).permutation(24)
    o, lse = oracle.attention_materialised(q, k, v, 0.5)
    o2, lse2 = oracle.attention_materialised(q, k[:, :, perm], v[:, :, perm], 0.5)
    assert np.allclose(o, o2, rtol=0, atol=1e-14)
    assert np.allclose(lse, lse2, rtol=0, atol=1e-14)


def test_matches_torch_sdpa_float64_unmasked_and_causal():
    torch = pytest.importorskip("torch")
    q, k, v = rand_qkv(2, 3, 33, 8, seed=41)
    for causal in (False, True):
        ref = torch.nn.functional.scaled_dot_product_attention(
            torch.from_numpy(q), torch.from_numpy(k), torch.from_numpy(v),
            is_causal=causal, scale=0.4).numpy()
        o, _ = oracle.attention_materialised(q, k, v, 0.4, causal)
        assert np.max(np.abs(o - ref)) <= 1e-13


# ---------------------------------------------------------------------------
# High-precision brute force on tiny inputs
# ---------------------------------------------------------------------------

def _brute_force_decimal(q, k, v, scale, causal, length):
    """Definition of attention in 60-digit decimal arithmetic, with plain
    exp(s) (no max subtraction) and plain loops; returns (o, lse) as float."""
    getcontext().prec = 60
    N, d = q.shape
    Nk = k.shape[0]
    L = Nk if length is None else min(max(length, 0), Nk)
    sc = Decimal(float(scale))
    o = np.zeros((N, v.shape[1]))
    lse = np.zeros(N)
    for i in range(N):
        num = [Decimal(0)] * v.shape[1]
        den = Decimal(0)
        for j in range(Nk):
            # query i sits at sequence position i + Nk - N (bottom-right)
            if j >= L or (causal and j > i + Nk - N):
                continue
            s = sc * sum(Decimal(float(q[i, t])) * Decimal(float(k[j, t])) for t in range(d))
            w = s.exp()
            den += w
            for t in range(v.shape[1]):
                num[t] += w * Decimal(float(v[j, t]))
        if den == 0:
            o[i] = 0.0
            lse[i] = -np.inf
        else:
            o[i] = [float(x / den) for x in num]
            lse[i] = float(den.ln())
    return o, lse


def test_brute_force_every_mask_combination_tiny():
    rng = np.random.default_rng(2024)
    for N in range(1, 6):
        q = rng.standard_normal((1, 1, N, 3))
        k = rng.standard_normal((1, 1, N, 3))
        v = rng.standard_normal((1, 1, N, 2))
        for causal in (False, True):
            for L in range(0, N + 1):
                lengths = np.array([L])
                ref_o, ref_l = _brute_force_decimal(q[0, 0], k[0, 0], v[0, 0], 0.8, causal, L)
                oa, la = oracle.attention_materialised(q, k, v, 0.8, causal, lengths)
                assert np.max(np.abs(oa[0, 0] - ref_o)) <= 1e-14
                assert np.array_equal(np.isneginf(la[0, 0]), np.isneginf(ref_l))
                fin = np.isfinite(ref_l)
                assert np.max(np.abs(la[0, 0][fin] - ref_l[fin]), initial=0) <= 1e-14
                for T in range(1, N + 1):
                    ob, lb = oracle.attention_online(q, k, v, 0.8, causal, lengths, tile=T)
                    assert np.max(np.abs(ob[0, 0] - ref_o)) <= 1e-14
                    assert np.array_equal(np.isneginf(lb[0, 0]), np.isneginf(ref_l))


def test_online_row_matches_brute_force_with_masks():
    rng = np.random.default_rng(99)
    for trial in range(20):
        n = int(rng.integers(1, 12))
        s = rng.normal(0, 3, n)
        s[rng.random(n) < 0.3] = -np.inf
        vals = rng.standard_normal((n, 3))
        getcontext().prec = 60
        den = sum((Decimal(float(x)).exp() for x in s if np.isfinite(x)), Decimal(0))
        if den == 0:
            ref = np.zeros(3)
        else:
            ref = np.array([float(sum(Decimal(float(x)).exp() * Decimal(float(vals[j, t]))
                                      for j, x in enumerate(s) if np.isfinite(x)) / den)
                            for t in range(3)])
        for T in (1, 2, 3, 5, 16):
            out = oracle.online_row(s, vals, tile=T)
            assert np.max(np.abs(out - ref)) <= 1e-14


def test_fewer_queries_are_the_last_rows_of_the_square_problem():
    """Causal attention of Nq queries against Nk keys equals the last Nq rows
    of the square causal problem whose queries end with them (the rows before
    do not influence later rows), for every key length."""
    rng = np.random.default_rng(31)
    Nk, Nq, d = 23, 7, 5
    k, v = rng.standard_normal((2, 1, 1, Nk, d))
    q_full = rng.standard_normal((1, 1, Nk, d))
    for length in (None, np.array([0]), np.array([3]), np.array([20]), np.array([23])):
        o_sq, l_sq = oracle.attention_materialised(q_full, k, v, 0.7, True, length)
        o_r, l_r = oracle.attention_materialised(q_full[:, :, Nk - Nq:], k, v, 0.7, True, length)
        assert np.array_equal(np.isneginf(l_r), np.isneginf(l_sq[:, :, Nk - Nq:]))
        assert np.max(np.abs(o_r - o_sq[:, :, Nk - Nq:])) <= 1e-13
        fin = np.isfinite(l_r)
        if fin.any():
            assert np.max(np.abs(l_r[fin] - l_sq[:, :, Nk - Nq:][fin])) <= 1e-13
        # the online route agrees
        o_b, l_b = oracle.attention_online(q_full[:, :, Nk - Nq:], k, v, 0.7, True, length, tile=4)
        assert np.max(np.abs(o_b - o_r)) <= 1e-13


def test_more_queries_than_keys_leave_the_first_rows_empty():
    """With Nq > Nk the first Nq - Nk queries precede every key: O = 0 and
    LSE = -inf; the remaining rows are the square problem over the Nk keys."""
    rng = np.random.default_rng(32)
    Nk, Nq, d = 9, 14, 4
    q = rng.standard_normal((1, 2, Nq, d))
    k, v = rng.standard_normal((2, 1, 2, Nk, d))
    o, lse = oracle.attention_materialised(q, k, v, 0.5, True)
    assert np.all(o[:, :, :Nq - Nk] == 0.0) and np.all(np.isneginf(lse[:, :, :Nq - Nk]))
    o_sq, l_sq = oracle.attention_materialised(q[:, :, Nq - Nk:], k, v, 0.5, True)
    assert np.max(np.abs(o[:, :, Nq - Nk:] - o_sq)) <= 1e-14
    assert np.max(np.abs(lse[:, :, Nq - Nk:] - l_sq)) <= 1e-14


def test_one_causal_query_sees_the_whole_cache():
    """Nq = 1 with the causal mask is decoding: the query sees every valid key,
    as the independent decode routine computes it."""
    rng = np.random.default_rng(33)
    B, H, Nk, d = 3, 2, 40, 6
    q = rng.standard_normal((B, H, 1, d))
    k, v = rng.standard_normal((2, B, H, Nk, d))
    lengths = np.array([40, 17, 0])
    o, lse = oracle.attention_materialised(q, k, v, 0.3, True, lengths)
    o_d, l_d = oracle.attention_decode(q[:, :, 0], k, v, 0.3, lengths)
    assert np.max(np.abs(o[:, :, 0] - o_d)) <= 1e-13
    assert np.array_equal(np.isneginf(lse[:, :, 0]), np.isneginf(l_d))
    fin = np.isfinite(l_d)
    assert fin.sum() == 4        # sequence 2 has an empty cache
    assert np.max(np.abs(lse[:, :, 0][fin] - l_d[fin])) <= 1e-13


def test_rectangular_backward_matches_finite_differences():
    rng = np.random.default_rng(34)
    for Nq, Nk, lengths in ((3, 7, None), (6, 4, None), (4, 8, np.array([5]))):
        q = rng.standard_normal((1, 1, Nq, 3))
        k, v = rng.standard_normal((2, 1, 1, Nk, 3))
        do = rng.standard_normal((1, 1, Nq, 3))
        o, lse = oracle.attention_materialised(q, k, v, 0.8, True, lengths)
        g = oracle.attention_backward(q, k, v, o, do, lse, 0.8, True, lengths)
        fd = oracle.finite_difference_grads(q, k, v, do, 0.8, True, lengths)
        for a, b in zip(g, fd):
            assert np.max(np.abs(a - b)) <= 1e-6


def test_rectangular_and_rows_helper():
    q, k, v = rand_qkv(1, 1, 9, 4, seed=5, Nk=14)
    o, lse = oracle.attention_materialised(q, k, v, 0.5, causal=True, lengths=np.array([11]))
    ref_o, ref_l = _brute_force_decimal(q[0, 0], k[0, 0], v[0, 0], 0.5, True, 11)
    assert np.max(np.abs(o[0, 0] - ref_o)) <= 1e-14
    rows = np.array([0, 4, 8])
    o_r, l_r = oracle.attention_rows(q[0, 0], k[0, 0], v[0, 0], rows, 0.5, True, 11)
    assert np.array_equal(o_r, o[0, 0, rows]) and np.array_equal(l_r, lse[0, 0, rows])


# ---------------------------------------------------------------------------
# Packed batches: each sequence is its own problem
# ---------------------------------------------------------------------------

def _pack(t, starts, lens):
    """Rows starts[b] .. starts[b] + lens[b] of each padded [B, H, L, d]
    sequence, back to back: [H, sum(lens), d]."""
    return np.concatenate([t[b, :, s0:s0 + n] for b, (s0, n) in enumerate(zip(starts, lens))],
                          axis=1)


def _cu(lens):
    return np.concatenate([[0], np.cumsum(lens)]).astype(np.int64)


def test_packed_batch_equals_the_padded_batch_with_key_lengths():
    """Sequences of lengths L_b packed back to back give, row for row, what the
    padded batch with key lengths L_b gives on its first L_b rows: the padded
    route masks keys by length, the packed one slices each sequence out."""
    rng = np.random.default_rng(41)
    H, d, Lmax = 2, 4, 11
    lens = [5, 0, 11, 1, 7]
    B = len(lens)
    qp, kp, vp = (rng.standard_normal((B, H, Lmax, d)) for _ in range(3))
    zero = [0] * B
    q, k, v = (_pack(t, zero, lens) for t in (qp, kp, vp))
    for causal in (False, True):
        o, lse = oracle.attention_packed(q, k, v, _cu(lens), _cu(lens), 0.6, causal)
        o_p, l_p = oracle.attention_materialised(qp, kp, vp, 0.6, causal, np.array(lens))
        assert np.max(np.abs(o - _pack(o_p, zero, lens))) <= 1e-13
        assert np.max(np.abs(lse - _pack(l_p[..., None], zero, lens)[..., 0])) <= 1e-13


def test_packed_queries_are_the_last_rows_of_each_sequence():
    """Sequence b holding the last nq_b of its Lk_b query positions against
    its Lk_b keys equals rows Lk_b - nq_b .. Lk_b of the padded batch with
    key lengths Lk_b (causal: the per-sequence offset is Lk_b - nq_b); a
    sequence with more queries than keys leaves its first rows empty."""
    rng = np.random.default_rng(42)
    H, d, Lmax = 2, 3, 12
    lk = [6, 9, 3, 12, 4]
    lq = [6, 2, 0, 1, 4]
    B = len(lk)
    qp, kp, vp = (rng.standard_normal((B, H, Lmax, d)) for _ in range(3))
    starts = [a - b for a, b in zip(lk, lq)]
    q = _pack(qp, starts, lq)
    k, v = (_pack(t, [0] * B, lk) for t in (kp, vp))
    for causal in (False, True):
        o, lse = oracle.attention_packed(q, k, v, _cu(lq), _cu(lk), 0.45, causal)
        o_p, l_p = oracle.attention_materialised(qp, kp, vp, 0.45, causal, np.array(lk))
        assert np.max(np.abs(o - _pack(o_p, starts, lq))) <= 1e-13
        assert np.max(np.abs(lse - _pack(l_p[..., None], starts, lq)[..., 0])) <= 1e-13
    # 7 queries against 3 keys: the first 4 precede every key
    q7 = rng.standard_normal((H, 7, d))
    k3, v3 = rng.standard_normal((2, H, 3, d))
    o, lse = oracle.attention_packed(q7, k3, v3, [0, 7], [0, 3], 0.5, True)
    assert np.all(o[:, :4] == 0.0) and np.all(np.isneginf(lse[:, :4]))
    assert np.all(np.isfinite(lse[:, 4:]))


def test_packed_backward_equals_the_padded_backward():
    """Gradients of a packed batch equal those of the padded batch with key
    lengths L_b when dO is zero on the padding rows (padding queries then add
    nothing to dK and dV); the padded backward is pinned by finite
    differences."""
    rng = np.random.default_rng(43)
    H, d, Lmax = 1, 3, 8
    lens = [3, 8, 0, 5]
    B = len(lens)
    qp, kp, vp, dop = (rng.standard_normal((B, H, Lmax, d)) for _ in range(4))
    for b, n in enumerate(lens):
        dop[b, :, n:] = 0.0
    zero = [0] * B
    q, k, v, do = (_pack(t, zero, lens) for t in (qp, kp, vp, dop))
    for causal in (False, True):
        o, lse = oracle.attention_packed(q, k, v, _cu(lens), _cu(lens), 0.7, causal)
        got = oracle.attention_backward_packed(q, k, v, o, do, lse, _cu(lens), _cu(lens), 0.7,
                                               causal)
        o_p, l_p = oracle.attention_materialised(qp, kp, vp, 0.7, causal, np.array(lens))
        ref = oracle.attention_backward(qp, kp, vp, o_p, dop, l_p, 0.7, causal, np.array(lens))
        for a, r in zip(got, ref):
            assert np.max(np.abs(a - _pack(r, zero, lens))) <= 1e-13


def test_packed_rows_outside_every_sequence_stay_empty():
    """Rows that no sequence owns (a gap, a tail) get O = 0, LSE = -inf and
    zero gradients; a packed sequence never reads them."""
    rng = np.random.default_rng(44)
    q, k, v, do = (rng.standard_normal((2, 10, 4)) for _ in range(4))
    cu_q, cu_k = [1, 4, 4, 8], [0, 5, 6, 9]
    o, lse = oracle.attention_packed(q, k, v, cu_q, cu_k, 0.5, True)
    assert np.all(o[:, [0, 8, 9]] == 0.0) and np.all(np.isneginf(lse[:, [0, 8, 9]]))
    dq, dk, dv = oracle.attention_backward_packed(q, k, v, o, do, lse, cu_q, cu_k, 0.5, True)
    assert np.all(dq[:, [0, 8, 9]] == 0.0) and np.all(dk[:, 9] == 0.0) and np.all(dv[:, 9] == 0.0)
    # sequence 2 (keys 5 .. 6, no queries) has zero key gradients
    assert np.all(dk[:, 5] == 0.0) and np.all(dv[:, 5] == 0.0)
    # changing the unowned rows changes nothing owned
    q2, k2 = q.copy(), k.copy()
    q2[:, [0, 8, 9]] = 9.0
    k2[:, 9] = -7.0
    o2, lse2 = oracle.attention_packed(q2, k2, v, cu_q, cu_k, 0.5, True)
    assert np.array_equal(o2[:, 1:8], o[:, 1:8]) and np.array_equal(lse2[:, 1:8], lse[:, 1:8])


# ---------------------------------------------------------------------------
# Backward: finite differences and invariants
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("causal,lengths", [(False, None), (True, None),
                                            (True, np.array([0, 3])), (False, np.array([5, 2]))])
def test_backward_matches_finite_differences(causal, lengths):
    rng = np.random.default_rng(77)
    B, H, N, d = 2, 1, 6, 3
    q, k, v = (rng.standard_normal((B, H, N, d)) for _ in range(3))
    do = rng.standard_normal((B, H, N, d))
    scale = 0.9
    o, lse = oracle.attention_materialised(q, k, v, scale, causal, lengths)
    dq, dk, dv = oracle.attention_backward(q, k, v, o, do, lse, scale, causal, lengths)
    fq, fk, fv = oracle.finite_difference_grads(q, k, v, do, scale, causal, lengths)
    for a, f in ((dq, fq), (dk, fk), (dv, fv)):
        err = np.max(np.abs(a - f)) / max(1.0, np.max(np.abs(f)))
        assert err <= 1e-7


def test_backward_matches_torch_autograd_float64():
    torch = pytest.importorskip("torch")
    rng = np.random.default_rng(5)
    B, H, N, d = 1, 2, 19, 4
    q, k, v, do = (rng.standard_normal((B, H, N, d)) for _ in range(4))
    lengths = np.array([13])
    scale = 0.5
    o, lse = oracle.attention_materialised(q, k, v, scale, True, lengths)
    dq, dk, dv = oracle.attention_backward(q, k, v, o, do, lse, scale, True, lengths)
    tq, tk, tv = (torch.tensor(x, requires_grad=True) for x in (q, k, v))
    mask = torch.from_numpy(oracle.visible_mask(np.arange(N), N, True, 13))
    s = scale * tq @ tk.transpose(-1, -2)
    s = s.masked_fill(~mask, float("-inf"))
    out = torch.softmax(s, dim=-1) @ tv
    (out * torch.from_numpy(do)).sum().backward()
    assert np.max(np.abs(out.detach().numpy() - o)) <= 1e-14
    for a, t in ((dq, tq), (dk, tk), (dv, tv)):
        assert np.max(np.abs(a - t.grad.numpy())) <= 1e-13


def test_backward_invariants():
    rng = np.random.default_rng(123)
    B, H, N, d = 2, 2, 40, 8
    q, k, v, do = (rng.standard_normal((B, H, N, d)) for _ in range(4))
    lengths = np.array([0, 29])
    scale = 0.35
    o, lse = oracle.attention_materialised(q, k, v, scale, True, lengths)
    dq, dk, dv = oracle.attention_backward(q, k, v, o, do, lse, scale, True, lengths)
    # every row of dS sums to zero, so the key gradients sum to zero
    assert np.max(np.abs(dk.sum(axis=2))) <= 1e-12
    # sum_j dV_j equals the sum of dO over rows that see something
    nonempty = np.isfinite(lse)
    for b in range(B):
        for h in range(H):
            assert np.allclose(dv[b, h].sum(axis=0), do[b, h][nonempty[b, h]].sum(axis=0),
                               rtol=0, atol=1e-12)
    # rows with a single visible key (causal row 0) and empty rows have dQ = 0
    assert np.all(np.abs(dq[1, :, 0]) <= 1e-15)
    assert np.all(dq[0] == 0.0) and np.all(dk[0] == 0.0) and np.all(dv[0] == 0.0)
    # keys beyond the length get no gradient
    assert np.all(dk[1, :, 29:] == 0.0) and np.all(dv[1, :, 29:] == 0.0)


# ---------------------------------------------------------------------------
# Decoding against a cache and merging partial results over key parts
# ---------------------------------------------------------------------------

def test_merge_reproduces_toy_two_tiles():
    # each tile of the toy is one part: (o, lse) = (10, 0) and (20, ln 2)
    g = golden("toy_two_tiles.json")
    o, lse = oracle.merge_states(np.array([[10.0], [20.0]]), np.array([0.0, math.log(2.0)]))
    assert o[0] == pytest.approx(g["output"]["numerator"] / g["output"]["denominator"], rel=1e-15)
    # LSE = m + ln l after the last tile
    assert lse == pytest.approx(math.log(2.0) + math.log(g["after_tile_2"]["l"]), rel=1e-15)


def test_merge_reproduces_six_score_running_sum():
    g = golden("six_scores.json")
    s = np.array(g["scores"], dtype=np.float64)
    t = g["tile"]
    parts = [math.log(np.exp(s[i:i + t]).sum()) for i in range(0, len(s), t)]
    _, lse = oracle.merge_states(np.zeros((len(parts), 1)), np.array(parts))
    # the page's rescaled sum is l relative to the final maximum 4.0
    assert round(math.exp(lse - 4.0), g["printed_decimals"]) == g["after_block_2"]["l"]


def _sdpa_decode(q, k, v, scale, lengths):
    import torch
    B, H, N, d = k.shape
    o = np.zeros((B, H, v.shape[3]))
    lse = np.full((B, H), -np.inf)
    for b in range(B):
        L = N if lengths is None else int(min(max(lengths[b], 0), N))
        if L == 0:
            continue
        qt = torch.from_numpy(q[b][:, None, :])            # [H, 1, d]
        kt = torch.from_numpy(np.ascontiguousarray(k[b, :, :L]))
        vt = torch.from_numpy(np.ascontiguousarray(v[b, :, :L]))
        o[b] = torch.nn.functional.scaled_dot_product_attention(qt, kt, vt, scale=scale)[:, 0].numpy()
        lse[b] = torch.logsumexp(scale * (kt @ qt.transpose(1, 2))[..., 0], dim=-1).numpy()
    return o, lse


@pytest.mark.parametrize("chunk", [None, 1, 3, 7, 16, 64])
def test_decode_matches_torch_sdpa_with_lengths(chunk):
    rng = np.random.default_rng(11)
    B, H, N, d = 3, 2, 41, 8
    q = rng.standard_normal((B, H, d)) * 3.0
    k = rng.standard_normal((B, H, N, d))
    v = rng.standard_normal((B, H, N, d))
    lengths = np.array([41, 17, 1])
    o, lse = oracle.attention_decode(q, k, v, 0.4, lengths, chunk=chunk)
    ro, rl = _sdpa_decode(q, k, v, 0.4, lengths)
    np.testing.assert_allclose(o, ro, rtol=0, atol=1e-12)
    np.testing.assert_allclose(lse, rl, rtol=0, atol=1e-12)


def test_decode_closed_forms():
    rng = np.random.default_rng(12)
    B, H, N, d = 3, 2, 9, 4
    k = rng.standard_normal((B, H, N, d))
    v = rng.standard_normal((B, H, N, d))
    # zero query: every visible key weighs the same
    lengths = np.array([9, 4, 0])
    o, lse = oracle.attention_decode(np.zeros((B, H, d)), k, v, 1.0, lengths, chunk=2)
    np.testing.assert_allclose(o[0], v[0].mean(axis=1), atol=1e-14)
    np.testing.assert_allclose(o[1], v[1, :, :4].mean(axis=1), atol=1e-14)
    np.testing.assert_allclose(lse[:2], np.log([[9.0, 9.0], [4.0, 4.0]]), atol=1e-14)
    # an empty cache gives the empty-row policy
    assert np.all(o[2] == 0.0) and np.all(np.isneginf(lse[2]))
    # one visible key: the output is that value row, LSE its scaled score
    q = rng.standard_normal((B, H, d))
    o, lse = oracle.attention_decode(q, k, v, 0.7, np.array([1, 1, 1]), chunk=3)
    np.testing.assert_allclose(o, v[:, :, 0], atol=1e-14)
    np.testing.assert_allclose(lse, 0.7 * np.einsum("bhd,bhd->bh", q, k[:, :, 0]), atol=1e-14)


def test_merge_associativity_and_order():
    rng = np.random.default_rng(13)
    o = rng.standard_normal((6, 5))
    lse = rng.standard_normal(6) * 4.0
    lse[2] = -np.inf
    whole_o, whole_l = oracle.merge_states(o, lse)
    a_o, a_l = oracle.merge_states(o[:4], lse[:4])
    b_o, b_l = oracle.merge_states(o[4:], lse[4:])
    two_o, two_l = oracle.merge_states(np.stack([a_o, b_o]), np.array([a_l, b_l]))
    np.testing.assert_allclose(two_o, whole_o, atol=1e-14)
    assert two_l == pytest.approx(whole_l, abs=1e-14)
    perm = rng.permutation(6)
    p_o, p_l = oracle.merge_states(o[perm], lse[perm])
    np.testing.assert_allclose(p_o, whole_o, atol=1e-14)
    assert p_l == pytest.approx(whole_l, abs=1e-14)


def test_merge_is_finite_at_large_lse():
    # parts with weights 1 : 3 at lse near 1000 (exp overflows without the max)
    o = np.array([[1.0, 0.0], [0.0, 1.0]])
    lse = np.array([1000.0, 1000.0 + math.log(3.0)])
    out, l = oracle.merge_states(o, lse)
    np.testing.assert_allclose(out, [0.25, 0.75], atol=1e-15)
    assert l == pytest.approx(1000.0 + math.log(4.0), abs=1e-12)


def test_merge_empty_parts():
    o = np.array([[5.0], [7.0], [9.0]])
    out, l = oracle.merge_states(o, np.array([-np.inf, 0.5, -np.inf]))
    assert out[0] == 7.0 and l == 0.5
    out, l = oracle.merge_states(o, np.array([-np.inf, -np.inf, -np.inf]))
    assert out[0] == 0.0 and np.isneginf(l)
