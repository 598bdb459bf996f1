"""Pins for compression, visibility, indexer scores and top-k selection.

Each oracle function is checked against something other than itself: exact
rational arithmetic, Python-integer brute force, brute-force enumeration of
blocks, a sort under an explicit key, and the hand-worked cases in
tests/golden/hand_worked.json."""
import json
import os
from fractions import Fraction

import numpy as np
import pytest
from hypothesis import given, settings, strategies as st

import oracle
from oracle.csa_hca import compress_to_cache
from workloads import bf16_normal, int8_uniform, rng

GOLDEN = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "hand_worked.json")))


# ---------------------------------------------------------------- golden (hand-worked)

@pytest.mark.parametrize("case", GOLDEN["kv_compress"])
def test_golden_compress(case):
    got = oracle.kv_compress(np.array(case["x"], float), case["c"])
    assert np.array_equal(got, np.array(case["expect"], float).reshape(got.shape))


@pytest.mark.parametrize("case", GOLDEN["index_scores"])
def test_golden_scores(case):
    got = oracle.index_scores(np.array(case["q"], np.int8), np.array(case["k"], np.int8))
    assert got.tolist() == case["expect"]


@pytest.mark.parametrize("case", GOLDEN["n_visible"])
def test_golden_visibility(case):
    got = [oracle.n_visible(p, case["c"], case["n_entries"]) for p in case["pos"]]
    assert got == case["expect"]


@pytest.mark.parametrize("case", GOLDEN["topk_select"])
def test_golden_topk(case):
    got = oracle.topk_select(np.array(case["scores"]), case["n_vis"], case["k"])
    assert got.tolist() == case["expect"]


# ---------------------------------------------------------------- compression

def test_compress_exact_rational_mean():
    g = rng(900, 0, 0)
    for c in (1, 2, 3, 4, 7, 8):
        bits = bf16_normal(g, (5 * c + c - 1, 6))
        x = oracle.bf16_bits_to_f64(bits)
        got = oracle.kv_compress(x, c)
        assert got.shape == (5, 6)
        for j in range(5):
            for d in range(6):
                exact = sum(Fraction(float(v)) for v in x[j * c:(j + 1) * c, d]) / c
                assert got[j, d] == float(exact)  # correctly rounded mean


def test_compress_identity_constant_tail():
    x = np.arange(40, dtype=float).reshape(10, 4)
    assert np.array_equal(oracle.kv_compress(x, 1), x)
    const = np.full((128 * 3 + 5, 8), -1.375)
    y = oracle.kv_compress(const, 128)
    assert y.shape == (3, 8) and np.all(y == -1.375)
    # tail rows never leak into an entry
    x2 = x.copy()
    x2[8:] = 1e9
    assert np.array_equal(oracle.kv_compress(x2, 4), oracle.kv_compress(x, 4))


def test_compress_linear():
    g = np.random.default_rng(1)
    a, b = g.standard_normal((64, 16)), g.standard_normal((64, 16))
    lhs = oracle.kv_compress(2.0 * a + b, 4)
    rhs = 2.0 * oracle.kv_compress(a, 4) + oracle.kv_compress(b, 4)
    assert np.allclose(lhs, rhs, rtol=0, atol=1e-14)


def test_compress_concatenation():
    # compressing context and appended tokens separately equals compressing the whole
    # sequence when the context length is a multiple of c (prefill append)
    g = rng(901, 0, 0)
    x = oracle.bf16_bits_to_f64(bf16_normal(g, (64, 8)))
    whole = compress_to_cache(x, 4)
    parts = np.concatenate([compress_to_cache(x[:40], 4), compress_to_cache(x[40:], 4)])
    assert np.array_equal(whole, parts)


# ---------------------------------------------------------------- visibility

@pytest.mark.parametrize("c", [1, 2, 4, 5, 128])
def test_visibility_brute_force(c):
    n_entries = 9
    for pos in range(0, c * 12):
        ends = [j * c + c - 1 for j in range(n_entries)]
        brute = sum(1 for e in ends if e < pos)
        assert oracle.n_visible(pos, c, n_entries) == brute


def test_visibility_prefill_shape():
    # 4096 queries after 262144 context tokens, c = 4: entry 66559 is never visible
    nv = [oracle.n_visible(262144 + i, 4, 66560) for i in range(4096)]
    assert nv[0] == 65536 and nv[3] == 65536 and nv[4] == 65537 and max(nv) == 66559


# ---------------------------------------------------------------- indexer scores

def test_scores_python_int_brute_force():
    g = rng(902, 0, 0)
    q = int8_uniform(g, (64,))
    k = int8_uniform(g, (50, 64))
    got = oracle.index_scores(q, k)
    for j in range(50):
        assert got[j] == sum(int(a) * int(b) for a, b in zip(q.tolist(), k[j].tolist()))


def test_scores_match_float64_blas():
    # fp64 products and sums of int8 values are exact below 2^53
    g = rng(903, 0, 0)
    q = int8_uniform(g, (64,))
    k = int8_uniform(g, (4096, 64))
    ref = k.astype(np.float64) @ q.astype(np.float64)
    assert np.array_equal(oracle.index_scores(q, k), ref.astype(np.int64))
    assert np.abs(ref).max() <= 64 * 127 * 127


# ---------------------------------------------------------------- top-k

def _brute_topk(s, n_vis, k):
    order = sorted(range(n_vis), key=lambda j: (-int(s[j]), j))
    return sorted(order[:k])


@settings(max_examples=300, deadline=None)
@given(st.lists(st.integers(-6, 6), min_size=0, max_size=40), st.integers(0, 45),
       st.integers(1, 45))
def test_topk_brute_force(scores, n_vis, k):
    s = np.array(scores, dtype=np.int64)
    n_vis = min(n_vis, len(scores))
    assert oracle.topk_select(s, n_vis, k).tolist() == _brute_topk(s, n_vis, k)


def test_topk_all_equal_and_k_ge_n():
    s = np.full(100, 42)
    assert oracle.topk_select(s, 100, 7).tolist() == list(range(7))
    s = np.arange(30)[::-1]
    assert oracle.topk_select(s, 20, 50).tolist() == list(range(20))
    assert oracle.topk_select(s, 0, 5).tolist() == []


def test_topk_masked_entries_never_selected():
    s = np.array([1, 2, 3, 1000, 1000])
    assert oracle.topk_select(s, 3, 2).tolist() == [1, 2]


def test_topk_threshold_tie():
    # 3 entries above the threshold, 4 tied at it, k = 5: the two lowest tied indices win
    s = np.array([0, 5, 9, 5, 9, 5, 9, 5, 1])
    assert oracle.topk_select(s, 9, 5).tolist() == [1, 2, 3, 4, 6]


def test_topk_selects_largest_scores():
    g = rng(904, 0, 0)
    s = oracle.index_scores(int8_uniform(g, (64,)), int8_uniform(g, (5000, 64)))
    sel = oracle.topk_select(s, 5000, 300)
    rest = np.setdiff1d(np.arange(5000), sel)
    assert len(sel) == 300 and np.all(np.diff(sel) > 0)
    assert s[sel].min() >= s[rest].max()


def test_scores_extreme_int8_codes():
    """The int8 type's whole range, -128 included: a query and a key of all -128 reach
    64 * 2^14 = 2^20 exactly (Python integers); no other pair reaches it, the next
    reachable score being 63 * 2^14 + 128 * 127 = 2^20 - 128; the lowest is
    64 * (-128) * 127."""
    q = np.full(64, -128, np.int8)
    keys = np.full((4, 64), -128, np.int8)
    keys[1, 0] = -127                      # one product 128 * 127
    keys[2] = 127                          # the lowest score
    keys[3, :32] = 127                     # half and half: -2^13 * 128 + ...
    want = [sum(int(a) * int(b) for a, b in zip(q, k)) for k in keys]
    assert want[0] == 1 << 20 and want[1] == (1 << 20) - 128 and want[2] == -64 * 128 * 127
    assert oracle.index_scores(q, keys).tolist() == want
    # the two top scores keep their order in the selection (ties by index otherwise)
    assert oracle.topk_select(oracle.index_scores(q, keys), 4, 1).tolist() == [0]
    assert oracle.topk_select(oracle.index_scores(q, keys[1:]), 3, 1).tolist() == [0]


# ---------------------------------------------------------------- many-row forms

def test_scores_rows_equal_per_row_scores():
    """The fp64-product form gives index_scores' exact integers row by row, including
    the extreme codes (a query and keys of all -128 reach 2^20)."""
    g = rng(700, 0, 0)
    K = int8_uniform(g, (3000, 64))
    Q = int8_uniform(g, (37, 64))
    K[::50] = -128
    K[1::50] = 127
    Q[0] = -128
    Q[1] = 127
    S = oracle.index_scores_rows(Q, K)
    assert S.dtype == np.int64 and S.shape == (37, 3000)
    for r in range(37):
        assert np.array_equal(S[r], oracle.index_scores(Q[r], K)), r
    assert S[0, 0] == 1 << 20


def test_scores_fp4_rows_equal_per_row_scores():
    g = rng(700, 1, 0)
    K = g.integers(0, 256, (2000, 32)).astype(np.uint8)
    Q = g.integers(0, 256, (23, 32)).astype(np.uint8)
    K[0] = 0x77          # +6 in both nibbles
    Q[0] = 0x77
    S = oracle.index_scores_fp4_rows(Q, K)
    for r in range(23):
        assert np.array_equal(S[r], oracle.index_scores_fp4(Q[r], K)), r
    assert S[0, 0] == 64 * 36 * 256


@pytest.mark.parametrize("spread", [3, 200, 1 << 20])
def test_topk_rows_equal_per_row_selection(spread):
    """Row by row the same selection as topk_select, with heavy ties (spread 3), n_vis
    of 0, below k, exactly k, between k and n, and n, and k above n."""
    g = rng(701, spread % 97, 0)
    n, k = 700, 64
    S = g.integers(-spread, spread + 1, (40, n))
    nv = np.array([0, 1, k - 1, k, k + 1, n - 1, n] + list(g.integers(0, n + 1, 33)))
    for kk in (k, 1, n + 5):
        T = oracle.topk_select_rows(S, nv, kk)
        assert T.shape == (40, kk)
        for r in range(40):
            ref = oracle.topk_select(S[r], int(nv[r]), kk)
            assert np.array_equal(T[r, :len(ref)], ref), (kk, r)
            assert np.all(T[r, len(ref):] == -1), (kk, r)
