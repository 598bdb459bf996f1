"""Pins for the oracle's FP4 indexer (E2M1 codes, packed two per byte, scores as
exact integers J = 256 * sum q k).

Witnesses: the E2M1 value table of the OCP Microscaling specification, a hand-packed
byte, a packer written here, Python-integer brute force, the exactly pinned int8
scorer applied to the doubled values, the score bound reached by its extreme codes,
and the composed query against the int8 path's selection rule."""
import numpy as np
import pytest

import oracle
from workloads import bf16_normal, fp4_uniform, rng

# E2M1 element values, codes 0..15 (OCP Microscaling Formats v1.0, FP4 E2M1 table)
E2M1_TABLE = [0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0,
              -0.0, -0.5, -1.0, -1.5, -2.0, -3.0, -4.0, -6.0]


def test_value_table():
    v = oracle.fp4_values(np.arange(16))
    assert list(v) == E2M1_TABLE
    assert np.signbit(v[8])                       # code 8 is negative zero
    assert np.all(oracle.fp4_values(np.arange(16) + 16) == v)   # only the low 4 bits count


def test_unpack_nibble_order():
    assert list(oracle.fp4_unpack(np.array([0x21], np.uint8))) == [1, 2]
    assert list(oracle.fp4_unpack(np.array([[0xF0, 0x0F]], np.uint8))[0]) == [0, 15, 15, 0]
    g = rng(950, 0, 0)
    codes = g.integers(0, 16, size=(5, 64))
    packed = (codes[:, 0::2] | (codes[:, 1::2] << 4)).astype(np.uint8)
    assert np.array_equal(oracle.fp4_unpack(packed), codes)


def _py_score(qb, kb):
    """Python integers: (2q)(2k) summed; 2 * an E2M1 value is an integer."""
    twice = [0, 1, 2, 3, 4, 6, 8, 12]
    def val2(c):
        return -twice[c & 7] if c & 8 else twice[c & 7]
    tot = 0
    for i in range(len(qb)):
        for sh in (0, 4):
            tot += val2((int(qb[i]) >> sh) & 15) * val2((int(kb[i]) >> sh) & 15)
    return tot


def test_scores_brute_force():
    g = rng(951, 0, 0)
    q, k = fp4_uniform(g, (32,)), fp4_uniform(g, (200, 32))
    s = oracle.index_scores_fp4(q, k)
    assert s.dtype == np.int64
    assert [int(x) for x in s] == [64 * _py_score(q, k[j]) for j in range(200)]


def test_scores_equal_int8_scorer_on_doubled_values():
    g = rng(952, 0, 0)
    q, k = fp4_uniform(g, (32,)), fp4_uniform(g, (1000, 32))
    q2 = (2 * oracle.fp4_values(oracle.fp4_unpack(q))).astype(np.int8)
    k2 = (2 * oracle.fp4_values(oracle.fp4_unpack(k))).astype(np.int8)
    assert np.array_equal(oracle.index_scores_fp4(q, k), 64 * oracle.index_scores(q2, k2))


def test_score_bound_and_zero():
    six, msix = 0x77, 0xFF                       # both nibbles +6, both -6
    q = np.full(32, six, np.uint8)
    assert oracle.index_scores_fp4(q, np.full((1, 32), six, np.uint8))[0] == 589824
    assert oracle.index_scores_fp4(q, np.full((1, 32), msix, np.uint8))[0] == -589824
    assert oracle.index_scores_fp4(q, np.full((1, 32), 0x88, np.uint8))[0] == 0   # -0 codes
    g = rng(953, 0, 0)
    s = oracle.index_scores_fp4(fp4_uniform(g, (32,)), fp4_uniform(g, (5000, 32)))
    assert np.abs(s).max() <= 589824 < (1 << 20) and np.all(s % 64 == 0)


@pytest.mark.parametrize("pos", [7, 3000])
def test_composed_query(pos):
    g = rng(954, pos, 0)
    N, H, c, k = 900, 16, 4, 100
    Kc = oracle.bf16_bits_to_f64(bf16_normal(g, (N, 128)))
    Vc = oracle.bf16_bits_to_f64(bf16_normal(g, (N, 128)))
    q = oracle.bf16_bits_to_f64(bf16_normal(g, (H, 128)))
    qf, kf = fp4_uniform(g, (32,)), fp4_uniform(g, (N, 32))
    r = oracle.csa_query_fp4(q, qf, pos, Kc, Vc, kf, c, k, 0.0884)
    n_vis = min(pos // c, N)
    s = oracle.index_scores_fp4(qf, kf)[:n_vis]
    want = sorted(sorted(range(n_vis), key=lambda j: (-int(s[j]), j))[:k])
    assert list(r["idx"]) == want and r["n_vis"] == n_vis
    o, lse, _ = oracle.attention(q, Kc[want], Vc[want], 0.0884)
    assert np.array_equal(r["o"], o)
