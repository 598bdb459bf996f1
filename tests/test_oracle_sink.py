"""Pins for the oracle's attention sink (one extra logit per head in the softmax
normalisation, with a zero value row).

Witnesses: Python-loop sums on a tiny case, torch's scaled_dot_product_attention
with the sink built as a real key (logit z, value 0), the closed form for equal
logits, the reduction to plain attention for a sink of -inf, the logistic fold of a
sink into a finished result (how the GPU path applies it), the limits of a huge sink
and of no entries, and the composed CSA / HCA queries with the window branch."""
import math

import numpy as np
import pytest
import torch

import oracle
from workloads import bf16_normal, int8_uniform, rng

SCALE = 1.0 / math.sqrt(128)


def _bf16(g, shape, std=1.0):
    return oracle.bf16_bits_to_f64(bf16_normal(g, shape, std))


def test_tiny_by_hand():
    q = [[1.0, -0.5], [0.25, 2.0]]
    K, V = [[0.5, 1.0], [-1.0, 0.5]], [[2.0, 0.0], [1.0, -1.0]]
    z = [0.3, -1.7]
    o, lse, p = oracle.attention_sink(np.array(q), np.array(K), np.array(V), 0.5, np.array(z))
    for h in range(2):
        ls = [0.5 * (q[h][0] * k[0] + q[h][1] * k[1]) for k in K]
        den = math.exp(z[h]) + sum(math.exp(x) for x in ls)
        for d in range(2):
            want = sum(math.exp(x) * v[d] for x, v in zip(ls, V)) / den
            assert abs(o[h, d] - want) < 1e-15
        assert abs(lse[h] - math.log(den)) < 1e-15
        assert abs(p[h].sum() - (1 - math.exp(z[h]) / den)) < 1e-15


def test_matches_torch_sdpa_with_a_sink_key():
    g = rng(940, 0, 0)
    H, n = 16, 300
    q, K, V = _bf16(g, (H, 128)), _bf16(g, (n, 128)), _bf16(g, (n, 128))
    z = g.standard_normal(H) * 3.0
    o, lse, _ = oracle.attention_sink(q, K, V, SCALE, z)
    for h in range(H):
        ks = (z[h] / SCALE) * q[h] / (q[h] @ q[h])       # scale * q_h . ks = z_h
        K2 = torch.from_numpy(np.concatenate([K, ks[None]]))
        V2 = torch.from_numpy(np.concatenate([V, np.zeros((1, 128))]))
        ref = torch.nn.functional.scaled_dot_product_attention(
            torch.from_numpy(q[h])[None, None, None], K2[None, None], V2[None, None],
            scale=SCALE)[0, 0, 0].numpy()
        assert np.allclose(o[h], ref, rtol=0, atol=1e-13)
        lg = SCALE * (K2.numpy() @ q[h])
        assert abs(lse[h] - np.logaddexp.reduce(lg)) < 1e-12


def test_equal_logits_closed_form():
    g = rng(941, 0, 0)
    n, H = 37, 4
    q, V = _bf16(g, (H, 128)), _bf16(g, (n, 128))
    z = np.array([-2.0, 0.0, 1.5, 4.0])
    o, lse, _ = oracle.attention_sink(q, np.zeros((n, 128)), V, SCALE, z)   # every logit 0
    for h in range(H):
        assert np.allclose(o[h], n / (n + math.exp(z[h])) * V.mean(axis=0), rtol=0, atol=1e-14)
        assert abs(lse[h] - math.log(n + math.exp(z[h]))) < 1e-14


def test_minus_infinity_sink_is_plain_attention():
    g = rng(942, 0, 0)
    q, K, V = _bf16(g, (16, 128), 4.0), _bf16(g, (200, 128)), _bf16(g, (200, 128))
    o, lse, p = oracle.attention_sink(q, K, V, SCALE, np.full(16, -np.inf))
    o2, lse2, p2 = oracle.attention(q, K, V, SCALE)
    assert np.allclose(o, o2, rtol=0, atol=1e-15) and np.allclose(lse, lse2, rtol=0, atol=1e-15)
    assert np.allclose(p, p2, rtol=0, atol=1e-15)


def test_fold_into_a_finished_result():
    """The sink applied after the fact: o * sigmoid(lse - z), lse -> logaddexp(lse, z)."""
    g = rng(943, 0, 0)
    q, K, V = _bf16(g, (64, 128), 2.0), _bf16(g, (500, 128)), _bf16(g, (500, 128))
    z = g.standard_normal(64) * 4.0
    o, lse, _ = oracle.attention_sink(q, K, V, SCALE, z)
    o0, lse0, _ = oracle.attention(q, K, V, SCALE)
    f = 1.0 / (1.0 + np.exp(z - lse0))
    assert np.allclose(o, o0 * f[:, None], rtol=0, atol=1e-14)
    assert np.allclose(lse, np.logaddexp(lse0, z), rtol=0, atol=1e-13)


def test_limits():
    g = rng(944, 0, 0)
    q, K, V = _bf16(g, (8, 128)), _bf16(g, (50, 128)), _bf16(g, (50, 128))
    _, lse0, _ = oracle.attention(q, K, V, SCALE)
    o, lse, p = oracle.attention_sink(q, K, V, SCALE, lse0 + 50.0)   # the sink takes ~all weight
    assert np.abs(o).max() <= math.exp(-49.0) * np.abs(V).max()
    assert np.allclose(lse, lse0 + 50.0, rtol=0, atol=1e-12)
    # no entries: o = 0, lse = the sink (or -inf without one)
    o, lse, p = oracle.attention_sink(q, np.zeros((0, 128)), np.zeros((0, 128)), SCALE,
                                      np.array([0.5, -np.inf] * 4))
    assert np.array_equal(o, np.zeros((8, 128))) and p.shape == (8, 0)
    assert np.array_equal(lse, np.array([0.5, -np.inf] * 4))


@pytest.mark.parametrize("pos", [3, 4096 + 77])
def test_composed_queries(pos):
    g = rng(945, pos, 0)
    c, N, H = 4, 1100, 16
    Kc, Vc = _bf16(g, (N, 128)), _bf16(g, (N, 128))
    kidx, q, qi = int8_uniform(g, (N, 64)), _bf16(g, (H, 128)), int8_uniform(g, (64,))
    pos0 = max(0, pos - 150)
    Kw, Vw = _bf16(g, (150, 128)), _bf16(g, (150, 128))
    z = g.standard_normal(H)
    r = oracle.csa_query_sink(q, qi, pos, Kc, Vc, kidx, c, 64, SCALE, z, Kw, Vw, pos0, 128)
    lo, hi = r["window"]
    o, lse, _ = oracle.attention_sink(q, np.concatenate([Kc[r["idx"]], Kw[lo:hi]]),
                                      np.concatenate([Vc[r["idx"]], Vw[lo:hi]]), SCALE, z)
    assert np.array_equal(r["o"], o) and np.array_equal(r["lse"], lse)
    # a sink of -inf and no window: the plain queries
    a = oracle.csa_query(q, qi, pos, Kc, Vc, kidx, c, 64, SCALE)
    b = oracle.csa_query_sink(q, qi, pos, Kc, Vc, kidx, c, 64, SCALE, np.full(H, -np.inf))
    assert np.array_equal(a["idx"], b["idx"]) and np.allclose(a["o"], b["o"], rtol=0, atol=1e-15)
    h1 = oracle.hca_query_swa(q, pos, Kc, Vc, 4, SCALE, Kw, Vw, pos0, 128)
    h2 = oracle.hca_query_sink(q, pos, Kc, Vc, 4, SCALE, np.full(H, -np.inf), Kw, Vw, pos0, 128)
    assert np.allclose(h1["o"], h2["o"], rtol=0, atol=1e-15)
    assert np.allclose(h1["lse"], h2["lse"], rtol=0, atol=1e-15)
