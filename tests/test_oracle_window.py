"""Pins for the oracle's sliding-window branch (window tokens, one softmax over the
compressed entries and the window's raw tokens).

Witnesses: a set-based brute force of the window range, torch's
scaled_dot_product_attention over the concatenated keys, Python-loop sums on a tiny
case, the reduction to the compressed branch alone (empty window) and to the window
alone (no visible compressed entry), the log-sum-exp merge of two separately
computed branches, and invariance to the order of the window's tokens."""
import math

import numpy as np
import pytest
import torch

import oracle
from workloads import bf16_normal, int8_uniform, rng

SCALE = 1.0 / math.sqrt(128)


def _bf16(g, shape, std=1.0):
    return oracle.bf16_bits_to_f64(bf16_normal(g, shape, std))


def test_window_tokens_brute_force():
    for pos in range(0, 40):
        for w in (0, 1, 3, 8, 128):
            for pos0 in (0, 5, 17, 30):
                for n_buf in (0, 1, 6, 20):
                    want = [t - pos0 for t in range(pos0, pos0 + n_buf) if pos - w <= t < pos]
                    lo, hi = oracle.window_tokens(pos, w, pos0, n_buf)
                    assert list(range(lo, hi)) == want, (pos, w, pos0, n_buf)
                    assert 0 <= lo <= hi <= n_buf


def test_tiny_union_by_hand():
    q = [[1.0, -0.5]]
    K, V = [[0.5, 1.0]], [[2.0, 0.0]]
    Kw, Vw = [[1.0, 1.0], [-1.0, 0.0]], [[0.0, 1.0], [1.0, -1.0]]
    o, lse, p = oracle.attention_union(np.array(q), np.array(K), np.array(V), np.array(Kw),
                                       np.array(Vw), 0.5)
    keys, vals = K + Kw, V + Vw
    ls = [0.5 * (q[0][0] * k[0] + q[0][1] * k[1]) for k in keys]
    ws = [math.exp(x) for x in ls]
    for d in range(2):
        assert abs(o[0, d] - sum(wj * v[d] for wj, v in zip(ws, vals)) / sum(ws)) < 1e-15
    assert abs(lse[0] - math.log(sum(ws))) < 1e-15
    assert abs(p.sum() - 1.0) < 1e-15


def test_union_matches_torch_sdpa():
    g = rng(930, 0, 0)
    q, K, V = _bf16(g, (16, 128)), _bf16(g, (200, 128)), _bf16(g, (200, 128))
    Kw, Vw = _bf16(g, (128, 128)), _bf16(g, (128, 128))
    o, lse, _ = oracle.attention_union(q, K, V, Kw, Vw, SCALE)
    ref = torch.nn.functional.scaled_dot_product_attention(
        torch.from_numpy(q)[None, :, None, :], torch.from_numpy(np.concatenate([K, Kw]))[None, None],
        torch.from_numpy(np.concatenate([V, Vw]))[None, None], scale=SCALE)[0, :, 0, :].numpy()
    assert np.allclose(o, ref, rtol=0, atol=1e-13)


def test_lse_merge_of_separate_branches():
    """The union equals the two branches attended separately and merged by their
    log-sum-exp weights, which is how the GPU path combines them."""
    g = rng(931, 0, 0)
    q = _bf16(g, (8, 128), 4.0)
    K, V = _bf16(g, (50, 128)), _bf16(g, (50, 128))
    Kw, Vw = _bf16(g, (30, 128)), _bf16(g, (30, 128))
    o, lse, _ = oracle.attention_union(q, K, V, Kw, Vw, SCALE)
    o1, l1, _ = oracle.attention(q, K, V, SCALE)
    o2, l2, _ = oracle.attention(q, Kw, Vw, SCALE)
    m = np.maximum(l1, l2)
    a, b = np.exp(l1 - m), np.exp(l2 - m)
    merged = (a[:, None] * o1 + b[:, None] * o2) / (a + b)[:, None]
    assert np.allclose(o, merged, rtol=0, atol=1e-14)
    assert np.allclose(lse, m + np.log(a + b), rtol=0, atol=1e-13)


def test_empty_window_is_the_compressed_branch():
    g = rng(932, 0, 0)
    c, n, pos = 4, 300, 1203
    Kc, Vc = _bf16(g, (n, 128)), _bf16(g, (n, 128))
    kidx, q, qi = int8_uniform(g, (n, 64)), _bf16(g, (16, 128)), int8_uniform(g, (64,))
    Kw, Vw = _bf16(g, (128, 128)), _bf16(g, (128, 128))
    a = oracle.csa_query(q, qi, pos, Kc, Vc, kidx, c, 40, SCALE)
    b = oracle.csa_query_swa(q, qi, pos, Kc, Vc, kidx, c, 40, SCALE, Kw, Vw, pos - 128, 0)
    assert b["window"] == (128, 128) and np.array_equal(a["idx"], b["idx"])
    assert np.array_equal(a["o"], b["o"]) and np.array_equal(a["lse"], b["lse"])
    h1 = oracle.hca_query(q, pos, Kc, Vc, 4, SCALE)
    h2 = oracle.hca_query_swa(q, pos, Kc, Vc, 4, SCALE, Kw, Vw, 0, 0)
    assert np.array_equal(h1["o"], h2["o"])


def test_window_alone_before_the_first_block():
    """A query before the first complete block sees no compressed entry: only the
    window, i.e. plain attention over the tokens before it."""
    g = rng(933, 0, 0)
    raw_k, raw_v = _bf16(g, (3, 128)), _bf16(g, (3, 128))
    q = _bf16(g, (16, 128))
    Kc, Vc = np.zeros((0, 128)), np.zeros((0, 128))
    r = oracle.hca_query_swa(q, 3, Kc, Vc, 128, SCALE, raw_k, raw_v, 0, 128)
    assert r["n_vis"] == 0 and r["window"] == (0, 3)
    o, lse, _ = oracle.attention(q, raw_k, raw_v, SCALE)
    assert np.array_equal(r["o"], o) and np.array_equal(r["lse"], lse)


def test_window_order_does_not_matter():
    g = rng(934, 0, 0)
    q = _bf16(g, (16, 128), 4.0)
    K, V = _bf16(g, (20, 128)), _bf16(g, (20, 128))
    Kw, Vw = _bf16(g, (64, 128)), _bf16(g, (64, 128))
    perm = g.permutation(64)
    a = oracle.attention_union(q, K, V, Kw, Vw, SCALE)
    b = oracle.attention_union(q, K, V, Kw[perm], Vw[perm], SCALE)
    assert np.allclose(a[0], b[0], rtol=0, atol=1e-14)


@pytest.mark.parametrize("pos", [5, 130, 4096 + 77])
def test_csa_swa_is_attention_over_selected_plus_window(pos):
    """The CSA window query attends exactly the selected entries and the window's
    tokens: the same as attention over those rows gathered by hand."""
    g = rng(935, pos, 0)
    c, N = 4, 1100
    Kc, Vc = _bf16(g, (N, 128)), _bf16(g, (N, 128))
    kidx, q, qi = int8_uniform(g, (N, 64)), _bf16(g, (16, 128)), int8_uniform(g, (64,))
    pos0 = max(0, pos - 160)
    Kw, Vw = _bf16(g, (160, 128)), _bf16(g, (160, 128))
    r = oracle.csa_query_swa(q, qi, pos, Kc, Vc, kidx, c, 64, SCALE, Kw, Vw, pos0, 128)
    lo, hi = r["window"]
    want = [t - pos0 for t in range(pos0, pos0 + 160) if pos - 128 <= t < pos]
    assert list(range(lo, hi)) == want
    o, lse, _ = oracle.attention(q, np.concatenate([Kc[r["idx"]], Kw[lo:hi]]),
                                 np.concatenate([Vc[r["idx"]], Vw[lo:hi]]), SCALE)
    assert np.array_equal(r["o"], o)
