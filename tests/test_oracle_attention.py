"""Pins for the oracle's attention and the composed CSA / HCA / hybrid / prefill steps.

Witnesses: torch's scaled_dot_product_attention and scipy's logsumexp/softmax
(independent library routines), closed forms (constant keys, constant values),
invariants (rows sum to 1, permutation of the KV order), reductions between the
methods (CSA at ratio 1 with top-k = all is plain attention; CSA with top-k =
all equals HCA over the same cache), Python-loop brute force on tiny shapes and
the hand-worked cases in tests/golden/hand_worked.json."""
import json
import math
import os

import numpy as np
import pytest
import scipy.special
import torch

import oracle
from oracle.csa_hca import compress_to_cache, to_bf16_values
from workloads import bf16_normal, int8_uniform, rng

GOLDEN = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "hand_worked.json")))
SCALE = 1.0 / math.sqrt(128)


def _bf16(g, shape, std=1.0):
    return oracle.bf16_bits_to_f64(bf16_normal(g, shape, std))


@pytest.mark.parametrize("case", GOLDEN["attention"])
def test_golden_attention(case):
    o, lse, p = oracle.attention(np.array(case["q"], float), np.array(case["K"], float),
                                 np.array(case["V"], float), case["scale"])
    assert np.allclose(o, np.array(case["expect_o"]), rtol=0, atol=1e-15)
    assert np.allclose(lse, np.array(case["expect_lse"]), rtol=0, atol=1e-15)


def test_attention_matches_torch_sdpa():
    g = rng(910, 0, 0)
    q, K, V = _bf16(g, (16, 128)), _bf16(g, (300, 128)), _bf16(g, (300, 128))
    o, lse, p = oracle.attention(q, K, V, SCALE)
    ref = torch.nn.functional.scaled_dot_product_attention(
        torch.from_numpy(q)[None, :, None, :], torch.from_numpy(K)[None, None],
        torch.from_numpy(V)[None, None], scale=SCALE)[0, :, 0, :].numpy()
    assert np.allclose(o, ref, rtol=0, atol=1e-13)
    assert np.allclose(lse, scipy.special.logsumexp(SCALE * q @ K.T, axis=1), atol=1e-12)
    assert np.allclose(p, scipy.special.softmax(SCALE * q @ K.T, axis=1), atol=1e-15)


def test_attention_tiny_brute_force():
    q = [[0.5, -1.0], [2.0, 0.25]]
    K = [[1.0, 0.0], [0.0, 1.0], [-1.0, 1.0]]
    V = [[1.0, 2.0], [3.0, -1.0], [0.0, 0.5]]
    o, lse, _ = oracle.attention(np.array(q), np.array(K), np.array(V), 0.7)
    for h in range(2):
        ls = [0.7 * sum(q[h][d] * K[j][d] for d in range(2)) for j in range(3)]
        w = [math.exp(x) for x in ls]
        for d in range(2):
            assert abs(o[h, d] - sum(w[j] * V[j][d] for j in range(3)) / sum(w)) < 1e-15
        assert abs(lse[h] - math.log(sum(w))) < 1e-15


def test_rows_sum_to_one_and_peaky():
    g = rng(911, 0, 0)
    q, K, V = _bf16(g, (64, 128)) * 16, _bf16(g, (513, 128)), _bf16(g, (513, 128))
    o, lse, p = oracle.attention(q, K, V, SCALE)
    assert np.all(np.abs(p.sum(axis=1) - 1) < 1e-12)
    assert np.all(np.isfinite(o)) and np.all(np.isfinite(lse))
    assert np.allclose(p, scipy.special.softmax(SCALE * q @ K.T, axis=1), atol=1e-14)


def test_constant_keys_and_values():
    g = rng(912, 0, 0)
    q, V = _bf16(g, (8, 128)), _bf16(g, (40, 128))
    Kc = np.tile(_bf16(g, (1, 128)), (40, 1))
    o, _, p = oracle.attention(q, Kc, V, SCALE)
    assert np.allclose(p, 1 / 40, atol=1e-15)
    assert np.allclose(o, V.mean(axis=0)[None], atol=1e-14)
    Vc = np.tile(_bf16(g, (1, 128)), (40, 1))
    o, _, _ = oracle.attention(q, _bf16(g, (40, 128)), Vc, SCALE)
    assert np.allclose(o, Vc[:8], atol=1e-14)


def test_empty_attention():
    o, lse, p = oracle.attention(np.ones((4, 128)), np.zeros((0, 128)), np.zeros((0, 128)), SCALE)
    assert np.all(o == 0) and np.all(lse == -np.inf) and p.shape == (4, 0)


def test_kv_permutation_invariance():
    g = rng(913, 0, 0)
    q, K, V = _bf16(g, (16, 128)), _bf16(g, (200, 128)), _bf16(g, (200, 128))
    perm = np.random.default_rng(0).permutation(200)
    o1, l1, _ = oracle.attention(q, K, V, SCALE)
    o2, l2, _ = oracle.attention(q, K[perm], V[perm], SCALE)
    assert np.allclose(o1, o2, atol=1e-14) and np.allclose(l1, l2, atol=1e-13)


# ---------------------------------------------------------------- composed steps

def _csa_inputs(cfg, n, h=16, std=1.0):
    g = rng(cfg, 0, 0)
    return (_bf16(g, (h, 128)), int8_uniform(g, (64,)), _bf16(g, (n, 128), std),
            _bf16(g, (n, 128), std), int8_uniform(g, (n, 64)))


def test_csa_ratio1_topk_all_is_vanilla_attention():
    # c = 1 and top-k = all: every raw token is its own entry and all are attended
    g = rng(914, 0, 0)
    raw_k, raw_v = bf16_normal(g, (96, 128)), bf16_normal(g, (96, 128))
    q, qi, kidx = _bf16(g, (16, 128)), int8_uniform(g, (64,)), int8_uniform(g, (96, 64))
    Kc = oracle.bf16_bits_to_f64(compress_to_cache(oracle.bf16_bits_to_f64(raw_k), 1))
    Vc = oracle.bf16_bits_to_f64(compress_to_cache(oracle.bf16_bits_to_f64(raw_v), 1))
    r = oracle.csa_decode(q, qi, 96, Kc, Vc, kidx, 1, 96, SCALE)
    ref = torch.nn.functional.scaled_dot_product_attention(
        torch.from_numpy(q)[None, :, None, :],
        torch.from_numpy(oracle.bf16_bits_to_f64(raw_k))[None, None],
        torch.from_numpy(oracle.bf16_bits_to_f64(raw_v))[None, None], scale=SCALE)
    assert r["idx"].tolist() == list(range(96))
    assert np.allclose(r["o"], ref[0, :, 0, :].numpy(), atol=1e-13)


def test_csa_topk_all_equals_hca_dense():
    q, qi, K, V, kidx = _csa_inputs(915, 333, h=64)
    a = oracle.csa_decode(q, qi, 333 * 4 + 3, K, V, kidx, 4, 10 ** 6, SCALE)
    b = oracle.hca_decode(q, 333 * 4 + 3, K, V, 4, SCALE)
    assert a["n_vis"] == b["n_vis"] == 333
    assert np.allclose(a["o"], b["o"], atol=1e-14) and np.allclose(a["lse"], b["lse"], atol=1e-13)


def test_csa_attends_exactly_the_selected_entries():
    q, qi, K, V, kidx = _csa_inputs(916, 500)
    r = oracle.csa_decode(q, qi, 2000, K, V, kidx, 4, 37, SCALE)
    s = oracle.index_scores(qi, kidx)
    assert len(r["idx"]) == 37 and s[r["idx"]].min() >= np.delete(s, r["idx"]).max()
    o, _, _ = oracle.attention(q, K[r["idx"]], V[r["idx"]], SCALE)
    assert np.array_equal(o, r["o"])
    # a row that is not selected cannot change the output
    K2, V2 = K.copy(), V.copy()
    other = np.setdiff1d(np.arange(500), r["idx"])[:50]
    K2[other] = 100.0
    V2[other] = -100.0
    assert np.array_equal(oracle.csa_decode(q, qi, 2000, K2, V2, kidx, 4, 37, SCALE)["o"], r["o"])


def test_csa_permutation_of_entries():
    # permuting compressed entries together with their indexer keys permutes the
    # selection and leaves the output unchanged when no tie sits at the threshold
    q, qi, K, V, kidx = _csa_inputs(917, 400)
    s = oracle.index_scores(qi, kidx)
    k = 50
    thr = np.sort(s)[::-1][k - 1]
    assert np.sum(s == thr) == 1 and np.sort(s)[::-1][k] != thr  # tie-free at the threshold
    perm = np.random.default_rng(1).permutation(400)
    a = oracle.csa_decode(q, qi, 1600, K, V, kidx, 4, k, SCALE)
    b = oracle.csa_decode(q, qi, 1600, K[perm], V[perm], kidx[perm], 4, k, SCALE)
    assert sorted(perm[b["idx"]].tolist()) == a["idx"].tolist()
    assert np.allclose(a["o"], b["o"], atol=1e-14)


def test_hca_visibility_and_tail():
    q, _, K, V, _ = _csa_inputs(918, 10)
    r = oracle.hca_decode(q, 10 * 128 + 127, K, V, 128, SCALE)
    assert r["n_vis"] == 10
    r = oracle.hca_query(q, 5 * 128 + 127, K, V, 128, SCALE)   # a query inside block 5
    o, _, _ = oracle.attention(q, K[:5], V[:5], SCALE)
    assert r["n_vis"] == 5 and np.array_equal(r["o"], o)


def test_hybrid_interleaves_csa_and_hca():
    layers = []
    for li in range(4):
        q, qi, K, V, kidx = _csa_inputs(920 + li, 64)
        layers.append(dict(q=q, q_idx=qi, Kc=K, Vc=V, k_idx=kidx, c=4, topk=8, m=4))
    out = oracle.hybrid_decode(layers, 256, SCALE)
    for li, r in enumerate(out):
        L = layers[li]
        if li % 2 == 0:
            assert len(r["idx"]) == 8
            o, _, _ = oracle.attention(L["q"], L["Kc"][r["idx"]], L["Vc"][r["idx"]], SCALE)
        else:
            assert "idx" not in r
            o, _, _ = oracle.attention(L["q"], L["Kc"], L["Vc"], SCALE)
        assert np.array_equal(o, r["o"])


def test_prefill_block_causal_visibility():
    g = rng(921, 0, 0)
    ctx, new, c, h = 64, 32, 4, 16
    raw_k, raw_v = _bf16(g, (ctx + new, 128)), _bf16(g, (ctx + new, 128))
    Kc = to_bf16_values(oracle.kv_compress(raw_k[:ctx], c))
    Vc = to_bf16_values(oracle.kv_compress(raw_v[:ctx], c))
    n_tot = (ctx + new) // c
    kidx = int8_uniform(g, (n_tot, 64))
    q, qi = _bf16(g, (new, h, 128)), int8_uniform(g, (new, 64))
    nk, nv, res = oracle.csa_prefill(q, qi, ctx, Kc, Vc, raw_k[ctx:], raw_v[ctx:], kidx, c, 6,
                                     SCALE)
    assert np.array_equal(nk, compress_to_cache(raw_k, c)[ctx // c:])
    full_k = oracle.bf16_bits_to_f64(compress_to_cache(raw_k, c))
    full_v = oracle.bf16_bits_to_f64(compress_to_cache(raw_v, c))
    for i, r in res.items():
        pos = ctx + i
        vis = [j for j in range(n_tot) if j * c + c - 1 < pos]   # blocks ended before pos
        assert r["n_vis"] == len(vis)
        s = oracle.index_scores(qi[i], kidx)
        best = sorted(vis, key=lambda j: (-int(s[j]), j))[:6]
        assert r["idx"].tolist() == sorted(best)
        o, _, _ = oracle.attention(q[i], full_k[r["idx"]], full_v[r["idx"]], SCALE)
        assert np.array_equal(o, r["o"])
