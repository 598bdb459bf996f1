"""csa_index_select_noalloc (the library's own per-device scratch as the workspace)
against csa_index_select with a caller workspace: bit-exact idx, count and n_vis, on
calls in a row, the second with a smaller batch, fewer entries and a smaller k, so that
whatever the first call left in the scratch must not reach the second's result, and a
third in the prefill form (16 or more query rows per sequence, no workspace)."""
import numpy as np
import pytest
import torch

import long_context_attention_19_amd as lca
from gpu_util import DEV, i64_dev, i8_dev, offsets, step
from workloads import int8_uniform, rng

pytestmark = pytest.mark.gpu


def _case(g, Ns, nq, c):
    kk = int8_uniform(g, (max(sum(Ns), 1), 64))
    qq = int8_uniform(g, (sum(nq), 64))
    q_pos = []
    for b, n in enumerate(Ns):
        for i in range(nq[b]):
            q_pos.append(n * c + 1 if i == 0 else int(g.integers(0, n * c + 3)))
    return kk, qq, q_pos


def _outputs(rows, k):
    return (torch.full((max(rows, 1), k), -5, dtype=torch.int32, device=DEV),
            torch.full((max(rows, 1),), -5, dtype=torch.int32, device=DEV),
            torch.full((max(rows, 1),), -5, dtype=torch.int32, device=DEV))


def test_noalloc_matches_workspace_form():
    g = rng(700, 0, 0)
    c = 4
    calls = [([120000, 70001, 0, 5000, 2049, 300000], [2, 1, 1, 3, 1, 2], 2048),
             ([9000, 2100], [1, 1], 256),
             ([30000, 7000], [20, 33], 512)]   # the prefill form (16 or more query rows)
    for n_call, (Ns, nq, k) in enumerate(calls):
        kk, qq, q_pos = _case(g, Ns, nq, c)
        B, max_q, max_n = len(Ns), max(nq), max(max(Ns), 1)
        ent_off, q_off = offsets(Ns), offsets(nq)
        rows = int(q_off[-1])
        kd, qd = i8_dev(kk), i8_dev(qq)
        qo, qp, eo = i64_dev(q_off), i64_dev(q_pos), i64_dev(ent_off)
        ws = lca.workspace(lca.csa_index_select_workspace_bytes(B, max_q, max_n, k))
        assert lca.csa_index_select_workspace_bytes(B, max_q, max_n, k) <= 8 << 20
        ref = _outputs(rows, k)
        step(f"csa_index_select (workspace) call={n_call} B={B} max_q={max_q} k={k}")
        lca.csa_index_select(qd, qo, qp, kd, eo, B, max_q, max_n, c, k, *ref, ws=ws)
        torch.cuda.synchronize()
        got = _outputs(rows, k)
        step(f"csa_index_select_noalloc call={n_call} B={B} max_q={max_q} k={k}")
        lca.csa_index_select_noalloc(qd, qo, qp, kd, eo, B, max_q, max_n, c, k, *got)
        torch.cuda.synchronize()
        for name, a, b in zip(("idx", "count", "n_vis"), ref, got):
            a, b = a.cpu().numpy(), b.cpu().numpy()
            assert np.array_equal(a[:rows], b[:rows]), (n_call, name)
        cnt = got[1].cpu().numpy()[:rows]
        assert np.all(cnt >= 0) and np.all(cnt <= k), n_call
        # n_vis NULL: the scratch holds it; idx and count unchanged
        got2 = _outputs(rows, k)
        step(f"csa_index_select_noalloc n_vis=NULL call={n_call}")
        lca.csa_index_select_noalloc(qd, qo, qp, kd, eo, B, max_q, max_n, c, k, got2[0], got2[1])
        torch.cuda.synchronize()
        assert torch.equal(got2[0][:rows].cpu(), ref[0][:rows].cpu()), n_call
        assert torch.equal(got2[1][:rows].cpu(), ref[1][:rows].cpu()), n_call


def test_noalloc_rejects_a_batch_beyond_the_scratch():
    g = rng(700, 1, 0)
    kd = i8_dev(int8_uniform(g, (64, 64)))
    qd = i8_dev(int8_uniform(g, (27, 64)))
    qo, qp = i64_dev(np.arange(28)), i64_dev(np.full(27, 4 << 22))
    eo = i64_dev(np.zeros(28, np.int64))
    idx, cnt, nv = _outputs(27, 2048)
    with pytest.raises(lca.LcaError, match="scratch"):
        lca.csa_index_select_noalloc(qd, qo, qp, kd, eo, 27, 1, 1 << 22, 4, 2048, idx, cnt, nv)
    assert int(cnt[0]) == -5        # rejected before anything ran
