"""Batch invariance of the hybrid step: a sequence's outputs (attention out and lse of
every layer, the CSA layers' selected indices) are bit-identical whether it runs alone,
inside a few sequences, or inside the 16-sequence batch, and a repeated step gives the
same bits.  The stack is 8 layers (4 CSA c=4 top-k 2048, 4 HCA m=128, interleaved) over
ragged contexts of 65,536..1,048,576 tokens, 64 heads: the decode stack at full size,
with bf16 cache rows and int8 indexer codes, with FP4 indexer codes, and with mixed
FP8 / bf16 cache rows.  Inputs are drawn on the GPU from seeded generators; no oracle is
involved (the parity of these kernels against the oracle is covered elsewhere)."""
import numpy as np
import pytest
import torch

import long_context_attention_19_amd as lca
from gpu_util import DEV, i64_dev, offsets, step
from long_context_attention_19_amd.pipeline import HybridStep
from workloads import gen
from workloads.gen import device_fp4_uniform, device_kv8_normal

pytestmark = pytest.mark.gpu

HEADS, SCALE = 64, 128 ** -0.5


def _stack(L, fmt):
    """Per layer: kind, ratio, entry counts and device tensors for the whole batch."""
    tg = torch.Generator(device=DEV)
    tg.manual_seed(9100)
    B = len(L)
    layers = []
    for li in range(8):
        csa = li % 2 == 0
        ratio = 4 if csa else 128
        Ns = [int(x) // ratio for x in L]
        tot = sum(Ns)
        if fmt == "kv8":   # mixed rows: dims 0..63 FP8 E4M3, 64..127 bf16
            k = device_kv8_normal(tot, 9200 + 2 * li, ratio ** -0.5, DEV)
            v = device_kv8_normal(tot, 9201 + 2 * li, ratio ** -0.5, DEV)
        else:
            k = torch.randn(tot, 128, generator=tg, device=DEV).mul_(ratio ** -0.5).bfloat16()
            v = torch.randn(tot, 128, generator=tg, device=DEV).mul_(ratio ** -0.5).bfloat16()
        d = dict(csa=csa, ratio=ratio, Ns=Ns, k=k, v=v,
                 q=torch.randn(B, HEADS, 128, generator=tg, device=DEV).bfloat16())
        if csa and fmt == "fp4":   # packed E2M1 codes, 32 bytes per vector
            d["k_idx"] = device_fp4_uniform((tot, 32), 9300 + li, DEV)
            d["q_idx"] = device_fp4_uniform((B, 32), 9400 + li, DEV)
        elif csa:
            d["k_idx"] = torch.randint(-127, 128, (tot, 64), generator=tg, device=DEV,
                                       dtype=torch.int8)
            d["q_idx"] = torch.randint(-127, 128, (B, 64), generator=tg, device=DEV,
                                       dtype=torch.int8)
        layers.append(d)
    return layers


def _run(stack, L, seqs, fmt):
    """The hybrid step over the sequences `seqs` of the stack; returns per layer
    (out, lse, idx, count) on the host."""
    B = len(seqs)
    specs = []
    for d in stack:
        off = offsets(d["Ns"])
        Ns = [d["Ns"][j] for j in seqs]
        # the chosen sequences' rows, packed in order (a contiguous slice when alone)
        if B == 1:
            j = seqs[0]
            sl = slice(int(off[j]), int(off[j + 1]))
            k, v = d["k"][sl], d["v"][sl]
            ki = d["k_idx"][sl] if d["csa"] else None
        else:
            parts = [slice(int(off[j]), int(off[j + 1])) for j in seqs]
            k = torch.cat([d["k"][s] for s in parts])
            v = torch.cat([d["v"][s] for s in parts])
            ki = torch.cat([d["k_idx"][s] for s in parts]) if d["csa"] else None
        s = dict(kind=lca.LCA_LAYER_CSA if d["csa"] else lca.LCA_LAYER_HCA, ratio=d["ratio"],
                 max_entries=max(max(Ns), 1), q=d["q"][seqs].contiguous(), k_cmp=k, v_cmp=v,
                 ent_off=i64_dev(offsets(Ns)),
                 out=torch.empty(B, HEADS, 128, dtype=torch.bfloat16, device=DEV),
                 lse=torch.empty(B, HEADS, dtype=torch.float32, device=DEV))
        if d["csa"]:
            s.update(topk=2048, k_idx=ki, q_idx=d["q_idx"][seqs].contiguous())
            if fmt == "fp4":
                s["idx_format"] = lca.LCA_IDX_FP4
        if fmt == "kv8":
            s["kv_format"] = lca.LCA_KV_MIXED
        specs.append(s)
    hs = HybridStep(specs, B, 1, HEADS)
    hs.run(i64_dev(np.arange(B + 1)), i64_dev([L[j] for j in seqs]), SCALE)
    torch.cuda.synchronize()
    res = []
    for Ld in hs.layers:
        res.append((Ld["out"].view(torch.int16).cpu().numpy(), Ld["lse"].cpu().numpy(),
                    Ld["idx"].cpu().numpy() if "idx" in Ld else None,
                    Ld["count"].cpu().numpy() if "count" in Ld else None))
    return res


@pytest.mark.parametrize("fmt", ["bf16_int8", "fp4", "kv8"])
def test_hybrid_step_batch_invariant(fmt):
    L = gen.ragged_lengths(gen.rng(3, 0, gen.T_LEN), 16, 65536, 1048576)
    step(f"batch invariance {fmt}: building the 16-sequence 8-layer stack")
    stack = _stack(L, fmt)
    step(f"batch invariance {fmt}: full batch, twice")
    full = _run(stack, L, list(range(16)), fmt)
    again = _run(stack, L, list(range(16)), fmt)
    for li, (a, b) in enumerate(zip(full, again)):
        for x, y in zip(a, b):
            assert x is None or np.array_equal(x, y), f"layer {li}: repeated step differs"
    order = np.argsort(L)
    cases = [[int(order[-1])], [int(order[0])], [int(order[8])],
             [int(order[3]), int(order[15]), int(order[7])]]
    for seqs in cases:
        step(f"batch invariance {fmt}: sequences {seqs} (contexts {[int(L[j]) for j in seqs]})")
        sub = _run(stack, L, seqs, fmt)
        for li, (fo, fl, fi, fc) in enumerate(full):
            so, sl, si, sc = sub[li]
            for r, j in enumerate(seqs):
                assert np.array_equal(so[r], fo[j]), f"layer {li} seq {j}: out differs"
                assert np.array_equal(sl[r], fl[j]), f"layer {li} seq {j}: lse differs"
                if fi is not None:
                    assert sc[r] == fc[j] and np.array_equal(si[r], fi[j]), \
                        f"layer {li} seq {j}: selection differs"
