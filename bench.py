#!/usr/bin/env python3
"""Benchmark of the CSA/HCA compressed-KV attention step on one MI355X.

    python bench.py [--steps K] [--warmup W] [--workload NAME] [--no-cpu-baseline]

Prints ONE JSON line.  The default workload is the 8-layer hybrid decode stack
(CSA on even layers, HCA on odd layers; 16 sequences with context lengths drawn
uniformly from 65,536..1,048,576 tokens; 64 query heads on one KV head).  A
"step" is one decode token for every sequence through all layers.  Inputs are
seeded, synthetic and resident in HBM before timing starts.

Reported: whole-step tokens/s and HBM GB/s (algorithmic bytes / step time), the
dominant kernel's roofline (algorithmic bytes per launch / its average launch
time, timed with HIP events on the stream it runs on) and the oracle's
throughput on the host CPU for a bounded sample of the same workload.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import sys
import time

import numpy as np

HBM_PEAK_GBS = 8000.0
ROOT = os.path.dirname(os.path.abspath(__file__))
METRIC = "decode tokens/s and achieved HBM GB/s (% peak), CSA+HCA at 1M ctx, 1 GPU"


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=100)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", default="hybrid_decode_1m")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-sample-seqs", type=int, default=16)
    ap.add_argument("--kernel-reps", type=int, default=50)
    return ap.parse_args()


# ------------------------------------------------------------------ inputs
def _lengths(wl):
    from workloads import gen
    if wl.ctx_len is not None:
        return np.full(wl.batch, wl.ctx_len, dtype=np.int64)
    return gen.ragged_lengths(gen.rng(wl.cfg_id, 0, gen.T_LEN), wl.batch, *wl.ctx_range)


def _offsets(counts):
    return np.concatenate([[0], np.cumsum(counts)]).astype(np.int64)


def build_hybrid(wl, torch, lca, dev):
    """Per layer: compressed K/V drawn directly as bf16 N(0, 1/ratio), int8 indexer."""
    from workloads import gen
    L = _lengths(wl)
    B, H = wl.batch, wl.heads
    layers, host = [], []
    for li in range(wl.n_layers):
        csa = li % 2 == 0
        ratio = wl.c if csa else wl.m
        N = L // ratio
        ent_off = _offsets(N)
        tot = int(ent_off[-1])
        std = 1.0 / math.sqrt(ratio)
        d = dict(kind=lca.LCA_LAYER_CSA if csa else lca.LCA_LAYER_HCA, ratio=ratio,
                 max_entries=int(N.max()),
                 q=gen.device_bf16_normal((B, H, 128), gen.seed_of(wl.cfg_id, li, gen.T_Q), device=dev),
                 k_cmp=gen.device_bf16_normal((tot, 128), gen.seed_of(wl.cfg_id, li, gen.T_CMP_K), std, dev),
                 v_cmp=gen.device_bf16_normal((tot, 128), gen.seed_of(wl.cfg_id, li, gen.T_CMP_V), std, dev),
                 ent_off=torch.tensor(ent_off, device=dev),
                 out=torch.empty(B, H, 128, dtype=torch.bfloat16, device=dev),
                 lse=torch.empty(B, H, dtype=torch.float32, device=dev))
        if csa:
            d.update(topk=wl.topk,
                     k_idx=gen.device_int8_uniform((tot, 64), gen.seed_of(wl.cfg_id, li, gen.T_KIDX), dev),
                     q_idx=gen.device_int8_uniform((B, 64), gen.seed_of(wl.cfg_id, li, gen.T_QIDX), dev))
        layers.append(d)
        host.append(dict(N=N, ent_off=ent_off, csa=csa, ratio=ratio))
    return L, layers, host


def hybrid_bytes(L, wl):
    """Algorithmic HBM bytes of one hybrid step: indexer keys, gathered / streamed K+V,
    queries and outputs (see the per-kernel figures in the design notes)."""
    tot = 0
    qo = wl.heads * 128 * 2 * 2
    for li in range(wl.n_layers):
        if li % 2 == 0:
            N = L // wl.c
            tot += int(np.sum(64 * N + np.minimum(N, wl.topk) * 512 + 64 + qo))
        else:
            N = L // wl.m
            tot += int(np.sum(N * 512 + qo))
    return tot


# ------------------------------------------------------------------ cpu baseline
def cpu_baseline_hybrid(wl, L, layers, host, torch, nseq):
    """The oracle on the host for `nseq` sequences through all layers (one decode token each)."""
    import oracle
    try:
        from threadpoolctl import threadpool_limits
        limiter = threadpool_limits(limits=1)
    except Exception:  # pragma: no cover
        limiter = None
    scale = 1.0 / math.sqrt(128)
    elapsed = 0.0
    for b in range(nseq):
        for li, (d, h) in enumerate(zip(layers, host)):
            s, e = int(h["ent_off"][b]), int(h["ent_off"][b + 1])
            bits = lambda t: t.view(torch.int16).cpu().numpy().view(np.uint16)
            Kc = oracle.bf16_bits_to_f64(bits(d["k_cmp"][s:e]))
            Vc = oracle.bf16_bits_to_f64(bits(d["v_cmp"][s:e]))
            q = oracle.bf16_bits_to_f64(bits(d["q"][b]))
            if h["csa"]:
                kidx = d["k_idx"][s:e].cpu().numpy()
                qidx = d["q_idx"][b].cpu().numpy()
                t0 = time.perf_counter()
                oracle.csa_decode(q, qidx, int(L[b]), Kc, Vc, kidx, h["ratio"], wl.topk, scale)
                elapsed += time.perf_counter() - t0
            else:
                t0 = time.perf_counter()
                oracle.hca_decode(q, int(L[b]), Kc, Vc, h["ratio"], scale)
                elapsed += time.perf_counter() - t0
            del Kc, Vc
    if limiter is not None:
        limiter.unregister() if hasattr(limiter, "unregister") else None
    return {"value": nseq / elapsed, "unit": "tokens/s", "cores": 1, "kind": "oracle",
            "sample": f"{nseq} of {wl.batch} sequences x {wl.n_layers} layers, one decode token "
                      f"each; oracle seconds {elapsed:.2f}, input transfer excluded, BLAS 1 thread"}


# ------------------------------------------------------------------ profiles
def traffic_from_profile(kernel_tag, src_files):
    """HBM traffic per launch measured by rocprofv3 counters, if the committed
    summary was taken on the current kernel source (matching hash); else None."""
    path = os.path.join(ROOT, "profiles", "traffic.json")
    if not os.path.exists(path):
        return None
    try:
        rec = json.load(open(path)).get(kernel_tag)
    except Exception:
        return None
    if not rec:
        return None
    h = hashlib.sha256()
    for f in src_files:
        h.update(open(os.path.join(ROOT, f), "rb").read())
    return rec.get("bytes_per_launch") if rec.get("source_sha256") == h.hexdigest() else None


# ------------------------------------------------------------------ main
def main():
    args = parse()
    if args.gpus != 1:
        print(json.dumps({"error": "this build runs on one GPU only; multi-GPU runs are not "
                          "supported (--gpus must be 1)"}))
        sys.exit(2)
    import torch
    sys.path.insert(0, ROOT)
    import long_context_attention_19_amd as lca
    from long_context_attention_19_amd.pipeline import HybridStep
    import workloads

    wl = workloads.get(args.workload)
    if wl.kind != "hybrid_decode":
        print(json.dumps({"error": f"bench times the hybrid decode stack; {wl.name} is covered by "
                          "the parity tests"}))
        sys.exit(2)
    dev = "cuda"
    torch.cuda.init()
    L, layers, host = build_hybrid(wl, torch, lca, dev)
    hs = HybridStep(layers, wl.batch, 1, wl.heads, dev)
    q_off = torch.arange(wl.batch + 1, dtype=torch.int64, device=dev)
    q_pos = torch.tensor(L, dtype=torch.int64, device=dev)
    scale = 1.0 / math.sqrt(128)
    stream = torch.cuda.current_stream()
    torch.cuda.synchronize()

    for _ in range(args.warmup):
        hs.run(q_off, q_pos, scale)
    torch.cuda.synchronize()
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    ev0.record(stream)
    for _ in range(args.steps):
        hs.run(q_off, q_pos, scale)
    ev1.record(stream)
    torch.cuda.synchronize()
    ms = ev0.elapsed_time(ev1) / args.steps
    step_bytes = hybrid_bytes(L, wl)
    tokens = wl.batch

    # dominant kernel: the indexer score stream of the CSA layers, timed alone with the
    # same launch shape (fused histogram on) on this stream
    csa = [(d, h) for d, h in zip(layers, host) if h["csa"]]
    rows = wl.batch
    max_n = max(d["max_entries"] for d, _ in csa)
    scores = torch.empty(rows, (max_n + 3) // 4 * 4, dtype=torch.int32, device=dev)
    n_vis = torch.empty(rows, dtype=torch.int32, device=dev)
    hws = lca.workspace(lca.csa_topk_workspace_bytes(rows, max_n, wl.topk))
    for d, _ in csa:   # warm
        lca.csa_index_score(d["q_idx"], q_off, q_pos, d["k_idx"], d["ent_off"], wl.batch, 1,
                            d["max_entries"], wl.c, scores, n_vis, ws=hws)
    torch.cuda.synchronize()
    k0, k1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    k0.record(stream)
    for r in range(args.kernel_reps):
        d, _ = csa[r % len(csa)]
        lca.csa_index_score(d["q_idx"], q_off, q_pos, d["k_idx"], d["ent_off"], wl.batch, 1,
                            d["max_entries"], wl.c, scores, n_vis, ws=hws)
    k1.record(stream)
    torch.cuda.synchronize()
    k_ms = k0.elapsed_time(k1) / args.kernel_reps
    k_bytes = float(np.mean([int(np.sum(h["N"])) * (64 + 4) + rows * 64 for _, h in csa]))
    k_gbs = k_bytes / (k_ms * 1e-3) / 1e9

    line = {
        "metric": METRIC,
        "value": tokens / (ms * 1e-3),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16+int8",
        "data": "synthetic",
        "config": {"workload": wl.name, "batch": wl.batch,
                   "ctx_len": f"uniform {wl.ctx_range[0]}..{wl.ctx_range[1]} (mean {int(L.mean())})",
                   "layers": f"{wl.n_layers} (CSA c={wl.c} top-k={wl.topk} d_idx=64 / HCA m={wl.m})",
                   "heads": wl.heads, "kv_heads": 1, "head_dim": 128, "query_tokens": 1},
        "hbm_gbs": step_bytes / (ms * 1e-3) / 1e9,
        "hbm_frac": step_bytes / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS,
        "step_bytes": step_bytes,
        "roofline": {"kernel": "index_score_kernel<true> (CSA indexer scores + fused radix histogram)",
                     "bound": "hbm", "achieved": k_gbs, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": k_gbs / HBM_PEAK_GBS, "avg_launch_us": k_ms * 1e3,
                     "bytes_per_launch": k_bytes,
                     "traffic": traffic_from_profile(
                         "index_score_kernel", ["long_context_attention_19_amd/csrc/index_score.hip"])},
        "cpu_baseline": None,
    }
    if not args.no_cpu_baseline:
        line["cpu_baseline"] = cpu_baseline_hybrid(wl, L, layers, host, torch,
                                                   min(args.cpu_sample_seqs, wl.batch))
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
