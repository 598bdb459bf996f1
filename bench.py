#!/usr/bin/env python3
"""Benchmark of the CSA/HCA compressed-KV attention step on one MI355X.

    python bench.py [--steps K] [--warmup W] [--workload NAME] [--no-cpu-baseline]

Prints ONE JSON line.  The default workload is the 8-layer hybrid decode stack
(CSA on even layers, HCA on odd layers; 16 sequences with context lengths drawn
uniformly from 65,536..1,048,576 tokens; 64 query heads on one KV head); the
other workloads (csa_decode_8k, hca_decode_128k, csa_decode_1m,
csa_prefill_256k, hybrid_decode_1m_swa: the stack with a 128-token sliding window on
every layer, hybrid_decode_1m_swa_sink: that and a per-head attention sink on every
layer, hybrid_decode_1m_fp4: the stack with the FP4 indexer, hybrid_decode_1m_kv8: the
stack over mixed FP8 / bf16 KV rows, csa_decode_1m_fp4: the 1M CSA decode with the FP4
indexer, csa_prefill_256k_fp4: the prefill chunk with the FP4 indexer) can be named with
--workload.  A step is one pass of the
workload's whole path over one batch; inputs are seeded, synthetic and resident
in HBM before timing starts.  Decode workloads smaller than the 256 MB
last-level cache rotate input replicas so that each step reads from HBM.

Reported: whole-step tokens/s and HBM GB/s (algorithmic bytes / step time), the
dominant kernel's roofline (algorithmic bytes or flops per launch / its average
launch time, timed with HIP events on the stream it runs on) and the oracle's
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

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0
BF16_PEAK_TFLOPS = 2500.0
METRIC = "decode tokens/s and achieved HBM GB/s (% peak), CSA+HCA at 1M ctx, 1 GPU"
SCALE = 1.0 / math.sqrt(128)
QO_BYTES_PER_HEAD = 128 * 2 * 2   # bf16 query row in, bf16 output row out


def parse(argv=None):
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=100)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", default="hybrid_decode_1m")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-sample", type=int, default=0, help="oracle sample size (0 = default)")
    ap.add_argument("--kernel-reps", type=int, default=50)
    ap.add_argument("--copy-probe", type=int, default=0, metavar="BYTES",
                    help="only run 10 plain device copies of BYTES bytes (counter calibration)")
    ap.add_argument("--no-graph", action="store_true",
                    help="enqueue each step eagerly instead of replaying captured HIP graphs")
    ap.add_argument("--no-extra", action="store_true",
                    help="the hybrid workload alone: skip the 1M CSA decode measured beside it")
    return ap.parse_args(argv)


def _bits(t):
    import torch
    return t.contiguous().view(torch.int16).cpu().numpy().view(np.uint16)


def _src_hash(files):
    h = hashlib.sha256()
    for f in files:
        h.update(open(os.path.join(ROOT, f), "rb").read())
    return h.hexdigest()


def traffic_from_profile(tag, src_files, workload):
    """HBM bytes per launch from the committed rocprofv3 counter summary, only if
    it was taken on this workload and on the current kernel source (matching hash);
    else None."""
    path = os.path.join(ROOT, "profiles", "traffic.json")
    if not os.path.exists(path):
        return None
    try:
        rec = json.load(open(path)).get(f"{tag} @ {workload}")
    except Exception:
        return None
    if not rec or rec.get("workload", "").split(" ")[0] != workload:
        return None
    if rec.get("source_sha256") != _src_hash(src_files):
        return None
    return rec.get("bytes_per_launch")


def _dtype(wl):
    """Arithmetic types of the step: bf16 attention, the indexer's codes (CSA layers),
    FP8 halves of mixed cache rows."""
    parts = ["bf16"]
    if wl.kv8:
        parts.append("fp8")
    if wl.kind != "hca_decode":
        parts.append("fp4" if wl.idx_fp4 else "int8")
    return "+".join(parts)


CPU_BUDGET_S = 12.0   # oracle time the cpu_baseline leg aims for
INDEX_REPS = 10       # back-to-back index-pass launches per timed step (its launch duration)


def _timed_reps(fn, budget):
    """Mean time of fn() over repeated calls until `budget` seconds are spent (at least
    one call; the inputs are converted once, outside the timing)."""
    spent, reps = 0.0, 0
    while reps == 0 or spent < budget:
        t0 = time.perf_counter()
        fn()
        spent += time.perf_counter() - t0
        reps += 1
    return spent / reps, spent, reps


def host_cores() -> int:
    """Host cores this process may run on (its CPU affinity), capped by OMP_NUM_THREADS
    where the environment sets it (a shared host's per-job share)."""
    n = len(os.sched_getaffinity(0))
    try:
        cap = int(os.environ.get("OMP_NUM_THREADS", "0"))
    except ValueError:
        cap = 0
    return max(1, min(n, cap) if cap > 0 else n)


class _HostThreads:
    """Run the oracle with its BLAS pool at the host's core count (host_cores())."""

    def __enter__(self):
        self.cores = host_cores()
        try:
            from threadpoolctl import threadpool_limits
            self._lim = threadpool_limits(limits=self.cores)
        except Exception:  # pragma: no cover
            self._lim = None
        return self

    def __exit__(self, *a):
        if self._lim is not None:
            self._lim.restore_original_limits()


# ====================================================================== runners
class _Capture:
    """One HIP graph per input replica: a step is then a single graph launch."""
    R = 1

    def capture(self):
        torch = self.torch
        self.step(0)                       # eager first: creates the library's streams
        torch.cuda.synchronize()
        graphs = []
        for r in range(self.R):
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g):
                self.step(r)
            graphs.append(g)
        torch.cuda.synchronize()
        return graphs


class HybridRunner(_Capture):
    """8 independent layers, CSA (even) / HCA (odd), one decode token per sequence."""
    dominant_tag = "ds_chunk_kernel"
    dominant_src = ["long_context_attention_19_amd/csrc/decode_select.hip"]

    def __init__(self, wl, device="cuda"):
        import torch
        import long_context_attention_19_amd as lca
        from long_context_attention_19_amd.pipeline import HybridStep
        from workloads import device as wdev
        self.wl, self.lca, self.torch = wl, lca, torch
        self.L, self.layers = wdev.hybrid_inputs(wl, device)
        B, H = wl.batch, wl.heads
        specs = []
        for d in self.layers:
            s = dict(kind=lca.LCA_LAYER_CSA if d["csa"] else lca.LCA_LAYER_HCA, ratio=d["ratio"],
                     max_entries=d["max_entries"], q=d["q"], k_cmp=d["k_cmp"], v_cmp=d["v_cmp"],
                     ent_off=d["ent_off_dev"],
                     out=torch.empty(B, H, 128, dtype=torch.bfloat16, device=device),
                     lse=torch.empty(B, H, dtype=torch.float32, device=device))
            if d["csa"]:
                s.update(topk=wl.topk, k_idx=d["k_idx"], q_idx=d["q_idx"])
                if wl.idx_fp4:
                    s.update(idx_format=lca.LCA_IDX_FP4)
            if wl.kv8:
                s.update(kv_format=lca.LCA_KV_MIXED)
            if wl.window:
                s.update(win_k=d["win_k"], win_v=d["win_v"], win_off=d["win_off_dev"],
                         win_pos0=d["win_pos0_dev"], window=wl.window)
            if wl.sink:
                s.update(sink=d["sink_dev"])
            specs.append(s)
        self.hs = HybridStep(specs, B, 1, H, device)
        self.q_off = torch.arange(B + 1, dtype=torch.int64, device=device)
        self.q_pos = torch.tensor(self.L, dtype=torch.int64, device=device)
        self.tokens_per_step = B
        # dominant kernel: the CSA indexer scores (+ fused histogram) launch of the step
        self._csa = [d for d in self.layers if d["csa"]]

    @property
    def outputs(self):
        return self.hs.layers

    def step(self, i=0):
        self.hs.run(self.q_off, self.q_pos, SCALE)

    def step_bytes(self):
        wl, tot = self.wl, 0
        for d in self.layers:
            N = d["N"]
            kv = 2 * 192 if wl.kv8 else 512   # K + V bytes per attended entry
            if d["csa"]:
                kb = 32 if wl.idx_fp4 else 64   # indexer key / query bytes
                tot += int(np.sum(kb * N + np.minimum(N, wl.topk) * kv + kb))
            else:
                tot += int(np.sum(N * kv))
            tot += wl.batch * wl.heads * QO_BYTES_PER_HEAD
            if wl.window:   # window K/V rows, and the merge's re-read of out and lse
                tot += int(np.sum(d["win_n"]) * 512) + wl.batch * wl.heads * QO_BYTES_PER_HEAD
            if wl.sink:     # the sink logits
                tot += wl.heads * 4
        return tot

    def dominant_ms(self, reps):
        """Average duration of the step's indexer-score launch (all CSA layers in one
        launch), from HIP events the library records on the stream it runs on, over
        `reps` eager steps of the same configuration."""
        lca, torch = self.lca, self.torch
        lca.hybrid_timing_enable(True, index_reps=INDEX_REPS)
        try:
            t = []
            for _ in range(max(1, reps)):
                self.step()
                t.append(lca.hybrid_timing_read())
        finally:
            torch.cuda.synchronize()
            lca.hybrid_timing_enable(False)
        self.phase_ms = [float(np.mean([x[p] for x in t])) for p in range(len(t[0]))]
        return self.phase_ms[0]

    def dominant_units(self):
        n = float(sum(int(np.sum(d["N"])) for d in self._csa))
        kb = 32 if self.wl.idx_fp4 else 64
        fmt = "FP4 (FP4 MFMA)" if self.wl.idx_fp4 else "int8 (v_dot4)"
        return {"bound": "hbm", "per_launch": n * kb + len(self._csa) * self.wl.batch * kb,
                "unit": "GB/s",
                "kernel": f"ds_chunk_kernel ({len(self._csa)} CSA layers in one launch): {fmt} "
                          "indexer scores in LDS, per-chunk top-k candidates (no score matrix)",
                "per_unit": f"{kb} B per compressed entry (indexer key read) + {kb} B per query"}

    def cpu_baseline(self, n):
        import oracle
        wl, torch = self.wl, self.torch
        n = n or wl.batch
        per_call = CPU_BUDGET_S / (n * len(self.layers))
        t_tok, spent, calls = 0.0, 0.0, 0
        with _HostThreads() as ht:
            for b in range(n):
                for d in self.layers:
                    s, e = int(d["ent_off"][b]), int(d["ent_off"][b + 1])
                    if wl.kv8:
                        Kc = oracle.kv8_values(d["k_cmp"][s:e].cpu().numpy())
                        Vc = oracle.kv8_values(d["v_cmp"][s:e].cpu().numpy())
                    else:
                        Kc = oracle.bf16_bits_to_f64(_bits(d["k_cmp"][s:e]))
                        Vc = oracle.bf16_bits_to_f64(_bits(d["v_cmp"][s:e]))
                    q = oracle.bf16_bits_to_f64(_bits(d["q"][b]))
                    L = int(self.L[b])
                    if wl.window:
                        ws, we = int(d["win_off"][b]), int(d["win_off"][b + 1])
                        Kw = oracle.bf16_bits_to_f64(_bits(d["win_k"][ws:we]))
                        Vw = oracle.bf16_bits_to_f64(_bits(d["win_v"][ws:we]))
                        p0 = int(d["win_pos0"][b])
                    if wl.sink:
                        z = d["sink"].astype(np.float64)
                        Kw_, Vw_, p0_, w_ = (Kw, Vw, p0, wl.window) if wl.window else (None, None, 0, 0)
                        if d["csa"]:
                            kidx, qidx = d["k_idx"][s:e].cpu().numpy(), d["q_idx"][b].cpu().numpy()
                            fn = lambda: oracle.csa_query_sink(q, qidx, L, Kc, Vc, kidx, d["ratio"],
                                                               wl.topk, SCALE, z, Kw_, Vw_, p0_, w_)
                        else:
                            fn = lambda: oracle.hca_query_sink(q, L, Kc, Vc, d["ratio"], SCALE, z,
                                                               Kw_, Vw_, p0_, w_)
                    elif d["csa"] and wl.idx_fp4:
                        kidx, qidx = d["k_idx"][s:e].cpu().numpy(), d["q_idx"][b].cpu().numpy()
                        fn = lambda: oracle.csa_query_fp4(q, qidx, L, Kc, Vc, kidx, d["ratio"],
                                                          wl.topk, SCALE)
                    elif d["csa"]:
                        kidx, qidx = d["k_idx"][s:e].cpu().numpy(), d["q_idx"][b].cpu().numpy()
                        if wl.window:
                            fn = lambda: oracle.csa_query_swa(q, qidx, L, Kc, Vc, kidx, d["ratio"],
                                                              wl.topk, SCALE, Kw, Vw, p0, wl.window)
                        else:
                            fn = lambda: oracle.csa_decode(q, qidx, L, Kc, Vc, kidx, d["ratio"],
                                                           wl.topk, SCALE)
                    elif wl.window:
                        fn = lambda: oracle.hca_query_swa(q, L, Kc, Vc, d["ratio"], SCALE, Kw, Vw,
                                                          p0, wl.window)
                    else:
                        fn = lambda: oracle.hca_decode(q, L, Kc, Vc, d["ratio"], SCALE)
                    mean, sp, r = _timed_reps(fn, per_call)
                    t_tok += mean
                    spent += sp
                    calls += r
        return {"value": n / t_tok, "unit": "tokens/s", "cores": ht.cores, "kind": "oracle",
                "sample": f"{n} of {wl.batch} sequences through all {wl.n_layers} layers, one "
                          f"decode token each; {calls} oracle layer calls, {spent:.1f} s of "
                          f"oracle time (transfers and conversions excluded)"}


class CsaDecodeRunner(_Capture):
    """CSA decode over caches compressed from raw tokens (compression is setup).  The
    step is the library's layer-stack step with one CSA layer: the candidate index
    pass, the top-k selection and the sparse attention; one step object per input
    replica (distinct indexer keys, queries and outputs)."""
    dominant_tag = "ds_chunk_kernel"
    dominant_src = ["long_context_attention_19_amd/csrc/decode_select.hip"]

    def __init__(self, wl, device="cuda", replicas=None):
        import torch
        import long_context_attention_19_amd as lca
        from long_context_attention_19_amd.pipeline import HybridStep
        from workloads import device as wdev
        self.wl, self.lca, self.torch = wl, lca, torch
        per_step = wl.batch * (wl.ctx_len // wl.c) * (32 if wl.idx_fp4 else 64)
        R = replicas or max(1, min(16, math.ceil(1.0e9 / per_step)))
        self.inp = wdev.decode_raw_inputs(wl, device, R)
        inp = self.inp
        n_tot = int(inp["ent_off"][-1])
        self.k_cmp = torch.empty(n_tot, 128, dtype=torch.bfloat16, device=device)
        self.v_cmp = torch.empty(n_tot, 128, dtype=torch.bfloat16, device=device)
        T = int(inp["L"].max())
        lca.kv_compress(inp["raw_k"], inp["tok_off_dev"], wl.batch, T, wl.c, self.k_cmp,
                        inp["ent_off_dev"])
        lca.kv_compress(inp["raw_v"], inp["tok_off_dev"], wl.batch, T, wl.c, self.v_cmp,
                        inp["ent_off_dev"])
        self.max_entries = int(inp["N"].max())
        self.steps = []
        for r in inp["replicas"]:
            spec = dict(kind=lca.LCA_LAYER_CSA, ratio=wl.c, topk=wl.topk,
                        max_entries=self.max_entries, q=r["q"], q_idx=r["q_idx"],
                        k_idx=r["k_idx"], k_cmp=self.k_cmp, v_cmp=self.v_cmp,
                        ent_off=inp["ent_off_dev"],
                        out=torch.empty(wl.batch, wl.heads, 128, dtype=torch.bfloat16,
                                        device=device),
                        lse=torch.empty(wl.batch, wl.heads, dtype=torch.float32, device=device))
            if wl.idx_fp4:
                spec["idx_format"] = lca.LCA_IDX_FP4
            self.steps.append(HybridStep([spec], wl.batch, 1, wl.heads, device))
        self.q_off = torch.arange(wl.batch + 1, dtype=torch.int64, device=device)
        self.q_pos = torch.tensor(inp["L"], dtype=torch.int64, device=device)
        self.tokens_per_step = wl.batch
        self.R = R

    def layer(self, i=0):
        """The layer dict of replica i: its inputs and its idx / count / out / lse."""
        return self.steps[i % self.R].layers[0]

    def step(self, i=0):
        self.steps[i % self.R].run(self.q_off, self.q_pos, SCALE)

    def step_bytes(self):
        N, wl = self.inp["N"], self.wl
        kb = 32 if wl.idx_fp4 else 64   # indexer key / query bytes
        return int(np.sum(kb * N + np.minimum(N, wl.topk) * 512 + kb)) + \
            wl.batch * wl.heads * QO_BYTES_PER_HEAD

    def dominant_ms(self, reps):
        """Average duration of the step's index pass (scores and candidates), from HIP
        events the library records around it on its stream, over `reps` eager steps."""
        lca, torch = self.lca, self.torch
        lca.hybrid_timing_enable(True, index_reps=INDEX_REPS)
        try:
            t = []
            for i in range(max(1, reps)):
                self.step(i)
                t.append(lca.hybrid_timing_read())
        finally:
            torch.cuda.synchronize()
            lca.hybrid_timing_enable(False)
        self.phase_ms = [float(np.mean([x[p] for x in t])) for p in range(len(t[0]))]
        return self.phase_ms[0]

    def dominant_units(self):
        n = int(np.sum(self.inp["N"]))
        kb = 32 if self.wl.idx_fp4 else 64
        fmt = "FP4 (FP4 MFMA)" if self.wl.idx_fp4 else "int8 (v_dot4)"
        return {"bound": "hbm", "per_launch": n * kb + self.wl.batch * kb, "unit": "GB/s",
                "kernel": f"ds_chunk_kernel: {fmt} indexer scores in LDS, per-chunk top-k "
                          "candidates (no score matrix)",
                "per_unit": f"{kb} B per compressed entry (indexer key read) + {kb} B per query"}

    def cpu_baseline(self, n):
        import oracle
        wl, inp = self.wl, self.inp
        n = n or wl.batch
        r = inp["replicas"][0]
        t_tok, spent, calls = 0.0, 0.0, 0
        with _HostThreads() as ht:
            for b in range(n):
                s, e = int(inp["ent_off"][b]), int(inp["ent_off"][b + 1])
                Kc = oracle.bf16_bits_to_f64(_bits(self.k_cmp[s:e]))
                Vc = oracle.bf16_bits_to_f64(_bits(self.v_cmp[s:e]))
                kidx, qidx = r["k_idx"][s:e].cpu().numpy(), r["q_idx"][b].cpu().numpy()
                q = oracle.bf16_bits_to_f64(_bits(r["q"][b]))
                L = int(inp["L"][b])
                query = oracle.csa_query_fp4 if wl.idx_fp4 else oracle.csa_decode
                mean, sp, rp = _timed_reps(
                    lambda: query(q, qidx, L, Kc, Vc, kidx, wl.c, wl.topk, SCALE),
                    CPU_BUDGET_S / n)
                t_tok += mean
                spent += sp
                calls += rp
        return {"value": n / t_tok, "unit": "tokens/s", "cores": ht.cores, "kind": "oracle",
                "sample": f"{n} of {wl.batch} sequences, one decode token each over the "
                          f"compressed cache; {calls} oracle calls, {spent:.1f} s of oracle time"}


class HcaDecodeRunner(_Capture):
    dominant_tag = "hca_dense_attn"
    dominant_src = ["long_context_attention_19_amd/csrc/attention.hip"]

    def __init__(self, wl, device="cuda", replicas=None):
        import torch
        import long_context_attention_19_amd as lca
        from long_context_attention_19_amd.pipeline import HcaStep
        from workloads import device as wdev
        self.wl, self.lca, self.torch = wl, lca, torch
        self.inp = wdev.decode_raw_inputs(wl, device, 1)
        inp = self.inp
        n_tot = int(inp["ent_off"][-1])
        T = int(inp["L"].max())
        k0 = torch.empty(n_tot, 128, dtype=torch.bfloat16, device=device)
        v0 = torch.empty(n_tot, 128, dtype=torch.bfloat16, device=device)
        lca.kv_compress(inp["raw_k"], inp["tok_off_dev"], wl.batch, T, wl.m, k0, inp["ent_off_dev"])
        lca.kv_compress(inp["raw_v"], inp["tok_off_dev"], wl.batch, T, wl.m, v0, inp["ent_off_dev"])
        per_step = n_tot * 512
        self.R = replicas or max(1, min(256, math.ceil(1.0e9 / per_step)))
        # replicas at distinct addresses so each step streams its caches from HBM
        self.caches = [(k0, v0)] + [(k0.clone(), v0.clone()) for _ in range(self.R - 1)]
        self.st = HcaStep(wl.batch, 1, int(inp["N"].max()), wl.heads, wl.m, device)
        self.q_off = torch.arange(wl.batch + 1, dtype=torch.int64, device=device)
        self.q_pos = torch.tensor(inp["L"], dtype=torch.int64, device=device)
        self.out = torch.empty(wl.batch, wl.heads, 128, dtype=torch.bfloat16, device=device)
        self.lse = torch.empty(wl.batch, wl.heads, dtype=torch.float32, device=device)
        self.tokens_per_step = wl.batch

    def step(self, i=0):
        k, v = self.caches[i % self.R]
        self.st.run(self.inp["replicas"][0]["q"], k, v, self.inp["ent_off_dev"], self.q_off,
                    self.q_pos, SCALE, self.out, self.lse)

    def step_bytes(self):
        return int(np.sum(self.inp["N"])) * 512 + self.wl.batch * self.wl.heads * QO_BYTES_PER_HEAD

    def dominant_launch(self):
        self._i = getattr(self, "_i", 0) + 1
        self.step(self._i)

    def dominant_units(self):
        return {"bound": "hbm", "per_launch": self.step_bytes(), "unit": "GB/s",
                "kernel": "hca_dense_attn (attn_dma_kernel + split combine)",
                "per_unit": "512 B per visible entry (K+V bf16) + 512 B per head (q in, o out)"}

    def cpu_baseline(self, n):
        import oracle
        wl, inp = self.wl, self.inp
        n = n or wl.batch
        k, v = self.caches[0]
        t_tok, spent, calls = 0.0, 0.0, 0
        with _HostThreads() as ht:
            for b in range(n):
                s, e = int(inp["ent_off"][b]), int(inp["ent_off"][b + 1])
                Kc, Vc = oracle.bf16_bits_to_f64(_bits(k[s:e])), oracle.bf16_bits_to_f64(_bits(v[s:e]))
                q = oracle.bf16_bits_to_f64(_bits(inp["replicas"][0]["q"][b]))
                L = int(inp["L"][b])
                mean, sp, rp = _timed_reps(lambda: oracle.hca_decode(q, L, Kc, Vc, wl.m, SCALE),
                                           CPU_BUDGET_S / n)
                t_tok += mean
                spent += sp
                calls += rp
        return {"value": n / t_tok, "unit": "tokens/s", "cores": ht.cores, "kind": "oracle",
                "sample": f"{n} of {wl.batch} sequences; {calls} oracle calls, {spent:.1f} s "
                          f"of oracle time"}


class PrefillRunner(_Capture):
    """Chunked prefill: compress the new tokens into the cache, then score, select and
    attend for every new query token under block-causal visibility."""
    dominant_tag = "csa_sparse_attn"
    dominant_src = ["long_context_attention_19_amd/csrc/attention.hip"]

    def __init__(self, wl, device="cuda", replicas=None):
        import torch
        import long_context_attention_19_amd as lca
        from long_context_attention_19_amd.pipeline import CsaStep
        from workloads import device as wdev
        self.wl, self.lca, self.torch = wl, lca, torch
        self.inp = wdev.prefill_inputs(wl, device)
        inp = self.inp
        ctx, new, c = wl.ctx_len, wl.new_tokens, wl.c
        self.n_ctx = ctx // c
        self.k_cmp = torch.zeros(inp["n_ent"], 128, dtype=torch.bfloat16, device=device)
        self.v_cmp = torch.zeros(inp["n_ent"], 128, dtype=torch.bfloat16, device=device)
        i64 = lambda a: torch.tensor(a, dtype=torch.int64, device=device)
        lca.kv_compress(inp["raw_k_ctx"], i64([0, ctx]), 1, ctx, c, self.k_cmp, i64([0, self.n_ctx]))
        lca.kv_compress(inp["raw_v_ctx"], i64([0, ctx]), 1, ctx, c, self.v_cmp, i64([0, self.n_ctx]))
        self.new_tok_off = i64([0, new])
        self.new_ent_off = i64([0, new // c])
        self.ent_off = i64([0, inp["n_ent"]])
        self.q_off = i64([0, new])
        self.q_pos = torch.arange(ctx, ctx + new, dtype=torch.int64, device=device)
        self.st = CsaStep(1, new, inp["n_ent"], wl.heads, wl.topk, c, device, fp4=wl.idx_fp4)
        self.out = torch.empty(new, wl.heads, 128, dtype=torch.bfloat16, device=device)
        self.lse = torch.empty(new, wl.heads, dtype=torch.float32, device=device)
        self.tokens_per_step = new

    def step(self, i=0):
        wl, inp, lca = self.wl, self.inp, self.lca
        new, c = wl.new_tokens, wl.c
        lca.kv_compress(inp["new_k"], self.new_tok_off, 1, new, c, self.k_cmp[self.n_ctx:],
                        self.new_ent_off)
        lca.kv_compress(inp["new_v"], self.new_tok_off, 1, new, c, self.v_cmp[self.n_ctx:],
                        self.new_ent_off)
        self.st.run(inp["q"], inp["q_idx"], self.q_off, self.q_pos, inp["k_idx"], self.k_cmp,
                    self.v_cmp, self.ent_off, SCALE, self.out, self.lse)

    def step_bytes(self):
        wl = self.wl
        new = wl.new_tokens
        kb = 32 if wl.idx_fp4 else 64   # indexer key / query bytes
        return (new * 128 * 2 * 2 + (new // wl.c) * 512 + self.inp["n_ent"] * kb + new * kb +
                new * wl.heads * QO_BYTES_PER_HEAD + self.inp["n_ent"] * 512)

    def dominant_launch(self):
        self.st.attend(self.inp["q"], self.k_cmp, self.v_cmp, self.ent_off, self.q_off, SCALE,
                       self.out, self.lse)

    def dominant_units(self):
        wl = self.wl
        flops = wl.new_tokens * wl.heads * wl.topk * 128 * 4.0
        return {"bound": "mfma", "per_launch": flops, "unit": "TFLOP/s",
                "kernel": "csa_sparse_attn (attn_dma_kernel, bf16 MFMA)",
                "per_unit": "4*128 flops per (query, head, selected entry)"}

    def cpu_baseline(self, n):
        import oracle
        wl, inp = self.wl, self.inp
        Kc = oracle.bf16_bits_to_f64(_bits(self.k_cmp))
        Vc = oracle.bf16_bits_to_f64(_bits(self.v_cmp))
        kidx = inp["k_idx"].cpu().numpy()
        # query tokens spread over the chunk, until the budget is spent (or n given)
        order = np.random.default_rng(0).permutation(wl.new_tokens)
        t_or, done = 0.0, 0
        with _HostThreads() as ht:
            for i in order:
                if (n and done >= n) or (not n and t_or >= CPU_BUDGET_S):
                    break
                q = oracle.bf16_bits_to_f64(_bits(inp["q"][i]))
                qi = inp["q_idx"][i].cpu().numpy()
                t0 = time.perf_counter()
                query = oracle.csa_query_fp4 if wl.idx_fp4 else oracle.csa_query
                query(q, qi, wl.ctx_len + int(i), Kc, Vc, kidx, wl.c, wl.topk, SCALE)
                t_or += time.perf_counter() - t0
                done += 1
        return {"value": done / t_or, "unit": "tokens/s", "cores": ht.cores, "kind": "oracle",
                "sample": f"{done} of {wl.new_tokens} query tokens (random order) after "
                          f"compression ({t_or:.1f} s of oracle time)"}


RUNNERS = {"hybrid_decode": HybridRunner, "csa_decode": CsaDecodeRunner,
           "hca_decode": HcaDecodeRunner, "csa_prefill": PrefillRunner}


def make_runner(wl, device="cuda"):
    return RUNNERS[wl.kind](wl, device)


def _time(fn, n, stream, torch):
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    e0.record(stream)
    for i in range(n):
        fn(i)
    e1.record(stream)
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) / n


def _measure(run, args, stream, torch):
    """W warm-up steps, then the mean time of K steps (HIP-graph replays unless
    --no-graph), bracketed by device synchronisations."""
    torch.cuda.synchronize()
    if args.no_graph:
        step_fn = run.step
    else:
        graphs = run.capture()
        step_fn = lambda i: graphs[i % len(graphs)].replay()
    for i in range(args.warmup):
        step_fn(i)
    return _time(step_fn, args.steps, stream, torch)


def _extra_csa_1m(args, stream, torch):
    """The 1M-context CSA decode (4 sequences of 1,048,576 tokens, top-k 2048), timed the
    same way in the same process: its step time, tokens/s, HBM rate and phases."""
    import workloads
    wl = workloads.get("csa_decode_1m")
    run = make_runner(wl)
    ms = _measure(run, args, stream, torch)
    k_ms = run.dominant_ms(args.kernel_reps)
    u = run.dominant_units()
    sb = run.step_bytes()
    out = {"workload": wl.name, "ms_per_step": ms, "tokens_per_s": run.tokens_per_step / (ms * 1e-3),
           "step_bytes": sb, "hbm_gbs": sb / (ms * 1e-3) / 1e9,
           "hbm_frac": sb / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS,
           "phases_ms": dict(zip(["index_pass", "selection", "attention"], run.phase_ms)),
           "index_pass": {"avg_launch_us": k_ms * 1e3, "per_launch": u["per_launch"],
                          "achieved_gbs": u["per_launch"] / (k_ms * 1e-3) / 1e9,
                          "frac": u["per_launch"] / (k_ms * 1e-3) / 1e9 / HBM_PEAK_GBS}}
    del run
    torch.cuda.synchronize()
    torch.cuda.empty_cache()
    return out


def main(argv=None):
    args = parse(argv)
    if args.gpus != 1:
        print(json.dumps({"error": "one GPU only: the step runs on a single GPU's share of the "
                                   "work and has no multi-GPU path; run with --gpus 1"}),
              flush=True)
        sys.exit(2)
    import torch
    import workloads

    if args.copy_probe:
        a = torch.ones(args.copy_probe, dtype=torch.uint8, device="cuda")
        b = torch.empty_like(a)
        stream = torch.cuda.current_stream()
        ms = _time(lambda i: b.copy_(a), 10, stream, torch)
        print(json.dumps({"copy_probe_bytes": args.copy_probe, "ms": ms,
                          "gbs_read_plus_write": 2 * args.copy_probe / (ms * 1e-3) / 1e9}), flush=True)
        return
    wl = workloads.get(args.workload)
    torch.cuda.init()
    run = make_runner(wl)
    stream = torch.cuda.current_stream()
    ms = _measure(run, args, stream, torch)
    sb = run.step_bytes()

    # dominant kernel: inside the step where the runner can time it there, else alone
    # with the same launch shape on the same stream
    if hasattr(run, "dominant_ms"):
        k_ms = run.dominant_ms(args.kernel_reps)
    else:
        for i in range(3):
            run.dominant_launch()
        k_ms = _time(lambda i: run.dominant_launch(), args.kernel_reps, stream, torch)
    u = run.dominant_units()
    scale_u = 1e9 if u["unit"] == "GB/s" else 1e12
    peak = HBM_PEAK_GBS if u["bound"] == "hbm" else BF16_PEAK_TFLOPS
    achieved = u["per_launch"] / (k_ms * 1e-3) / scale_u
    cfg = {"workload": wl.name, "batch": wl.batch, "heads": wl.heads, "kv_heads": 1,
           "head_dim": 128}
    if wl.ctx_len is None:
        cfg["ctx_len"] = f"uniform {wl.ctx_range[0]}..{wl.ctx_range[1]}"
    else:
        cfg["ctx_len"] = wl.ctx_len
    if wl.kind == "hybrid_decode":
        cfg["layers"] = f"{wl.n_layers} (CSA c={wl.c} top-k={wl.topk} d_idx=64 / HCA m={wl.m})"
    elif wl.kind == "hca_decode":
        cfg["m"] = wl.m
    else:
        cfg.update(c=wl.c, topk=wl.topk, d_idx=64)
    if wl.new_tokens:
        cfg["new_tokens"] = wl.new_tokens
    if wl.window:
        cfg["window"] = wl.window
    if wl.sink:
        cfg["sink"] = "per-head logits on every layer"
    if wl.idx_fp4:
        cfg["indexer"] = "FP4 E2M1 (32 B per key)"
    if wl.kv8:
        cfg["kv_storage"] = "mixed rows: FP8 E4M3 dims 0..63, bf16 dims 64..127 (192 B)"
    line = {
        "metric": METRIC,
        "value": run.tokens_per_step / (ms * 1e-3),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": _dtype(wl),
        "data": "synthetic",
        "config": cfg,
        "launch": "eager" if args.no_graph else f"hip-graph replay ({getattr(run, 'R', 1)} replica graphs)",
        "hbm_gbs": sb / (ms * 1e-3) / 1e9,
        "hbm_frac": sb / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS,
        "step_bytes": sb,
        "roofline": {"kernel": u["kernel"], "bound": u["bound"], "achieved": achieved,
                     "peak": peak, "unit": u["unit"], "frac": achieved / peak,
                     "avg_launch_us": k_ms * 1e3,
                     "avg_launch_source": (f"HIP events the library records on its stream around "
                                           f"{INDEX_REPS} back-to-back launches of the index pass "
                                           f"in eager steps, per launch" if hasattr(run, "dominant_ms")
                                           else "HIP events around repeated launches of the same "
                                                "shape on the step's stream"),
                     "per_launch": u["per_launch"],
                     "per_unit": u["per_unit"],
                     "traffic": traffic_from_profile(run.dominant_tag, run.dominant_src,
                                                     wl.name)},
        "cpu_baseline": None,
    }
    if hasattr(run, "phase_ms"):
        line["phases_ms"] = dict(zip(["index_pass", "selection", "attention"], run.phase_ms))
    if not args.no_cpu_baseline:
        line["cpu_baseline"] = run.cpu_baseline(args.cpu_sample)
    if wl.name == "hybrid_decode_1m" and not args.no_extra:
        del run
        torch.cuda.synchronize()
        torch.cuda.empty_cache()
        line["csa_decode_1m"] = _extra_csa_1m(args, stream, torch)
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
