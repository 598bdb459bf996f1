"""Full-size inputs for the five workloads, drawn on the GPU (seeded Philox).

Input generation only: raw tokens, compressed entries drawn directly where the
workload says so, int8 indexer vectors, queries and lengths.  Nothing here
computes any step of the method; raw tokens are compressed by the caller.
Every tensor's seed is seed_of(workload id, layer, tensor id[, replica]).
"""
from __future__ import annotations

import math

import numpy as np

from . import gen
from .configs import Workload


def lengths(wl: Workload) -> np.ndarray:
    if wl.ctx_len is not None:
        return np.full(wl.batch, wl.ctx_len, dtype=np.int64)
    return gen.ragged_lengths(gen.rng(wl.cfg_id, 0, gen.T_LEN), wl.batch, *wl.ctx_range)


def offsets(counts) -> np.ndarray:
    return np.concatenate([[0], np.cumsum(np.asarray(counts, dtype=np.int64))]).astype(np.int64)


def hybrid_inputs(wl: Workload, device="cuda"):
    """Per layer (CSA on even layers, HCA on odd): compressed K/V drawn directly as
    bf16 N(0, 1/ratio) (the distribution of a mean of `ratio` N(0,1) tokens, without
    materialising ~36 GB of raw tokens), int8 indexer keys/queries, bf16 queries."""
    import torch

    L = lengths(wl)
    B, H = wl.batch, wl.heads
    layers = []
    for li in range(wl.n_layers):
        csa = li % 2 == 0
        ratio = wl.c if csa else wl.m
        N = L // ratio
        ent_off = offsets(N)
        tot = int(ent_off[-1])
        std = 1.0 / math.sqrt(ratio)
        d = dict(csa=csa, ratio=ratio, N=N, ent_off=ent_off, max_entries=int(N.max()),
                 q=gen.device_bf16_normal((B, H, 128), gen.seed_of(wl.cfg_id, li, gen.T_Q),
                                          device=device),
                 k_cmp=(gen.device_kv8_normal(tot, gen.seed_of(wl.cfg_id, li, gen.T_CMP_K), std, device)
                        if wl.kv8 else
                        gen.device_bf16_normal((tot, 128), gen.seed_of(wl.cfg_id, li, gen.T_CMP_K),
                                               std, device)),
                 v_cmp=(gen.device_kv8_normal(tot, gen.seed_of(wl.cfg_id, li, gen.T_CMP_V), std, device)
                        if wl.kv8 else
                        gen.device_bf16_normal((tot, 128), gen.seed_of(wl.cfg_id, li, gen.T_CMP_V),
                                               std, device)),
                 ent_off_dev=torch.tensor(ent_off, device=device))
        if csa and wl.idx_fp4:   # packed FP4 codes, 32 bytes per vector
            d["k_idx"] = gen.device_fp4_uniform((tot, 32), gen.seed_of(wl.cfg_id, li, gen.T_KFP4),
                                                device)
            d["q_idx"] = gen.device_fp4_uniform((B, 32), gen.seed_of(wl.cfg_id, li, gen.T_QFP4),
                                                device)
        elif csa:
            d["k_idx"] = gen.device_int8_uniform((tot, 64), gen.seed_of(wl.cfg_id, li, gen.T_KIDX),
                                                 device)
            d["q_idx"] = gen.device_int8_uniform((B, 64), gen.seed_of(wl.cfg_id, li, gen.T_QIDX),
                                                 device)
        if wl.window:
            # state buffer: the last `window` raw tokens of each sequence, N(0,1)
            nbuf = np.minimum(L, wl.window)
            boff = offsets(nbuf)
            d["win_n"] = nbuf
            d["win_off"] = boff
            d["win_pos0"] = (L - nbuf).astype(np.int64)
            d["win_k"] = gen.device_bf16_normal((int(boff[-1]), 128),
                                                gen.seed_of(wl.cfg_id, li, gen.T_WIN_K), device=device)
            d["win_v"] = gen.device_bf16_normal((int(boff[-1]), 128),
                                                gen.seed_of(wl.cfg_id, li, gen.T_WIN_V), device=device)
            d["win_off_dev"] = torch.tensor(boff, device=device)
            d["win_pos0_dev"] = torch.tensor(d["win_pos0"], device=device)
        if wl.sink:   # per-head sink logits, fp32 N(0, 1)
            d["sink"] = gen.rng(wl.cfg_id, li, gen.T_SINK).standard_normal(H).astype(np.float32)
            d["sink_dev"] = torch.from_numpy(d["sink"]).to(device)
        layers.append(d)
    return L, layers


def decode_raw_inputs(wl: Workload, device="cuda", replicas: int = 1):
    """Raw K/V tokens N(0,1) for every sequence (to be compressed by the caller),
    plus, per replica r, indexer keys, indexer queries and queries (replica 0 uses
    the base seeds; others add r to the seed key)."""
    import torch

    L = lengths(wl)
    tok_off = offsets(L)
    T = int(tok_off[-1])
    raw_k = gen.device_bf16_normal((T, 128), gen.seed_of(wl.cfg_id, 0, gen.T_RAW_K), device=device)
    raw_v = gen.device_bf16_normal((T, 128), gen.seed_of(wl.cfg_id, 0, gen.T_RAW_V), device=device)
    ratio = wl.c if wl.kind == "csa_decode" else wl.m
    N = L // ratio
    ent_off = offsets(N)
    reps = []
    for r in range(replicas):
        d = dict(q=gen.device_bf16_normal((wl.batch, wl.heads, 128),
                                          gen.seed_of(wl.cfg_id, 0, gen.T_Q, r), device=device))
        if wl.kind == "csa_decode":
            if wl.idx_fp4:   # packed FP4 codes, 32 bytes per vector
                d["k_idx"] = gen.device_fp4_uniform((int(ent_off[-1]), 32),
                                                    gen.seed_of(wl.cfg_id, 0, gen.T_KFP4, r), device)
                d["q_idx"] = gen.device_fp4_uniform((wl.batch, 32),
                                                    gen.seed_of(wl.cfg_id, 0, gen.T_QFP4, r), device)
            else:
                d["k_idx"] = gen.device_int8_uniform((int(ent_off[-1]), 64),
                                                     gen.seed_of(wl.cfg_id, 0, gen.T_KIDX, r), device)
                d["q_idx"] = gen.device_int8_uniform((wl.batch, 64),
                                                     gen.seed_of(wl.cfg_id, 0, gen.T_QIDX, r), device)
        reps.append(d)
    return dict(L=L, tok_off=tok_off, raw_k=raw_k, raw_v=raw_v, ratio=ratio, N=N, ent_off=ent_off,
                tok_off_dev=torch.tensor(tok_off, device=device),
                ent_off_dev=torch.tensor(ent_off, device=device), replicas=reps)


def prefill_inputs(wl: Workload, device="cuda"):
    """Context raw tokens (ctx_len), the new raw tokens (new_tokens), indexer keys for
    all ctx/c + new/c entries, and per-new-token queries and indexer queries (packed FP4
    codes, 32 bytes per vector, for a workload with the FP4 indexer)."""
    ctx, new, c = wl.ctx_len, wl.new_tokens, wl.c
    n_ent = ctx // c + new // c
    return dict(
        raw_k_ctx=gen.device_bf16_normal((ctx, 128), gen.seed_of(wl.cfg_id, 0, gen.T_RAW_K),
                                         device=device),
        raw_v_ctx=gen.device_bf16_normal((ctx, 128), gen.seed_of(wl.cfg_id, 0, gen.T_RAW_V),
                                         device=device),
        new_k=gen.device_bf16_normal((new, 128), gen.seed_of(wl.cfg_id, 0, gen.T_NEW_K),
                                     device=device),
        new_v=gen.device_bf16_normal((new, 128), gen.seed_of(wl.cfg_id, 0, gen.T_NEW_V),
                                     device=device),
        k_idx=(gen.device_fp4_uniform((n_ent, 32), gen.seed_of(wl.cfg_id, 0, gen.T_KFP4), device)
               if wl.idx_fp4 else
               gen.device_int8_uniform((n_ent, 64), gen.seed_of(wl.cfg_id, 0, gen.T_KIDX), device)),
        q=gen.device_bf16_normal((new, wl.heads, 128), gen.seed_of(wl.cfg_id, 0, gen.T_Q),
                                 device=device),
        q_idx=(gen.device_fp4_uniform((new, 32), gen.seed_of(wl.cfg_id, 0, gen.T_QFP4), device)
               if wl.idx_fp4 else
               gen.device_int8_uniform((new, 64), gen.seed_of(wl.cfg_id, 0, gen.T_QIDX), device)),
        n_ent=n_ent,
    )
