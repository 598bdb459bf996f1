"""Composed steps over the C ABI: buffer allocation and call order only.

CsaStep   selection, then csa_sparse_attn.  Selection is csa_index_select (scores
          never written: its candidate form for decode, its sweep form for chunked
          prefill of 16 or more queries per sequence), or, with fused=False, the pair
          csa_index_score (with the fused first radix pass) -> csa_topk_select; the
          FP4 indexer takes the _fp4 forms of the same calls.
HcaStep   hca_dense_attn.
HybridStep  hybrid_layer_step over a list of CSA / HCA layers.

Buffers are allocated once per shape; every call after that only enqueues
kernels on the current stream.
"""
from __future__ import annotations

import torch

from . import (LCA_IDX_FP4, LCA_IDX_INT8, LCA_KV_BF16, LCA_KV_MIXED, LCA_LAYER_CSA, LCA_LAYER_HCA,
               attn_workspace_bytes, csa_index_score, csa_index_score_fp4, csa_index_select,
               csa_index_select_fp4, csa_index_select_workspace_bytes,
               csa_sparse_attn, csa_sparse_attn_kv8, csa_topk_select, csa_topk_workspace_bytes,
               hca_dense_attn, hca_dense_attn_kv8, hybrid_layer_step, hybrid_workspace_bytes,
               make_layers, workspace)


SELECT_MIN_Q = 16   # query tokens per sequence from which csa_index_select applies


def _round4(n: int) -> int:
    return max(4, (n + 3) // 4 * 4)


class CsaStep:
    """fused: True (default) selects with csa_index_select; False with the two-call
    path, which materialises the scores in self.scores.  fp4: the
    indexer query / keys are packed FP4 codes (the _fp4 scoring and selection calls);
    kv8: the cache holds mixed FP8 / bf16 rows (csa_sparse_attn_kv8)."""

    def __init__(self, batch, max_q, max_entries, heads, topk, c, device="cuda", splits=0,
                 fused=None, fp4=False, kv8=False):
        self.batch, self.max_q, self.max_entries = batch, max_q, max_entries
        self.heads, self.topk, self.c, self.splits = heads, topk, c, splits
        rows = batch * max_q
        self.rows = rows
        self.fp4, self.kv8 = fp4, kv8
        self.fused = True if fused is None else fused
        self.n_vis = torch.empty(rows, dtype=torch.int32, device=device)
        self.idx = torch.empty(rows, topk, dtype=torch.int32, device=device)
        self.count = torch.empty(rows, dtype=torch.int32, device=device)
        if self.fused:
            self.sws = workspace(csa_index_select_workspace_bytes(batch, max_q, max_entries, topk),
                                 device)
        else:
            self.scores = torch.empty(rows, _round4(max_entries), dtype=torch.int32,
                                      device=device)
            self.tws = workspace(csa_topk_workspace_bytes(rows, max_entries, topk), device)
        self.aws = workspace(attn_workspace_bytes(rows, heads, max_q, splits), device)

    def select(self, q_idx, q_off, q_pos, k_idx, ent_off, stream=None):
        if self.fused:
            sel = csa_index_select_fp4 if self.fp4 else csa_index_select
            sel(q_idx, q_off, q_pos, k_idx, ent_off, self.batch, self.max_q, self.max_entries,
                self.c, self.topk, self.idx, self.count, self.n_vis, ws=self.sws, stream=stream)
            return
        score = csa_index_score_fp4 if self.fp4 else csa_index_score
        score(q_idx, q_off, q_pos, k_idx, ent_off, self.batch, self.max_q, self.max_entries,
              self.c, self.scores, self.n_vis, ws=self.tws, stream=stream)
        csa_topk_select(self.scores, self.rows, self.max_entries, self.n_vis, self.topk, self.idx,
                        self.count, self.tws, hist_ready=True, stream=stream)

    def attend(self, q, k_cmp, v_cmp, ent_off, q_off, scale, out, lse=None, stream=None):
        attn = csa_sparse_attn_kv8 if self.kv8 else csa_sparse_attn
        attn(q, k_cmp, v_cmp, ent_off, q_off, self.batch, self.max_q, self.idx, self.count,
             self.topk, scale, out, lse, ws=self.aws, splits=self.splits, stream=stream)

    def run(self, q, q_idx, q_off, q_pos, k_idx, k_cmp, v_cmp, ent_off, scale, out, lse=None,
            stream=None):
        self.select(q_idx, q_off, q_pos, k_idx, ent_off, stream)
        self.attend(q, k_cmp, v_cmp, ent_off, q_off, scale, out, lse, stream)


class HcaStep:
    """kv8: the cache holds mixed rows (hca_dense_attn_kv8)."""

    def __init__(self, batch, max_q, max_entries, heads, m, device="cuda", splits=0, kv8=False):
        self.batch, self.max_q, self.max_entries, self.heads, self.m = batch, max_q, max_entries, heads, m
        self.splits, self.kv8 = splits, kv8
        self.aws = workspace(attn_workspace_bytes(batch * max_q, heads, max_q, splits), device)

    def run(self, q, k_cmp, v_cmp, ent_off, q_off, q_pos, scale, out, lse=None, stream=None):
        attn = hca_dense_attn_kv8 if self.kv8 else hca_dense_attn
        attn(q, k_cmp, v_cmp, ent_off, q_off, q_pos, self.batch, self.max_q, self.max_entries,
             self.m, scale, out, lse, ws=self.aws, splits=self.splits, stream=stream)


class HybridStep:
    """layers: dicts with kind, ratio, topk, max_entries and the layer's tensors
    (q, q_idx, k_cmp, v_cmp, k_idx, ent_off, out, lse), optionally a sliding window
    (win_k, win_v, win_off, win_pos0, window), per-head sink logits (sink) and, for CSA
    layers, idx_format (LCA_IDX_FP4: packed FP4 indexer codes), and kv_format (LCA_KV_MIXED:
    mixed FP8 / bf16 cache rows); idx / count of CSA layers are allocated here when absent."""

    def __init__(self, layers, batch, max_q, heads, device="cuda"):
        rows = batch * max_q
        self.layers = []
        for L in layers:
            L = dict(L)
            if L["kind"] == LCA_LAYER_CSA:
                L.setdefault("idx", torch.empty(rows, L["topk"], dtype=torch.int32, device=device))
                L.setdefault("count", torch.empty(rows, dtype=torch.int32, device=device))
            self.layers.append(L)
        self.arr = make_layers(self.layers)
        self.batch, self.max_q, self.heads = batch, max_q, heads
        self.ws = workspace(hybrid_workspace_bytes(self.arr, batch, max_q, heads), device)

    def run(self, q_off, q_pos, scale, head_dim=128, stream=None):
        hybrid_layer_step(self.arr, q_off, q_pos, self.batch, self.max_q, self.heads, head_dim,
                          scale, self.ws, stream=stream)


__all__ = ["CsaStep", "HcaStep", "HybridStep", "LCA_LAYER_CSA", "LCA_LAYER_HCA", "LCA_IDX_INT8",
           "LCA_IDX_FP4", "LCA_KV_BF16", "LCA_KV_MIXED"]
