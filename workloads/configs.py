"""Workload shapes.

The method ("DeepSeek-V4: Towards Highly Efficient Million-Token Context
Intelligence Review", dimensionstp.github.io, section 3-2 item 2, component and
config tables) fixes the compression ratios (4 tokens per CSA entry, 128 per
HCA entry) and the interleaving of CSA and HCA layers.  Batch sizes, context
lengths, head counts, top-k sizes, the pooling operator and the int8 indexer are
synthetic choices of the workload specification, reproduced here as data.
"""
from __future__ import annotations

from dataclasses import dataclass, field
from typing import Optional, Tuple


@dataclass(frozen=True)
class Workload:
    name: str
    cfg_id: int            # seed namespace
    kind: str              # csa_decode | hca_decode | hybrid_decode | csa_prefill
    batch: int
    ctx_len: Optional[int]              # fixed context length (tokens) or None when ragged
    ctx_range: Optional[Tuple[int, int]] = None   # inclusive range for ragged lengths
    heads: int = 64
    head_dim: int = 128
    c: int = 4             # CSA compression ratio
    m: int = 128           # HCA compression ratio
    topk: int = 2048
    d_idx: int = 64
    n_layers: int = 1
    new_tokens: int = 0    # prefill: query tokens appended after ctx_len
    direct_entries: bool = False   # draw compressed entries directly (no raw tokens)
    window: int = 0        # sliding-window branch: raw tokens before the query (0: none)
    sink: bool = False     # per-head attention-sink logits on every layer
    idx_fp4: bool = False  # FP4 (E2M1) indexer query / keys instead of int8
    kv8: bool = False      # mixed KV rows: dims 0..63 FP8 E4M3, dims 64..127 bf16
    notes: str = field(default="", compare=False)

    @property
    def scale(self) -> float:
        return 1.0 / float(self.head_dim) ** 0.5


WORKLOADS = {
    # single-sequence CSA decode over an 8K context
    "csa_decode_8k": Workload(
        name="csa_decode_8k", cfg_id=0, kind="csa_decode", batch=1, ctx_len=8192,
        heads=16, topk=256),
    # HCA decode, 8 sequences of 128K tokens
    "hca_decode_128k": Workload(
        name="hca_decode_128k", cfg_id=1, kind="hca_decode", batch=8, ctx_len=131072,
        heads=64),
    # CSA decode, 4 sequences of 1M tokens
    "csa_decode_1m": Workload(
        name="csa_decode_1m", cfg_id=2, kind="csa_decode", batch=4, ctx_len=1048576,
        heads=64, topk=2048),
    # the same with the FP4 indexer (32 B per key instead of 64)
    "csa_decode_1m_fp4": Workload(
        name="csa_decode_1m_fp4", cfg_id=2, kind="csa_decode", batch=4, ctx_len=1048576,
        heads=64, topk=2048, idx_fp4=True),
    # 8-layer hybrid stack (CSA on even layers, HCA on odd), 16 ragged sequences
    "hybrid_decode_1m": Workload(
        name="hybrid_decode_1m", cfg_id=3, kind="hybrid_decode", batch=16, ctx_len=None,
        ctx_range=(65536, 1048576), heads=64, topk=2048, n_layers=8, direct_entries=True,
        notes="compressed entries drawn directly as bf16 N(0, 1/ratio)"),
    # the same stack with the sliding-window branch (128 raw tokens) on every layer
    "hybrid_decode_1m_swa": Workload(
        name="hybrid_decode_1m_swa", cfg_id=3, kind="hybrid_decode", batch=16, ctx_len=None,
        ctx_range=(65536, 1048576), heads=64, topk=2048, n_layers=8, direct_entries=True,
        window=128,
        notes="compressed entries drawn directly as bf16 N(0, 1/ratio); state buffers of the "
              "last 128 raw tokens drawn as bf16 N(0, 1)"),
    # the same stack with the window branch and an attention sink on every layer: the
    # attention as the method lists it (compressed entries, window, sink)
    "hybrid_decode_1m_swa_sink": Workload(
        name="hybrid_decode_1m_swa_sink", cfg_id=3, kind="hybrid_decode", batch=16, ctx_len=None,
        ctx_range=(65536, 1048576), heads=64, topk=2048, n_layers=8, direct_entries=True,
        window=128, sink=True,
        notes="compressed entries drawn directly as bf16 N(0, 1/ratio); state buffers of the "
              "last 128 raw tokens drawn as bf16 N(0, 1); sink logits fp32 N(0, 1) per head"),
    # the stack with the FP4 indexer on its CSA layers (packed E2M1 codes, 32 B per key)
    "hybrid_decode_1m_fp4": Workload(
        name="hybrid_decode_1m_fp4", cfg_id=3, kind="hybrid_decode", batch=16, ctx_len=None,
        ctx_range=(65536, 1048576), heads=64, topk=2048, n_layers=8, direct_entries=True,
        idx_fp4=True,
        notes="compressed entries drawn directly as bf16 N(0, 1/ratio); FP4 indexer codes "
              "uniform over the 16 E2M1 codes"),
    # the stack over mixed KV storage rows (FP8 for dims 0..63, bf16 for the RoPE dims)
    "hybrid_decode_1m_kv8": Workload(
        name="hybrid_decode_1m_kv8", cfg_id=3, kind="hybrid_decode", batch=16, ctx_len=None,
        ctx_range=(65536, 1048576), heads=64, topk=2048, n_layers=8, direct_entries=True,
        kv8=True,
        notes="compressed entries drawn directly as N(0, 1/ratio), stored as 192-byte mixed "
              "rows (FP8 E4M3 dims 0..63, bf16 dims 64..127)"),
    # CSA chunked prefill: 4096 new tokens after a 256K context
    "csa_prefill_256k": Workload(
        name="csa_prefill_256k", cfg_id=4, kind="csa_prefill", batch=1, ctx_len=262144,
        heads=64, topk=2048, new_tokens=4096),
    # the same chunk with the FP4 indexer (packed E2M1 query and key codes)
    "csa_prefill_256k_fp4": Workload(
        name="csa_prefill_256k_fp4", cfg_id=4, kind="csa_prefill", batch=1, ctx_len=262144,
        heads=64, topk=2048, new_tokens=4096, idx_fp4=True,
        notes="FP4 indexer codes uniform over the 16 E2M1 codes"),
}


def get(name: str) -> Workload:
    return WORKLOADS[name]
