"""Seeded generators.

Every stream is keyed by (workload id, layer, tensor id) through numpy's
SeedSequence, so any tensor can be regenerated on its own.  Tensor ids:

    0 raw K tokens     1 raw V tokens     2 indexer keys      3 queries
    4 indexer queries  5 context lengths  6 compressed K (direct)
    7 compressed V (direct)  8 new raw K (prefill)  9 new raw V (prefill)
    10, 11 window state K / V   12 sink logits   13 FP4 indexer keys   14 FP4 indexer queries

Host generation (numpy PCG64) is exact and reproducible on any CPU; it is what
the parity tests use.  The device generators (torch Philox on the GPU) exist
for inputs of several GiB that numpy would take minutes to draw; they are
seeded from the same SeedSequence and their values are read back to the host
whenever the oracle needs them.
"""
from __future__ import annotations

import numpy as np

T_RAW_K, T_RAW_V, T_KIDX, T_Q, T_QIDX, T_LEN, T_CMP_K, T_CMP_V, T_NEW_K, T_NEW_V = range(10)
T_WIN_K, T_WIN_V = 10, 11   # sliding-window state buffers (raw tokens)
T_SINK = 12                  # per-head attention-sink logits
T_KFP4, T_QFP4 = 13, 14       # FP4 indexer keys / queries (packed E2M1 codes)


def seed_of(cfg_id: int, layer: int, tensor_id: int, replica: int = 0) -> int:
    key = [cfg_id, layer, tensor_id] + ([replica] if replica else [])
    return int(np.random.SeedSequence(key).generate_state(1, dtype=np.uint64)[0] >> 1)


def rng(cfg_id: int, layer: int, tensor_id: int, replica: int = 0) -> np.random.Generator:
    key = [cfg_id, layer, tensor_id] + ([replica] if replica else [])
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence(key)))


def bf16_bits_from_f32(x: np.ndarray) -> np.ndarray:
    """Round float32 draws to bf16 storage (round to nearest, ties to even).

    Finite inputs only (the draws are Gaussian); returns uint16 bit patterns."""
    b = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32).astype(np.uint64)
    b = b + 0x7FFF + ((b >> 16) & 1)
    return (b >> 16).astype(np.uint16)


def bf16_normal(gen: np.random.Generator, shape, std: float = 1.0) -> np.ndarray:
    """bf16 bit patterns of N(0, std^2) draws."""
    x = gen.standard_normal(size=shape, dtype=np.float32)
    if std != 1.0:
        x = (x.astype(np.float64) * std).astype(np.float32)
    return bf16_bits_from_f32(x)


def int8_uniform(gen: np.random.Generator, shape) -> np.ndarray:
    """int8 uniform over the 255 integers -127..127 inclusive."""
    return gen.integers(-127, 128, size=shape, dtype=np.int8)


def _e4m3_table():
    """Non-negative finite FP8 E4M3 values by code 0..126 (exponent bias 7, 3 mantissa
    bits, subnormals below 2^-6); ascending in the code."""
    codes = np.arange(127)
    e, m = codes >> 3, codes & 7
    return np.where(e == 0, m * 2.0 ** -9, (1.0 + m / 8.0) * 2.0 ** (e - 7.0))


def fp8_e4m3_bits(x) -> np.ndarray:
    """Round to FP8 E4M3 codes: nearest value, ties to the even code, saturating at
    +-448 (the storage rounding of the mixed KV rows)."""
    x = np.asarray(x, dtype=np.float64)
    vals = _e4m3_table()
    a = np.minimum(np.abs(x), vals[-1])
    hi = np.clip(np.searchsorted(vals, a), 1, len(vals) - 1)
    lo = hi - 1
    dl, dh = a - vals[lo], vals[hi] - a
    pick = np.where(dl < dh, lo, np.where(dh < dl, hi, np.where(lo % 2 == 0, lo, hi)))
    return (pick | np.where(np.signbit(x), 128, 0)).astype(np.uint8)


def kv8_rows(x) -> np.ndarray:
    """Mixed KV rows [N, 192] uint8 from values [N, 128]: dims 0..63 as FP8 E4M3 codes,
    dims 64..127 as bf16 (little-endian)."""
    x = np.asarray(x, dtype=np.float32).reshape(-1, 128)
    lo = fp8_e4m3_bits(x[:, :64])
    hi = bf16_bits_from_f32(np.ascontiguousarray(x[:, 64:])).astype("<u2").view(np.uint8)
    return np.concatenate([lo, hi.reshape(-1, 128)], axis=1)


def kv8_normal(gen: np.random.Generator, n: int, std: float = 1.0) -> np.ndarray:
    """Mixed KV rows of N(0, std^2) float32 draws."""
    x = gen.standard_normal(size=(n, 128), dtype=np.float32)
    if std != 1.0:
        x = (x.astype(np.float64) * std).astype(np.float32)
    return kv8_rows(x)


def fp4_uniform(gen: np.random.Generator, shape) -> np.ndarray:
    """Packed FP4 codes: uint8 bytes uniform over 0..255, i.e. two codes per byte, each
    uniform over the 16 E2M1 codes."""
    return gen.integers(0, 256, size=shape, dtype=np.uint8)


def ragged_lengths(gen: np.random.Generator, n: int, lo: int, hi: int) -> np.ndarray:
    """n integers uniform over lo..hi inclusive."""
    return gen.integers(lo, hi + 1, size=n, dtype=np.int64)


# --------------------------------------------------------------------------------------
# device-side generation for multi-GiB inputs


def _torch_gen(seed: int, device):
    import torch

    g = torch.Generator(device=device)
    g.manual_seed(seed)
    return g


def device_bf16_normal(shape, seed: int, std: float = 1.0, device="cuda", out=None):
    """torch.bfloat16 tensor of N(0, std^2) draws made on the device (Philox).

    Drawn in slabs so the float32 staging buffer stays small."""
    import torch

    g = _torch_gen(seed, device)
    if out is None:
        out = torch.empty(shape, dtype=torch.bfloat16, device=device)
    flat = out.view(-1)
    slab = 1 << 26
    for s in range(0, flat.numel(), slab):
        e = min(flat.numel(), s + slab)
        tmp = torch.randn(e - s, generator=g, device=device, dtype=torch.float32)
        if std != 1.0:
            tmp.mul_(std)
        flat[s:e].copy_(tmp)
    return out


def device_int8_uniform(shape, seed: int, device="cuda"):
    import torch

    g = _torch_gen(seed, device)
    return torch.randint(-127, 128, shape, generator=g, device=device, dtype=torch.int8)


def device_fp4_uniform(shape, seed: int, device="cuda"):
    """Packed FP4 codes (uint8, two per byte, each uniform over the 16 codes), on the device."""
    import torch

    g = _torch_gen(seed, device)
    return torch.randint(0, 256, shape, generator=g, device=device, dtype=torch.uint8)


def device_kv8_normal(n: int, seed: int, std: float = 1.0, device="cuda"):
    """Mixed KV rows [n, 192] uint8 of N(0, std^2) draws made on the device: dims 0..63
    rounded to FP8 E4M3 (nearest even, saturating), dims 64..127 to bf16."""
    import torch

    g = _torch_gen(seed, device)
    out = torch.empty((n, 192), dtype=torch.uint8, device=device)
    slab = 1 << 19
    for s0 in range(0, n, slab):
        e = min(n, s0 + slab)
        x = torch.randn((e - s0, 128), generator=g, device=device, dtype=torch.float32)
        if std != 1.0:
            x.mul_(std)
        out[s0:e, :64] = x[:, :64].clamp(-448.0, 448.0).to(torch.float8_e4m3fn).view(torch.uint8)
        out[s0:e, 64:] = x[:, 64:].to(torch.bfloat16).contiguous().view(torch.uint8)
    return out
