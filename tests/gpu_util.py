"""Helpers for the GPU parity tests: host <-> device transfers and comparisons.

Parity bars (the workload's stated tolerances): indexer scores, n_vis, selected
index sets and counts bit-exact; compressed entries bit-exact (both sides round
an exact fp64 mean once); attention outputs within rel-L2 <= 1e-2 and
max-abs <= 2e-2 of the fp64 oracle, lse within 2e-2 absolute."""
import sys

import numpy as np
import torch

import oracle

REL_L2 = 1e-2
MAX_ABS = 2e-2
LSE_ABS = 2e-2
DEV = "cuda"


def step(msg: str):
    """Name the case before each GPU step, flushed, so a fault can be attributed."""
    print(f"[gpu-case] {msg}", flush=True)
    sys.stdout.flush()


def bf16_dev(bits: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).to(DEV)


def bf16_bits(t: torch.Tensor) -> np.ndarray:
    return t.detach().contiguous().view(torch.int16).cpu().numpy().view(np.uint16)


def bf16_vals(t: torch.Tensor) -> np.ndarray:
    return oracle.bf16_bits_to_f64(bf16_bits(t))


def i64_dev(a) -> torch.Tensor:
    return torch.tensor(np.asarray(a, dtype=np.int64), device=DEV)


def i8_dev(a: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(a)).to(DEV)


def offsets(counts) -> np.ndarray:
    return np.concatenate([[0], np.cumsum(np.asarray(counts, dtype=np.int64))]).astype(np.int64)


def assert_attn_close(got: np.ndarray, ref: np.ndarray, what: str):
    got = np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    err = got - ref
    den = np.linalg.norm(ref)
    rel = np.linalg.norm(err) / den if den > 0 else np.linalg.norm(err)
    mx = np.abs(err).max() if err.size else 0.0
    assert rel <= REL_L2 and mx <= MAX_ABS, f"{what}: rel-L2 {rel:.3e} max-abs {mx:.3e}"
    return rel, mx


def assert_lse_close(got: np.ndarray, ref: np.ndarray, what: str):
    got = np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    inf = np.isinf(ref)
    assert np.array_equal(np.isinf(got), inf) and np.all(got[inf] == ref[inf]), f"{what}: lse inf"
    if (~inf).any():
        d = np.abs(got[~inf] - ref[~inf]).max()
        assert d <= LSE_ABS, f"{what}: lse max diff {d:.3e}"
