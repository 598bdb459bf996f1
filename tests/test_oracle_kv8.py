"""Pins for the oracle's mixed KV storage rows (dims 0..63 FP8 E4M3, dims 64..127 bf16).

Witnesses: torch's float8_e4m3fn decoder on all 256 codes, values of the OCP E4M3
table, torch's bf16 decoder for the high half, hand-built rows, and the rounding
error bound of a round trip through the row encoder."""
import numpy as np
import torch

import oracle
from workloads import bf16_bits_from_f32, bf16_normal, fp8_e4m3_bits, kv8_rows, rng


def test_e4m3_against_torch_all_codes():
    v = oracle.fp8_e4m3_values(np.arange(256))
    t = torch.arange(256, dtype=torch.uint8).view(torch.float8_e4m3fn).double().numpy()
    nan = np.isnan(t)
    assert list(np.nonzero(nan)[0]) == [0x7F, 0xFF]
    assert np.array_equal(np.isnan(v), nan)
    assert np.array_equal(v[~nan], t[~nan])
    assert np.array_equal(np.signbit(v[~nan]), np.signbit(t[~nan]))


def test_e4m3_table_values():
    v = oracle.fp8_e4m3_values
    assert v(0x38) == 1.0 and v(0xB8) == -1.0 and v(0x7E) == 448.0 and v(0x40) == 2.0
    assert v(0x08) == 2.0 ** -6 and v(0x01) == 2.0 ** -9 and v(0x07) == 7 * 2.0 ** -9
    assert v(0x00) == 0.0 and np.signbit(v(0x80))


def test_rows_by_hand():
    row = np.zeros(192, np.uint8)
    row[0], row[63] = 0x38, 0xC0                      # dim 0 = 1.0, dim 63 = -2.0
    row[64:66] = [0x80, 0x3F]                         # dim 64 = bf16 0x3F80 = 1.0 (little-endian)
    row[190:192] = [0x40, 0xC0]                       # dim 127 = bf16 0xC040 = -3.0
    x = oracle.kv8_values(row[None])
    assert x.shape == (1, 128)
    assert x[0, 0] == 1.0 and x[0, 63] == -2.0 and x[0, 64] == 1.0 and x[0, 127] == -3.0
    assert np.count_nonzero(x) == 4


def test_high_half_matches_torch_bf16():
    g = rng(960, 0, 0)
    x = g.standard_normal((50, 128)).astype(np.float32)
    rows = kv8_rows(x)
    hi = torch.from_numpy(np.ascontiguousarray(rows[:, 64:])).view(torch.bfloat16).double().numpy()
    assert np.array_equal(oracle.kv8_values(rows)[:, 64:], hi)
    assert np.array_equal(rows[:, 64:].view("<u2"), bf16_bits_from_f32(np.ascontiguousarray(x[:, 64:])))


def test_round_trip_error_bound():
    g = rng(961, 0, 0)
    x = (g.standard_normal((400, 128)) * 0.5).astype(np.float32)
    d = oracle.kv8_values(kv8_rows(x))
    lo, xl = d[:, :64], x[:, :64].astype(np.float64)
    normal = np.abs(xl) >= 2.0 ** -6
    assert np.all(np.abs(lo - xl)[normal] <= np.abs(xl)[normal] * 2.0 ** -4)   # half an ulp, 3 bits
    assert np.all(np.abs(lo - xl)[~normal] <= 2.0 ** -10)                      # subnormal spacing / 2
    hi, xh = d[:, 64:], x[:, 64:].astype(np.float64)
    assert np.all(np.abs(hi - xh) <= np.abs(xh) * 2.0 ** -8)
    assert np.array_equal(fp8_e4m3_bits(np.array([1000.0, -1000.0])), np.array([0x7E, 0xFE], np.uint8))


# ------------------------------------------------------------------ the encoder
def test_e4m3_round_returns_every_finite_code():
    codes = np.array([c for c in range(256) if c & 0x7F != 0x7F])
    vals = oracle.fp8_e4m3_values(codes)
    assert np.array_equal(oracle.fp8_e4m3_round(vals), codes.astype(np.uint8))


def test_e4m3_round_midpoints_go_to_the_even_code():
    mags = oracle.fp8_e4m3_values(np.arange(0x7F))          # 0 .. 448, increasing
    for i in range(len(mags) - 1):
        mid = (mags[i] + mags[i + 1]) / 2
        want = i if i % 2 == 0 else i + 1
        assert oracle.fp8_e4m3_round(mid) == want, i
        assert oracle.fp8_e4m3_round(-mid) == want | 128, i
        eps = (mags[i + 1] - mags[i]) / 64
        assert oracle.fp8_e4m3_round(mid - eps) == i and oracle.fp8_e4m3_round(mid + eps) == i + 1


def test_e4m3_round_saturates_and_keeps_the_sign_of_zero():
    r = oracle.fp8_e4m3_round
    for x in (448.0, 449.0, 464.0, 480.0, 1e9, np.inf):
        assert r(x) == 0x7E and r(-x) == 0xFE
    assert r(0.0) == 0x00 and r(-0.0) == 0x80
    assert r(2.0 ** -11) == 0x00 and r(-(2.0 ** -11)) == 0x80   # below half the least subnormal
    assert r(2.0 ** -10) == 0x00                                 # exactly half: ties to even (0)
    assert r(3 * 2.0 ** -10) == 0x02                             # 1.5 subnormal steps: to 2
    assert r(3 * 2.0 ** -11) == 0x01                             # 0.75 of a step: to 1


def test_e4m3_round_matches_torch_in_range():
    """torch's float8_e4m3fn conversion rounds to nearest, ties to even, inside the
    finite range; float32 inputs make its float step exact."""
    g = rng(960, 0, 0)
    x = np.concatenate([g.standard_normal(20000) * s for s in (0.003, 0.05, 1.0, 30.0, 120.0)])
    x = np.clip(x, -440.0, 440.0).astype(np.float32)
    t = torch.from_numpy(x).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(oracle.fp8_e4m3_round(x.astype(np.float64)), t)


# ------------------------------------------------------------------ compression into mixed rows
def test_compress_kv8_constant_blocks_and_layout():
    x = np.zeros((8, 128))
    x[:4, 0], x[4:, 0] = 1.0, -2.0            # dim 0: blocks of 1.0 and -2.0
    x[:4, 64], x[4:, 127] = 1.0, -3.0         # dims 64 / 127 in the bf16 half
    rows = oracle.compress_to_cache_kv8(x, 4)
    assert rows.shape == (2, 192) and rows.dtype == np.uint8
    assert rows[0, 0] == 0x38 and rows[1, 0] == 0xC0
    assert list(rows[0, 64:66]) == [0x80, 0x3F] and list(rows[1, 190:192]) == [0x40, 0xC0]
    assert np.count_nonzero(rows) == 6


def test_compress_kv8_error_bound_and_tail():
    """Each stored value is the block mean rounded once: within half a step of the
    format at the mean's magnitude (FP8: 3 mantissa bits, bf16: 8), and the tail of
    T mod c tokens forms no row."""
    g = rng(961, 0, 0)
    x = oracle.bf16_bits_to_f64(bf16_normal(g, (4 * 50 + 3, 128), 2.0))
    rows = oracle.compress_to_cache_kv8(x, 4)
    assert rows.shape == (50, 192)
    mean = x[:200].reshape(50, 4, 128).mean(axis=1)
    got = oracle.kv8_values(rows)
    lo_err = np.abs(got[:, :64] - mean[:, :64])
    lo_bound = np.maximum(np.exp2(np.floor(np.log2(np.abs(mean[:, :64]) + 1e-300)) - 4), 2.0 ** -10)
    assert np.all(lo_err <= lo_bound)
    hi_err = np.abs(got[:, 64:] - mean[:, 64:])
    assert np.all(hi_err <= np.abs(mean[:, 64:]) * 2.0 ** -8 + 1e-300)
