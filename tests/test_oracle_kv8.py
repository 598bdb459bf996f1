"""Pins for the oracle's mixed KV storage rows (dims 0..63 FP8 E4M3, dims 64..127 bf16).

Witnesses: torch's float8_e4m3fn decoder on all 256 codes, values of the OCP E4M3
table, torch's bf16 decoder for the high half, hand-built rows, and the rounding
error bound of a round trip through the row encoder."""
import numpy as np
import torch

import oracle
from workloads import bf16_bits_from_f32, fp8_e4m3_bits, kv8_rows, rng


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
