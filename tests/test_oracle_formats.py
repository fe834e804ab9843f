"""Pins of the oracle's number formats against the pages' printed constants,
hand-worked values and torch's independent casts."""

import os

import numpy as np
import pytest
import torch

from oracle import formats as F
from conftest import GOLDEN


def _read_golden(name):
    rows = []
    with open(os.path.join(GOLDEN, name)) as f:
        for line in f:
            line = line.strip()
            if line and not line.startswith("#"):
                rows.append(line.split())
    return rows


# ---------------------------------------------------------------- E4M3FN


def test_e4m3_grid_constants():
    v = F.E4M3_VALUES
    assert F.E4M3_MAX == 448.0  # "E4M3 max 448"
    assert v[0x7E] == 448.0 and v[0xFE] == -448.0
    assert np.isnan(v[0x7F]) and np.isnan(v[0xFF])
    assert np.isfinite(v).sum() == 254
    assert v[0x01] == 2.0 ** -9 and v[0x08] == 2.0 ** -6 and v[0x38] == 1.0
    pos = v[:0x7F]
    assert np.all(np.diff(pos) > 0)
    # sign bit flips sign only
    assert np.array_equal(v[0x80:0xFF], -v[0x00:0x7F])


def test_e4m3_hand_worked():
    for u, code, val in _read_golden("e4m3_scale1.txt"):
        c = int(F.e4m3_encode(np.float64(float(u))))
        assert c == int(code, 16), (u, hex(c), code)
        assert F.e4m3_decode(c) == float(val)
        assert np.signbit(F.e4m3_decode(c)) == val.startswith("-")


def test_e4m3_all_bf16_values_vs_torch():
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    with np.errstate(invalid="ignore"):
        vals = F.bf16_from_bits(bits).astype(np.float64)
    ok = np.isfinite(vals) & (np.abs(vals) <= 448.0)
    u = vals[ok]
    ours = F.e4m3_encode(u)
    ref = torch.from_numpy(u.astype(np.float32)).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(ours, ref)
    # beyond 448 every finite value saturates
    big = vals[np.isfinite(vals) & (np.abs(vals) > 448.0)]
    codes = F.e4m3_encode(big)
    assert np.all((codes == 0x7E) | (codes == 0xFE))


def test_e4m3_random_f32_vs_torch():
    g = np.random.default_rng(1)
    u = (g.standard_normal(200000) * np.exp(g.uniform(-14, 6, 200000))).astype(np.float32)
    u = np.clip(u, -448, 448)
    ours = F.e4m3_encode(u.astype(np.float64))
    ref = torch.from_numpy(u).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(ours, ref)


def test_e4m3_brute_force_nearest():
    """Nearest-value search over the whole signed table (independent of the
    sorted-grid search the encoder uses)."""
    g = np.random.default_rng(2)
    u = g.uniform(-500, 500, 3000)
    u = np.concatenate([u, g.uniform(-0.05, 0.05, 3000)])
    table = F.E4M3_VALUES
    finite = np.where(np.isfinite(table))[0]
    for x in u:
        d = np.abs(table[finite] - min(max(x, -448.0), 448.0))
        best = finite[d == d.min()]
        best = [c for c in best if np.signbit(table[c]) == np.signbit(x) or table[c] != 0]
        if len(best) > 1:  # tie: even mantissa
            best = [c for c in best if (c & 1) == 0]
        assert int(F.e4m3_encode(x)) == best[0], x


# ---------------------------------------------------------------- E2M1 / E8M0


def test_e2m1_grid_constants():
    pos = F.E2M1_VALUES[:8]
    assert list(pos) == [0, 0.5, 1, 1.5, 2, 3, 4, 6]
    assert F.E2M1_MAX == 6.0  # "max 6"
    assert F.E2M1_EMAX == 2 and 6.0 == 1.5 * 2.0 ** F.E2M1_EMAX  # "emax=2"
    assert np.array_equal(F.E2M1_VALUES[8:], -pos)


def test_e2m1_ties_and_saturation():
    # ties go to the even code
    cases = {0.25: 0, 0.75: 2, 1.25: 2, 1.75: 4, 2.5: 4, 3.5: 6, 5.0: 6,
             0.3: 1, 2.6: 5, 5.1: 7, 6.0: 7, 7.9: 7, 100.0: 7}
    for v, c in cases.items():
        assert int(F.e2m1_encode(v)) == c, v
        assert int(F.e2m1_encode(-v)) == c | 8, v
    assert int(F.e2m1_encode(-0.0)) == 8
    assert int(F.e2m1_encode(-0.1)) == 8


def test_e8m0_decode():
    assert F.e8m0_decode(127) == 1.0
    assert F.e8m0_decode(0) == 2.0 ** -127
    assert F.e8m0_decode(254) == 2.0 ** 127
    assert np.isnan(F.e8m0_decode(255))


# ---------------------------------------------------------------- INT8 / bf16


def test_int8_hand_worked_and_range():
    for x, c in _read_golden("int8_scale1.txt"):
        assert int(F.int8_encode(float(x))) == int(c), x
    codes = F.int8_encode(np.linspace(-1000, 1000, 10001))
    assert codes.min() == -128 and codes.max() == 127


def test_bf16_round_vs_torch():
    g = np.random.default_rng(3)
    x = (g.standard_normal(300000) * np.exp(g.uniform(-80, 80, 300000))).astype(np.float32)
    x = np.concatenate([x, np.float32([0.0, -0.0, 1.0, 1.00390625, 1.005859375, 3e38, 1e-40])])
    ref = torch.from_numpy(x).to(torch.bfloat16).to(torch.float32).numpy()
    ours = F.bf16_round(x.astype(np.float64)).astype(np.float32)
    assert np.array_equal(ours.view(np.uint32), ref.view(np.uint32))


def test_bf16_round_single_rounding_from_fp64():
    # 1 + 2^-8 + 2^-30 must round up in one step (a detour through float32
    # would first drop the 2^-30 and then tie to even, rounding down).
    x = 1.0 + 2.0 ** -8 + 2.0 ** -30
    assert F.bf16_round(x) == 1.0 + 2.0 ** -7
    assert F.bf16_round(1.0 + 2.0 ** -8) == 1.0
