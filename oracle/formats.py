"""Number formats of the FA quantization modes, built from their bit layouts.

TEST INFRASTRUCTURE ONLY (see ``oracle/__init__``).

Each grid is built by enumerating every code of the format and decoding its
bit fields; encoders pick the nearest grid value by search over that table,
with ties sent to the code whose least-significant mantissa bit is 0.

Pins (tests/test_oracle_formats.py):
* E4M3FN: largest finite value 448 (msModelSlim "FA 量化" page, 分支组合 /
  组合 2: "E4M3 max 448"; the MindIE SD "量化" page, FA量化 / 块量化 names the
  type ``float8_e4m3fn``); encoder cross-checked against torch's independent
  ``float8_e4m3fn`` cast on every bf16 value with |u| <= 448.
* E2M1: largest value 6 and largest exponent 2 ("FA 量化" page, 组合 3:
  "emax=2, max 6"); E8M0 shared exponent for blocks of 32 (same passage).
* INT8: code range [-128, 127] (MindIE SD "量化" page, Linear量化 / 通用原理,
  the INT8 mapping figure), symmetric with no offset ("FA 量化" page, 组合 1).
* bf16 rounding cross-checked against torch's bf16 cast of float32 values.
"""

import numpy as np

# --------------------------------------------------------------------------
# FP8 E4M3FN: 1 sign, 4 exponent (bias 7), 3 mantissa bits; no infinities;
# S.1111.111 is NaN.  Subnormals: exponent field 0 -> m/8 * 2^-6.
# --------------------------------------------------------------------------


def _e4m3_decode_code(code: int) -> float:
    sign = -1.0 if code & 0x80 else 1.0
    e = (code >> 3) & 0xF
    m = code & 0x7
    if e == 0xF and m == 0x7:
        return float("nan")
    if e == 0:
        return sign * (m / 8.0) * 2.0 ** -6
    return sign * (1.0 + m / 8.0) * 2.0 ** (e - 7)


E4M3_VALUES = np.array([_e4m3_decode_code(c) for c in range(256)], dtype=np.float64)
# Non-negative finite codes 0x00..0x7E are increasing in value.
_E4M3_POS = E4M3_VALUES[:0x7F].copy()
E4M3_MAX = float(_E4M3_POS[-1])  # 448.0
E4M3_EMAX = 8  # exponent of the largest normal (448 = 1.75 * 2^8)


def _nearest_code(a: np.ndarray, grid: np.ndarray) -> np.ndarray:
    """Index of the grid value nearest to each a >= 0 (grid ascending,
    index == code), ties to the even index, saturating at the last entry."""
    a = np.asarray(a, dtype=np.float64)
    n = grid.size
    hi = np.clip(np.searchsorted(grid, a, side="left"), 0, n - 1)
    lo = np.clip(hi - 1, 0, n - 1)
    dlo = np.abs(a - grid[lo])
    dhi = np.abs(grid[hi] - a)
    pick_hi = (dhi < dlo) | ((dhi == dlo) & (hi % 2 == 0))
    idx = np.where(pick_hi, hi, lo)
    idx = np.where(a >= grid[-1], n - 1, idx)
    return idx.astype(np.int64)


def e4m3_encode(u) -> np.ndarray:
    """Nearest E4M3FN code (uint8) to each value u, round half to even,
    |u| > 448 saturating to +-448 (0x7E / 0xFE), sign kept (so -0 and tiny
    negatives give 0x80).  NaN input is rejected."""
    u = np.asarray(u, dtype=np.float64)
    if np.isnan(u).any():
        raise ValueError("NaN input to e4m3_encode")
    code = _nearest_code(np.abs(u), _E4M3_POS)
    sign = np.signbit(u).astype(np.int64) << 7
    return (code | sign).astype(np.uint8)


def e4m3_decode(code) -> np.ndarray:
    return E4M3_VALUES[np.asarray(code, dtype=np.uint8)]


def e4m3_neighbors(a):
    """For a >= 0: the two adjacent non-negative E4M3 values (lo <= a <= hi)
    and the midpoint between them; used for the tie allowance."""
    a = np.asarray(a, dtype=np.float64)
    hi = np.clip(np.searchsorted(_E4M3_POS, a, side="left"), 1, _E4M3_POS.size - 1)
    lo = hi - 1
    return _E4M3_POS[lo], _E4M3_POS[hi]


# --------------------------------------------------------------------------
# E2M1 (FP4): 1 sign, 2 exponent (bias 1), 1 mantissa bit.
# Exponent field 0 is subnormal: m/2 * 2^0.
# --------------------------------------------------------------------------


def _e2m1_decode_code(code: int) -> float:
    sign = -1.0 if code & 0x8 else 1.0
    e = (code >> 1) & 0x3
    m = code & 0x1
    if e == 0:
        return sign * (m / 2.0)
    return sign * (1.0 + m / 2.0) * 2.0 ** (e - 1)


E2M1_VALUES = np.array([_e2m1_decode_code(c) for c in range(16)], dtype=np.float64)
_E2M1_POS = E2M1_VALUES[:8].copy()  # 0, .5, 1, 1.5, 2, 3, 4, 6
E2M1_MAX = float(_E2M1_POS[-1])  # 6.0
E2M1_EMAX = 2  # exponent of the largest normal (6 = 1.5 * 2^2)


def e2m1_encode(v) -> np.ndarray:
    """Nearest E2M1 code (0..15) to v, ties to even code, |v| > 6 saturating
    to 6, sign in bit 3 (sign kept: -0 -> 0x8)."""
    v = np.asarray(v, dtype=np.float64)
    if np.isnan(v).any():
        raise ValueError("NaN input to e2m1_encode")
    code = _nearest_code(np.abs(v), _E2M1_POS)
    sign = np.signbit(v).astype(np.int64) << 3
    return (code | sign).astype(np.uint8)


def e2m1_decode(code) -> np.ndarray:
    return E2M1_VALUES[np.asarray(code, dtype=np.uint8) & 0xF]


def e2m1_neighbors(a):
    a = np.asarray(a, dtype=np.float64)
    hi = np.clip(np.searchsorted(_E2M1_POS, a, side="left"), 1, _E2M1_POS.size - 1)
    lo = hi - 1
    return _E2M1_POS[lo], _E2M1_POS[hi]


# --------------------------------------------------------------------------
# E8M0: an unsigned power-of-two exponent, bias 127; 0xFF is NaN.
# --------------------------------------------------------------------------


def e8m0_decode(byte) -> np.ndarray:
    b = np.asarray(byte, dtype=np.int64)
    out = np.ldexp(1.0, b - 127).astype(np.float64)
    return np.where(b == 255, np.nan, out)


# --------------------------------------------------------------------------
# INT8, symmetric: code = clip(round_half_even(u), -128, 127).
# --------------------------------------------------------------------------


def int8_encode(u) -> np.ndarray:
    u = np.asarray(u, dtype=np.float64)
    return np.clip(np.rint(u), -128, 127).astype(np.int8)


# --------------------------------------------------------------------------
# fp32 / bf16 rounding.
# --------------------------------------------------------------------------


def fl32(x) -> np.ndarray:
    """Round to float32 (IEEE round to nearest even)."""
    return np.asarray(x, dtype=np.float64).astype(np.float32)


def bf16_round(x) -> np.ndarray:
    """Round real values (given in fp64) once to the nearest bf16 value
    (8 significant bits, round half to even); returned as float64."""
    x = np.asarray(x, dtype=np.float64)
    _, e = np.frexp(x)  # x = m * 2^e, 0.5 <= |m| < 1
    e = np.maximum(e, -125)  # below 2^-126 the quantum is the subnormal 2^-133
    quantum = np.ldexp(1.0, e - 8)
    r = np.rint(x / quantum) * quantum
    big = np.abs(r) > 3.3895313892515355e38
    return np.where(big, np.copysign(np.inf, x), r)


def bf16_bits(x) -> np.ndarray:
    """uint16 bit patterns of bf16-representable float values."""
    f = np.asarray(x, dtype=np.float32)
    return (f.view(np.uint32) >> 16).astype(np.uint16)


def bf16_from_bits(b) -> np.ndarray:
    b = np.asarray(b, dtype=np.uint16).astype(np.uint32) << 16
    return b.view(np.float32)
