"""Pins of the oracle's quantizers: hand-worked blocks, printed constants,
symmetry, scale counts, brute-force nearest codes, and rotation invariance."""

import os

import numpy as np
import pytest

from oracle import formats as F
from oracle import quantize as Q
from conftest import GOLDEN


def test_int8_per_head_scale1_golden():
    rows = []
    with open(os.path.join(GOLDEN, "int8_scale1.txt")) as f:
        rows = [l.split() for l in f if l.strip() and not l.startswith("#")]
    xs = np.array([float(r[0]) for r in rows], dtype=np.float32)
    want = np.array([int(r[1]) for r in rows])
    amax = np.float32([127.0])
    s = Q.int8_scales(amax)
    assert s[0] == 1.0
    codes = Q.quantize_int8_per_head(xs.reshape(1, 1, 1, -1), s)
    assert np.array_equal(codes.ravel(), want)


def test_int8_per_head_symmetric_no_offset_and_scale_count():
    g = np.random.default_rng(5)
    x = g.standard_normal((2, 3, 16, 64)).astype(np.float32)
    amax = Q.calibrate_amax(x)
    assert amax.shape == (3,)  # one scale per head ("overhead = number of heads")
    s = Q.int8_scales(amax)
    c = Q.quantize_int8_per_head(x, s)
    cn = Q.quantize_int8_per_head(-x, s)
    assert np.array_equal(cn.astype(int), -c.astype(int))  # no -128 reached within amax
    assert int(Q.quantize_int8_per_head(np.zeros((1, 3, 1, 64), np.float32), s).max()) == 0
    # the calibrated amax maps to +-127 exactly
    for h in range(3):
        assert np.abs(c[:, h]).max() == 127


def test_calibration_running_max():
    g = np.random.default_rng(6)
    a = g.standard_normal((1, 4, 8, 32)).astype(np.float32)
    b = 3 * g.standard_normal((2, 4, 8, 32)).astype(np.float32)
    run = Q.calibrate_amax(b, Q.calibrate_amax(a))
    assert np.array_equal(run, np.maximum(np.abs(a).max(axis=(0, 2, 3)), np.abs(b).max(axis=(0, 2, 3))))


def test_int8_brute_force_tiny():
    g = np.random.default_rng(7)
    x = g.standard_normal((1, 2, 4, 32)).astype(np.float32)
    s = np.float32([0.02, 0.05])  # scales small enough that some values clamp
    c = Q.quantize_int8_per_head(x, s)
    for h in range(2):
        for v, code in zip(x[0, h].ravel(), c[0, h].ravel()):
            u = np.float32(v) / s[h]
            cands = np.arange(-128, 128)
            d = np.abs(cands - float(u))
            best = cands[d == d.min()]
            if best.size > 1:
                best = best[best % 2 == 0]
            assert code == best[0]


def test_fp8_per_token_row_max_hits_448():
    g = np.random.default_rng(8)
    x = (g.standard_normal((1, 2, 64, 128)) * np.exp(g.standard_normal((1, 2, 64, 1)))).astype(np.float32)
    codes, s = Q.quantize_fp8_per_token(x)
    assert s.shape == (1, 2, 64)
    am = np.abs(x).argmax(axis=3)
    top = np.take_along_axis(codes, am[..., None], axis=3)[..., 0]
    assert np.all((top == 0x7E) | (top == 0xFE))
    # dequantization error bounded by half a step of the E4M3 grid (3 bits)
    deq = Q.dequantize_per_token(codes, s, F.e4m3_decode)
    rel = np.abs(deq - x) / np.maximum(np.abs(x), s[..., None] * 2.0 ** -6)
    assert rel.max() <= 2.0 ** -4 + 1e-12


def test_fp8_per_token_zero_row_and_sign():
    x = np.zeros((1, 1, 2, 64), np.float32)
    x[0, 0, 1, :] = -5e-4
    x[0, 0, 1, 0] = 448.0
    codes, s = Q.quantize_fp8_per_token(x)
    assert s[0, 0, 0] == 1.0 and np.all(codes[0, 0, 0] == 0)
    assert s[0, 0, 1] == 1.0
    assert codes[0, 0, 1, 0] == 0x7E
    assert np.all(codes[0, 0, 1, 1:] == 0x80)  # -5e-4 < 2^-10: signed zero


def test_fp8_per_token_brute_force_tiny():
    g = np.random.default_rng(9)
    x = (g.standard_normal((1, 1, 3, 32)) * 10).astype(np.float32)
    codes, s = Q.quantize_fp8_per_token(x)
    finite = np.where(np.isfinite(F.E4M3_VALUES))[0]
    for r in range(3):
        for v, code in zip(x[0, 0, r], codes[0, 0, r]):
            u = float(np.float32(v) / s[0, 0, r])
            d = np.abs(F.E4M3_VALUES[finite] - u)
            best = finite[d == d.min()]
            if best.size > 1:
                best = best[best % 2 == 0]
            assert code == best[0]


def _read_mx_golden():
    out = []
    with open(os.path.join(GOLDEN, "mxfp4_blocks.txt")) as f:
        for line in f:
            if not line.strip() or line.startswith("#"):
                continue
            vals, e8, codes, deq = [p.split() for p in line.split("|")]
            out.append(([float(v) for v in vals], int(e8[0]),
                        [int(c, 16) for c in codes], [float(d) for d in deq]))
    return out


def test_mxfp4_golden_blocks():
    for vals, e8, codes, deq in _read_mx_golden():
        x = np.zeros((1, 1, 1, 32), np.float32)
        x[0, 0, 0, :len(vals)] = vals
        packed, e = Q.quantize_mxfp4(x)
        assert e.ravel()[0] == e8
        un = Q.unpack_fp4(packed).ravel()
        assert list(un[:len(codes)]) == codes
        assert np.all(un[len(codes):] == 0)
        d = Q.dequantize_mxfp4(packed, e).ravel()
        assert np.array_equal(d[:len(deq)], np.array(deq))
        assert list(np.signbit(d[:len(deq)])) == [s.startswith("-") for s in map(str, deq)]


def test_mxfp4_exponent_rule_pins_emax2_max6():
    g = np.random.default_rng(10)
    x = (g.standard_t(4, (2, 3, 17, 128)) * np.exp2(g.integers(-20, 20, (2, 3, 17, 1)))).astype(np.float32)
    packed, e8 = Q.quantize_mxfp4(x)
    E = e8.astype(np.int64) - 127
    amax = np.abs(x.reshape(2, 3, 17, 4, 32)).max(axis=4)
    # amax in [4, 8) * 2^E  (E = floor(log2 amax) - 2)
    assert np.all(amax >= 4.0 * np.exp2(E)) and np.all(amax < 8.0 * np.exp2(E))
    codes = Q.unpack_fp4(packed).reshape(2, 3, 17, 4, 32)
    top = np.take_along_axis(codes, np.abs(x.reshape(2, 3, 17, 4, 32)).argmax(axis=4)[..., None], axis=4)
    assert np.all(np.isin(top & 7, [6, 7]))  # block max lands on 4 or 6 (max 6)
    deq = Q.dequantize_mxfp4(packed, e8)
    assert np.all(np.abs(deq).reshape(2, 3, 17, 4, 32).max(axis=4) <= 6.0 * np.exp2(E))


def test_mxfp4_zero_block_and_tiny():
    x = np.zeros((1, 1, 1, 64), np.float32)
    x[0, 0, 0, 32] = 1e-40  # subnormal amax: exponent clamps to -127
    packed, e8 = Q.quantize_mxfp4(x)
    assert list(e8.ravel()) == [0, 0]
    assert np.all(Q.unpack_fp4(packed) == 0)


def test_mxfp4_brute_force_tiny():
    g = np.random.default_rng(11)
    x = g.standard_t(4, (1, 1, 2, 64)).astype(np.float32)
    packed, e8 = Q.quantize_mxfp4(x)
    codes = Q.unpack_fp4(packed)
    for r in range(2):
        for b in range(2):
            blk = x[0, 0, r, 32 * b:32 * b + 32].astype(np.float64)
            scale = 2.0 ** (int(e8[0, 0, r, b]) - 127)
            for v, c in zip(blk, codes[0, 0, r, 32 * b:32 * b + 32]):
                d = np.abs(F.E2M1_VALUES * scale - min(max(v, -6 * scale), 6 * scale))
                best = np.where(d == d.min())[0]
                best = [k for k in best if np.signbit(F.E2M1_VALUES[k]) == np.signbit(v) or F.E2M1_VALUES[k] != 0]
                if len(best) > 1:
                    best = [k for k in best if k % 2 == 0]
                assert c == best[0]


def test_rotation_identity_permutation_and_invariance():
    g = np.random.default_rng(12)
    x = F.bf16_round(g.standard_normal((1, 2, 8, 64))).astype(np.float32)
    assert np.array_equal(Q.rotate(x, np.eye(64)), x)
    perm = np.eye(64)[g.permutation(64)]
    assert np.array_equal(Q.rotate(x, perm), x @ perm)
    # orthogonal R leaves Q K^T unchanged (before the bf16 rounding)
    a = g.standard_normal((64, 64))
    r, _ = np.linalg.qr(a)
    q = g.standard_normal((5, 64))
    k = g.standard_normal((7, 64))
    assert np.allclose((q @ r) @ (k @ r).T, q @ k.T, atol=1e-12)
    # rotate rounds once to bf16: within half a bf16 ulp of the exact product
    y = Q.rotate(x, r)
    exact = x.astype(np.float64) @ r
    ulp = np.exp2(np.floor(np.log2(np.abs(exact))) - 7)
    assert np.all(np.abs(y - exact) <= 0.5 * ulp + 1e-30)


def test_fp8_block_quant():
    g = np.random.default_rng(13)
    y = g.standard_normal((2, 3, 300, 64)).astype(np.float32)
    codes, s = Q.quantize_fp8_block(y, 128)
    assert s.shape == (2, 3, 3)  # 128 + 128 + 44: the partial last block is its own
    for i, sl in enumerate([slice(0, 128), slice(128, 256), slice(256, 300)]):
        am = np.abs(y[:, :, sl]).max(axis=(2, 3))
        assert np.array_equal(s[:, :, i], (am / np.float32(448)).astype(np.float32))
    # block of one token is per-token quantization
    c1, s1 = Q.quantize_fp8_block(y, 1)
    c2, s2 = Q.quantize_fp8_per_token(y)
    assert np.array_equal(c1, c2) and np.array_equal(s1, s2)


def test_correctly_rounded_divide_at_ties():
    with open(os.path.join(GOLDEN, "divide_ties.txt")) as f:
        rows = [l.split() for l in f if l.strip() and not l.startswith("#")]
    for mode, amax, x, want in rows:
        if mode == "int8":
            s = Q.int8_scales(np.float32([float(amax)]))
            c = int(Q.quantize_int8_per_head(np.float32([[[[float(x)]]]]), s).ravel()[0])
            assert c == int(want), (x, c)
        else:
            row = np.zeros((1, 1, 1, 32), np.float32)
            row[0, 0, 0, 0] = float(amax)
            row[0, 0, 0, 1] = float(x)
            codes, s = Q.quantize_fp8_per_token(row)
            assert int(codes.ravel()[1]) == int(want, 16), (x, hex(codes.ravel()[1]))


# ---- sibling FA modes: FP8 per-head static, INT8 per-token dynamic, MXFP8


def test_fp8_per_head_calibrated_max_and_saturation():
    g = np.random.default_rng(14)
    x = g.standard_normal((2, 3, 16, 64)).astype(np.float32)
    s = Q.fp8_scales(Q.calibrate_amax(x))
    c = Q.quantize_fp8_per_head(x, s)
    # the calibrated maximum of every head encodes to +-448 exactly
    for h in range(3):
        top = c[:, h].ravel()[np.abs(x[:, h]).argmax()]
        assert top in (0x7E, 0xFE)
    # symmetric: negation flips only the sign bit
    assert np.array_equal(Q.quantize_fp8_per_head(-x, s), c ^ 0x80)
    # beyond the calibrated range codes saturate at 448 (no NaN code)
    big = np.full((1, 3, 1, 64), 1e6, np.float32)
    assert np.all(Q.quantize_fp8_per_head(big, s) == 0x7E)
    assert np.all(Q.quantize_fp8_per_head(-big, s) == 0xFE)


def test_fp8_per_head_brute_force_tiny():
    g = np.random.default_rng(15)
    x = (g.standard_normal((1, 2, 3, 32)) * 4).astype(np.float32)
    s = np.float32([0.01, 0.003])
    c = Q.quantize_fp8_per_head(x, s)
    finite = np.where(np.isfinite(F.E4M3_VALUES))[0]
    for h in range(2):
        for v, code in zip(x[0, h].ravel(), c[0, h].ravel()):
            u = float(np.float32(v) / s[h])
            u = min(max(u, -448.0), 448.0)
            d = np.abs(F.E4M3_VALUES[finite] - u)
            best = finite[d == d.min()]
            if best.size > 1:
                best = best[best % 2 == 0]
            assert code == best[0]


def test_int8_per_token_rows():
    g = np.random.default_rng(16)
    x = (g.standard_normal((1, 2, 40, 64)) * np.exp(g.standard_normal((1, 2, 40, 1)))).astype(np.float32)
    x[0, 1, 7] = 0.0
    codes, s = Q.quantize_int8_per_token(x)
    assert s.shape == (1, 2, 40) and codes.dtype == np.int8
    am = np.abs(x).argmax(axis=3)
    top = np.take_along_axis(codes, am[..., None], axis=3)[..., 0].astype(int)
    nz = np.abs(x).max(axis=3) > 0
    assert np.all(np.abs(top[nz]) == 127)  # each row's max maps to +-127
    assert s[0, 1, 7] == 1.0 and np.all(codes[0, 1, 7] == 0)
    assert np.array_equal(s[nz], (np.abs(x).max(axis=3)[nz] / np.float32(127)).astype(np.float32))
    # brute force on a few rows: nearest integer of the fp32 quotient, ties to even
    for r in range(3):
        for v, code in zip(x[0, 0, r], codes[0, 0, r]):
            u = float(np.float32(v) / s[0, 0, r])
            cands = np.arange(-128, 128)
            d = np.abs(cands - u)
            best = cands[d == d.min()]
            if best.size > 1:
                best = best[best % 2 == 0]
            assert int(code) == best[0]


def test_mxfp8_hand_worked_block():
    # amax 3: floor(log2 3) = 1, E = 1 - 8 = -7, x * 2^7:
    #   1 -> 128 = 2^7 (0x70); 0.5 -> 64 (0x68); -3 -> -384 = -1.5 * 2^8 (0xFC);
    #   0.001 -> 0.128, nearest E4M3 0.125 = 2^-3 (0x20); 1e-6 -> 1.28e-4 < 2^-10: 0
    x = np.zeros((1, 1, 1, 32), np.float32)
    x[0, 0, 0, :5] = [1.0, 0.5, -3.0, 0.001, 1e-6]
    codes, e8 = Q.quantize_mxfp8(x)
    assert int(e8.ravel()[0]) == 127 - 7
    assert list(codes.ravel()[:5]) == [0x70, 0x68, 0xFC, 0x20, 0x00]
    assert np.all(codes.ravel()[5:] == 0)
    # amax 1.9375: E = -8, 1.9375 * 256 = 496 lies in (448, 512): saturates to 448
    x[0, 0, 0, :5] = [1.9375, 0, 0, 0, 0]
    codes, e8 = Q.quantize_mxfp8(x)
    assert int(e8.ravel()[0]) == 127 - 8 and int(codes.ravel()[0]) == 0x7E


def test_mxfp8_exponent_rule_pins_emax8_max448():
    g = np.random.default_rng(17)
    x = (g.standard_t(4, (2, 3, 17, 128)) * np.exp2(g.integers(-20, 20, (2, 3, 17, 1)))).astype(np.float32)
    codes, e8 = Q.quantize_mxfp8(x)
    E = e8.astype(np.int64) - 127
    amax = np.abs(x.reshape(2, 3, 17, 4, 32)).max(axis=4)
    # amax in [256, 512) * 2^E  (E = floor(log2 amax) - 8, 448 = 1.75 * 2^8)
    assert np.all(amax >= 256.0 * np.exp2(E)) and np.all(amax < 512.0 * np.exp2(E))
    deq = Q.dequantize_mxfp8(codes, e8)
    assert np.all(np.abs(deq).reshape(2, 3, 17, 4, 32).max(axis=4) <= 448.0 * np.exp2(E))


def test_mxfp8_elements_match_torch_float8_cast():
    """torch's float8_e4m3fn cast (an independent implementation) of the
    exactly scaled block values x * 2^-E, clamped to +-448 first (torch gives
    NaN from 464 up)."""
    torch = pytest.importorskip("torch")
    g = np.random.default_rng(18)
    x = (g.standard_t(3, (1, 4, 33, 64)) * np.exp2(g.integers(-30, 30, (1, 4, 33, 1)))).astype(np.float32)
    x[0, 0, 0, :32] = 0.0
    codes, e8 = Q.quantize_mxfp8(x)
    E = e8.astype(np.int64) - 127
    v = np.ldexp(x.reshape(1, 4, 33, 2, 32).astype(np.float64), -E[..., None])
    v = np.clip(v, -448.0, 448.0).reshape(x.shape).astype(np.float32)
    ref = torch.from_numpy(v).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(codes, ref)
    assert list(e8[0, 0, 0]) == [0, e8[0, 0, 0, 1]]  # all-zero block: E = -127
