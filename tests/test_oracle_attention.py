"""Pins of the oracle's attention: softmax attention (torch SDPA, an
independent library) when P is not quantized; closed forms where the P rule
is exact; hand-worked two-key values; tile-order invariance."""

import math

import numpy as np
import pytest
import torch

from oracle import attention as A
from oracle import formats as F


def _sdpa(q, k, v, causal, scale=None):
    t = lambda a: torch.from_numpy(np.ascontiguousarray(a, dtype=np.float64))
    o = torch.nn.functional.scaled_dot_product_attention(t(q), t(k), t(v), is_causal=causal, scale=scale)
    return o.numpy()


@pytest.mark.parametrize("S,D,causal", [(100, 64, False), (128, 64, True), (300, 128, False),
                                        (300, 64, True), (513, 32, True)])
def test_exact_p_equals_softmax_attention(S, D, causal):
    g = np.random.default_rng(S + D)
    q, k, v = (g.standard_normal((2, 2, S, D)) * 1.5 for _ in range(3))
    o = A.attention(q, k, v, "exact", causal=causal)
    assert np.allclose(o, _sdpa(q, k, v, causal), rtol=0, atol=1e-12)


def test_row_sampling_is_exact():
    g = np.random.default_rng(1)
    q, k, v = (g.standard_normal((1, 2, 400, 64)) for _ in range(3))
    rows = np.array([0, 5, 127, 128, 399])
    full = A.attention(q, k, v, "int8", causal=True)
    part = A.attention(q, k, v, "int8", causal=True, rows=rows)
    assert np.array_equal(full[:, :, rows], part)


def _two_key(p_rule, v_scale=None):
    """Two keys in one tile with scores 0 and -1: q = e0 * sqrt(D), k0 = 0,
    k1 = -e0  -> s = (0, -1) with sm_scale 1/sqrt(D)."""
    D = 64
    q = np.zeros((1, 1, 1, D)); q[..., 0] = math.sqrt(D)
    k = np.zeros((1, 1, 2, D)); k[0, 0, 1, 0] = -1.0
    v = np.zeros((1, 1, 2, D)); v[0, 0, 0, 1] = 1.0; v[0, 0, 1, 2] = 1.0
    if v_scale is not None:
        v[0, 0, 1, 2] = v_scale[0, 0, 1]  # v1 = s_v1 * code 1
    return A.attention(q, k, v, p_rule, v_scale=v_scale)[0, 0, 0], v


def test_two_key_hand_worked_int8():
    # p = (1, e^-1); 127 e^-1 = 46.72 -> 47
    o, _ = _two_key("int8")
    den = 1 + math.exp(-1)
    assert o[1] == pytest.approx(1 / den, abs=1e-15)
    assert o[2] == pytest.approx((47 / 127) / den, abs=1e-15)


def test_two_key_hand_worked_fp8():
    # equal V scales: 448 e^-1 = 164.81 -> E4M3 160 (step 16 in [128, 256))
    vs = np.ones((1, 1, 2))
    o, _ = _two_key("fp8", vs)
    den = 1 + math.exp(-1)
    assert o[2] == pytest.approx((160 / 448) / den, abs=1e-15)
    # V scales (1, 0.5): sigma = 1, w1 = 0.5: 448*0.5*e^-1 = 82.4 -> 80 (step 8);
    # Pq1 = 80 / (448*0.5); v1 = 0.5
    vs = np.array([[[1.0, 0.5]]])
    o, _ = _two_key("fp8", vs)
    assert o[2] == pytest.approx((80 / 224) * 0.5 / den, abs=1e-15)


def test_two_key_hand_worked_mxfp4():
    # group amax 1 -> E = -2; p * 4 = (4, 1.4715) -> (4, 1.5) -> Pq = (1, 0.375)
    o, _ = _two_key("mxfp4")
    den = 1 + math.exp(-1)
    assert o[1] == pytest.approx(1 / den, abs=1e-15)
    assert o[2] == pytest.approx(0.375 / den, abs=1e-15)


def test_two_key_hand_worked_int8_per_key_v_scale():
    # V scales (1, 0.5): sigma = 1, w1 = 0.5: 127 * 0.5 * e^-1 = 23.36 -> 23;
    # Pq1 = 23 / 63.5, v1 = 0.5 (code 1 times its scale)
    vs = np.array([[[1.0, 0.5]]])
    o, _ = _two_key("int8", vs)
    den = 1 + math.exp(-1)
    assert o[1] == pytest.approx(1 / den, abs=1e-15)
    assert o[2] == pytest.approx((23 / 63.5) * 0.5 / den, abs=1e-15)
    # one V scale for the tile: the per-head rule (no scale given)
    o1, _ = _two_key("int8", np.full((1, 1, 2), 0.37))
    o0, _ = _two_key("int8")
    assert np.array_equal(o1[:2], o0[:2])


def test_two_key_hand_worked_mxfp8():
    # group amax 1 -> E = floor(log2 1) - 8 = -8; p * 256 = (256, 94.18):
    # 94.18 lies in [64, 128) where E4M3 steps by 8 -> 96; Pq = (1, 0.375)
    o, _ = _two_key("mxfp8")
    den = 1 + math.exp(-1)
    assert o[1] == pytest.approx(1 / den, abs=1e-15)
    assert o[2] == pytest.approx(0.375 / den, abs=1e-15)


def test_two_key_hand_worked_bf16():
    # p = (1, e^-1); e^-1 = 1.4715177 * 2^-2, 7 fraction bits: 188.35 / 128
    # -> 188 / 128 -> Pq1 = 0.3671875
    o, _ = _two_key("bf16")
    den = 1 + math.exp(-1)
    assert o[1] == pytest.approx(1 / den, abs=1e-15)
    assert o[2] == pytest.approx(0.3671875 / den, abs=1e-15)


@pytest.mark.parametrize("rule", ["int8", "fp8", "mxfp4", "mxfp8", "bf16"])
def test_equal_scores_give_mean_of_v(rule):
    g = np.random.default_rng(2)
    S, D = 300, 64
    q = np.zeros((1, 1, 5, D))
    k = g.standard_normal((1, 1, S, D))
    v = g.standard_normal((1, 1, S, D))
    vs = np.full((1, 1, S), 0.37)
    o = A.attention(q, k, v, rule, v_scale=vs)
    assert np.allclose(o, v.mean(axis=2, keepdims=True), atol=1e-13)


@pytest.mark.parametrize("rule", ["int8", "fp8", "mxfp4", "mxfp8", "bf16", "exact"])
def test_dominant_key(rule):
    g = np.random.default_rng(3)
    S, D = 260, 64
    q = np.zeros((1, 1, 1, D)); q[..., 0] = 1.0
    k = np.zeros((1, 1, S, D)); k[0, 0, 200, 0] = 4000.0
    v = g.standard_normal((1, 1, S, D))
    o = A.attention(q, k, v, rule, v_scale=np.ones((1, 1, S)))
    assert np.allclose(o[0, 0, 0], v[0, 0, 200], atol=1e-13)


@pytest.mark.parametrize("rule", ["int8", "fp8", "mxfp4", "mxfp8", "bf16"])
def test_tile_local_max(rule):
    """Tile 0: one key with a large score; tile 1: 128 keys of one lower
    score.  With each tile's probabilities taken relative to its own max the
    quantized P is exact in both tiles (1 and 0/1), so O is exactly softmax
    attention.  Taking tile 1 relative to the running max would quantize
    e^{b-a} instead and miss this."""
    g = np.random.default_rng(4)
    D = 64
    q = np.zeros((1, 1, 1, D)); q[..., 0] = math.sqrt(D)
    k = np.zeros((1, 1, 256, D))
    k[0, 0, 0, 0] = 2.0       # score a = 2
    k[0, 0, 1:128, 0] = -60.0  # p underflows far below any code step
    k[0, 0, 128:, 0] = 0.3    # score b = 0.3 for the whole second tile
    v = g.standard_normal((1, 1, 256, D))
    o = A.attention(q, k, v, rule, v_scale=np.ones((1, 1, 256)))
    ref = _sdpa(q, k, v, False)
    assert np.allclose(o, ref, atol=1e-12)


@pytest.mark.parametrize("rule", ["fp8", "int8"])
def test_sigma_is_per_tile(rule):
    """Equal scores, V scale 1 in tile 0 and 0.3 in tile 1: sigma per tile
    makes w = 1 everywhere and P exact (O = mean v); a global sigma would
    quantize 448*0.3 = 134.4 -> 128 (127*0.3 = 38.1 -> 38) in tile 1."""
    g = np.random.default_rng(5)
    D = 64
    q = np.zeros((1, 1, 1, D))
    k = g.standard_normal((1, 1, 256, D))
    v = g.standard_normal((1, 1, 256, D))
    vs = np.concatenate([np.ones(128), np.full(128, 0.3)]).reshape(1, 1, 256)
    o = A.attention(q, k, v, rule, v_scale=vs)
    assert np.allclose(o[0, 0, 0], v[0, 0].mean(axis=0), atol=1e-13)


@pytest.mark.parametrize("rule", ["int8", "fp8", "mxfp4", "mxfp8", "bf16"])
def test_tile_order_invariance(rule):
    g = np.random.default_rng(6)
    S, D = 512, 64
    q, k, v = (g.standard_normal((1, 1, S, D)) * 2 for _ in range(3))
    vs = np.exp(g.standard_normal((1, 1, S)))
    o = A.attention(q, k, v, rule, v_scale=vs)
    perm = np.concatenate([np.arange(t * 128, t * 128 + 128) for t in [2, 0, 3, 1]])
    o2 = A.attention(q, k[:, :, perm], v[:, :, perm], rule, v_scale=vs[:, :, perm])
    assert np.allclose(o, o2, atol=1e-13)


def test_quantized_close_to_exact():
    """Each rule stays close to softmax attention on typical data (rule
    sanity: int8/e4m3 P errors are ~1e-2 relative Frobenius)."""
    g = np.random.default_rng(7)
    q, k, v = (g.standard_normal((1, 2, 256, 64)) for _ in range(3))
    ref = A.attention(q, k, v, "exact")
    for rule, tol in [("int8", 0.05), ("fp8", 0.06), ("mxfp4", 0.25), ("mxfp8", 0.06), ("bf16", 0.01)]:
        o = A.attention(q, k, v, rule, v_scale=np.ones((1, 2, 256)))
        err = np.linalg.norm(o - ref) / np.linalg.norm(ref)
        assert 1e-4 < err < tol, (rule, err)


def test_allowance_flags_ties():
    # p = exp(-x) with 127 p exactly at a half-integer up to 2^-13 relative
    D = 64
    t = 46.5 / 127
    s1 = math.log(t)
    q = np.zeros((1, 1, 1, D)); q[..., 0] = math.sqrt(D)
    k = np.zeros((1, 1, 2, D)); k[0, 0, 1, 0] = s1
    v = np.ones((1, 1, 2, D))
    o, T, n = A.attention(q, k, v, "int8", allowance=True)
    assert n == 1
    assert T[0, 0, 0, 0] == pytest.approx((1 / 127) / (1 + t), rel=1e-9)


def _top_key_code(rule, sv0, sv1):
    """Two keys: key 0 holds the tile maximum (p = 1), key 1's p underflows,
    so O[1] = code(qmax w_0) / (qmax w_0) * vhat_0 with vhat_0 = s_v0 * 1.
    Returns the code the oracle took for the maximum: O[1] * qmax w_0 / vhat_0."""
    D = 64
    q = np.zeros((1, 1, 1, D)); q[..., 0] = math.sqrt(D)
    k = np.zeros((1, 1, 2, D)); k[0, 0, 1, 0] = -200.0  # p1 = e^-200 rounds to code 0
    v = np.zeros((1, 1, 2, D)); v[0, 0, 0, 1] = sv0; v[0, 0, 1, 2] = sv1
    vs = np.array([[[sv0, sv1]]], dtype=np.float64)
    o = A.attention(q, k, v, rule, v_scale=vs)[0, 0, 0]
    qmax = 448.0 if rule == "fp8" else 127.0
    return o[1] * (qmax * sv0 / max(sv0, sv1)) / sv0


def test_fp8_code_of_the_maximum_is_decided_exactly():
    """The probability code of the tile's maximum (p = 1) is decided on the
    exact 448 w_j (the reading of the P rule: V's scale folded into P, then
    E4M3 round-to-nearest-even).  Hand-worked: V amaxes 2.125 and 14 give
    fp32 scales s0 = fl32(2.125/448) and s1 = 14/448 = 2^-5 exactly, so
    448 w_0 = 448 * 32 * fl32(2.125/448) = 68 (1 + e) with e the (positive)
    rounding error of fl32(2.125/448): just above the 64 / 72 midpoint, code
    72.  An fp32 multiplier fl32(448 fl32(w_0)) rounds to 68.0 exactly and
    would give the even code 64."""
    s0 = float(np.float32(2.125) / np.float32(448))
    s1 = float(np.float32(14.0) / np.float32(448))
    assert s1 == 2.0 ** -5 and 448 * 32 * s0 > 68.0  # the hand-worked premises
    assert float(np.float32(448) * (np.float32(s0) / np.float32(s1))) == 68.0
    assert _top_key_code("fp8", s0, s1) == pytest.approx(72.0, rel=1e-12)


def test_fp8_code_of_the_maximum_at_an_exact_tie():
    """448 w_j exactly on the 64 / 72 midpoint: s0 = 17/128, sigma = 7/8 give
    448 * (17/128) / (7/8) = 68 exactly, so round-half-even takes 64."""
    assert _top_key_code("fp8", 17.0 / 128.0, 7.0 / 8.0) == pytest.approx(64.0, rel=1e-12)
    # and just above the tie (s0 one fp32 ulp larger): 72
    s0_up = float(np.nextafter(np.float32(17.0 / 128.0), np.float32(1.0)))
    assert _top_key_code("fp8", s0_up, 7.0 / 8.0) == pytest.approx(72.0, rel=1e-12)


def test_int8_code_of_the_maximum_is_decided_exactly():
    """INT8 per-token V: 127 w_j = 127 * (93/256) / (127/128) = 46.5 exactly
    rounds half to even, to 46; one fp32 ulp more in s_v,j gives 47, one
    less 46."""
    s0, sig = 93.0 / 256.0, 127.0 / 128.0
    assert 127 * s0 / sig == 46.5
    assert _top_key_code("int8", s0, sig) == pytest.approx(46.0, rel=1e-12)
    up = float(np.nextafter(np.float32(s0), np.float32(1.0)))
    dn = float(np.nextafter(np.float32(s0), np.float32(0.0)))
    assert _top_key_code("int8", up, sig) == pytest.approx(47.0, rel=1e-12)
    assert _top_key_code("int8", dn, sig) == pytest.approx(46.0, rel=1e-12)


def test_bf16_rule_is_one_rounding_of_p():
    """Against torch's bf16 cast (an independent rounding): every quantized
    probability is the bf16 value nearest to the exact p."""
    g = np.random.default_rng(8)
    p = np.exp(-np.abs(g.standard_normal((3, 2, 128))) * 4)
    pq, step, near = A._quantize_p(p, "bf16")
    ref = torch.from_numpy(p.astype(np.float32)).to(torch.bfloat16).to(torch.float64).numpy()
    # the float32 detour of the reference can only differ at exact ties
    assert np.mean(pq == ref) > 0.999
    assert np.all(np.abs(pq - p) <= step / 2 * (1 + 1e-12))
