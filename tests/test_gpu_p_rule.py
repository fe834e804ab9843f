"""GPU parity of the probability code of each tile's maximum when V has one
scale per token (FP8 and INT8 per-token V; "FA 量化" page, 组合 2, with V's
scale folded into P).  Under the P rule the code of the key that holds the
tile maximum (p = 1) is the round-to-nearest-even of the exact
qmax s_v,j / sigma_t, so V scales whose ratio sits exactly on a code
midpoint, one fp32 ulp beside it, or within fp32 rounding of it (scales
derived from bf16 amaxes) must take the exact rule's code.

The operands are built by hand: query i and key j share a one-hot channel
when j = i (mod 128), which gives one dominant key per query and tile with a
score margin of ~70 (every other p underflows to code 0).  In the centered
variant the dominant score is 0 and the others -70 (query i is -big on
every channel but its own, which is 0), so |m| is small and the kernel's
fused exponent argument (p within a few ulps of 1 at the maximum) is the
one exercised; otherwise m is ~70 nats.  Each output is
sum_t code(qmax w_j) * sigma_t / qmax * vhat_j / (number of tiles) up to
fp32 rounding, and any code decided on the wrong side of a midpoint moves it
by at least 1/16 of a tile's term.  The bar is therefore far tighter than
the general attention tolerance: 1e-5 of the largest output."""

import numpy as np
import pytest
import torch

import quantized_attention_fa_amd as faq
from oracle import attention as OA
from oracle import formats as F

pytestmark = pytest.mark.gpu

DEV = "cuda:0"
D = 128


def _e4m3_mids(lo, hi):
    """E4M3 code midpoints in [lo, hi]."""
    pos = F.E4M3_VALUES[:0x7F]
    m = (pos[1:] + pos[:-1]) / 2
    return m[(m >= lo) & (m <= hi)]


def _v_scales(rule, nt, g):
    """Per-key V scales [nt * 128] (fp32 values), tile by tile: key 127 of
    each tile holds sigma_t; the other keys sit exactly on a midpoint of the
    code grid of qmax s / sigma, one fp32 ulp beside one, on bf16-derived
    ratios, or at random."""
    qmax = 448.0 if rule == "fp8" else 127.0
    out = np.zeros(nt * 128, np.float64)
    f32 = lambda x: float(np.float32(x))
    for t in range(nt):
        kind = t % 4
        if kind < 2:
            # sigma = 7 / 8 * 2^k (fp8) or 127 / 128 * 2^k (int8): qmax s / sigma
            # is the midpoint itself when s = mid * 2^k / 64 (fp8) or
            # (n + 1/2) * 2^k / 128 (int8)
            k = int(g.integers(-6, 3))
            if rule == "fp8":
                sig = 0.875 * 2.0 ** k
                mids = _e4m3_mids(2.0 ** -3, 440.0)
                s = g.choice(mids, 127) * 2.0 ** k / 64.0
            else:
                sig = 127.0 / 128.0 * 2.0 ** k
                s = (g.integers(0, 127, 127) + 0.5) * 2.0 ** k / 128.0
            s = s.astype(np.float32)
            if kind == 1:  # one ulp up or down
                up = g.random(127) < 0.5
                s = np.where(up, np.nextafter(s, np.float32(np.inf)), np.nextafter(s, np.float32(0.0)))
            s = np.minimum(s, np.float32(sig))
            out[t * 128:t * 128 + 127] = s
            out[t * 128 + 127] = sig
        elif kind == 2:
            # scales of bf16 amaxes, s = fl32(a / qmax): sigma's amax is
            # qmax / 64 * 2^j (fp8: 7 * 2^j) or qmax * 2^j (int8), so sigma is
            # a power of two, and the other amaxes are code midpoints times
            # sigma (at most 8 significant bits): qmax s / sigma is then the
            # midpoint times (1 + the rounding error of fl32(a / qmax)) -
            # within fp32 rounding of the tie, on the side that error gives
            j = int(g.integers(-4, 5))
            if rule == "fp8":
                a_sig = 7.0 * 2.0 ** j
                mids = g.choice(_e4m3_mids(2.0 ** -2, 440.0), 127)
            else:
                a_sig = 127.0 * 2.0 ** j
                mids = g.integers(0, 127, 127) + 0.5
            sig = f32(np.float32(a_sig) / np.float32(qmax))
            a = mids * sig  # exactly representable (short significands)
            assert np.all(torch.from_numpy(a).to(torch.bfloat16).double().numpy() == a)
            out[t * 128:t * 128 + 127] = (a.astype(np.float32) / np.float32(qmax)).astype(np.float32)
            out[t * 128 + 127] = sig
        else:
            s = g.uniform(0.05, 1.0, 128).astype(np.float32)
            out[t * 128:t * 128 + 128] = s
    return out


def _fp32_multiplier_codes(rule, sv, nt):
    """Codes an fp32 multiplier fl32(qmax fl32(s / sigma)) would give at p = 1
    (the reading the rule does not take), and the exact rule's codes."""
    qmax = 448.0 if rule == "fp8" else 127.0
    s = sv.reshape(nt, 128)
    sig = s.max(axis=1, keepdims=True)
    m32 = (np.float32(qmax) * (s.astype(np.float32) / sig.astype(np.float32))).astype(np.float64)
    ex = qmax * s / sig
    enc = F.e4m3_encode if rule == "fp8" else (lambda u: np.rint(u))
    return enc(m32), enc(ex)


def _qtensor(dtype, codes, scales, S):
    cfg = faq.QConfig("fp8_e4m3" if dtype == "fp8" else "int8", "per_token")
    return faq.QTensor(cfg, (1, 1, S, D), codes.to(DEV), scales.to(DEV))


def _build(qk, vrule, nt, skv, seed, centered=False):
    """Q [128 queries], K / V [skv keys] codes and scales of one head."""
    g = np.random.default_rng(seed)
    big = 0x7E if qk == "fp8" else 127  # the largest code of the Q / K format
    sq = 1.0 / 16.0 if qk == "fp8" else 1.0 / 4.0
    qc = np.zeros((1, 1, 128, D), np.uint8 if qk == "fp8" else np.int8)
    if centered:
        qc[...] = (0x80 | big) if qk == "fp8" else -big  # -big everywhere ...
        qc[0, 0, np.arange(128), np.arange(128)] = 0  # ... but the own channel
    else:
        qc[0, 0, np.arange(128), np.arange(128)] = big
    kc = np.zeros((1, 1, skv, D), qc.dtype)
    kc[0, 0, np.arange(skv), np.arange(skv) % 128] = big
    sv = _v_scales(vrule, nt, g)[:skv]
    if vrule == "fp8":
        mag = g.integers(0x30, 0x7F, (skv, D)).astype(np.uint8)
        vc = (mag | (g.integers(0, 2, (skv, D)) << 7).astype(np.uint8)).reshape(1, 1, skv, D)
        vhat = F.e4m3_decode(vc) * sv[None, None, :, None]
    else:
        vc = g.integers(-127, 128, (1, 1, skv, D)).astype(np.int8)
        vc[vc == 0] = 1
        vhat = vc.astype(np.float64) * sv[None, None, :, None]
    qs = np.full(128, sq, np.float32)
    ks = np.full(skv, sq, np.float32)
    dq = (F.e4m3_decode(qc) if qk == "fp8" else qc.astype(np.float64)) * sq
    dk = (F.e4m3_decode(kc) if qk == "fp8" else kc.astype(np.float64)) * sq
    tq = _qtensor(qk, torch.from_numpy(qc), torch.from_numpy(qs), 128)
    tk = _qtensor(qk, torch.from_numpy(kc), torch.from_numpy(ks), skv)
    tv = _qtensor(vrule, torch.from_numpy(vc), torch.from_numpy(sv.astype(np.float32)), skv)
    return (tq, tk, tv), (dq, dk, vhat, sv.reshape(1, 1, skv))


# (Q/K format, V format, key tiles, keys): FP8 and INT8 per-token V with Q/K
# of their own configuration (specialised kernels) and of the other one
# (the general score mode); 3 tiles run without key splits (the ping-pong
# kernel for FP8 scores), 16 tiles split the keys (128 queries per head);
# a ragged last tile leaves some queries without their one-hot key there,
# so every key of that tile ties at the maximum (p = 1 for all of them).
CASES = [("fp8", "fp8", 3, 384, False), ("fp8", "fp8", 16, 2048, False), ("fp8", "fp8", 4, 428, False),
         ("int8", "int8", 3, 384, False), ("int8", "int8", 16, 2048, False), ("int8", "int8", 16, 2000, False),
         ("fp8", "int8", 16, 2048, False), ("int8", "fp8", 3, 384, False),
         ("fp8", "fp8", 3, 384, True), ("fp8", "fp8", 16, 2048, True), ("fp8", "fp8", 4, 428, True),
         ("int8", "int8", 3, 384, True), ("int8", "int8", 16, 2000, True), ("fp8", "int8", 16, 2048, True),
         ("int8", "fp8", 3, 384, True)]


@pytest.mark.parametrize("qk,vrule,nt,skv,centered", CASES)
def test_code_of_the_tile_maximum(qk, vrule, nt, skv, centered):
    tens, (dq, dk, vhat, sv) = _build(qk, vrule, nt, skv, seed=nt * 1000 + skv + (qk == "fp8") * 7 + (vrule == "fp8"),
                                      centered=centered)
    # the crafted scales must separate the exact rule from an fp32 multiplier
    m32, ex = _fp32_multiplier_codes(vrule, np.pad(sv[0, 0], (0, nt * 128 - skv)), nt)
    assert (m32 != ex).sum() >= 16
    o = faq.fa_quant_attention(*tens, out_dtype=torch.float32)
    torch.cuda.synchronize()
    got = o.cpu().numpy().astype(np.float64)
    ref = OA.attention(dq, dk, vhat, vrule, v_scale=sv)
    err = np.abs(got - ref)
    tol = 1e-5 * np.abs(ref).max()
    assert err.max() <= tol, (f"{qk}/{vrule} nt={nt} S={skv}: {int((err > tol).sum())} outputs off by more "
                              f"than {tol:.2e} (max {err.max():.3e})")
