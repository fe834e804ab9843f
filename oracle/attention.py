"""Attention on dequantized low-bit operands, in fp64.

TEST INFRASTRUCTURE ONLY (see ``oracle/__init__``).

What the pages fix: Q, K and V all enter attention quantized, so both the
score product Q K^T and the weighted sum with V take low-bit operands
("FA 量化" page, 概述); attention runs in the FP8 domain and its output is
dequantized back to the original precision (MindIE SD "量化" page, FA量化 /
技术特点, FP8 Attention).  The flash-attention structure (tiles, online
softmax) is the one of the FlashAttention reference the "FA 量化" page cites.

What the pages leave open, and the reading taken here.  The pages print no
value for this rule; its arithmetic is pinned by closed forms worked by hand
(two keys in one tile, for every rule, with and without per-key V scales),
invariants (tile-order invariance, the tile-local maximum, sigma per tile)
and special cases (exact p equals softmax attention; equal scores give the
mean of V; a dominant key gives its V):

* Keys are cut into P-tiles of 128 keys aligned to absolute key index.  For
  each query row i and tile t with at least one unmasked key:
  m_it = max_j s_ij, p_ij = exp(s_ij - m_it), L_it = sum_j p_ij (unquantized).
* p enters the PV product quantized to the mode's own type with a static
  scale (0 <= p <= 1).  With sigma_t = max over the tile's keys of the
  per-key V scale and w_j = s_v,j / sigma_t (the V scale folded into P; w = 1
  when V has one scale per tile - per-head and token-block scopes - or when
  no V scale is given):
    - 'int8':  Pq = rne(127 p w_j) / (127 w_j);
    - 'fp8':   Pq = E4M3(448 p w_j) / (448 w_j);
    the code is decided on the exact product (the multiplier qmax w_j is
    formed as (qmax s_v,j) / sigma_t with one rounding of an fp64 quotient,
    which lands on a rounding boundary exactly when the exact value does);
    - 'mxfp4': the MXFP4 quantizer applied along keys, 32-key groups aligned
               to absolute key index, masked keys counting as p = 0;
    - 'mxfp8': the same with the MXFP8 quantizer (E4M3 elements, emax 8);
    - 'bf16':  V not quantized (an unconfigured branch, "fa3_quant 配置说明"
               §2.3): the product takes P in bf16, Pq = bf16_rne(p);
    - 'exact': Pq = p (no quantization; reduces to softmax attention).
  C_it = sum_j Pq_ij vhat_j with vhat the exactly dequantized V.
* Combine: M_i = max_t m_it; O_i = sum_t e^{m_it-M_i} C_it / sum_t e^{m_it-M_i} L_it.
* Scores s_ij = (qhat_i . khat_j) * sm_scale with sm_scale = 1/sqrt(D) by
  default; under causal masking key j > query i is excluded (Sq == Skv).
"""

import numpy as np

from . import formats as F
from .quantize import mx_shared_exponent

# P rule -> qmax of its static probability scale
_PQMAX = {"int8": 127.0, "fp8": F.E4M3_MAX}

P_TILE = 128
MX_GROUP = 32
TIE_REL = 2.0 ** -12


def _quantize_p(p, rule, mult=None):
    """Dequantized quantized probabilities for one row-chunk, per tile.

    p: [nr, nt, 128] fp64 (masked -> 0); mult: [nt, 128] the multiplier
    qmax w_j = qmax s_v,j / sigma_t ('int8' / 'fp8'; None means w = 1).
    Returns (Pq, step, near) where `near` flags elements whose pre-rounding
    value lies within 2^-12 (relative) of a rounding boundary and `step` is
    the size of the code step such an element may flip by (in p units)."""
    if rule == "exact":
        z = np.zeros_like(p)
        return p.copy(), z, z.astype(bool)
    if rule in _PQMAX:
        # The code is decided on u = qmax p w_j and the dequantized value
        # divides by qmax w_j.  For the tile's own maximum (p = 1) u is the
        # multiplier itself: qmax s_v,j / sigma_t, exact up to one fp64
        # rounding, which keeps every exact tie on its tie and every
        # non-tie (at least ~2^-29 away from a boundary for fp32 scales) on
        # its own side.
        qmax = _PQMAX[rule]
        if mult is None:
            mult = np.full(p.shape[1:], qmax)
        mult = mult[None, :, :]
        scale = mult
        u = p * mult
        if rule == "int8":
            pq = np.rint(u) / scale
            frac = u - np.floor(u)
            near = (np.abs(frac - 0.5) <= TIE_REL * u) & (u > 0)
            step = 1.0 / scale * np.ones_like(p)
        else:
            pq = F.e4m3_decode(F.e4m3_encode(u)) / scale
            lo, hi = F.e4m3_neighbors(u)
            mid = 0.5 * (lo + hi)
            near = (np.abs(u - mid) <= TIE_REL * u) & (u > 0)
            step = (hi - lo) / scale
        return pq, step, near
    if rule == "bf16":
        pq = F.bf16_round(p)
        _, e = np.frexp(np.where(p > 0, p, 1.0))
        ulp = np.ldexp(1.0, np.maximum(e, -125) - 8)  # bf16 spacing at p
        frac = p / ulp - np.floor(p / ulp)
        near = (np.abs(frac - 0.5) <= TIE_REL * p / ulp) & (p > 0)
        return pq, ulp, near
    if rule in ("mxfp4", "mxfp8"):
        if rule == "mxfp4":
            enc, dec, nbr, emax, vmax = F.e2m1_encode, F.e2m1_decode, F.e2m1_neighbors, F.E2M1_EMAX, F.E2M1_MAX
        else:
            enc, dec, nbr, emax, vmax = F.e4m3_encode, F.e4m3_decode, F.e4m3_neighbors, F.E4M3_EMAX, F.E4M3_MAX
        nr, nt, n = p.shape
        g = p.reshape(nr, nt, n // MX_GROUP, MX_GROUP)
        amax = g.max(axis=3)
        E = mx_shared_exponent(amax, emax=emax)
        v = np.ldexp(g, -E[..., None])
        pq = np.ldexp(dec(enc(v)), E[..., None])
        lo, hi = nbr(v)
        mid = 0.5 * (lo + hi)
        near = (np.abs(v - mid) <= TIE_REL * v) & (v > 0) & (v < vmax)
        step = np.ldexp(hi - lo, E[..., None])
        # A group whose amax sits just off a power of two may take the other
        # shared exponent; every element of it may then move by up to the
        # larger grid's top step plus the saturation of the top binade:
        # 3 * 2^(E+1) for E2M1, 3 * 2^(E+5) for E4M3.  amax == 1 exactly
        # (the tile's own maximum) is exact on both sides and is not a tie.
        k = np.rint(np.log2(np.where(amax > 0, amax, 1.0)))
        gnear = (np.abs(amax - np.exp2(k)) <= TIE_REL * amax) & (amax > 0) & (amax != 1.0)
        gstep = 3.0 * np.ldexp(1.0, E + (1 if rule == "mxfp4" else 5))
        near = near | gnear[..., None]
        step = np.where(gnear[..., None], np.maximum(step, gstep[..., None]), step)
        return (pq.reshape(nr, nt, n), step.reshape(nr, nt, n),
                near.reshape(nr, nt, n))
    raise ValueError(f"unknown P rule {rule!r}")


def attention(qhat, khat, vhat, p_rule, *, v_scale=None, causal=False,
              sm_scale=None, rows=None, allowance=False, chunk=128):
    """Quantized-domain flash attention reference.

    qhat: [B,H,Sq,D]; khat, vhat: [B,H,Skv,D] dequantized values.
    v_scale: [B,H,Skv] per-key V scale, folded into P by the 'int8' and 'fp8'
    rules (None: w = 1).
    rows: optional sorted array of query rows to evaluate (for every (b,h)).
    Returns O [B,H,R,D] fp64, plus (T [B,H,R,D], n_tie) when allowance=True:
    T is the tie allowance - the sum, over probability elements near a
    rounding boundary, of one code step * |vhat| * e^{m-M} / denominator."""
    qhat = np.asarray(qhat, dtype=np.float64)
    khat = np.asarray(khat, dtype=np.float64)
    vhat = np.asarray(vhat, dtype=np.float64)
    B, H, Sq, D = qhat.shape
    Skv = khat.shape[2]
    if causal and Sq != Skv:
        raise ValueError("causal attention needs Sq == Skv")
    if sm_scale is None:
        sm_scale = 1.0 / np.sqrt(D)
    if rows is None:
        rows = np.arange(Sq)
    rows = np.asarray(rows, dtype=np.int64)
    nt = -(-Skv // P_TILE)
    pad = nt * P_TILE - Skv
    key_idx = np.arange(nt * P_TILE)
    out = np.zeros((B, H, rows.size, D))
    tall = np.zeros((B, H, rows.size, D)) if allowance else None
    n_tie = 0
    for b in range(B):
        for h in range(H):
            k = khat[b, h]
            v = np.concatenate([vhat[b, h], np.zeros((pad, D))], axis=0)
            vt = v.reshape(nt, P_TILE, D)
            mult = None
            if p_rule in _PQMAX and v_scale is not None:
                # sigma_t = the tile's largest V scale; qmax w_j = qmax s_v,j / sigma_t
                qmax = _PQMAX[p_rule]
                sv = np.asarray(v_scale[b, h], dtype=np.float64)
                svp = np.concatenate([sv, np.zeros(pad)]).reshape(nt, P_TILE)
                sigma = svp.max(axis=1, keepdims=True)
                mult = np.where(svp > 0, (qmax * svp) / np.where(sigma > 0, sigma, 1.0), qmax)
            for c0 in range(0, rows.size, chunk):
                r = rows[c0:c0 + chunk]
                s = (qhat[b, h, r] @ k.T) * sm_scale  # [nr, Skv]
                valid = np.ones((r.size, nt * P_TILE), dtype=bool)
                valid[:, Skv:] = False
                if causal:
                    valid &= key_idx[None, :] <= r[:, None]
                sp = np.full((r.size, nt * P_TILE), -np.inf)
                sp[:, :Skv] = s
                sp = np.where(valid, sp, -np.inf).reshape(r.size, nt, P_TILE)
                vmask = valid.reshape(r.size, nt, P_TILE)
                m_t = sp.max(axis=2)  # -inf for fully masked tiles
                live = np.isfinite(m_t)
                m_safe = np.where(live, m_t, 0.0)
                p = np.where(vmask, np.exp(sp - m_safe[..., None]), 0.0)
                L_t = p.sum(axis=2)
                pq, step, near = _quantize_p(p, p_rule, mult=mult)
                C_t = np.matmul(pq.transpose(1, 0, 2), vt).transpose(1, 0, 2)  # [nr, nt, D]
                M = np.where(live, m_t, -np.inf).max(axis=1)
                f = np.where(live, np.exp(m_safe - M[:, None]), 0.0)  # e^{m_t - M}
                den = (f * L_t).sum(axis=1)
                num = (f[..., None] * C_t).sum(axis=1)
                out[b, h, c0:c0 + r.size] = num / den[:, None]
                if allowance:
                    t_el = np.where(near & vmask, step, 0.0) * f[..., None]
                    n_tie += int((near & vmask).sum())
                    tr = np.matmul(t_el.transpose(1, 0, 2), np.abs(vt)).sum(axis=0)
                    tall[b, h, c0:c0 + r.size] = tr / den[:, None]
    if allowance:
        return out, tall, n_tie
    return out

