"""Scalar-semantics quantizers of the FA quantization modes.

TEST INFRASTRUCTURE ONLY (see ``oracle/__init__``).

Tensors are BNSD ``[B, H, S, D]`` arrays of real values (float32 holding the
fp32 or bf16 inputs exactly).  Scale arithmetic is float32 with IEEE
round-to-nearest-even (numpy float32 division is correctly rounded); every
other step is exact or goes through the encoders of ``oracle.formats``.

Pins (tests/test_oracle_quantize.py): the hand-worked values under
``tests/golden/``, symmetry and zero-offset, scale counts, brute-force
nearest-code search on tiny tensors, the exponent rule against the printed
"emax=2, max 6", and the rotation invariance of Q K^T.
"""

import numpy as np

from . import formats as F

QMAX_INT8 = 127.0
QMAX_FP8 = F.E4M3_MAX  # 448
MX_BLOCK = 32


def _as_f32(x) -> np.ndarray:
    x = np.asarray(x)
    if x.dtype != np.float32:
        x = x.astype(np.float32)
    return x


def _scale_from_amax(amax, qmax) -> np.ndarray:
    """fl32(amax / qmax); an all-zero group gets scale 1 (the pages are
    silent on amax == 0; with scale 1 every code is 0)."""
    amax = _as_f32(amax)
    s = (amax / np.float32(qmax)).astype(np.float32)
    return np.where(amax == 0, np.float32(1.0), s).astype(np.float32)


def _div32(x, s) -> np.ndarray:
    """fl32(x / s): float32 division, correctly rounded."""
    return (_as_f32(x) / _as_f32(s)).astype(np.float32)


# --------------------------------------------------------------------------
# 组合 1 - INT8 per-head static ("FA 量化" page, 分支组合 / 组合 1; the
# fa3_quant config page, §2.1 default qconfig int8 / per_head / symmetric /
# minmax, §2.2 method minmax).  One scale per attention head, calibrated
# offline by min-max and then frozen; symmetric, no offset.
# --------------------------------------------------------------------------


def calibrate_amax(x, amax=None) -> np.ndarray:
    """Running per-head max|x| over calibration tensors: amax[h] =
    max(amax[h], max over b, s, d of |x[b, h, s, d]|).  Exact."""
    x = _as_f32(x)
    cur = np.abs(x).max(axis=(0, 2, 3)).astype(np.float32)
    if amax is None:
        return cur
    return np.maximum(_as_f32(amax), cur)


def int8_scales(amax) -> np.ndarray:
    """Per-head INT8 scale fl32(amax / 127)."""
    return _scale_from_amax(amax, QMAX_INT8)


def fp8_scales(amax) -> np.ndarray:
    """Per-head FP8 scale fl32(amax / 448) (the FP8 variant of FA PerHead)."""
    return _scale_from_amax(amax, QMAX_FP8)


def quantize_int8_per_head(x, scale) -> np.ndarray:
    """code = clip(rne(fl32(x / scale[h])), -128, 127) as int8 [B,H,S,D]."""
    x = _as_f32(x)
    s = _as_f32(scale).reshape(1, -1, 1, 1)
    return F.int8_encode(_div32(x, s))


def quantize_fp8_per_head(x, scale) -> np.ndarray:
    """FA PerHead, FP8 variant ("FA 量化" page, 该类下的模式清单: per-head
    static INT8/FP8; "量化模式" page, 模式索引 / FA 量化, FP8 per-head static):
    code = E4M3(fl32(x / scale[h])), saturating at +-448 for inputs beyond
    the calibrated range.  uint8 E4M3 bit patterns [B,H,S,D]."""
    x = _as_f32(x)
    s = _as_f32(scale).reshape(1, -1, 1, 1)
    return F.e4m3_encode(_div32(x, s))


def dequantize_per_head(codes, scale, decode=None) -> np.ndarray:
    vals = codes.astype(np.float64) if decode is None else decode(codes)
    return vals * _as_f32(scale).astype(np.float64).reshape(1, -1, 1, 1)


# --------------------------------------------------------------------------
# 组合 2 - FP8 E4M3 per-token dynamic ("FA 量化" page, 分支组合 / 组合 2):
# one scale per token row, computed online from that row's max|x|.
# --------------------------------------------------------------------------


def quantize_fp8_per_token(x):
    """Per (b,h,s) row over D: s = fl32(amax / 448); code = E4M3(fl32(x / s)).
    Returns (codes uint8 [B,H,S,D], scales float32 [B,H,S])."""
    x = _as_f32(x)
    amax = np.abs(x).max(axis=3)
    s = _scale_from_amax(amax, QMAX_FP8)
    codes = F.e4m3_encode(_div32(x, s[..., None]))
    return codes, s


def quantize_int8_per_token(x):
    """FA PerToken, INT8 variant ("FA 量化" page, 该类下的模式清单: per-token
    dynamic INT8/FP8): per (b,h,s) row s = fl32(amax / 127) and
    code = clip(rne(fl32(x / s)), -128, 127).  Returns (codes int8 [B,H,S,D],
    scales float32 [B,H,S])."""
    x = _as_f32(x)
    amax = np.abs(x).max(axis=3)
    s = _scale_from_amax(amax, QMAX_INT8)
    return F.int8_encode(_div32(x, s[..., None])), s


def dequantize_per_token(codes, scales, decode) -> np.ndarray:
    return decode(codes) * _as_f32(scales).astype(np.float64)[..., None]


# --------------------------------------------------------------------------
# 组合 3 - MXFP4 per-block dynamic ("FA 量化" page, 分支组合 / 组合 3):
# 32 consecutive elements along head_dim share one E8M0 exponent; elements
# are E2M1 (largest exponent 2, largest value 6).
# --------------------------------------------------------------------------


def mx_shared_exponent(amax, emax=F.E2M1_EMAX) -> np.ndarray:
    """E = clamp(floor(log2 amax) - emax, -127, 127), read exactly from the
    binary exponent of amax; amax == 0 gives -127.  emax is the exponent of
    the element format's largest normal: 2 for E2M1 (max 6 = 1.5 * 2^2),
    8 for E4M3 (max 448 = 1.75 * 2^8)."""
    amax = np.asarray(amax, dtype=np.float64)
    _, e = np.frexp(amax)  # amax = m * 2^e, 0.5 <= m < 1  =>  floor(log2) = e - 1
    E = (e - 1) - emax
    E = np.where(amax == 0, -127, E)
    return np.clip(E, -127, 127).astype(np.int64)


def quantize_mxfp4(x):
    """Returns (packed codes uint8 [B,H,S,D/2] with element 2i in the low
    nibble, E8M0 bytes uint8 [B,H,S,D/32])."""
    x = _as_f32(x)
    B, H, S, D = x.shape
    if D % MX_BLOCK:
        raise ValueError("head_dim must be a multiple of 32 for MXFP4")
    blk = x.reshape(B, H, S, D // MX_BLOCK, MX_BLOCK).astype(np.float64)
    E = mx_shared_exponent(np.abs(blk).max(axis=4))
    v = np.ldexp(blk, -E[..., None])  # exact power-of-two scaling
    codes = F.e2m1_encode(v).reshape(B, H, S, D)
    packed = (codes[..., 0::2] | (codes[..., 1::2] << 4)).astype(np.uint8)
    return packed, (E + 127).astype(np.uint8)


def quantize_mxfp8(x):
    """FA PerBlock, MXFP8 variant ("FA 量化" page, 该类下的模式清单: block
    shared-exponent MXFP8/MXFP4; "量化模式" page, 模式索引 / FA 量化): the
    组合 3 structure - 32 consecutive elements along head_dim share one E8M0
    exponent - with E4M3 elements, whose largest normal exponent is 8 (max
    448): E = clamp(floor(log2 amax) - 8, -127, 127), element =
    E4M3(x * 2^-E) with ties to even, saturating at 448 (block values in
    (448, 512) * 2^E).  Returns (codes uint8 [B,H,S,D] E4M3 bit patterns,
    E8M0 bytes uint8 [B,H,S,D/32])."""
    x = _as_f32(x)
    B, H, S, D = x.shape
    if D % MX_BLOCK:
        raise ValueError("head_dim must be a multiple of 32 for MXFP8")
    blk = x.reshape(B, H, S, D // MX_BLOCK, MX_BLOCK).astype(np.float64)
    E = mx_shared_exponent(np.abs(blk).max(axis=4), emax=F.E4M3_EMAX)
    v = np.ldexp(blk, -E[..., None])  # exact power-of-two scaling
    codes = F.e4m3_encode(v).reshape(B, H, S, D)
    return codes, (E + 127).astype(np.uint8)


def dequantize_mxfp8(codes, e8m0) -> np.ndarray:
    codes = np.asarray(codes, dtype=np.uint8)
    B, H, S, D = codes.shape
    vals = F.e4m3_decode(codes).reshape(B, H, S, D // MX_BLOCK, MX_BLOCK)
    scale = F.e8m0_decode(e8m0)[..., None]
    return (vals * scale).reshape(B, H, S, D)


def unpack_fp4(packed) -> np.ndarray:
    packed = np.asarray(packed, dtype=np.uint8)
    lo = packed & 0xF
    hi = packed >> 4
    out = np.empty(packed.shape[:-1] + (packed.shape[-1] * 2,), dtype=np.uint8)
    out[..., 0::2] = lo
    out[..., 1::2] = hi
    return out


def dequantize_mxfp4(packed, e8m0) -> np.ndarray:
    codes = unpack_fp4(packed)
    B, H, S, D = codes.shape
    vals = F.e2m1_decode(codes).reshape(B, H, S, D // MX_BLOCK, MX_BLOCK)
    scale = F.e8m0_decode(e8m0)[..., None]
    return (vals * scale).reshape(B, H, S, D)


# --------------------------------------------------------------------------
# Rotate -> FP8 block quant (MindIE SD "量化" page, FA量化 / 技术特点:
# 旋转 applies the pretrained q_rot / k_rot to Q and K; 块量化 quantizes the
# rotated Q/K/V dynamically to float8_e4m3fn with block size 128 for Q and
# 256 for K/V).
# --------------------------------------------------------------------------


def rotate(x, R) -> np.ndarray:
    """Y = bf16_rne(X . R): each output element is the dot product of a
    token row of X with a column of R in fp64 (an error far below one bf16
    ulp), rounded once to bf16.  Returned as float32 (exact)."""
    x = np.asarray(x, dtype=np.float64)
    R = np.asarray(R, dtype=np.float64)
    return F.bf16_round(x @ R).astype(np.float32)


def quantize_fp8_block(y, block_tokens):
    """One scale per (b, h, block of `block_tokens` tokens x all of D):
    s = fl32(amax / 448), code = E4M3(fl32(y / s)).  A partial last block is
    its own block.  Returns (codes uint8 [B,H,S,D], scales float32
    [B,H,ceil(S/bt)])."""
    y = _as_f32(y)
    B, H, S, D = y.shape
    nb = -(-S // block_tokens)
    amax = np.zeros((B, H, nb), dtype=np.float32)
    for i in range(nb):
        sl = y[:, :, i * block_tokens:(i + 1) * block_tokens, :]
        amax[:, :, i] = np.abs(sl).max(axis=(2, 3))
    s = _scale_from_amax(amax, QMAX_FP8)
    s_tok = np.repeat(s, block_tokens, axis=2)[:, :, :S]
    codes = F.e4m3_encode(_div32(y, s_tok[..., None]))
    return codes, s


def block_scales_per_token(scales, block_tokens, S) -> np.ndarray:
    """Expand per-block scales [B,H,nb] to per-token [B,H,S]."""
    return np.repeat(np.asarray(scales, dtype=np.float32), block_tokens, axis=2)[:, :, :S]
