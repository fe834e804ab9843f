"""C ABI checks that need no GPU: the library loads, exports every function
include/fa_quant.h declares, and rejects bad arguments before any HIP call."""

import ctypes
import os
import re

import pytest

from conftest import ROOT
import quantized_attention_fa_amd as faq
from quantized_attention_fa_amd import _abi

HEADER = os.path.join(ROOT, "include", "fa_quant.h")


def _declared():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(fa_quant\w*|fa_quantize)\s*\(", text)))


def test_exports_match_header():
    names = _declared()
    assert set(names) == set(_abi.EXPORTS)
    lib = _abi.lib()
    for n in names:
        assert hasattr(lib, n), n
    # nothing else with the prefix is exported
    out = os.popen(f"nm -D --defined-only {_abi.LIB_PATH}").read()
    exported = set(re.findall(r" T (fa_quant\w*|fa_quantize)\b", out))
    assert exported == set(names)


def test_status_strings():
    lib = _abi.lib()
    for st in range(-7, 1):
        s = lib.fa_quant_status_string(st).decode()
        assert s and s != "unknown status"
    assert lib.fa_quant_status_string(-99).decode() == "unknown status"


def _cfg(dtype, scope, bt=0, sym=1, method=0):
    return _abi.faq_qconfig(dtype, scope, sym, method, bt)


def test_size_queries():
    lib = _abi.lib()
    shp = _abi.faq_shape(2, 3, 300, 128)
    B = ctypes.byref
    c = _cfg(_abi.FAQ_INT8, _abi.FAQ_PER_HEAD)
    assert lib.fa_quant_codes_bytes(B(c), B(shp)) == 2 * 3 * 300 * 128
    assert lib.fa_quant_scales_bytes(B(c), B(shp)) == 3 * 4
    c = _cfg(_abi.FAQ_FP8_E4M3, _abi.FAQ_PER_TOKEN)
    assert lib.fa_quant_scales_bytes(B(c), B(shp)) == 2 * 3 * 300 * 4
    c = _cfg(_abi.FAQ_MXFP4, _abi.FAQ_PER_BLOCK)
    assert lib.fa_quant_codes_bytes(B(c), B(shp)) == 2 * 3 * 300 * 64
    assert lib.fa_quant_scales_bytes(B(c), B(shp)) == 2 * 3 * 300 * 4
    c = _cfg(_abi.FAQ_FP8_E4M3, _abi.FAQ_PER_TOKEN_BLOCK, 256)
    assert lib.fa_quant_scales_bytes(B(c), B(shp)) == 2 * 3 * 2 * 4
    # sibling modes: FP8 per-head, INT8 per-token, MXFP8 per-block
    c = _cfg(_abi.FAQ_FP8_E4M3, _abi.FAQ_PER_HEAD)
    assert lib.fa_quant_codes_bytes(B(c), B(shp)) == 2 * 3 * 300 * 128
    assert lib.fa_quant_scales_bytes(B(c), B(shp)) == 3 * 4
    c = _cfg(_abi.FAQ_INT8, _abi.FAQ_PER_TOKEN)
    assert lib.fa_quant_codes_bytes(B(c), B(shp)) == 2 * 3 * 300 * 128
    assert lib.fa_quant_scales_bytes(B(c), B(shp)) == 2 * 3 * 300 * 4
    c = _cfg(_abi.FAQ_MXFP8, _abi.FAQ_PER_BLOCK)
    assert lib.fa_quant_codes_bytes(B(c), B(shp)) == 2 * 3 * 300 * 128
    assert lib.fa_quant_scales_bytes(B(c), B(shp)) == 2 * 3 * 300 * 4
    # combinations outside the mode list stay unsupported (size 0)
    for dt, sc in [(_abi.FAQ_MXFP8, _abi.FAQ_PER_TOKEN), (_abi.FAQ_INT8, _abi.FAQ_PER_BLOCK),
                   (_abi.FAQ_MXFP4, _abi.FAQ_PER_HEAD), (_abi.FAQ_INT8, _abi.FAQ_PER_TOKEN_BLOCK)]:
        c = _cfg(dt, sc, 128)
        assert lib.fa_quant_codes_bytes(B(c), B(shp)) == 0
    # unsupported combinations report 0
    assert lib.fa_quant_codes_bytes(B(_cfg(_abi.FAQ_INT8, _abi.FAQ_PER_BLOCK)), B(shp)) == 0
    assert lib.fa_quant_codes_bytes(B(c), B(_abi.faq_shape(1, 1, 4, 96))) == 0


FAKE = ctypes.c_void_p(0x1000)  # never dereferenced: validation fails first


def _quantize(cfg, shape, static=None, rot=None, out_cfg=None, out_shape=None, xdt=_abi.FAQ_T_BF16, dbg=None):
    lib = _abi.lib()
    qt = _abi.faq_qtensor(out_cfg or cfg, out_shape or shape, 0x2000, 0x3000)
    return lib.fa_quantize(FAKE, xdt, ctypes.byref(shape), ctypes.byref(cfg), static, rot, ctypes.byref(qt), dbg, None)


def test_quantize_validation():
    shp = _abi.faq_shape(1, 2, 64, 128)
    head = _cfg(_abi.FAQ_INT8, _abi.FAQ_PER_HEAD)
    # static per-head without calibration data is an error ("FA 量化" 组合 1)
    assert _quantize(head, shp) == _abi.FAQ_ERR_NOT_CALIBRATED
    tok = _cfg(_abi.FAQ_FP8_E4M3, _abi.FAQ_PER_TOKEN)
    assert _quantize(tok, shp, static=FAKE) == _abi.FAQ_ERR_INVALID_ARG
    assert _quantize(tok, _abi.faq_shape(1, 2, 64, 96)) == _abi.FAQ_ERR_UNSUPPORTED
    assert _quantize(tok, shp, out_shape=_abi.faq_shape(1, 2, 65, 128)) == _abi.FAQ_ERR_SHAPE
    assert _quantize(tok, shp, out_cfg=_cfg(_abi.FAQ_MXFP4, _abi.FAQ_PER_BLOCK)) == _abi.FAQ_ERR_INVALID_ARG
    assert _quantize(_cfg(_abi.FAQ_FP8_E4M3, _abi.FAQ_PER_TOKEN, sym=0), shp) == _abi.FAQ_ERR_UNSUPPORTED
    assert _quantize(_cfg(_abi.FAQ_FLOAT, _abi.FAQ_PER_TOKEN), shp) == _abi.FAQ_ERR_UNSUPPORTED
    assert _quantize(_cfg(7, _abi.FAQ_PER_TOKEN), shp) == _abi.FAQ_ERR_INVALID_ARG
    assert _quantize(tok, shp, rot=FAKE) == _abi.FAQ_ERR_UNSUPPORTED
    blk = _cfg(_abi.FAQ_FP8_E4M3, _abi.FAQ_PER_TOKEN_BLOCK, 128)
    assert _quantize(blk, shp, xdt=_abi.FAQ_T_F32) == _abi.FAQ_ERR_UNSUPPORTED
    assert _quantize(blk, shp, dbg=FAKE) == _abi.FAQ_ERR_INVALID_ARG
    assert _quantize(_cfg(_abi.FAQ_FP8_E4M3, _abi.FAQ_PER_TOKEN_BLOCK, 0), shp) == _abi.FAQ_ERR_INVALID_ARG
    assert _quantize(_cfg(_abi.FAQ_FP8_E4M3, _abi.FAQ_PER_TOKEN_BLOCK, 64), shp) == _abi.FAQ_ERR_UNSUPPORTED
    assert _quantize(tok, _abi.faq_shape(1, -2, 64, 128)) == _abi.FAQ_ERR_INVALID_ARG
    assert _quantize(tok, _abi.faq_shape(1, 2, 64, 128, 2)) == _abi.FAQ_ERR_INVALID_ARG  # unknown layout
    assert _quantize(tok, _abi.faq_shape(1 << 20, 1 << 10, 1 << 10, 128)) == _abi.FAQ_ERR_INVALID_ARG  # rows >= 2^31
    lib = _abi.lib()
    assert lib.fa_quant_calibrate(FAKE, 5, ctypes.byref(shp), FAKE, None) == _abi.FAQ_ERR_INVALID_ARG
    assert lib.fa_quant_calibrate(FAKE, 1, ctypes.byref(shp), None, None) == _abi.FAQ_ERR_INVALID_ARG
    assert lib.fa_quant_scales_from_amax(FAKE, 4, _abi.FAQ_MXFP4, FAKE, None) == _abi.FAQ_ERR_UNSUPPORTED
    assert lib.fa_quant_scales_from_amax(FAKE, -1, _abi.FAQ_INT8, FAKE, None) == _abi.FAQ_ERR_INVALID_ARG


def _qt(cfg, shape):
    return _abi.faq_qtensor(cfg, shape, 0x2000, 0x3000)


def _attn(q, k, v, causal=0, ws_bytes=1 << 40, out_dtype=_abi.FAQ_T_BF16, sm=0.0):
    return _abi.lib().fa_quant_attention(ctypes.byref(q), ctypes.byref(k), ctypes.byref(v), sm, causal, FAKE,
                                         out_dtype, FAKE, ws_bytes, None)


def test_attention_validation():
    tok = _cfg(_abi.FAQ_FP8_E4M3, _abi.FAQ_PER_TOKEN)
    s = _abi.faq_shape(1, 2, 256, 128)
    q, k, v = _qt(tok, s), _qt(tok, s), _qt(tok, s)
    lib = _abi.lib()
    need = lib.fa_quant_attention_workspace_bytes(ctypes.byref(q), ctypes.byref(k), ctypes.byref(v))
    assert need >= 2 * 256 * 128
    assert _attn(q, k, v, ws_bytes=need - 1) == _abi.FAQ_ERR_WORKSPACE
    assert _attn(q, k, _qt(tok, _abi.faq_shape(1, 2, 255, 128))) == _abi.FAQ_ERR_SHAPE
    assert _attn(q, _qt(tok, _abi.faq_shape(1, 3, 256, 128)), v) == _abi.FAQ_ERR_SHAPE
    qs = _qt(tok, _abi.faq_shape(1, 2, 100, 128))
    assert _attn(qs, k, v, causal=1) == _abi.FAQ_ERR_SHAPE
    mx = _cfg(_abi.FAQ_MXFP4, _abi.FAQ_PER_BLOCK)
    assert _attn(q, k, v, out_dtype=9) == _abi.FAQ_ERR_INVALID_ARG
    assert _attn(q, k, v, causal=2) == _abi.FAQ_ERR_INVALID_ARG
    assert _attn(q, k, v, sm=-1.0) == _abi.FAQ_ERR_INVALID_ARG
    assert _attn(q, k, v, sm=float("nan")) == _abi.FAQ_ERR_INVALID_ARG
    # per-branch configurations: every combination of the three branches
    # runs (fa3_quant 配置说明 §2.3); pairs without a specialised score
    # kernel widen Q and K to bf16, and K's bf16 image (2 bytes per element)
    # is part of their workspace
    ws = lambda a, b, c: lib.fa_quant_attention_workspace_bytes(ctypes.byref(_qt(a, s)), ctypes.byref(_qt(b, s)),
                                                                ctypes.byref(_qt(c, s)))
    b1 = _cfg(_abi.FAQ_FP8_E4M3, _abi.FAQ_PER_TOKEN_BLOCK, 128)
    b2 = _cfg(_abi.FAQ_FP8_E4M3, _abi.FAQ_PER_TOKEN_BLOCK, 256)
    fl = _cfg(_abi.FAQ_FLOAT, _abi.FAQ_PER_HEAD)
    i8t = _cfg(_abi.FAQ_INT8, _abi.FAQ_PER_TOKEN)
    i8h = _cfg(_abi.FAQ_INT8, _abi.FAQ_PER_HEAD)
    m8 = _cfg(_abi.FAQ_MXFP8, _abi.FAQ_PER_BLOCK)
    i8h0 = _cfg(_abi.FAQ_INT8, _abi.FAQ_PER_HEAD)
    for ok in [(b1, b2, b2), (b1, b2, fl), (fl, fl, tok), (fl, fl, mx), (fl, fl, fl), (tok, tok, fl), (i8t, i8t, i8t),
               (i8h0, i8h0, i8h0)]:
        assert ws(*ok) >= 256, ok  # INT8 per-head needs no re-layout but still reports a size
    for mixed in [(tok, tok, i8t), (fl, tok, tok), (tok, fl, fl), (i8t, tok, tok), (mx, mx, tok), (mx, m8, i8h),
                  (i8h, i8t, mx), (tok, b1, fl)]:
        assert ws(*mixed) >= 2 * 2 * 256 * 128, mixed
    assert _attn(_qt(mx, s), _qt(i8h, s), _qt(tok, s), ws_bytes=ws(mx, i8h, tok) - 1) == _abi.FAQ_ERR_WORKSPACE
    # a head's K / V rows must span less than 4 GiB (32-bit row offsets):
    # BSND bf16 with S = 2^20, H = 20, D = 128 spans about 2^20 * 20 * 256
    # bytes (5 GiB)
    big = _abi.faq_shape(1, 20, 1 << 20, 128, _abi.FAQ_LAYOUT_BSND)
    assert _attn(_qt(fl, big), _qt(fl, big), _qt(fl, big)) == _abi.FAQ_ERR_UNSUPPORTED
    ok_big = _abi.faq_shape(1, 20, 1 << 20, 128, _abi.FAQ_LAYOUT_BNSD)  # 256 MiB per head
    assert lib.fa_quant_attention_workspace_bytes(ctypes.byref(_qt(fl, ok_big)), ctypes.byref(_qt(fl, ok_big)),
                                                  ctypes.byref(_qt(fl, ok_big))) > 0
    # unquantized branches need no scales; quantized ones do
    nos = _abi.faq_qtensor(tok, s, 0x2000, None)
    assert _attn(nos, k, v) == _abi.FAQ_ERR_INVALID_ARG
    assert lib.fa_quant_attention(None, ctypes.byref(k), ctypes.byref(v), 0.0, 0, FAKE, 1, FAKE, 1, None) \
        == _abi.FAQ_ERR_INVALID_ARG


def test_fa3_config_rules():
    # qconfig and details together are an error (fa3_quant 配置说明 §2.1 constraint)
    with pytest.raises(faq.FaQuantError) as e:
        faq.resolve_fa3_config(faq.QConfig("fp8_e4m3", "per_token"), {"fa_q": None})
    assert e.value.status == _abi.FAQ_ERR_CONFIG_CONFLICT
    # neither: int8 / per_head / symmetric / minmax for all three branches
    d = faq.resolve_fa3_config()
    assert all(c == faq.QConfig("int8", "per_head", True, "minmax") for c in d.values())
    # details: unlisted branches stay unquantized
    d = faq.resolve_fa3_config(details={"fa_k": faq.QConfig("fp8_e4m3", "per_token")})
    assert d["fa_q"] is None and d["fa_v"] is None and d["fa_k"].dtype == "fp8_e4m3"
    with pytest.raises(faq.FaQuantError):
        faq.resolve_fa3_config(details={"fa_x": None})


def test_package_has_no_oracle_dependency():
    import sys
    pkg_dir = os.path.join(ROOT, "quantized_attention_fa_amd")
    for dirpath, _, files in os.walk(pkg_dir):
        for f in files:
            if f.endswith((".py", ".hip", ".h", ".cpp")):
                text = open(os.path.join(dirpath, f), encoding="utf-8").read()
                assert "oracle" not in re.findall(r"\bimport\s+(\w+)|from\s+(\w+)", text).__str__(), f
