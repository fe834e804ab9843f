"""ctypes declarations of the C ABI in include/fa_quant.h."""

import ctypes
import os

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libfaquant.so")
PROBE_LIB_PATH = os.path.join(_PKG, "libfaquant_probe.so")

# faq_status
FAQ_OK = 0
FAQ_ERR_INVALID_ARG = -1
FAQ_ERR_UNSUPPORTED = -2
FAQ_ERR_CONFIG_CONFLICT = -3
FAQ_ERR_NOT_CALIBRATED = -4
FAQ_ERR_SHAPE = -5
FAQ_ERR_HIP = -6
FAQ_ERR_WORKSPACE = -7

# faq_dtype
FAQ_FLOAT, FAQ_INT8, FAQ_FP8_E4M3, FAQ_MXFP4, FAQ_MXFP8 = 0, 1, 2, 3, 4
FAQ_LAYOUT_BNSD, FAQ_LAYOUT_BSND = 0, 1
# faq_scope
FAQ_PER_HEAD, FAQ_PER_TOKEN, FAQ_PER_BLOCK, FAQ_PER_TOKEN_BLOCK = 0, 1, 2, 3
# faq_tdtype
FAQ_T_F32, FAQ_T_BF16 = 0, 1

EXPORTS = (
    "fa_quant_codes_bytes",
    "fa_quant_scales_bytes",
    "fa_quant_calibrate",
    "fa_quant_scales_from_amax",
    "fa_quantize",
    "fa_quant_attention_workspace_bytes",
    "fa_quant_attention",
    "fa_quant_attention_static_ws",
    "fa_quant_status_string",
)
FA_QUANT_STATIC_WORKSPACE_BYTES = 64 << 20


class faq_qconfig(ctypes.Structure):
    _fields_ = [
        ("dtype", ctypes.c_int32),
        ("scope", ctypes.c_int32),
        ("symmetric", ctypes.c_int32),
        ("method", ctypes.c_int32),
        ("block_tokens", ctypes.c_int32),
    ]


class faq_shape(ctypes.Structure):
    _fields_ = [("B", ctypes.c_int64), ("H", ctypes.c_int64), ("S", ctypes.c_int64), ("D", ctypes.c_int64),
                ("layout", ctypes.c_int64)]


class faq_qtensor(ctypes.Structure):
    _fields_ = [
        ("cfg", faq_qconfig),
        ("shape", faq_shape),
        ("codes", ctypes.c_void_p),
        ("scales", ctypes.c_void_p),
    ]


_P = ctypes.POINTER
_vp = ctypes.c_void_p


def _declare(lib):
    lib.fa_quant_codes_bytes.argtypes = [_P(faq_qconfig), _P(faq_shape)]
    lib.fa_quant_codes_bytes.restype = ctypes.c_size_t
    lib.fa_quant_scales_bytes.argtypes = [_P(faq_qconfig), _P(faq_shape)]
    lib.fa_quant_scales_bytes.restype = ctypes.c_size_t
    lib.fa_quant_calibrate.argtypes = [_vp, ctypes.c_int32, _P(faq_shape), _vp, _vp]
    lib.fa_quant_calibrate.restype = ctypes.c_int32
    lib.fa_quant_scales_from_amax.argtypes = [_vp, ctypes.c_int64, ctypes.c_int32, _vp, _vp]
    lib.fa_quant_scales_from_amax.restype = ctypes.c_int32
    lib.fa_quantize.argtypes = [_vp, ctypes.c_int32, _P(faq_shape), _P(faq_qconfig), _vp, _vp,
                                _P(faq_qtensor), _vp, _vp]
    lib.fa_quantize.restype = ctypes.c_int32
    lib.fa_quant_attention_workspace_bytes.argtypes = [_P(faq_qtensor)] * 3
    lib.fa_quant_attention_workspace_bytes.restype = ctypes.c_size_t
    lib.fa_quant_attention.argtypes = [_P(faq_qtensor), _P(faq_qtensor), _P(faq_qtensor), ctypes.c_float,
                                       ctypes.c_int32, _vp, ctypes.c_int32, _vp, ctypes.c_size_t, _vp]
    lib.fa_quant_attention.restype = ctypes.c_int32
    lib.fa_quant_attention_static_ws.argtypes = [_P(faq_qtensor), _P(faq_qtensor), _P(faq_qtensor), ctypes.c_float,
                                                 ctypes.c_int32, _vp, ctypes.c_int32, _vp]
    lib.fa_quant_attention_static_ws.restype = ctypes.c_int32
    lib.fa_quant_status_string.argtypes = [ctypes.c_int32]
    lib.fa_quant_status_string.restype = ctypes.c_char_p
    return lib


_LIB = None


def lib():
    """The loaded product library.  There is no fallback: a missing build is
    an error."""
    global _LIB
    if _LIB is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(
                f"{LIB_PATH} is missing: build it with `python -m quantized_attention_fa_amd.build`")
        _LIB = _declare(ctypes.CDLL(LIB_PATH))
    return _LIB


def probe_lib():
    if not os.path.exists(PROBE_LIB_PATH):
        raise RuntimeError(f"{PROBE_LIB_PATH} is missing: build the package first")
    return ctypes.CDLL(PROBE_LIB_PATH)
