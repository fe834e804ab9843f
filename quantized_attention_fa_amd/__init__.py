"""MI355X-native FA quantization: quantize Q/K/V and attend on low-bit operands.

Thin Python layer over the C ABI of ``include/fa_quant.h`` (ctypes).  It only
marshals arguments - torch supplies device memory and the current stream;
every step of the computation runs in the HIP kernels of ``libfaquant.so``.

Configuration follows the msModelSlim ``fa3_quant`` processor page
("fa3_quant 配置说明"): §2.1 FA3QuantProcessorConfig (``qconfig`` and
``details`` are mutually exclusive; with neither, the default is int8 /
per_head / symmetric / minmax), §2.2 QConfig fields, §2.3 FA3AttentionDetails
(per-branch fa_q / fa_k / fa_v; an unconfigured branch is not quantized).
"""

import ctypes
from dataclasses import dataclass, field
from typing import Dict, Optional

import torch

from . import _abi
from ._abi import (FAQ_FP8_E4M3, FAQ_INT8, FAQ_MXFP4, FAQ_MXFP8, FAQ_FLOAT, FAQ_PER_BLOCK, FAQ_PER_HEAD,
                   FAQ_PER_TOKEN, FAQ_PER_TOKEN_BLOCK, FAQ_T_BF16, FAQ_T_F32)

__all__ = [
    "QConfig", "QTensor", "FaQuantError", "resolve_fa3_config", "default_qconfig", "float_branch",
    "fa_quant_calibrate", "fa_quant_scales_from_amax", "fa_quantize",
    "fa_quant_attention", "fa_quant_attention_workspace_bytes", "fa_quant_attention_static_ws",
    "fa_quant_codes_bytes", "fa_quant_scales_bytes", "fa_quant_status_string",
]

_DTYPES = {"float": FAQ_FLOAT, "int8": FAQ_INT8, "fp8_e4m3": FAQ_FP8_E4M3, "mxfp4": FAQ_MXFP4,
           "mxfp8": FAQ_MXFP8}
_SCOPES = {"per_head": FAQ_PER_HEAD, "per_token": FAQ_PER_TOKEN, "per_block": FAQ_PER_BLOCK,
           "per_token_block": FAQ_PER_TOKEN_BLOCK}
_METHODS = {"minmax": 0}
# Q/K/V memory layouts ("量化" page, 注意事项: BNSD and BSND)
_LAYOUTS = {"bnsd": _abi.FAQ_LAYOUT_BNSD, "bsnd": _abi.FAQ_LAYOUT_BSND}


class FaQuantError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        super().__init__(f"{where}: {fa_quant_status_string(status)} (status {status})")


@dataclass(frozen=True)
class QConfig:
    """One tensor's quantization ("fa3_quant 配置说明" §2.2)."""
    dtype: str
    scope: str
    symmetric: bool = True
    method: str = "minmax"
    block_tokens: int = 0  # per_token_block only

    def to_c(self) -> _abi.faq_qconfig:
        if self.dtype not in _DTYPES or self.scope not in _SCOPES:
            raise FaQuantError(_abi.FAQ_ERR_UNSUPPORTED, f"QConfig({self.dtype}, {self.scope})")
        method = _METHODS.get(self.method, -1)
        return _abi.faq_qconfig(_DTYPES[self.dtype], _SCOPES[self.scope], int(bool(self.symmetric)),
                                method, int(self.block_tokens))


def default_qconfig() -> QConfig:
    """The fa3_quant default when no qconfig is given (§2.1)."""
    return QConfig("int8", "per_head", True, "minmax")


def resolve_fa3_config(qconfig: Optional[QConfig] = None,
                       details: Optional[Dict[str, Optional[QConfig]]] = None) -> Dict[str, Optional[QConfig]]:
    """Per-branch configs {fa_q, fa_k, fa_v} from a processor config: qconfig
    and details together are an error; neither gives the default for all three
    branches; details leaves unlisted branches unquantized (None)."""
    if qconfig is not None and details is not None:
        raise FaQuantError(_abi.FAQ_ERR_CONFIG_CONFLICT, "resolve_fa3_config")
    if details is not None:
        unknown = set(details) - {"fa_q", "fa_k", "fa_v"}
        if unknown:
            raise FaQuantError(_abi.FAQ_ERR_INVALID_ARG, f"resolve_fa3_config: unknown branch {sorted(unknown)}")
        return {b: details.get(b) for b in ("fa_q", "fa_k", "fa_v")}
    q = qconfig if qconfig is not None else default_qconfig()
    return {"fa_q": q, "fa_k": q, "fa_v": q}


@dataclass
class QTensor:
    """Quantized tensor: device codes + scales and their config.  `shape` is
    the logical (B, H, S, D); the codes are laid out as `layout` ("bnsd" or
    "bsnd"); scales are indexed (b, h, s)."""
    cfg: QConfig
    shape: tuple
    codes: torch.Tensor
    scales: torch.Tensor
    layout: str = "bnsd"

    def to_c(self) -> _abi.faq_qtensor:
        return _abi.faq_qtensor(self.cfg.to_c(), _abi.faq_shape(*self.shape, _LAYOUTS[self.layout]),
                                self.codes.data_ptr(), self.scales.data_ptr())


def float_branch(x: torch.Tensor, layout: str = "bnsd") -> QTensor:
    """An unquantized branch ("fa3_quant 配置说明" §2.3: a branch without a
    configuration is not quantized): the bf16 tensor itself, passed to
    fa_quant_attention as a QTensor of dtype "float" (no scales)."""
    shape = _bnsd(x, "float_branch", layout)
    if x.dtype != torch.bfloat16:
        raise FaQuantError(_abi.FAQ_ERR_UNSUPPORTED, "float_branch: unquantized branches are bf16")
    return QTensor(QConfig("float", "per_head"), shape, x, torch.empty(0, dtype=torch.uint8, device=x.device),
                   layout)


def fa_quant_status_string(status: int) -> str:
    return _abi.lib().fa_quant_status_string(int(status)).decode()


def _check(status: int, where: str):
    if status != _abi.FAQ_OK:
        raise FaQuantError(status, where)


def _stream(t: torch.Tensor):
    return ctypes.c_void_p(torch.cuda.current_stream(t.device).cuda_stream)


def _tdtype(t: torch.Tensor) -> int:
    if t.dtype == torch.float32:
        return FAQ_T_F32
    if t.dtype == torch.bfloat16:
        return FAQ_T_BF16
    raise FaQuantError(_abi.FAQ_ERR_UNSUPPORTED, f"input dtype {t.dtype}")


def _bnsd(x: torch.Tensor, where: str, layout: str = "bnsd") -> tuple:
    """Logical (B, H, S, D) of a contiguous device tensor in `layout`."""
    if x.dim() != 4 or not x.is_contiguous() or not x.is_cuda:
        raise FaQuantError(_abi.FAQ_ERR_INVALID_ARG, f"{where}: need a contiguous CUDA 4-d tensor")
    if layout not in _LAYOUTS:
        raise FaQuantError(_abi.FAQ_ERR_INVALID_ARG, f"{where}: layout must be 'bnsd' or 'bsnd'")
    d = tuple(int(s) for s in x.shape)
    return d if layout == "bnsd" else (d[0], d[2], d[1], d[3])


def _physical(shape: tuple, layout: str, last: int) -> tuple:
    B, H, S, _ = shape
    return (B, H, S, last) if layout == "bnsd" else (B, S, H, last)


def _check_buffer(t: torch.Tensor, nbytes: int, device, where: str):
    """A caller-supplied device buffer: contiguous, on `device`, holding at
    least `nbytes` bytes (the C ABI cannot check sizes)."""
    if not isinstance(t, torch.Tensor) or not t.is_cuda or t.device != device or not t.is_contiguous():
        raise FaQuantError(_abi.FAQ_ERR_INVALID_ARG, f"{where}: need a contiguous CUDA tensor on {device}")
    if t.numel() * t.element_size() < nbytes:
        raise FaQuantError(_abi.FAQ_ERR_INVALID_ARG,
                           f"{where}: {t.numel() * t.element_size()} bytes, need {nbytes}")


def _check_qtensor(t: QTensor, device, where: str):
    """Codes and scales of a QTensor large enough for its config and shape."""
    if t.cfg.dtype == "float":
        B, H, S, D = t.shape
        _check_buffer(t.codes, 2 * B * H * S * D, device, f"{where} (bf16 values)")
        if t.codes.dtype != torch.bfloat16:
            raise FaQuantError(_abi.FAQ_ERR_UNSUPPORTED, f"{where}: unquantized branches are bf16")
        return
    c, s = t.cfg.to_c(), _abi.faq_shape(*t.shape, _LAYOUTS[t.layout])
    nc = int(_abi.lib().fa_quant_codes_bytes(ctypes.byref(c), ctypes.byref(s)))
    ns = int(_abi.lib().fa_quant_scales_bytes(ctypes.byref(c), ctypes.byref(s)))
    _check_buffer(t.codes, nc, device, f"{where} (codes)")
    _check_buffer(t.scales, ns, device, f"{where} (scales)")


def fa_quant_codes_bytes(cfg: QConfig, shape) -> int:
    c, s = cfg.to_c(), _abi.faq_shape(*shape)
    return int(_abi.lib().fa_quant_codes_bytes(ctypes.byref(c), ctypes.byref(s)))


def fa_quant_scales_bytes(cfg: QConfig, shape) -> int:
    c, s = cfg.to_c(), _abi.faq_shape(*shape)
    return int(_abi.lib().fa_quant_scales_bytes(ctypes.byref(c), ctypes.byref(s)))


def fa_quant_calibrate(x: torch.Tensor, amax: torch.Tensor, layout: str = "bnsd") -> torch.Tensor:
    """Running per-head max|x| into `amax` (float32 [H] on the device)."""
    shape = _bnsd(x, "fa_quant_calibrate", layout)
    if amax.dtype != torch.float32 or amax.numel() != shape[1] or not amax.is_cuda:
        raise FaQuantError(_abi.FAQ_ERR_INVALID_ARG, "fa_quant_calibrate: amax must be float32 [H] on the GPU")
    s = _abi.faq_shape(*shape, _LAYOUTS[layout])
    _check(_abi.lib().fa_quant_calibrate(x.data_ptr(), _tdtype(x), ctypes.byref(s), amax.data_ptr(), _stream(x)),
           "fa_quant_calibrate")
    return amax


def fa_quant_scales_from_amax(amax: torch.Tensor, dtype: str = "int8", out: torch.Tensor = None) -> torch.Tensor:
    if amax.dtype != torch.float32 or not amax.is_cuda or not amax.is_contiguous():
        raise FaQuantError(_abi.FAQ_ERR_INVALID_ARG, "fa_quant_scales_from_amax: amax must be contiguous float32 "
                                                     "on the GPU")
    out = torch.empty_like(amax) if out is None else out
    if out.dtype != torch.float32:
        raise FaQuantError(_abi.FAQ_ERR_INVALID_ARG, "fa_quant_scales_from_amax: out must be float32")
    _check_buffer(out, 4 * amax.numel(), amax.device, "fa_quant_scales_from_amax out")
    _check(_abi.lib().fa_quant_scales_from_amax(amax.data_ptr(), amax.numel(), _DTYPES[dtype], out.data_ptr(),
                                                _stream(amax)), "fa_quant_scales_from_amax")
    return out


def fa_quantize(x: torch.Tensor, cfg: QConfig, static_scale: torch.Tensor = None, rot: torch.Tensor = None,
                debug_rotated: torch.Tensor = None, out: QTensor = None, layout: str = "bnsd") -> QTensor:
    """Quantize one branch; x and its codes are laid out as `layout`."""
    shape = _bnsd(x, "fa_quantize", layout)
    lib = _abi.lib()
    c, s = cfg.to_c(), _abi.faq_shape(*shape, _LAYOUTS[layout])
    if out is None:
        nc = lib.fa_quant_codes_bytes(ctypes.byref(c), ctypes.byref(s))
        ns = lib.fa_quant_scales_bytes(ctypes.byref(c), ctypes.byref(s))
        if nc == 0 and ns == 0 and x.numel() > 0:
            raise FaQuantError(_abi.FAQ_ERR_UNSUPPORTED, f"fa_quantize: {cfg}")
        cdt = torch.int8 if cfg.dtype == "int8" else torch.uint8
        codes = torch.empty(nc, dtype=cdt, device=x.device)
        if cfg.dtype in ("mxfp4", "mxfp8"):
            cd = shape[3] // 2 if cfg.dtype == "mxfp4" else shape[3]
            codes = codes.view(*_physical(shape, layout, cd))
            scales = torch.empty(ns, dtype=torch.uint8, device=x.device).view(shape[0], shape[1], shape[2],
                                                                               shape[3] // 32)
        else:
            codes = codes.view(*_physical(shape, layout, shape[3]))
            scales = torch.empty(max(ns // 4, 0), dtype=torch.float32, device=x.device)
        out = QTensor(cfg, shape, codes, scales, layout)
    else:
        if out.cfg != cfg or tuple(out.shape) != shape or out.layout != layout:
            raise FaQuantError(_abi.FAQ_ERR_INVALID_ARG, "fa_quantize: out was made for another config, "
                                                         "shape or layout")
        _check_qtensor(out, x.device, "fa_quantize out")
    if static_scale is not None:
        _check_buffer(static_scale, 4 * shape[1], x.device, "fa_quantize static_scale")
    if rot is not None:
        _check_buffer(rot, 2 * shape[3] * shape[3], x.device, "fa_quantize rot")
    if debug_rotated is not None:
        _check_buffer(debug_rotated, 2 * x.numel(), x.device, "fa_quantize debug_rotated")
    qt = out.to_c()
    st = lib.fa_quantize(x.data_ptr(), _tdtype(x), ctypes.byref(s), ctypes.byref(c),
                         static_scale.data_ptr() if static_scale is not None else None,
                         rot.data_ptr() if rot is not None else None, ctypes.byref(qt),
                         debug_rotated.data_ptr() if debug_rotated is not None else None, _stream(x))
    _check(st, "fa_quantize")
    return out


def fa_quant_attention_workspace_bytes(q: QTensor, k: QTensor, v: QTensor) -> int:
    qc, kc, vc = q.to_c(), k.to_c(), v.to_c()
    return int(_abi.lib().fa_quant_attention_workspace_bytes(ctypes.byref(qc), ctypes.byref(kc), ctypes.byref(vc)))


def fa_quant_attention(q: QTensor, k: QTensor, v: QTensor, sm_scale: float = 0.0, causal: bool = False,
                       out_dtype=torch.bfloat16, out: torch.Tensor = None,
                       workspace: torch.Tensor = None) -> torch.Tensor:
    lib = _abi.lib()
    qc, kc, vc = q.to_c(), k.to_c(), v.to_c()
    dev = q.codes.device
    for t, name in ((q, "q"), (k, "k"), (v, "v")):
        _check_qtensor(t, dev, f"fa_quant_attention {name}")
    if out is None:
        out = torch.empty(_physical(q.shape, q.layout, q.shape[3]), dtype=out_dtype, device=dev)
    odt = FAQ_T_BF16 if out.dtype == torch.bfloat16 else FAQ_T_F32 if out.dtype == torch.float32 else -1
    if odt >= 0:
        B, H, Sq, D = q.shape
        _check_buffer(out, B * H * Sq * D * out.element_size(), dev, "fa_quant_attention out")
    need = int(lib.fa_quant_attention_workspace_bytes(ctypes.byref(qc), ctypes.byref(kc), ctypes.byref(vc)))
    if workspace is None:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=dev)
    else:
        _check_buffer(workspace, need, dev, "fa_quant_attention workspace")
    st = lib.fa_quant_attention(ctypes.byref(qc), ctypes.byref(kc), ctypes.byref(vc), float(sm_scale),
                                int(bool(causal)), out.data_ptr(), odt, workspace.data_ptr(),
                                workspace.numel(), _stream(out))
    _check(st, "fa_quant_attention")
    return out


def fa_quant_attention_static_ws(q: QTensor, k: QTensor, v: QTensor, out: torch.Tensor, sm_scale: float = 0.0,
                                 causal: bool = False) -> torch.Tensor:
    """fa_quant_attention without a workspace and without any allocation:
    the library's static per-GPU workspace (calls on one GPU must not
    overlap).  `out` is required (bf16 or float32, q's shape and layout)."""
    lib = _abi.lib()
    qc, kc, vc = q.to_c(), k.to_c(), v.to_c()
    dev = q.codes.device
    for t, name in ((q, "q"), (k, "k"), (v, "v")):
        _check_qtensor(t, dev, f"fa_quant_attention_static_ws {name}")
    odt = FAQ_T_BF16 if out.dtype == torch.bfloat16 else FAQ_T_F32 if out.dtype == torch.float32 else -1
    if odt >= 0:
        B, H, Sq, D = q.shape
        _check_buffer(out, B * H * Sq * D * out.element_size(), dev, "fa_quant_attention_static_ws out")
    st = lib.fa_quant_attention_static_ws(ctypes.byref(qc), ctypes.byref(kc), ctypes.byref(vc), float(sm_scale),
                                          int(bool(causal)), out.data_ptr(), odt, _stream(out))
    _check(st, "fa_quant_attention_static_ws")
    return out
