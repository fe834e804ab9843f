"""fa_quant_attention_static_ws (the entry point for callers that cannot
allocate: its workspace is a static per-GPU array) against
fa_quant_attention on the same quantized operands, through the C ABI: the
two run the same kernels, so the outputs must be equal bit for bit.  Each
case makes two calls in a row, the second on a smaller input (the array
keeps the first call's contents, which the second must never read), and a
call whose workspace need exceeds the array is refused before any launch."""

import numpy as np
import pytest
import torch

import quantized_attention_fa_amd as faq
from quantized_attention_fa_amd import _abi
from synth import make_inputs

pytestmark = pytest.mark.gpu

DEV = "cuda:0"
STATIC = {"int8_head": "int8", "fp8_head": "fp8_e4m3"}


def _cfg(mode):
    return {"int8_head": faq.QConfig("int8", "per_head"), "fp8_token": faq.QConfig("fp8_e4m3", "per_token"),
            "mxfp4": faq.QConfig("mxfp4", "per_block"), "int8_token": faq.QConfig("int8", "per_token")}[mode]


def _operands(cfg, shape, mode, q_len=None):
    w = make_inputs(cfg, shape=shape, calib_batch=1, q_len=q_len)
    qts = []
    for br, x in enumerate((w.q, w.k, w.v)):
        x = x.to(DEV)
        sc = None
        if mode in STATIC:
            amax = torch.zeros(shape[1], dtype=torch.float32, device=DEV)
            faq.fa_quant_calibrate(x, amax)
            sc = faq.fa_quant_scales_from_amax(amax, STATIC[mode])
        qts.append(faq.fa_quantize(x, _cfg(mode), static_scale=sc))
    return qts


def _both(qts, causal, out_dtype=torch.float32):
    ref = faq.fa_quant_attention(*qts, causal=causal, out_dtype=out_dtype)
    got = torch.full_like(ref, float("nan"))
    faq.fa_quant_attention_static_ws(*qts, out=got, causal=causal)
    torch.cuda.synchronize()
    return ref, got


# (workload, first shape, second (smaller) shape, mode, causal, q_len):
# FP8 per-token (K / V^T re-layout images), MXFP4 (V^T image, K exponents),
# INT8 per-token (multipliers and sigma), INT8 per-head decode (key-split
# partial results and their merge)
CASES = [
    (3, (1, 4, 2048, 128), (1, 2, 700, 64), "fp8_token", False, None),
    (4, (1, 4, 1536, 128), (1, 1, 300, 128), "mxfp4", False, None),
    (7, (2, 2, 1024, 128), (1, 2, 257, 128), "int8_token", True, None),
    (2, (2, 4, 4096, 128), (1, 2, 1000, 128), "int8_head", False, 16),
]


@pytest.mark.parametrize("cfg,big,small,mode,causal,q_len", CASES)
def test_static_workspace_matches_workspace_entry(cfg, big, small, mode, causal, q_len):
    first = _operands(cfg, big, mode, q_len)
    need = faq.fa_quant_attention_workspace_bytes(*first)
    assert 0 < need <= _abi.FA_QUANT_STATIC_WORKSPACE_BYTES
    ref1, got1 = _both(first, causal)
    second = _operands(cfg, small, mode, q_len)
    ref2, got2 = _both(second, causal)
    assert torch.equal(ref1, got1), f"first call ({big})"
    assert torch.equal(ref2, got2), f"second, smaller call ({small})"
    # bf16 output through the static workspace too
    ref3, got3 = _both(second, causal, torch.bfloat16)
    assert torch.equal(ref3.view(torch.int16), got3.view(torch.int16))


def test_static_workspace_too_small_is_refused():
    # FP8 per-token [1,24,8192,128]: the bf16 K image and the V^T codes of
    # 1536 key tiles need 72 MiB, more than the array holds
    qts = _operands(3, (1, 24, 8192, 128), "fp8_token")
    assert faq.fa_quant_attention_workspace_bytes(*qts) > _abi.FA_QUANT_STATIC_WORKSPACE_BYTES
    out = torch.full((1, 24, 8192, 128), 7.0, dtype=torch.float32, device=DEV)
    with pytest.raises(faq.FaQuantError) as e:
        faq.fa_quant_attention_static_ws(*qts, out=out)
    assert e.value.status == _abi.FAQ_ERR_WORKSPACE
    torch.cuda.synchronize()
    assert bool((out == 7.0).all())  # nothing was launched
