"""GPU checks of the BSND layout ("量化" page, 注意事项: Q/K/V in BNSD or BSND).
Quantizing a BSND tensor must give the same codes (in BSND) and the same
scales as quantizing its BNSD copy, bit for bit; attention on BSND operands
(all or some of them) must give exactly the BNSD result, in Q's layout; one
case is also checked against the oracle directly."""

import numpy as np
import pytest
import torch

import quantized_attention_fa_amd as faq
from gpu_helpers import DEV, GpuRun, MODE_CFG, STATIC_DTYPE, check_attention, oracle_attention, small_workload

pytestmark = pytest.mark.gpu

MODES = [(2, "int8_head"), (6, "fp8_head"), (3, "fp8_token"), (7, "int8_token"), (4, "mxfp4"), (8, "mxfp8"),
         (5, "rot_fp8_block")]


def _bsnd(t):
    return t.permute(0, 2, 1, 3).contiguous()


@pytest.mark.parametrize("cfg,mode", MODES)
@pytest.mark.parametrize("shape", [(1, 3, 300, 128), (2, 2, 257, 64)])
def test_quantize_bsnd_equals_bnsd(cfg, mode, shape):
    w = small_workload(cfg, shape)
    for br, x in enumerate((w.q, w.k, w.v)):
        xb = x.to(DEV)
        xs = _bsnd(xb)
        static = None
        if mode in STATIC_DTYPE:
            a1 = torch.zeros(shape[1], dtype=torch.float32, device=DEV)
            a2 = torch.zeros(shape[1], dtype=torch.float32, device=DEV)
            faq.fa_quant_calibrate(xb, a1)
            faq.fa_quant_calibrate(xs, a2, layout="bsnd")
            assert torch.equal(a1, a2)
            static = faq.fa_quant_scales_from_amax(a1, STATIC_DTYPE[mode]) * 0.9  # some values saturate
        cfgq = MODE_CFG[mode](w.spec, br)
        rot = w.rot.to(DEV) if (w.rot is not None and br < 2) else None
        d1 = torch.empty_like(xb) if rot is not None else None
        d2 = torch.empty_like(xs) if rot is not None else None
        q1 = faq.fa_quantize(xb, cfgq, static_scale=static, rot=rot, debug_rotated=d1)
        q2 = faq.fa_quantize(xs, cfgq, static_scale=static, rot=rot, debug_rotated=d2, layout="bsnd")
        torch.cuda.synchronize()
        assert q2.codes.shape[1] == shape[2]  # codes are BSND
        assert torch.equal(_bsnd(q2.codes), q1.codes), (mode, br)
        assert torch.equal(q2.scales, q1.scales), (mode, br)
        if rot is not None:
            assert torch.equal(_bsnd(d2), d1)


def _to_layout(qt, layout):
    if layout == "bnsd":
        return qt
    return faq.QTensor(qt.cfg, qt.shape, _bsnd(qt.codes), qt.scales, "bsnd")


CASES = [
    (2, (1, 3, 300, 128), True, None),
    (3, (2, 2, 257, 64), False, None),
    (4, (1, 3, 300, 128), False, None),
    (5, (1, 2, 384, 128), False, None),
    (7, (1, 3, 300, 128), True, None),
    (8, (1, 2, 257, 128), False, None),
    (6, (1, 3, 300, 128), False, ("fp8_head", "fp8_head", "float")),
    (3, (1, 3, 300, 128), False, ("float", "float", "float")),
]


@pytest.mark.parametrize("cfg,shape,causal,modes", CASES)
@pytest.mark.parametrize("layouts", [("bsnd", "bsnd", "bsnd"), ("bsnd", "bnsd", "bsnd"), ("bnsd", "bsnd", "bnsd")])
def test_attention_bsnd_equals_bnsd(cfg, shape, causal, modes, layouts):
    w = small_workload(cfg, shape)
    run = GpuRun(w, modes=modes)
    ref32 = run.attention(torch.float32, causal=causal)
    ref16 = run.attention(torch.bfloat16, causal=causal)
    q, k, v = (_to_layout(t, l) for t, l in zip(run.qt, layouts))
    o32 = faq.fa_quant_attention(q, k, v, causal=causal, out_dtype=torch.float32)
    o16 = faq.fa_quant_attention(q, k, v, causal=causal, out_dtype=torch.bfloat16)
    torch.cuda.synchronize()
    if layouts[0] == "bsnd":
        assert o32.shape[1] == shape[2]
        o32, o16 = _bsnd(o32), _bsnd(o16)
    assert torch.equal(o32, ref32)
    assert torch.equal(o16, ref16)
    if layouts == ("bsnd", "bsnd", "bsnd") and cfg == 3 and modes is None:
        check_attention(o32.cpu().numpy(), oracle_attention(run, causal=causal), "bsnd vs oracle")


@pytest.mark.parametrize("cfg", [2, 3])
def test_full_size_bsnd_equals_bnsd(cfg):
    """At the bench's full sizes (INT8 per-head prefill: four-wave kernel;
    FP8 per-token video: ping-pong kernel): quantizing the BSND inputs gives
    the BSND codes and the same scales, and attention on BSND operands gives
    the BNSD result bit for bit, in BSND."""
    from synth import make_inputs
    w = make_inputs(cfg)
    run = GpuRun(w)
    for br, x in enumerate(run.x):
        qt = faq.fa_quantize(_bsnd(x), run.qt[br].cfg, static_scale=run.static[br], layout="bsnd")
        torch.cuda.synchronize()
        assert torch.equal(_bsnd(qt.codes), run.qt[br].codes), br
        assert torch.equal(qt.scales, run.qt[br].scales), br
        del qt
    ref32 = run.attention(torch.float32)
    q, k, v = (_to_layout(t, "bsnd") for t in run.qt)
    o32 = faq.fa_quant_attention(q, k, v, causal=w.spec["causal"], out_dtype=torch.float32)
    torch.cuda.synchronize()
    assert o32.shape[1] == w.shape[2]
    assert torch.equal(_bsnd(o32), ref32)
