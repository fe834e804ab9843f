"""GPU parity of decode: a few queries per head (Sq = 1..16) against a long
quantized key/value cache.  Such calls split the keys across workgroups on
128-key tile boundaries and merge the partial results; since probabilities
are quantized per tile against the tile's own maximum, the merged output
must meet the same bar against the oracle as an unsplit call.  Every mode,
unquantized V and no quantization, ragged cache lengths, BSND operands."""

import numpy as np
import pytest
import torch

import quantized_attention_fa_amd as faq
from synth import make_inputs
from gpu_helpers import GpuRun, bf16_of, check_attention, oracle_attention, small_workload

pytestmark = pytest.mark.gpu

DECODE = [
    (2, (1, 2, 1000, 128), 1, None),
    (2, (2, 3, 777, 128), 16, None),
    (2, (2, 3, 777, 64), 16, None),
    (3, (1, 2, 1000, 128), 5, None),
    (4, (1, 2, 1000, 128), 16, None),
    (5, (1, 2, 1100, 128), 16, None),
    (6, (1, 2, 1000, 64), 3, None),
    (7, (1, 2, 777, 128), 16, None),
    (8, (1, 2, 1000, 128), 1, None),
    (3, (1, 2, 1000, 128), 16, ("fp8_token", "fp8_token", "float")),
    (2, (1, 2, 1000, 128), 7, ("float", "float", "float")),
    (2, (2, 2, 1000, 128), 16, ("fp8_token", "int8_head", "int8_head")),
    (4, (1, 2, 1000, 64), 4, ("float", "mxfp4", "fp8_token")),
    # a long sequence over few heads splits keys too (Sq = Skv, not causal)
    (3, (1, 2, 1024, 64), None, None),
]


@pytest.mark.parametrize("cfg,shape,q_len,modes", DECODE)
def test_decode_against_oracle(cfg, shape, q_len, modes):
    w = small_workload(cfg, shape, q_len=q_len)
    run = GpuRun(w, modes=modes)
    o32 = run.attention(torch.float32, causal=False).cpu().numpy()
    assert o32.shape == (shape[0], shape[1], q_len or shape[2], shape[3])
    check_attention(o32, oracle_attention(run, causal=False), f"decode cfg{cfg} {shape} q_len={q_len} {modes}")
    o16 = run.attention(torch.bfloat16, causal=False)
    assert np.array_equal(o16.view(torch.int16).cpu().numpy(), bf16_of(o32))


@pytest.mark.parametrize("cfg", [7, 2])
def test_decode_bsnd_equals_bnsd(cfg):
    w = small_workload(cfg, (2, 3, 1000, 128), q_len=9)
    run = GpuRun(w)
    ref = run.attention(torch.float32, causal=False)
    bs = lambda qt: faq.QTensor(qt.cfg, qt.shape, qt.codes.permute(0, 2, 1, 3).contiguous(), qt.scales, "bsnd")
    o = faq.fa_quant_attention(bs(run.qt[0]), bs(run.qt[1]), bs(run.qt[2]), out_dtype=torch.float32)
    torch.cuda.synchronize()
    assert torch.equal(o.permute(0, 2, 1, 3), ref)


def test_decode_full_size():
    w = make_inputs(11)
    run = GpuRun(w)
    o = run.attention(torch.float32).cpu().numpy()
    check_attention(o, oracle_attention(run), "int8 per-head decode, full size")
