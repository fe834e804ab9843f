"""GPU parity of the quantized attention in every FA mode (INT8 / FP8
per-head, INT8 / FP8 per-token, MXFP4 / MXFP8 per-block, rotate + FP8 token
blocks): the HIP output (fp32) against the oracle run on the same quantized
codes - relative Frobenius <= 1e-3 and
max |error| <= 2e-3 + tie allowance - on multi-tile shapes with ragged tails,
causal and not, and at the full workload sizes on sampled query rows.  The
bf16 output must be the round-to-nearest-even of the fp32 output, bit for
bit."""

import numpy as np
import pytest
import torch

from synth import make_inputs, sample_rows
from gpu_helpers import GpuRun, bf16_of, check_attention, oracle_attention, small_workload

pytestmark = pytest.mark.gpu

SMALL = [
    (1, (1, 2, 128, 64), False),
    (1, (1, 2, 300, 64), False),
    (2, (1, 2, 300, 128), True),
    (2, (2, 2, 384, 128), True),
    (2, (1, 1, 200, 64), True),
    (3, (1, 2, 300, 128), False),
    (3, (1, 2, 257, 64), False),
    (3, (1, 2, 384, 128), True),
    (4, (1, 2, 300, 128), False),
    (4, (1, 2, 256, 64), False),
    (4, (1, 2, 300, 128), True),
    (5, (1, 2, 300, 128), False),
    (5, (1, 2, 640, 128), True),
    (6, (1, 2, 300, 128), True),
    (6, (1, 2, 257, 64), False),
    (7, (1, 2, 300, 128), False),
    (7, (1, 2, 257, 64), False),
    (7, (1, 2, 384, 128), True),
    (8, (1, 2, 300, 128), False),
    (8, (1, 2, 256, 64), False),
    (8, (1, 2, 300, 128), True),
]


@pytest.mark.parametrize("cfg,shape,causal", SMALL)
def test_attention_small(cfg, shape, causal):
    w = small_workload(cfg, shape)
    run = GpuRun(w)
    o32 = run.attention(torch.float32, causal=causal).cpu().numpy()
    ref = oracle_attention(run, causal=causal)
    check_attention(o32, ref, f"cfg{cfg} {shape} causal={causal}")
    o16 = run.attention(torch.bfloat16, causal=causal)
    assert np.array_equal(o16.view(torch.int16).cpu().numpy(), bf16_of(o32))


def test_attention_custom_scale_and_determinism():
    w = small_workload(3, (1, 2, 300, 128))
    run = GpuRun(w)
    a = run.attention(torch.float32, sm_scale=0.05).cpu().numpy()
    b = run.attention(torch.float32, sm_scale=0.05).cpu().numpy()
    assert np.array_equal(a, b)  # run twice, bitwise equal
    check_attention(a, oracle_attention(run, sm_scale=0.05), "sm_scale 0.05")


@pytest.mark.parametrize("cfg,rows_per_bh", [(1, None), (2, 24), (3, 8), (4, 24), (5, 8), (6, 24), (7, 8),
                                             (8, 24)])
def test_full_size_attention(cfg, rows_per_bh):
    w = make_inputs(cfg)
    run = GpuRun(w)
    o = run.attention(torch.float32)
    S = w.shape[2]
    rows = None if rows_per_bh is None else sample_rows(cfg, S, rows_per_bh, edge=4)
    got = o.cpu().numpy() if rows is None else o[:, :, torch.from_numpy(rows).to(o.device)].cpu().numpy()
    check_attention(got, oracle_attention(run, rows=rows), f"cfg{cfg} full size")
