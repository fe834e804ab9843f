"""Degenerate and extreme cases on the GPU, every mode, against the oracle:
all-zero tensors (scale 1, codes 0, uniform attention over zero values), a
single key, a single query, a one-key ragged last tile, score ranges so wide
that each row's softmax is one-hot, and calls with nothing to compute."""

import numpy as np
import pytest
import torch

import quantized_attention_fa_amd as faq
from gpu_helpers import DEV, GpuRun, check_attention, oracle_attention, small_workload

pytestmark = pytest.mark.gpu

MODES = [(2, "int8_head"), (6, "fp8_head"), (3, "fp8_token"), (7, "int8_token"), (4, "mxfp4"), (8, "mxfp8"),
         (5, "rot_fp8_block"), (3, "float")]


def _run(cfg, mode, shape, q_len=None, scale_q=1.0, zero=False):
    w = small_workload(cfg, shape, q_len=q_len)
    if zero:
        w.q.zero_(); w.k.zero_(); w.v.zero_()
        for c in w.calib:
            for t in c:
                t.zero_()
    if scale_q != 1.0:
        w.q.mul_(scale_q)
        for t in (w.calib[0] if w.calib else []):
            t.mul_(scale_q)
    return GpuRun(w, modes=None if mode != "float" else ("float",) * 3)


@pytest.mark.parametrize("cfg,mode", MODES)
def test_all_zero_tensors(cfg, mode):
    run = _run(cfg, mode, (1, 2, 200, 128), zero=True)
    for br in range(3):
        if mode != "float":
            assert int(run.qt[br].codes.abs().max() if run.qt[br].codes.dtype == torch.int8
                       else (run.qt[br].codes & 0x7F).max()) == 0
    o = run.attention(torch.float32, causal=False).cpu().numpy()
    assert not np.isnan(o).any() and np.all(o == 0)
    check_attention(o, oracle_attention(run, causal=False), f"zeros {mode}")


@pytest.mark.parametrize("cfg,mode", MODES)
@pytest.mark.parametrize("shape,q_len,causal", [((1, 2, 1, 128), None, False), ((1, 2, 1, 64), None, True),
                                                ((2, 1, 129, 128), 3, False), ((1, 3, 1, 128), 1, False)])
def test_tiny_and_ragged(cfg, mode, shape, q_len, causal):
    run = _run(cfg, mode, shape, q_len=q_len)
    o = run.attention(torch.float32, causal=causal).cpu().numpy()
    check_attention(o, oracle_attention(run, causal=causal), f"{mode} {shape} q_len={q_len} causal={causal}")
    if shape[2] == 1:  # one key: the output is that key's (dequantized) value
        from gpu_helpers import dequant
        v, _ = dequant(run, 2)
        assert np.allclose(o, np.broadcast_to(v, o.shape), rtol=0, atol=2e-3 * max(1.0, np.abs(v).max()))


@pytest.mark.parametrize("cfg,mode", MODES)
def test_one_hot_softmax(cfg, mode):
    """Q scaled by 200: score gaps of hundreds, every row's weights are one
    key; no overflow, no NaN."""
    run = _run(cfg, mode, (1, 2, 300, 128), scale_q=200.0)
    o = run.attention(torch.float32, causal=False).cpu().numpy()
    check_attention(o, oracle_attention(run, causal=False), f"one-hot {mode}")


def test_nothing_to_compute():
    w = small_workload(3, (1, 2, 256, 128))
    run = GpuRun(w)
    q0 = faq.QTensor(run.qt[0].cfg, (1, 2, 0, 128), run.qt[0].codes[:, :, :0], run.qt[0].scales)
    out = faq.fa_quant_attention(q0, run.qt[1], run.qt[2], out_dtype=torch.float32)
    assert out.numel() == 0
    x = torch.empty((0, 2, 64, 128), dtype=torch.bfloat16, device=DEV)
    qt = faq.fa_quantize(x, faq.QConfig("mxfp8", "per_block"))
    assert qt.codes.numel() == 0
    k0 = faq.QTensor(run.qt[1].cfg, (1, 2, 0, 128), run.qt[1].codes[:, :, :0], run.qt[1].scales)
    with pytest.raises(faq.FaQuantError):
        faq.fa_quant_attention(run.qt[0], k0, k0)


@pytest.mark.parametrize("shift,q_len,causal,S", [(30, None, False, 256), (50, None, False, 256),
                                                  (30, 5, False, 640), (40, None, True, 384)])
def test_mxfp4_value_exponent_spread(shift, q_len, causal, S):
    """MXFP4 values whose 32-key groups span more binades than one E5M2
    image holds: the odd keys' V rows are scaled by 2^-shift (a group's
    exponents then spread over shift + ~3 binades), and Q and K put the
    weight on those keys (scores ~11 above the even keys', whose
    probabilities quantize to 0), so every output comes from the small
    elements and the relative error sees them.  Spreads up to 57 are exact
    through the second image; also with key splits (a short query set: a
    split starts past tile 0) and under the causal mask."""
    w = small_workload(4, (1, 2, S, 128), q_len=q_len)
    g = torch.Generator().manual_seed(101 + shift)
    B, H, Sq, D = w.q.shape
    u = torch.randn((1, H, 1, D), generator=g)
    u = u / u.norm(dim=-1, keepdim=True)
    sign = torch.where(torch.arange(S) % 2 == 1, 1.0, -1.0).reshape(1, 1, S, 1)
    q = 8.0 * u + 0.3 * torch.randn((B, H, Sq, D), generator=g)
    k = 8.0 * sign * u + 0.3 * torch.randn((B, H, S, D), generator=g)
    v = w.v.float() * torch.where(torch.arange(S) % 2 == 1, 2.0 ** -shift, 1.0).reshape(1, 1, S, 1)
    w.q.copy_(q.to(w.q.dtype)); w.k.copy_(k.to(w.k.dtype)); w.v.copy_(v.to(w.v.dtype))
    run = GpuRun(w)
    o = run.attention(torch.float32, causal=causal).cpu().numpy()
    o_ref, T, n_tie = oracle_attention(run, causal=causal)
    # the outputs are the small elements', except, under the causal mask,
    # rows at a 32-key group start (row 0, 32, ...): the last group they see
    # holds one even key alone, whose probability takes that group's
    # exponent and a nonzero code; those rows are checked on their own
    big = (np.arange(Sq) % 32 == 0) if causal else np.zeros(Sq, bool)
    assert np.abs(o_ref[:, :, ~big]).max() < 2.0 ** (-shift + 6)
    for h in range(H):
        sl = (slice(None), slice(h, h + 1), ~big)
        check_attention(o[sl], (o_ref[sl], T[sl], n_tie), f"mxfp4 V spread 2^-{shift} q_len={q_len} causal={causal} head {h}")
    if causal:
        sl = (slice(None), slice(None), big)
        check_attention(o[sl], (o_ref[sl], T[sl], n_tie), f"mxfp4 V spread 2^-{shift} causal group-start rows")
