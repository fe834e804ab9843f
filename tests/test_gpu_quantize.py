"""GPU parity of the quantization kernels: codes and scales bit-exact against
the oracle, on small multi-tile shapes with ragged tails, on hand-built edge
values, and at the full workload sizes (sampled rows / blocks there)."""

import numpy as np
import pytest
import torch

import quantized_attention_fa_amd as faq
from oracle import formats as F
from oracle import quantize as OQ
from synth import CONFIGS, make_inputs
from gpu_helpers import DEV, GpuRun, _parity_log, oracle_pool_map, small_workload

pytestmark = pytest.mark.gpu


def _np(t):
    return t.to(torch.float32).cpu().numpy() if t.dtype == torch.bfloat16 else t.cpu().numpy()


@pytest.mark.parametrize("shape,dtype", [((1, 2, 128, 64), torch.float32), ((2, 3, 300, 128), torch.bfloat16),
                                         ((1, 4, 77, 64), torch.bfloat16), ((2, 2, 513, 128), torch.float32)])
def test_int8_per_head_small(shape, dtype):
    g = np.random.default_rng(sum(shape))
    x = (g.standard_normal(shape) * np.exp(g.standard_normal((1, shape[1], 1, 1)))).astype(np.float32)
    xt = torch.from_numpy(x).to(dtype)
    xn = _np(xt)
    amax = torch.zeros(shape[1], dtype=torch.float32, device=DEV)
    faq.fa_quant_calibrate(xt[:, :, : shape[2] // 2].contiguous().to(DEV), amax)
    faq.fa_quant_calibrate(xt.to(DEV), amax)
    ref_amax = OQ.calibrate_amax(xn, OQ.calibrate_amax(xn[:, :, : shape[2] // 2]))
    assert np.array_equal(amax.cpu().numpy(), ref_amax)
    sc = faq.fa_quant_scales_from_amax(amax, "int8")
    assert np.array_equal(sc.cpu().numpy(), OQ.int8_scales(ref_amax))
    # scales tighter than the data so some values clamp to -128 / 127
    tight = sc * 0.8
    qt = faq.fa_quantize(xt.to(DEV), faq.QConfig("int8", "per_head"), static_scale=tight)
    want = OQ.quantize_int8_per_head(xn, tight.cpu().numpy())
    assert np.array_equal(qt.codes.cpu().numpy(), want)
    assert np.array_equal(qt.scales.cpu().numpy(), tight.cpu().numpy())


def test_int8_divide_ties():
    """Quotients that sit within an ulp of a rounding tie (see
    tests/golden/divide_ties.txt): the GPU's division must be correctly
    rounded."""
    x = np.zeros((1, 1, 4, 64), np.float32)
    x[0, 0, 0, :4] = [72, 74, -72, 144]
    x[0, 0, 1, :3] = [148, 74, -74]
    sc = torch.tensor([np.float32(144) / np.float32(127)], device=DEV)
    qt = faq.fa_quantize(torch.from_numpy(x).to(DEV), faq.QConfig("int8", "per_head"), static_scale=sc)
    assert np.array_equal(qt.codes.cpu().numpy(), OQ.quantize_int8_per_head(x, sc.cpu().numpy()))
    assert qt.codes.cpu().numpy()[0, 0, 0, 0] == 63


def test_int8_scales_and_inputs_at_the_extremes():
    """Heads whose scale lies outside the fast division's range (2^-90,
    2^90), inputs far beyond the scale (codes saturate), subnormal inputs and
    signed zeros: every code still equals clamp(rne(fl32(x / s)))."""
    g = np.random.default_rng(11)
    x = (g.standard_normal((1, 6, 40, 64)) * 3).astype(np.float32)
    x[0, :, 0, :8] = [1e30, -1e30, 3e38, -3e38, 1e-40, -1e-40, 0.0, -0.0]
    x[0, 1] *= 2.0 ** -95  # tiny head, tiny scale
    x[0, 2] *= 2.0 ** 95  # huge head, huge scale
    x[0, 3] *= 2.0 ** -120  # mostly subnormal values
    for dtype in (torch.float32, torch.bfloat16):
        xt = torch.from_numpy(x).to(dtype)
        xn = _np(xt)
        sc = np.array([0.02, 2.0 ** -96, 2.0 ** 93, 2.0 ** -126, 1e-3, 7.0], np.float32)
        sct = torch.from_numpy(sc).to(DEV)
        qt = faq.fa_quantize(xt.to(DEV), faq.QConfig("int8", "per_head"), static_scale=sct)
        assert np.array_equal(qt.codes.cpu().numpy(), OQ.quantize_int8_per_head(xn, sc))


def test_fp8_rows_at_the_extremes():
    """Per-token and token-block FP8 on rows whose amax puts the scale
    outside the fast division's range, rows of subnormals, huge rows and
    signed zeros."""
    g = np.random.default_rng(12)
    x = g.standard_normal((1, 2, 256, 128)).astype(np.float32)
    x[0, 0, 0] *= 1e-30
    x[0, 0, 1] *= 1e30
    x[0, 0, 2] *= 1e-39
    x[0, 0, 3, :4] = [0.0, -0.0, -1e-20, 1.0]
    x[0, 0, 4] = -0.0
    x[0, 1, :128] *= 2.0 ** -100  # a whole token block of tiny values
    x[0, 1, 128:] *= 2.0 ** 100
    for dtype in (torch.float32, torch.bfloat16):
        xt = torch.from_numpy(x).to(dtype)
        xn = _np(xt)
        qt = faq.fa_quantize(xt.to(DEV), faq.QConfig("fp8_e4m3", "per_token"))
        codes, s = OQ.quantize_fp8_per_token(xn)
        assert np.array_equal(qt.scales.cpu().numpy().reshape(s.shape), s)
        assert np.array_equal(qt.codes.cpu().numpy(), codes)
    xt = torch.from_numpy(x).to(torch.bfloat16)
    xn = _np(xt)
    for bt in (128, 256):
        qt = faq.fa_quantize(xt.to(DEV), faq.QConfig("fp8_e4m3", "per_token_block", block_tokens=bt))
        codes, s = OQ.quantize_fp8_block(xn, bt)
        assert np.array_equal(qt.codes.cpu().numpy(), codes)
        assert np.array_equal(qt.scales.cpu().numpy().reshape(s.shape), s)


@pytest.mark.parametrize("shape,dtype", [((1, 2, 128, 64), torch.float32), ((2, 3, 300, 128), torch.bfloat16),
                                         ((1, 1, 1000, 128), torch.bfloat16), ((1, 2, 37, 64), torch.bfloat16)])
def test_fp8_per_token_small(shape, dtype):
    g = np.random.default_rng(sum(shape) + 1)
    x = (g.standard_normal(shape) * np.exp(2 * g.standard_normal(shape[:3] + (1,)))).astype(np.float32)
    x[..., 0, :] = 0.0  # all-zero row: scale 1, codes 0
    x[..., 1, :] = -1e-6
    x[..., 1, 0] = 1.0  # tiny negatives -> 0x80
    xt = torch.from_numpy(x).to(dtype)
    xn = _np(xt)
    qt = faq.fa_quantize(xt.to(DEV), faq.QConfig("fp8_e4m3", "per_token"))
    codes, s = OQ.quantize_fp8_per_token(xn)
    assert np.array_equal(qt.scales.cpu().numpy().reshape(s.shape), s)
    assert np.array_equal(qt.codes.cpu().numpy(), codes)


def test_fp8_divide_ties_and_grid():
    """Rows whose quotients hit E4M3 ties and the whole positive grid."""
    rows = []
    r = np.zeros(128, np.float32); r[:4] = [452, 169.5, -169.5, 1.0]; rows.append(r)
    r = np.zeros(128, np.float32); r[:3] = [466, 349.5, 3.0]; rows.append(r)
    grid = F.E4M3_VALUES[:0x7F].astype(np.float32)
    mids = ((grid[1:] + grid[:-1]) / 2).astype(np.float32)
    vals = np.concatenate([grid, mids, -grid, -mids])
    for i in range(0, vals.size, 127):
        r = np.zeros(128, np.float32); r[0] = 448.0; chunk = vals[i:i + 127]; r[1:1 + chunk.size] = chunk
        rows.append(r)
    x = np.stack(rows).reshape(1, 1, len(rows), 128)
    qt = faq.fa_quantize(torch.from_numpy(x).to(DEV), faq.QConfig("fp8_e4m3", "per_token"))
    codes, s = OQ.quantize_fp8_per_token(x)
    assert np.array_equal(qt.codes.cpu().numpy(), codes)
    assert np.array_equal(qt.scales.cpu().numpy().reshape(s.shape), s)


@pytest.mark.parametrize("shape,dtype", [((1, 2, 128, 64), torch.float32), ((2, 3, 300, 128), torch.bfloat16),
                                         ((1, 1, 999, 128), torch.bfloat16)])
def test_mxfp4_small(shape, dtype):
    g = np.random.default_rng(sum(shape) + 2)
    x = (g.standard_t(4, shape) * np.exp2(g.integers(-30, 30, shape[:3] + (1,)))).astype(np.float32)
    x[..., 0, :] = 0.0
    xt = torch.from_numpy(x).to(dtype)
    xn = _np(xt)
    qt = faq.fa_quantize(xt.to(DEV), faq.QConfig("mxfp4", "per_block"))
    packed, e8 = OQ.quantize_mxfp4(xn)
    assert np.array_equal(qt.scales.cpu().numpy(), e8)
    assert np.array_equal(qt.codes.cpu().numpy(), packed)


def test_mxfp4_ties_and_saturation():
    """Blocks with amax = 7 * 2^E (elements above 6 saturate) and elements on
    every E2M1 tie, for a spread of exponents."""
    ties = np.array([0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0, 6.5, 7.0, 0.1, 0.0, -0.0], np.float32)
    rows = []
    for E in [-130, -100, -20, -3, 0, 5, 60, 125]:
        blk = np.zeros(32, np.float32)
        blk[: ties.size] = ties
        blk[ties.size: 2 * ties.size] = -ties
        blk[-1] = 7.0
        rows.append(np.ldexp(blk, E).astype(np.float32))
    x = np.stack([np.concatenate([r, r[::-1], r, r]) for r in rows]).reshape(1, 1, len(rows), 128)
    qt = faq.fa_quantize(torch.from_numpy(x).to(DEV), faq.QConfig("mxfp4", "per_block"))
    packed, e8 = OQ.quantize_mxfp4(x)
    assert np.array_equal(qt.scales.cpu().numpy(), e8)
    assert np.array_equal(qt.codes.cpu().numpy(), packed)


@pytest.mark.parametrize("bt,S", [(128, 300), (256, 300), (256, 512), (128, 77)])
def test_fp8_block_small(bt, S):
    g = np.random.default_rng(bt + S)
    x = g.standard_normal((2, 3, S, 128)).astype(np.float32)
    x[1, 2] *= 1e-3
    xt = torch.from_numpy(x).to(torch.bfloat16)
    qt = faq.fa_quantize(xt.to(DEV), faq.QConfig("fp8_e4m3", "per_token_block", block_tokens=bt))
    codes, s = OQ.quantize_fp8_block(_np(xt), bt)
    assert np.array_equal(qt.scales.cpu().numpy().reshape(s.shape), s)
    assert np.array_equal(qt.codes.cpu().numpy(), codes)


def _check_rotated(y_gpu, x, R, label="rotate"):
    """The GPU rounds an fp32-accumulated product X.R to bf16, the oracle the
    exact one (fp64).  Where the exact value lies within the fp32
    accumulation error of a bf16 rounding boundary the two may round apart:
    by one bf16 ulp, or by more where X.R cancels (|y| far below
    sum_i |x_i| |R_ij|), which the fp32 bound D * 2^-22 * sum_i |x_i| |R_ij|
    covers.  Elements whose bound is under a quarter ulp must agree within
    one ulp; the equal fraction (measured, logged) must be >= 99.9 %."""
    y_ref = OQ.rotate(x, R)
    diff = np.abs(y_gpu.astype(np.float64) - y_ref)
    ulp = np.exp2(np.floor(np.log2(np.maximum(np.abs(y_ref), 1e-30))) - 7)
    D = R.shape[0]
    acc = D * 2.0 ** -22 * (np.abs(x.astype(np.float64)) @ np.abs(R.astype(np.float64)))
    eq = float(np.mean(diff == 0))
    over1 = diff > ulp * 1.0001
    _parity_log({"case": label, "elements": int(diff.size), "equal_fraction": eq,
                 "over_1ulp": int(over1.sum()), "max_ulps": float((diff / ulp).max()) if diff.size else 0.0,
                 "over_1ulp_with_small_bound": int((over1 & (acc < 0.25 * ulp)).sum())})
    assert np.all(diff <= ulp * 1.0001 + acc)
    assert not np.any(over1 & (acc < 0.25 * ulp))
    assert eq >= 0.999
    return eq


@pytest.mark.parametrize("bt,S,D", [(128, 300, 128), (256, 300, 128), (128, 256, 64), (256, 70, 64)])
def test_rotate_block_small(bt, S, D):
    g = np.random.default_rng(bt + S + D)
    x = g.standard_normal((2, 2, S, D)).astype(np.float32)
    x[:, :, :, 3] *= 30
    xt = torch.from_numpy(x).to(torch.bfloat16)
    a = g.standard_normal((D, D))
    qm, rm = np.linalg.qr(a)
    R = torch.from_numpy((qm * np.sign(np.diag(rm))).astype(np.float32)).to(torch.bfloat16)
    dbg = torch.empty_like(xt, device=DEV)
    qt = faq.fa_quantize(xt.to(DEV), faq.QConfig("fp8_e4m3", "per_token_block", block_tokens=bt),
                         rot=R.to(DEV), debug_rotated=dbg)
    y = _np(dbg)
    _check_rotated(y, _np(xt), _np(R), f"rotate bt={bt} S={S} D={D}")
    codes, s = OQ.quantize_fp8_block(y, bt)
    assert np.array_equal(qt.scales.cpu().numpy().reshape(s.shape), s)
    assert np.array_equal(qt.codes.cpu().numpy(), codes)


# ---------------------------------------------------------------- sibling modes


@pytest.mark.parametrize("shape,dtype", [((1, 2, 128, 64), torch.float32), ((2, 3, 300, 128), torch.bfloat16),
                                         ((1, 4, 77, 64), torch.bfloat16)])
def test_fp8_per_head_small(shape, dtype):
    g = np.random.default_rng(sum(shape) + 3)
    x = (g.standard_normal(shape) * np.exp(g.standard_normal((1, shape[1], 1, 1)))).astype(np.float32)
    xt = torch.from_numpy(x).to(dtype)
    xn = _np(xt)
    amax = torch.zeros(shape[1], dtype=torch.float32, device=DEV)
    faq.fa_quant_calibrate(xt.to(DEV), amax)
    ref_amax = OQ.calibrate_amax(xn)
    sc = faq.fa_quant_scales_from_amax(amax, "fp8_e4m3")
    assert np.array_equal(sc.cpu().numpy(), OQ.fp8_scales(ref_amax))
    # scales tighter than the data: values beyond the calibrated range saturate
    for f in (1.0, 0.7):
        s2 = sc * f
        qt = faq.fa_quantize(xt.to(DEV), faq.QConfig("fp8_e4m3", "per_head"), static_scale=s2)
        assert np.array_equal(qt.codes.cpu().numpy(), OQ.quantize_fp8_per_head(xn, s2.cpu().numpy()))
        assert np.array_equal(qt.scales.cpu().numpy(), s2.cpu().numpy())


def test_fp8_per_head_at_the_extremes():
    """Scales outside the fast division's range, inputs far beyond the scale
    (saturate at 448, never NaN), subnormals and signed zeros."""
    g = np.random.default_rng(13)
    x = (g.standard_normal((1, 6, 40, 64)) * 3).astype(np.float32)
    x[0, :, 0, :8] = [1e30, -1e30, 3e38, -3e38, 1e-40, -1e-40, 0.0, -0.0]
    x[0, 1] *= 2.0 ** -95
    x[0, 2] *= 2.0 ** 95
    x[0, 3] *= 2.0 ** -120
    sc = np.array([0.02, 2.0 ** -96, 2.0 ** 93, 2.0 ** -126, 1e-3, 7.0], np.float32)
    for dtype in (torch.float32, torch.bfloat16):
        xt = torch.from_numpy(x).to(dtype)
        xn = _np(xt)
        qt = faq.fa_quantize(xt.to(DEV), faq.QConfig("fp8_e4m3", "per_head"), static_scale=torch.from_numpy(sc).to(DEV))
        assert np.array_equal(qt.codes.cpu().numpy(), OQ.quantize_fp8_per_head(xn, sc))


@pytest.mark.parametrize("shape,dtype", [((1, 2, 128, 64), torch.float32), ((2, 3, 300, 128), torch.bfloat16),
                                         ((1, 1, 1000, 128), torch.bfloat16)])
def test_int8_per_token_small(shape, dtype):
    g = np.random.default_rng(sum(shape) + 4)
    x = (g.standard_normal(shape) * np.exp(2 * g.standard_normal(shape[:3] + (1,)))).astype(np.float32)
    x[..., 0, :] = 0.0
    x[..., 1, :] = -1e-6
    x[..., 1, 0] = 1.0
    xt = torch.from_numpy(x).to(dtype)
    xn = _np(xt)
    qt = faq.fa_quantize(xt.to(DEV), faq.QConfig("int8", "per_token"))
    codes, s = OQ.quantize_int8_per_token(xn)
    assert np.array_equal(qt.scales.cpu().numpy().reshape(s.shape), s)
    assert np.array_equal(qt.codes.cpu().numpy(), codes)


def test_int8_per_token_rows_at_the_extremes():
    g = np.random.default_rng(14)
    x = g.standard_normal((1, 2, 64, 128)).astype(np.float32)
    x[0, 0, 0] *= 1e-30
    x[0, 0, 1] *= 1e30
    x[0, 0, 2] *= 1e-39
    x[0, 0, 3, :4] = [0.0, -0.0, -1e-20, 1.0]
    x[0, 0, 4] = -0.0
    x[0, 1, 5, :3] = [254.0, 1.0, 3.0]  # 127 * x / 254: exact half-integers
    for dtype in (torch.float32, torch.bfloat16):
        xt = torch.from_numpy(x).to(dtype)
        xn = _np(xt)
        qt = faq.fa_quantize(xt.to(DEV), faq.QConfig("int8", "per_token"))
        codes, s = OQ.quantize_int8_per_token(xn)
        assert np.array_equal(qt.scales.cpu().numpy().reshape(s.shape), s)
        assert np.array_equal(qt.codes.cpu().numpy(), codes)


@pytest.mark.parametrize("shape,dtype", [((1, 2, 128, 64), torch.float32), ((2, 3, 300, 128), torch.bfloat16),
                                         ((1, 1, 999, 128), torch.bfloat16)])
def test_mxfp8_small(shape, dtype):
    g = np.random.default_rng(sum(shape) + 5)
    x = (g.standard_t(4, shape) * np.exp2(g.integers(-30, 30, shape[:3] + (1,)))).astype(np.float32)
    x[..., 0, :] = 0.0
    xt = torch.from_numpy(x).to(dtype)
    xn = _np(xt)
    qt = faq.fa_quantize(xt.to(DEV), faq.QConfig("mxfp8", "per_block"))
    codes, e8 = OQ.quantize_mxfp8(xn)
    assert np.array_equal(qt.scales.cpu().numpy(), e8)
    assert np.array_equal(qt.codes.cpu().numpy(), codes)


def test_mxfp8_ties_saturation_and_exponent_range():
    """Blocks whose maximum sits in (448, 512) * 2^E (saturates), elements on
    E4M3 ties and in the subnormal range, at exponents from the clamp at
    -127 to the top of fp32."""
    grid = F.E4M3_VALUES[:0x7F]
    mids = (grid[1:] + grid[:-1]) / 2
    rows = []
    for E in [-140, -127, -100, -20, -9, 0, 7, 60, 119]:
        blk = np.concatenate([[500.0], mids[::4][:15], -grid[::8][:16]])[:32]
        rows.append(np.ldexp(blk, E).astype(np.float32))
    x = np.stack([np.concatenate([r, r[::-1], -r, r]) for r in rows]).reshape(1, 1, len(rows), 128)
    qt = faq.fa_quantize(torch.from_numpy(x).to(DEV), faq.QConfig("mxfp8", "per_block"))
    codes, e8 = OQ.quantize_mxfp8(x)
    assert np.array_equal(qt.scales.cpu().numpy(), e8)
    assert np.array_equal(qt.codes.cpu().numpy(), codes)


def test_empty_tensor_is_a_no_op():
    x = torch.empty((1, 2, 0, 128), dtype=torch.bfloat16, device=DEV)
    qt = faq.fa_quantize(x, faq.QConfig("fp8_e4m3", "per_token"))
    assert qt.codes.numel() == 0
    amax = torch.zeros(2, device=DEV)
    faq.fa_quant_calibrate(x, amax)
    assert amax.sum().item() == 0


# ---------------------------------------------------------------- full sizes


def _rows_check(run, br):
    """Oracle recomputation of every token row from the GPU's inputs, head by
    head on a thread pool; codes and scales compared bit for bit."""
    w = run.w
    B, H, S, D = w.shape
    x = (w.q, w.k, w.v)[br]
    codes_gpu = run.qt[br].codes.cpu().numpy()
    sc = run.qt[br].scales
    scales_gpu = (sc.view(B, H, S) if run.mode in ("fp8_token", "int8_token") else sc).cpu().numpy()
    static = run.static[br].cpu().numpy() if run.static[br] is not None else None

    def one(bh):
        b, h = divmod(bh, H)
        xs = x[b:b + 1, h:h + 1].to(torch.float32).numpy()
        cg = codes_gpu[b:b + 1, h:h + 1]
        if run.mode == "fp8_token":
            codes, s = OQ.quantize_fp8_per_token(xs)
        elif run.mode == "int8_token":
            codes, s = OQ.quantize_int8_per_token(xs)
        elif run.mode == "mxfp4":
            codes, s = OQ.quantize_mxfp4(xs)
        elif run.mode == "mxfp8":
            codes, s = OQ.quantize_mxfp8(xs)
        elif run.mode == "int8_head":
            codes, s = OQ.quantize_int8_per_head(xs, static[h:h + 1]), None
        elif run.mode == "fp8_head":
            codes, s = OQ.quantize_fp8_per_head(xs, static[h:h + 1]), None
        else:
            raise AssertionError(run.mode)
        assert np.array_equal(cg, codes), (run.mode, br, b, h)
        if s is not None:
            assert np.array_equal(scales_gpu[b:b + 1, h:h + 1], s), (run.mode, br, b, h)

    oracle_pool_map(one, range(B * H))


def _calib_check(run):
    w = run.w
    scales = OQ.int8_scales if run.mode == "int8_head" else OQ.fp8_scales
    for br in range(3):
        ref = None
        for c in w.calib[br]:
            ref = OQ.calibrate_amax(c.to(torch.float32).numpy(), ref)
        assert np.array_equal(run.amax[br].cpu().numpy(), ref)
        assert np.array_equal(run.static[br].cpu().numpy(), scales(ref))


def _blocks_check(run, br):
    """Every token block of the rotate path, head by head: rotated values
    against the oracle's (_check_rotated), then codes and scales bit-exact
    against the oracle's block quantizer run on the GPU's rotated values."""
    w = run.w
    B, H, S, D = w.shape
    bt = run.qt[br].cfg.block_tokens
    nb = -(-S // bt)
    scales = run.qt[br].scales.view(B, H, nb).cpu().numpy()
    codes_gpu = run.qt[br].codes.cpu().numpy()
    xs = (w.q, w.k, w.v)[br]
    ys = run.rotated[br].cpu() if br < 2 else None
    R = w.rot.to(torch.float32).numpy()

    def one(bh):
        b, h = divmod(bh, H)
        x = xs[b:b + 1, h:h + 1].to(torch.float32).numpy()
        if br < 2:
            y = ys[b:b + 1, h:h + 1].to(torch.float32).numpy()
            eq = _check_rotated(y, x, R, f"cfg{w.cfg} branch {br} rotated (b={b}, h={h}) full size")
        else:
            y, eq = x, 1.0
        codes, s = OQ.quantize_fp8_block(y, bt)
        assert np.array_equal(codes_gpu[b:b + 1, h:h + 1], codes), (b, h)
        assert np.array_equal(scales[b:b + 1, h:h + 1], s), (b, h)
        return eq

    eqs = oracle_pool_map(one, range(B * H))
    if br < 2:
        _parity_log({"case": f"cfg{w.cfg} branch {br} rotated, all heads", "equal_fraction_min": min(eqs),
                     "equal_fraction_mean": float(np.mean(eqs))})


@pytest.mark.parametrize("cfg", [1, 2, 3, 4, 5, 6, 7, 8])
def test_full_size_quantize(cfg):
    w = make_inputs(cfg)
    run = GpuRun(w, keep_rotated=(cfg == 5))
    if run.static[0] is not None:
        _calib_check(run)
    for br in range(3):
        if cfg == 5:
            _blocks_check(run, br)
        else:
            _rows_check(run, br)
