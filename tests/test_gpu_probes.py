"""Single-instruction probes of the gfx950 facts the kernels rely on, each
checked against a CPU reference built from the oracle's format tables:

* MFMA operand layouts (i8 16x16x64, bf16 16x16x32, f8f6f4 16x16x128 with
  E2M1 operands and per-lane E8M0 scales; 32x32 forms of each, and the
  32x32x64 f8f6f4 with E5M2 A and E2M1 B, whose scales follow K blocks);
* the K order of 8-bit f8f6f4 operands (lane group g: bytes 0-15 at K
  16g.., bytes 16-31 at K 64+16g..), which differs from the 4-bit one;
* the f8f6f4 MFMA sums 8-bit products with limited precision (the reason the
  FP8 attention runs its score products on the bf16 MFMA), the bf16 MFMA
  does not; it adds its accumulator input exactly;
* hardware conversions: f32 -> E4M3 (OCP, nearest even), f32 -> E2M1 with a
  power-of-two scale (x / scale, saturating), E4M3 -> bf16 and
  E2M1 * scale -> bf16 (both exact);
* the lane mapping of the LDS copy (global_load_lds) and of the
  transposing LDS read of bytes (ds_read_b64_tr_b8);
* LDS reads of fixed lane patterns (the workload the LDS bank-conflict
  counter is read on).
"""

import ctypes

import numpy as np
import pytest
import torch

from oracle import formats as F
from quantized_attention_fa_amd import _abi

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


@pytest.fixture(scope="module")
def lib():
    return _abi.probe_lib()


def _d(a):
    return torch.from_numpy(np.ascontiguousarray(a)).to(DEV)


def _p(t):
    return ctypes.c_void_p(t.data_ptr())


def _pack4(codes):
    return (codes[:, 0::2] | (codes[:, 1::2] << 4)).astype(np.uint8)


def _f8f6f4(lib, A, Bt, fa, fb, sa=None, sb=None, scaled=0):
    sa = np.full((16, 4), 127, np.uint8) if sa is None else sa
    sb = np.full((16, 4), 127, np.uint8) if sb is None else sb
    keep = [_d(A), _d(Bt), _d(sa), _d(sb)]
    C = torch.zeros((16, 16), dtype=torch.float32, device=DEV)
    assert lib.faq_probe_mfma_f8f6f4(*[_p(t) for t in keep], fa, fb, scaled, _p(C)) == 0
    return C.cpu().numpy().astype(np.float64)


def test_mfma_i8_layout(lib):
    g = np.random.default_rng(0)
    A = g.integers(-128, 128, (16, 64)).astype(np.int8)
    B = g.integers(-128, 128, (16, 64)).astype(np.int8)
    C = torch.zeros((16, 16), dtype=torch.int32, device=DEV)
    a, b = _d(A), _d(B)
    assert lib.faq_probe_mfma_i8(_p(a), _p(b), _p(C)) == 0
    assert np.array_equal(C.cpu().numpy(), A.astype(np.int64) @ B.astype(np.int64).T)


def test_mfma_bf16_layout_and_precision(lib):
    g = np.random.default_rng(1)
    # E4M3-valued operands (exact in bf16) with per-row magnitudes spread out
    qa = np.clip(g.standard_normal((16, 32)) * np.exp(2 * g.standard_normal((16, 1))), -448, 448)
    kb = np.clip(g.standard_normal((16, 32)) * np.exp(2 * g.standard_normal((16, 1))), -448, 448)
    A = F.e4m3_decode(F.e4m3_encode(qa)).astype(np.float32)
    B = F.e4m3_decode(F.e4m3_encode(kb)).astype(np.float32)
    a = torch.from_numpy(A).to(torch.bfloat16).to(DEV)
    b = torch.from_numpy(B).to(torch.bfloat16).to(DEV)
    C = torch.zeros((16, 16), dtype=torch.float32, device=DEV)
    assert lib.faq_probe_mfma_bf16(_p(a), _p(b), _p(C)) == 0
    ref = A.astype(np.float64) @ B.astype(np.float64).T
    bound = 32 * 2.0 ** -22 * (np.abs(A).astype(np.float64) @ np.abs(B).astype(np.float64).T)
    assert np.all(np.abs(C.cpu().numpy() - ref) <= bound)


def test_mfma32_bf16_layout(lib):
    """v_mfma_f32_32x32x16_bf16: lane (i, h) holds K elements 8h..8h+7 of
    row i; accumulator r is row 8(r/4) + 4h + r%4 of column i."""
    g = np.random.default_rng(21)
    A = g.integers(-8, 9, (32, 16)).astype(np.float32)
    B = g.integers(-8, 9, (32, 16)).astype(np.float32)
    a = torch.from_numpy(A).to(torch.bfloat16).to(DEV)
    b = torch.from_numpy(B).to(torch.bfloat16).to(DEV)
    C = torch.zeros((32, 32), dtype=torch.float32, device=DEV)
    assert lib.faq_probe_mfma32_bf16(_p(a), _p(b), _p(C)) == 0
    assert np.array_equal(C.cpu().numpy(), A @ B.T)


def test_mfma32_i8_layout(lib):
    g = np.random.default_rng(22)
    A = g.integers(-128, 128, (32, 32)).astype(np.int8)
    B = g.integers(-128, 128, (32, 32)).astype(np.int8)
    C = torch.zeros((32, 32), dtype=torch.int32, device=DEV)
    a, b = _d(A), _d(B)
    assert lib.faq_probe_mfma32_i8(_p(a), _p(b), _p(C)) == 0
    assert np.array_equal(C.cpu().numpy(), A.astype(np.int64) @ B.astype(np.int64).T)


def test_mfma32_fp8_layout(lib):
    """v_mfma_f32_32x32x64_f8f6f4 with E4M3 operands (the FP8 value product):
    lane (i, h) holds bytes 32h..32h+31 of row i of A and of B^T, paired
    byte for byte (whatever K order the hardware gives them), accumulator r
    is row 8(r/4) + 4h + r%4 of column i.  Values of a narrow exponent range
    keep every sum exact."""
    g = np.random.default_rng(24)
    vals = np.array([0.5, 0.75, 1.0, 1.25, 1.5, 2.0, 2.5, 3.0])
    A = vals[g.integers(0, 8, (32, 64))] * np.where(g.random((32, 64)) < 0.5, -1.0, 1.0)
    B = vals[g.integers(0, 8, (32, 64))] * np.where(g.random((32, 64)) < 0.5, -1.0, 1.0)
    a, b = _d(F.e4m3_encode(A)), _d(F.e4m3_encode(B))
    C = torch.zeros((32, 32), dtype=torch.float32, device=DEV)
    assert lib.faq_probe_mfma32_fp8(_p(a), _p(b), _p(C)) == 0
    assert np.array_equal(C.cpu().numpy().astype(np.float64), A @ B.T)


def test_mfma32_fp4_scaled_layout(lib):
    """v_mfma_scale_f32_32x32x64_f8f6f4 with E2M1 operands: lane (i, h) holds
    elements 32h..32h+31 of row i (16 bytes) and that block's E8M0 scale."""
    g = np.random.default_rng(23)
    ca = g.integers(0, 16, (32, 64)).astype(np.uint8)
    cb = g.integers(0, 16, (32, 64)).astype(np.uint8)
    sa = g.integers(125, 130, (32, 2)).astype(np.uint8)
    sb = g.integers(125, 130, (32, 2)).astype(np.uint8)
    va = F.e2m1_decode(ca) * np.repeat(2.0 ** (sa.astype(np.float64) - 127), 32, axis=1)
    vb = F.e2m1_decode(cb) * np.repeat(2.0 ** (sb.astype(np.float64) - 127), 32, axis=1)
    keep = [_d(_pack4(ca)), _d(_pack4(cb)), _d(sa), _d(sb)]
    C = torch.zeros((32, 32), dtype=torch.float32, device=DEV)
    assert lib.faq_probe_mfma32_fp4(*[_p(t) for t in keep], _p(C)) == 0
    assert np.array_equal(C.cpu().numpy().astype(np.float64), va @ vb.T)


def _e5m2_decode(codes):
    """E5M2 (OCP FP8, bias 15, subnormals at 2^-16 steps); no Inf/NaN codes
    are used here."""
    c = np.asarray(codes).astype(np.int64)
    e, m = (c >> 2) & 0x1F, c & 3
    mag = np.where(e == 0, m * 2.0 ** -16, (1 + m / 4) * 2.0 ** (e - 15))
    return np.where(c & 0x80, -mag, mag)


# K position of byte p (lane half p // 32, byte p % 32) of an 8-bit operand
# of the 32x32x64 f8f6f4 MFMA, against the 4-bit operand's elements (lane
# half h holds elements 32h .. 32h + 31 in order)
MFMA32_8BIT_K = [16 * (p // 32) + p % 32 if p % 32 < 16 else 32 + 16 * (p // 32) + p % 32 - 16 for p in range(64)]


def _mfma32_bf8_fp4(lib, A, Bp, sa, sb):
    keep = [_d(A), _d(Bp), _d(sa), _d(sb)]
    C = torch.zeros((32, 32), dtype=torch.float32, device=DEV)
    assert lib.faq_probe_mfma32_bf8_fp4(*[_p(t) for t in keep], _p(C)) == 0
    return C.cpu().numpy().astype(np.float64)


def test_mfma32_bf8_fp4_k_order(lib):
    """E5M2 A times E2M1 B on v_mfma_scale_f32_32x32x64_f8f6f4 (the MXFP4
    value product), each A byte's K position read off bit-encoded B rows: in
    lane half h, bytes 0-15 sit at K 16h.., bytes 16-31 at K 32 + 16h..,
    while the E2M1 elements of B are in order."""
    kappa = np.full(64, -1)
    ones = np.full((32, 2), 127, np.uint8)
    for m in range(2):
        A = np.zeros((32, 64), np.uint8)
        for i in range(32):
            A[i, 32 * m + i] = 0x3C  # 1.0
        Bc = np.zeros((32, 64), np.uint8)
        for j in range(6):
            Bc[j, [q for q in range(64) if (q >> j) & 1]] = 2  # 1.0
        C = _mfma32_bf8_fp4(lib, A, _pack4(Bc), ones, ones)
        for i in range(32):
            kappa[32 * m + i] = int(sum(int(round(C[i, j])) << j for j in range(6)))
    assert kappa.tolist() == MFMA32_8BIT_K


def test_mfma32_bf8_fp4_values(lib):
    """The same instruction on E5M2 values e2m1 * 2^-k (k = 0..15, down to
    the E5M2 subnormals) with E8M0 scales per row and K block: each row's
    products span < 2^6 within a block, so the sums are exact."""
    g = np.random.default_rng(25)
    e2m1_mag = np.array([0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0])
    k = g.integers(0, 16, (32, 1))  # one shift per row: its products span < 2^8
    Aval = e2m1_mag[g.integers(0, 7, (32, 64))] * 2.0 ** -k.astype(np.float64)
    Aval *= np.where(g.random((32, 64)) < 0.5, -1.0, 1.0)
    grid = np.arange(256)
    dec = _e5m2_decode(grid)
    lut = {float(v): int(c) for c, v in zip(grid, dec) if (c & 0x7F) < 0x7C}
    A = np.vectorize(lambda v: lut[float(v)])(Aval).astype(np.uint8)
    assert np.array_equal(_e5m2_decode(A), Aval)
    Bc = g.integers(0, 16, (32, 64)).astype(np.uint8)
    # block scales within 2^5 of 1: the two block sums stay exact in fp32
    sa = g.integers(125, 131, (32, 2)).astype(np.uint8)
    sb = g.integers(125, 131, (32, 2)).astype(np.uint8)
    C = _mfma32_bf8_fp4(lib, A, _pack4(Bc), sa, sb)
    Ak = np.zeros_like(Aval)
    Ak[:, MFMA32_8BIT_K] = Aval  # A in K order
    # the scale of lane half h applies to K block h (K 32h .. 32h + 31), not
    # to the bytes that lane holds
    ref = (Ak * np.repeat(F.e8m0_decode(sa), 32, axis=1)) @ (
        F.e2m1_decode(Bc) * np.repeat(F.e8m0_decode(sb), 32, axis=1)).T
    assert np.array_equal(C, ref)


def test_mfma_fp4_scaled_layout(lib):
    g = np.random.default_rng(2)
    ca = g.integers(0, 16, (16, 128)).astype(np.uint8)
    cb = g.integers(0, 16, (16, 128)).astype(np.uint8)
    sa = g.integers(110, 140, (16, 4)).astype(np.uint8)
    sb = g.integers(110, 140, (16, 4)).astype(np.uint8)
    C = _f8f6f4(lib, _pack4(ca), _pack4(cb), 4, 4, sa, sb, 1)
    va = F.e2m1_decode(ca) * np.repeat(F.e8m0_decode(sa), 32, axis=1)
    vb = F.e2m1_decode(cb) * np.repeat(F.e8m0_decode(sb), 32, axis=1)
    ref = va @ vb.T
    # products inside a 32-block share one scale and span < 2^8, so each
    # block sum is exact; the blocks are then added in fp32
    bound = 4 * 2.0 ** -23 * (np.abs(va) @ np.abs(vb).T)
    assert np.all(np.abs(C - ref) <= bound)


def test_mfma_8bit_k_order(lib):
    """Bit-encoded pairing of each E4M3 operand byte with an E2M1 nibble."""
    kappa = np.full(128, -1)
    for m in range(8):
        A = np.zeros((16, 128), np.uint8)
        for i in range(16):
            A[i, 16 * m + i] = 0x38  # 1.0
        Bc = np.zeros((16, 128), np.uint8)
        for j in range(7):
            Bc[j, [q for q in range(128) if (q >> j) & 1]] = 2  # 1.0
        C = _f8f6f4(lib, A, _pack4(Bc), 0, 4)
        for i in range(16):
            kappa[16 * m + i] = int(sum(int(round(C[i, j])) << j for j in range(7)))
    want = [16 * (p // 32) + p % 32 if p % 32 < 16 else 64 + 16 * (p // 32) + p % 32 - 16 for p in range(128)]
    assert kappa.tolist() == want


def test_mfma_fp8_accumulation_is_truncating(lib):
    """One product of 448 and fifteen of 2^-7 in the same 16-group: the
    f8f6f4 MFMA keeps about 12 fractional bits below the group's largest
    product, so part of the small sum is lost (exact: 448 + 127/128)."""
    A = np.zeros((16, 128), np.uint8)
    A[:, 0] = 0x7E
    A[:, 1:] = int(F.e4m3_encode(2.0 ** -7))
    Bt = np.full((16, 128), 0x38, np.uint8)
    C = _f8f6f4(lib, A, Bt, 0, 0)
    exact = 448 + 127 * 2.0 ** -7
    assert C[0, 0] < exact and exact - C[0, 0] < 2.0 ** -4


def test_mfma32_fp8_accumulator_input_is_added_exactly(lib):
    """The 32x32x64 f8f6f4 MFMA adds its accumulator input at fp32
    precision, not aligned with the products: a large C plus small products
    comes back as the correctly rounded sum (the FP8 value product
    accumulates into the running output this way)."""
    f = lib.faq_probe_mfma32_fp8_acc
    one = int(F.e4m3_encode(1.0))
    for cin, pv, n in [(2.0 ** 20, 1.0, 64), (2.0 ** 20, 1.0, 1), (1024.0, 2.0 ** -7, 64), (1024.0, 2.0 ** -7, 1),
                       (-(2.0 ** 20), 1.0, 64), (2.0 ** 12, 2.0 ** -3, 64)]:
        A = np.zeros((32, 64), np.uint8)
        A[:, :n] = int(F.e4m3_encode(pv))
        Bt = np.full((32, 64), one, np.uint8)
        keep = [_d(A), _d(Bt), _d(np.full((32, 32), cin, np.float32))]
        C = torch.zeros((32, 32), dtype=torch.float32, device=DEV)
        assert f(*[_p(t) for t in keep], _p(C)) == 0
        got = C.cpu().numpy().astype(np.float64)
        assert np.all(got == float(np.float32(cin + n * pv))), (cin, pv, n, got[0, 0])


def test_cvt_f32_to_u8_rounds_to_nearest_even(lib):
    """v_cvt_pk_u8_f32 on [0, 128) (the INT8 probability codes): round to
    nearest, ties to even (the value phase takes a tie's side from this
    conversion)."""
    x = np.concatenate([np.arange(0, 127) + 0.5, np.arange(0, 127) + 0.25, np.arange(0, 127) + 0.75,
                        np.nextafter(np.arange(0, 127) + 0.5, 0), np.nextafter(np.arange(0, 127) + 0.5, 1e9),
                        [0.0, 127.0]]).astype(np.float32)
    xd = _d(x)
    out = torch.zeros(x.size, dtype=torch.uint8, device=DEV)
    assert lib.faq_probe_cvt_u8(_p(xd), x.size, _p(out)) == 0
    want = np.rint(x.astype(np.float64)).astype(np.uint8)
    assert np.array_equal(out.cpu().numpy(), want)


def test_cvt_f32_to_e4m3_and_fp4(lib):
    grid = F.E4M3_VALUES[:0x7F]
    mids = (grid[1:] + grid[:-1]) / 2
    g = np.random.default_rng(3)
    x = np.concatenate([grid, mids, mids * (1 + 2.0 ** -20), mids * (1 - 2.0 ** -20), -grid, -mids,
                        g.uniform(-448, 448, 4000), g.standard_normal(4000) * 0.01, [0.0, -0.0, -1e-6]]).astype(np.float32)
    xt = _d(x)
    outs = [torch.zeros(x.size, dtype=torch.uint8, device=DEV) for _ in range(4)]
    for scale in (1.0, 0.25, 2.0 ** -10, 8.0):
        assert lib.faq_probe_cvt(_p(xt), x.size, ctypes.c_float(scale), *[_p(o) for o in outs]) == 0
        e4, _, f4, sw = [o.cpu().numpy() for o in outs]
        ref4 = F.e4m3_encode(x.astype(np.float64))
        assert np.array_equal(e4, ref4)
        assert np.array_equal(sw, ref4)
        assert np.array_equal(f4, F.e2m1_encode(x.astype(np.float64) / scale))


def test_cvt_up_to_bf16(lib):
    words = np.arange(1 << 16, dtype=np.uint32)
    words = words | (words[::-1] << 16)
    codes = words.view(np.uint8).reshape(-1, 4)
    finite = np.isfinite(F.E4M3_VALUES[codes]).all(axis=1)
    words = words[finite]
    codes = codes[finite]
    w = _d(words)
    n = words.size
    outs = [torch.zeros(n, dtype=torch.int32, device=DEV) for _ in range(3)]
    for scale in (1.0, 2.0 ** -3, 2.0 ** 5):
        assert lib.faq_probe_cvt_up(_p(w), n, ctypes.c_float(scale), *[_p(o) for o in outs]) == 0
        lo, hi, f4 = [o.cpu().numpy().view(np.uint32) for o in outs]
        bf = lambda u: F.bf16_from_bits((u & 0xffff).astype(np.uint16)).astype(np.float64), \
            lambda u: F.bf16_from_bits((u >> 16).astype(np.uint16)).astype(np.float64)
        assert np.array_equal(bf[0](lo), F.E4M3_VALUES[codes[:, 0]])
        assert np.array_equal(bf[1](lo), F.E4M3_VALUES[codes[:, 1]])
        assert np.array_equal(bf[0](hi), F.E4M3_VALUES[codes[:, 2]])
        assert np.array_equal(bf[1](hi), F.E4M3_VALUES[codes[:, 3]])
        assert np.array_equal(bf[0](f4), F.e2m1_decode(codes[:, 0] & 0xF) * scale)
        assert np.array_equal(bf[1](f4), F.e2m1_decode(codes[:, 0] >> 4) * scale)


def test_global_load_lds_layout(lib):
    """Each lane's 16 bytes land at the instruction's LDS address + 16 * lane
    (the attention kernel stages its K / V^T tiles this way)."""
    g = np.random.default_rng(4)
    src = g.integers(0, 256, 1024).astype(np.uint8)
    perm = g.permutation(64).astype(np.int32)
    s_d, p_d = _d(src), _d(perm)
    out = torch.zeros(2048, dtype=torch.uint8, device=DEV)
    assert lib.faq_probe_global_load_lds(_p(s_d), _p(p_d), _p(out)) == 0
    o = out.cpu().numpy()
    assert not o[:1024].any()
    want = src.reshape(64, 16)[perm].reshape(-1)
    assert np.array_equal(o[1024:], want)


def test_lds_transposing_read_layout(lib):
    """ds_read_b64_tr_b8: in each 16-lane group, lane l receives as byte k
    byte l % 8 of the 8 bytes source lane 2 k + (l / 8) % 2 points at (the
    INT8 value product reads V rows this way)."""
    g = np.random.default_rng(5)
    src = g.integers(0, 256, 1024).astype(np.uint8)
    offs = (8 * g.integers(0, 128, 64)).astype(np.int32)
    s_d, o_d = _d(src), _d(offs)
    out = torch.zeros(512, dtype=torch.uint8, device=DEV)
    assert lib.faq_probe_lds_tr8(_p(s_d), _p(o_d), _p(out)) == 0
    o = out.cpu().numpy().reshape(64, 8)
    want = np.zeros((64, 8), dtype=np.uint8)
    for lane in range(64):
        for k in range(8):
            srcl = 16 * (lane >> 4) + 2 * k + ((lane >> 3) & 1)
            want[lane, k] = src[offs[srcl] + (lane & 7)]
    assert np.array_equal(o, want)


def _qk_row(r):
    return 64 * ((r >> 2) & 1) + 4 * (r >> 3) + (r & 3)


def _half_swap(row):
    return row ^ ((row >> 3) & 8)


# Byte offsets per lane of the LDS read patterns (width, offsets).  The
# K-operand pattern is the one the attention kernel's score MFMA reads: lane
# half h takes 16-byte column h of a chunk-major tile, lane j of the half K
# row qk_row(j) (plain row order); the half-swapped variant puts rows 64..
# in the other 8-row half, which a plain 64 x 4-byte bank model predicts to
# be the conflict-free one.
LDS_PATTERNS = [
    ("b128_contiguous", 16, [16 * l for l in range(64)]),
    ("b128_k_operand_half_swapped", 16, [2048 * (l // 32) + 16 * _half_swap(_qk_row(l % 32)) for l in range(64)]),
    ("b128_k_operand", 16, [2048 * (l // 32) + 16 * _qk_row(l % 32) for l in range(64)]),
    ("b128_stride32", 16, [32 * l for l in range(64)]),
    ("b128_8lane_groups_1k_apart", 16, [16 * (l % 8) + 1024 * (l // 8) for l in range(64)]),
    ("b128_broadcast", 16, [0] * 64),
    ("b64_contiguous", 8, [8 * l for l in range(64)]),
    ("b32_contiguous", 4, [4 * l for l in range(64)]),
]


def test_lds_read_patterns(lib):
    """Each pattern's reads return the addressed words (the launches, in this
    order, are the workload of the LDS bank-conflict counter calibration)."""
    f = lib.faq_probe_lds_read
    f.argtypes = [ctypes.POINTER(ctypes.c_int), ctypes.c_int, ctypes.c_int, ctypes.c_void_p]
    f.restype = ctypes.c_int
    reps = 1024
    words = (np.arange(4096, dtype=np.uint64) * 2654435761) % (1 << 32)
    for name, width, offs in LDS_PATTERNS:
        assert all(0 <= o <= 16384 - width and o % width == 0 for o in offs), name
        out = torch.zeros(64 * width // 4, dtype=torch.int32, device=DEV)
        arr = (ctypes.c_int * 64)(*offs)
        assert f(arr, width, reps, _p(out)) == 0, name
        got = out.cpu().numpy().view(np.uint32).reshape(64, width // 4).astype(np.uint64)
        want = np.array([[(reps * int(words[o // 4 + k])) % (1 << 32) for k in range(width // 4)] for o in offs],
                        dtype=np.uint64)
        assert np.array_equal(got, want), name
    bad = (ctypes.c_int * 64)(*([8] * 64))
    out = torch.zeros(256, dtype=torch.int32, device=DEV)
    assert f(bad, 16, 1, _p(out)) == -1  # misaligned for a 16-byte read
