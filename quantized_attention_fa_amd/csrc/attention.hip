// Flash-style attention on quantized Q/K/V for gfx950.
//
// Both products take the low-bit operands ("FA 量化" page, 概述) on MFMA.
// Each branch is configured on its own ("fa3_quant 配置说明" page, §2.3
// FA3AttentionDetails; an unconfigured branch is not quantized), so the
// score product Q K^T follows the (shared) configuration of Q and K and the
// value product P V follows V's:
//
//   scores, by the Q/K configuration
//     INT8 per-head   v_mfma_i32_32x32x32_i8, exact int32 scores
//     INT8 per-token  the same; the per-key K scale multiplies the scores
//     FP8 E4M3        v_mfma_f32_32x32x16_bf16 on the exact bf16 images of
//                     the E4M3 codes.  The f8f6f4 MFMA sums each group of
//                     products aligned to the group's largest with about 12
//                     fractional bits, so score errors reach ~1e-4 of
//                     amax_q * amax_k and move probability codes; the bf16
//                     MFMA accumulates these exact products at fp32 precision.
//     MXFP4           v_mfma_scale_f32_32x32x64_f8f6f4 with E2M1 operands and
//                     their E8M0 block exponents as MFMA scales (exact:
//                     products within a block span < 2^8)
//     MXFP8           the bf16 MFMA; each row widened relative to its
//                     largest block exponent (exact), the row exponents
//                     scale the scores
//     unquantized     the bf16 MFMA on the bf16 inputs
//   values, by V's configuration, with the probabilities P quantized to
//   V's type
//     INT8            int8 P, v_mfma_i32_32x32x32_i8, exact int32 sums
//     FP8 E4M3        per-token V: E4M3 P times the E4M3 V codes on
//                     v_mfma_scale_f32_32x32x64_f8f6f4 (unscaled),
//                     accumulating into O (the instruction adds its
//                     accumulator input exactly; the alignment error of its
//                     products enters O linearly); V with one scale per
//                     tile: E4M3 P on the bf16 MFMA (exact images)
//     MXFP4           with MXFP4 Q and K: E2M1 P with its 32-key group
//                     exponents as the B scales of the block-scaled f8f6f4
//                     MFMA, times V re-expressed per (32-key group, 32-channel
//                     block) as E5M2 under one E8M0 A scale (V's own
//                     exponents run along D, the MFMA's scales along keys);
//                     exact for exponent spreads up to 57 within a group (a
//                     second image and product past 28); the instruction
//                     sums the products to about 2^-12 of the largest
//     MXFP4 / MXFP8   otherwise: MX-quantized P on the bf16 MFMA, V exact in
//                     bf16
//     unquantized     bf16 P on the bf16 MFMA
// The output is dequantized to bf16 (or fp32) ("量化" page, FA量化 / FP8
// Attention).
//
// Probability rule (the pages leave it open; this is the library's contract):
// keys are cut into 128-key tiles aligned to absolute key index; per query
// row and tile, m = max score, p = exp(s - m) is quantized with a static
// scale relative to that tile maximum (int8: rne(127 p w_j); E4M3: 448 p w_j
// with w_j = s_v,j / max_tile s_v, 1 when V has one scale per tile; MXFP4 /
// MXFP8: the MX quantizer over 32-key groups; unquantized V: bf16 of p),
// the tile sum L uses unquantized p, and tiles combine with the usual
// running-max rescale, O = sum_t e^{m_t-M} C_t / sum_t e^{m_t-M} L_t.
//
// Kernel shape: each tile runs in a score phase (S^T = K Q^T, mostly MFMA)
// and a value phase (probabilities, P quantization, O^T += V^T P^T, mostly
// vector work).  Four-wave kernel (INT8 and MXFP4 scores, and every call
// with key splits): a workgroup is 4 waves and 128 queries of one (b,h);
// two workgroups share a CU.  Ping-pong kernel (bf16 score products without
// key splits): 8 waves in two 128-query groups, the second one phase behind
// the first, so the two waves of a SIMD are always in different phases; K
// and V^T tiles are double-buffered.
// Each wave owns 32 queries: one 32x32 MFMA column block for both products.
// Scores are computed transposed (S^T = K Q^T): a lane holds one query and,
// with the K rows fed to the MFMA permuted (qk_row), 64 consecutive keys of
// the tile, i.e. two whole 32-key MX groups.  The row max and sum need one
// cross-lane step, and the lane's probabilities are already the B operand of
// O^T = V^T P^T.  V^T comes from a per-call workspace with its key columns in
// the order the lanes hold their probabilities (FP8 / MXFP8 K widened there
// to bf16 too).  INT8 per-head V needs no workspace: its tile is copied as
// rows and read through the transposing LDS read (prefill), or loaded into
// registers and transposed by the kernel (key splits).
//
// LDS tiles are chunk-major: 16-byte column c of every row, then column c+1.
// An operand read takes one column per lane half (distinct rows of it), which
// runs without bank conflicts (measured on the fixed lane pattern), and every
// operand address is a per-lane base plus a constant.  In the four-wave
// kernel the K tile of t+1 is copied (global_load_lds) while P V of tile t
// runs, and V^T of tile t while the scores of t are computed: two barriers
// per tile.
//
// Workgroups are numbered so that all query tiles of one (b,h) land on the
// same XCD (workgroups are dealt to the 8 XCDs round robin), which keeps a
// head's K/V tiles in that XCD's L2; causal grids run the longest query
// tiles first.

#include <climits>
#include <type_traits>

#include "common.h"
#include "launch.h"

namespace faq {
namespace {

typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef int i32x16 __attribute__((ext_vector_type(16)));

constexpr int NW = 4;          // waves per workgroup
constexpr int NTHR = NW * 64;  // threads per workgroup
constexpr int BM = NW * 32;    // queries per workgroup
constexpr int BN = 128;        // keys per tile = probability tile
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLog2_127 = 6.9886846867721655f, kLog2_448 = 8.807354922057604f;

// Key order.  Output row R of the 32x32 block kb of S^T reads K row
// 16 kb + qk_row(R); the accumulator puts row 8 (r/4) + 4 h + r%4 in
// register r of lane half h, so register r of block kb in lane half h is
// key 64 h + 16 kb + r.
FAQ_DEV int qk_row(int R) { return 64 * ((R >> 2) & 1) + 4 * (R >> 3) + (R & 3); }

// LDS slot of K row `row` within a 16-byte column: the row itself.  The
// score MFMA's K operand read (lane j of half h: row qk_row(j) of column h)
// has no bank conflicts in this order (SQ_LDS_BANK_CONFLICT on the fixed
// pattern is 0).  Swapping the 8-row halves of rows 64.., which a plain
// 64 x 4-byte bank model predicts to spread the read over all banks,
// measures 4 conflict cycles per read: gfx950 maps addresses to banks with
// more than the low address bits.
FAQ_DEV int kslot(int row) { return row; }

// Key at column p of a V^T tile.  bf16 P V (32x32x16): k-step 2 kb + s of
// the tile takes, in lane half h, registers 8 s .. 8 s + 7 of block kb:
// column p = 32 kb + 16 s + 8 h + t <-> key 64 h + 16 kb + 8 s + t.
// int8 P V (32x32x32): k-step kb takes registers 0..15 of block kb:
// column p = 32 kb + 16 h + r <-> key 64 h + 16 kb + r.
// E4M3 P V for per-token V (32x32x64 f8f6f4): k-step s takes, in lane half h, the 32 bytes
// of blocks 2 s and 2 s + 1 (keys 64 h + 32 s + 0..31); A and B pair their
// bytes position by position, so column p <-> key p (natural order): lane
// (i, h) reads 16-byte columns 4 h + 2 s and 4 h + 2 s + 1 of row i.
FAQ_DEV int vt_key_bf16(int p) { return 64 * ((p >> 3) & 1) + 16 * (p >> 5) + 8 * ((p >> 4) & 1) + (p & 7); }
FAQ_DEV int vt_key_i8(int p) { return 64 * ((p >> 4) & 1) + 16 * (p >> 5) + (p & 15); }

// Two E4M3 bytes (the low half-word of `w`, or the high one when HI) -> two
// bf16, times the power of two `sc` (exact while the values stay in bf16's
// normal range).
template <bool HI>
FAQ_DEV uint32_t e4m3x2_to_bf16x2(uint32_t w, float sc = 1.0f) {
  return __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8((int)w, sc, HI));
}

// Eight E2M1 codes (the four bytes of `w`, element 2i in the low nibble of
// byte i) -> eight bf16, times the power of two `sc`.
FAQ_DEV uint4 e2m1x8_to_bf16x8(uint32_t w, float sc) {
  return make_uint4(__builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, sc, 0)),
                    __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, sc, 1)),
                    __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, sc, 2)),
                    __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, sc, 3)));
}

// Two INT8 codes (bytes B and B + 1 of `w`) -> two bf16, exactly.
template <int B>
FAQ_DEV uint32_t i8x2_to_bf16x2(uint32_t w) {
  const float a = (float)(int8_t)(w >> (8 * B)), b = (float)(int8_t)(w >> (8 * B + 8));
  return (__float_as_uint(a) >> 16) | (__float_as_uint(b) & 0xffff0000u);
}

// Eight elements of a row, from `row` (bytes) at element e0 (a multiple of
// 8), widened exactly to bf16 relative to 2^-E_rel for the MX formats: the
// general score mode's operand.  ex: the row's E8M0 bytes (MX only).
FAQ_DEV uint4 widen8(int fmt, const uint8_t* row, int e0, const uint8_t* ex, int erow) {
  switch (fmt) {
    case FMT_BF16: return *reinterpret_cast<const uint4*>(row + 2 * e0);
    case FMT_INT8: {
      const uint2 a = *reinterpret_cast<const uint2*>(row + e0);
      return make_uint4(i8x2_to_bf16x2<0>(a.x), i8x2_to_bf16x2<2>(a.x), i8x2_to_bf16x2<0>(a.y),
                        i8x2_to_bf16x2<2>(a.y));
    }
    case FMT_MX4: {
      const float sc = __builtin_amdgcn_ldexpf(1.0f, (int)ex[e0 >> 5] - erow);
      return e2m1x8_to_bf16x8(*reinterpret_cast<const uint32_t*>(row + e0 / 2), sc);
    }
    default: {  // FP8, MX8 (E4M3 codes)
      const float sc = fmt == FMT_MX8 ? __builtin_amdgcn_ldexpf(1.0f, (int)ex[e0 >> 5] - erow) : 1.0f;
      const uint2 a = *reinterpret_cast<const uint2*>(row + e0);
      return make_uint4(__builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8((int)a.x, sc, false)),
                        __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8((int)a.x, sc, true)),
                        __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8((int)a.y, sc, false)),
                        __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8((int)a.y, sc, true)));
    }
  }
}

// Bytes of a row of D elements in a branch format.
FAQ_DEV int fmt_row_bytes(int fmt, int D) { return fmt == FMT_BF16 ? 2 * D : (fmt == FMT_MX4 ? D / 2 : D); }

// 2^e as a float for e in [-126, 127] (a normal number, built from its bits).
FAQ_DEV float pow2f(int e) { return __uint_as_float((uint32_t)(e + 127) << 23); }

// Max / sum over the two lanes holding one query (l and l ^ 32).
FAQ_DEV float halves_max(float x) {
  const auto a = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(a[0]), __uint_as_float(a[1]));
}
FAQ_DEV float halves_sum(float x) {
  const auto a = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(a[0]) + __uint_as_float(a[1]);
}

// Code of u under the hardware conversions the value phase uses (E4M3 or
// unsigned 8-bit, round to nearest even).
FAQ_DEV uint32_t p_code(float u, bool e4m3) {
  return e4m3 ? ((uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(u, 0.0f, 0, false) & 0xffu)
              : (__builtin_amdgcn_cvt_pk_u8_f32(u, 0u, 0u) & 0xffu);
}

// The probability multiplier qmax w_j = qmax s_v,j / sigma_t of a key whose
// V scale varies along the tile (per-token V), as an fp32 value that the
// code grid (E4M3 for qmax 448, integers for 127) rounds like the exact
// quotient, with room to spare: the tile maximum (p = 1 exactly) must take
// the code of the exact product even when its p carries the few-ulp error
// of the fused exponent argument.  u is the fp64 quotient (one rounding):
// an exact tie stays on the tie, and every other quotient of fp32 scales
// lies at least ~2^-29 (relative) from a boundary.  A quotient within
// 2^-15 (relative) of the nearest code boundary b is moved to b (1 +- 2^-15)
// on its own side; an exact tie to the side of the code round-to-nearest-
// even gives b.  Other quotients keep their fp32 rounding, which cannot
// cross b.  Away from the maximum the multiplier then differs from the
// quotient by at most 2^-15, so a key's code can differ from the exact
// rule's only if its product lies that close to a boundary.
FAQ_DEV float p_multiplier(float sv, float sigma, bool e4m3) {
  const double u = (e4m3 ? 448.0 : 127.0) * (double)sv / (double)sigma;
  const float mu = (float)u;
  float b;  // the code boundary nearest to mu
  if (e4m3) {
    int e;
    (void)__builtin_frexpf(mu, &e);
    const float step = __builtin_amdgcn_ldexpf(1.0f, max(e - 1, -6) - 3);  // E4M3 spacing at mu
    b = (__builtin_rintf(mu / step - 0.5f) + 0.5f) * step;
  } else {
    b = __builtin_rintf(mu - 0.5f) + 0.5f;
  }
  const double d = u - (double)b;
  const float gap = b * 0x1p-15f;
  if (d == 0.0) return p_code(b - gap, e4m3) == p_code(b, e4m3) ? b - gap : b + gap;
  if (d > 0.0 && d < (double)gap) return b + gap;
  if (d < 0.0 && -d < (double)gap) return b - gap;
  return mu;
}

// Geometry of the LDS tiles, from the score mode QK and the value mode PV.
template <int QK, int PV, int D>
struct Cfg {
  static constexpr bool QI8 = QK == QK_I8H || QK == QK_I8T;                                 // int8 score MFMA
  static constexpr bool QBF =
      QK == QK_F8T || QK == QK_F8C || QK == QK_MX8 || QK == QK_BF || QK == QK_GEN;  // bf16 score MFMA
  static constexpr bool QIMG = QK == QK_F8T || QK == QK_F8C || QK == QK_MX8 || QK == QK_GEN;  // K widened
  static constexpr bool KSC =
      QK == QK_I8T || QK == QK_F8T || QK == QK_F8C || QK == QK_MX8 || QK == QK_GEN;  // per-key K floats
  static constexpr bool PI8 = PV == PV_I8H || PV == PV_I8T;  // int8 value MFMA
  // E4M3 value MFMA (f8f6f4) for per-token V.  The instruction sums its
  // products to about 2^-12 of the largest, an error of ~2^-12 |O| per
  // output: within the absolute bar for per-token V, whose codes are
  // normalised row by row, but not for V with one scale per tile, whose
  // outlier channels carry outputs of tens; those keep the bf16 product.
  static constexpr bool PF8 = PV == PV_F8W;
  static constexpr bool PMX = PV == PV_MX4 || PV == PV_MX8;  // MX probability groups
  // MXFP4 Q, K and V: the value product on the block-scaled f8f6f4 MFMA,
  // E2M1 P (its 32-key group exponents as B scales) times V re-expressed
  // per (32-key group, 32-channel block) as E5M2 with one E8M0 A scale.
  // A tile whose V exponents spread too far for one image takes a second
  // one and a second product (a per-tile flag).
  static constexpr bool PF4 = QK == QK_MX4 && PV == PV_MX4;
  static constexpr bool PVW = PV == PV_I8T || PV == PV_F8W;  // per-key V scale folded into P
  static constexpr bool SIG = PVW || PV == PV_F8C;            // sigma_t per tile
  static constexpr int KROW = QI8 ? D : (QBF ? 2 * D : D / 2);  // bytes of a K row in LDS
  static constexpr int KBYTES = BN * KROW;
  static constexpr int NB = D / 32;  // MX blocks per row
  // per-key extras: after the K tile the K scales (floats; MXFP8: 2^ of
  // the row exponent) or the MXFP4 K block exponents; after the V^T tile
  // the multipliers qmax w_j (floats), then sigma_t (one float, padded to
  // 16 bytes), which the value phase reads after the K buffer is refilled
  static constexpr int XKBYTES = QK == QK_MX4 ? BN * NB : (KSC ? BN * 4 : 0);
  static constexpr int XVW = PVW ? BN * 4 : 0;  // offset of sigma_t in the V extras
  // MXFP4 values: 16 bytes of scales of the first E5M2 image (byte 4 g + b:
  // key group g, channel block b), 16 of the second, then the tile's flag
  // word (nonzero: the second image is used)
  static constexpr int XVBYTES = PF4 ? 48 : XVW + (SIG ? 16 : 0);
  static constexpr int XBYTES = XKBYTES + XVBYTES;  // per tile in the workspace
  static constexpr int VROW = (PI8 || PF8) ? BN : 2 * BN;  // bytes of a V^T row
  static constexpr int VBYTES = D * VROW;
  static constexpr int VF4BYTES = D * BN;  // MXFP4 values: one E5M2 image (half of the slot)
  // INT8 per-head V: the tile is copied straight from the V rows
  // (chunk-major, like K) and the value MFMA reads it through the
  // transposing LDS reads, so no V^T image is made.  (For bf16 V the same
  // scheme doubles the LDS read instructions of the value product and
  // measured slower than the V^T image.)
  static constexpr bool VROWS = PV == PV_I8H;
  // nothing to prepare: no K image, no per-key extras, V read as rows
  static constexpr bool NOPREP = VROWS && !QIMG && XKBYTES == 0 && XVBYTES == 0;
  static constexpr int KS = QI8 ? D / 32 : (QBF ? D / 16 : D / 64);  // score k-steps
  static constexpr int DB = D / 32;                                  // 32-channel output blocks
};

// ------------------------------------------------------------------------
// Workspace layout (per (b,h), per 128-key tile t):
//   vt  : V^T of the tile as its LDS image (chunk-major, columns in the lane
//         key order): INT8 or per-token E4M3 codes (1 byte) or bf16 values
//         (2 bytes: E4M3 codes of V with one scale per tile, exact MX
//         values, or the unquantized V).  MXFP4 Q, K and V: the E5M2 image
//         (1 byte, natural key order) in the first half of a 2-byte slot,
//         a flagged tile's second E5M2 image in the other half
//   kb  : FP8 / MXFP8 scores: K widened to bf16 as its LDS image (rows past
//         the end are 0; MXFP8 relative to the row's largest block exponent)
//   aux : K extras (K scales; MXFP8 row scales 2^(E_row); MXFP4 K block
//         exponents, 128 rows x D/32 bytes, 127 past the end), then V
//         extras (the multipliers qmax w_j; sigma_t = max over the tile's
//         keys of s_v,j for FP8 / INT8 per-token and FP8 with one V scale
//         per tile; MXFP4 values: the E5M2 images' E8M0 scales and the
//         tile's flag)
// ------------------------------------------------------------------------
struct WsLayout {
  size_t vt_off, kb_off, aux_off, part_off, total;
};

// Key splits: with few query tiles per head (decode: a handful of queries
// against a long cache) the (b,h, query tile) grid cannot fill 256 CUs, so
// the key tiles are split across workgroups, tps tiles each, for about 512
// workgroups: one full round at two per CU, each streaming a long run of
// tiles (fewer, longer splits measure faster than more rounds of short
// ones).  Causal attention (Sq == Skv) never splits.
struct KvSplit {
  int nsplit, tps;
};

inline KvSplit kv_split(int64_t B, int64_t H, int64_t Sq, int64_t Skv, int causal) {
  const int64_t nt = (Skv + BN - 1) / BN;
  const int64_t base = B * H * ((Sq + BM - 1) / BM);
  if (causal || base >= 1024 || nt < 4) return KvSplit{1, (int)nt};
  int64_t want = (512 + base - 1) / base;
  if (want > nt / 2) want = nt / 2;
  if (want > 64) want = 64;  // the merge keeps one split per lane
  const int64_t tps = (nt + want - 1) / want;
  return KvSplit{(int)((nt + tps - 1) / tps), (int)tps};
}

inline WsLayout ws_layout(int qk, int pv, int64_t B, int64_t H, int64_t Sq, int64_t Skv, int64_t D,
                          int causal) {
  const int64_t nt = (Skv + BN - 1) / BN;
  const size_t tiles = (size_t)(B * H * nt);
  const bool pi8 = pv == PV_I8H || pv == PV_I8T;
  const bool pf8 = pv == PV_F8W;
  const bool qimg = qk == QK_F8T || qk == QK_F8C || qk == QK_MX8 || qk == QK_GEN;
  const bool ksc = qk == QK_I8T || qimg;
  const bool pvw = pv == PV_I8T || pv == PV_F8W;
  const bool sig = pvw || pv == PV_F8C;
  const bool pf4 = qk == QK_MX4 && pv == PV_MX4;
  const size_t xk = qk == QK_MX4 ? BN * (D / 32) : (ksc ? BN * 4 : 0);
  const size_t xv = pf4 ? 48 : (pvw ? BN * 4 : 0) + (sig ? 16 : 0);
  auto up = [](size_t x) { return (x + 255) & ~size_t(255); };
  WsLayout l{};
  const bool vrows = pv == PV_I8H;  // V read as rows, no V^T image
  l.vt_off = 0;
  l.kb_off = up(vrows ? 0 : tiles * D * BN * ((pi8 || pf8) ? 1 : 2));
  l.aux_off = l.kb_off + up(qimg ? tiles * BN * D * 2 : 0);
  l.part_off = l.aux_off + up(tiles * (xk + xv));
  const KvSplit sp = kv_split(B, H, Sq, Skv, causal);
  l.total = l.part_off + up(sp.nsplit > 1 ? (size_t)sp.nsplit * B * H * Sq * (D + 2) * 4 : 0);
  if (l.total < 256) l.total = 256;  // valid operands never report 0 (that means invalid)
  return l;
}

// ------------------------------------------------------------------------
// Per-call re-layout.  grid = (tiles, B*H), 256 threads; one 128-key tile.
//   K (by QK): FP8 / MXFP8 the bf16 image (MXFP8 rows relative to their
//              largest block exponent); the per-key K scales (INT8 / FP8
//              per-token, FP8 one-per-tile, MXFP8 2^(E_row)); MXFP4 the K
//              block exponents.
//   V (by PV): the V^T image: INT8 codes, E4M3 codes widened to bf16, MX
//              values exact in bf16, or the unquantized bf16 values; the
//              per-key multipliers qmax w_j and sigma_t.  None for INT8
//              per-head V (read as rows by the attention kernel); a pair of
//              INT8 per-head Q/K with such V needs no re-layout at all.
// Float scales of K and V are read at b * sb + h * sh + key / blk
// (per-token: blk 1; token blocks: blk tokens; per-head: sb 0, sh 1, one
// block).
// ------------------------------------------------------------------------
struct PrepArgs {
  const uint8_t* k;
  const void* ks;
  const uint8_t* v;
  const void* vs;
  RowMap kmap, vmap;  // rows of K and V codes (BNSD or BSND)
  int64_t H, Skv, nt, ksb, ksh, vsb, vsh;
  int kblk, vblk;
  int kfmt;  // general score mode: K's BranchFmt
  uint8_t* vt;
  uint8_t* kb;
  uint8_t* aux;
};

template <int QK, int PV, int D>
__global__ __launch_bounds__(256) void k_prep(const PrepArgs a) {
  using C = Cfg<QK, PV, D>;
  constexpr int NB = D / 32;
  // bytes of a V row: packed E2M1, bf16, or one-byte codes
  constexpr int VR = PV == PV_MX4 ? D / 2 : (PV == PV_BF ? 2 * D : D);
  constexpr bool VEX = PV == PV_MX4 || PV == PV_MX8;
  __shared__ uint8_t tile[BN][VR + 4];
  __shared__ uint8_t vex[VEX ? BN : 1][NB];
  __shared__ float red[4];
  // MXFP4 values: per (row, channel block) the exponent byte where the
  // block holds a nonzero code (else 0 / 255), the scales of the two E5M2
  // images, and the tile's flag (second image used)
  __shared__ uint8_t ehi[C::PF4 ? BN : 1][NB], elo[C::PF4 ? BN : 1][NB];
  __shared__ uint8_t gsc[4][NB], gsc1[4][NB];
  __shared__ int vwide;
  const int t = blockIdx.x;
  const int64_t bh = blockIdx.y;
  const int64_t k0 = (int64_t)t * BN;
  const int64_t tile_id = bh * a.nt + t;
  const int64_t b_ = bh / a.H, h_ = bh % a.H;
  uint8_t* auxt = a.aux + tile_id * C::XBYTES;
  // V rows -> LDS (not for V read as rows by the attention kernel)
  for (int c = threadIdx.x; c < (C::VROWS ? 0 : BN * (VR / 16)); c += 256) {
    const int kl = c / (VR / 16), cc = c % (VR / 16);
    uint4 val = make_uint4(0, 0, 0, 0);
    if (k0 + kl < a.Skv) val = *reinterpret_cast<const uint4*>(a.v + a.vmap.row(b_, h_, k0 + kl) * VR + cc * 16);
    uint32_t* dst = reinterpret_cast<uint32_t*>(&tile[kl][cc * 16]);
    dst[0] = val.x; dst[1] = val.y; dst[2] = val.z; dst[3] = val.w;
  }
  if (VEX) {
    for (int c = threadIdx.x; c < BN * NB; c += 256) {
      const int kl = c / NB, b = c % NB;
      vex[kl][b] = k0 + kl < a.Skv ? reinterpret_cast<const uint8_t*>(a.vs)[(bh * a.Skv + k0 + kl) * NB + b]
                                   : (uint8_t)127;
    }
  }
  // K image, 16 codes (two 16-byte image columns) per item
  if (QK == QK_GEN) {
    const int rb = fmt_row_bytes(a.kfmt, D);
    for (int c = threadIdx.x; c < BN * (D / 16); c += 256) {
      const int kl = c / (D / 16), cc = c % (D / 16);
      uint4 lo = make_uint4(0, 0, 0, 0), hi = make_uint4(0, 0, 0, 0);
      if (k0 + kl < a.Skv) {
        const uint8_t* row = a.k + a.kmap.row(b_, h_, k0 + kl) * rb;
        const uint8_t* ke = reinterpret_cast<const uint8_t*>(a.ks) + (bh * a.Skv + k0 + kl) * NB;
        int emax = 0;
        if (a.kfmt == FMT_MX4 || a.kfmt == FMT_MX8)
          for (int b = 0; b < NB; ++b) emax = max(emax, (int)ke[b]);
        lo = widen8(a.kfmt, row, 16 * cc, ke, emax);
        hi = widen8(a.kfmt, row, 16 * cc + 8, ke, emax);
      }
      uint8_t* img = a.kb + tile_id * C::KBYTES + kslot(kl) * 16;
      *reinterpret_cast<uint4*>(img + (2 * cc) * BN * 16) = lo;
      *reinterpret_cast<uint4*>(img + (2 * cc + 1) * BN * 16) = hi;
    }
  } else if (C::QIMG) {
    for (int c = threadIdx.x; c < BN * (D / 16); c += 256) {
      const int kl = c / (D / 16), cc = c % (D / 16);
      uint4 kv = make_uint4(0, 0, 0, 0);
      float sc = 1.0f;
      if (k0 + kl < a.Skv) {
        kv = *reinterpret_cast<const uint4*>(a.k + a.kmap.row(b_, h_, k0 + kl) * D + cc * 16);
        if (QK == QK_MX8) {
          const uint8_t* ke = reinterpret_cast<const uint8_t*>(a.ks) + (bh * a.Skv + k0 + kl) * NB;
          int emax = 0;
#pragma unroll
          for (int b = 0; b < NB; ++b) emax = max(emax, (int)ke[b]);
          sc = __builtin_amdgcn_ldexpf(1.0f, (int)ke[cc >> 1] - emax);
        }
      }
      uint8_t* img = a.kb + tile_id * C::KBYTES + kslot(kl) * 16;
      *reinterpret_cast<uint4*>(img + (2 * cc) * BN * 16) =
          make_uint4(e4m3x2_to_bf16x2<false>(kv.x, sc), e4m3x2_to_bf16x2<true>(kv.x, sc),
                     e4m3x2_to_bf16x2<false>(kv.y, sc), e4m3x2_to_bf16x2<true>(kv.y, sc));
      *reinterpret_cast<uint4*>(img + (2 * cc + 1) * BN * 16) =
          make_uint4(e4m3x2_to_bf16x2<false>(kv.z, sc), e4m3x2_to_bf16x2<true>(kv.z, sc),
                     e4m3x2_to_bf16x2<false>(kv.w, sc), e4m3x2_to_bf16x2<true>(kv.w, sc));
    }
  }
  // K extras
  if (QK == QK_MX4) {
    for (int c = threadIdx.x; c < BN * NB; c += 256) {
      const int kl = c / NB, b = c % NB;
      auxt[c] = k0 + kl < a.Skv ? reinterpret_cast<const uint8_t*>(a.ks)[(bh * a.Skv + k0 + kl) * NB + b]
                                : (uint8_t)127;
    }
  }
  const int kl = threadIdx.x;
  if (C::KSC && kl < BN) {
    float sk = 0.0f;
    const bool kmx = QK == QK_MX8 || (QK == QK_GEN && (a.kfmt == FMT_MX4 || a.kfmt == FMT_MX8));
    if (k0 + kl < a.Skv) {
      if (QK == QK_GEN && a.kfmt == FMT_BF16) {
        sk = 1.0f;
      } else if (kmx) {
        const uint8_t* ke = reinterpret_cast<const uint8_t*>(a.ks) + (bh * a.Skv + k0 + kl) * NB;
        int emax = 0;
#pragma unroll
        for (int b = 0; b < NB; ++b) emax = max(emax, (int)ke[b]);
        sk = __builtin_amdgcn_ldexpf(1.0f, emax - 127);
      } else {
        sk = reinterpret_cast<const float*>(a.ks)[(bh / a.H) * a.ksb + (bh % a.H) * a.ksh + (k0 + kl) / a.kblk];
      }
    }
    reinterpret_cast<float*>(auxt)[kl] = sk;
  }
  __syncthreads();
  // V^T image.  item i: column c = i / D, row d = i % D (consecutive
  // threads write consecutive 16-byte slots of one column)
  uint8_t* img = a.vt + tile_id * C::VBYTES;
  constexpr int VCOLS = C::VROW / 16;
  if constexpr (C::PF4) {
    // MXFP4 values, re-expressed per (32-key group g, channel block b):
    // element e2m1 * 2^(E_j - 127) = (e2m1 * 2^(E_j - A)) * 2^(A - 127)
    // with A = max(E_max - 13, 0) (E_max over the group's rows whose block
    // holds a nonzero code): the largest element becomes at most
    // 6 * 2^13 < 57344 and every element with E_j - A in [-15, 13] is an
    // exact E5M2 value (e2m1 has at most two significant bits; E5M2 keeps
    // three down to its subnormal step 2^-16).  A nonzero element with
    // E_j < A - 15 flags the tile: such elements go to a second image
    // under A1 = max(A - 29, 0), exact for E_j >= A1 - 15, i.e. exponent
    // spreads up to 57 within a group; an element beyond that (below
    // 2^-55 of its group's largest) is left out.
    if (threadIdx.x == 0) vwide = 0;
    for (int c = threadIdx.x; c < BN * NB; c += 256) {
      const int kl = c / NB, b = c % NB;
      const uint32_t* w = reinterpret_cast<const uint32_t*>(&tile[kl][16 * b]);
      const bool nz = ((w[0] | w[1] | w[2] | w[3]) & 0x77777777u) != 0u;  // magnitude bits; rows past the end are 0
      ehi[kl][b] = nz ? vex[kl][b] : (uint8_t)0;
      elo[kl][b] = nz ? vex[kl][b] : (uint8_t)255;
    }
    __syncthreads();
    if (threadIdx.x < 4 * NB) {
      const int g = threadIdx.x / NB, b = threadIdx.x % NB;
      int mx = 0, mn = 255;
      for (int r = 0; r < 32; ++r) {
        mx = max(mx, (int)ehi[32 * g + r][b]);
        mn = min(mn, (int)elo[32 * g + r][b]);
      }
      const int sa = max(mx - 13, 0), sa1 = max(sa - 29, 0);
      gsc[g][b] = (uint8_t)sa;
      gsc1[g][b] = (uint8_t)sa1;
      auxt[C::XKBYTES + 4 * g + b] = (uint8_t)sa;
      auxt[C::XKBYTES + 16 + 4 * g + b] = (uint8_t)sa1;
      if (mn != 255 && mn < sa - 15) vwide = 1;
    }
    __syncthreads();
    if (threadIdx.x == 0) *reinterpret_cast<uint32_t*>(auxt + C::XKBYTES + 32) = (uint32_t)vwide;
  }
  if (C::PF4) {
    // the E5M2 image(s), keys in natural order: column c holds keys
    // 16 c .. 16 c + 15 of row d; a flagged tile's second image follows
    // the first
    auto image = [&](auto two) __attribute__((always_inline)) {
      constexpr bool TWO = decltype(two)::value;
      for (int i = threadIdx.x; i < (BN / 16) * D; i += 256) {
        const int c = i / D, d = i % D, b = d >> 5;
        const int sa = gsc[c >> 1][b], sa1 = gsc1[c >> 1][b];
        uint32_t w[4], w1[4];
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          float f[4], f1[4];
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            const int key = 16 * c + 4 * q + r;
            const uint32_t nib = (tile[key][d >> 1] >> (4 * (d & 1))) & 0xfu;
            const uint32_t mag = nib & 7u;
            const float fm = mag < 2 ? 0.5f * (float)mag
                                     : (float)(1u << ((mag >> 1) - 1)) * (1.0f + 0.5f * (float)(mag & 1u));
            const int e = (int)vex[key][b];
            const bool in0 = mag != 0 && e >= sa - 15;
            const float x0 = in0 ? __builtin_amdgcn_ldexpf(fm, e - sa) : 0.0f;
            f[r] = (nib & 8u) ? -x0 : x0;
            if (TWO) {
              const bool in1 = mag != 0 && !in0 && e >= sa1 - 15;
              const float x1 = in1 ? __builtin_amdgcn_ldexpf(fm, e - sa1) : 0.0f;
              f1[r] = (nib & 8u) ? -x1 : x1;
            }
          }
          int pk = __builtin_amdgcn_cvt_pk_bf8_f32(f[0], f[1], 0, false);
          pk = __builtin_amdgcn_cvt_pk_bf8_f32(f[2], f[3], pk, true);
          w[q] = (uint32_t)pk;
          if (TWO) {
            int pk1 = __builtin_amdgcn_cvt_pk_bf8_f32(f1[0], f1[1], 0, false);
            pk1 = __builtin_amdgcn_cvt_pk_bf8_f32(f1[2], f1[3], pk1, true);
            w1[q] = (uint32_t)pk1;
          }
        }
        *reinterpret_cast<uint4*>(img + (c * D + d) * 16) = make_uint4(w[0], w[1], w[2], w[3]);
        if (TWO)
          *reinterpret_cast<uint4*>(img + C::VF4BYTES + (c * D + d) * 16) = make_uint4(w1[0], w1[1], w1[2], w1[3]);
      }
    };
    if (vwide != 0) image(std::true_type{});
    else image(std::false_type{});
  }
  for (int i = threadIdx.x; i < ((C::VROWS || C::PF4) ? 0 : VCOLS * D); i += 256) {
    const int c = i / D, d = i % D;
    uint32_t w[4];
    if (C::PI8 || C::PF8) {
      // one byte per code; E4M3 values: keys in their natural order
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        uint32_t acc = 0;
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int p = 16 * c + 4 * q + r;
          acc |= (uint32_t)tile[C::PF8 ? p : vt_key_i8(p)][d] << (8 * r);
        }
        w[q] = acc;
      }
    } else {
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int key0 = vt_key_bf16(8 * c + 2 * q), key1 = vt_key_bf16(8 * c + 2 * q + 1);
        if (PV == PV_BF) {
          w[q] = (uint32_t)*reinterpret_cast<const uint16_t*>(&tile[key0][2 * d]) |
                 ((uint32_t)*reinterpret_cast<const uint16_t*>(&tile[key1][2 * d]) << 16);
        } else if (PV == PV_MX4) {
          uint32_t pair = 0;
#pragma unroll
          for (int hh = 0; hh < 2; ++hh) {
            const int key = hh ? key1 : key0;
            const uint32_t nib = (tile[key][d >> 1] >> (4 * (d & 1))) & 0xfu;
            const uint32_t mag = nib & 7u;
            // E2M1 magnitude: 0, .5, 1, 1.5, 2, 3, 4, 6; times 2^(e8m0 - 127)
            const float fm = mag < 2 ? 0.5f * (float)mag
                                     : (float)(1u << ((mag >> 1) - 1)) * (1.0f + 0.5f * (float)(mag & 1u));
            float f = __builtin_amdgcn_ldexpf(fm, (int)vex[key][d >> 5] - 127);
            f = (nib & 8u) ? -f : f;
            pair |= (__float_as_uint(f) >> 16) << (16 * hh);  // exact: at most 2 significant bits
          }
          w[q] = pair;
        } else {
          const uint32_t pair = (uint32_t)tile[key0][d] | ((uint32_t)tile[key1][d] << 8);
          w[q] = e4m3x2_to_bf16x2<false>(pair);
          if (PV == PV_MX8) {
            // the exact value code * 2^(E - 127), rounded to bf16 (exact
            // within bf16's normal range)
            const float f0 = __builtin_amdgcn_ldexpf(bf16_lo(w[q]), (int)vex[key0][d >> 5] - 127);
            const float f1 = __builtin_amdgcn_ldexpf(bf16_hi(w[q]), (int)vex[key1][d >> 5] - 127);
            w[q] = f32_to_bf16_bits(f0) | (f32_to_bf16_bits(f1) << 16);
          }
        }
      }
    }
    *reinterpret_cast<uint4*>(img + (c * D + d) * 16) = make_uint4(w[0], w[1], w[2], w[3]);
  }
  // V extras: sigma_t and the multipliers qmax w_j
  if (C::SIG) {
    float sv = 0.0f;
    if (kl < BN && k0 + kl < a.Skv)
      sv = reinterpret_cast<const float*>(a.vs)[(bh / a.H) * a.vsb + (bh % a.H) * a.vsh + (k0 + kl) / a.vblk];
    float m = wave_max(sv);
    if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = m;
    __syncthreads();
    m = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
    if (C::PVW && kl < BN)
      reinterpret_cast<float*>(auxt + C::XKBYTES)[kl] = (sv > 0.0f) ? p_multiplier(sv, m, PV == PV_F8W) : 0.0f;
    if (threadIdx.x == 0) reinterpret_cast<float*>(auxt + C::XKBYTES + C::XVW)[0] = m;
  }
}

// ------------------------------------------------------------------------
// The attention kernel.
// ------------------------------------------------------------------------
struct KParams {
  int64_t H, BH, Sq, Skv, nt;
  int nqt;
  RowMap qmap, kmap, omap;  // rows of Q codes, K codes (when gathered) and the output
  const uint8_t* q;      // Q codes or bf16 values
  const void* qs;        // Q scales
  const uint8_t* k;      // K codes / bf16 values, or the bf16 K images in the workspace
  const void* ks;        // INT8 per-head: K scale
  const uint8_t* vt;     // V^T images in the workspace
  const uint8_t* aux;    // per-tile K extras, then V extras (see Cfg)
  const float* vs_head;  // INT8 per-head V: V scale
  int64_t q_sb, q_sh;    // float Q scale index b * q_sb + h * q_sh + i / q_block
  int q_block;
  int qfmt;              // general score mode: Q's BranchFmt
  float c_log2;  // sm_scale * log2(e)
  void* out;
  int out_bf16;
  // split keys (non-causal): split c of a (b,h, query tile) runs tiles
  // [c tps, (c + 1) tps) and leaves its unnormalized O, running reference M
  // and sum L in part (nsplit > 1) for k_combine
  int nsplit, tps;
  float* part;
  // direct V (INT8 codes, decode): V rows read from the codes and transposed
  // into the LDS V^T tile by the kernel itself, no re-layout pass
  const uint8_t* vcodes;
  RowMap vmap;
};

// Partial results of split c: O at part + ((c BH + bh) Sq + i) D, then
// (M, L) pairs after all nsplit BH Sq rows of O.
FAQ_DEV float* part_o(float* part, int c, int64_t BH, int64_t Sq, int64_t bh, int64_t i, int D) {
  return part + (((int64_t)c * BH + bh) * Sq + i) * D;
}
FAQ_DEV float* part_ml(float* part, int nsplit, int c, int64_t BH, int64_t Sq, int64_t bh, int64_t i, int D) {
  return part + (int64_t)nsplit * BH * Sq * D + (((int64_t)c * BH + bh) * Sq + i) * 2;
}

using lptr = __attribute__((address_space(3))) void*;

// One 16-byte global -> LDS copy per lane (lane i of the wave to
// lds + 16 i) from base + off, base wave-uniform, off the lane's 32-bit
// byte offset: global_load_lds_dwordx4 written out in its SGPR-base form
// (the address is one VGPR, no 64-bit per-lane address arithmetic), so
// that the compiler does not track the copy: its completion is waited for
// only where the kernel says so (vmcnt), never before reads of other LDS
// buffers.  The instruction has no result registers; M0 holds the wave's
// LDS base.  M0 is a reserved register the compiler does not treat as
// clobberable, so the attention kernels issue no other M0-using
// instruction: all their LDS copies go through this form (their assembly
// has no M0 access outside these blocks).
FAQ_DEV void copy16(const uint8_t* base, uint32_t off, uint8_t* lds) {
  const uint32_t m = (uint32_t)(uintptr_t)(lptr)lds;
  asm volatile("s_mov_b32 m0, %2\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, %1" : : "v"(off), "s"(base), "s"(m)
               : "memory");
}

// Copy NCH 16-byte chunks global -> LDS with NT threads.  The workgroup
// moves one round of NT chunks per step (one global_load_lds_dwordx4 per
// wave, 1 KiB); chunk p = NT i + 64 wave + lane lands at lds + 16 p and
// comes from base + i rstride + loff: loff is the lane's 32-bit byte
// offset (the same register in every round), rstride a wave-uniform
// stride added to the scalar base.
template <int NCH, int NT>
FAQ_DEV void stage(uint8_t* lds, const uint8_t* base, int wave, int lane, uint32_t loff, uint32_t rstride) {
  // the tile base is a wave-uniform value held in SGPRs; hiding it from the
  // optimizer keeps it from turning every copy into a 64-bit per-lane
  // pointer carried across loop iterations
  asm volatile("" : "+s"(base));
  constexpr int ROUNDS = NCH / NT;
#pragma unroll
  for (int i = 0; i < ROUNDS; ++i) {
    const int grp = i * NT + wave * 64;
    copy16(base + (size_t)i * rstride, loff, lds + grp * 16);
  }
  constexpr int REM = NCH - ROUNDS * NT;  // < one round: the first waves take it
  if (REM > 0) {
    const int grp = ROUNDS * NT + wave * 64;
    if (grp < NCH) {
      if (REM % 64 == 0 || grp + lane < NCH) copy16(base + (size_t)ROUNDS * rstride, loff, lds + grp * 16);
    }
  }
}

// Copies (global_load_lds instructions) wave `wave` of NT threads issues
// for NCH chunks: the full rounds, plus one if it takes part in the rest.
template <int NCH, int NT>
FAQ_DEV int stage_loads(int wave) {
  return NCH / NT + ((NCH / NT) * NT + wave * 64 < NCH ? 1 : 0);
}

// s_waitcnt vmcnt(n) for a wave-uniform n (the count must be an immediate)
FAQ_DEV void wait_vm(int n) {
  switch (n) {
    case 0: __builtin_amdgcn_s_waitcnt(0x0F70); break;
    case 1: __builtin_amdgcn_s_waitcnt(0x0F71); break;
    case 2: __builtin_amdgcn_s_waitcnt(0x0F72); break;
    case 3: __builtin_amdgcn_s_waitcnt(0x0F73); break;
    case 4: __builtin_amdgcn_s_waitcnt(0x0F74); break;
    case 5: __builtin_amdgcn_s_waitcnt(0x0F75); break;
    case 6: __builtin_amdgcn_s_waitcnt(0x0F76); break;
    case 7: __builtin_amdgcn_s_waitcnt(0x0F77); break;
    case 8: __builtin_amdgcn_s_waitcnt(0x0F78); break;
    case 9: __builtin_amdgcn_s_waitcnt(0x0F79); break;
    case 10: __builtin_amdgcn_s_waitcnt(0x0F7A); break;
    case 11: __builtin_amdgcn_s_waitcnt(0x0F7B); break;
    case 12: __builtin_amdgcn_s_waitcnt(0x0F7C); break;
    default: __builtin_amdgcn_s_waitcnt(0x0F70); break;  // (never above 12 here)
  }
}

// Transposing LDS read of bytes (gfx950): within each 16-lane group, lane l
// receives as its byte k byte l % 8 of the 8 bytes source lane
// 2 k + (l / 8) % 2 points at.
using v2i = int __attribute__((ext_vector_type(2)));
FAQ_DEV v2i lds_tr8(const uint8_t* p) {
  return __builtin_amdgcn_ds_read_tr8_b64_v2i32((__attribute__((address_space(3))) v2i*)p);
}

template <class T>
FAQ_DEV T lds_ld(const uint8_t* p) {
  return *reinterpret_cast<const T*>(p);
}

// PP (ping-pong): eight waves in two groups of four, each group a 128-query
// tile; the second group runs one phase behind the first, so each SIMD
// holds one wave computing scores (MFMA) while the other computes
// probabilities and their products (vector work), and the two overlap.  K
// and V^T tiles are double-buffered.
template <int QK, int PV, int D, bool CAUSAL, bool VDIR = false, bool PP = false>
__global__ __launch_bounds__(PP ? 2 * NTHR : NTHR, PP ? 1 : 2) void k_attn(const KParams p) {
  using G = Cfg<QK, PV, D>;
  constexpr int NWK = PP ? 2 * NW : NW;  // waves per workgroup
  constexpr int NTK = NWK * 64;          // threads per workgroup
  static_assert(NTK % 256 == 0, "tile copies: an even number of 128-lane columns per round");
  constexpr int BMK = NWK * 32;          // queries per workgroup
  static_assert(!(PP && VDIR), "ping-pong tiles come from the workspace");
  static_assert(!(G::PF4 && (PP || VDIR)), "MXFP4 value tiles: four-wave kernel");
  static_assert(!VDIR || (G::PI8 && D == 128), "direct V: int8 codes, D = 128");
  constexpr int KS = G::KS, DB = G::DB, NB = G::NB;
  // per-key K scales multiply the scores (per-token scopes, MXFP8 rows); a
  // K scale constant over the tile folds into the exponent factor
  constexpr bool PERKEY = QK == QK_I8T || QK == QK_F8T || QK == QK_MX8 || QK == QK_GEN;
  constexpr bool KCONST = QK == QK_F8C;
  static_assert(!(G::PMX && QK == QK_I8H), "MX probabilities need the float score path");
  // K (+ its per-key extras) and V^T tiles in separate LDS objects: V(t)
  // is copied while the scores and probabilities of tile t are computed
  // from K(t), and K(t+1) while the products with V(t) run.  As distinct
  // objects the compiler knows an LDS read of one does not alias a copy in
  // flight into the other, so it never waits for the copy.
  constexpr int KSZ = G::KBYTES + G::XKBYTES, VSZ = G::VBYTES + G::XVBYTES;
  __shared__ __attribute__((aligned(1024))) uint8_t kbuf[KSZ];
  __shared__ __attribute__((aligned(1024))) uint8_t vbuf[VSZ];
  // ping-pong: the second K and V^T buffers (odd tiles of the work item);
  // direct V: the second K buffer
  __shared__ __attribute__((aligned(PP || VDIR ? 1024 : 16))) uint8_t kbuf1[PP || VDIR ? KSZ : 16];
  __shared__ __attribute__((aligned(PP ? 1024 : 16))) uint8_t vbuf1[PP ? VSZ : 16];

  const int tid = threadIdx.x, lane = tid & 63, j = lane & 31, h = lane >> 5;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  __builtin_assume(wave >= 0 && wave < NWK);
  const int grp = PP ? wave >> 2 : 0;  // ping-pong group

  // ---- work item: (b,h), query tile and key split
  int64_t bh;
  int qt;
  const int split = p.nsplit > 1 ? (int)(blockIdx.x % p.nsplit) : 0;
  {
    const int L = p.nsplit > 1 ? (int)(blockIdx.x / p.nsplit) : (int)blockIdx.x, nqt = p.nqt;
    const int BH = (int)p.BH;
    if ((BH & 7) == 0) {
      const int xcd = L & 7, jj = L >> 3, per = BH >> 3;
      if (CAUSAL) { qt = nqt - 1 - jj / per; bh = xcd + 8 * (jj % per); }
      else { bh = xcd + 8 * (jj / nqt); qt = jj % nqt; }
    } else {
      if (CAUSAL) { qt = nqt - 1 - L / BH; bh = L % BH; }
      else { bh = L / nqt; qt = L % nqt; }
    }
  }
  const int64_t hd = bh % p.H;
  const int Sq = (int)p.Sq, Skv = (int)p.Skv, nt = (int)p.nt;
  const int q0 = qt * BMK + wave * 32;  // this wave's first query
  const int qi = q0 + j;               // this lane's query
  const bool act = q0 < Sq;            // uniform per wave: any query to compute
  const int64_t bb = bh / p.H;
  // K rows gathered from the codes: row r of head (b, h) at kbase + r kstride
  const uint8_t* kbase = p.k + (G::QIMG ? bh * nt * (int64_t)G::KBYTES : p.kmap.row(bb, hd, 0) * G::KROW);
  const uint32_t kstride = (uint32_t)(p.kmap.ss * G::KROW);
  const uint8_t* vtbase = p.vt + bh * nt * (int64_t)G::VBYTES;
  const uint8_t* auxbase = p.aux + bh * nt * (int64_t)G::XBYTES;

  // ---- Q operands (B of S^T = K Q^T): lane (j, h) holds, for k-step ks,
  // the K-slice [K/2 h, K/2 h + K/2) of the instruction's K range
  bf16x8 qbf[G::QBF ? KS : 1];       // bf16 (images of E4M3 codes, or the inputs)
  i32x4 qi8[G::QI8 ? KS : 1];        // INT8: 16 codes
  i32x8 qmx[QK == QK_MX4 ? KS : 1];  // MXFP4: 32 E2M1 codes (16 bytes used)
  int qsc[QK == QK_MX4 ? KS : 1];    // MXFP4: their E8M0 exponents
  float cq;
  {
    const bool ok = qi < Sq;
    const int64_t qrow_i = bh * p.Sq + (ok ? qi : 0);      // logical row (scales)
    const int64_t qmem = p.qmap.row(bb, hd, ok ? qi : 0);  // memory row (codes)
    // per-token / token-block / per-head float Q scale of this query
    const int64_t qsi = (bh / p.H) * p.q_sb + hd * p.q_sh + (ok ? qi : 0) / p.q_block;
    if (QK == QK_GEN) {
      // any format, widened exactly (MX relative to the row's largest block
      // exponent, which scales the scores); once per workgroup, so the
      // format is a runtime switch
      const int fmt = p.qfmt;
      const uint8_t* qrow = p.q + qmem * fmt_row_bytes(fmt, D);
      const bool mx = fmt == FMT_MX4 || fmt == FMT_MX8;
      const uint8_t* qe = reinterpret_cast<const uint8_t*>(p.qs) + qrow_i * NB;
      int emax = 0;
      if (mx && ok)
        for (int b = 0; b < NB; ++b) emax = max(emax, (int)qe[b]);
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
        uint4 a = make_uint4(0, 0, 0, 0);
        if (ok) a = widen8(fmt, qrow, 16 * ks + 8 * h, qe, emax);
        qbf[ks] = __builtin_bit_cast(bf16x8, a);
      }
      if (fmt == FMT_BF16) cq = p.c_log2;
      else if (mx) cq = __builtin_amdgcn_ldexpf(1.0f, (ok ? emax : 127) - 127) * p.c_log2;
      else cq = (ok ? reinterpret_cast<const float*>(p.qs)[qsi] : 1.0f) * p.c_log2;
    } else if (QK == QK_BF) {
      const uint8_t* qrow = p.q + qmem * (2 * D);
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
        uint4 a = make_uint4(0, 0, 0, 0);
        if (ok) a = *reinterpret_cast<const uint4*>(qrow + 32 * ks + 16 * h);
        qbf[ks] = __builtin_bit_cast(bf16x8, a);
      }
      cq = p.c_log2;
    } else if (G::QBF) {
      const uint8_t* qrow = p.q + qmem * D;
      // MXFP8: the row relative to its largest block exponent
      int eb[QK == QK_MX8 ? NB : 1], emax = 127;
      if (QK == QK_MX8) {
        const uint8_t* qe = reinterpret_cast<const uint8_t*>(p.qs) + qrow_i * NB;
        emax = 0;
#pragma unroll
        for (int b = 0; b < NB; ++b) {
          eb[b] = ok ? (int)qe[b] : 127;
          emax = max(emax, eb[b]);
        }
      }
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
        uint2 a = make_uint2(0, 0);
        if (ok) a = *reinterpret_cast<const uint2*>(qrow + 16 * ks + 8 * h);
        const float sc = QK == QK_MX8 ? __builtin_amdgcn_ldexpf(1.0f, eb[ks >> 1] - emax) : 1.0f;
        qbf[ks] = __builtin_bit_cast(bf16x8, i32x4{(int)e4m3x2_to_bf16x2<false>(a.x, sc),
                                                  (int)e4m3x2_to_bf16x2<true>(a.x, sc),
                                                  (int)e4m3x2_to_bf16x2<false>(a.y, sc),
                                                  (int)e4m3x2_to_bf16x2<true>(a.y, sc)});
      }
      if (QK == QK_MX8) cq = __builtin_amdgcn_ldexpf(1.0f, emax - 127) * p.c_log2;
      else cq = (ok ? reinterpret_cast<const float*>(p.qs)[qsi] : 1.0f) * p.c_log2;
    } else if (G::QI8) {
      const uint8_t* qrow = p.q + qmem * D;
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
        uint4 a = make_uint4(0, 0, 0, 0);
        if (ok) a = *reinterpret_cast<const uint4*>(qrow + 32 * ks + 16 * h);
        qi8[ks] = i32x4{(int)a.x, (int)a.y, (int)a.z, (int)a.w};
      }
      const float* qs = reinterpret_cast<const float*>(p.qs);
      if (QK == QK_I8H) cq = qs[hd] * reinterpret_cast<const float*>(p.ks)[hd] * p.c_log2;
      else cq = (ok ? qs[qsi] : 1.0f) * p.c_log2;
    } else {
      const uint8_t* qrow = p.q + qmem * (D / 2);
      const uint8_t* qe = reinterpret_cast<const uint8_t*>(p.qs) + qrow_i * NB;
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
        uint4 a = make_uint4(0, 0, 0, 0);
        int sc = 127;
        if (ok) {
          a = *reinterpret_cast<const uint4*>(qrow + 32 * ks + 16 * h);
          sc = qe[2 * ks + h];
        }
        qmx[ks] = i32x8{(int)a.x, (int)a.y, (int)a.z, (int)a.w, 0, 0, 0, 0};
        qsc[ks] = sc;
      }
      cq = p.c_log2;
    }
  }

  // ---- operand addresses in a K / V^T buffer: per-lane offsets, constant
  // offsets per step
  const int kop_off = h * (BN * 16) + kslot(qk_row(j)) * 16;  // + ks 2 BN 16 + kb 256
  const int vop_off = h * (D * 16) + j * 16;                  // + kstep 2 D 16 + db 512
  const int vop8_off = (4 * h * D + j) * 16;                  // E4M3 V^T: + s 2 D 16 + db 512 (+ D 16)
  // E5M2 V^T (MXFP4 values): the 8-bit A operand of the 32x32x64 f8f6f4
  // MFMA holds, in lane half h, K 16 h .. 16 h + 15 in bytes 0-15 and K
  // 32 + 16 h .. in bytes 16-31, while the E2M1 P operand holds K 32 h' ..
  // 32 h' + 31 in order (keys 64 h' + 32 s + 0..31).  So byte b < 16 of
  // lane half h is key 32 s + 16 h + b (image column 2 s + h) and byte
  // 16 + b key 64 + 32 s + 16 h + b (column 4 + 2 s + h).
  const int vop4_off = (h * D + j) * 16;                      // + s 2 D 16 + db 512 (+ 4 D 16)
  const int xk_off = G::KBYTES + 256 * h;                     // the lane's keys' K scales (floats)
  const int xv_off = G::VBYTES + 256 * h;                     // their qmax w_j (floats)
  const int xmx_off = G::KBYTES + qk_row(j) * NB + h;         // MXFP4: + 16 kb NB + 2 ks
  // V read as rows: the tile is chunk-major (16-byte column c of the key
  // rows, key in slot key ^ VSWZ (c & 1), which keeps the two 16-lane
  // groups of one read in distinct banks).  The A operand of the value MFMA
  // (rows = channels, k = the keys in P's lane order: k-position 16 h + r
  // is key 64 h + 16 kb + r) comes from two transposing reads rd: in
  // 16-lane group g = lane / 16, source lane s points at bytes 8 (s % 2) ..
  // + 7 of channel chunk g % 2 of key 64 (g / 2) + 16 kb + 8 rd + s / 2, so
  // output lane l holds channel 16 (g % 2) + l % 16 of keys 8 rd .. + 7.
  // Offsets at kb = db = 0; kb adds 256 bytes, db 4096.
  constexpr int VSWZ = 8;
  int vtr_off[2] = {0, 0};
  if (G::VROWS && !VDIR) {
    const int g = lane >> 4, s = lane & 15;
#pragma unroll
    for (int rd = 0; rd < 2; ++rd) {
      const int c = g & 1, key = 64 * (g >> 1) + 8 * rd + (s >> 1);
      vtr_off[rd] = c * (BN * 16) + (key ^ (VSWZ * (c & 1))) * 16 + 8 * (s & 1);
    }
  }

  // ---- tile copies.  K: FP8 / MXFP8 copy the bf16 image from the
  // workspace; the other modes gather K rows into the chunk-major layout
  // (round i of a lane moves column (NTK / 128) i + pw / 128 of slot
  // pw % 128, i.e.
  // of K row kslot(pw % 128); rows past the end re-read the last row,
  // masked).
  const int pw = wave * 64 + lane;
  const uint32_t loff_lin = (uint32_t)pw * 16;  // chunk i NTK + pw of a contiguous image
  const int krow = kslot(pw & (BN - 1));
  auto issue_k = [&](int t, uint8_t* kb) {
    if (G::QIMG) {
      stage<G::KBYTES / 16, NTK>(kb, kbase + (int64_t)t * G::KBYTES, wave, lane, loff_lin,
                                             NTK * 16);
    } else {
      const uint32_t roff = (uint32_t)min(t * BN + krow, Skv - 1) * kstride + (uint32_t)((pw >> 7) * 16);
      stage<G::KBYTES / 16, NTK>(kb, kbase, wave, lane, roff, (NTK / 128) * 16);
    }
    if (G::XKBYTES > 0)
      stage<G::XKBYTES / 16, NTK>(kb + G::KBYTES, auxbase + (int64_t)t * G::XBYTES, wave, lane,
                                              loff_lin, NTK * 16);
  };
  // direct V: thread (cc, g) = (tid / 32, tid % 32) moves the 16 keys of
  // V^T column cc (keys 64 (cc & 1) + 16 (cc >> 1) + r) times channels
  // 4 g .. 4 g + 3: 16 four-byte row loads, four 4x4 byte transposes, and
  // four 16-byte chunks of V^T rows 4 g .. 4 g + 3
  uint32_t vreg[VDIR ? 16 : 1];
  const int vcc = tid >> 5, vg = tid & 31;
  const int vkey0 = 64 * (vcc & 1) + 16 * (vcc >> 1);
  const uint8_t* vrow = VDIR ? p.vcodes + p.vmap.row(bb, hd, 0) * D + 4 * vg : nullptr;
  // (every thread issues exactly 16 loads - rows past the end re-read the
  // last row and are zeroed when stored - so the wait for the K copy issued
  // before them can count them)
  auto load_v = [&](int t) {
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int key = t * BN + vkey0 + r;
      vreg[r] = *reinterpret_cast<const uint32_t*>(vrow + (int64_t)min(key, Skv - 1) * p.vmap.ss * D);
    }
  };
  auto store_vt = [&](int t) {
#pragma unroll
    for (int r = 0; r < 16; ++r)
      if (t * BN + vkey0 + r >= Skv) vreg[r] = 0u;
    uint32_t o[4][4];  // [channel j][4-key group]
#pragma unroll
    for (int kg = 0; kg < 4; ++kg) {
      const uint32_t w0 = vreg[4 * kg], w1 = vreg[4 * kg + 1], w2 = vreg[4 * kg + 2], w3 = vreg[4 * kg + 3];
      const uint32_t t0 = __builtin_amdgcn_perm(w1, w0, 0x05010400u), t1 = __builtin_amdgcn_perm(w1, w0, 0x07030602u);
      const uint32_t t2 = __builtin_amdgcn_perm(w3, w2, 0x05010400u), t3 = __builtin_amdgcn_perm(w3, w2, 0x07030602u);
      o[0][kg] = __builtin_amdgcn_perm(t2, t0, 0x05040100u);
      o[1][kg] = __builtin_amdgcn_perm(t2, t0, 0x07060302u);
      o[2][kg] = __builtin_amdgcn_perm(t3, t1, 0x05040100u);
      o[3][kg] = __builtin_amdgcn_perm(t3, t1, 0x07060302u);
    }
#pragma unroll
    for (int jj = 0; jj < 4; ++jj)
      *reinterpret_cast<uint4*>(vbuf + (vcc * D + 4 * vg + jj) * 16) = make_uint4(o[jj][0], o[jj][1], o[jj][2], o[jj][3]);
  };
  // V rows (read as rows): the rows of head (b, h) at vrows + r vrstride
  constexpr int VRB = G::PI8 ? D : 2 * D;  // bytes of a V row
  const uint8_t* vrows = (G::VROWS && !VDIR) ? p.vcodes + p.vmap.row(bb, hd, 0) * VRB : nullptr;
  const uint32_t vrstride = (uint32_t)(p.vmap.ss * VRB);
  // f4: copy only the first E5M2 image of an MXFP4 value tile
  auto issue_v = [&](int t, uint8_t* vb, bool f4 = false) {
    if (G::PF4 && f4) {
      stage<G::VF4BYTES / 16, NTK>(vb, vtbase + (int64_t)t * G::VBYTES, wave, lane, loff_lin, NTK * 16);
    } else if (G::VROWS && !VDIR) {
      // chunk i NTK + pw: column c = i (NTK / 128) + pw / 128, slot pw % 128
      // holding key slot ^ VSWZ (c & 1) (NTK / 128 is even: c & 1 is the
      // same in every round)
      const int c0 = pw >> 7;
      const int key = (pw & (BN - 1)) ^ (VSWZ * (c0 & 1));
      stage<G::VBYTES / 16, NTK>(vb, vrows, wave, lane,
                                     (uint32_t)min(t * BN + key, Skv - 1) * vrstride + (uint32_t)(c0 * 16),
                                     (NTK / 128) * 16);
    } else {
      stage<G::VBYTES / 16, NTK>(vb, vtbase + (int64_t)t * G::VBYTES, wave, lane, loff_lin, NTK * 16);
    }
    if (G::XVBYTES > 0)
      stage<G::XVBYTES / 16, NTK>(vb + G::VBYTES, auxbase + (int64_t)t * G::XBYTES + G::XKBYTES, wave, lane,
                                      loff_lin, NTK * 16);
  };
  // copies each tile costs this wave (the wait counts of the ping-pong loop)
  const int kloads = stage_loads<G::KBYTES / 16, NTK>(wave) +
                     (G::XKBYTES > 0 ? stage_loads<G::XKBYTES / 16, NTK>(wave) : 0);
  const int vloads = stage_loads<G::VBYTES / 16, NTK>(wave) +
                     (G::XVBYTES > 0 ? stage_loads<G::XVBYTES / 16, NTK>(wave) : 0);

  // Row state (each lane holds its query's; both halves agree).  O holds
  // the output relative to a reference factor fref: the true accumulator is
  // O * fref (int8 values keep fref = 1 and fold their per-tile factor in
  // with an fma; the bf16 value product rescales O once per tile and lets
  // the P V MFMA accumulate straight into it).
  float M = -INFINITY, L = 0.f, fref = 1.f;
  // MXFP4 values: the current tile's flag (nonzero: a second E5M2 image)
  uint32_t vwide = 1;
  auto load_vwide = [&](int t) -> uint32_t {
    return __builtin_amdgcn_readfirstlane(
        *reinterpret_cast<const uint32_t*>(auxbase + (int64_t)t * G::XBYTES + G::XKBYTES + 32));
  };
  f32x16 O[DB];
#pragma unroll
  for (int db = 0; db < DB; ++db) O[db] = f32x16{};

  // per-group query range (ping-pong: group g holds queries
  // [qt BMK + 128 g, qt BMK + 128 g + 128)) and its causal diagonal tile
  const int gq0 = qt * BMK + 128 * grp;
  const int qlast = min(Sq, (qt + 1) * BMK) - 1;           // the workgroup's
  const int qlast_g = min(Sq, gq0 + 128) - 1;               // the group's
  const int dtile = gq0 / BN;
  const int t_beg = split * p.tps;
  const int t_end = CAUSAL ? min(nt, qlast / BN + 1) : min(nt, t_beg + p.tps);
  const int t_end_g = CAUSAL ? min(t_end, qlast_g / BN + 1) : t_end;
  const float vscale_i8 = (PV == PV_I8H) ? p.vs_head[hd] * (1.0f / 127.0f) : 1.0f;
  // valid keys of this lane's query: [0, lim)
  const int lim = CAUSAL ? min(Skv, qi + 1) : Skv;

  // ---- one tile in two phases.  Scores: S^T = K Q^T, per-key scales,
  // masking, the tile maximum and the row's combination factors.  Values:
  // probabilities, tile sum, the quantized P operand and O^T += V^T P^T.
  // The score phase leaves its state here for the value phase.
  f32x16 S[4];
  i32x16 SI[4];
  float rscale = 1.f, ce = cq, ms = 0.f, bt = 0.f;
  float gmax[2] = {-INFINITY, -INFINITY};
  auto phase_scores = [&](const int t, const uint8_t* kb) __attribute__((always_inline)) {
      const int k0 = t * BN;
      // the ragged last tile and the causal diagonal need a per-key validity
      // test; the other tiles skip it (uniform branch)
      const bool masked = (k0 + BN > Skv) || (CAUSAL && t == dtile);
      const int rel = lim - k0 - 64 * h;  // key 64 h + 16 kb + r is valid when 16 kb + r < rel
      const uint8_t* kop_base = kb + kop_off;
      const float* xk = reinterpret_cast<const float*>(kb + xk_off);
      const uint8_t* xmx = kb + xmx_off;
      rscale = 1.f; ce = cq; ms = 0.f; bt = 0.f;
      gmax[0] = -INFINITY; gmax[1] = -INFINITY;
      if (act) {
        // ---- S^T = K Q^T: four 32-key blocks, two at a time (two
        // independent accumulation chains keep the MFMA pipe full)
#pragma unroll
        for (int pr = 0; pr < 2; ++pr) {
#pragma unroll
          for (int ks = 0; ks < KS; ++ks) {
#pragma unroll
            for (int kk = 0; kk < 2; ++kk) {
              const int kb = 2 * pr + kk;
              const uint8_t* a = kop_base + ks * (2 * BN * 16) + kb * 256;
              if (G::QBF) {
                if (ks == 0) S[kb] = f32x16{};
                S[kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(lds_ld<bf16x8>(a), qbf[ks], S[kb], 0, 0, 0);
              } else if (G::QI8) {
                if (ks == 0) SI[kb] = i32x16{};
                const uint4 v = lds_ld<uint4>(a);
                SI[kb] = __builtin_amdgcn_mfma_i32_32x32x32_i8(i32x4{(int)v.x, (int)v.y, (int)v.z, (int)v.w}, qi8[ks],
                                                               SI[kb], 0, 0, 0);
              } else {
                if (ks == 0) S[kb] = f32x16{};
                const uint4 v = lds_ld<uint4>(a);
                const int sc = xmx[16 * kb * NB + 2 * ks];
                S[kb] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(
                    i32x8{(int)v.x, (int)v.y, (int)v.z, (int)v.w, 0, 0, 0, 0}, qmx[ks], S[kb], 4, 4, 0, sc, 0, qsc[ks]);
              }
            }
          }
        }

        // ---- per-key K scale, masking, tile maximum
        float m;
        if (QK == QK_I8H) {
          if (!masked) {
            // exact int32 scores (|s| < 2^21): max in integers, converted once
            int mi = INT_MIN;
#pragma unroll
            for (int kb = 0; kb < 4; ++kb)
#pragma unroll
              for (int r = 0; r < 16; r += 2) mi = max(max(mi, SI[kb][r]), SI[kb][r + 1]);  // v_max3_i32
            m = (float)mi;
#pragma unroll
            for (int kb = 0; kb < 4; ++kb)
#pragma unroll
              for (int r = 0; r < 16; ++r) S[kb][r] = (float)SI[kb][r];
          } else {
            m = -INFINITY;
#pragma unroll
            for (int kb = 0; kb < 4; ++kb)
#pragma unroll
              for (int r = 0; r < 16; ++r) {
                S[kb][r] = (16 * kb + r < rel) ? (float)SI[kb][r] : -INFINITY;
                m = fmaxf(m, S[kb][r]);
              }
          }
        } else {
          if (QK == QK_I8T) {
#pragma unroll
            for (int kb = 0; kb < 4; ++kb)
#pragma unroll
              for (int r = 0; r < 16; ++r) S[kb][r] = (float)SI[kb][r];
          }
          if (PERKEY) {
#pragma unroll
            for (int kb = 0; kb < 4; ++kb)
#pragma unroll
              for (int q4 = 0; q4 < 4; ++q4) {
                const float4 sk = *reinterpret_cast<const float4*>(xk + 16 * kb + 4 * q4);
                S[kb][4 * q4 + 0] *= sk.x; S[kb][4 * q4 + 1] *= sk.y;
                S[kb][4 * q4 + 2] *= sk.z; S[kb][4 * q4 + 3] *= sk.w;
              }
          }
          if (masked) {
#pragma unroll
            for (int kb = 0; kb < 4; ++kb)
#pragma unroll
              for (int r = 0; r < 16; ++r) S[kb][r] = (16 * kb + r < rel) ? S[kb][r] : -INFINITY;
          }
#pragma unroll
          for (int g2 = 0; g2 < 2; ++g2) {
            float x = -INFINITY;
#pragma unroll
            for (int kb = 2 * g2; kb < 2 * g2 + 2; ++kb)
#pragma unroll
              for (int r = 0; r < 16; r += 2) x = fmaxf(fmaxf(x, S[kb][r]), S[kb][r + 1]);  // v_max3
            gmax[g2] = x;  // MX probabilities: the lane's 32-key group maxima
          }
          m = fmaxf(gmax[0], gmax[1]);
        }
        m = halves_max(m);

        // ---- the row's combination factors: a rescales what was
        // accumulated so far, bt weights this tile
        if (KCONST) ce = cq * xk[-64 * h];  // the tile's K scale
        const float ml = m * ce;  // tile max, log2 units (M is kept in these units)
        float Mn, a;
        if (G::PI8) {
          // lazy reference: keep the running reference unless this tile's max
          // exceeds it by more than 2^8 (tile weights stay <= 2^8, far from
          // overflow), so O is rescaled only when the max jumps
          const bool jump = ml > M + 8.0f;
          Mn = jump ? ml : M;
          a = jump ? __builtin_amdgcn_exp2f(M - ml) : 1.0f;
        } else {
          Mn = fmaxf(M, ml);
          a = __builtin_amdgcn_exp2f(M - Mn);
        }
        bt = (m == -INFINITY) ? 0.0f : __builtin_amdgcn_exp2f(ml - Mn);
        M = Mn;
        // a row whose tile is negligible (bt < 2^-64) keeps its reference
        // and contributes nothing, which keeps O bounded (bf16 value
        // product; the value phase takes the new reference factor)
        const bool live = G::PI8 || bt >= 0x1p-64f;
        rscale = a;
        L *= a;
        // a row that is not live takes +inf as its reference, so all its p are 0
        ms = (m == -INFINITY) ? 0.0f : (live ? m : INFINITY);
      }
  };
  auto phase_values = [&](const int t, const uint8_t* vb) __attribute__((always_inline)) {
      // the vector-heavy phase issues first when both waves of a SIMD are
      // ready, so the other wave's products fill the matrix unit meanwhile
      __builtin_amdgcn_s_setprio(1);
      const uint8_t* vop_base = vb + vop_off;
      const float* xv = reinterpret_cast<const float*>(vb + xv_off);
      const float sig_t = G::SIG ? *reinterpret_cast<const float*>(vb + G::VBYTES + G::XVW) : 1.0f;
      if (act) {
        // ---- probabilities, tile sum, the quantized P operand and
        // O^T += V^T P^T
        float ls0 = 0.f, ls1 = 0.f;
        if (G::PI8) {
          // the running max moves rarely once a row has seen its largest
          // scores: rescale only when some row of the wave needs it (before
          // the probabilities, so that they and their products share a block)
          if (__builtin_amdgcn_ballot_w64(rscale != 1.0f) != 0) {
#pragma unroll
            for (int db = 0; db < DB; ++db) O[db] *= rscale;
          }
          // per-head: 127 p = 2^((s - m) ce + log2 127), s - m exact (integer
          // scores).  When every row of the wave has |m ce| <= 64 (log2
          // units: all but extreme score magnitudes) the subtraction folds
          // into the fma, 2^(s ce + (log2 127 - m ce)): the argument then
          // carries the roundings of m ce and of that constant, below
          // 1.2e-5, a relative error of p ~30x under the 2^-12 of a code
          // near its rounding boundary (and 127 p at the maximum stays
          // within 1e-5 of 127, whose code it keeps).  Larger |m ce| would
          // carry ~2^-24 |m ce|, so those waves keep the subtraction.
          // per-token: the same fold, 2^(s ce - m ce) times 127 w_j: p at
          // the maximum within 3e-6 of 1, and the multiplier is kept 2^-15
          // off every code boundary, so the maximum keeps the exact rule's
          // code; other waves take p = 1 exactly at the maximum.
          i32x4 P[4];
          auto probs = [&](auto fused) __attribute__((always_inline)) {
            const float c127 = kLog2_127 - ms * ce;
#pragma unroll
            for (int kb = 0; kb < 4; ++kb) {
#pragma unroll
              for (int w = 0; w < 4; ++w) {
                float4 vm4;
                if (PV == PV_I8T) vm4 = *reinterpret_cast<const float4*>(xv + 16 * kb + 4 * w);
                const float vm[4] = {vm4.x, vm4.y, vm4.z, vm4.w};
                uint32_t word = 0, u[4];
#pragma unroll
                for (int b = 0; b < 4; ++b) {
                  const float x = S[kb][4 * w + b];
                  float pv;
                  if (PV == PV_I8H)
                    pv = decltype(fused)::value ? __builtin_amdgcn_exp2f(__builtin_fmaf(x, ce, c127))
                                                : __builtin_amdgcn_exp2f(__builtin_fmaf(x - ms, ce, kLog2_127));
                  else
                    pv = decltype(fused)::value ? __builtin_amdgcn_exp2f(__builtin_fmaf(x, ce, -ms * ce))
                                                : __builtin_amdgcn_exp2f((x - ms) * ce);
                  if (b & 1) ls1 += pv; else ls0 += pv;
                  if (PV == PV_I8T) {
                    // 2^23 + rne(127 p w_j) (ulp 1 in [2^23, 2^24), one
                    // rounding of the exact product, ties to even): the
                    // code is the low byte (0 <= 127 p w_j < 127.5)
                    u[b] = __builtin_bit_cast(uint32_t, __builtin_fmaf(pv, vm[b], 0x1p23f));
                  } else {
                    word = __builtin_amdgcn_cvt_pk_u8_f32(pv, (uint32_t)b, word);  // rne(127 p)
                  }
                }
                if (PV == PV_I8T) {
                  // bytes 0 of u0..u3 -> bytes 0..3: two pairs, then the pairs
                  const uint32_t lo = __builtin_amdgcn_perm(u[1], u[0], 0x0c0c0400u);
                  const uint32_t hi = __builtin_amdgcn_perm(u[3], u[2], 0x0c0c0400u);
                  word = __builtin_amdgcn_perm(hi, lo, 0x05040100u);
                }
                P[kb][w] = (int)word;
              }
            }
          };
          if (__builtin_amdgcn_ballot_w64(!(fabsf(ms * ce) <= 64.0f)) == 0)
            probs(std::true_type{});
          else
            probs(std::false_type{});
          L += halves_sum(ls0 + ls1) * (PV == PV_I8H ? bt * (1.0f / 127.0f) : bt);
          const float bv = PV == PV_I8H ? bt * vscale_i8 : bt * sig_t * (1.0f / 127.0f);
          // two output blocks at a time: two independent accumulation chains
#pragma unroll
          for (int d2 = 0; d2 < DB; d2 += 2) {
            i32x16 C[2] = {i32x16{}, i32x16{}};
#pragma unroll
            for (int kb = 0; kb < 4; ++kb)
#pragma unroll
              for (int dd = 0; dd < 2; ++dd) {
                i32x4 va;
                if (G::VROWS && !VDIR) {
                  const v2i lo = lds_tr8(vb + vtr_off[0] + kb * 256 + (d2 + dd) * 4096);
                  const v2i hi = lds_tr8(vb + vtr_off[1] + kb * 256 + (d2 + dd) * 4096);
                  va = i32x4{lo.x, lo.y, hi.x, hi.y};
                } else {
                  const uint4 v = lds_ld<uint4>(vop_base + kb * (2 * D * 16) + (d2 + dd) * 512);
                  va = i32x4{(int)v.x, (int)v.y, (int)v.z, (int)v.w};
                }
                C[dd] = __builtin_amdgcn_mfma_i32_32x32x32_i8(va, P[kb], C[dd], 0, 0, 0);
              }
#pragma unroll
            for (int dd = 0; dd < 2; ++dd)
#pragma unroll
              for (int r = 0; r < 16; ++r) O[d2 + dd][r] = __builtin_fmaf((float)C[dd][r], bv, O[d2 + dd][r]);
          }
        } else {
          // bf16 value product: the new reference factor f = bt (times
          // sigma_t / 448 for FP8 values; a row that is not live keeps its
          // own), rescale, then per 32-key block: probabilities, the bf16 P
          // operand of its two k-steps, and their products
          {
            float ft = bt;
            if (PV == PV_F8W || PV == PV_F8C) ft *= sig_t * (1.0f / 448.0f);
            const bool live = bt >= 0x1p-64f;
            rscale = live ? fref * rscale * __builtin_amdgcn_rcpf(ft) : rscale;
            fref = live ? ft : fref;
          }
#pragma unroll
          for (int db = 0; db < DB; ++db) O[db] *= rscale;
          float sc = 1.0f, isc = 1.0f;
          i32x8 p8[2];  // E4M3 values: the P codes of the two 64-key k-steps
          // The exponent argument.  (s - m) ce: exactly 0 at the tile
          // maximum, where p = 1 exactly.  The value modes fold the
          // subtraction when every row of the wave has |m ce| <= 64 (log2
          // units): s ce + c0, c0 = -m ce, one instruction per score.  That argument carries the rounding of
          // m ce, below 2^-18 absolute: p within 1e-5 (relative) of the
          // exact value, inside the 2^-12 a code counts as tied near a
          // boundary, and at the maximum within 2e-6 of 1, which keeps the
          // code there: the per-token multiplier is kept 2^-15 off every
          // boundary, 448 p (one V scale per tile) and bf16(p) stay 448 and
          // 1, and an MX group takes its exponent from the unfused form.
          // Other waves take (s - m) ce: per-token E4M3 values through a
          // second copy of the probability loop (their products come after
          // it); the other modes by shifting S in place and folding with
          // m = 0, the same roundings as the unfused form, since their
          // products are interleaved with the probabilities and a second
          // copy of that loop spills.
          auto values = [&](auto fused) __attribute__((always_inline)) {
          const float c0 = -ms * ce;
#pragma unroll
          for (int kb = 0; kb < 4; ++kb) {
            if (G::PMX && (kb & 1) == 0) {
              // this lane's keys of blocks kb, kb + 1 are one MX group:
              // group max -> shared exponent; p -> E2M1 / E4M3 of p / 2^E,
              // times 2^E, exact in bf16.  The exponent comes from the
              // unfused p of the group's largest score (exactly 1 at the
              // tile maximum); a fused p lies within 1e-5 of it, so the
              // group maximum still lands at [4, 8) 2^E (E2M1, saturating
              // to 6) or [256, 512) 2^E (E4M3, 448) and keeps its code.
              const float pmax = __builtin_amdgcn_exp2f((gmax[kb >> 1] - ms) * ce);
              const int E = PV == PV_MX4 ? mx_exponent(pmax) : mx_exponent<8>(pmax);
              sc = E > -127 ? pow2f(E) : 1.0f;
              isc = E > -127 ? pow2f(-E) : 1.0f;
            }
#pragma unroll
            for (int s2 = 0; s2 < 2; ++s2) {
              float pv[8];
#pragma unroll
              for (int t8 = 0; t8 < 8; ++t8) {
                const float x = S[kb][8 * s2 + t8];
                // 448 p (one V scale per tile) or p
                float arg;
                if constexpr (decltype(fused)::value) arg = __builtin_fmaf(x, ce, PV == PV_F8C ? c0 + kLog2_448 : c0);
                else arg = PV == PV_F8C ? __builtin_fmaf(x - ms, ce, kLog2_448) : (x - ms) * ce;
                pv[t8] = __builtin_amdgcn_exp2f(arg);
                if (t8 & 1) ls1 += pv[t8]; else ls0 += pv[t8];
              }
              i32x4 pop;
              if (PV == PV_F8W || PV == PV_F8C) {
                // E4M3 of 448 p w_j (round to nearest even): the f8f6f4
                // operand (per-token V), or its exact bf16 image
                if (PV == PV_F8W) {
                  const float4 v0 = *reinterpret_cast<const float4*>(xv + 16 * kb + 8 * s2);
                  const float4 v1 = *reinterpret_cast<const float4*>(xv + 16 * kb + 8 * s2 + 4);
                  pv[0] *= v0.x; pv[1] *= v0.y; pv[2] *= v0.z; pv[3] *= v0.w;
                  pv[4] *= v1.x; pv[5] *= v1.y; pv[6] *= v1.z; pv[7] *= v1.w;
                }
                int e0 = __builtin_amdgcn_cvt_pk_fp8_f32(pv[0], pv[1], 0, false);
                e0 = __builtin_amdgcn_cvt_pk_fp8_f32(pv[2], pv[3], e0, true);
                int e1 = __builtin_amdgcn_cvt_pk_fp8_f32(pv[4], pv[5], 0, false);
                e1 = __builtin_amdgcn_cvt_pk_fp8_f32(pv[6], pv[7], e1, true);
                if (G::PF8) {
                  // the codes of keys 16 kb + 8 s2 .. + 7 of the lane's half:
                  // bytes 16 (kb % 2) + 8 s2 .. of k-step kb / 2
                  p8[kb >> 1][4 * (kb & 1) + 2 * s2] = e0;
                  p8[kb >> 1][4 * (kb & 1) + 2 * s2 + 1] = e1;
                  continue;
                }
                pop = i32x4{(int)e4m3x2_to_bf16x2<false>((uint32_t)e0), (int)e4m3x2_to_bf16x2<true>((uint32_t)e0),
                            (int)e4m3x2_to_bf16x2<false>((uint32_t)e1), (int)e4m3x2_to_bf16x2<true>((uint32_t)e1)};
              } else if (PV == PV_MX8) {
                // E4M3 of p / 2^E (exact scaling; the group maximum lies in
                // [256, 512) and saturates above 448), then back times 2^E
                float u[8];
#pragma unroll
                for (int t8 = 0; t8 < 8; ++t8) u[t8] = fminf(pv[t8] * isc, 448.0f);
                int e0 = __builtin_amdgcn_cvt_pk_fp8_f32(u[0], u[1], 0, false);
                e0 = __builtin_amdgcn_cvt_pk_fp8_f32(u[2], u[3], e0, true);
                int e1 = __builtin_amdgcn_cvt_pk_fp8_f32(u[4], u[5], 0, false);
                e1 = __builtin_amdgcn_cvt_pk_fp8_f32(u[6], u[7], e1, true);
                pop = i32x4{(int)e4m3x2_to_bf16x2<false>((uint32_t)e0, sc),
                            (int)e4m3x2_to_bf16x2<true>((uint32_t)e0, sc),
                            (int)e4m3x2_to_bf16x2<false>((uint32_t)e1, sc),
                            (int)e4m3x2_to_bf16x2<true>((uint32_t)e1, sc)};
              } else if (PV == PV_MX4) {
                // each pair through byte 0: E2M1(p / 2^E), then back times 2^E
#pragma unroll
                for (int b = 0; b < 4; ++b) {
                  const uint32_t f4 = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(0u, pv[2 * b], pv[2 * b + 1], sc, 0);
                  pop[b] = (int)__builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(f4, sc, 0));
                }
              } else {
                // unquantized V: p rounded to bf16 (nearest even)
#pragma unroll
                for (int b = 0; b < 4; ++b) {
                  const bf16x2 pr2 = {(__bf16)pv[2 * b], (__bf16)pv[2 * b + 1]};
                  pop[b] = (int)__builtin_bit_cast(uint32_t, pr2);
                }
              }
              const bf16x8 pb = __builtin_bit_cast(bf16x8, pop);
              const int kst = 2 * kb + s2;
#pragma unroll
              for (int db = 0; db < DB; ++db)
                O[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
                    lds_ld<bf16x8>(vop_base + kst * (2 * D * 16) + db * 512), pb, O[db], 0, 0, 0);
            }
          }
          };
          // MXFP4 Q, K and V, tile with an E5M2 V^T image: per 32-key group
          // (k-step s: the lane's keys 64 h + 32 s + 0..31, one MX group)
          // the group exponent E as in the bf16 path, the E2M1 codes of
          // p / 2^E packed eight to a word (the B operand, E + 127 its
          // scale), then O^T += V^T P^T on the block-scaled f8f6f4 MFMA
          // with the E5M2 image as A (its scale per key group and channel
          // block), accumulating into the rescaled O.  The products are
          // those of the exact values; the instruction sums them to about
          // 2^-12 of the largest, an error that enters O linearly.
          auto values_f4 = [&]() __attribute__((always_inline)) {
            const float c0 = -ms * ce;
            const uint8_t* vop4 = vb + vop4_off;
#pragma unroll
            for (int s = 0; s < 2; ++s) {
              const float pmax = __builtin_amdgcn_exp2f((gmax[s] - ms) * ce);
              const int E = mx_exponent(pmax);
              const float psc = E > -127 ? pow2f(E) : 1.0f;
              const int pe = E > -127 ? E + 127 : 127;
              i32x8 pb = {0, 0, 0, 0, 0, 0, 0, 0};
#pragma unroll
              for (int kk = 0; kk < 2; ++kk)
#pragma unroll
                for (int s2 = 0; s2 < 2; ++s2) {
                  float pv[8];
#pragma unroll
                  for (int t8 = 0; t8 < 8; ++t8) {
                    pv[t8] = __builtin_amdgcn_exp2f(__builtin_fmaf(S[2 * s + kk][8 * s2 + t8], ce, c0));
                    if (t8 & 1) ls1 += pv[t8]; else ls0 += pv[t8];
                  }
                  // keys 16 kk + 8 s2 + 0..7 of the group: nibbles of word 2 kk + s2
                  uint32_t w = 0;
                  w = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w, pv[0], pv[1], psc, 0);
                  w = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w, pv[2], pv[3], psc, 1);
                  w = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w, pv[4], pv[5], psc, 2);
                  w = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w, pv[6], pv[7], psc, 3);
                  pb[2 * kk + s2] = (int)w;
                }
              // E5M2 scales of key group 2 h + s: byte b for channel block b
              const uint32_t vsc = *reinterpret_cast<const uint32_t*>(vb + G::VBYTES + 4 * (2 * h + s));
#pragma unroll
              for (int db = 0; db < DB; ++db) {
                const uint8_t* a = vop4 + (2 * s * D + 32 * db) * 16;
                const uint4 lo = lds_ld<uint4>(a), hi = lds_ld<uint4>(a + 4 * D * 16);
                const i32x8 va = {(int)lo.x, (int)lo.y, (int)lo.z, (int)lo.w,
                                  (int)hi.x, (int)hi.y, (int)hi.z, (int)hi.w};
                O[db] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(va, pb, O[db], 1, 4, 0,
                                                                        (int)((vsc >> (8 * db)) & 0xffu), 0, pe);
              }
              if (vwide != 0) {
                // flagged tile: the elements the first image leaves out are
                // in the second one (upper half of the slot), its scales
                // after the first image's
                const uint32_t vsc1 = *reinterpret_cast<const uint32_t*>(vb + G::VBYTES + 16 + 4 * (2 * h + s));
#pragma unroll
                for (int db = 0; db < DB; ++db) {
                  const uint8_t* a = vop4 + G::VF4BYTES + (2 * s * D + 32 * db) * 16;
                  const uint4 lo = lds_ld<uint4>(a), hi = lds_ld<uint4>(a + 4 * D * 16);
                  const i32x8 va = {(int)lo.x, (int)lo.y, (int)lo.z, (int)lo.w,
                                    (int)hi.x, (int)hi.y, (int)hi.z, (int)hi.w};
                  O[db] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(va, pb, O[db], 1, 4, 0,
                                                                          (int)((vsc1 >> (8 * db)) & 0xffu), 0, pe);
                }
              }
            }
          };
          if constexpr (G::PF8) {
            if (__builtin_amdgcn_ballot_w64(!(fabsf(ms * ce) <= 64.0f)) == 0) values(std::true_type{});
            else values(std::false_type{});
          } else {
            // rare: a wave with a large |m ce| shifts its scores (and MX
            // group maxima) instead
            if (__builtin_amdgcn_ballot_w64(!(fabsf(ms * ce) <= 64.0f)) != 0) {
#pragma unroll
              for (int kb = 0; kb < 4; ++kb)
#pragma unroll
                for (int r = 0; r < 16; ++r) S[kb][r] -= ms;
              if (G::PMX) {
                gmax[0] -= ms;
                gmax[1] -= ms;
              }
              ms = 0.0f;
            }
            if constexpr (G::PF4) values_f4();
            else values(std::true_type{});
          }
          if (G::PF8) {
            // O^T += V^T P^T on the f8f6f4 MFMA (E4M3 x E4M3), straight into
            // the rescaled O: the MFMA adds its accumulator input at fp32
            // precision and sums its products to about 2^-12 of the largest,
            // an error that enters O linearly (no code is decided after it).
            // The DB output blocks are independent chains of two MFMAs each.
            const uint8_t* vop8 = vb + vop8_off;
#pragma unroll
            for (int s = 0; s < 2; ++s)
#pragma unroll
              for (int db = 0; db < DB; ++db) {
                const uint8_t* a = vop8 + (2 * s * D + 32 * db) * 16;
                const uint4 lo = lds_ld<uint4>(a), hi = lds_ld<uint4>(a + D * 16);
                const i32x8 va = {(int)lo.x, (int)lo.y, (int)lo.z, (int)lo.w,
                                  (int)hi.x, (int)hi.y, (int)hi.z, (int)hi.w};
                O[db] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(va, p8[s], O[db], 0, 0, 0, 0, 0, 0);
              }
          }
          const float lsc = PV == PV_F8C ? (1.0f / 448.0f) : 1.0f;
          L += halves_sum(ls0 + ls1) * (bt * lsc);
        }
      }
      __builtin_amdgcn_s_setprio(0);
  };

  if (VDIR) {
    // direct V (decode): the rows of V(t + 1) are loaded into registers and
    // K(t + 2) is copied into the other K buffer while the products of
    // tile t and the scores of t + 1 run.  K copies are not tracked by the
    // compiler; the wait for the V rows (vmcnt(0) before they are stored)
    // also covers the K copy issued before them, and the barriers drain
    // nothing else.
    // (K(t) lives in the buffer of t's parity)
    issue_k(t_beg, (t_beg & 1) ? kbuf1 : kbuf);
    if (t_beg + 1 < t_end) issue_k(t_beg + 1, (t_beg & 1) ? kbuf : kbuf1);
    load_v(t_beg);
    __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0)
    barrier_lds();
#pragma clang loop unroll(disable)
    for (int t = t_beg; t < t_end; ++t) {
      uint8_t* kb = (t & 1) ? kbuf1 : kbuf;
      phase_scores(t, kb);
      // V(t) and K(t + 1) have landed; V^T(t) goes into the LDS tile (every
      // wave finished the products of t - 1 at the last barrier)
      __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0)
      store_vt(t);
      barrier_lds();
      // every wave is done with K(t): its buffer takes K(t + 2)
      if (t + 2 < t_end) issue_k(t + 2, kb);
      if (t + 1 < t_end) load_v(t + 1);
      phase_values(t, vbuf);
      barrier_lds();
    }
  } else if (!PP) {
    issue_k(t_beg, kbuf);
    // MXFP4 values: each tile's flag is read one tile ahead
    uint32_t vwide_next = G::PF4 && t_beg < t_end ? load_vwide(t_beg) : 1u;
    __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0)
    __syncthreads();
#pragma clang loop unroll(disable)
    for (int t = t_beg; t < t_end; ++t) {
      if (G::PF4) {
        vwide = vwide_next;
        if (t + 1 < t_end) vwide_next = load_vwide(t + 1);
      }
      issue_v(t, vbuf, vwide == 0);
      phase_scores(t, kbuf);
      // V(t) has landed everywhere and every wave is done with K(t)
      __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0)
      __syncthreads();
      if (t + 1 < t_end) issue_k(t + 1, kbuf);
      phase_values(t, vbuf);
      // K(t+1) has landed everywhere and every wave is done with V(t)
      __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0)
      __syncthreads();
    }
  } else {
    // Slots separated by workgroup barriers.  Slot 2r: group 0 scores tile
    // r while group 1 takes the values of tile r - 1; slot 2r + 1: group 0
    // the values of r, group 1 the scores of r.  Copies: slot 2r issues
    // K(r + 1), slot 2r + 1 issues V(r + 1), each into the buffer of its
    // tile's parity; the tile a slot needs next has landed at its end,
    // while the copy it issued may stay in flight (vmcnt of that copy).
    // r counts tiles from t_beg; even r use kbuf / vbuf, odd r kbuf1 / vbuf1
    // (separate objects, so the compiler sees that reads of one buffer never
    // alias copies into the other).
    const int nr = t_end - t_beg, nr_g = t_end_g - t_beg;
    auto slot_k = [&](int r, auto odd) __attribute__((always_inline)) {  // issue K(r) into its buffer
      if (r < nr) issue_k(t_beg + r, decltype(odd)::value ? kbuf1 : kbuf);
      return r < nr ? kloads : 0;
    };
    auto slot_v = [&](int r, auto odd) __attribute__((always_inline)) {
      if (r < nr) issue_v(t_beg + r, decltype(odd)::value ? vbuf1 : vbuf);
      return r < nr ? vloads : 0;
    };
    using Even = std::integral_constant<bool, false>;
    using Odd = std::integral_constant<bool, true>;
    // tile r (parity ODD) of this wave: its two slots
    auto tile = [&](int r, auto odd) __attribute__((always_inline)) {
      constexpr bool O1 = decltype(odd)::value;
      using Next = std::integral_constant<bool, !O1>;
      const uint8_t* kb = O1 ? kbuf1 : kbuf;
      const uint8_t* vb = O1 ? vbuf1 : vbuf;
      int n;
      // scores of r: group 0 in slot 2r (issues K(r + 1)), group 1 in slot
      // 2r + 1 (issues V(r + 1))
      if (grp == 0) n = slot_k(r + 1, Next{});
      else n = slot_v(r + 1, Next{});
      if (r < nr_g) phase_scores(t_beg + r, kb);
      wait_vm(n);
      barrier_lds();
      // values of r: group 0 in slot 2r + 1 (issues V(r + 1)), group 1 in
      // slot 2r + 2 (issues K(r + 2))
      if (grp == 0) n = slot_v(r + 1, Next{});
      else n = slot_k(r + 2, odd);
      if (r < nr_g) phase_values(t_beg + r, vb);
      wait_vm(n);
      barrier_lds();
    };
    // prologue: the Q operands are in registers (so that no wait for them
    // lands inside the loop, where it would also wait for the copies);
    // K(0) lands before slot 0, V(0) during it
    __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0)
    issue_k(t_beg, kbuf);
    issue_v(t_beg, vbuf);
    wait_vm(vloads);
    barrier_lds();
    if (grp == 1) {  // slot 0 of group 1: no work, its share of K(1)
      wait_vm(slot_k(1, Odd{}));
      barrier_lds();
    }
#pragma clang loop unroll(disable)
    for (int r = 0; r < nr; r += 2) {
      tile(r, Even{});
      if (r + 1 < nr) tile(r + 1, Odd{});
    }
    if (grp == 0) {  // the last slot: group 1 finishes, no copies left
      __builtin_amdgcn_s_waitcnt(0x0F70);
      barrier_lds();
    }
  }

  // ---- a key split leaves its partial result: O times its reference
  // factor (unnormalized, relative to the running reference M), M and L
  if (p.nsplit > 1) {
    if (qi < Sq) {
      float* po = part_o(p.part, split, p.BH, p.Sq, bh, qi, D);
#pragma unroll
      for (int db = 0; db < DB; ++db)
#pragma unroll
        for (int a4 = 0; a4 < 4; ++a4)
          *reinterpret_cast<float4*>(po + 32 * db + 8 * a4 + 4 * h) =
              make_float4(O[db][4 * a4] * fref, O[db][4 * a4 + 1] * fref, O[db][4 * a4 + 2] * fref,
                          O[db][4 * a4 + 3] * fref);
      if (h == 0)
        *reinterpret_cast<float2*>(part_ml(p.part, p.nsplit, split, p.BH, p.Sq, bh, qi, D)) = make_float2(M, L);
    }
    return;
  }

  // ---- normalize, store: register r of block db is channel
  // 32 db + 8 (r / 4) + 4 h + r % 4 of query qi
  if (qi < Sq) {
    const float inv = fref / L;
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
      for (int a4 = 0; a4 < 4; ++a4) {
        const int64_t off = p.omap.row(bb, hd, qi) * D + 32 * db + 8 * a4 + 4 * h;
        const float o0 = O[db][4 * a4] * inv, o1 = O[db][4 * a4 + 1] * inv;
        const float o2 = O[db][4 * a4 + 2] * inv, o3 = O[db][4 * a4 + 3] * inv;
        if (p.out_bf16) {
          const uint32_t w0 = f32_to_bf16_bits(o0) | (f32_to_bf16_bits(o1) << 16);
          const uint32_t w1 = f32_to_bf16_bits(o2) | (f32_to_bf16_bits(o3) << 16);
          *reinterpret_cast<uint2*>(reinterpret_cast<uint16_t*>(p.out) + off) = make_uint2(w0, w1);
        } else {
          *reinterpret_cast<float4*>(reinterpret_cast<float*>(p.out) + off) = make_float4(o0, o1, o2, o3);
        }
      }
  }
}

// ------------------------------------------------------------------------
// Merge of the key splits: one wave per (b,h, query), D / 64 channels per
// lane.  M* = max_c M_c; O = sum_c 2^(M_c - M*) O_c / sum_c 2^(M_c - M*) L_c
// (M is kept in log2 units).
// ------------------------------------------------------------------------
template <int D>
__global__ __launch_bounds__(256) void k_combine(const float* __restrict__ part, int nsplit, int64_t BH, int64_t H,
                                                 int64_t Sq, RowMap omap, void* __restrict__ out, int out_bf16) {
  constexpr int CPL = D / 64;  // channels per lane
  const int64_t row = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (row >= BH * Sq) return;
  const int lane = threadIdx.x & 63;
  const int64_t bh = row / Sq, i = row % Sq;
  float* pp = const_cast<float*>(part);
  // lane c < nsplit holds split c's (M, L); its weight 2^(M_c - M*)
  float2 ml = make_float2(-INFINITY, 0.0f);
  if (lane < nsplit) ml = *reinterpret_cast<const float2*>(part_ml(pp, nsplit, lane, BH, Sq, bh, i, D));
  const float Ms = wave_max(ml.x);
  const float wgt = lane < nsplit ? __builtin_amdgcn_exp2f(ml.x - Ms) : 0.0f;
  float den = wgt * ml.y;
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) den += __shfl_xor(den, m, 64);
  float num[CPL] = {};
  for (int c = 0; c < nsplit; ++c) {
    const float wc = __shfl(wgt, c, 64);
    const float* po = part_o(pp, c, BH, Sq, bh, i, D) + lane * CPL;
#pragma unroll
    for (int k = 0; k < CPL; ++k) num[k] = __builtin_fmaf(wc, po[k], num[k]);
  }
  const float inv = 1.0f / den;
  const int64_t off = omap.row(bh / H, bh % H, i) * D + lane * CPL;
  if (out_bf16) {
    uint16_t* o = reinterpret_cast<uint16_t*>(out) + off;
#pragma unroll
    for (int k = 0; k < CPL; ++k) o[k] = (uint16_t)f32_to_bf16_bits(num[k] * inv);
  } else {
    float* o = reinterpret_cast<float*>(out) + off;
#pragma unroll
    for (int k = 0; k < CPL; ++k) o[k] = num[k] * inv;
  }
}

template <int QK, int PV, int D>
hipError_t launch_d(const AttnArgs& a, const WsLayout& l, hipStream_t st) {
  using G = Cfg<QK, PV, D>;
  const int64_t nt = (a.Skv + BN - 1) / BN;
  uint8_t* ws = reinterpret_cast<uint8_t*>(a.ws);
  PrepArgs pa{};
  pa.k = (const uint8_t*)a.k_codes; pa.ks = a.k_scales;
  pa.v = (const uint8_t*)a.v_codes; pa.vs = a.v_scales;
  pa.kmap = a.kmap; pa.vmap = a.vmap;
  pa.H = a.H; pa.Skv = a.Skv; pa.nt = nt;
  pa.ksb = a.k_sb; pa.ksh = a.k_sh; pa.kblk = a.k_block;
  pa.vsb = a.v_sb; pa.vsh = a.v_sh; pa.vblk = a.v_block;
  pa.kfmt = a.kfmt;
  pa.vt = ws + l.vt_off; pa.kb = ws + l.kb_off; pa.aux = ws + l.aux_off;
  const KvSplit sp = kv_split(a.B, a.H, a.Sq, a.Skv, a.causal);
  // decode with INT8 per-head V: the kernel transposes V itself
  constexpr bool VDIR_OK = QK == QK_I8H && PV == PV_I8H && D == 128;
  const bool vdir = VDIR_OK && sp.nsplit > 1;
  hipError_t e = hipSuccess;
  if (!vdir && !G::NOPREP) {
    k_prep<QK, PV, D><<<dim3((unsigned)nt, (unsigned)(a.B * a.H)), 256, 0, st>>>(pa);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  KParams p{};
  p.H = a.H; p.BH = a.B * a.H; p.Sq = a.Sq; p.Skv = a.Skv; p.nt = nt;
  p.nqt = (int)((a.Sq + BM - 1) / BM);
  p.qmap = a.qmap; p.kmap = a.kmap; p.omap = a.qmap;
  p.q = (const uint8_t*)a.q_codes; p.qs = a.q_scales;
  p.k = G::QIMG ? ws + l.kb_off : (const uint8_t*)a.k_codes;
  p.ks = a.k_scales;
  p.vt = ws + l.vt_off;
  p.aux = ws + l.aux_off;
  p.vs_head = (const float*)a.v_scales;
  p.q_sb = a.q_sb; p.q_sh = a.q_sh; p.q_block = a.q_block;
  p.qfmt = a.qfmt;
  p.c_log2 = a.sm_scale * kLog2e;
  p.out = a.out; p.out_bf16 = a.out_bf16;
  p.nsplit = sp.nsplit; p.tps = sp.tps;
  p.part = reinterpret_cast<float*>(ws + l.part_off);
  p.vcodes = (const uint8_t*)a.v_codes; p.vmap = a.vmap;
  dim3 grid((unsigned)(p.nqt * p.BH * sp.nsplit));
  if constexpr (VDIR_OK) {
    if (vdir) {
      k_attn<QK, PV, D, false, true><<<grid, NTHR, 0, st>>>(p);  // splits are never causal
      e = hipGetLastError();
      if (e != hipSuccess) return e;
      k_combine<D><<<(unsigned)((p.BH * p.Sq + 3) / 4), 256, 0, st>>>(p.part, sp.nsplit, p.BH, a.H, a.Sq, a.qmap,
                                                                     a.out, a.out_bf16);
      return hipGetLastError();
    }
  }
  if constexpr (G::QBF) {
    if (sp.nsplit == 1) {
      // bf16 score products, no key split: the ping-pong kernel, 256
      // queries per workgroup (INT8 / MXFP4 scores keep the four-wave
      // kernel, which is faster for them)
      p.nqt = (int)((a.Sq + 2 * BM - 1) / (2 * BM));
      const dim3 g2((unsigned)(p.nqt * p.BH));
      if (a.causal) k_attn<QK, PV, D, true, false, true><<<g2, 2 * NTHR, 0, st>>>(p);
      else k_attn<QK, PV, D, false, false, true><<<g2, 2 * NTHR, 0, st>>>(p);
      return hipGetLastError();
    }
  }
  if (a.causal) k_attn<QK, PV, D, true><<<grid, NTHR, 0, st>>>(p);
  else k_attn<QK, PV, D, false><<<grid, NTHR, 0, st>>>(p);  // key splits are never causal
  e = hipGetLastError();
  if (e != hipSuccess || sp.nsplit == 1) return e;
  k_combine<D><<<(unsigned)((p.BH * p.Sq + 3) / 4), 256, 0, st>>>(p.part, sp.nsplit, p.BH, a.H, a.Sq, a.qmap, a.out,
                                                                 a.out_bf16);
  return hipGetLastError();
}

template <int QK, int PV>
hipError_t launch_pair(const AttnArgs& a, const WsLayout& l, hipStream_t st) {
  return a.D == 128 ? launch_d<QK, PV, 128>(a, l, st) : launch_d<QK, PV, 64>(a, l, st);
}

// Quantized Q and K: V of their own configuration, or unquantized V.
template <int QK, int PV_OWN>
hipError_t launch_qk(const AttnArgs& a, const WsLayout& l, hipStream_t st) {
  if (a.pv == PV_BF) return launch_pair<QK, PV_BF>(a, l, st);
  return launch_pair<QK, PV_OWN>(a, l, st);
}

}  // namespace

bool attn_pair_supported(int qk, int pv) {
  if (pv == PV_BF || qk == QK_BF || qk == QK_GEN) return true;
  switch (qk) {
    case QK_I8H: return pv == PV_I8H;
    case QK_I8T: return pv == PV_I8T;
    case QK_F8T: return pv == PV_F8W;
    case QK_F8C: return pv == PV_F8C;
    case QK_MX4: return pv == PV_MX4;
    case QK_MX8: return pv == PV_MX8;
    default: return false;
  }
}

size_t attn_workspace_bytes(int qk, int pv, int64_t B, int64_t H, int64_t Sq, int64_t Skv, int64_t D, int causal) {
  return ws_layout(qk, pv, B, H, Sq, Skv, D, causal).total;
}

hipError_t launch_attention(const AttnArgs& a, hipStream_t st) {
  const WsLayout l = ws_layout(a.qk, a.pv, a.B, a.H, a.Sq, a.Skv, a.D, a.causal);
  switch (a.qk) {
    case QK_I8H: return launch_qk<QK_I8H, PV_I8H>(a, l, st);
    case QK_I8T: return launch_qk<QK_I8T, PV_I8T>(a, l, st);
    case QK_F8T: return launch_qk<QK_F8T, PV_F8W>(a, l, st);
    case QK_F8C: return launch_qk<QK_F8C, PV_F8C>(a, l, st);
    case QK_MX4: return launch_qk<QK_MX4, PV_MX4>(a, l, st);
    case QK_MX8: return launch_qk<QK_MX8, PV_MX8>(a, l, st);
    case QK_GEN:
      // any Q/K formats with any value mode
      switch (a.pv) {
        case PV_I8H: return launch_pair<QK_GEN, PV_I8H>(a, l, st);
        case PV_I8T: return launch_pair<QK_GEN, PV_I8T>(a, l, st);
        case PV_F8W: return launch_pair<QK_GEN, PV_F8W>(a, l, st);
        case PV_F8C: return launch_pair<QK_GEN, PV_F8C>(a, l, st);
        case PV_MX4: return launch_pair<QK_GEN, PV_MX4>(a, l, st);
        case PV_MX8: return launch_pair<QK_GEN, PV_MX8>(a, l, st);
        default: return launch_pair<QK_GEN, PV_BF>(a, l, st);
      }
    default:
      // unquantized Q and K with any value mode
      switch (a.pv) {
        case PV_I8H: return launch_pair<QK_BF, PV_I8H>(a, l, st);
        case PV_I8T: return launch_pair<QK_BF, PV_I8T>(a, l, st);
        case PV_F8W: return launch_pair<QK_BF, PV_F8W>(a, l, st);
        case PV_F8C: return launch_pair<QK_BF, PV_F8C>(a, l, st);
        case PV_MX4: return launch_pair<QK_BF, PV_MX4>(a, l, st);
        case PV_MX8: return launch_pair<QK_BF, PV_MX8>(a, l, st);
        default: return launch_pair<QK_BF, PV_BF>(a, l, st);
      }
  }
}

}  // namespace faq
