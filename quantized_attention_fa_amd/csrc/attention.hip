// Flash-style attention on quantized Q/K/V for gfx950.
//
// Both products take the low-bit operands ("FA 量化" page, 概述) on MFMA:
//   INT8 per-head  v_mfma_i32_16x16x64_i8 for Q K^T and P V (int8 P):
//                  exact int32 accumulation.
//   FP8 E4M3       v_mfma_f32_16x16x32_bf16 on the exact bf16 images of the
//                  E4M3 codes (Q, K, V and the E4M3 probabilities).  The
//                  f8f6f4 MFMA sums each group of 16 products aligned to the
//                  group's largest with about 12 fractional bits, so score
//                  errors reach ~1e-4 of amax_q * amax_k and move probability
//                  codes; the bf16 MFMA accumulates these exact products at
//                  fp32 precision.
//   MXFP4          Q K^T on v_mfma_scale_f32_16x16x128_f8f6f4 with E2M1
//                  operands and their E8M0 block exponents as MFMA scales
//                  (exact: products within a block span < 2^8); P V on the
//                  bf16 MFMA with P = E2M1 * 2^E and V dequantized exactly.
// The output is dequantized to bf16 (or fp32) ("量化" page, FA量化 / FP8
// Attention).
//
// Probability rule (the pages leave it open; this is the library's contract):
// keys are cut into 128-key tiles aligned to absolute key index; per query
// row and tile, m = max score, p = exp(s - m) is quantized with a static
// scale relative to that tile maximum (int8: rne(127 p); E4M3: 448 p w_j with
// w_j = s_v,j / max_tile s_v; MXFP4: the MX quantizer over 32-key groups),
// the tile sum L uses unquantized p, and tiles combine with the usual
// running-max rescale, O = sum_t e^{m_t-M} C_t / sum_t e^{m_t-M} L_t.
//
// Kernel shape: one workgroup = 8 waves = 256 queries of one (b,h); each
// wave owns 32 queries as two 16-query MFMA column blocks, and all eight
// share each K / V^T tile.  Tiles stream from global memory straight into
// LDS (global_load_lds, 16 bytes per lane), double buffered: the copy of
// tile t+1 runs while tile t is computed, with one barrier per tile.
// Scores are computed transposed (S^T = K Q^T), so a lane holds one query
// and a run of keys: the row max needs only two cross-lane steps, and the
// lane's probabilities are already the B operand of O^T = V^T P^T.  V comes
// from a per-call workspace already transposed per 128-key tile, with its
// keys permuted to match the order in which a lane holds its probabilities
// (FP8: K and V^T widened there to their exact bf16 images).
//
// Workgroups are numbered so that all query tiles of one (b,h) land on the
// same XCD (workgroups are dealt to the 8 XCDs round robin), which keeps a
// head's K/V tiles in that XCD's L2; causal grids run the longest query
// tiles first.

#include <climits>

#include "common.h"
#include "launch.h"

namespace faq {
namespace {

// Waves per workgroup: INT8 runs two 4-wave workgroups per CU (their
// tiles fit twice in LDS, and the two waves sharing a SIMD then come from
// independent workgroups, so one's softmax overlaps the other's MFMAs);
// FP8 and MXFP4 tiles are larger and run one 8-wave workgroup per CU.
template <int MODE>
struct Waves {
  static constexpr int NW = MODE == ATTN_INT8 ? 4 : 8;
  static constexpr int NTHR = NW * 64;  // threads per workgroup
  static constexpr int BM = NW * 32;    // queries per workgroup
  static constexpr int WG_PER_CU = 8 / NW;
};
constexpr int BN = 128;        // keys per tile = probability tile
constexpr float kLog2e = 1.4426950408889634f;

// Key order inside a V^T tile.  A lane of lane-group g (g = lane / 16) holds,
// for query column l16, the scores of MFMA block b (16 keys) at output rows
// 4g + r.  The K rows fed to block b are chosen per mode:
//   INT8, FP8: row 16b + i            -> lane g holds keys 16b + 4g + r
//   MXFP4:     row 32(i/4) + 4b + i%4 -> lane g holds keys 32g + 4b + r (one
//                                        32-key MX group per lane)
// The probabilities then feed O^T = V^T P^T as the B operand without moving
// between lanes, so V^T's columns are stored in the order the lanes hold
// their keys:
//   INT8 (i8 MFMA, 16 K-bytes per lane): column 32g + 4b + r <-> key 16b + 4g + r
//   FP8 / MXFP4 (bf16 MFMA 16x16x32, 8 K-elements per lane and block kk, the
//   lane's blocks b = 2kk and 2kk+1): column 32kk + 8g + t <-> key
//     FP8:   16(2kk + t/4) + 4g + t%4
//     MXFP4: 32g + 8kk + t
FAQ_DEV int vt_key_int8(int col) { return 16 * ((col >> 2) & 7) + 4 * (col >> 5) + (col & 3); }
FAQ_DEV int vt_key_fp8(int col) {
  const int kk = col >> 5, g = (col >> 3) & 3, t = col & 7;
  return 16 * (2 * kk + (t >> 2)) + 4 * g + (t & 3);
}
FAQ_DEV int vt_key_mx(int col) {
  const int kk = col >> 5, g = (col >> 3) & 3, t = col & 7;
  return 32 * g + 8 * kk + t;
}

// Row of the K tile read by lane-row i of MFMA block b in the MXFP4 kernel.
FAQ_DEV int k_row_mx(int b, int i) { return 32 * (i >> 2) + 4 * b + (i & 3); }

// XOR swizzles of the 16-byte chunks of a tile row.  An MFMA operand read
// has 16 consecutive lanes fetch the same chunk column of 16 consecutive
// rows; the LDS serves 64 banks (256 bytes) per cycle, so those 16 reads
// must land in 16 distinct 16-byte bank groups.  Each swizzle depends only
// on row bits that are the same for rows i and 16b + i, so an operand
// address is a per-lane base plus a constant offset per block.
FAQ_DEV int swz8(int row) { return (row >> 1) & 7; }   // 128-byte rows
FAQ_DEV int swz4(int row) { return (row >> 2) & 3; }   // 64-byte rows
FAQ_DEV int swz_mx(int row) { return (row >> 5) & 3; } // MXFP4 K rows (64 bytes, rows 32(i/4) + 4b + i%4)

// Two E4M3 bytes (the low half-word of `w`, or the high one when HI) -> two
// bf16, exactly.
template <bool HI>
FAQ_DEV uint32_t e4m3x2_to_bf16x2(uint32_t w) {
  return __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8((int)w, 1.0f, HI));
}

// Geometry of one LDS tile buffer: K rows, V^T rows, then per-key extras
// (FP8: K scale and 448 w_j as floats; MXFP4: the K block exponents).
template <int MODE, int D>
struct Geo {
  static constexpr int KROW = MODE == ATTN_INT8 ? D : (MODE == ATTN_FP8 ? 2 * D : D / 2);
  static constexpr int KCH = KROW / 16;  // 16-byte chunks per K row
  static constexpr int KBYTES = BN * KROW;
  static constexpr int VROW = MODE == ATTN_INT8 ? BN : 2 * BN;
  static constexpr int VCH = VROW / 16;
  static constexpr int VBYTES = D * VROW;
  static constexpr int XBYTES = MODE == ATTN_FP8 ? 2 * BN * 4 : (MODE == ATTN_MX ? BN * (D / 32) : 0);
  static constexpr int VOFF = KBYTES;
  static constexpr int XOFF = KBYTES + VBYTES;
  static constexpr int BUF = XOFF + XBYTES;
  // swizzled chunk of K row `row`
  FAQ_DEV int kswz(int row) {
    if (MODE == ATTN_INT8) return KCH == 8 ? swz8(row) : swz4(row);
    if (MODE == ATTN_FP8) return row & (KCH - 1);
    return KCH == 4 ? swz_mx(row) : 0;
  }
  FAQ_DEV int vswz(int row) { return MODE == ATTN_INT8 ? swz8(row) : (row & (VCH - 1)); }
};

// ------------------------------------------------------------------------
// Workspace layout (per (b,h), per 128-key tile t):
//   vt  : V^T of the tile, D rows x 128 keys: INT8 codes (1 byte) or, for
//         FP8 and MXFP4, the exact values in bf16 (2 bytes)
//   kb  : FP8: K widened to bf16, 128 rows x D (rows past the end are 0)
//   aux : FP8: 128 K scales then 128 multipliers 448 * w_j (floats);
//         MXFP4: the K block exponents, 128 rows x D/32 bytes (127 past
//         the end)
//   sig : FP8: sigma_t = max over the tile's keys of s_v,j
// ------------------------------------------------------------------------
struct WsLayout {
  size_t vt_off, kb_off, aux_off, sig_off, total;
};

inline WsLayout ws_layout(int mode, int64_t B, int64_t H, int64_t Skv, int64_t D) {
  const int64_t nt = (Skv + BN - 1) / BN;
  const size_t tiles = (size_t)(B * H * nt);
  auto up = [](size_t x) { return (x + 255) & ~size_t(255); };
  WsLayout l{};
  l.vt_off = 0;
  l.kb_off = up(tiles * D * BN * (mode == ATTN_INT8 ? 1 : 2));
  l.aux_off = l.kb_off + up(mode == ATTN_FP8 ? tiles * BN * D * 2 : 0);
  const size_t aux = mode == ATTN_FP8 ? tiles * 2 * BN * 4 : (mode == ATTN_MX ? tiles * BN * (D / 32) : 0);
  l.sig_off = l.aux_off + up(aux);
  l.total = l.sig_off + up(mode == ATTN_FP8 ? tiles * 4 : 0);
  return l;
}

// ------------------------------------------------------------------------
// Per-call re-layout.  grid = (tiles, B*H), 256 threads; one 128-key tile.
//   INT8 : V^T codes in the lane key order.
//   FP8  : K and V^T widened to bf16 (V^T in the lane key order), the
//          per-key K scales and 448 w_j, and sigma_t.
// ------------------------------------------------------------------------
template <int D, bool FP8>
__global__ __launch_bounds__(256) void k_prep(const uint8_t* __restrict__ k, const float* __restrict__ ks,
                                              const uint8_t* __restrict__ v, const float* __restrict__ vs,
                                              int64_t Skv, int kv_block, int64_t nt, uint8_t* __restrict__ vt,
                                              uint16_t* __restrict__ kb, float* __restrict__ aux,
                                              float* __restrict__ sig) {
  __shared__ uint8_t tile[BN][D + 4];
  __shared__ float red[4];
  const int t = blockIdx.x;
  const int64_t bh = blockIdx.y;
  const int64_t k0 = (int64_t)t * BN;
  const int64_t tile_id = bh * nt + t;
  const uint8_t* src = v + (bh * Skv + k0) * D;
  constexpr int CPR = D / 16;  // 16-byte chunks per key row
  for (int c = threadIdx.x; c < BN * CPR; c += 256) {
    const int kl = c / CPR, cc = c % CPR;
    uint4 val = make_uint4(0, 0, 0, 0);
    if (k0 + kl < Skv) val = *reinterpret_cast<const uint4*>(src + (int64_t)kl * D + cc * 16);
    uint32_t* dst = reinterpret_cast<uint32_t*>(&tile[kl][cc * 16]);
    dst[0] = val.x; dst[1] = val.y; dst[2] = val.z; dst[3] = val.w;
    if (FP8) {
      // K row chunk widened to bf16 (32 bytes)
      uint4 kv = make_uint4(0, 0, 0, 0);
      if (k0 + kl < Skv) kv = *reinterpret_cast<const uint4*>(k + (bh * Skv + k0 + kl) * D + cc * 16);
      uint16_t* kd = kb + (tile_id * BN + kl) * D + cc * 16;
      *reinterpret_cast<uint4*>(kd) = make_uint4(e4m3x2_to_bf16x2<false>(kv.x), e4m3x2_to_bf16x2<true>(kv.x),
                                                 e4m3x2_to_bf16x2<false>(kv.y), e4m3x2_to_bf16x2<true>(kv.y));
      *reinterpret_cast<uint4*>(kd + 8) = make_uint4(e4m3x2_to_bf16x2<false>(kv.z), e4m3x2_to_bf16x2<true>(kv.z),
                                                     e4m3x2_to_bf16x2<false>(kv.w), e4m3x2_to_bf16x2<true>(kv.w));
    }
  }
  __syncthreads();
  if (FP8) {
    uint16_t* out = reinterpret_cast<uint16_t*>(vt) + tile_id * (int64_t)D * BN;
    for (int c = threadIdx.x; c < D * (BN / 8); c += 256) {
      const int d = c / (BN / 8), c8 = (c % (BN / 8)) * 8;
      uint32_t w[4];
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const uint32_t pair = (uint32_t)tile[vt_key_fp8(c8 + 2 * q)][d] | ((uint32_t)tile[vt_key_fp8(c8 + 2 * q + 1)][d] << 8);
        w[q] = e4m3x2_to_bf16x2<false>(pair);
      }
      *reinterpret_cast<uint4*>(out + (int64_t)d * BN + c8) = make_uint4(w[0], w[1], w[2], w[3]);
    }
    const int kl = threadIdx.x;
    float s = 0.0f, sk = 0.0f;
    if (kl < BN && k0 + kl < Skv) {
      const int64_t nblk = (Skv + kv_block - 1) / kv_block;
      s = vs[bh * nblk + (k0 + kl) / kv_block];
      sk = ks[bh * nblk + (k0 + kl) / kv_block];
    }
    float m = wave_max(s);
    if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = m;
    __syncthreads();
    m = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
    if (kl < BN) {
      aux[tile_id * 2 * BN + kl] = sk;
      aux[tile_id * 2 * BN + BN + kl] = (s > 0.0f) ? 448.0f * (s / m) : 0.0f;
    }
    if (threadIdx.x == 0) sig[tile_id] = m;
  } else {
    uint8_t* out = vt + tile_id * (int64_t)D * BN;
    for (int c = threadIdx.x; c < D * (BN / 16); c += 256) {
      const int d = c / (BN / 16), j = c % (BN / 16);
      uint32_t w[4];
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        uint32_t acc = 0;
#pragma unroll
        for (int r = 0; r < 4; ++r) acc |= (uint32_t)tile[vt_key_int8(16 * j + 4 * q + r)][d] << (8 * r);
        w[q] = acc;
      }
      *reinterpret_cast<uint4*>(out + (int64_t)d * BN + 16 * j) = make_uint4(w[0], w[1], w[2], w[3]);
    }
  }
}

// ------------------------------------------------------------------------
// MXFP4 re-layout: V^T per tile as the exact bf16 values E2M1 * 2^E (E from
// the token's 32-channel block), in the lane key order; K block exponents
// per tile (127 = 2^0 past the end).
// ------------------------------------------------------------------------
template <int D>
__global__ __launch_bounds__(256) void k_prep_mx(const uint8_t* __restrict__ v, const uint8_t* __restrict__ ve,
                                                 const uint8_t* __restrict__ ke, int64_t Skv, int64_t nt,
                                                 uint16_t* __restrict__ vt, uint8_t* __restrict__ kex) {
  constexpr int NB = D / 32;
  __shared__ uint8_t codes[BN][D / 2 + 4];
  __shared__ uint8_t ex[BN][NB];
  const int t = blockIdx.x;
  const int64_t bh = blockIdx.y;
  const int64_t k0 = (int64_t)t * BN;
  const int64_t tile_id = bh * nt + t;
  for (int c = threadIdx.x; c < BN * (D / 32); c += 256) {
    const int kl = c / (D / 32), cc = c % (D / 32);  // 16-byte chunks of the packed row
    uint4 val = make_uint4(0, 0, 0, 0);
    if (k0 + kl < Skv) val = *reinterpret_cast<const uint4*>(v + (bh * Skv + k0 + kl) * (D / 2) + cc * 16);
    uint32_t* dst = reinterpret_cast<uint32_t*>(&codes[kl][cc * 16]);
    dst[0] = val.x; dst[1] = val.y; dst[2] = val.z; dst[3] = val.w;
  }
  for (int c = threadIdx.x; c < BN * NB; c += 256) {
    const int kl = c / NB, b = c % NB;
    const bool ok = k0 + kl < Skv;
    ex[kl][b] = ok ? ve[(bh * Skv + k0 + kl) * NB + b] : (uint8_t)127;
    kex[tile_id * BN * NB + c] = ok ? ke[(bh * Skv + k0 + kl) * NB + b] : (uint8_t)127;
  }
  __syncthreads();
  uint16_t* out = vt + tile_id * (int64_t)D * BN;
  // 8 output columns (16 bytes) per item
  for (int c = threadIdx.x; c < D * (BN / 8); c += 256) {
    const int d = c / (BN / 8), c8 = (c % (BN / 8)) * 8;
    uint32_t w[4];
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      uint32_t pair = 0;
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const int key = vt_key_mx(c8 + 2 * q + h);
        const uint32_t nib = (codes[key][d >> 1] >> (4 * (d & 1))) & 0xfu;
        const uint32_t mag = nib & 7u;
        // E2M1 magnitude: 0, .5, 1, 1.5, 2, 3, 4, 6; times 2^(e8m0 - 127)
        const float fm = mag < 2 ? 0.5f * (float)mag
                                 : (float)(1u << ((mag >> 1) - 1)) * (1.0f + 0.5f * (float)(mag & 1u));
        float f = __builtin_amdgcn_ldexpf(fm, (int)ex[key][d >> 5] - 127);
        f = (nib & 8u) ? -f : f;
        pair |= (__float_as_uint(f) >> 16) << (16 * h);  // exact: at most 2 significant bits
      }
      w[q] = pair;
    }
    *reinterpret_cast<uint4*>(out + (int64_t)d * BN + c8) = make_uint4(w[0], w[1], w[2], w[3]);
  }
}

// ------------------------------------------------------------------------
// The attention kernel.
// ------------------------------------------------------------------------
struct KParams {
  int64_t H, BH, Sq, Skv, nt;
  int nqt;
  const uint8_t* q;
  const void* qs;
  const uint8_t* k;      // INT8 / MXFP4: K codes; FP8: bf16 K tiles in the workspace
  const void* ks;        // INT8: per-head K scale
  const uint8_t* vt;     // V^T tiles in the workspace
  const uint8_t* aux;    // FP8: K scales + 448 w_j; MXFP4: K exponents (per tile)
  const float* sig;      // FP8: sigma_t
  const float* vs_head;  // INT8: per-head V scale
  int q_block;
  float c_log2;  // sm_scale * log2(e)
  void* out;
  int out_bf16;
};

using gptr = const __attribute__((address_space(1))) void*;
using lptr = __attribute__((address_space(3))) void*;

// Copy NCH 16-byte chunks global -> LDS.  The workgroup moves one round of
// NW * 64 chunks per step (one global_load_lds_dwordx4 per wave, 1 KiB);
// chunk p = 512 i + 64 wave + lane lands at lds + 16 p and comes from
// base + off(i), off being the lane's 32-bit byte offset in round i.
template <int NCH, int NW, class Off>
FAQ_DEV void stage(uint8_t* lds, const uint8_t* base, int wave, int lane, Off off) {
  // the tile base is a wave-uniform value held in SGPRs; hiding it from the
  // optimizer keeps it from turning every copy into a 64-bit per-lane
  // pointer carried across loop iterations
  asm volatile("" : "+s"(base));
  constexpr int ROUNDS = NCH / (NW * 64);
#pragma unroll
  for (int i = 0; i < ROUNDS; ++i) {
    const int grp = i * NW * 64 + wave * 64;
    __builtin_amdgcn_global_load_lds((gptr)(base + (uint32_t)off(i)), (lptr)(lds + grp * 16), 16, 0, 0);
  }
  constexpr int REM = NCH - ROUNDS * NW * 64;  // < one round: the first waves take it
  if (REM > 0) {
    const int grp = ROUNDS * NW * 64 + wave * 64;
    if (grp < NCH) {
      if (REM % 64 == 0 || grp + lane < NCH)
        __builtin_amdgcn_global_load_lds((gptr)(base + (uint32_t)off(ROUNDS)), (lptr)(lds + grp * 16), 16, 0, 0);
    }
  }
}

// KVC (FP8 only): the K and V scales are constant over each 128-key tile
// (token blocks of a multiple of 128 keys), so the K scale folds into the
// query's exponent factor and every w_j is 1.
template <int MODE, int D, bool CAUSAL, bool KVC>
__global__ __launch_bounds__(Waves<MODE>::NTHR, Waves<MODE>::WG_PER_CU) void k_attn(const KParams p) {
  constexpr int NW = Waves<MODE>::NW;
  constexpr int BM = Waves<MODE>::BM;
  constexpr int RB = NW * 64 * 16;  // bytes one staging round moves
  using G = Geo<MODE, D>;
  constexpr int DB = D / 16;  // 16-channel output blocks
  constexpr int NB = D / 32;  // MX blocks per row
  constexpr int KK = D / 32;  // bf16 MFMA steps over D
  // two tile buffers as separate objects: with the loop unrolled by two
  // every LDS read names one of them statically, so the compiler knows it
  // does not alias the copy in flight into the other and need not wait
  __shared__ __attribute__((aligned(1024))) uint8_t buf0[G::BUF];
  __shared__ __attribute__((aligned(1024))) uint8_t buf1[G::BUF];

  const int tid = threadIdx.x, lane = tid & 63, l16 = lane & 15, g = lane >> 4;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  __builtin_assume(wave >= 0 && wave < NW);

  // ---- work item: (b,h) and query tile
  int64_t bh;
  int qt;
  {
    const int L = blockIdx.x, nqt = p.nqt;
    const int BH = (int)p.BH;
    if ((BH & 7) == 0) {
      const int xcd = L & 7, j = L >> 3, per = BH >> 3;
      if (CAUSAL) { qt = nqt - 1 - j / per; bh = xcd + 8 * (j % per); }
      else { bh = xcd + 8 * (j / nqt); qt = j % nqt; }
    } else {
      if (CAUSAL) { qt = nqt - 1 - L / BH; bh = L % BH; }
      else { bh = L / nqt; qt = L % nqt; }
    }
  }
  const int64_t h = bh % p.H;
  const int Sq = (int)p.Sq, Skv = (int)p.Skv, nt = (int)p.nt;
  const int qw = qt * BM + wave * 32;  // this wave's first query
  // last tile this wave computes: its diagonal tile under causal masking
  // (none when its queries are all past the end); every tile otherwise
  // (rows past the end are computed on row 0's data and never stored)
  const int wdiag = CAUSAL ? (qw < Sq ? qw / BN : -1) : INT_MAX;
  const uint8_t* kbase = p.k + (MODE == ATTN_FP8 ? bh * nt * (int64_t)BN : bh * (int64_t)Skv) * G::KROW;
  const uint8_t* vtbase = p.vt + bh * nt * (int64_t)G::VBYTES;
  const uint8_t* auxbase = p.aux + bh * nt * (int64_t)G::XBYTES;

  // ---- Q operands and per-query factors
  bf16x8 qw8[2][KK];  // FP8: the bf16 images of the E4M3 codes per bf16 MFMA step
  i32x4 qi8[2][2];    // INT8: 16 bytes per lane per 64-wide step
  i32x4 qmx[2];       // MXFP4: 32 E2M1 per lane
  int qsc[2];
  float cq[2];
#pragma unroll
  for (int qb = 0; qb < 2; ++qb) {
    const int qi = qw + qb * 16 + l16;
    const bool ok = qi < Sq;
    const uint8_t* qrow = p.q + (bh * p.Sq + (ok ? qi : 0)) * (MODE == ATTN_MX ? D / 2 : D);
    if (MODE == ATTN_FP8) {
#pragma unroll
      for (int kk = 0; kk < KK; ++kk) {
        uint2 a = make_uint2(0, 0);
        if (ok) a = *reinterpret_cast<const uint2*>(qrow + 32 * kk + 8 * g);
        qw8[qb][kk] = __builtin_bit_cast(bf16x8, i32x4{(int)e4m3x2_to_bf16x2<false>(a.x), (int)e4m3x2_to_bf16x2<true>(a.x),
                                                       (int)e4m3x2_to_bf16x2<false>(a.y), (int)e4m3x2_to_bf16x2<true>(a.y)});
      }
      const float* qs = reinterpret_cast<const float*>(p.qs);
      const int64_t nqs = (p.Sq + p.q_block - 1) / p.q_block;
      cq[qb] = (ok ? qs[bh * nqs + qi / p.q_block] : 1.0f) * p.c_log2;
    } else if (MODE == ATTN_INT8) {
#pragma unroll
      for (int kk = 0; kk < 2; ++kk) {
        i32x4 v = {0, 0, 0, 0};
        if (ok && 64 * kk < D) {
          const uint4 a = *reinterpret_cast<const uint4*>(qrow + 64 * kk + 16 * g);
          v = i32x4{(int)a.x, (int)a.y, (int)a.z, (int)a.w};
        }
        qi8[qb][kk] = v;
      }
      const float* qs = reinterpret_cast<const float*>(p.qs);
      const float* ks = reinterpret_cast<const float*>(p.ks);
      cq[qb] = qs[h] * ks[h] * p.c_log2;
    } else {
      i32x4 v = {0, 0, 0, 0};
      int sc = 127;
      if (ok && 32 * g < D) {
        const uint4 a = *reinterpret_cast<const uint4*>(qrow + 16 * g);
        v = i32x4{(int)a.x, (int)a.y, (int)a.z, (int)a.w};
        sc = reinterpret_cast<const uint8_t*>(p.qs)[(bh * p.Sq + qi) * NB + g];
      }
      qmx[qb] = v;
      qsc[qb] = sc;
      cq[qb] = p.c_log2;
    }
  }

  // ---- tile copy into LDS buffer `buf`.  A lane's chunk in round i is
  // row i * (NW * 64 / CH) + r0, column c0 of the tile: the same swizzled
  // column every round, RB bytes further on.
  const int pw = wave * 64 + lane;
  const int kr0 = pw / G::KCH;
  const uint32_t koff0 = (uint32_t)(((pw % G::KCH) ^ G::kswz(kr0)) << 4);
  const uint32_t voff0 = (uint32_t)((pw / G::VCH) * G::VROW + (((pw % G::VCH) ^ G::vswz(pw / G::VCH)) << 4));
  auto issue = [&](int t, uint8_t* buf) {
    const int k0 = t * BN;
    if (MODE == ATTN_FP8) {
      // bf16 K tiles in the workspace, padded with zero rows
      stage<G::KBYTES / 16, NW>(buf, kbase + (int64_t)k0 * G::KROW, wave, lane,
                            [&](int i) { return (uint32_t)(i * RB + kr0 * G::KROW) + koff0; });
    } else {
      // K codes: rows past the end are re-read from the last row (masked)
      stage<G::KBYTES / 16, NW>(buf, kbase, wave, lane, [&](int i) {
        const int kr = min(k0 + i * (NW * 64 / G::KCH) + kr0, Skv - 1);
        return (uint32_t)(kr * G::KROW) + koff0;
      });
    }
    stage<G::VBYTES / 16, NW>(buf + G::VOFF, vtbase + (int64_t)t * G::VBYTES, wave, lane,
                          [&](int i) { return (uint32_t)(i * RB) + voff0; });
    if (MODE != ATTN_INT8)
      stage<G::XBYTES / 16, NW>(buf + G::XOFF, auxbase + (int64_t)t * G::XBYTES, wave, lane,
                            [&](int i) { return (uint32_t)(i * RB + pw * 16); });
  };

  // Row state.  O holds the output of each row relative to a reference
  // factor fref: the true accumulator is O * fref (INT8 keeps fref = 1 and
  // folds its per-tile factor in with an fma; the bf16-MFMA modes rescale O
  // once per tile and let the PV MFMA accumulate straight into it).
  float M[2] = {-INFINITY, -INFINITY}, L[2] = {0.f, 0.f}, fref[2] = {1.f, 1.f};
  f32x4 O[2][DB];
#pragma unroll
  for (int qb = 0; qb < 2; ++qb)
#pragma unroll
    for (int db = 0; db < DB; ++db) O[qb][db] = f32x4{0.f, 0.f, 0.f, 0.f};

  const int qlast = min(Sq, (qt + 1) * BM) - 1;
  const int t_end = CAUSAL ? min(nt, qlast / BN + 1) : nt;
  const float vscale_i8 = (MODE == ATTN_INT8) ? p.vs_head[h] * (1.0f / 127.0f) : 1.0f;

  auto step = [&](int t, const uint8_t* cur, uint8_t* nxt) __attribute__((always_inline)) {
    const int k0 = t * BN;
    // this wave's copies of tile t have landed; the barrier makes every
    // wave's copies visible and retires all reads of the other buffer
    __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0)
    __syncthreads();
    if (t + 1 < t_end) issue(t + 1, nxt);
    if (t > wdiag) return;
    // the ragged last tile and the causal diagonal need a per-key validity
    // test; the other tiles skip it (uniform branch)
    const bool masked = (k0 + BN > Skv) || (CAUSAL && t == wdiag);
    const uint8_t* Kt = cur;
    const uint8_t* Vl = cur + G::VOFF;
    const float* Xt = reinterpret_cast<const float*>(cur + G::XOFF);

    // One query block at a time: scores, tile max, probabilities and the
    // quantized P operand of block qb, so only one block's scores are held
    // in registers (the K operands are read once per query block).
    i32x4 pi8[2][2];   // INT8: rne(127 p) bytes, keys in vt_key_int8 order
    i32x4 pbf[2][4];   // FP8 / MXFP4: bf16 images of the quantized p, per step kk
    float rscale[2], bvi8[2];
    bool rescale_any = false;
#pragma unroll
    for (int qb = 0; qb < 2; ++qb) {
      // The two query blocks read the same K operands and per-key factors;
      // an opaque zero offset keeps the compiler from reusing the first
      // block's reads (which would hold them all in registers) - LDS reads
      // are cheap, registers are not.
      int zq = 0;
      asm volatile("" : "+v"(zq));
      const uint8_t* Kl = Kt + zq;
      const float* Xf = Xt + zq;
      const uint8_t* Xb = reinterpret_cast<const uint8_t*>(Xt) + zq;
      // ---- S^T = K Q^T: score of (query qb*16 + l16, key of block b at
      // output row 4g + r).  Operands of block b+1 are read from LDS while
      // block b multiplies, and the VALU work on block b-1 fills the MFMA
      // shadow; a scheduling fence closes each step, which bounds the
      // registers held by operands in flight.
      f32x4 s[8];
      int mi = INT_MIN;
      if (MODE == ATTN_FP8) {
        bf16x8 kop[1][KK];
        auto kload = [&](int bb, bf16x8 (&dst)[KK]) {
#pragma unroll
          for (int kk = 0; kk < KK; ++kk)
            dst[kk] = *reinterpret_cast<const bf16x8*>(&Kl[(16 * bb + l16) * G::KROW + (((4 * kk + g) ^ G::kswz(l16)) << 4)]);
        };
        auto kscale = [&](int bb) {
          const float4 skv = *reinterpret_cast<const float4*>(&Xf[16 * bb + 4 * g]);
          s[bb][0] *= skv.x; s[bb][1] *= skv.y; s[bb][2] *= skv.z; s[bb][3] *= skv.w;
        };
        // (one block of K operands in flight: 16 registers each)
#pragma unroll
        for (int bb = 0; bb < 8; ++bb) {
          kload(bb, kop[0]);
          s[bb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kop[0][0], qw8[qb][0], f32x4{0.f, 0.f, 0.f, 0.f}, 0, 0, 0);
#pragma unroll
          for (int kk = 1; kk < KK; ++kk)
            s[bb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kop[0][kk], qw8[qb][kk], s[bb], 0, 0, 0);
          if (!KVC && bb > 0) kscale(bb - 1);
          __builtin_amdgcn_sched_barrier(0);
        }
        if (!KVC) kscale(7);
      } else if (MODE == ATTN_INT8) {
        constexpr int K8 = D / 64;
        constexpr int PD = 3;  // K operand blocks in flight
        i32x4 kop[PD + 1][K8];
        i32x4 si[2];
        auto kload = [&](int bb, i32x4 (&dst)[K8]) {
#pragma unroll
          for (int kk = 0; kk < K8; ++kk) {
            const uint4 v = *reinterpret_cast<const uint4*>(&Kl[(16 * bb + l16) * G::KROW + (((4 * kk + g) ^ G::kswz(l16)) << 4)]);
            dst[kk] = i32x4{(int)v.x, (int)v.y, (int)v.z, (int)v.w};
          }
        };
        // exact int32 scores (|s| < 2^21): the float conversion is exact
        auto post = [&](int bb) {
          const i32x4 v = si[bb & 1];
          if (!masked) mi = max(mi, max(max(v[0], v[1]), max(v[2], v[3])));
          s[bb] = f32x4{(float)v[0], (float)v[1], (float)v[2], (float)v[3]};
        };
#pragma unroll
        for (int bb = 0; bb < PD; ++bb) kload(bb, kop[bb]);
#pragma unroll
        for (int bb = 0; bb < 8; ++bb) {
          if (bb + PD < 8) kload(bb + PD, kop[(bb + PD) % (PD + 1)]);
          const int ko = bb % (PD + 1);
          si[bb & 1] = __builtin_amdgcn_mfma_i32_16x16x64_i8(kop[ko][0], qi8[qb][0], i32x4{0, 0, 0, 0}, 0, 0, 0);
#pragma unroll
          for (int kk = 1; kk < K8; ++kk)
            si[bb & 1] = __builtin_amdgcn_mfma_i32_16x16x64_i8(kop[ko][kk], qi8[qb][kk], si[bb & 1], 0, 0, 0);
          if (bb > 0) post(bb - 1);
          __builtin_amdgcn_sched_barrier(0);
        }
        post(7);
      } else {
        i32x8 kop[2];
        int ksc[2];
        auto kload = [&](int bb, i32x8& dst, int& sc) {
          const int row = k_row_mx(bb, l16);
          dst = i32x8{0, 0, 0, 0, 0, 0, 0, 0};
          sc = 127;
          if (32 * g < D) {
            const uint4 v = *reinterpret_cast<const uint4*>(&Kl[row * G::KROW + ((g ^ G::kswz(row)) << 4)]);
            dst = i32x8{(int)v.x, (int)v.y, (int)v.z, (int)v.w, 0, 0, 0, 0};
            sc = Xb[row * NB + g];
          }
        };
        const i32x4 qv = qmx[qb];
        const i32x8 qop = {qv[0], qv[1], qv[2], qv[3], 0, 0, 0, 0};
        kload(0, kop[0], ksc[0]);
#pragma unroll
        for (int bb = 0; bb < 8; ++bb) {
          if (bb + 1 < 8) kload(bb + 1, kop[(bb + 1) & 1], ksc[(bb + 1) & 1]);
          s[bb] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(kop[bb & 1], qop, f32x4{0.f, 0.f, 0.f, 0.f},
                                                                   4, 4, 0, ksc[bb & 1], 0, qsc[qb]);
          __builtin_amdgcn_sched_barrier(0);
        }
      }

      if (masked) {
        // key kl of the tile is valid when kl < lim; the lane's own part of
        // kl is folded into the limit so the rest is an immediate
        const int qi = qw + qb * 16 + l16;
        const int lim = (CAUSAL ? min(Skv, qi + 1) : Skv) - k0;
        const int rel = lim - (MODE == ATTN_MX ? 32 * g : 4 * g);
#pragma unroll
        for (int bb = 0; bb < 8; ++bb)
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            const int kc = (MODE == ATTN_MX) ? (4 * bb + r) : (16 * bb + r);
            s[bb][r] = (kc < rel) ? s[bb][r] : -INFINITY;
          }
      }

      // ---- tile max, then the row combination factors: a rescales what
      // was accumulated so far, bt weights this tile
      float m;
      if (MODE == ATTN_INT8 && !masked) {
        m = (float)mi;
      } else {
        m = -INFINITY;
#pragma unroll
        for (int bb = 0; bb < 8; ++bb) m = fmaxf(fmaxf(m, fmaxf(s[bb][0], s[bb][1])), fmaxf(s[bb][2], s[bb][3]));
      }
      const float mlane = m;  // max over this lane's keys (MXFP4: its 32-key group)
      m = rows4_max(m);
      // exponent factor of this row and tile: scores times ce are log2 units
      const float ce = (MODE == ATTN_FP8 && KVC) ? cq[qb] * Xf[0] : cq[qb];
      const float ml = m * ce;  // tile max, log2 units (M is kept in these units)
      float Mn, a;
      if (MODE == ATTN_INT8) {
        // lazy reference: keep the running reference unless this tile's max
        // exceeds it by more than 2^8 (tile weights stay <= 2^8, far from
        // overflow), so O is rescaled only when the max jumps
        const bool jump = ml > M[qb] + 8.0f;
        Mn = jump ? ml : M[qb];
        a = jump ? __builtin_amdgcn_exp2f(M[qb] - ml) : 1.0f;
      } else {
        Mn = fmaxf(M[qb], ml);
        a = __builtin_amdgcn_exp2f(M[qb] - Mn);
      }
      const float bt = (m == -INFINITY) ? 0.0f : __builtin_amdgcn_exp2f(ml - Mn);
      M[qb] = Mn;
      // bf16-MFMA modes: new reference factor f = bt (times sigma_t / 448
      // for FP8); a row whose tile is negligible (bt < 2^-64) keeps its
      // reference and contributes nothing, which keeps O bounded.
      bool live = true;
      if (MODE == ATTN_INT8) {
        rscale[qb] = a;
        bvi8[qb] = bt * vscale_i8;
      } else {
        float ft = bt;
        if (MODE == ATTN_FP8) ft *= p.sig[bh * nt + t] * (1.0f / 448.0f);
        live = bt >= 0x1p-64f;
        rscale[qb] = live ? (fref[qb] * a / ft) : a;
        fref[qb] = live ? ft : fref[qb];
      }
      rescale_any |= (rscale[qb] != 1.0f);

      // ---- probabilities, tile sum and the quantized P operand.  A row
      // that is not live takes +inf as its reference, so all its p are 0.
      // INT8 and KVC fold the static P scale into the exponent (127 p and
      // 448 p come out of the exp); their sums are scaled back once.
      const float ms = (m == -INFINITY) ? 0.0f : (live ? m : INFINITY);
      constexpr float kLog2_127 = 6.9886846867721655f, kLog2_448 = 8.807354922057604f;
      const float mc = ms * ce - kLog2_127;
      float ls[2] = {0.f, 0.f};
#pragma unroll
      for (int bb = 0; bb < 8; ++bb) {
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          float pv;
          if (MODE == ATTN_INT8) {
            // 127 p = 2^(s ce - (m ce - log2 127)); at the maximum this may
            // differ from 127 by an ulp, which cannot move rne(127 p)
            pv = __builtin_amdgcn_exp2f(__builtin_fmaf(s[bb][r], ce, -mc));
          } else if (MODE == ATTN_FP8 && KVC) {
            // 448 p (w = 1): at the maximum within an ulp of 448, whose code
            // both roundings give
            pv = __builtin_amdgcn_exp2f(__builtin_fmaf(s[bb][r] - ms, ce, kLog2_448));
          } else {
            // (x - m) is exactly 0 at the tile maximum, so p = 1 there exactly
            pv = __builtin_amdgcn_exp2f((s[bb][r] - ms) * ce);
          }
          s[bb][r] = pv;
          ls[r & 1] += pv;
        }
        if (MODE == ATTN_INT8) {
          // rne(127 p), saturated to [0, 255], packed byte by byte
          uint32_t w = __builtin_amdgcn_cvt_pk_u8_f32(s[bb][0], 0u, 0u);
          w = __builtin_amdgcn_cvt_pk_u8_f32(s[bb][1], 1u, w);
          w = __builtin_amdgcn_cvt_pk_u8_f32(s[bb][2], 2u, w);
          w = __builtin_amdgcn_cvt_pk_u8_f32(s[bb][3], 3u, w);
          pi8[qb][bb >> 2][bb & 3] = (int)w;
        } else if (MODE == ATTN_FP8) {
          // E4M3 of 448 p w_j (round to nearest even), then its exact bf16 image
          int e8;
          if (KVC) {
            e8 = __builtin_amdgcn_cvt_pk_fp8_f32(s[bb][0], s[bb][1], 0, false);
            e8 = __builtin_amdgcn_cvt_pk_fp8_f32(s[bb][2], s[bb][3], e8, true);
          } else {
            const float4 vm = *reinterpret_cast<const float4*>(&Xf[BN + 16 * bb + 4 * g]);
            e8 = __builtin_amdgcn_cvt_pk_fp8_f32(s[bb][0] * vm.x, s[bb][1] * vm.y, 0, false);
            e8 = __builtin_amdgcn_cvt_pk_fp8_f32(s[bb][2] * vm.z, s[bb][3] * vm.w, e8, true);
          }
          pbf[qb][bb >> 1][2 * (bb & 1)] = (int)e4m3x2_to_bf16x2<false>((uint32_t)e8);
          pbf[qb][bb >> 1][2 * (bb & 1) + 1] = (int)e4m3x2_to_bf16x2<true>((uint32_t)e8);
        }
      }
      if (MODE == ATTN_MX) {
        // this lane's 32 keys are one MX group: local max -> shared
        // exponent; p -> E2M1(p / 2^E) * 2^E, exact in bf16.  The group's
        // largest p is the same function of the lane's largest score.
        const float pmax = __builtin_amdgcn_exp2f((mlane - ms) * ce);
        const int E = mx_exponent(pmax);
        const float sc = E > -127 ? __uint_as_float((uint32_t)(E + 127) << 23) : 1.0f;
#pragma unroll
        for (int bb = 0; bb < 8; ++bb) {
#pragma unroll
          for (int hh = 0; hh < 2; ++hh) {
            const uint32_t f4 = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(0u, s[bb][2 * hh], s[bb][2 * hh + 1], sc, 0);
            const int v2 = (int)__builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(f4, sc, 0));
            pbf[qb][bb >> 1][2 * (bb & 1) + hh] = v2;
          }
        }
      }
      const float lscale = MODE == ATTN_INT8 ? 1.0f / 127.0f : ((MODE == ATTN_FP8 && KVC) ? 1.0f / 448.0f : 1.0f);
      L[qb] = L[qb] * a + rows4_sum(ls[0] + ls[1]) * (bt * lscale);
      __builtin_amdgcn_sched_barrier(0);
    }

    // ---- O^T += V^T P^T (per 16-channel block), V operands of block db+1
    // read while block db multiplies
    if (MODE == ATTN_INT8) {
      const bool do_rescale = __any(rescale_any);
      constexpr int PD = 3;  // V operand blocks in flight
      i32x4 vop[PD + 1][2], ci[2][2];
      auto vload = [&](int db, i32x4 (&dst)[2]) {
#pragma unroll
        for (int h2 = 0; h2 < 2; ++h2) {
          const uint4 v = *reinterpret_cast<const uint4*>(&Vl[(16 * db + l16) * G::VROW + (((2 * g + h2) ^ G::vswz(l16)) << 4)]);
          dst[h2] = i32x4{(int)v.x, (int)v.y, (int)v.z, (int)v.w};
        }
      };
      auto accum = [&](int db) {
#pragma unroll
        for (int qb = 0; qb < 2; ++qb)
#pragma unroll
          for (int r = 0; r < 4; ++r) O[qb][db][r] = __builtin_fmaf((float)ci[qb][db & 1][r], bvi8[qb], O[qb][db][r]);
      };
      // the running max moves rarely once a row has seen its largest
      // scores: rescale only when some row of the wave needs it
      if (do_rescale) {
#pragma unroll
        for (int qb = 0; qb < 2; ++qb)
#pragma unroll
          for (int db = 0; db < DB; ++db)
#pragma unroll
            for (int r = 0; r < 4; ++r) O[qb][db][r] *= rscale[qb];
      }
#pragma unroll
      for (int db = 0; db < PD && db < DB; ++db) vload(db, vop[db]);
#pragma unroll
      for (int db = 0; db < DB; ++db) {
        if (db + PD < DB) vload(db + PD, vop[(db + PD) % (PD + 1)]);
        const int vo = db % (PD + 1);
#pragma unroll
        for (int qb = 0; qb < 2; ++qb) {
          ci[qb][db & 1] = __builtin_amdgcn_mfma_i32_16x16x64_i8(vop[vo][0], pi8[qb][0], i32x4{0, 0, 0, 0}, 0, 0, 0);
          ci[qb][db & 1] = __builtin_amdgcn_mfma_i32_16x16x64_i8(vop[vo][1], pi8[qb][1], ci[qb][db & 1], 0, 0, 0);
        }
        if (db > 0) accum(db - 1);
        __builtin_amdgcn_sched_barrier(0);
      }
      accum(DB - 1);
    } else {
      bf16x8 vop[2][4];
      auto vload = [&](int db, bf16x8 (&dst)[4]) {
#pragma unroll
        for (int kk = 0; kk < 4; ++kk)
          dst[kk] = *reinterpret_cast<const bf16x8*>(&Vl[(16 * db + l16) * G::VROW + (((4 * kk + g) ^ G::vswz(l16)) << 4)]);
      };
      vload(0, vop[0]);
#pragma unroll
      for (int db = 0; db < DB; ++db) {
        if (db + 1 < DB) vload(db + 1, vop[(db + 1) & 1]);
        // the reference factor moves almost every tile: rescale unconditionally
#pragma unroll
        for (int qb = 0; qb < 2; ++qb)
#pragma unroll
          for (int r = 0; r < 4; ++r) O[qb][db][r] *= rscale[qb];
#pragma unroll
        for (int kk = 0; kk < 4; ++kk)
#pragma unroll
          for (int qb = 0; qb < 2; ++qb)
            O[qb][db] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(vop[db & 1][kk], __builtin_bit_cast(bf16x8, pbf[qb][kk]),
                                                                O[qb][db], 0, 0, 0);
        __builtin_amdgcn_sched_barrier(0);
      }
    }
  };

  issue(0, buf0);
#pragma clang loop unroll(disable)
  for (int t = 0; t < t_end; t += 2) {
    step(t, buf0, buf1);
    if (t + 1 < t_end) step(t + 1, buf1, buf0);
  }

  // ---- normalize, store
#pragma unroll
  for (int qb = 0; qb < 2; ++qb) {
    const int qi = qw + qb * 16 + l16;
    if (qi >= Sq) continue;
    const float inv = fref[qb] / L[qb];
#pragma unroll
    for (int db = 0; db < DB; ++db) {
      const int64_t off = (bh * p.Sq + qi) * D + 16 * db + 4 * g;
      const float o0 = O[qb][db][0] * inv, o1 = O[qb][db][1] * inv;
      const float o2 = O[qb][db][2] * inv, o3 = O[qb][db][3] * inv;
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

template <int MODE, int D>
hipError_t launch_mode_d(const AttnArgs& a, const WsLayout& l, hipStream_t st) {
  const int64_t nt = (a.Skv + BN - 1) / BN;
  uint8_t* ws = reinterpret_cast<uint8_t*>(a.ws);
  dim3 pgrid((unsigned)nt, (unsigned)(a.B * a.H));
  if (MODE == ATTN_MX) {
    k_prep_mx<D><<<pgrid, 256, 0, st>>>((const uint8_t*)a.v_codes, (const uint8_t*)a.v_scales,
                                        (const uint8_t*)a.k_scales, a.Skv, nt,
                                        reinterpret_cast<uint16_t*>(ws + l.vt_off), ws + l.aux_off);
  } else {
    k_prep<D, MODE == ATTN_FP8><<<pgrid, 256, 0, st>>>(
        (const uint8_t*)a.k_codes, (const float*)a.k_scales, (const uint8_t*)a.v_codes, (const float*)a.v_scales,
        a.Skv, a.kv_block, nt, ws + l.vt_off, reinterpret_cast<uint16_t*>(ws + l.kb_off),
        reinterpret_cast<float*>(ws + l.aux_off), reinterpret_cast<float*>(ws + l.sig_off));
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  KParams p{};
  p.H = a.H; p.BH = a.B * a.H; p.Sq = a.Sq; p.Skv = a.Skv; p.nt = nt;
  p.nqt = (int)((a.Sq + Waves<MODE>::BM - 1) / Waves<MODE>::BM);
  p.q = (const uint8_t*)a.q_codes; p.qs = a.q_scales;
  p.k = MODE == ATTN_FP8 ? ws + l.kb_off : (const uint8_t*)a.k_codes;
  p.ks = a.k_scales;
  p.vt = ws + l.vt_off;
  p.aux = ws + l.aux_off;
  p.sig = reinterpret_cast<const float*>(ws + l.sig_off);
  p.vs_head = (const float*)a.v_scales;
  p.q_block = a.q_block;
  p.c_log2 = a.sm_scale * kLog2e;
  p.out = a.out; p.out_bf16 = a.out_bf16;
  dim3 grid((unsigned)(p.nqt * p.BH));
  if constexpr (MODE == ATTN_FP8) {
    if (a.kv_block % BN == 0) {
      if (a.causal) k_attn<MODE, D, true, true><<<grid, Waves<MODE>::NTHR, 0, st>>>(p);
      else k_attn<MODE, D, false, true><<<grid, Waves<MODE>::NTHR, 0, st>>>(p);
      return hipGetLastError();
    }
  }
  {
    if (a.causal) k_attn<MODE, D, true, false><<<grid, Waves<MODE>::NTHR, 0, st>>>(p);
    else k_attn<MODE, D, false, false><<<grid, Waves<MODE>::NTHR, 0, st>>>(p);
  }
  return hipGetLastError();
}

}  // namespace

size_t attn_workspace_bytes(int mode, int64_t B, int64_t H, int64_t Skv, int64_t D) {
  return ws_layout(mode, B, H, Skv, D).total;
}

hipError_t launch_attention(const AttnArgs& a, hipStream_t st) {
  const WsLayout l = ws_layout(a.mode, a.B, a.H, a.Skv, a.D);
  switch (a.mode) {
    case ATTN_INT8: return a.D == 128 ? launch_mode_d<ATTN_INT8, 128>(a, l, st) : launch_mode_d<ATTN_INT8, 64>(a, l, st);
    case ATTN_FP8: return a.D == 128 ? launch_mode_d<ATTN_FP8, 128>(a, l, st) : launch_mode_d<ATTN_FP8, 64>(a, l, st);
    default: return a.D == 128 ? launch_mode_d<ATTN_MX, 128>(a, l, st) : launch_mode_d<ATTN_MX, 64>(a, l, st);
  }
}

}  // namespace faq
