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
// Kernel shape: one workgroup = 4 waves = 128 queries of one (b,h); each
// wave owns 32 queries as two 16-query MFMA column blocks.  Scores are
// computed transposed (S^T = K Q^T), so a lane holds one query and a run of
// keys: the row max needs only two cross-lane steps, and the lane's
// probabilities are already the B operand of O^T = V^T P^T.  K is staged in
// LDS row-major (XOR-swizzled 16-byte chunks; FP8 codes widened to bf16 on
// the way); V comes from the workspace already transposed per 128-key tile,
// with its keys permuted to match the order in which a lane holds its
// probabilities.

#include <climits>

#include "common.h"
#include "launch.h"

namespace faq {
namespace {

constexpr int BM = 128;  // queries per workgroup
constexpr int BN = 128;  // keys per tile = probability tile
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

template <bool B>
struct BoolC {
  static constexpr bool value = B;
};

// Row of the K tile read by lane-row i of MFMA block b in the MXFP4 kernel.
FAQ_DEV int k_row_mx(int b, int i) { return 32 * (i >> 2) + 4 * b + (i & 3); }

// XOR swizzles of 16-byte chunks (bank spreading for the operand reads).
FAQ_DEV int swz8(int row) { return (row ^ (row >> 3)) & 7; }
FAQ_DEV int swz4(int row) { return (row ^ (row >> 3)) & 3; }
FAQ_DEV int swz_mx(int row) {
  return ((((row >> 1) & 1) | (((row >> 5) & 1) << 1)) ^ ((row >> 5) & 3)) & 3;
}
// bf16 rows: 16 rows read together hit 16 distinct chunks of a 256-byte row
FAQ_DEV int swz_bf(int row, int nch) { return row & (nch - 1); }

// Two E4M3 bytes (the low half-word of `w`, or the high one when HI) -> two
// bf16, exactly.
template <bool HI>
FAQ_DEV uint32_t e4m3x2_to_bf16x2(uint32_t w) {
  return __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8((int)w, 1.0f, HI));
}

// ------------------------------------------------------------------------
// Workspace layout (per (b,h), per 128-key tile t):
//   vt  : V^T of the tile, D rows x 128 keys: INT8 / E4M3 codes (1 byte) or,
//         for MXFP4, the exactly dequantized values in bf16 (2 bytes)
//   aux : FP8 only: 128 floats 448 * w_j = 448 * s_v,j / sigma_t
//   sig : FP8 only: sigma_t = max over the tile's keys of s_v,j
// ------------------------------------------------------------------------
struct WsLayout {
  size_t vt_off, aux_off, sig_off, total;
};

inline WsLayout ws_layout(int mode, int64_t B, int64_t H, int64_t Skv, int64_t D) {
  const int64_t nt = (Skv + BN - 1) / BN;
  const int64_t tiles = B * H * nt;
  auto up = [](size_t x) { return (x + 255) & ~size_t(255); };
  const size_t vbytes = (mode == ATTN_MX) ? 2 : 1;
  WsLayout l{};
  l.vt_off = 0;
  l.aux_off = up((size_t)tiles * D * BN * vbytes);
  const size_t aux = (mode == ATTN_FP8) ? (size_t)tiles * BN * 4 : 0;
  const size_t sig = (mode == ATTN_FP8) ? (size_t)tiles * 4 : 0;
  l.sig_off = l.aux_off + up(aux);
  l.total = l.sig_off + up(sig);
  return l;
}

// ------------------------------------------------------------------------
// V re-layout, INT8 / FP8 (1-byte codes): V^T per tile in the lane key
// order; FP8 also gets sigma_t and the per-key multipliers 448 * w_j.
// grid = (tiles, B*H), 256 threads.
// ------------------------------------------------------------------------
template <int D, bool FP8>
__global__ __launch_bounds__(256) void k_prep_v(const uint8_t* __restrict__ v, const float* __restrict__ vs,
                                                int64_t Skv, int kv_block, int64_t nt,
                                                uint8_t* __restrict__ vt, float* __restrict__ vmul,
                                                float* __restrict__ sig) {
  __shared__ uint8_t tile[BN][D + 4];
  __shared__ float red[4];
  const int t = blockIdx.x;
  const int64_t bh = blockIdx.y;
  const int64_t k0 = (int64_t)t * BN;
  const uint8_t* src = v + (bh * Skv + k0) * D;
  constexpr int CPR = D / 16;  // 16-byte chunks per key row
  for (int c = threadIdx.x; c < BN * CPR; c += 256) {
    const int kl = c / CPR, cc = c % CPR;
    uint4 val = make_uint4(0, 0, 0, 0);
    if (k0 + kl < Skv) val = *reinterpret_cast<const uint4*>(src + (int64_t)kl * D + cc * 16);
    uint32_t* dst = reinterpret_cast<uint32_t*>(&tile[kl][cc * 16]);
    dst[0] = val.x; dst[1] = val.y; dst[2] = val.z; dst[3] = val.w;
  }
  __syncthreads();
  uint8_t* out = vt + ((bh * nt) + t) * (int64_t)D * BN;
  for (int c = threadIdx.x; c < D * (BN / 16); c += 256) {
    const int d = c / (BN / 16), j = c % (BN / 16);
    uint32_t w[4];
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      uint32_t acc = 0;
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int col = 16 * j + 4 * q + r;
        const int key = FP8 ? vt_key_fp8(col) : vt_key_int8(col);
        acc |= (uint32_t)tile[key][d] << (8 * r);
      }
      w[q] = acc;
    }
    *reinterpret_cast<uint4*>(out + (int64_t)d * BN + 16 * j) = make_uint4(w[0], w[1], w[2], w[3]);
  }
  if (FP8) {
    const int kl = threadIdx.x;
    float s = 0.0f;
    if (kl < BN && k0 + kl < Skv) s = vs[bh * ((Skv + kv_block - 1) / kv_block) + (k0 + kl) / kv_block];
    float m = wave_max(s);
    if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = m;
    __syncthreads();
    m = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
    if (kl < BN) vmul[(bh * nt + t) * BN + kl] = (s > 0.0f) ? 448.0f * (s / m) : 0.0f;
    if (threadIdx.x == 0) sig[bh * nt + t] = m;
  }
}

// ------------------------------------------------------------------------
// V re-layout, MXFP4: V^T per tile as the exact bf16 values E2M1 * 2^E
// (E from the token's 32-channel block), in the lane key order.
// ------------------------------------------------------------------------
template <int D>
__global__ __launch_bounds__(256) void k_prep_v_mx(const uint8_t* __restrict__ v,
                                                   const uint8_t* __restrict__ ve, int64_t Skv,
                                                   int64_t nt, uint16_t* __restrict__ vt) {
  constexpr int NB = D / 32;
  __shared__ uint8_t codes[BN][D / 2 + 4];
  __shared__ uint8_t ex[BN][NB];
  const int t = blockIdx.x;
  const int64_t bh = blockIdx.y;
  const int64_t k0 = (int64_t)t * BN;
  for (int c = threadIdx.x; c < BN * (D / 32); c += 256) {
    const int kl = c / (D / 32), cc = c % (D / 32);  // 16-byte chunks of the packed row
    uint4 val = make_uint4(0, 0, 0, 0);
    if (k0 + kl < Skv) val = *reinterpret_cast<const uint4*>(v + (bh * Skv + k0 + kl) * (D / 2) + cc * 16);
    uint32_t* dst = reinterpret_cast<uint32_t*>(&codes[kl][cc * 16]);
    dst[0] = val.x; dst[1] = val.y; dst[2] = val.z; dst[3] = val.w;
  }
  for (int c = threadIdx.x; c < BN * NB; c += 256) {
    const int kl = c / NB, b = c % NB;
    ex[kl][b] = (k0 + kl < Skv) ? ve[(bh * Skv + k0 + kl) * NB + b] : (uint8_t)127;
  }
  __syncthreads();
  uint16_t* out = vt + ((bh * nt) + t) * (int64_t)D * BN;
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
  int64_t H, Sq, Skv, nt;
  const uint8_t* q;
  const void* qs;
  const uint8_t* k;
  const void* ks;
  const uint8_t* vt;
  const float* vmul;
  const float* sig;
  const float* vs_head;  // INT8: per-head V scale
  int q_block, kv_block;
  float c_log2;  // sm_scale * log2(e)
  void* out;
  int out_bf16;
};

// Raw bytes of one K/V tile (plus its per-key scale data) held in registers
// between the prefetch issued before a tile's compute and the commit to LDS
// at the start of the next one, so global-memory latency overlaps compute.
template <int MODE, int D>
struct TileRegs {
  static constexpr int KSRC = (MODE == ATTN_MX) ? D / 2 : D;             // K bytes per key row
  static constexpr int VSRC = (MODE == ATTN_MX) ? 2 * BN : BN;            // V^T bytes per channel row
  static constexpr int NK = BN * KSRC / 16 / 256;                         // 16-byte chunks per thread
  static constexpr int NV = D * VSRC / 16 / 256;
  uint4 k[NK];
  uint4 v[NV];
  float sc;       // FP8: K scale of key tid (tid < 128) or 448 w of key tid-128
  uint32_t kex;   // MXFP4: 2 K exponent bytes
};

template <int MODE, int D, bool CAUSAL>
__global__ __launch_bounds__(256, 2) void k_attn(const KParams p) {
  // K tile in LDS: INT8 codes (D bytes/row), FP8 widened to bf16 (2D bytes),
  // MXFP4 packed E2M1 (D/2 bytes)
  constexpr int KB = (MODE == ATTN_MX) ? D / 2 : (MODE == ATTN_FP8 ? 2 * D : D);
  constexpr int KCH = KB / 16;                           // 16-byte chunks per K row
  constexpr int VB = (MODE == ATTN_INT8) ? BN : 2 * BN;  // bytes per V^T row in LDS
  constexpr int VCH = VB / 16;
  constexpr int DB = D / 16;  // 16-channel output blocks
  constexpr int NB = D / 32;  // MX blocks per row
  constexpr int KK = D / 32;  // bf16 MFMA steps over D
  using TR = TileRegs<MODE, D>;
  constexpr int KSCH = TR::KSRC / 16;  // source chunks per K row
  constexpr int VSCH = TR::VSRC / 16;  // source chunks per V^T row
  __shared__ __attribute__((aligned(16))) uint8_t k_lds[BN * KB];
  __shared__ __attribute__((aligned(16))) uint8_t v_lds[D * VB];
  __shared__ __attribute__((aligned(16))) float sk_lds[BN];
  __shared__ __attribute__((aligned(16))) float vm_lds[BN];
  __shared__ __attribute__((aligned(4))) uint8_t kex_lds[BN * NB];

  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63, l16 = lane & 15, g = lane >> 4;
  const int64_t bh = blockIdx.y;
  const int64_t h = bh % p.H;
  const int nqt = (int)((p.Sq + BM - 1) / BM);
  const int qt = CAUSAL ? (nqt - 1 - (int)blockIdx.x) : (int)blockIdx.x;
  const int qbase = qt * BM + wave * 32;
  const int Skv = (int)p.Skv;
  const uint8_t* kbase = p.k + bh * p.Skv * TR::KSRC;
  const uint8_t* vtbase = p.vt + bh * p.nt * (int64_t)D * TR::VSRC;

  // ---- Q operands and per-query factors
  uint2 q8[2][KK];   // FP8: the E4M3 bytes of each bf16 MFMA step (widened per step)
  i32x4 qi8[2][2];   // INT8: 16 bytes per lane per 64-wide step
  i32x4 qmx[2];      // MXFP4: 32 E2M1 per lane
  int qsc[2];
  float cq[2];
#pragma unroll
  for (int qb = 0; qb < 2; ++qb) {
    const int qi = qbase + qb * 16 + l16;
    const bool ok = qi < p.Sq;
    const uint8_t* qrow = p.q + (bh * p.Sq + (ok ? qi : 0)) * TR::KSRC;
    if (MODE == ATTN_FP8) {
#pragma unroll
      for (int kk = 0; kk < KK; ++kk) {
        uint2 a = make_uint2(0, 0);
        if (ok) a = *reinterpret_cast<const uint2*>(qrow + 32 * kk + 8 * g);
        q8[qb][kk] = a;
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

  // ---- tile prefetch (registers) and commit (LDS)
  auto prefetch = [&](int t, TR& r) {
    const int k0 = t * BN;
#pragma unroll
    for (int i = 0; i < TR::NK; ++i) {
      const int c = i * 256 + tid, row = c / KSCH, cc = c % KSCH;
      r.k[i] = make_uint4(0, 0, 0, 0);
      if (k0 + row < Skv) r.k[i] = *reinterpret_cast<const uint4*>(kbase + (int64_t)(k0 + row) * TR::KSRC + cc * 16);
    }
    const uint8_t* vsrc = vtbase + (int64_t)t * D * TR::VSRC;
#pragma unroll
    for (int i = 0; i < TR::NV; ++i) {
      const int c = i * 256 + tid;
      r.v[i] = *reinterpret_cast<const uint4*>(vsrc + c * 16);
    }
    if (MODE == ATTN_FP8) {
      if (tid < BN) {
        const float* ks = reinterpret_cast<const float*>(p.ks);
        const int64_t nks = (p.Skv + p.kv_block - 1) / p.kv_block;
        r.sc = (k0 + tid < Skv) ? ks[bh * nks + (k0 + tid) / p.kv_block] : 0.0f;
      } else {
        r.sc = p.vmul[(bh * p.nt + t) * BN + (tid - BN)];
      }
    }
    if (MODE == ATTN_MX) {
      // 2 exponent bytes per thread (BN * NB <= 512)
      const uint8_t* kes = reinterpret_cast<const uint8_t*>(p.ks);
      uint32_t w = 0x7f7fu;
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        const int c = 2 * tid + j;
        if (c < BN * NB && k0 + c / NB < Skv) w = (w & ~(0xffu << (8 * j))) | ((uint32_t)kes[(bh * p.Skv + k0) * NB + c] << (8 * j));
      }
      r.kex = w;
    }
  };
  auto commit = [&](const TR& r) {
#pragma unroll
    for (int i = 0; i < TR::NK; ++i) {
      const int c = i * 256 + tid, row = c / KSCH, cc = c % KSCH;
      const uint4 val = r.k[i];
      if (MODE == ATTN_FP8) {
        const int sw = swz_bf(row, KCH);
        const uint4 lo = make_uint4(e4m3x2_to_bf16x2<false>(val.x), e4m3x2_to_bf16x2<true>(val.x),
                                    e4m3x2_to_bf16x2<false>(val.y), e4m3x2_to_bf16x2<true>(val.y));
        const uint4 hi = make_uint4(e4m3x2_to_bf16x2<false>(val.z), e4m3x2_to_bf16x2<true>(val.z),
                                    e4m3x2_to_bf16x2<false>(val.w), e4m3x2_to_bf16x2<true>(val.w));
        *reinterpret_cast<uint4*>(&k_lds[row * KB + (((2 * cc) ^ sw) * 16)]) = lo;
        *reinterpret_cast<uint4*>(&k_lds[row * KB + (((2 * cc + 1) ^ sw) * 16)]) = hi;
      } else {
        const int sw = (MODE == ATTN_MX) ? (KCH == 4 ? swz_mx(row) : 0) : (KCH == 8 ? swz8(row) : swz4(row));
        *reinterpret_cast<uint4*>(&k_lds[row * KB + ((cc ^ sw) * 16)]) = val;
      }
    }
#pragma unroll
    for (int i = 0; i < TR::NV; ++i) {
      const int c = i * 256 + tid, row = c / VSCH, cc = c % VSCH;
      const uint4 val = r.v[i];
      if (MODE == ATTN_INT8) {
        *reinterpret_cast<uint4*>(&v_lds[row * VB + ((cc ^ swz8(row)) * 16)]) = val;
      } else if (MODE == ATTN_FP8) {
        const int sw = swz_bf(row, VCH);
        const uint4 lo = make_uint4(e4m3x2_to_bf16x2<false>(val.x), e4m3x2_to_bf16x2<true>(val.x),
                                    e4m3x2_to_bf16x2<false>(val.y), e4m3x2_to_bf16x2<true>(val.y));
        const uint4 hi = make_uint4(e4m3x2_to_bf16x2<false>(val.z), e4m3x2_to_bf16x2<true>(val.z),
                                    e4m3x2_to_bf16x2<false>(val.w), e4m3x2_to_bf16x2<true>(val.w));
        *reinterpret_cast<uint4*>(&v_lds[row * VB + (((2 * cc) ^ sw) * 16)]) = lo;
        *reinterpret_cast<uint4*>(&v_lds[row * VB + (((2 * cc + 1) ^ sw) * 16)]) = hi;
      } else {
        *reinterpret_cast<uint4*>(&v_lds[row * VB + ((cc ^ swz_bf(row, VCH)) * 16)]) = val;
      }
    }
    if (MODE == ATTN_FP8) {
      if (tid < BN) sk_lds[tid] = r.sc;
      else vm_lds[tid - BN] = r.sc;
    }
    if (MODE == ATTN_MX) {
      if (2 * tid < BN * NB) *reinterpret_cast<uint16_t*>(&kex_lds[2 * tid]) = (uint16_t)r.kex;
    }
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

  const int t_end = CAUSAL ? (qt + 1 < (int)p.nt ? qt + 1 : (int)p.nt) : (int)p.nt;
  const float vscale_i8 = (MODE == ATTN_INT8) ? p.vs_head[h] * (1.0f / 127.0f) : 1.0f;

  TR regs;
  prefetch(0, regs);
  for (int t = 0; t < t_end; ++t) {
    const int k0 = t * BN;
    __syncthreads();  // every wave is done reading the previous tile
    commit(regs);
    __syncthreads();
    if (t + 1 < t_end) prefetch(t + 1, regs);  // in flight during this tile's compute
    // the ragged last tile and the causal diagonal need a per-key validity
    // test; the other tiles skip it (uniform branch)
    const bool masked = (k0 + BN > Skv) || (CAUSAL && t == qt);

    // ---- S^T = K Q^T: score of (query qb*16 + l16, key of block b at
    // output row 4g + r)
    f32x4 s[2][8];
    if (MODE == ATTN_FP8) {
#pragma unroll
      for (int b = 0; b < 8; ++b) s[0][b] = s[1][b] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int kk = 0; kk < KK; ++kk) {
        bf16x8 qop[2];
#pragma unroll
        for (int qb = 0; qb < 2; ++qb)
          qop[qb] = __builtin_bit_cast(bf16x8, i32x4{(int)e4m3x2_to_bf16x2<false>(q8[qb][kk].x),
                                                     (int)e4m3x2_to_bf16x2<true>(q8[qb][kk].x),
                                                     (int)e4m3x2_to_bf16x2<false>(q8[qb][kk].y),
                                                     (int)e4m3x2_to_bf16x2<true>(q8[qb][kk].y)});
#pragma unroll
        for (int b = 0; b < 8; ++b) {
          const int row = 16 * b + l16;
          const bf16x8 kop =
              *reinterpret_cast<const bf16x8*>(&k_lds[row * KB + (((4 * kk + g) ^ swz_bf(row, KCH)) * 16)]);
#pragma unroll
          for (int qb = 0; qb < 2; ++qb)
            s[qb][b] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kop, qop[qb], s[qb][b], 0, 0, 0);
        }
      }
    } else if (MODE == ATTN_INT8) {
#pragma unroll
      for (int b = 0; b < 8; ++b) {
        const int row = 16 * b + l16;
        i32x4 si[2] = {i32x4{0, 0, 0, 0}, i32x4{0, 0, 0, 0}};
#pragma unroll
        for (int kk = 0; kk < D / 64; ++kk) {
          const int cc = 4 * kk + g;
          const int sw = (KCH == 8 ? swz8(row) : swz4(row));
          const uint4 a = *reinterpret_cast<const uint4*>(&k_lds[row * KB + ((cc ^ sw) * 16)]);
          const i32x4 kop = {(int)a.x, (int)a.y, (int)a.z, (int)a.w};
#pragma unroll
          for (int qb = 0; qb < 2; ++qb)
            si[qb] = __builtin_amdgcn_mfma_i32_16x16x64_i8(kop, qi8[qb][kk], si[qb], 0, 0, 0);
        }
        // exact int32 scores (|s| < 2^21): the float conversion is exact
#pragma unroll
        for (int qb = 0; qb < 2; ++qb)
          s[qb][b] = f32x4{(float)si[qb][0], (float)si[qb][1], (float)si[qb][2], (float)si[qb][3]};
      }
    } else {
#pragma unroll
      for (int b = 0; b < 8; ++b) {
        const int row = k_row_mx(b, l16);
        i32x8 kop = {0, 0, 0, 0, 0, 0, 0, 0};
        int ksc = 127;
        if (32 * g < D) {
          const int sw = (KCH == 4 ? swz_mx(row) : 0);
          const uint4 a = *reinterpret_cast<const uint4*>(&k_lds[row * KB + ((g ^ sw) * 16)]);
          kop = i32x8{(int)a.x, (int)a.y, (int)a.z, (int)a.w, 0, 0, 0, 0};
          ksc = kex_lds[row * NB + g];
        }
#pragma unroll
        for (int qb = 0; qb < 2; ++qb) {
          const i32x4 qv = qmx[qb];
          const i32x8 qop = {qv[0], qv[1], qv[2], qv[3], 0, 0, 0, 0};
          s[qb][b] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(kop, qop, f32x4{0.f, 0.f, 0.f, 0.f},
                                                                      4, 4, 0, ksc, 0, qsc[qb]);
        }
      }
    }

    // ---- scores in "t units" (t * cq is the log2-domain score)
    if (MODE == ATTN_FP8) {
#pragma unroll
      for (int b = 0; b < 8; ++b) {
        const float4 skv = *reinterpret_cast<const float4*>(&sk_lds[16 * b + 4 * g]);
#pragma unroll
        for (int qb = 0; qb < 2; ++qb) {
          s[qb][b][0] *= skv.x; s[qb][b][1] *= skv.y; s[qb][b][2] *= skv.z; s[qb][b][3] *= skv.w;
        }
      }
    }
    if (masked) {
#pragma unroll
      for (int qb = 0; qb < 2; ++qb) {
        const int qi = qbase + qb * 16 + l16;
        const int lim = (CAUSAL ? min(Skv, qi + 1) : Skv) - k0;  // keys kl < lim are valid
#pragma unroll
        for (int b = 0; b < 8; ++b)
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            const int kl = (MODE == ATTN_MX) ? (32 * g + 4 * b + r) : (16 * b + 4 * g + r);
            s[qb][b][r] = (kl < lim) ? s[qb][b][r] : -INFINITY;
          }
      }
    }
    float mt[2];
#pragma unroll
    for (int qb = 0; qb < 2; ++qb) {
      float m = -INFINITY;
      if (MODE == ATTN_INT8 && !masked) {
        // exact integer scores: integer max (no float canonicalization)
        int mi = INT_MIN;
#pragma unroll
        for (int b = 0; b < 8; ++b)
          mi = max(max(mi, max((int)s[qb][b][0], (int)s[qb][b][1])), max((int)s[qb][b][2], (int)s[qb][b][3]));
        m = (float)mi;
      } else {
#pragma unroll
        for (int b = 0; b < 8; ++b)
          m = fmaxf(fmaxf(m, fmaxf(s[qb][b][0], s[qb][b][1])), fmaxf(s[qb][b][2], s[qb][b][3]));
      }
      mt[qb] = rows4_max(m);
    }

    // ---- probabilities, tile sums, quantized P operands, row combination
    i32x8 pi8[2];      // INT8: rne(127 p) bytes, keys in vt_key_int8 order
    i32x4 pbf[2][4];   // FP8 / MXFP4: bf16 images of the quantized p, per step kk
    float rscale[2], bvi8[2];
    bool rescale_any = false;
#pragma unroll
    for (int qb = 0; qb < 2; ++qb) {
      const float m = mt[qb];
      const float msafe = (m == -INFINITY) ? 0.0f : m;
      float lsum = 0.0f, pmax = 0.0f;
      if (MODE == ATTN_INT8) {
        // p = 2^(s cq - m cq); p at the maximum may differ from 1 by an ulp,
        // which cannot move rne(127 p)
        const float mc = msafe * cq[qb];
#pragma unroll
        for (int b = 0; b < 8; ++b)
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            const float pv = __builtin_amdgcn_exp2f(__builtin_fmaf(s[qb][b][r], cq[qb], -mc));
            s[qb][b][r] = pv;
            lsum += pv;
          }
      } else {
#pragma unroll
        for (int b = 0; b < 8; ++b)
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            // (x - m) is exactly 0 at the tile maximum, so p = 1 there exactly
            const float pv = __builtin_amdgcn_exp2f((s[qb][b][r] - msafe) * cq[qb]);
            s[qb][b][r] = pv;
            lsum += pv;
            if (MODE == ATTN_MX) pmax = fmaxf(pmax, pv);
          }
      }
      lsum = rows4_sum(lsum);

      // online combination of tiles
      const float mnew = fmaxf(M[qb], m);
      const float a = __builtin_amdgcn_exp2f((M[qb] - mnew) * cq[qb]);
      const float bt = (m == -INFINITY) ? 0.0f : __builtin_amdgcn_exp2f((m - mnew) * cq[qb]);
      L[qb] = L[qb] * a + lsum * bt;
      M[qb] = mnew;

      if (MODE == ATTN_INT8) {
        int w[8];
#pragma unroll
        for (int b = 0; b < 8; ++b) {
          // rne(127 p) lands in the low byte of fma(p, 127, 1.5 * 2^23)
          const uint32_t f0 = __float_as_uint(__builtin_fmaf(s[qb][b][0], 127.0f, 12582912.0f));
          const uint32_t f1 = __float_as_uint(__builtin_fmaf(s[qb][b][1], 127.0f, 12582912.0f));
          const uint32_t f2 = __float_as_uint(__builtin_fmaf(s[qb][b][2], 127.0f, 12582912.0f));
          const uint32_t f3 = __float_as_uint(__builtin_fmaf(s[qb][b][3], 127.0f, 12582912.0f));
          const uint32_t lo = __builtin_amdgcn_perm(f1, f0, 0x0c0c0400u);
          const uint32_t hi = __builtin_amdgcn_perm(f3, f2, 0x0c0c0400u);
          w[b] = (int)__builtin_amdgcn_perm(hi, lo, 0x05040100u);
        }
        pi8[qb] = i32x8{w[0], w[1], w[2], w[3], w[4], w[5], w[6], w[7]};
        rscale[qb] = a;
        bvi8[qb] = bt * vscale_i8;
        rescale_any |= (a != 1.0f);
      } else {
        // bf16-MFMA modes: new reference factor f = bt (times sigma_t / 448
        // for FP8); a row whose tile is negligible (bt < 2^-64) keeps its
        // reference and contributes nothing, which keeps O bounded.
        float ft = bt;
        if (MODE == ATTN_FP8) ft *= p.sig[bh * p.nt + t] * (1.0f / 448.0f);
        const bool live = bt >= 0x1p-64f;
        const float r = live ? (fref[qb] * a / ft) : a;
        fref[qb] = live ? ft : fref[qb];
        rscale[qb] = r;
        rescale_any |= (r != 1.0f);
        if (MODE == ATTN_FP8) {
#pragma unroll
          for (int b = 0; b < 8; ++b) {
            const float4 vm = *reinterpret_cast<const float4*>(&vm_lds[16 * b + 4 * g]);
            // E4M3 of 448 p w_j (round to nearest even), then its exact bf16 image
            int e8 = __builtin_amdgcn_cvt_pk_fp8_f32(s[qb][b][0] * vm.x, s[qb][b][1] * vm.y, 0, false);
            e8 = __builtin_amdgcn_cvt_pk_fp8_f32(s[qb][b][2] * vm.z, s[qb][b][3] * vm.w, e8, true);
            pbf[qb][b >> 1][2 * (b & 1)] = live ? (int)e4m3x2_to_bf16x2<false>((uint32_t)e8) : 0;
            pbf[qb][b >> 1][2 * (b & 1) + 1] = live ? (int)e4m3x2_to_bf16x2<true>((uint32_t)e8) : 0;
          }
        } else {
          // this lane's 32 keys are one MX group: local max -> shared
          // exponent; p -> E2M1(p / 2^E) * 2^E, exact in bf16
          const int E = mx_exponent(pmax);
          const float sc = E > -127 ? __uint_as_float((uint32_t)(E + 127) << 23) : 1.0f;
#pragma unroll
          for (int b = 0; b < 8; ++b) {
#pragma unroll
            for (int hh = 0; hh < 2; ++hh) {
              const uint32_t f4 =
                  __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(0u, s[qb][b][2 * hh], s[qb][b][2 * hh + 1], sc, 0);
              const int v2 = (int)__builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(f4, sc, 0));
              pbf[qb][b >> 1][2 * (b & 1) + hh] = live ? v2 : 0;
            }
          }
        }
      }
    }

    // ---- O^T += V^T P^T (per 16-channel block)
    const bool do_rescale = __any(rescale_any);
#pragma unroll
    for (int db = 0; db < DB; ++db) {
      const int row = 16 * db + l16;
      if (do_rescale) {
#pragma unroll
        for (int qb = 0; qb < 2; ++qb)
#pragma unroll
          for (int r = 0; r < 4; ++r) O[qb][db][r] *= rscale[qb];
      }
      if (MODE == ATTN_INT8) {
        const uint4 a = *reinterpret_cast<const uint4*>(&v_lds[row * VB + (((2 * g) ^ swz8(row)) * 16)]);
        const uint4 c = *reinterpret_cast<const uint4*>(&v_lds[row * VB + (((2 * g + 1) ^ swz8(row)) * 16)]);
        const i32x4 v0 = {(int)a.x, (int)a.y, (int)a.z, (int)a.w};
        const i32x4 v1 = {(int)c.x, (int)c.y, (int)c.z, (int)c.w};
#pragma unroll
        for (int qb = 0; qb < 2; ++qb) {
          const i32x4 p0 = {pi8[qb][0], pi8[qb][1], pi8[qb][2], pi8[qb][3]};
          const i32x4 p1 = {pi8[qb][4], pi8[qb][5], pi8[qb][6], pi8[qb][7]};
          i32x4 ci = __builtin_amdgcn_mfma_i32_16x16x64_i8(v0, p0, i32x4{0, 0, 0, 0}, 0, 0, 0);
          ci = __builtin_amdgcn_mfma_i32_16x16x64_i8(v1, p1, ci, 0, 0, 0);
#pragma unroll
          for (int r = 0; r < 4; ++r) O[qb][db][r] = __builtin_fmaf((float)ci[r], bvi8[qb], O[qb][db][r]);
        }
      } else {
        const int sw = swz_bf(row, VCH);
#pragma unroll
        for (int kk = 0; kk < 4; ++kk) {
          const bf16x8 vop = *reinterpret_cast<const bf16x8*>(&v_lds[row * VB + (((4 * kk + g) ^ sw) * 16)]);
#pragma unroll
          for (int qb = 0; qb < 2; ++qb)
            O[qb][db] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(vop, __builtin_bit_cast(bf16x8, pbf[qb][kk]),
                                                                O[qb][db], 0, 0, 0);
        }
      }
    }
  }

  // ---- normalize, store
#pragma unroll
  for (int qb = 0; qb < 2; ++qb) {
    const int qi = qbase + qb * 16 + l16;
    if (qi >= p.Sq) continue;
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
  uint8_t* vt = ws + l.vt_off;
  dim3 pgrid((unsigned)nt, (unsigned)(a.B * a.H));
  if (MODE == ATTN_MX) {
    k_prep_v_mx<D><<<pgrid, 256, 0, st>>>((const uint8_t*)a.v_codes, (const uint8_t*)a.v_scales, a.Skv, nt,
                                          reinterpret_cast<uint16_t*>(vt));
  } else {
    k_prep_v<D, MODE == ATTN_FP8><<<pgrid, 256, 0, st>>>(
        (const uint8_t*)a.v_codes, (const float*)a.v_scales, a.Skv, a.kv_block, nt, vt,
        reinterpret_cast<float*>(ws + l.aux_off), reinterpret_cast<float*>(ws + l.sig_off));
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  KParams p{};
  p.H = a.H; p.Sq = a.Sq; p.Skv = a.Skv; p.nt = nt;
  p.q = (const uint8_t*)a.q_codes; p.qs = a.q_scales;
  p.k = (const uint8_t*)a.k_codes; p.ks = a.k_scales;
  p.vt = vt;
  p.vmul = reinterpret_cast<const float*>(ws + l.aux_off);
  p.sig = reinterpret_cast<const float*>(ws + l.sig_off);
  p.vs_head = (const float*)a.v_scales;
  p.q_block = a.q_block; p.kv_block = a.kv_block;
  p.c_log2 = a.sm_scale * kLog2e;
  p.out = a.out; p.out_bf16 = a.out_bf16;
  dim3 grid((unsigned)((a.Sq + BM - 1) / BM), (unsigned)(a.B * a.H));
  if (a.causal) k_attn<MODE, D, true><<<grid, 256, 0, st>>>(p);
  else k_attn<MODE, D, false><<<grid, 256, 0, st>>>(p);
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
