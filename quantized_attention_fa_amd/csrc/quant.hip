// Q/K/V quantization kernels for gfx950.
//
// All of them are HBM-bound streaming kernels: 16-byte loads and stores,
// several loads in flight per thread before any arithmetic, reductions
// across lanes with shuffles.  The arithmetic is bit-exact with respect to
// the formats' definitions:
//   scale = fl32(amax / qmax) (IEEE division; amax == 0 -> 1),
//   u     = fl32(x / scale)   (correctly rounded: one fma correction of
//                              x * RN(1 / scale), see div_rn),
//   code  = nearest code to u, ties to even, saturating (hardware E4M3 and
//           E2M1 conversions, an exact integer rounding for INT8).
// Formats and granularities follow the msModelSlim "FA 量化" page
// (分支组合, 组合 1-3) and the MindIE SD "量化" page (FA量化 / 技术特点).

#include "common.h"
#include "launch.h"

namespace faq {
namespace {

constexpr int kThreads = 256;

// Logical row (b H + h) S + s of memory row r (BSND memory rows run
// (b, s, h); rows below 2^32).  The per-row quantizers walk memory rows in
// order, so neighbouring threads read neighbouring rows in either layout,
// and place each row's scales at its logical index.
FAQ_DEV int64_t logical_row(const RowMap& m, int64_t r, uint32_t H, uint32_t S) {
  if (m.ident) return r;
  const uint32_t r32 = (uint32_t)r, bs = r32 / H, h = r32 - bs * H, b = bs / S, s = bs - b * S;
  return ((int64_t)b * H + h) * S + s;
}

// Element offset of element i (0 <= i < S D) of the (b, h) slice: rows of D
// = 2^dsh elements, consecutive tokens m.ss rows apart.
FAQ_DEV int64_t slice_off(int64_t row0, int64_t i, const RowMap& m, int dsh) {
  return ((row0 + (i >> dsh) * m.ss) << dsh) + (i & ((1 << dsh) - 1));
}

// ------------------------------------------------------------------------
// Min-max calibration: amax[h] = max(amax[h], max |x[b,h,:,:]|).
// grid = (chunks per (b,h) slice, B*H); the float bits of a non-negative
// value order like unsigned integers, so the running max is an atomicMax.
// ------------------------------------------------------------------------
template <typename T>
__global__ __launch_bounds__(kThreads) void k_calibrate(const T* __restrict__ x, RowMap rm, int dsh, int64_t per_bh,
                                                        int H, float* __restrict__ amax) {
  constexpr int U = 4;
  const int64_t bh = blockIdx.y;
  const int64_t row0 = rm.row(bh / H, bh % H, 0);
  float m = 0.0f;
  for (int64_t c0 = (int64_t)blockIdx.x * kThreads * 8 * U; c0 < per_bh;
       c0 += (int64_t)gridDim.x * kThreads * 8 * U) {
    float v[U][8];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int64_t i = c0 + ((int64_t)u * kThreads + threadIdx.x) * 8;
      if (i < per_bh) {
        load8(x + slice_off(row0, i, rm, dsh), v[u]);
      } else {
#pragma unroll
        for (int k = 0; k < 8; ++k) v[u][k] = 0.0f;
      }
    }
#pragma unroll
    for (int u = 0; u < U; ++u)
#pragma unroll
      for (int k = 0; k < 8; ++k) m = fmaxf(m, fabsf(v[u][k]));
  }
  m = wave_max(m);
  __shared__ float red[kThreads / 64];
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = m;
  __syncthreads();
  if (threadIdx.x == 0) {
    m = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
    atomicMax(reinterpret_cast<unsigned int*>(amax + (bh % H)), __float_as_uint(m));
  }
}

__global__ void k_scales_from_amax(const float* amax, int64_t H, float qmax, float* scale) {
  const int64_t h = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (h < H) scale[h] = scale_from_amax(amax[h], qmax);
}

// ------------------------------------------------------------------------
// Per-head static: INT8 code = clamp(rne(x / scale[h]), -128, 127); FP8
// code = E4M3(x / scale[h]) saturating at +-448 (FA PerHead, INT8 / FP8).
// grid = (chunks per (b,h) slice, B*H); 16 elements per thread-vector.
// ------------------------------------------------------------------------
template <bool FAST, bool FP8, typename T>
FAQ_DEV void head_slice(const T* __restrict__ src, uint8_t* __restrict__ dst, int64_t row0, const RowMap& rm,
                        int dsh, int64_t per_bh, float s) {
  constexpr int U = 1;
  const float r = 1.0f / s;
  for (int64_t c0 = (int64_t)blockIdx.x * kThreads * 16 * U; c0 < per_bh;
       c0 += (int64_t)gridDim.x * kThreads * 16 * U) {
    float v[U][16];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int64_t i = c0 + ((int64_t)u * kThreads + threadIdx.x) * 16;
      if (i < per_bh) {
        const int64_t o = slice_off(row0, i, rm, dsh);
        float a[8], b[8];
        load8(src + o, a);
        load8(src + o + 8, b);
#pragma unroll
        for (int k = 0; k < 8; ++k) { v[u][k] = a[k]; v[u][8 + k] = b[k]; }
      }
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int64_t i = c0 + ((int64_t)u * kThreads + threadIdx.x) * 16;
      if (i < per_bh) {
        uint32_t w[4];
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          if (FP8) {
            w[j] = e4m3_sat_code_word<FAST>(v[u] + 4 * j, s, r);
          } else {
            uint32_t c[4];
#pragma unroll
            for (int k = 0; k < 4; ++k) c[k] = int8_code_word<FAST>(v[u][4 * j + k], s, r);
            w[j] = pack_low_bytes(c[0], c[1], c[2], c[3]);
          }
        }
        *reinterpret_cast<uint4*>(dst + slice_off(row0, i, rm, dsh)) = make_uint4(w[0], w[1], w[2], w[3]);
      }
    }
  }
}

template <typename T, bool FP8>
__global__ __launch_bounds__(kThreads) void k_quant_head(const T* __restrict__ x,
                                                         const float* __restrict__ scale, RowMap rm, int dsh,
                                                         int64_t per_bh, int H,
                                                         uint8_t* __restrict__ codes) {
  const int64_t bh = blockIdx.y;
  const float s = scale[bh % H];
  const int64_t row0 = rm.row(bh / H, bh % H, 0);
  // the head's scale picks the division path once for the whole slice
  if (div_fast_ok(s)) head_slice<true, FP8>(x, codes, row0, rm, dsh, per_bh, s);
  else head_slice<false, FP8>(x, codes, row0, rm, dsh, per_bh, s);
}

// ------------------------------------------------------------------------
// Per-token dynamic: one scale per (b,h,s) row of D elements, FP8 E4M3
// (s = amax / 448) or INT8 (s = amax / 127) (FA PerToken, FP8 / INT8).
// D/16 threads per row, 16 elements per thread.
// ------------------------------------------------------------------------
template <typename T, int D, bool I8>
__global__ __launch_bounds__(kThreads) void k_quant_token(const T* __restrict__ x, int64_t rows, RowMap rm,
                                                          uint32_t H, uint32_t S, uint8_t* __restrict__ codes,
                                                          float* __restrict__ scales) {
  constexpr int EPT = 16, TPR = D / EPT, RPB = kThreads / TPR, U = 1;
  const int sub = threadIdx.x % TPR, rin = threadIdx.x / TPR;
  for (int64_t r0 = (int64_t)blockIdx.x * RPB * U; r0 < rows; r0 += (int64_t)gridDim.x * RPB * U) {
    float v[U][EPT];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int64_t row = r0 + u * RPB + rin;
      if (row < rows) {
        const int64_t mr = row;  // memory row
        float a[8], b[8];
        load8(x + mr * D + sub * EPT, a);
        load8(x + mr * D + sub * EPT + 8, b);
#pragma unroll
        for (int k = 0; k < 8; ++k) { v[u][k] = a[k]; v[u][8 + k] = b[k]; }
      } else {
#pragma unroll
        for (int k = 0; k < EPT; ++k) v[u][k] = 0.0f;
      }
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int64_t row = r0 + u * RPB + rin;
      float m = 0.0f;
#pragma unroll
      for (int k = 0; k < EPT; ++k) m = fmaxf(m, fabsf(v[u][k]));
      m = group_max<TPR>(m);
      const float s = scale_from_amax(m, I8 ? 127.0f : 448.0f);
      uint32_t w[4];
      if (I8) int8_code_words<EPT>(v[u], s, w);
      else e4m3_code_words<EPT>(v[u], s, w);
      if (row < rows) {
        *reinterpret_cast<uint4*>(codes + row * D + sub * EPT) = make_uint4(w[0], w[1], w[2], w[3]);
        if (sub == 0) scales[logical_row(rm, row, H, S)] = s;
      }
    }
  }
}

// ------------------------------------------------------------------------
// MXFP4 per-block: 32 consecutive elements along D share an E8M0 exponent.
// D/8 threads per row; 4 threads per 32-element block.
// ------------------------------------------------------------------------
template <typename T, int D>
__global__ __launch_bounds__(kThreads) void k_quant_mxfp4(const T* __restrict__ x, int64_t rows, RowMap rm,
                                                          uint32_t H, uint32_t S, uint8_t* __restrict__ codes,
                                                          uint8_t* __restrict__ e8m0) {
  constexpr int TPR = D / 8, RPB = kThreads / TPR, U = 2, NB = D / 32;
  const int sub = threadIdx.x % TPR, rin = threadIdx.x / TPR;
  const int lane = threadIdx.x & 63;
  for (int64_t r0 = (int64_t)blockIdx.x * RPB * U; r0 < rows; r0 += (int64_t)gridDim.x * RPB * U) {
    float v[U][8];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int64_t row = r0 + u * RPB + rin;
      if (row < rows) {
        load8(x + row * D + sub * 8, v[u]);  // memory row
      } else {
#pragma unroll
        for (int k = 0; k < 8; ++k) v[u][k] = 0.0f;
      }
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int64_t row = r0 + u * RPB + rin;
      float m = 0.0f;
#pragma unroll
      for (int k = 0; k < 8; ++k) m = fmaxf(m, fabsf(v[u][k]));
      m = group_max<4>(m);
      const int E = mx_exponent(m);
      // hardware E2M1 of x / 2^E (exact division by a power of two;
      // nearest, ties to even, saturating at 6, sign kept)
      const float sc = __uint_as_float((uint32_t)(E > -127 ? E + 127 : 127) << 23);
      uint32_t packed = 0;
      packed = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(packed, v[u][0], v[u][1], sc, 0);
      packed = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(packed, v[u][2], v[u][3], sc, 1);
      packed = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(packed, v[u][4], v[u][5], sc, 2);
      packed = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(packed, v[u][6], v[u][7], sc, 3);
      if (__builtin_expect(__builtin_amdgcn_ballot_w64(E == -127) != 0, 0)) {
        // 2^-127 is not a normal float: blocks with zero or subnormal amax
        // scale with ldexp and encode in software
        if (E == -127) {
          packed = 0;
#pragma unroll
          for (int k = 0; k < 8; ++k)
            packed |= enc_e2m1(__builtin_amdgcn_ldexpf(v[u][k], 127)) << (4 * k);
        }
      }
      // gather the row's NB exponent bytes into the row's first lane
      uint32_t eb = (uint32_t)(E + 127);
      uint32_t word = eb;
#pragma unroll
      for (int j = 1; j < NB; ++j) word |= (uint32_t)__shfl(eb, lane + 4 * j, 64) << (8 * j);
      if (row < rows) {
        *reinterpret_cast<uint32_t*>(codes + row * (D / 2) + sub * 4) = packed;
        if (sub == 0) {
          const int64_t lr = logical_row(rm, row, H, S);
          if (NB == 4) *reinterpret_cast<uint32_t*>(e8m0 + lr * NB) = word;
          else *reinterpret_cast<uint16_t*>(e8m0 + lr * NB) = (uint16_t)word;
        }
      }
    }
  }
}

// ------------------------------------------------------------------------
// MXFP8 per-block: 32 consecutive elements along D share an E8M0 exponent
// E = floor(log2 amax) - 8; elements are E4M3 of x / 2^E (exact scaling),
// saturating at 448 (FA PerBlock, MXFP8).  D/8 threads per row, 4 per block.
// ------------------------------------------------------------------------
template <typename T, int D>
__global__ __launch_bounds__(kThreads) void k_quant_mxfp8(const T* __restrict__ x, int64_t rows, RowMap rm,
                                                          uint32_t H, uint32_t S, uint8_t* __restrict__ codes,
                                                          uint8_t* __restrict__ e8m0) {
  constexpr int TPR = D / 8, RPB = kThreads / TPR, U = 2, NB = D / 32;
  const int sub = threadIdx.x % TPR, rin = threadIdx.x / TPR;
  const int lane = threadIdx.x & 63;
  for (int64_t r0 = (int64_t)blockIdx.x * RPB * U; r0 < rows; r0 += (int64_t)gridDim.x * RPB * U) {
    float v[U][8];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int64_t row = r0 + u * RPB + rin;
      if (row < rows) {
        load8(x + row * D + sub * 8, v[u]);  // memory row
      } else {
#pragma unroll
        for (int k = 0; k < 8; ++k) v[u][k] = 0.0f;
      }
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int64_t row = r0 + u * RPB + rin;
      float m = 0.0f;
#pragma unroll
      for (int k = 0; k < 8; ++k) m = fmaxf(m, fabsf(v[u][k]));
      m = group_max<4>(m);
      const int E = mx_exponent<8>(m);
      // x / 2^E is exact wherever it can reach a nonzero code; the block
      // maximum lies in [256, 512) and saturates above 448
      float q[8];
#pragma unroll
      for (int k = 0; k < 8; ++k)
        q[k] = with_sign_of(__builtin_amdgcn_fmed3f(__builtin_amdgcn_ldexpf(v[u][k], -E), -448.0f, 448.0f), v[u][k]);
      int w0 = __builtin_amdgcn_cvt_pk_fp8_f32(q[0], q[1], 0, false);
      w0 = __builtin_amdgcn_cvt_pk_fp8_f32(q[2], q[3], w0, true);
      int w1 = __builtin_amdgcn_cvt_pk_fp8_f32(q[4], q[5], 0, false);
      w1 = __builtin_amdgcn_cvt_pk_fp8_f32(q[6], q[7], w1, true);
      // gather the row's NB exponent bytes into the row's first lane
      uint32_t eb = (uint32_t)(E + 127);
      uint32_t word = eb;
#pragma unroll
      for (int j = 1; j < NB; ++j) word |= (uint32_t)__shfl(eb, lane + 4 * j, 64) << (8 * j);
      if (row < rows) {
        *reinterpret_cast<uint2*>(codes + row * D + sub * 8) = make_uint2((uint32_t)w0, (uint32_t)w1);
        if (sub == 0) {
          const int64_t lr = logical_row(rm, row, H, S);
          if (NB == 4) *reinterpret_cast<uint32_t*>(e8m0 + lr * NB) = word;
          else *reinterpret_cast<uint16_t*>(e8m0 + lr * NB) = (uint16_t)word;
        }
      }
    }
  }
}

// ------------------------------------------------------------------------
// FP8 E4M3 token-block quantization without rotation (the V branch of the
// rotate path): one scale per (b,h, BT tokens x D).  bf16 input.
// One workgroup per block; the block stays in registers between the amax
// reduction and the encode.
// ------------------------------------------------------------------------
template <int D, int BT>
__global__ __launch_bounds__(kThreads) void k_quant_fp8_block(const uint16_t* __restrict__ x, RowMap rm, int H,
                                                              int64_t S, int nblk,
                                                              uint8_t* __restrict__ codes,
                                                              float* __restrict__ scales) {
  constexpr int NV = BT * D / (kThreads * 8);
  const int64_t bh = blockIdx.y;
  const int blk = blockIdx.x;
  const int64_t tok0 = (int64_t)blk * BT;
  const int64_t ntok = (S - tok0) < BT ? (S - tok0) : BT;
  // element e of the block: token tok0 + e / D, channel e % D
  const int64_t row0 = rm.row(bh / H, bh % H, tok0);
  auto off = [&](int e) { return (row0 + (int64_t)(e / D) * rm.ss) * D + e % D; };
  uint4 raw[NV];
  float m = 0.0f;
#pragma unroll
  for (int i = 0; i < NV; ++i) {
    const int e = (i * kThreads + threadIdx.x) * 8;
    raw[i] = (e / D < ntok) ? *reinterpret_cast<const uint4*>(x + off(e)) : make_uint4(0, 0, 0, 0);
  }
#pragma unroll
  for (int i = 0; i < NV; ++i) {
    const uint32_t w[4] = {raw[i].x, raw[i].y, raw[i].z, raw[i].w};
#pragma unroll
    for (int j = 0; j < 4; ++j) m = fmaxf(m, fmaxf(fabsf(bf16_lo(w[j])), fabsf(bf16_hi(w[j]))));
  }
  m = wave_max(m);
  __shared__ float red[kThreads / 64];
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = m;
  __syncthreads();
  m = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
  const float s = scale_from_amax(m, 448.0f);
#pragma unroll
  for (int i = 0; i < NV; ++i) {
    const int e = (i * kThreads + threadIdx.x) * 8;
    if (e / D < ntok) {
      const uint32_t w[4] = {raw[i].x, raw[i].y, raw[i].z, raw[i].w};
      float f[8];
#pragma unroll
      for (int j = 0; j < 4; ++j) { f[2 * j] = bf16_lo(w[j]); f[2 * j + 1] = bf16_hi(w[j]); }
      uint32_t c[2];
      e4m3_code_words<8>(f, s, c);
      *reinterpret_cast<uint2*>(codes + off(e)) = make_uint2(c[0], c[1]);
    }
  }
  if (threadIdx.x == 0) scales[bh * nblk + blk] = s;
}

// ------------------------------------------------------------------------
// Rotation + FP8 token-block quantization (Q and K of the rotate path):
//   Y = bf16_rne(X . R),  then per (b,h, BT tokens): s = fl32(amax|Y| / 448),
//   code = E4M3(fl32(Y / s)).
// Y^T = R^T X^T on the bf16 MFMA (16x16x32, fp32 accumulate): the A operand
// is R^T from LDS (staged once per workgroup; the workgroup then walks
// blocks in a grid-stride loop), the B operand is X read straight from
// global memory (each lane's 8 bf16 are contiguous in a token row).  The
// accumulator holds, per lane, 4 consecutive output channels of one token.
// One wave per 32 tokens: BT/32 waves per workgroup.
// ------------------------------------------------------------------------
template <int D, int BT>
__global__ __launch_bounds__(BT * 2) void k_rot_fp8_block(const uint16_t* __restrict__ x,
                                                          const uint16_t* __restrict__ rot, RowMap rm, int H,
                                                          int64_t S, int nblk, int64_t nwork,
                                                          uint8_t* __restrict__ codes,
                                                          float* __restrict__ scales,
                                                          uint16_t* __restrict__ dbg) {
  constexpr int NW = BT / 32, NT = BT * 2, KK = D / 32, DB = D / 16, RS = D + 8;
  __shared__ uint16_t rt[D * RS];  // R^T, one padded row per output channel
  __shared__ float red[NW];
  for (int i = threadIdx.x; i < D * D; i += NT) {
    const int k = i / D, n = i % D;
    rt[n * RS + k] = rot[i];
  }
  __syncthreads();
  const int w = threadIdx.x >> 6, lane = threadIdx.x & 63, l16 = lane & 15, g = lane >> 4;
  for (int64_t work = blockIdx.x; work < nwork; work += gridDim.x) {
    const int64_t bh = work / nblk;
    const int blk = (int)(work % nblk);
    const int64_t tok0 = (int64_t)blk * BT + w * 32;
    const int64_t row0 = rm.row(bh / H, bh % H, 0);  // token tok is row row0 + tok rm.ss
    bf16x8 xb[2][KK];
#pragma unroll
    for (int tb = 0; tb < 2; ++tb) {
      const int64_t tok = tok0 + tb * 16 + l16;
#pragma unroll
      for (int kk = 0; kk < KK; ++kk) {
        uint4 r = make_uint4(0, 0, 0, 0);
        if (tok < S) r = *reinterpret_cast<const uint4*>(x + (row0 + tok * rm.ss) * D + kk * 32 + g * 8);
        xb[tb][kk] = __builtin_bit_cast(bf16x8, r);
      }
    }
    f32x4 acc[2][DB];
#pragma unroll
    for (int db = 0; db < DB; ++db) {
      acc[0][db] = f32x4{0.f, 0.f, 0.f, 0.f};
      acc[1][db] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int kk = 0; kk < KK; ++kk) {
        const bf16x8 a =
            *reinterpret_cast<const bf16x8*>(&rt[(db * 16 + l16) * RS + kk * 32 + g * 8]);
        acc[0][db] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, xb[0][kk], acc[0][db], 0, 0, 0);
        acc[1][db] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, xb[1][kk], acc[1][db], 0, 0, 0);
      }
    }
    // round to bf16 (the rotated tensor is bf16; the hardware conversion
    // rounds to nearest even), block max
    float m = 0.0f;
#pragma unroll
    for (int tb = 0; tb < 2; ++tb)
#pragma unroll
      for (int db = 0; db < DB; ++db)
#pragma unroll
        for (int r = 0; r < 4; r += 2) {
          const bf16x2 y = {(__bf16)acc[tb][db][r], (__bf16)acc[tb][db][r + 1]};
          const uint32_t yw = __builtin_bit_cast(uint32_t, y);
          acc[tb][db][r] = bf16_lo(yw);
          acc[tb][db][r + 1] = bf16_hi(yw);
          m = fmaxf(m, fmaxf(fabsf(acc[tb][db][r]), fabsf(acc[tb][db][r + 1])));
        }
    m = wave_max(m);
    if (lane == 0) red[w] = m;
    __syncthreads();
    m = red[0];
#pragma unroll
    for (int i = 1; i < NW; ++i) m = fmaxf(m, red[i]);
    __syncthreads();  // red is rewritten by the next block
    const float s = scale_from_amax(m, 448.0f);
#pragma unroll
    for (int tb = 0; tb < 2; ++tb) {
      const int64_t tok = tok0 + tb * 16 + l16;
      if (tok >= S) continue;
      float y[4 * DB];
#pragma unroll
      for (int db = 0; db < DB; ++db)
#pragma unroll
        for (int r = 0; r < 4; ++r) y[4 * db + r] = acc[tb][db][r];
      uint32_t c[DB];
      e4m3_code_words<4 * DB>(y, s, c);
#pragma unroll
      for (int db = 0; db < DB; ++db) {
        const int64_t off = (row0 + tok * rm.ss) * D + db * 16 + g * 4;
        *reinterpret_cast<uint32_t*>(codes + off) = c[db];
        if (dbg) {
          // y holds bf16 values: their top halves are the bf16 bits
          const float* yd = y + 4 * db;
          const uint32_t b0 = (__float_as_uint(yd[0]) >> 16) | (__float_as_uint(yd[1]) & 0xffff0000u);
          const uint32_t b1 = (__float_as_uint(yd[2]) >> 16) | (__float_as_uint(yd[3]) & 0xffff0000u);
          *reinterpret_cast<uint2*>(dbg + off) = make_uint2(b0, b1);
        }
      }
    }
    if (threadIdx.x == 0) scales[bh * nblk + blk] = s;
  }
}

inline unsigned grid_chunks(int64_t n, int64_t per_block, unsigned cap) {
  int64_t g = (n + per_block - 1) / per_block;
  if (g < 1) g = 1;
  return (unsigned)(g > cap ? cap : g);
}

}  // namespace

// ---------------------------------------------------------------- launchers

hipError_t launch_calibrate(const void* x, int x_dtype, const faq_shape& s, float* amax,
                            hipStream_t st) {
  const int64_t per_bh = s.S * s.D;
  const RowMap rm = row_map(s);
  const int dsh = s.D == 128 ? 7 : 6;
  dim3 grid(grid_chunks(per_bh, kThreads * 8 * 4, 65535), (unsigned)(s.B * s.H));
  if (x_dtype == FAQ_T_BF16)
    k_calibrate<uint16_t><<<grid, kThreads, 0, st>>>((const uint16_t*)x, rm, dsh, per_bh, (int)s.H, amax);
  else
    k_calibrate<float><<<grid, kThreads, 0, st>>>((const float*)x, rm, dsh, per_bh, (int)s.H, amax);
  return hipGetLastError();
}

hipError_t launch_scales_from_amax(const float* amax, int64_t H, float qmax, float* scale,
                                   hipStream_t st) {
  k_scales_from_amax<<<(unsigned)((H + 255) / 256), 256, 0, st>>>(amax, H, qmax, scale);
  return hipGetLastError();
}

template <bool FP8>
static hipError_t head_q(const void* x, int x_dtype, const faq_shape& s, const float* scale,
                         uint8_t* codes, hipStream_t st) {
  const int64_t per_bh = s.S * s.D;
  const RowMap rm = row_map(s);
  const int dsh = s.D == 128 ? 7 : 6;
  dim3 grid(grid_chunks(per_bh, kThreads * 16 * 1, 65535), (unsigned)(s.B * s.H));
  if (x_dtype == FAQ_T_BF16)
    k_quant_head<uint16_t, FP8><<<grid, kThreads, 0, st>>>((const uint16_t*)x, scale, rm, dsh, per_bh, (int)s.H,
                                                           codes);
  else
    k_quant_head<float, FP8><<<grid, kThreads, 0, st>>>((const float*)x, scale, rm, dsh, per_bh, (int)s.H, codes);
  return hipGetLastError();
}

hipError_t launch_quant_int8_head(const void* x, int x_dtype, const faq_shape& s,
                                  const float* scale, int8_t* codes, hipStream_t st) {
  return head_q<false>(x, x_dtype, s, scale, reinterpret_cast<uint8_t*>(codes), st);
}

hipError_t launch_quant_fp8_head(const void* x, int x_dtype, const faq_shape& s,
                                 const float* scale, uint8_t* codes, hipStream_t st) {
  return head_q<true>(x, x_dtype, s, scale, codes, st);
}

template <int D, bool I8>
static hipError_t token_d(const void* x, int x_dtype, const faq_shape& s, uint8_t* codes,
                          float* scales, hipStream_t st) {
  constexpr int RPB = kThreads / (D / 16);
  const int64_t rows = s.B * s.H * s.S;
  const RowMap rm = row_map(s);
  const unsigned grid = grid_chunks(rows, RPB * 1, 1u << 20);
  if (x_dtype == FAQ_T_BF16)
    k_quant_token<uint16_t, D, I8><<<grid, kThreads, 0, st>>>((const uint16_t*)x, rows, rm, (uint32_t)s.H,
                                                              (uint32_t)s.S, codes, scales);
  else
    k_quant_token<float, D, I8><<<grid, kThreads, 0, st>>>((const float*)x, rows, rm, (uint32_t)s.H,
                                                           (uint32_t)s.S, codes, scales);
  return hipGetLastError();
}

hipError_t launch_quant_fp8_token(const void* x, int x_dtype, const faq_shape& s,
                                  uint8_t* codes, float* scales, hipStream_t st) {
  return s.D == 128 ? token_d<128, false>(x, x_dtype, s, codes, scales, st)
                    : token_d<64, false>(x, x_dtype, s, codes, scales, st);
}

hipError_t launch_quant_int8_token(const void* x, int x_dtype, const faq_shape& s,
                                   int8_t* codes, float* scales, hipStream_t st) {
  uint8_t* c = reinterpret_cast<uint8_t*>(codes);
  return s.D == 128 ? token_d<128, true>(x, x_dtype, s, c, scales, st)
                    : token_d<64, true>(x, x_dtype, s, c, scales, st);
}

template <int D, bool FP4>
static hipError_t mx_d(const void* x, int x_dtype, const faq_shape& s, uint8_t* codes,
                       uint8_t* e8m0, hipStream_t st) {
  constexpr int RPB = kThreads / (D / 8);
  const int64_t rows = s.B * s.H * s.S;
  const RowMap rm = row_map(s);
  const uint32_t H = (uint32_t)s.H, S = (uint32_t)s.S;
  const unsigned grid = grid_chunks(rows, RPB * 2, 1u << 20);
  if (FP4) {
    if (x_dtype == FAQ_T_BF16)
      k_quant_mxfp4<uint16_t, D><<<grid, kThreads, 0, st>>>((const uint16_t*)x, rows, rm, H, S, codes, e8m0);
    else
      k_quant_mxfp4<float, D><<<grid, kThreads, 0, st>>>((const float*)x, rows, rm, H, S, codes, e8m0);
  } else {
    if (x_dtype == FAQ_T_BF16)
      k_quant_mxfp8<uint16_t, D><<<grid, kThreads, 0, st>>>((const uint16_t*)x, rows, rm, H, S, codes, e8m0);
    else
      k_quant_mxfp8<float, D><<<grid, kThreads, 0, st>>>((const float*)x, rows, rm, H, S, codes, e8m0);
  }
  return hipGetLastError();
}

hipError_t launch_quant_mxfp4(const void* x, int x_dtype, const faq_shape& s, uint8_t* codes,
                              uint8_t* e8m0, hipStream_t st) {
  return s.D == 128 ? mx_d<128, true>(x, x_dtype, s, codes, e8m0, st)
                    : mx_d<64, true>(x, x_dtype, s, codes, e8m0, st);
}

hipError_t launch_quant_mxfp8(const void* x, int x_dtype, const faq_shape& s, uint8_t* codes,
                              uint8_t* e8m0, hipStream_t st) {
  return s.D == 128 ? mx_d<128, false>(x, x_dtype, s, codes, e8m0, st)
                    : mx_d<64, false>(x, x_dtype, s, codes, e8m0, st);
}

template <int D, int BT>
static hipError_t fp8_block_d(const uint16_t* x, const faq_shape& s, uint8_t* codes,
                              float* scales, hipStream_t st) {
  const int nblk = (int)((s.S + BT - 1) / BT);
  dim3 grid((unsigned)nblk, (unsigned)(s.B * s.H));
  k_quant_fp8_block<D, BT><<<grid, kThreads, 0, st>>>(x, row_map(s), (int)s.H, s.S, nblk, codes, scales);
  return hipGetLastError();
}

hipError_t launch_quant_fp8_block(const uint16_t* x, const faq_shape& s, int block_tokens,
                                  uint8_t* codes, float* scales, hipStream_t st) {
  if (s.D == 128)
    return block_tokens == 128 ? fp8_block_d<128, 128>(x, s, codes, scales, st)
                               : fp8_block_d<128, 256>(x, s, codes, scales, st);
  return block_tokens == 128 ? fp8_block_d<64, 128>(x, s, codes, scales, st)
                             : fp8_block_d<64, 256>(x, s, codes, scales, st);
}

template <int D, int BT>
static hipError_t rot_block_d(const uint16_t* x, const uint16_t* rot, const faq_shape& s,
                              uint8_t* codes, float* scales, uint16_t* dbg, hipStream_t st) {
  const int nblk = (int)((s.S + BT - 1) / BT);
  const int64_t nwork = (int64_t)nblk * s.B * s.H;
  const unsigned grid = (unsigned)(nwork < 2048 ? nwork : 2048);
  k_rot_fp8_block<D, BT><<<grid, BT * 2, 0, st>>>(x, rot, row_map(s), (int)s.H, s.S, nblk, nwork, codes, scales,
                                                   dbg);
  return hipGetLastError();
}

hipError_t launch_rot_fp8_block(const uint16_t* x, const uint16_t* rot, const faq_shape& s,
                                int block_tokens, uint8_t* codes, float* scales,
                                uint16_t* debug_rotated, hipStream_t st) {
  if (s.D == 128)
    return block_tokens == 128
               ? rot_block_d<128, 128>(x, rot, s, codes, scales, debug_rotated, st)
               : rot_block_d<128, 256>(x, rot, s, codes, scales, debug_rotated, st);
  return block_tokens == 128 ? rot_block_d<64, 128>(x, rot, s, codes, scales, debug_rotated, st)
                             : rot_block_d<64, 256>(x, rot, s, codes, scales, debug_rotated, st);
}

}  // namespace faq
