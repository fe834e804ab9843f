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
// grid = (chunks per (b,h) slice, B*H).  A thread keeps U 16-byte loads in
// flight and reduces their magnitudes as integers: for finite values |x|
// orders like its magnitude bits (bf16: the low 15 bits of each half-word,
// two at a time with packed 16-bit max; fp32: the low 31 bits), so the max
// is exact.  The float bits of a non-negative value also order like
// unsigned integers, so the running max across workgroups and calls is an
// atomicMax (one per workgroup).
// ------------------------------------------------------------------------
template <typename T, int U>
__global__ __launch_bounds__(kThreads) void k_calibrate(const T* __restrict__ x, RowMap rm, int dsh, int64_t per_bh,
                                                        int H, float* __restrict__ amax) {
  constexpr int EPL = 16 / sizeof(T);  // elements per 16-byte load
  constexpr bool BF = sizeof(T) == 2;
  const int64_t bh = blockIdx.y;
  const int64_t row0 = rm.row(bh / H, bh % H, 0);
  uint32_t mb = 0;  // bf16: two packed 15-bit magnitudes; fp32: one 31-bit magnitude
  for (int64_t c0 = (int64_t)blockIdx.x * kThreads * EPL * U; c0 < per_bh;
       c0 += (int64_t)gridDim.x * kThreads * EPL * U) {
    uint4 v[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int64_t i = c0 + ((int64_t)u * kThreads + threadIdx.x) * EPL;
      v[u] = i < per_bh ? *reinterpret_cast<const uint4*>(x + slice_off(row0, i, rm, dsh)) : make_uint4(0, 0, 0, 0);
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const uint32_t w[4] = {v[u].x, v[u].y, v[u].z, v[u].w};
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        if (BF) {
          typedef unsigned short u16x2 __attribute__((ext_vector_type(2)));
          const u16x2 a = __builtin_bit_cast(u16x2, w[k] & 0x7fff7fffu);
          const u16x2 b = __builtin_bit_cast(u16x2, mb);
          mb = __builtin_bit_cast(uint32_t, __builtin_elementwise_max(a, b));
        } else {
          mb = max(mb, w[k] & 0x7fffffffu);
        }
      }
    }
  }
  if (BF) mb = max(mb & 0xffffu, mb >> 16) << 16;  // the larger half, as fp32 bits
  float m = __uint_as_float(mb);
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
// D/16 threads per row; two neighbouring lanes per 32-element block, whose
// maximum crosses them with one DPP swap (no LDS round trip); the lane
// holding the first half writes the block's exponent byte.
// ------------------------------------------------------------------------
template <typename T, int D>
__global__ __launch_bounds__(kThreads) void k_quant_mxfp4(const T* __restrict__ x, int64_t rows, RowMap rm,
                                                          uint32_t H, uint32_t S, uint8_t* __restrict__ codes,
                                                          uint8_t* __restrict__ e8m0) {
  constexpr int TPR = D / 16, RPB = kThreads / TPR, U = 2, NB = D / 32;
  const int sub = threadIdx.x % TPR, rin = threadIdx.x / TPR;
  for (int64_t r0 = (int64_t)blockIdx.x * RPB * U; r0 < rows; r0 += (int64_t)gridDim.x * RPB * U) {
    float a[U][8], b[U][8];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int64_t row = r0 + u * RPB + rin;
      if (row < rows) {
        load8(x + row * D + sub * 16, a[u]);  // memory row
        load8(x + row * D + sub * 16 + 8, b[u]);
      } else {
#pragma unroll
        for (int k = 0; k < 8; ++k) a[u][k] = b[u][k] = 0.0f;
      }
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int64_t row = r0 + u * RPB + rin;
      float m = 0.0f;
#pragma unroll
      for (int k = 0; k < 8; ++k) m = fmaxf(m, fmaxf(fabsf(a[u][k]), fabsf(b[u][k])));
      // the other half of the block: lane ^ 1 (quad_perm [1, 0, 3, 2])
      m = fmaxf(m, __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(m), 0xB1, 0xF, 0xF, false)));
      const int E = mx_exponent(m);
      // hardware E2M1 of x / 2^E (exact division by a power of two;
      // nearest, ties to even, saturating at 6, sign kept)
      const float sc = __uint_as_float((uint32_t)(E > -127 ? E + 127 : 127) << 23);
      uint32_t p0 = 0, p1 = 0;
      p0 = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(p0, a[u][0], a[u][1], sc, 0);
      p0 = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(p0, a[u][2], a[u][3], sc, 1);
      p0 = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(p0, a[u][4], a[u][5], sc, 2);
      p0 = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(p0, a[u][6], a[u][7], sc, 3);
      p1 = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(p1, b[u][0], b[u][1], sc, 0);
      p1 = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(p1, b[u][2], b[u][3], sc, 1);
      p1 = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(p1, b[u][4], b[u][5], sc, 2);
      p1 = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(p1, b[u][6], b[u][7], sc, 3);
      if (__builtin_expect(__builtin_amdgcn_ballot_w64(E == -127) != 0, 0)) {
        // 2^-127 is not a normal float: blocks with zero or subnormal amax
        // scale with ldexp and encode in software
        if (E == -127) {
          p0 = 0;
          p1 = 0;
#pragma unroll
          for (int k = 0; k < 8; ++k) {
            p0 |= enc_e2m1(__builtin_amdgcn_ldexpf(a[u][k], 127)) << (4 * k);
            p1 |= enc_e2m1(__builtin_amdgcn_ldexpf(b[u][k], 127)) << (4 * k);
          }
        }
      }
      if (row < rows) {
        *reinterpret_cast<uint2*>(codes + row * (D / 2) + sub * 8) = make_uint2(p0, p1);
        if ((sub & 1) == 0) e8m0[logical_row(rm, row, H, S) * NB + (sub >> 1)] = (uint8_t)(E + 127);
      }
    }
  }
}

// ------------------------------------------------------------------------
// MXFP8 per-block: 32 consecutive elements along D share an E8M0 exponent
// E = floor(log2 amax) - 8; elements are E4M3 of x / 2^E (exact scaling),
// saturating at 448 (FA PerBlock, MXFP8).  D/16 threads per row, two neighbouring
// lanes per block (one DPP swap for its maximum).
// ------------------------------------------------------------------------
template <typename T, int D>
__global__ __launch_bounds__(kThreads) void k_quant_mxfp8(const T* __restrict__ x, int64_t rows, RowMap rm,
                                                          uint32_t H, uint32_t S, uint8_t* __restrict__ codes,
                                                          uint8_t* __restrict__ e8m0) {
  constexpr int TPR = D / 16, RPB = kThreads / TPR, U = 2, NB = D / 32;
  const int sub = threadIdx.x % TPR, rin = threadIdx.x / TPR;
  for (int64_t r0 = (int64_t)blockIdx.x * RPB * U; r0 < rows; r0 += (int64_t)gridDim.x * RPB * U) {
    float v[U][16];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int64_t row = r0 + u * RPB + rin;
      float a[8], b[8];
      if (row < rows) {
        load8(x + row * D + sub * 16, a);  // memory row
        load8(x + row * D + sub * 16 + 8, b);
      } else {
#pragma unroll
        for (int k = 0; k < 8; ++k) a[k] = b[k] = 0.0f;
      }
#pragma unroll
      for (int k = 0; k < 8; ++k) { v[u][k] = a[k]; v[u][8 + k] = b[k]; }
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int64_t row = r0 + u * RPB + rin;
      float m = 0.0f;
#pragma unroll
      for (int k = 0; k < 16; ++k) m = fmaxf(m, fabsf(v[u][k]));
      // the other half of the block: lane ^ 1 (quad_perm [1, 0, 3, 2])
      m = fmaxf(m, __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(m), 0xB1, 0xF, 0xF, false)));
      const int E = mx_exponent<8>(m);
      // x / 2^E is exact wherever it can reach a nonzero code; the block
      // maximum lies in [256, 512) and saturates above 448
      float q[16];
#pragma unroll
      for (int k = 0; k < 16; ++k)
        q[k] = with_sign_of(__builtin_amdgcn_fmed3f(__builtin_amdgcn_ldexpf(v[u][k], -E), -448.0f, 448.0f), v[u][k]);
      uint32_t w[4];
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        int c = __builtin_amdgcn_cvt_pk_fp8_f32(q[4 * k], q[4 * k + 1], 0, false);
        c = __builtin_amdgcn_cvt_pk_fp8_f32(q[4 * k + 2], q[4 * k + 3], c, true);
        w[k] = (uint32_t)c;
      }
      if (row < rows) {
        *reinterpret_cast<uint4*>(codes + row * D + sub * 16) = make_uint4(w[0], w[1], w[2], w[3]);
        if ((sub & 1) == 0) e8m0[logical_row(rm, row, H, S) * NB + (sub >> 1)] = (uint8_t)(E + 127);
      }
    }
  }
}

// ------------------------------------------------------------------------
// Persistent walk over token blocks: workgroup g takes blocks g, g + grid,
// g + 2 grid, ... of the (b, h, block) order.  A position advances by the
// grid stride with carries (uniform scalar work): a division inside the
// loop would take vector registers that may still be the targets of loads
// in flight, which makes the compiler wait for all of them.
// ------------------------------------------------------------------------
struct BlockPos {
  int b, h, blk;
};

struct BlockWalk {
  int nblk, H, dblk, dh, db;  // blocks per head, heads, the grid stride split
  __device__ __forceinline__ BlockWalk(int grid, int nblk_, int H_) : nblk(nblk_), H(H_) {
    dblk = grid % nblk;
    const int dbh = grid / nblk;
    dh = dbh % H;
    db = dbh / H;
  }
  __device__ __forceinline__ BlockPos at(int work) const { return BlockPos{work / nblk / H, (work / nblk) % H, work % nblk}; }
  __device__ __forceinline__ BlockPos next(BlockPos p) const {
    p.blk += dblk;
    const int c = p.blk >= nblk ? 1 : 0;
    p.blk -= c * nblk;
    p.h += dh + c;  // < 2 H
    const int c2 = p.h >= H ? 1 : 0;
    p.h -= c2 * H;
    p.b += db + c2;
    return p;
  }
};

// ------------------------------------------------------------------------
// FP8 E4M3 token-block quantization without rotation (the V branch of the
// rotate path): one scale per (b,h, BT tokens x D).  bf16 input.
// Persistent workgroups walk the blocks; a block stays in registers between
// the amax reduction and the encode, and the next block's loads are issued
// before it is reduced (two register buffers; every load unconditional -
// rows past S re-read row S - 1 and are left out of the maximum and the
// stores - so the compiler's wait for one block leaves the next in
// flight).  The block maximum crosses the waves through LDS behind a
// barrier without a memory fence; alternating slots make one barrier per
// block enough.
// ------------------------------------------------------------------------
template <int D, int BT>
constexpr int fp8_block_threads() { return BT * D >= 256 * 128 ? 512 : kThreads; }

template <int D, int BT>
__global__ __launch_bounds__((fp8_block_threads<D, BT>()), 2) void k_quant_fp8_block(
    const uint16_t* __restrict__ x, RowMap rm, int H, int64_t S, int nblk, int nwork, uint8_t* __restrict__ codes,
    float* __restrict__ scales) {
  constexpr int NT = fp8_block_threads<D, BT>(), NW = NT / 64;
  constexpr int NV = BT * D / (NT * 8);  // 16-byte loads per thread and block
  __shared__ float red[2][NW];
  const int w = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const BlockWalk walk((int)gridDim.x, nblk, H);
  // element e of the block: token tok0 + e / D, channel e % D
  auto load = [&](BlockPos p, uint4(&raw)[NV]) __attribute__((always_inline)) {
    const int64_t tok0 = (int64_t)p.blk * BT;
    const int64_t row0 = rm.row(p.b, p.h, 0);
#pragma unroll
    for (int i = 0; i < NV; ++i) {
      const int e = (i * NT + threadIdx.x) * 8;
      const int64_t tok = min(tok0 + e / D, S - 1);
      raw[i] = *reinterpret_cast<const uint4*>(x + (row0 + tok * rm.ss) * D + e % D);
    }
  };
  auto process = [&](BlockPos p, const uint4(&raw)[NV], int slot) __attribute__((always_inline)) {
    const int64_t tok0 = (int64_t)p.blk * BT;
    const int64_t ntok = (S - tok0) < BT ? (S - tok0) : BT;
    const int64_t row0 = rm.row(p.b, p.h, 0);
    float m = 0.0f;
#pragma unroll
    for (int i = 0; i < NV; ++i) {
      const int e = (i * NT + threadIdx.x) * 8;
      const uint32_t wd[4] = {raw[i].x, raw[i].y, raw[i].z, raw[i].w};
      float mi = 0.0f;
#pragma unroll
      for (int j = 0; j < 4; ++j) mi = fmaxf(mi, fmaxf(fabsf(bf16_lo(wd[j])), fabsf(bf16_hi(wd[j]))));
      if (e / D < ntok) m = fmaxf(m, mi);
    }
    m = wave_max(m);
    if (lane == 0) red[slot][w] = m;
    barrier_lds();
    m = red[slot][0];
#pragma unroll
    for (int i = 1; i < NW; ++i) m = fmaxf(m, red[slot][i]);
    const float s = scale_from_amax(m, 448.0f);
#pragma unroll
    for (int i = 0; i < NV; ++i) {
      const int e = (i * NT + threadIdx.x) * 8;
      if (e / D < ntok) {
        const uint32_t wd[4] = {raw[i].x, raw[i].y, raw[i].z, raw[i].w};
        float f[8];
#pragma unroll
        for (int j = 0; j < 4; ++j) { f[2 * j] = bf16_lo(wd[j]); f[2 * j + 1] = bf16_hi(wd[j]); }
        uint32_t c[2];
        e4m3_code_words<8>(f, s, c);
        *reinterpret_cast<uint2*>(codes + (row0 + (tok0 + e / D) * rm.ss) * D + e % D) = make_uint2(c[0], c[1]);
      }
    }
    if (threadIdx.x == 0) scales[((int64_t)p.b * H + p.h) * nblk + p.blk] = s;
  };
  uint4 ra[NV], rc[NV];
  int work = (int)blockIdx.x;
  BlockPos pa = walk.at(work);
  load(pa, ra);
  for (;;) {
    const BlockPos pc = walk.next(pa);
    const bool more1 = work + (int)gridDim.x < nwork;
    load(more1 ? pc : pa, rc);
    process(pa, ra, 0);
    if (!more1) break;
    const BlockPos pn = walk.next(pc);
    const bool more2 = work + 2 * (int)gridDim.x < nwork;
    load(more2 ? pn : pc, ra);
    process(pc, rc, 1);
    if (!more2) break;
    pa = pn;
    work += 2 * (int)gridDim.x;
  }
}

// ------------------------------------------------------------------------
// Rotation + FP8 token-block quantization (Q and K of the rotate path):
//   Y = bf16_rne(X . R),  then per (b,h, BT tokens): s = fl32(amax|Y| / 448),
//   code = E4M3(fl32(Y / s)).
// Y^T = R^T X^T on the bf16 MFMA (16x16x32, fp32 accumulate): the A operand
// is R^T from LDS, the B operand X read straight from global memory (each
// lane's 8 bf16 are contiguous in a token row).  The accumulator holds, per
// lane, 4 consecutive output channels of one token.  One wave per 32
// tokens: BT/32 waves per workgroup.
// Persistent workgroups (as many as fit on the GPU at once) stage R^T once
// and walk the blocks; the X rows of the next block are loaded while the
// current one is rotated, reduced and encoded.  The block maximum crosses
// the waves through LDS behind a barrier without a memory fence, so those
// loads stay in flight across it (alternating reduction slots make one
// barrier per block enough: a slot is rewritten two blocks later, after
// every wave has passed the barrier that follows its last read).
// ------------------------------------------------------------------------
template <int D, int BT>
__global__ __launch_bounds__(BT * 2, 2) void k_rot_fp8_block(const uint16_t* __restrict__ x,
                                                          const uint16_t* __restrict__ rot, RowMap rm, int H,
                                                          int64_t S, int nblk, int nwork,
                                                          uint8_t* __restrict__ codes,
                                                          float* __restrict__ scales,
                                                          uint16_t* __restrict__ dbg) {
  constexpr int NW = BT / 32, NT = BT * 2, KK = D / 32, DB = D / 16, RS = D + 8;
  __shared__ uint16_t rt[D * RS];  // R^T, one padded row per output channel
  __shared__ float red[2][NW];
  // each wave's 32 x D codes on their way to memory: the accumulator gives
  // a lane 4 consecutive channels of one token, the stores want 16
  // contiguous bytes per lane (a 128-byte row per 8 lanes)
  constexpr int CR = D + 16;  // padded code row (bytes)
  __shared__ __attribute__((aligned(16))) uint8_t cst[NW][32 * CR];
  // R^T: 16-byte loads of R's rows k, each element to row n of rt
  for (int i = threadIdx.x; i < D * D / 8; i += NT) {
    const int k = i / (D / 8), n0 = (i % (D / 8)) * 8;
    const uint4 v = *reinterpret_cast<const uint4*>(rot + k * D + n0);
    const uint32_t wv[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      rt[(n0 + 2 * q) * RS + k] = (uint16_t)(wv[q] & 0xffffu);
      rt[(n0 + 2 * q + 1) * RS + k] = (uint16_t)(wv[q] >> 16);
    }
  }
  __syncthreads();
  const int w = threadIdx.x >> 6, lane = threadIdx.x & 63, l16 = lane & 15, g = lane >> 4;

  const int G = (int)gridDim.x;
  const BlockWalk walk(G, nblk, H);

  // X rows of block p (this wave's 32 tokens).  Every load is issued
  // unconditionally - rows past S re-read row S - 1 and are left out of the
  // block maximum and the stores - so that no branch separates the loads and
  // the compiler counts them exactly: the wait for the block being
  // processed leaves the next block's loads in flight.
  auto load = [&](BlockPos p, bf16x8(&xb)[2][KK]) __attribute__((always_inline)) {
    const int64_t tok0 = (int64_t)p.blk * BT + w * 32;
    const int64_t row0 = rm.row(p.b, p.h, 0);
#pragma unroll
    for (int tb = 0; tb < 2; ++tb) {
      const int64_t tok = min(tok0 + tb * 16 + l16, S - 1);
#pragma unroll
      for (int kk = 0; kk < KK; ++kk)
        xb[tb][kk] = __builtin_bit_cast(
            bf16x8, *reinterpret_cast<const uint4*>(x + (row0 + tok * rm.ss) * D + kk * 32 + g * 8));
    }
  };

  // rotate, block maximum, encode and store block p from its X rows
  auto process = [&](BlockPos p, const bf16x8(&xb)[2][KK], int slot) __attribute__((always_inline)) {
    const int64_t tok0 = (int64_t)p.blk * BT + w * 32;
    const int64_t row0 = rm.row(p.b, p.h, 0);  // token tok is row row0 + tok rm.ss
    f32x4 acc[2][DB];
#pragma unroll
    for (int db = 0; db < DB; ++db) {
      acc[0][db] = f32x4{0.f, 0.f, 0.f, 0.f};
      acc[1][db] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int kk = 0; kk < KK; ++kk) {
        const bf16x8 a = *reinterpret_cast<const bf16x8*>(&rt[(db * 16 + l16) * RS + kk * 32 + g * 8]);
        acc[0][db] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, xb[0][kk], acc[0][db], 0, 0, 0);
        acc[1][db] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, xb[1][kk], acc[1][db], 0, 0, 0);
      }
    }
    // round to bf16 (the rotated tensor is bf16; the hardware conversion
    // rounds to nearest even), block max over the tokens below S
    float m = 0.0f;
#pragma unroll
    for (int tb = 0; tb < 2; ++tb) {
      float mt = 0.0f;
#pragma unroll
      for (int db = 0; db < DB; ++db)
#pragma unroll
        for (int r = 0; r < 4; r += 2) {
          const bf16x2 y = {(__bf16)acc[tb][db][r], (__bf16)acc[tb][db][r + 1]};
          const uint32_t yw = __builtin_bit_cast(uint32_t, y);
          acc[tb][db][r] = bf16_lo(yw);
          acc[tb][db][r + 1] = bf16_hi(yw);
          mt = fmaxf(mt, fmaxf(fabsf(acc[tb][db][r]), fabsf(acc[tb][db][r + 1])));
        }
      if (tok0 + tb * 16 + l16 < S) m = fmaxf(m, mt);
    }
    m = wave_max(m);
    if (lane == 0) red[slot][w] = m;
    barrier_lds();
    m = red[slot][0];
#pragma unroll
    for (int i = 1; i < NW; ++i) m = fmaxf(m, red[slot][i]);
    const float s = scale_from_amax(m, 448.0f);
    uint8_t* cw = cst[w];
#pragma unroll
    for (int tb = 0; tb < 2; ++tb) {
      const int64_t tok = tok0 + tb * 16 + l16;
      float y[4 * DB];
#pragma unroll
      for (int db = 0; db < DB; ++db)
#pragma unroll
        for (int r = 0; r < 4; ++r) y[4 * db + r] = acc[tb][db][r];
      uint32_t c[DB];
      e4m3_code_words<4 * DB>(y, s, c);
#pragma unroll
      for (int db = 0; db < DB; ++db)
        *reinterpret_cast<uint32_t*>(cw + (tb * 16 + l16) * CR + db * 16 + g * 4) = c[db];
      if (tok >= S || !dbg) continue;
#pragma unroll
      for (int db = 0; db < DB; ++db) {
        const int64_t off = (row0 + tok * rm.ss) * D + db * 16 + g * 4;
        {
          // y holds bf16 values: their top halves are the bf16 bits
          const float* yd = y + 4 * db;
          const uint32_t b0 = (__float_as_uint(yd[0]) >> 16) | (__float_as_uint(yd[1]) & 0xffff0000u);
          const uint32_t b1 = (__float_as_uint(yd[2]) >> 16) | (__float_as_uint(yd[3]) & 0xffff0000u);
          *reinterpret_cast<uint2*>(dbg + off) = make_uint2(b0, b1);
        }
      }
    }
    // the wave's codes, 16 bytes per lane and store: 32 rows of D / 16
    // chunks (the LDS writes and reads of one wave are done in order)
#pragma unroll
    for (int i = 0; i < 32 * (D / 16) / 64; ++i) {
      const int c = i * 64 + lane, row = c / (D / 16), ch = c % (D / 16);
      const uint4 v = *reinterpret_cast<const uint4*>(cw + row * CR + ch * 16);
      const int64_t tok = tok0 + row;
      if (tok < S) *reinterpret_cast<uint4*>(codes + (row0 + tok * rm.ss) * D + ch * 16) = v;
    }
    if (threadIdx.x == 0) scales[((int64_t)p.b * H + p.h) * nblk + p.blk] = s;
  };

  // two register buffers of X rows, alternating: block b + grid is loaded
  // while block b is processed (past the last block the current one is
  // re-read and not processed; the exits are uniform over the workgroup:
  // they depend on the work index only).  The grid never exceeds nwork.
  bf16x8 xa[2][KK], xc[2][KK];
  int work = (int)blockIdx.x;
  BlockPos pa = walk.at(work);
  load(pa, xa);
  for (;;) {
    const BlockPos pc = walk.next(pa);
    const bool more1 = work + G < nwork;
    load(more1 ? pc : pa, xc);
    process(pa, xa, 0);
    if (!more1) break;
    const BlockPos pn = walk.next(pc);
    const bool more2 = work + 2 * G < nwork;
    load(more2 ? pn : pc, xa);
    process(pc, xc, 1);
    if (!more2) break;
    pa = pn;
    work += 2 * G;
  }
}

// Workgroups of `kernel` the GPU holds at once (per CU from the occupancy
// query, times the CUs), for persistent grids; queried once per kernel.
template <class K>
int resident_workgroups(K kernel, int threads) {
  static int resident = 0;
  if (resident == 0) {
    int dev = 0, per_cu = 0;
    hipDeviceProp_t prop;
    if (hipGetDevice(&dev) == hipSuccess && hipGetDeviceProperties(&prop, dev) == hipSuccess &&
        hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, kernel, threads, 0) == hipSuccess && per_cu > 0)
      resident = per_cu * prop.multiProcessorCount;
    else
      resident = 256;
  }
  return resident;
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
  // 16 loads of 16 bytes in flight per thread: 64 KiB per workgroup round
  constexpr int U = 16;
  if (x_dtype == FAQ_T_BF16) {
    dim3 grid(grid_chunks(per_bh, kThreads * 8 * U, 65535), (unsigned)(s.B * s.H));
    k_calibrate<uint16_t, U><<<grid, kThreads, 0, st>>>((const uint16_t*)x, rm, dsh, per_bh, (int)s.H, amax);
  } else {
    dim3 grid(grid_chunks(per_bh, kThreads * 4 * U, 65535), (unsigned)(s.B * s.H));
    k_calibrate<float, U><<<grid, kThreads, 0, st>>>((const float*)x, rm, dsh, per_bh, (int)s.H, amax);
  }
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
  // rows per workgroup and step (16 elements per thread); two steps per
  // workgroup round
  constexpr int RPB = kThreads / (D / 16);
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
  const int64_t nwork = (int64_t)nblk * s.B * s.H;
  constexpr int NT = fp8_block_threads<D, BT>();
  const int res = resident_workgroups(k_quant_fp8_block<D, BT>, NT);
  const unsigned grid = (unsigned)(nwork < res ? nwork : res);
  k_quant_fp8_block<D, BT><<<grid, NT, 0, st>>>(x, row_map(s), (int)s.H, s.S, nblk, (int)nwork, codes,
                                                       scales);
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
  const int res = resident_workgroups(k_rot_fp8_block<D, BT>, BT * 2);
  const unsigned grid = (unsigned)(nwork < res ? nwork : res);
  k_rot_fp8_block<D, BT><<<grid, BT * 2, 0, st>>>(x, rot, row_map(s), (int)s.H, s.S, nblk, (int)nwork, codes,
                                                   scales, dbg);
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
