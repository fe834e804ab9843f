// Test-only probes (built into a separate library, never into libfaquant):
// single-instruction kernels that pin the lane layout of the MFMA operands
// and scales, and the rounding of the hardware conversion instructions,
// against CPU references in the test suite.  Every kernel runs one wave on
// fixed-size buffers.

#include "common.h"

namespace {

// C[16][16] = A[16][64] . Bt[16][64]^T with v_mfma_i32_16x16x64_i8.
// Assumed layout: lane (i = l%16, g = l/16) holds A[i][16g .. 16g+15] and
// Bt[i][16g .. 16g+15]; C[4g + r][i] lands in accumulator r.
__global__ void k_probe_i8(const int8_t* A, const int8_t* Bt, int32_t* C) {
  const int l = threadIdx.x, i = l & 15, g = l >> 4;
  const uint4 a = *reinterpret_cast<const uint4*>(A + i * 64 + 16 * g);
  const uint4 b = *reinterpret_cast<const uint4*>(Bt + i * 64 + 16 * g);
  const i32x4 av = {(int)a.x, (int)a.y, (int)a.z, (int)a.w};
  const i32x4 bv = {(int)b.x, (int)b.y, (int)b.z, (int)b.w};
  const i32x4 c = __builtin_amdgcn_mfma_i32_16x16x64_i8(av, bv, i32x4{0, 0, 0, 0}, 0, 0, 0);
  for (int r = 0; r < 4; ++r) C[(4 * g + r) * 16 + i] = c[r];
}

// C = A[16][128] . Bt[16][128]^T with the f8f6f4 MFMA; element formats fa, fb
// (0 E4M3, 1 E5M2, 4 E2M1); row bytes 128 (8-bit) or 64 (4-bit).  Scales
// (E8M0 bytes) sa[i][g], sb[i][g] for row i and 32-element block g when
// `scaled`; lane (i, g) holds elements 32g..32g+31 of its row.
template <int FA, int FB>
__global__ void k_probe_f8f6f4(const uint8_t* A, const uint8_t* Bt, const uint8_t* sa,
                               const uint8_t* sb, int scaled, float* C) {
  const int l = threadIdx.x, i = l & 15, g = l >> 4;
  constexpr int RA = FA == 4 ? 64 : 128, RB = FB == 4 ? 64 : 128;
  i32x8 av = {0, 0, 0, 0, 0, 0, 0, 0}, bv = {0, 0, 0, 0, 0, 0, 0, 0};
  {
    const uint4* p = reinterpret_cast<const uint4*>(A + i * RA + g * (RA / 4));
    const uint4 x = p[0];
    av[0] = x.x; av[1] = x.y; av[2] = x.z; av[3] = x.w;
    if (FA != 4) { const uint4 y = p[1]; av[4] = y.x; av[5] = y.y; av[6] = y.z; av[7] = y.w; }
  }
  {
    const uint4* p = reinterpret_cast<const uint4*>(Bt + i * RB + g * (RB / 4));
    const uint4 x = p[0];
    bv[0] = x.x; bv[1] = x.y; bv[2] = x.z; bv[3] = x.w;
    if (FB != 4) { const uint4 y = p[1]; bv[4] = y.x; bv[5] = y.y; bv[6] = y.z; bv[7] = y.w; }
  }
  f32x4 c;
  if (scaled) {
    c = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(av, bv, f32x4{0.f, 0.f, 0.f, 0.f}, FA, FB, 0,
                                                         (int)sa[i * 4 + g], 0, (int)sb[i * 4 + g]);
  } else {
    c = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(av, bv, f32x4{0.f, 0.f, 0.f, 0.f}, FA, FB, 0, 0,
                                                         0, 0);
  }
  for (int r = 0; r < 4; ++r) C[(4 * g + r) * 16 + i] = c[r];
}

// C = A[16][32] . Bt[16][32]^T with v_mfma_f32_16x16x32_bf16; lane (i, g)
// holds elements 8g..8g+7.
__global__ void k_probe_bf16(const uint16_t* A, const uint16_t* Bt, float* C) {
  const int l = threadIdx.x, i = l & 15, g = l >> 4;
  const uint4 a = *reinterpret_cast<const uint4*>(A + i * 32 + 8 * g);
  const uint4 b = *reinterpret_cast<const uint4*>(Bt + i * 32 + 8 * g);
  const f32x4 c = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a),
                                                          __builtin_bit_cast(bf16x8, b),
                                                          f32x4{0.f, 0.f, 0.f, 0.f}, 0, 0, 0);
  for (int r = 0; r < 4; ++r) C[(4 * g + r) * 16 + i] = c[r];
}

// Conversions of n floats (n even): hardware E4M3 / E5M2 packs, the
// hardware scaled FP4 pack (with scale `fp4_scale`), and the software E4M3
// encoder, one output byte (or nibble byte) per input.
__global__ void k_probe_cvt(const float* x, int n, float fp4_scale, uint8_t* hw_e4m3, uint8_t* hw_e5m2,
                            uint8_t* hw_fp4, uint8_t* sw_e4m3) {
  const int i = 2 * ((int)(blockIdx.x * blockDim.x + threadIdx.x));
  if (i + 1 >= n + 1) return;
  const float a = x[i], b = (i + 1 < n) ? x[i + 1] : 0.0f;
  const int e4 = __builtin_amdgcn_cvt_pk_fp8_f32(a, b, 0, false);
  const int e5 = __builtin_amdgcn_cvt_pk_bf8_f32(a, b, 0, false);
  const unsigned f4 = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(0u, a, b, fp4_scale, 0);
  hw_e4m3[i] = (uint8_t)(e4 & 0xff);
  hw_e5m2[i] = (uint8_t)(e5 & 0xff);
  hw_fp4[i] = (uint8_t)(f4 & 0xf);
  sw_e4m3[i] = (uint8_t)enc_e4m3(a);
  if (i + 1 < n) {
    hw_e4m3[i + 1] = (uint8_t)((e4 >> 8) & 0xff);
    hw_e5m2[i + 1] = (uint8_t)((e5 >> 8) & 0xff);
    hw_fp4[i + 1] = (uint8_t)((f4 >> 4) & 0xf);
    sw_e4m3[i + 1] = (uint8_t)enc_e4m3(b);
  }
}

}  // namespace

extern "C" {

int faq_probe_mfma_i8(const int8_t* A, const int8_t* Bt, int32_t* C) {
  k_probe_i8<<<1, 64>>>(A, Bt, C);
  return (int)hipDeviceSynchronize();
}

int faq_probe_mfma_f8f6f4(const uint8_t* A, const uint8_t* Bt, const uint8_t* sa, const uint8_t* sb,
                          int fa, int fb, int scaled, float* C) {
#define FAQ_PROBE_CASE(X, Y)                                        \
  if (fa == X && fb == Y) {                                         \
    k_probe_f8f6f4<X, Y><<<1, 64>>>(A, Bt, sa, sb, scaled, C);      \
    return (int)hipDeviceSynchronize();                             \
  }
  FAQ_PROBE_CASE(0, 0)
  FAQ_PROBE_CASE(1, 1)
  FAQ_PROBE_CASE(4, 4)
  FAQ_PROBE_CASE(1, 4)
  FAQ_PROBE_CASE(0, 4)
#undef FAQ_PROBE_CASE
  return -1;
}

int faq_probe_mfma_bf16(const uint16_t* A, const uint16_t* Bt, float* C) {
  k_probe_bf16<<<1, 64>>>(A, Bt, C);
  return (int)hipDeviceSynchronize();
}

int faq_probe_cvt(const float* x, int n, float fp4_scale, uint8_t* hw_e4m3, uint8_t* hw_e5m2,
                  uint8_t* hw_fp4, uint8_t* sw_e4m3) {
  const int pairs = (n + 1) / 2;
  k_probe_cvt<<<(pairs + 255) / 256, 256>>>(x, n, fp4_scale, hw_e4m3, hw_e5m2, hw_fp4, sw_e4m3);
  return (int)hipDeviceSynchronize();
}

}  // extern "C"

namespace {
// C = A[16][32] . Bt[16][32]^T with the 16x16x32 fp8 MFMA (E4M3 x E4M3);
// lane (i, g) holds bytes 8g..8g+7 of its row.
__global__ void k_probe_fp8_k32(const uint8_t* A, const uint8_t* Bt, float* C) {
  const int l = threadIdx.x, i = l & 15, g = l >> 4;
  const long a = *reinterpret_cast<const long*>(A + i * 32 + 8 * g);
  const long b = *reinterpret_cast<const long*>(Bt + i * 32 + 8 * g);
  const f32x4 c = __builtin_amdgcn_mfma_f32_16x16x32_fp8_fp8(a, b, f32x4{0.f, 0.f, 0.f, 0.f}, 0, 0, 0);
  for (int r = 0; r < 4; ++r) C[(4 * g + r) * 16 + i] = c[r];
}
}  // namespace

extern "C" int faq_probe_mfma_fp8_k32(const uint8_t* A, const uint8_t* Bt, float* C) {
  k_probe_fp8_k32<<<1, 64>>>(A, Bt, C);
  return (int)hipDeviceSynchronize();
}

namespace {
// Up-conversions used by the attention kernels, one input word per thread:
// bf16 pairs of the two low / two high E4M3 bytes (scale 1), and the bf16
// pair of the two low E2M1 nibbles times `fp4_scale`.
__global__ void k_probe_cvt_up(const uint32_t* w, int n, float fp4_scale, uint32_t* e4_lo, uint32_t* e4_hi,
                               uint32_t* f4) {
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= n) return;
  e4_lo[i] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8((int)w[i], 1.0f, false));
  e4_hi[i] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8((int)w[i], 1.0f, true));
  f4[i] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w[i], fp4_scale, 0));
}
}  // namespace

extern "C" int faq_probe_cvt_up(const uint32_t* w, int n, float fp4_scale, uint32_t* e4_lo, uint32_t* e4_hi,
                                uint32_t* f4) {
  k_probe_cvt_up<<<(n + 255) / 256, 256>>>(w, n, fp4_scale, e4_lo, e4_hi, f4);
  return (int)hipDeviceSynchronize();
}

namespace {
// global_load_lds_dwordx4: each lane's 16 source bytes land at the LDS
// address given to the instruction plus 16 * lane.  One wave copies 64
// chunks src[perm[lane]] into bytes 1024..2047 of a zeroed 2 KiB buffer,
// which is then written out whole.
__global__ void k_probe_gll(const uint8_t* src, const int* perm, uint8_t* out) {
  __shared__ __attribute__((aligned(16))) uint8_t buf[2048];
  const int lane = threadIdx.x;
  for (int i = lane; i < 512; i += 64) reinterpret_cast<uint32_t*>(buf)[i] = 0u;
  __syncthreads();
  __builtin_amdgcn_global_load_lds((const __attribute__((address_space(1))) void*)(src + perm[lane] * 16),
                                   (__attribute__((address_space(3))) void*)(buf + 1024), 16, 0, 0);
  __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0)
  __syncthreads();
  for (int i = lane; i < 512; i += 64) reinterpret_cast<uint32_t*>(out)[i] = reinterpret_cast<uint32_t*>(buf)[i];
}
}  // namespace

// src: 1024 bytes; perm: 64 ints in [0, 64); out: 2048 bytes.
extern "C" int faq_probe_global_load_lds(const uint8_t* src, const int* perm, uint8_t* out) {
  k_probe_gll<<<1, 64>>>(src, perm, out);
  return (int)hipDeviceSynchronize();
}

namespace {
// ds_read_b64_tr_b8: 1 KiB of src in LDS; lane l reads through the
// transposing instruction at byte offset offs[l] (a multiple of 8, at most
// 1016) and writes its 8 bytes to out[8 l ..].
__global__ void k_probe_lds_tr8(const uint8_t* src, const int* offs, uint8_t* out) {
  __shared__ __attribute__((aligned(16))) uint8_t buf[1024];
  const int lane = threadIdx.x;
  for (int i = lane; i < 256; i += 64) reinterpret_cast<uint32_t*>(buf)[i] = reinterpret_cast<const uint32_t*>(src)[i];
  __syncthreads();
  typedef int v2i __attribute__((ext_vector_type(2)));
  const v2i v = __builtin_amdgcn_ds_read_tr8_b64_v2i32((__attribute__((address_space(3))) v2i*)(buf + offs[lane]));
  reinterpret_cast<uint32_t*>(out)[2 * lane] = (uint32_t)v.x;
  reinterpret_cast<uint32_t*>(out)[2 * lane + 1] = (uint32_t)v.y;
}
}  // namespace

// src: 1024 bytes; offs: 64 ints, multiples of 8 in [0, 1016]; out: 512 bytes.
extern "C" int faq_probe_lds_tr8(const uint8_t* src, const int* offs, uint8_t* out) {
  k_probe_lds_tr8<<<1, 64>>>(src, offs, out);
  return (int)hipDeviceSynchronize();
}

namespace {
// v_cvt_pk_u8_f32 on n floats, one byte each (byte 0 of a zero word).
__global__ void k_probe_cvt_u8(const float* x, int n, uint8_t* out) {
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) out[i] = (uint8_t)(__builtin_amdgcn_cvt_pk_u8_f32(x[i], 0, 0u) & 0xffu);
}
}  // namespace

extern "C" int faq_probe_cvt_u8(const float* x, int n, uint8_t* out) {
  k_probe_cvt_u8<<<(n + 255) / 256, 256>>>(x, n, out);
  return (int)hipDeviceSynchronize();
}

namespace {
// 32x32 MFMA shapes.  Assumed layout: lane (i = l%32, h = l/32) holds row i
// of A and of Bt at K elements [K/2 h, K/2 h + K/2) of the instruction's K;
// C[8(r/4) + 4h + r%4][i] lands in accumulator r (r = 0..15).
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef int i32x16 __attribute__((ext_vector_type(16)));

// v_mfma_f32_32x32x16_bf16: A, Bt [32][16] bf16.
__global__ void k_probe_mfma32_bf16(const uint16_t* A, const uint16_t* Bt, float* C) {
  const int l = threadIdx.x, i = l & 31, h = l >> 5;
  const uint4 a = *reinterpret_cast<const uint4*>(A + i * 16 + 8 * h);
  const uint4 b = *reinterpret_cast<const uint4*>(Bt + i * 16 + 8 * h);
  f32x16 c = {};
  c = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a), __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
  for (int r = 0; r < 16; ++r) C[(8 * (r / 4) + 4 * h + r % 4) * 32 + i] = c[r];
}

// v_mfma_i32_32x32x32_i8: A, Bt [32][32] int8.
__global__ void k_probe_mfma32_i8(const int8_t* A, const int8_t* Bt, int32_t* C) {
  const int l = threadIdx.x, i = l & 31, h = l >> 5;
  const uint4 a = *reinterpret_cast<const uint4*>(A + i * 32 + 16 * h);
  const uint4 b = *reinterpret_cast<const uint4*>(Bt + i * 32 + 16 * h);
  i32x16 c = {};
  c = __builtin_amdgcn_mfma_i32_32x32x32_i8(i32x4{(int)a.x, (int)a.y, (int)a.z, (int)a.w},
                                            i32x4{(int)b.x, (int)b.y, (int)b.z, (int)b.w}, c, 0, 0, 0);
  for (int r = 0; r < 16; ++r) C[(8 * (r / 4) + 4 * h + r % 4) * 32 + i] = c[r];
}

// v_mfma_scale_f32_32x32x64_f8f6f4 with E2M1 operands: A, Bt [32][32] bytes
// (64 elements per row, element 2k in the low nibble of byte k); E8M0 scales
// sa, sb [32][2] for row i and 32-element block h.
__global__ void k_probe_mfma32_fp4(const uint8_t* A, const uint8_t* Bt, const uint8_t* sa, const uint8_t* sb,
                                   float* C) {
  const int l = threadIdx.x, i = l & 31, h = l >> 5;
  const uint4 a = *reinterpret_cast<const uint4*>(A + i * 32 + 16 * h);
  const uint4 b = *reinterpret_cast<const uint4*>(Bt + i * 32 + 16 * h);
  const i32x8 av = {(int)a.x, (int)a.y, (int)a.z, (int)a.w, 0, 0, 0, 0};
  const i32x8 bv = {(int)b.x, (int)b.y, (int)b.z, (int)b.w, 0, 0, 0, 0};
  f32x16 c = {};
  c = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(av, bv, c, 4, 4, 0, (int)sa[i * 2 + h], 0, (int)sb[i * 2 + h]);
  for (int r = 0; r < 16; ++r) C[(8 * (r / 4) + 4 * h + r % 4) * 32 + i] = c[r];
}
}  // namespace

namespace {
// v_mfma_f32_32x32x64_f8f6f4 with E4M3 operands (no block scales): A, Bt
// [32][64] bytes; lane (i, h) holds bytes 32h .. 32h + 31 of row i of each.
// The hardware's K numbering of those 32 bytes does not matter as long as
// A and B use the same one, which this probe checks.
__global__ void k_probe_mfma32_fp8(const uint8_t* A, const uint8_t* Bt, float* C) {
  const int l = threadIdx.x, i = l & 31, h = l >> 5;
  const uint4* pa = reinterpret_cast<const uint4*>(A + i * 64 + 32 * h);
  const uint4* pb = reinterpret_cast<const uint4*>(Bt + i * 64 + 32 * h);
  const uint4 a0 = pa[0], a1 = pa[1], b0 = pb[0], b1 = pb[1];
  const i32x8 av = {(int)a0.x, (int)a0.y, (int)a0.z, (int)a0.w, (int)a1.x, (int)a1.y, (int)a1.z, (int)a1.w};
  const i32x8 bv = {(int)b0.x, (int)b0.y, (int)b0.z, (int)b0.w, (int)b1.x, (int)b1.y, (int)b1.z, (int)b1.w};
  f32x16 c = {};
  c = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(av, bv, c, 0, 0, 0, 0, 0, 0);
  for (int r = 0; r < 16; ++r) C[(8 * (r / 4) + 4 * h + r % 4) * 32 + i] = c[r];
}
}  // namespace

extern "C" int faq_probe_mfma32_fp8(const uint8_t* A, const uint8_t* Bt, float* C) {
  k_probe_mfma32_fp8<<<1, 64>>>(A, Bt, C);
  return (int)hipDeviceSynchronize();
}

extern "C" int faq_probe_mfma32_bf16(const uint16_t* A, const uint16_t* Bt, float* C) {
  k_probe_mfma32_bf16<<<1, 64>>>(A, Bt, C);
  return (int)hipDeviceSynchronize();
}

extern "C" int faq_probe_mfma32_i8(const int8_t* A, const int8_t* Bt, int32_t* C) {
  k_probe_mfma32_i8<<<1, 64>>>(A, Bt, C);
  return (int)hipDeviceSynchronize();
}

extern "C" int faq_probe_mfma32_fp4(const uint8_t* A, const uint8_t* Bt, const uint8_t* sa, const uint8_t* sb,
                                    float* C) {
  k_probe_mfma32_fp4<<<1, 64>>>(A, Bt, sa, sb, C);
  return (int)hipDeviceSynchronize();
}

namespace {
// v_mfma_scale_f32_32x32x64_f8f6f4 with E5M2 A and E2M1 B (the MXFP4 value
// product): A [32][64] bytes, lane (i, h) holds bytes 32h .. 32h + 31 of
// row i; Bt [32][32] bytes (64 elements per row, element 2k in the low
// nibble of byte k), lane (i, h) holds elements 32h .. 32h + 31; E8M0
// scales sa, sb [32][2] for row i and lane half h.
__global__ void k_probe_mfma32_bf8_fp4(const uint8_t* A, const uint8_t* Bt, const uint8_t* sa, const uint8_t* sb,
                                       float* C) {
  const int l = threadIdx.x, i = l & 31, h = l >> 5;
  const uint4* pa = reinterpret_cast<const uint4*>(A + i * 64 + 32 * h);
  const uint4 a0 = pa[0], a1 = pa[1];
  const uint4 b = *reinterpret_cast<const uint4*>(Bt + i * 32 + 16 * h);
  const i32x8 av = {(int)a0.x, (int)a0.y, (int)a0.z, (int)a0.w, (int)a1.x, (int)a1.y, (int)a1.z, (int)a1.w};
  const i32x8 bv = {(int)b.x, (int)b.y, (int)b.z, (int)b.w, 0, 0, 0, 0};
  f32x16 c = {};
  c = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(av, bv, c, 1, 4, 0, (int)sa[i * 2 + h], 0, (int)sb[i * 2 + h]);
  for (int r = 0; r < 16; ++r) C[(8 * (r / 4) + 4 * h + r % 4) * 32 + i] = c[r];
}
}  // namespace

extern "C" int faq_probe_mfma32_bf8_fp4(const uint8_t* A, const uint8_t* Bt, const uint8_t* sa, const uint8_t* sb,
                                        float* C) {
  k_probe_mfma32_bf8_fp4<<<1, 64>>>(A, Bt, sa, sb, C);
  return (int)hipDeviceSynchronize();
}

namespace {
// LDS read pattern: a 16 KiB LDS buffer holds word i = i * 2654435761 (mod
// 2^32); each of the 64 lanes reads W bytes at byte offset offs[lane],
// `reps` times (the address is made opaque per repetition, so every
// repetition issues its own ds_read), and writes the wrapped sum of its
// words.  Under SQ_INSTS_LDS / SQ_LDS_BANK_CONFLICT each launch gives the
// bank-conflict cycles of one access pattern.
struct LdsOffs {
  int v[64];
};
template <int W>
__global__ void k_probe_lds_read(const LdsOffs offs, int reps, uint32_t* out) {
  __shared__ __attribute__((aligned(16))) uint32_t buf[4096];
  const int lane = threadIdx.x;
  for (int i = lane; i < 4096; i += 64) buf[i] = (uint32_t)i * 2654435761u;
  __syncthreads();
  int off = offs.v[lane];
  uint32_t acc[W / 4] = {};
  for (int r = 0; r < reps; ++r) {
    asm volatile("" : "+v"(off));
    const uint8_t* p = reinterpret_cast<const uint8_t*>(buf) + off;
    if constexpr (W == 16) {
      const uint4 v = *reinterpret_cast<const uint4*>(p);
      acc[0] += v.x; acc[1] += v.y; acc[2] += v.z; acc[3] += v.w;
    } else if constexpr (W == 8) {
      const uint2 v = *reinterpret_cast<const uint2*>(p);
      acc[0] += v.x; acc[1] += v.y;
    } else {
      acc[0] += *reinterpret_cast<const uint32_t*>(p);
    }
  }
  for (int k = 0; k < W / 4; ++k) out[lane * (W / 4) + k] = acc[k];
}
}  // namespace

// offs: 64 host ints, multiples of width in [0, 16384 - width]; width 4, 8
// or 16; reps >= 0; out: 64 * width / 4 device words.  -1 on bad arguments.
extern "C" int faq_probe_lds_read(const int* offs, int width, int reps, uint32_t* out) {
  if (!offs || !out || reps < 0 || !(width == 4 || width == 8 || width == 16)) return -1;
  LdsOffs o;
  for (int i = 0; i < 64; ++i) {
    if (offs[i] < 0 || offs[i] > 16384 - width || offs[i] % width) return -1;
    o.v[i] = offs[i];
  }
  if (width == 16) k_probe_lds_read<16><<<1, 64>>>(o, reps, out);
  else if (width == 8) k_probe_lds_read<8><<<1, 64>>>(o, reps, out);
  else k_probe_lds_read<4><<<1, 64>>>(o, reps, out);
  return (int)hipDeviceSynchronize();
}

namespace {
// The same MFMA with an accumulator input: C = Cin + A . Bt^T, Cin and C
// [32][32] floats in the output layout above.
__global__ void k_probe_mfma32_fp8_acc(const uint8_t* A, const uint8_t* Bt, const float* Cin, float* C) {
  const int l = threadIdx.x, i = l & 31, h = l >> 5;
  const uint4* pa = reinterpret_cast<const uint4*>(A + i * 64 + 32 * h);
  const uint4* pb = reinterpret_cast<const uint4*>(Bt + i * 64 + 32 * h);
  const uint4 a0 = pa[0], a1 = pa[1], b0 = pb[0], b1 = pb[1];
  const i32x8 av = {(int)a0.x, (int)a0.y, (int)a0.z, (int)a0.w, (int)a1.x, (int)a1.y, (int)a1.z, (int)a1.w};
  const i32x8 bv = {(int)b0.x, (int)b0.y, (int)b0.z, (int)b0.w, (int)b1.x, (int)b1.y, (int)b1.z, (int)b1.w};
  f32x16 c;
  for (int r = 0; r < 16; ++r) c[r] = Cin[(8 * (r / 4) + 4 * h + r % 4) * 32 + i];
  c = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(av, bv, c, 0, 0, 0, 0, 0, 0);
  for (int r = 0; r < 16; ++r) C[(8 * (r / 4) + 4 * h + r % 4) * 32 + i] = c[r];
}
}  // namespace

extern "C" int faq_probe_mfma32_fp8_acc(const uint8_t* A, const uint8_t* Bt, const float* Cin, float* C) {
  k_probe_mfma32_fp8_acc<<<1, 64>>>(A, Bt, Cin, C);
  return (int)hipDeviceSynchronize();
}
