/*
 * fa_quant.h - C ABI of the MI355X (gfx950) FA-quantization library.
 *
 * Quantize the Q/K/V activations that feed flash attention, then run
 * attention on the low-bit operands.  Modes:
 *   - INT8 per-head static, scales from min-max calibration
 *     (msModelSlim "FA 量化" page, 分支组合 / 组合 1; default QConfig on the
 *     "fa3_quant 配置说明" page, §2.1);
 *   - FP8 E4M3 per-token dynamic ("FA 量化" page, 组合 2);
 *   - MXFP4 per-block dynamic, 32 elements along head_dim sharing one E8M0
 *     exponent ("FA 量化" page, 组合 3);
 *   - learned rotation of Q and K, then FP8 E4M3 block quantization with
 *     128-token Q blocks and 256-token K/V blocks (MindIE SD "量化" page,
 *     FA量化 / 技术特点: 旋转, 块量化, FP8 Attention);
 *   - the sibling modes of the FA mode list ("FA 量化" page, 该类下的模式清单;
 *     "量化模式" page, 模式索引 / FA 量化): FP8 per-head static, INT8
 *     per-token dynamic and MXFP8 per-block dynamic.
 *
 * Conventions shared by every entry point:
 *   - Tensors are contiguous, row-major, in one of the two layouts the
 *     "量化" page (注意事项) lists for Q/K/V: BNSD [B, H, S, D] or BSND
 *     [B, S, H, D] (faq_shape.layout).  Shapes are always given as the
 *     logical (B, H, S, D); scale arrays are always indexed (b, h, s) in
 *     that order, whatever the layout of the tensor.  D must be 64 or 128.
 *   - Every tensor pointer is a DEVICE pointer, except the descriptor structs
 *     themselves (faq_shape, faq_qconfig, faq_qtensor), which live in host
 *     memory and are read during the call only.  The caller owns every
 *     buffer; the library allocates nothing and keeps no state between
 *     calls; calls on different streams may run concurrently.
 *   - `stream` is a hipStream_t (NULL = the null stream).  All work is
 *     enqueued asynchronously on it; the return value reports argument
 *     validation and launch errors, not kernel completion.
 *   - Validation happens before any HIP call: a call that returns an error
 *     other than FAQ_ERR_HIP has enqueued nothing.
 */
#ifndef FA_QUANT_H
#define FA_QUANT_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  FAQ_OK = 0,
  FAQ_ERR_INVALID_ARG = -1,     /* NULL pointer, negative size, bad enum     */
  FAQ_ERR_UNSUPPORTED = -2,     /* valid but not implemented (D, dtype, ...) */
  FAQ_ERR_CONFIG_CONFLICT = -3, /* qconfig and details both given ("fa3_quant
                                   配置说明" §2.1 constraint); raised by the
                                   Python layer, reserved here              */
  FAQ_ERR_NOT_CALIBRATED = -4,  /* static per-head without scales ("FA 量化"
                                   组合 1: calibration data is required)     */
  FAQ_ERR_SHAPE = -5,           /* inconsistent shapes between tensors       */
  FAQ_ERR_HIP = -6,             /* the HIP runtime reported an error         */
  FAQ_ERR_WORKSPACE = -7        /* workspace missing or too small            */
} faq_status;

/* Quantized data type ("fa3_quant 配置说明" §2.2 QConfig.dtype, the subset the
   FA modes use: "FA 量化" page, 该类下的模式清单).  FAQ_FLOAT means "not
   quantized" ("fa3_quant 配置说明" §2.3: an unconfigured branch): attention
   accepts it for any of Q, K and V (the branch's bf16 values stand in for
   codes); fa_quantize and the size queries reject it (there is nothing to
   quantize). */
typedef enum { FAQ_FLOAT = 0, FAQ_INT8 = 1, FAQ_FP8_E4M3 = 2, FAQ_MXFP4 = 3, FAQ_MXFP8 = 4 } faq_dtype;

/* Quantization granularity (QConfig.scope):
   PER_HEAD        one float scale per head, shared over B and S  -> float[H]
   PER_TOKEN       one float scale per (b,h,s) row of D          -> float[B,H,S]
   PER_BLOCK       MX (MXFP4, MXFP8): one E8M0 byte per 32
                   consecutive d                                  -> uint8[B,H,S,D/32]
   PER_TOKEN_BLOCK one float scale per (b,h, block_tokens rows)  -> float[B,H,ceil(S/bt)] */
typedef enum {
  FAQ_PER_HEAD = 0,
  FAQ_PER_TOKEN = 1,
  FAQ_PER_BLOCK = 2,
  FAQ_PER_TOKEN_BLOCK = 3
} faq_scope;

/* Element type of float tensors (inputs, attention output). */
typedef enum { FAQ_T_F32 = 0, FAQ_T_BF16 = 1 } faq_tdtype;

typedef struct {
  int32_t dtype;        /* faq_dtype                                         */
  int32_t scope;        /* faq_scope                                         */
  int32_t symmetric;    /* must be 1: symmetric, no offset (组合 1)           */
  int32_t method;       /* 0 = minmax (QConfig.method)                       */
  int32_t block_tokens; /* PER_TOKEN_BLOCK only: 128 (the Q block of the
                           rotate path) or 256 (its K/V block), for any
                           branch; another positive value is
                           FAQ_ERR_UNSUPPORTED, zero or negative
                           FAQ_ERR_INVALID_ARG                                */
} faq_qconfig;

/* Memory layout of a tensor with logical shape (B, H, S, D). */
typedef enum { FAQ_LAYOUT_BNSD = 0, FAQ_LAYOUT_BSND = 1 } faq_layout;

typedef struct {
  int64_t B, H, S, D;
  int64_t layout; /* faq_layout; 0 (BNSD) when zero-initialised */
} faq_shape;

/* A quantized tensor: codes and scales in device memory.
   codes:  INT8       int8 [B,H,S,D]
           FP8_E4M3   uint8 E4M3FN bit patterns [B,H,S,D]
           MXFP4      uint8 [B,H,S,D/2], element 2i in the low nibble
           MXFP8      uint8 E4M3FN bit patterns [B,H,S,D]
           FLOAT      (attention only: an unquantized branch) the bf16
                      values [B,H,S,D]; scales unused (may be NULL)
           in shape.layout (BSND: [B,S,H,.] with the same last dimension)
   scales: see faq_scope.  fa_quant_codes_bytes / fa_quant_scales_bytes give
   the sizes. */
typedef struct {
  faq_qconfig cfg;
  faq_shape shape;
  void* codes;
  void* scales;
} faq_qtensor;

/* Buffer sizes in bytes for a quantized tensor; 0 if the combination of
   config and shape is invalid or unsupported. */
size_t fa_quant_codes_bytes(const faq_qconfig* cfg, const faq_shape* shape);
size_t fa_quant_scales_bytes(const faq_qconfig* cfg, const faq_shape* shape);

/* Min-max calibration for static per-head quantization ("FA 量化" 组合 1 and
   the minmax method of "fa3_quant 配置说明" §2.2): for every head h,
     amax[h] = max(amax[h], max over b, s, d of |x[b,h,s,d]|).
   `amax` is a device float[H], read and updated in place (a running max over
   calls, so calibration can span several batches and resume from a saved
   buffer); the caller zero-fills it before the first batch. */
faq_status fa_quant_calibrate(const void* x, int32_t x_dtype, const faq_shape* shape,
                              float* amax, void* stream);

/* Per-head scales from calibrated maxima: scale[h] = fl32(amax[h] / qmax) with
   qmax 127 (INT8) or 448 (FP8 E4M3), correctly rounded; amax == 0 gives 1.
   amax and scale are device float[H] (may alias). */
faq_status fa_quant_scales_from_amax(const float* amax, int64_t H, int32_t dtype,
                                     float* scale, void* stream);

/* Quantize one branch (Q, K or V).
   x           device [B,H,S,D] of x_dtype (F32 or BF16; the rotation path
               needs BF16).
   cfg         the branch's QConfig; must equal out->cfg.
   static_scale PER_HEAD only (INT8 or FP8): device float[H] from
               fa_quant_scales_from_amax (same dtype);
               NULL -> FAQ_ERR_NOT_CALIBRATED.  Must be NULL for other scopes.
               Copied into out->scales unless it is the same pointer.
   rot         PER_TOKEN_BLOCK only, optional: device bf16 [D,D] rotation R;
               the tensor is replaced by Y = bf16_rne(X . R) before block
               quantization ("量化" page, FA量化 / 技术特点: 旋转 of Q and K
               by q_rot / k_rot).  NULL = no rotation (the V branch).
   out         shape (layout included) must equal *shape: codes are
               written in the layout of x; codes/scales must hold the sizes
               the size queries report.
   debug_rotated optional device bf16 [B,H,S,D]: receives Y when rot != NULL.
   Codes and scales are bit-exact functions of the inputs:
     scale = fl32(amax / qmax) (amax == 0 -> 1), code = round-half-even of
     fl32(x / scale) onto the target grid, saturating (INT8 clamps to
     [-128,127]; E4M3 saturates at +-448 and keeps the sign of zero);
     FP8 per-head saturates inputs beyond the calibrated range at +-448;
     MXFP4: E = clamp(floor(log2 amax) - 2, -127, 127), E8M0 byte = E + 127,
     element = E2M1(x * 2^-E) with ties to even, saturating at 6;
     MXFP8: E = clamp(floor(log2 amax) - 8, -127, 127), element =
     E4M3(x * 2^-E), ties to even, saturating at 448. */
faq_status fa_quantize(const void* x, int32_t x_dtype, const faq_shape* shape,
                       const faq_qconfig* cfg, const float* static_scale, const void* rot,
                       faq_qtensor* out, void* debug_rotated, void* stream);

/* Device workspace (bytes) fa_quant_attention needs for these operands
   (V re-laid out tile by tile with its per-tile scale data - not for INT8
   per-head V, which the kernel reads as rows - and K widened to bf16 where
   its format has no MFMA path of its own; with few queries per head -
   decode - also the partial results of the key splits); enough for causal
   and non-causal calls; at least 256 for valid operands, 0 on invalid
   operands. */
size_t fa_quant_attention_workspace_bytes(const faq_qtensor* q, const faq_qtensor* k,
                                          const faq_qtensor* v);

/* Attention on quantized operands: both Q K^T and P V run on low-bit MFMA
   operands ("FA 量化" page, 概述), output dequantized to the original
   precision ("量化" page, FA量化 / FP8 Attention).
   q, k, v     each quantized in its own configuration ("fa3_quant 配置说明"
               §2.3) - INT8 or FP8 PER_HEAD / PER_TOKEN, MXFP4 or MXFP8
               PER_BLOCK, FP8/PER_TOKEN_BLOCK (128 or 256 tokens) - or
               FLOAT (bf16, not quantized).  Every combination runs: Q and
               K of one (dtype, scope) with V of theirs or FLOAT take
               kernels specialised to that pair (INT8 scores on INT8 MFMA,
               MXFP4 on the scaled f8f6f4 MFMA); any other mix widens Q and
               K exactly to bf16 (MX rows relative to their largest block
               exponent) and scores on bf16 MFMA.  With Q, K and V all
               MXFP4 the value product also runs on the scaled f8f6f4 MFMA:
               V is re-expressed per (32-key group, 32-channel block) as
               E5M2 under one E8M0 scale, exact while a group's block
               exponents span at most 57; an element more than 57 binades
               below its group's largest exponent (so below 2^-55 of that
               group's largest |V|) is left out.  B, H, D equal; k and v
               share S.  The rows of one head of k and of v must span
               less than 4 GiB (in BSND they lie H rows apart), else
               FAQ_ERR_UNSUPPORTED.
   sm_scale    softmax scale; 0 means 1/sqrt(D).
   causal      1: key j is masked for query i when j > i (needs Sq == Skv).
   out         device [B,H,Sq,D] in q's layout, out_dtype F32 or BF16
               (bf16 = the float result rounded to nearest even).  q, k and
               v may have different layouts.
   workspace   device buffer of at least fa_quant_attention_workspace_bytes.
   Short query sets (decode: a few queries per head against a long key
   cache) split the keys across workgroups on 128-key tile boundaries and
   merge the partial results; the probability rule below makes the split
   exact up to fp32 rounding.
   Probabilities enter the PV product quantized per 128-key tile relative
   to the tile's own row maximum: int8 round(127 p w_j) or E4M3 of
   448 p w_j, with w_j the key's V scale over the tile's largest (1 when V
   has one scale per tile), round to nearest even; the key holding the
   tile maximum (p = 1) takes the code of the exact 448 w_j / 127 w_j, the
   others that of their fp32 p times it; MXFP4 / MXFP8 over 32-key groups
   in the MX modes; bf16 of p for an unquantized V.  The softmax
   denominator uses unquantized p. */
faq_status fa_quant_attention(const faq_qtensor* q, const faq_qtensor* k, const faq_qtensor* v,
                              float sm_scale, int32_t causal, void* out, int32_t out_dtype,
                              void* workspace, size_t workspace_bytes, void* stream);

/* Size of the static workspace of fa_quant_attention_static_ws, per GPU. */
#define FA_QUANT_STATIC_WORKSPACE_BYTES ((size_t)64 << 20)

/* fa_quant_attention for callers that cannot allocate device memory (code
   under HIP graph capture, tight serving loops, harnesses that forbid
   allocation): the same operation, arguments and results, without a
   workspace argument.  The kernels' workspace is a static device array of
   FA_QUANT_STATIC_WORKSPACE_BYTES (64 MiB) on each GPU the library runs on,
   held until the process ends; the call allocates nothing (no hipMalloc,
   hipFree or allocating library routine).  A call whose workspace need
   (fa_quant_attention_workspace_bytes) exceeds the array returns
   FAQ_ERR_WORKSPACE and enqueues nothing.  Every call on one GPU shares
   that GPU's array: calls that overlap on one GPU (other streams, other
   host threads) race, and the caller must serialize them; the stream must
   belong to the current device.  The array's contents between calls are
   never read (each call writes all it reads). */
faq_status fa_quant_attention_static_ws(const faq_qtensor* q, const faq_qtensor* k, const faq_qtensor* v,
                                        float sm_scale, int32_t causal, void* out, int32_t out_dtype,
                                        void* stream);

/* Static, NUL-terminated description of a status code. */
const char* fa_quant_status_string(int32_t status);

#ifdef __cplusplus
}
#endif

#endif /* FA_QUANT_H */
