// Internal launchers shared between the C ABI layer and the kernel files.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/fa_quant.h"

namespace faq {

// ---- quantization (quant.hip)
hipError_t launch_calibrate(const void* x, int x_dtype, const faq_shape& s, float* amax,
                            hipStream_t st);
hipError_t launch_scales_from_amax(const float* amax, int64_t H, float qmax, float* scale,
                                   hipStream_t st);
hipError_t launch_quant_int8_head(const void* x, int x_dtype, const faq_shape& s,
                                  const float* scale, int8_t* codes, hipStream_t st);
hipError_t launch_quant_fp8_token(const void* x, int x_dtype, const faq_shape& s,
                                  uint8_t* codes, float* scales, hipStream_t st);
hipError_t launch_quant_fp8_head(const void* x, int x_dtype, const faq_shape& s,
                                 const float* scale, uint8_t* codes, hipStream_t st);
hipError_t launch_quant_int8_token(const void* x, int x_dtype, const faq_shape& s,
                                   int8_t* codes, float* scales, hipStream_t st);
hipError_t launch_quant_mxfp8(const void* x, int x_dtype, const faq_shape& s, uint8_t* codes,
                              uint8_t* e8m0, hipStream_t st);
hipError_t launch_quant_mxfp4(const void* x, int x_dtype, const faq_shape& s, uint8_t* codes,
                              uint8_t* e8m0, hipStream_t st);
hipError_t launch_quant_fp8_block(const uint16_t* x, const faq_shape& s, int block_tokens,
                                  uint8_t* codes, float* scales, hipStream_t st);
hipError_t launch_rot_fp8_block(const uint16_t* x, const uint16_t* rot, const faq_shape& s,
                                int block_tokens, uint8_t* codes, float* scales,
                                uint16_t* debug_rotated, hipStream_t st);

// ---- attention (attention.hip)
// INT8 per-head; FP8 (per-token, token-block or per-head); MXFP4;
// INT8 per-token; MXFP8.
enum AttnMode { ATTN_INT8 = 0, ATTN_FP8 = 1, ATTN_MX = 2, ATTN_I8TOK = 3, ATTN_MX8 = 4 };

struct AttnArgs {
  int mode;
  int64_t B, H, Sq, Skv, D;
  const void* q_codes;
  const void* q_scales;
  const void* k_codes;
  const void* k_scales;
  const void* v_codes;
  const void* v_scales;
  // float scales of per-token, token-block and per-head scopes sit at
  // b * sb + h * sh + token / block
  int q_block;   // tokens per Q scale (1 = per token)
  int kv_block;  // tokens per K/V scale (1 = per token)
  int64_t q_sb, q_sh, kv_sb, kv_sh;
  float sm_scale;
  int causal;
  void* out;
  int out_bf16;
  void* ws;
};

size_t attn_workspace_bytes(int mode, int64_t B, int64_t H, int64_t Skv, int64_t D);
hipError_t launch_attention(const AttnArgs& a, hipStream_t st);

}  // namespace faq
