// Internal launchers shared between the C ABI layer and the kernel files.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/fa_quant.h"

namespace faq {

// Row (in units of D elements) of token (b, h, s) of a contiguous tensor
// in either layout: BNSD rows are (b H + h) S + s, BSND rows (b S + s) H + h.
struct RowMap {
  int64_t sb, sh, ss;
  int ident;  // BNSD: logical row index == memory row index
  __host__ __device__ int64_t row(int64_t b, int64_t h, int64_t s) const { return b * sb + h * sh + s * ss; }
};

inline RowMap row_map(const faq_shape& s) {
  if (s.layout == FAQ_LAYOUT_BSND) return RowMap{s.S * s.H, 1, s.H, s.H == 1 ? 1 : 0};
  return RowMap{s.H * s.S, s.S, 1, 1};
}

// ---- quantization (quant.hip)
hipError_t launch_calibrate(const void* x, int x_dtype, const faq_shape& s, float* amax,
                            hipStream_t st);
// Every quantizer reads x and writes its codes in the layout of `s`; scales
// are indexed (b, h, s).
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
// Score modes, from the configuration Q and K share: INT8 per-head, INT8
// per-token, FP8 with per-token K scales, FP8 with one K scale per 128-key
// tile (per-head, token blocks), MXFP4, MXFP8, unquantized bf16; and the
// general mode for any other Q/K/V combination (Q and K of any formats
// widened exactly to bf16, per-query and per-key scale factors).
enum QkMode { QK_I8H = 0, QK_I8T, QK_F8T, QK_F8C, QK_MX4, QK_MX8, QK_BF, QK_GEN };
// Element formats of one branch for the general score mode.
enum BranchFmt { FMT_BF16 = 0, FMT_INT8, FMT_FP8, FMT_MX4, FMT_MX8 };
// Value modes, from V's configuration: INT8 per-head, INT8 per-token, FP8
// with per-token V scales (folded into P), FP8 with one V scale per tile,
// MXFP4, MXFP8, unquantized bf16.
enum PvMode { PV_I8H = 0, PV_I8T, PV_F8W, PV_F8C, PV_MX4, PV_MX8, PV_BF };

struct AttnArgs {
  int qk, pv;
  int qfmt, kfmt;  // BranchFmt of Q and K (general score mode)
  int64_t B, H, Sq, Skv, D;
  const void* q_codes;
  const void* q_scales;
  const void* k_codes;
  const void* k_scales;
  const void* v_codes;
  const void* v_scales;
  // float scales of per-token, token-block and per-head scopes sit at
  // b * sb + h * sh + token / block
  int q_block, k_block, v_block;
  int64_t q_sb, q_sh, k_sb, k_sh, v_sb, v_sh;
  RowMap qmap, kmap, vmap;  // memory rows of Q, K, V (the output takes Q's layout)
  float sm_scale;
  int causal;
  void* out;
  int out_bf16;
  void* ws;
};

// Pairs with kernels: Q, K and V of one configuration, or either side
// unquantized.
bool attn_pair_supported(int qk, int pv);
// Workspace of one call; it depends on Sq and causal through the key
// splits of short query sets (their partial results live there too).
size_t attn_workspace_bytes(int qk, int pv, int64_t B, int64_t H, int64_t Sq, int64_t Skv, int64_t D, int causal);
hipError_t launch_attention(const AttnArgs& a, hipStream_t st);

// The common body of the attention entry points (api.hip): validation
// before any HIP call, the workspace check, dispatch.  `fn` names the entry
// point in log lines.
faq_status attention_entry(const faq_qtensor* q, const faq_qtensor* k, const faq_qtensor* v, float sm_scale,
                           int32_t causal, void* out, int32_t out_dtype, void* workspace, size_t workspace_bytes,
                           void* stream, const char* fn);

}  // namespace faq
