// C ABI entry points: argument validation (host only, before any HIP call),
// size queries and kernel dispatch.

#include <math.h>
#include <stdio.h>
#include <stdlib.h>

#include "launch.h"

using namespace faq;

namespace {

bool log_enabled() {
  static const int on = [] {
    const char* e = getenv("FAQ_LOG");
    return (e && *e && *e != '0') ? 1 : 0;
  }();
  return on != 0;
}

faq_status fail(faq_status st, const char* fn, const char* why) {
  if (log_enabled()) fprintf(stderr, "[faquant] %s: %s (%s)\n", fn, why, fa_quant_status_string(st));
  return st;
}

faq_status hip_status(hipError_t e, const char* fn) {
  if (e == hipSuccess) return FAQ_OK;
  if (log_enabled()) fprintf(stderr, "[faquant] %s: HIP error %s\n", fn, hipGetErrorString(e));
  return FAQ_ERR_HIP;
}

// Non-negative sizes, a known layout, and rows (B H S) that index in 32 bits.
bool shape_ok(const faq_shape* s) {
  return s && s->B >= 0 && s->H >= 0 && s->S >= 0 && s->D >= 0 &&
         (s->layout == FAQ_LAYOUT_BNSD || s->layout == FAQ_LAYOUT_BSND) &&
         (s->H == 0 || s->S == 0 || s->B <= (int64_t)INT32_MAX / s->H / s->S);
}

bool d_supported(int64_t D) { return D == 64 || D == 128; }

int64_t numel(const faq_shape& s) { return s.B * s.H * s.S * s.D; }

bool same_shape(const faq_shape& a, const faq_shape& b) {
  return a.B == b.B && a.H == b.H && a.S == b.S && a.D == b.D && a.layout == b.layout;
}

bool same_cfg(const faq_qconfig& a, const faq_qconfig& b) {
  return a.dtype == b.dtype && a.scope == b.scope && a.symmetric == b.symmetric &&
         a.method == b.method && (a.scope != FAQ_PER_TOKEN_BLOCK || a.block_tokens == b.block_tokens);
}

// The (dtype, scope) pairs of the FA modes implemented here: per-head
// static INT8/FP8, per-token dynamic INT8/FP8, per-block MXFP4/MXFP8, and
// FP8 token blocks of the rotate path.
faq_status check_cfg(const faq_qconfig* c) {
  if (!c) return FAQ_ERR_INVALID_ARG;
  if (c->dtype < FAQ_FLOAT || c->dtype > FAQ_MXFP8) return FAQ_ERR_INVALID_ARG;
  if (c->scope < FAQ_PER_HEAD || c->scope > FAQ_PER_TOKEN_BLOCK) return FAQ_ERR_INVALID_ARG;
  if (c->symmetric != 1 || c->method != 0) return FAQ_ERR_UNSUPPORTED;
  if ((c->dtype == FAQ_INT8 || c->dtype == FAQ_FP8_E4M3) &&
      (c->scope == FAQ_PER_HEAD || c->scope == FAQ_PER_TOKEN))
    return FAQ_OK;
  if ((c->dtype == FAQ_MXFP4 || c->dtype == FAQ_MXFP8) && c->scope == FAQ_PER_BLOCK) return FAQ_OK;
  if (c->dtype == FAQ_FP8_E4M3 && c->scope == FAQ_PER_TOKEN_BLOCK) {
    if (c->block_tokens == 128 || c->block_tokens == 256) return FAQ_OK;
    return c->block_tokens > 0 ? FAQ_ERR_UNSUPPORTED : FAQ_ERR_INVALID_ARG;
  }
  return FAQ_ERR_UNSUPPORTED;
}

size_t codes_bytes(const faq_qconfig& c, const faq_shape& s) {
  const size_t n = (size_t)numel(s);
  return c.dtype == FAQ_MXFP4 ? n / 2 : n;
}

size_t scales_bytes(const faq_qconfig& c, const faq_shape& s) {
  switch (c.scope) {
    case FAQ_PER_HEAD: return (size_t)s.H * 4;
    case FAQ_PER_TOKEN: return (size_t)(s.B * s.H * s.S) * 4;
    case FAQ_PER_BLOCK: return (size_t)(s.B * s.H * s.S) * (size_t)(s.D / 32);
    default: return (size_t)(s.B * s.H * ((s.S + c.block_tokens - 1) / c.block_tokens)) * 4;
  }
}

}  // namespace

extern "C" {

const char* fa_quant_status_string(int32_t st) {
  switch (st) {
    case FAQ_OK: return "ok";
    case FAQ_ERR_INVALID_ARG: return "invalid argument";
    case FAQ_ERR_UNSUPPORTED: return "unsupported configuration";
    case FAQ_ERR_CONFIG_CONFLICT: return "qconfig and details are mutually exclusive";
    case FAQ_ERR_NOT_CALIBRATED: return "static per-head quantization needs calibrated scales";
    case FAQ_ERR_SHAPE: return "inconsistent shapes";
    case FAQ_ERR_HIP: return "HIP runtime error";
    case FAQ_ERR_WORKSPACE: return "workspace missing or too small";
    default: return "unknown status";
  }
}

size_t fa_quant_codes_bytes(const faq_qconfig* cfg, const faq_shape* shape) {
  if (check_cfg(cfg) != FAQ_OK || !shape_ok(shape) || !d_supported(shape->D)) return 0;
  return codes_bytes(*cfg, *shape);
}

size_t fa_quant_scales_bytes(const faq_qconfig* cfg, const faq_shape* shape) {
  if (check_cfg(cfg) != FAQ_OK || !shape_ok(shape) || !d_supported(shape->D)) return 0;
  return scales_bytes(*cfg, *shape);
}

faq_status fa_quant_calibrate(const void* x, int32_t x_dtype, const faq_shape* shape, float* amax,
                              void* stream) {
  static const char* fn = "fa_quant_calibrate";
  if (!shape_ok(shape)) return fail(FAQ_ERR_INVALID_ARG, fn, "shape");
  if (x_dtype != FAQ_T_F32 && x_dtype != FAQ_T_BF16) return fail(FAQ_ERR_INVALID_ARG, fn, "x_dtype");
  if (!d_supported(shape->D)) return fail(FAQ_ERR_UNSUPPORTED, fn, "head_dim must be 64 or 128");
  if (shape->H > 0 && !amax) return fail(FAQ_ERR_INVALID_ARG, fn, "amax is NULL");
  if (numel(*shape) == 0) return FAQ_OK;
  if (!x) return fail(FAQ_ERR_INVALID_ARG, fn, "x is NULL");
  return hip_status(launch_calibrate(x, x_dtype, *shape, amax, (hipStream_t)stream), fn);
}

faq_status fa_quant_scales_from_amax(const float* amax, int64_t H, int32_t dtype, float* scale,
                                     void* stream) {
  static const char* fn = "fa_quant_scales_from_amax";
  if (H < 0) return fail(FAQ_ERR_INVALID_ARG, fn, "H < 0");
  float qmax;
  if (dtype == FAQ_INT8) qmax = 127.0f;
  else if (dtype == FAQ_FP8_E4M3) qmax = 448.0f;
  else return fail(FAQ_ERR_UNSUPPORTED, fn, "dtype has no per-head static scale");
  if (H == 0) return FAQ_OK;
  if (!amax || !scale) return fail(FAQ_ERR_INVALID_ARG, fn, "NULL pointer");
  return hip_status(launch_scales_from_amax(amax, H, qmax, scale, (hipStream_t)stream), fn);
}

faq_status fa_quantize(const void* x, int32_t x_dtype, const faq_shape* shape, const faq_qconfig* cfg,
                       const float* static_scale, const void* rot, faq_qtensor* out,
                       void* debug_rotated, void* stream) {
  static const char* fn = "fa_quantize";
  if (!shape_ok(shape)) return fail(FAQ_ERR_INVALID_ARG, fn, "shape");
  if (x_dtype != FAQ_T_F32 && x_dtype != FAQ_T_BF16) return fail(FAQ_ERR_INVALID_ARG, fn, "x_dtype");
  const faq_status cs = check_cfg(cfg);
  if (cs != FAQ_OK) return fail(cs, fn, "qconfig");
  if (!d_supported(shape->D)) return fail(FAQ_ERR_UNSUPPORTED, fn, "head_dim must be 64 or 128");
  if (!out) return fail(FAQ_ERR_INVALID_ARG, fn, "out is NULL");
  if (!same_cfg(out->cfg, *cfg)) return fail(FAQ_ERR_INVALID_ARG, fn, "out->cfg differs from cfg");
  if (!same_shape(out->shape, *shape)) return fail(FAQ_ERR_SHAPE, fn, "out->shape differs from shape");
  const bool per_head = cfg->scope == FAQ_PER_HEAD;
  const bool tok_block = cfg->scope == FAQ_PER_TOKEN_BLOCK;
  if (per_head && !static_scale) return fail(FAQ_ERR_NOT_CALIBRATED, fn, "per-head scales missing");
  if (!per_head && static_scale) return fail(FAQ_ERR_INVALID_ARG, fn, "static_scale given for a dynamic scope");
  if (rot && !tok_block) return fail(FAQ_ERR_UNSUPPORTED, fn, "rotation needs the token-block scope");
  if (debug_rotated && !rot) return fail(FAQ_ERR_INVALID_ARG, fn, "debug_rotated without rot");
  if (tok_block && x_dtype != FAQ_T_BF16) return fail(FAQ_ERR_UNSUPPORTED, fn, "token-block path needs bf16 input");
  if (numel(*shape) == 0) {
    if (per_head && shape->H > 0 && out->scales != static_scale) {
      if (!out->scales) return fail(FAQ_ERR_INVALID_ARG, fn, "out->scales is NULL");
      return hip_status(hipMemcpyAsync(out->scales, static_scale, (size_t)shape->H * 4,
                                       hipMemcpyDeviceToDevice, (hipStream_t)stream), fn);
    }
    return FAQ_OK;
  }
  if (!x || !out->codes || !out->scales) return fail(FAQ_ERR_INVALID_ARG, fn, "NULL pointer");
  hipStream_t st = (hipStream_t)stream;
  hipError_t e = hipSuccess;
  switch (cfg->dtype) {
    case FAQ_INT8:
      if (per_head)
        e = launch_quant_int8_head(x, x_dtype, *shape, static_scale, (int8_t*)out->codes, st);
      else
        e = launch_quant_int8_token(x, x_dtype, *shape, (int8_t*)out->codes, (float*)out->scales, st);
      break;
    case FAQ_FP8_E4M3:
      if (per_head) {
        e = launch_quant_fp8_head(x, x_dtype, *shape, static_scale, (uint8_t*)out->codes, st);
      } else if (tok_block) {
        if (rot)
          e = launch_rot_fp8_block((const uint16_t*)x, (const uint16_t*)rot, *shape, cfg->block_tokens,
                                   (uint8_t*)out->codes, (float*)out->scales, (uint16_t*)debug_rotated, st);
        else
          e = launch_quant_fp8_block((const uint16_t*)x, *shape, cfg->block_tokens, (uint8_t*)out->codes,
                                     (float*)out->scales, st);
      } else {
        e = launch_quant_fp8_token(x, x_dtype, *shape, (uint8_t*)out->codes, (float*)out->scales, st);
      }
      break;
    case FAQ_MXFP8:
      e = launch_quant_mxfp8(x, x_dtype, *shape, (uint8_t*)out->codes, (uint8_t*)out->scales, st);
      break;
    default:
      e = launch_quant_mxfp4(x, x_dtype, *shape, (uint8_t*)out->codes, (uint8_t*)out->scales, st);
      break;
  }
  if (e == hipSuccess && per_head && out->scales != static_scale)
    e = hipMemcpyAsync(out->scales, static_scale, (size_t)shape->H * 4, hipMemcpyDeviceToDevice, st);
  return hip_status(e, fn);
}

// Where the float scale of token i of head (b, h) sits: b * sb + h * sh +
// i / block.  Per-head scales are one block spanning the sequence (rounded
// up to whole 128-key tiles).
static void scale_index(const faq_qconfig& c, const faq_shape& s, int* block, int64_t* sb, int64_t* sh) {
  if (c.scope == FAQ_PER_TOKEN_BLOCK) {
    const int64_t nb = (s.S + c.block_tokens - 1) / c.block_tokens;
    *block = c.block_tokens; *sh = nb; *sb = s.H * nb;
  } else if (c.scope == FAQ_PER_HEAD) {
    *block = (int)(((s.S > 0 ? s.S : 1) + 127) / 128 * 128); *sh = 1; *sb = 0;
  } else {
    *block = 1; *sh = s.S; *sb = s.H * s.S;
  }
}

static int qk_mode(const faq_qconfig& c) {
  switch (c.dtype) {
    case FAQ_FLOAT: return QK_BF;
    case FAQ_INT8: return c.scope == FAQ_PER_HEAD ? QK_I8H : QK_I8T;
    case FAQ_MXFP4: return QK_MX4;
    case FAQ_MXFP8: return QK_MX8;
    default: return c.scope == FAQ_PER_TOKEN ? QK_F8T : QK_F8C;  // per-head, 128/256-token blocks
  }
}

static int branch_fmt(const faq_qconfig& c) {
  switch (c.dtype) {
    case FAQ_FLOAT: return FMT_BF16;
    case FAQ_INT8: return FMT_INT8;
    case FAQ_MXFP4: return FMT_MX4;
    case FAQ_MXFP8: return FMT_MX8;
    default: return FMT_FP8;
  }
}

static int pv_mode(const faq_qconfig& c) {
  switch (c.dtype) {
    case FAQ_FLOAT: return PV_BF;
    case FAQ_INT8: return c.scope == FAQ_PER_HEAD ? PV_I8H : PV_I8T;
    case FAQ_MXFP4: return PV_MX4;
    case FAQ_MXFP8: return PV_MX8;
    default: return c.scope == FAQ_PER_TOKEN ? PV_F8W : PV_F8C;
  }
}

// Branch configurations for attention ("fa3_quant 配置说明" §2.3: each of
// fa_q / fa_k / fa_v configured on its own, an unconfigured branch not
// quantized - FAQ_FLOAT, bf16 values in `codes`).  Every combination runs:
// Q and K of one (dtype, scope) (token blocks may differ in size) with V of
// that configuration or unquantized take the specialised score kernels; any
// other combination takes the general score mode, which widens Q and K of
// any format exactly to bf16.
static faq_status attn_check(const faq_qtensor* q, const faq_qtensor* k, const faq_qtensor* v,
                             int* qk, int* pv, int* qfmt, int* kfmt, const char* fn) {
  if (!q || !k || !v) return fail(FAQ_ERR_INVALID_ARG, fn, "NULL tensor");
  for (const faq_qtensor* t : {q, k, v}) {
    if (t->cfg.dtype != FAQ_FLOAT) {
      const faq_status cs = check_cfg(&t->cfg);
      if (cs != FAQ_OK) return fail(cs, fn, "qconfig");
    }
    if (!shape_ok(&t->shape)) return fail(FAQ_ERR_INVALID_ARG, fn, "shape");
    if (!d_supported(t->shape.D)) return fail(FAQ_ERR_UNSUPPORTED, fn, "head_dim must be 64 or 128");
  }
  const bool same = q->cfg.dtype == k->cfg.dtype && (q->cfg.dtype == FAQ_FLOAT || q->cfg.scope == k->cfg.scope);
  *qk = same ? qk_mode(k->cfg) : QK_GEN;
  *pv = pv_mode(v->cfg);
  if (!attn_pair_supported(*qk, *pv)) *qk = QK_GEN;
  *qfmt = branch_fmt(q->cfg);
  *kfmt = branch_fmt(k->cfg);
  // the kernels address the K / V rows of one head with 32-bit byte
  // offsets: a head's rows must span less than 4 GiB (BSND rows are H rows
  // apart)
  for (const faq_qtensor* t : {k, v}) {
    const int64_t rb = t->cfg.dtype == FAQ_FLOAT ? 2 * t->shape.D
                       : (t->cfg.dtype == FAQ_MXFP4 ? t->shape.D / 2 : t->shape.D);
    const int64_t ss = t->shape.layout == FAQ_LAYOUT_BSND ? t->shape.H : 1;
    if (t->shape.S > 0 && ((t->shape.S - 1) * ss + 1) * rb >= ((int64_t)1 << 32))
      return fail(FAQ_ERR_UNSUPPORTED, fn, "the K / V rows of one head span 4 GiB or more");
  }
  if (q->shape.B != k->shape.B || q->shape.B != v->shape.B || q->shape.H != k->shape.H ||
      q->shape.H != v->shape.H || q->shape.D != k->shape.D || q->shape.D != v->shape.D ||
      k->shape.S != v->shape.S)
    return fail(FAQ_ERR_SHAPE, fn, "q/k/v shapes");
  return FAQ_OK;
}

size_t fa_quant_attention_workspace_bytes(const faq_qtensor* q, const faq_qtensor* k,
                                          const faq_qtensor* v) {
  int qk, pv, qf, kf;
  if (attn_check(q, k, v, &qk, &pv, &qf, &kf, "fa_quant_attention_workspace_bytes") != FAQ_OK) return 0;
  // the non-causal size: it covers causal calls too (they never split keys)
  return attn_workspace_bytes(qk, pv, k->shape.B, k->shape.H, q->shape.S, k->shape.S, k->shape.D, 0);
}

}  // extern "C"

// The body of the attention entry points: validation (before any HIP
// call), the workspace check, dispatch.
faq_status faq::attention_entry(const faq_qtensor* q, const faq_qtensor* k, const faq_qtensor* v,
                                float sm_scale, int32_t causal, void* out, int32_t out_dtype, void* workspace,
                                size_t workspace_bytes, void* stream, const char* fn) {
  int qk, pv, qf, kf;
  const faq_status cs = attn_check(q, k, v, &qk, &pv, &qf, &kf, fn);
  if (cs != FAQ_OK) return cs;
  if (out_dtype != FAQ_T_F32 && out_dtype != FAQ_T_BF16) return fail(FAQ_ERR_INVALID_ARG, fn, "out_dtype");
  if (causal != 0 && causal != 1) return fail(FAQ_ERR_INVALID_ARG, fn, "causal must be 0 or 1");
  if (!(sm_scale >= 0.0f) || isinf(sm_scale)) return fail(FAQ_ERR_INVALID_ARG, fn, "sm_scale");
  if (causal && q->shape.S != k->shape.S) return fail(FAQ_ERR_SHAPE, fn, "causal needs Sq == Skv");
  const int64_t B = q->shape.B, H = q->shape.H, Sq = q->shape.S, Skv = k->shape.S, D = q->shape.D;
  if (B * H * Sq == 0) return FAQ_OK;
  if (Skv == 0) return fail(FAQ_ERR_SHAPE, fn, "no keys");
  if (!out || !q->codes || !k->codes || !v->codes) return fail(FAQ_ERR_INVALID_ARG, fn, "NULL pointer");
  for (const faq_qtensor* t : {q, k, v})
    if (t->cfg.dtype != FAQ_FLOAT && !t->scales) return fail(FAQ_ERR_INVALID_ARG, fn, "NULL scales");
  const size_t need = attn_workspace_bytes(qk, pv, B, H, Sq, Skv, D, causal);
  if (workspace_bytes < need || !workspace) return fail(FAQ_ERR_WORKSPACE, fn, "workspace");
  AttnArgs a{};
  a.qk = qk;
  a.pv = pv;
  a.qfmt = qf; a.kfmt = kf;
  a.B = B; a.H = H; a.Sq = Sq; a.Skv = Skv; a.D = D;
  a.qmap = row_map(q->shape); a.kmap = row_map(k->shape); a.vmap = row_map(v->shape);
  a.q_codes = q->codes; a.q_scales = q->scales;
  a.k_codes = k->codes; a.k_scales = k->scales;
  a.v_codes = v->codes; a.v_scales = v->scales;
  scale_index(q->cfg, q->shape, &a.q_block, &a.q_sb, &a.q_sh);
  scale_index(k->cfg, k->shape, &a.k_block, &a.k_sb, &a.k_sh);
  scale_index(v->cfg, v->shape, &a.v_block, &a.v_sb, &a.v_sh);
  a.sm_scale = sm_scale == 0.0f ? 1.0f / sqrtf((float)D) : sm_scale;
  a.causal = causal;
  a.out = out;
  a.out_bf16 = out_dtype == FAQ_T_BF16;
  a.ws = workspace;
  return hip_status(launch_attention(a, (hipStream_t)stream), fn);
}

extern "C" faq_status fa_quant_attention(const faq_qtensor* q, const faq_qtensor* k, const faq_qtensor* v,
                                         float sm_scale, int32_t causal, void* out, int32_t out_dtype,
                                         void* workspace, size_t workspace_bytes, void* stream) {
  return attention_entry(q, k, v, sm_scale, causal, out, out_dtype, workspace, workspace_bytes, stream,
                         "fa_quant_attention");
}
