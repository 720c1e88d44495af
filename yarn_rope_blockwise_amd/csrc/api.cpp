// C ABI of libyrb: argument validation on the host, then kernel launches.
// Declarations and the contract of each call are in include/yrb.h.
//
// Nothing here allocates, synchronises or keeps state between calls.  Every
// check runs before the first launch, so an error return means nothing was
// queued.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <cstdint>

#include "../../include/yrb.h"
#include "kernels.h"

namespace {

using yrb::kBF16;
using yrb::kF32;

constexpr double kPi = 3.14159265358979323846;

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

int elem_size(int32_t dtype) { return dtype == YRB_BF16 ? 2 : 4; }

bool dtype_ok(int32_t dtype) { return dtype == YRB_BF16 || dtype == YRB_F32; }
bool dim_ok(int64_t d) { return d == 64 || d == 128; }

// Strides (elements) must keep every row start 16-byte aligned.
bool strides_aligned(const int64_t* s, int n, int32_t dtype) {
  const int64_t q = 16 / elem_size(dtype);
  for (int i = 0; i < n; ++i)
    if (s[i] % q != 0) return false;
  return true;
}
// Non-negative and below 2^31 elements (the kernels index rows in 32 bits).
bool strides_nonneg(const int64_t* s, int n) {
  for (int i = 0; i < n; ++i)
    if (s[i] < 0 || s[i] >= (int64_t(1) << 31)) return false;
  return true;
}

int hip_status(hipError_t e) { return e == hipSuccess ? YRB_OK : YRB_EHIP; }

// Launch-size limits.  A dispatch counts its work-items in 32 bits: with
// 256 per workgroup, at most 2^24 - 1 workgroups; the fp32 attention grid
// puts heads and batches in its y and z extents, each below 2^16.
constexpr int64_t kMaxBlocks = (int64_t(1) << 24) - 1;
constexpr int64_t kMaxItems = (int64_t(1) << 32) - 256;
constexpr int64_t kMaxYZ = 65535;
constexpr int64_t kLim31 = int64_t(1) << 31;

// a * b <= lim for a, b >= 0, without forming a product that may overflow.
bool mul_le(int64_t a, int64_t b, int64_t lim) { return a == 0 || b <= lim / a; }
// a + b < lim for a, b >= 0, likewise.
bool add_lt(int64_t a, int64_t b, int64_t lim) { return a < lim && b < lim - a; }

int check_config(const yrb_rope_config* c) {
  if (!c) return YRB_EINVAL;
  if (c->kind < YRB_ROPE_PLAIN || c->kind > YRB_ROPE_YARN) return YRB_EINVAL;
  if (!dim_ok(c->head_dim)) return YRB_EUNSUPPORTED;
  if (!(c->base > 1.0) || !std::isfinite(c->base)) return YRB_EINVAL;
  if (!(c->scale > 0.0) || !std::isfinite(c->scale)) return YRB_EINVAL;
  if (c->kind == YRB_ROPE_YARN) {
    if (c->orig_ctx <= 0) return YRB_EINVAL;
    if (!(c->alpha < c->beta) || !std::isfinite(c->alpha) || !std::isfinite(c->beta))
      return YRB_EINVAL;
  }
  return YRB_OK;
}

// theta'_i of one rescale, in fp64.
//  base frequencies theta_i = b^(-2i/d)        (tecvarsity Sec. 2)
//  PI   theta_i / s                             (tecvarsity Sec. 2; 14cs17 "Position Interpolation")
//  NTK  (b s^(d/(d-2)))^(-2i/d)                 (14cs17 "NTK-Aware Scaling"; the base change that
//                                                keeps pair 0 and scales the slowest pair by 1/s)
//  YARN r_i = L_train theta_i / (2 pi) turns per training window; g_i = clamp((r_i-alpha)/(beta-alpha));
//       theta'_i = (1-g_i) theta_i / s + g_i theta_i   (root18d "Not every RoPE dimension ...";
//                                                       tecvarsity Sec. 3)
void compute_theta(const yrb_rope_config* c, double* th) {
  const int half = c->head_dim / 2;
  const double d = c->head_dim;
  double base = c->base;
  if (c->kind == YRB_ROPE_NTK) base = c->base * std::pow(c->scale, d / (d - 2.0));
  for (int i = 0; i < half; ++i) {
    const double t = std::pow(base, -2.0 * i / d);
    double tp = t;
    if (c->kind == YRB_ROPE_PI) {
      tp = t / c->scale;
    } else if (c->kind == YRB_ROPE_YARN) {
      const double turns = (double)c->orig_ctx * t / (2.0 * kPi);
      double g = (turns - c->alpha) / (c->beta - c->alpha);
      g = g < 0.0 ? 0.0 : (g > 1.0 ? 1.0 : g);
      tp = (1.0 - g) * (t / c->scale) + g * t;
    }
    th[i] = tp;
  }
}

// Logit multiplier (0.1 ln s + 1)^2 for YaRN with s > 1 (tecvarsity Sec. 3 temperature;
// the square because the factor sits on both the query and the key rotation).
double attn_factor_of(const yrb_rope_config* c) {
  if (c->kind != YRB_ROPE_YARN || c->scale <= 1.0) return 1.0;
  const double ms = 0.1 * std::log(c->scale) + 1.0;
  return ms * ms;
}

}  // namespace

extern "C" {

const char* yrb_status_str(int status) {
  switch (status) {
    case YRB_OK: return "ok";
    case YRB_EINVAL: return "invalid argument";
    case YRB_EUNSUPPORTED: return "unsupported head_dim or dtype";
    case YRB_EALIGN: return "pointer or stride not 16-byte aligned";
    case YRB_EHIP: return "HIP launch error";
    default: return "unknown status";
  }
}

int rope_tables_build(const yrb_rope_config* cfg, int64_t pos0, int64_t n_pos, float* cos_sin,
                      double* inv_freq_out, double* attn_factor_out, void* stream) {
  int st = check_config(cfg);
  if (st) return st;
  if (pos0 < 0 || n_pos < 0) return YRB_EINVAL;
  if (n_pos > 0 && !cos_sin) return YRB_EINVAL;
  if (n_pos > 0 && !aligned16(cos_sin)) return YRB_EALIGN;
  if (!mul_le(n_pos, cfg->head_dim / 2, kMaxItems) || pos0 > (int64_t(1) << 50)) return YRB_EINVAL;
  double th[64];
  compute_theta(cfg, th);
  const int half = cfg->head_dim / 2;
  if (inv_freq_out)
    for (int i = 0; i < half; ++i) inv_freq_out[i] = th[i];
  if (attn_factor_out) *attn_factor_out = attn_factor_of(cfg);
  if (n_pos == 0) return YRB_OK;
  return hip_status(
      yrb::launch_rope_tables(th, half, pos0, n_pos, cos_sin, static_cast<hipStream_t>(stream)));
}

// theta'_i = theta_i / lambda_i for a caller's per-pair vector (tecvarsity
// Sec. 4, LongRoPE's non-uniform per-dimension scale).
int rope_tables_build_factors(int32_t head_dim, double base, const double* factors, int64_t pos0,
                              int64_t n_pos, float* cos_sin, double* inv_freq_out, void* stream) {
  if (!dim_ok(head_dim)) return YRB_EUNSUPPORTED;
  if (!(base > 1.0) || !std::isfinite(base)) return YRB_EINVAL;
  if (!factors) return YRB_EINVAL;
  const int half = head_dim / 2;
  for (int i = 0; i < half; ++i)
    if (!(factors[i] > 0.0) || !std::isfinite(factors[i])) return YRB_EINVAL;
  if (pos0 < 0 || n_pos < 0) return YRB_EINVAL;
  if (n_pos > 0 && !cos_sin) return YRB_EINVAL;
  if (n_pos > 0 && !aligned16(cos_sin)) return YRB_EALIGN;
  if (!mul_le(n_pos, half, kMaxItems) || pos0 > (int64_t(1) << 50)) return YRB_EINVAL;
  double th[64];
  const double d = head_dim;
  for (int i = 0; i < half; ++i) th[i] = std::pow(base, -2.0 * i / d) / factors[i];
  if (inv_freq_out)
    for (int i = 0; i < half; ++i) inv_freq_out[i] = th[i];
  if (n_pos == 0) return YRB_OK;
  return hip_status(
      yrb::launch_rope_tables(th, half, pos0, n_pos, cos_sin, static_cast<hipStream_t>(stream)));
}

int rope_apply(const void* x, void* y, int32_t dtype, int64_t B, int64_t S, int64_t H, int64_t D,
               const int64_t x_strides[3], const int64_t y_strides[3], const float* cos_sin,
               int64_t n_table_rows, int64_t pos_offset, const int32_t* pos_ids, void* stream) {
  return rope_apply_ex(x, y, dtype, B, S, H, D, x_strides, y_strides, cos_sin, n_table_rows,
                       pos_offset, pos_ids, YRB_LAYOUT_HALF, stream);
}

int rope_apply_ex(const void* x, void* y, int32_t dtype, int64_t B, int64_t S, int64_t H,
                  int64_t D, const int64_t x_strides[3], const int64_t y_strides[3],
                  const float* cos_sin, int64_t n_table_rows, int64_t pos_offset,
                  const int32_t* pos_ids, int32_t layout, void* stream) {
  if (layout != YRB_LAYOUT_HALF && layout != YRB_LAYOUT_INTERLEAVED) return YRB_EINVAL;
  if (!dtype_ok(dtype)) return YRB_EUNSUPPORTED;
  if (!dim_ok(D)) return YRB_EUNSUPPORTED;
  if (B < 0 || S < 0 || H < 0 || n_table_rows < 0 || pos_offset < 0) return YRB_EINVAL;
  if (!x_strides || !y_strides) return YRB_EINVAL;
  if (B == 0 || S == 0 || H == 0) return YRB_OK;
  // one workgroup row per token (S of them), head pairs in its y extent
  if (S > kMaxBlocks || H > kLim31 / 16) return YRB_EINVAL;
  if (!x || !y || !cos_sin) return YRB_EINVAL;
  if (!strides_nonneg(x_strides, 3) || !strides_nonneg(y_strides, 3)) return YRB_EINVAL;
  if (!aligned16(x) || !aligned16(y) || !aligned16(cos_sin)) return YRB_EALIGN;
  if (!strides_aligned(x_strides, 3, dtype) || !strides_aligned(y_strides, 3, dtype))
    return YRB_EALIGN;
  if (!pos_ids && (S > n_table_rows || pos_offset > n_table_rows - S)) return YRB_EINVAL;
  yrb::RopeArgs r{};
  r.x = x;
  r.y = y;
  for (int i = 0; i < 3; ++i) {
    r.xs[i] = x_strides[i];
    r.ys[i] = y_strides[i];
  }
  r.B = B;
  r.S = S;
  r.H = H;
  r.cos_sin = cos_sin;
  r.n_rows = n_table_rows;
  r.pos_offset = pos_offset;
  r.pos_ids = pos_ids;
  return hip_status(yrb::launch_rope_apply(dtype, (int)D, layout == YRB_LAYOUT_INTERLEAVED, r,
                                           static_cast<hipStream_t>(stream)));
}

namespace {

// Validation and launch shared by the prefill entry points: Sq queries at
// positions q_offset.., Sk keys at positions 0..; window > 0 turns on the
// sink+window mask (bf16 pipelined kernel).
int prefill_common(const void* q, const void* k, const void* v, void* o, int32_t dtype, int64_t B, int64_t Sq,
                   int64_t Sk, int64_t q_offset, int64_t Hq, int64_t Hkv, int64_t D, const int64_t strides[4][3],
                   const float* cos_sin, int64_t n_table_rows, float softmax_scale, int32_t causal,
                   int64_t n_sink, int64_t window, float* lse, void* workspace, void* stream) {
  if (!dtype_ok(dtype)) return YRB_EUNSUPPORTED;
  if (!dim_ok(D)) return YRB_EUNSUPPORTED;
  if (B < 0 || Sq < 0 || Sk < 0 || q_offset < 0 || Hq <= 0 || Hkv <= 0 || Hq % Hkv != 0) return YRB_EINVAL;
  if (causal != 0 && causal != 1) return YRB_EINVAL;
  if (!std::isfinite(softmax_scale) || !(softmax_scale > 0.f)) return YRB_EINVAL;
  if (!strides) return YRB_EINVAL;
  if (B == 0 || Sq == 0) return YRB_OK;
  if (!q || !o || (Sk > 0 && (!k || !v))) return YRB_EINVAL;
  if (!add_lt(q_offset, Sq, kLim31) || Sk >= kLim31 || Hq >= kLim31) return YRB_EINVAL;
  // grid: bf16, one workgroup per (256-row query tile, batch, head); fp32,
  // 64-row tiles with heads and batches in the y and z extents
  if (dtype == YRB_BF16 ? !mul_le(B, Hq, kMaxBlocks) || !mul_le((Sq + 255) / 256, B * Hq, kMaxBlocks)
                        : Hq > kMaxYZ || B > kMaxYZ)
    return YRB_EINVAL;
  for (int t = 0; t < 4; ++t) {
    if (!strides_nonneg(strides[t], 3)) return YRB_EINVAL;
    if (!strides_aligned(strides[t], 3, dtype)) return YRB_EALIGN;
  }
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(o) || !aligned16(lse) ||
      !aligned16(workspace))
    return YRB_EALIGN;
  if (cos_sin) {
    if (!aligned16(cos_sin)) return YRB_EALIGN;
    if (n_table_rows < 0 || q_offset + Sq > n_table_rows) return YRB_EINVAL;
  }
  hipStream_t s = static_cast<hipStream_t>(stream);
  yrb::AttnArgs a{};
  a.q = q;
  a.k = k;
  a.v = v;
  for (int i = 0; i < 3; ++i) {
    a.qs[i] = strides[0][i];
    a.ks[i] = strides[1][i];
    a.vs[i] = strides[2][i];
    a.os[i] = strides[3][i];
  }
  a.o = o;
  a.lse = lse;
  a.cos_sin = cos_sin;
  a.B = B;
  a.Sq = Sq;
  a.Sk = Sk;
  a.Hq = Hq;
  a.Hkv = Hkv;
  a.q_offset = q_offset;
  a.k_offset = 0;
  a.softmax_scale = softmax_scale;
  a.causal = causal;
  a.load_state = 0;
  a.store_state = 0;
  a.finalize = 1;
  a.claims = static_cast<unsigned*>(workspace);
  if (window > 0) {
    a.n_sink = (int)n_sink;
    a.window = (int)window;
    return hip_status(yrb::launch_attention_bf16_pp((int)D, a, s));
  }
  return hip_status(yrb::launch_attention(dtype, (int)D, a, s));
}

}  // namespace

int attn_prefill_blockwise(const void* q, const void* k, const void* v, void* o, int32_t dtype,
                           int64_t B, int64_t S, int64_t Hq, int64_t Hkv, int64_t D,
                           const int64_t strides[4][3], const float* cos_sin,
                           int64_t n_table_rows, float softmax_scale, int32_t causal, float* lse,
                           void* workspace, void* stream) {
  return prefill_common(q, k, v, o, dtype, B, S, S, 0, Hq, Hkv, D, strides, cos_sin, n_table_rows,
                        softmax_scale, causal, 0, 0, lse, workspace, stream);
}

int attn_prefill_sink_window(const void* q, const void* k, const void* v, void* o, int32_t dtype,
                             int64_t B, int64_t S, int64_t Hq, int64_t Hkv, int64_t D,
                             const int64_t strides[4][3], const float* cos_sin, int64_t n_table_rows,
                             float softmax_scale, int64_t n_sink, int64_t window, float* lse,
                             void* workspace, void* stream) {
  return attn_prefill_sink_window_chunk(q, k, v, o, dtype, B, S, S, Hq, Hkv, D, strides, 0, cos_sin, n_table_rows,
                                        softmax_scale, n_sink, window, lse, workspace, stream);
}

int attn_prefill_sink_window_chunk(const void* q, const void* k, const void* v, void* o, int32_t dtype,
                                   int64_t B, int64_t Sq, int64_t Sk, int64_t Hq, int64_t Hkv, int64_t D,
                                   const int64_t strides[4][3], int64_t q_offset, const float* cos_sin,
                                   int64_t n_table_rows, float softmax_scale, int64_t n_sink, int64_t window,
                                   float* lse, void* workspace, void* stream) {
  if (dtype != YRB_BF16) return YRB_EUNSUPPORTED;
  if (n_sink < 0 || window < 1 || Sq < 0 || Sk < 0 || q_offset < 0) return YRB_EINVAL;
  if (Sk >= (int64_t(1) << 30) || !add_lt(q_offset, Sq, int64_t(1) << 30)) return YRB_EINVAL;
  // A window reaching past position 0 from the last query sees every
  // earlier key: plain causal.  Sinks past Sk are all the keys there are.
  const int64_t q_end = q_offset + Sq;
  return prefill_common(q, k, v, o, dtype, B, Sq, Sk, q_offset, Hq, Hkv, D, strides, cos_sin, n_table_rows,
                        softmax_scale, 1, std::min(n_sink, Sk), std::min(window, std::max<int64_t>(q_end, 1)), lse,
                        workspace, stream);
}

int attn_block_accumulate(const void* q, const void* k_blk, const void* v_blk, int32_t dtype,
                          int64_t B, int64_t Sq, int64_t Sk, int64_t Hq, int64_t Hkv, int64_t D,
                          const int64_t strides[3][3], int64_t q_offset, int64_t k_offset,
                          const float* cos_sin, int64_t n_table_rows, float softmax_scale,
                          int32_t causal, float* o_acc, float* m, float* l,
                          int32_t flags, void* o_out, const int64_t o_strides[3], void* workspace,
                          void* stream) {
  if (!dtype_ok(dtype)) return YRB_EUNSUPPORTED;
  if (!dim_ok(D)) return YRB_EUNSUPPORTED;
  if (B < 0 || Sq < 0 || Sk < 0 || Hq <= 0 || Hkv <= 0 || Hq % Hkv != 0) return YRB_EINVAL;
  if (q_offset < 0 || k_offset < 0) return YRB_EINVAL;
  if (causal != 0 && causal != 1) return YRB_EINVAL;
  if (flags & ~(YRB_ACC_FIRST | YRB_ACC_FINALIZE)) return YRB_EINVAL;
  if (!std::isfinite(softmax_scale) || !(softmax_scale > 0.f)) return YRB_EINVAL;
  if (!strides) return YRB_EINVAL;
  const bool fin = (flags & YRB_ACC_FINALIZE) != 0;
  if (fin && !o_strides) return YRB_EINVAL;
  if (B == 0 || Sq == 0) return YRB_OK;
  if (!add_lt(q_offset, Sq, kLim31) || !add_lt(k_offset, Sk, kLim31) || Hq >= kLim31) return YRB_EINVAL;
  if (dtype == YRB_BF16 ? !mul_le(B, Hq, kMaxBlocks) || !mul_le((Sq + 255) / 256, B * Hq, kMaxBlocks)
                        : Hq > kMaxYZ || B > kMaxYZ)
    return YRB_EINVAL;
  if (!q || !o_acc || !m || !l) return YRB_EINVAL;
  if (Sk > 0 && (!k_blk || !v_blk)) return YRB_EINVAL;
  if (fin && !o_out) return YRB_EINVAL;
  for (int t = 0; t < 3; ++t) {
    if (!strides_nonneg(strides[t], 3)) return YRB_EINVAL;
    if (!strides_aligned(strides[t], 3, dtype)) return YRB_EALIGN;
  }
  if (fin && (!strides_nonneg(o_strides, 3))) return YRB_EINVAL;
  if (fin && !strides_aligned(o_strides, 3, dtype)) return YRB_EALIGN;
  if (!aligned16(q) || !aligned16(k_blk) || !aligned16(v_blk) || !aligned16(o_acc) ||
      !aligned16(o_out) || !aligned16(workspace))
    return YRB_EALIGN;
  const bool future = causal && k_offset > q_offset + Sq - 1;
  if (cos_sin) {
    if (!aligned16(cos_sin)) return YRB_EALIGN;
    if (q_offset + Sq > n_table_rows) return YRB_EINVAL;
  }
  hipStream_t s = static_cast<hipStream_t>(stream);
  yrb::AttnArgs a{};
  a.q = q;
  a.k = k_blk;
  a.v = v_blk;
  for (int i = 0; i < 3; ++i) {
    a.qs[i] = strides[0][i];
    a.ks[i] = strides[1][i];
    a.vs[i] = strides[2][i];
    a.os[i] = fin ? o_strides[i] : 0;
  }
  a.o = fin ? o_out : nullptr;
  a.lse = nullptr;
  a.o_acc = o_acc;
  a.m = m;
  a.l = l;
  a.cos_sin = cos_sin;
  a.B = B;
  a.Sq = Sq;
  a.Sk = future ? 0 : Sk;
  a.Hq = Hq;
  a.Hkv = Hkv;
  a.q_offset = q_offset;
  a.k_offset = k_offset;
  a.softmax_scale = softmax_scale;
  a.causal = causal;
  a.load_state = (flags & YRB_ACC_FIRST) ? 0 : 1;
  a.store_state = 1;
  a.finalize = fin ? 1 : 0;
  a.claims = static_cast<unsigned*>(workspace);
  return hip_status(yrb::launch_attention(dtype, (int)D, a, s));
}

namespace {

// Shared by the bf16 and fp8 decode entry points: validation, then the
// launch with the cache element type `cache_dtype` (q and o are bf16).
int decode_common(int cache_dtype, bool interleaved, const void* q, const void* k_cache, const void* v_cache, void* o,
                  int64_t B, int64_t Hq, int64_t Hkv, int64_t D, int64_t n_sink, int64_t window,
                  const int64_t q_strides[2], const int64_t cache_strides[3],
                  const int64_t o_strides[2], const int32_t* cache_len, const int32_t* ring_head,
                  const float* k_scale, const float* v_scale, const float* cos_sin,
                  int64_t n_table_rows, float softmax_scale, void* stream) {
  const int32_t dtype = YRB_BF16;   // q and o
  if (!dim_ok(D)) return YRB_EUNSUPPORTED;
  if (B < 0 || Hq <= 0 || Hkv <= 0 || Hq % Hkv != 0) return YRB_EINVAL;
  const int64_t g = Hq / Hkv;
  if (g != 1 && g != 2 && g != 4 && g != 8) return YRB_EUNSUPPORTED;
  if (n_sink < 0 || window < 1) return YRB_EINVAL;
  if (!add_lt(n_sink, window, kLim31)) return YRB_EINVAL;
  if (!std::isfinite(softmax_scale) || !(softmax_scale > 0.f)) return YRB_EINVAL;
  if (!q_strides || !cache_strides || !o_strides) return YRB_EINVAL;
  if (B == 0) return YRB_OK;
  if (!mul_le(B, Hkv, kMaxBlocks)) return YRB_EINVAL;   // at most one workgroup per (sequence, head)
  if (!q || !k_cache || !v_cache || !o || !cache_len || !cos_sin) return YRB_EINVAL;
  if (!strides_nonneg(q_strides, 2) || !strides_nonneg(cache_strides, 3) ||
      !strides_nonneg(o_strides, 2))
    return YRB_EINVAL;
  const int64_t cache_q = cache_dtype == yrb::kFP8E4M3 ? 16 : 8;   // elements per 16 bytes
  for (int i = 0; i < 3; ++i)
    if (cache_strides[i] % cache_q != 0) return YRB_EALIGN;
  // The kernel addresses a (sequence, head)'s cache with 32-bit offsets from
  // one base: an entry index and the entry stride in bytes below 2^24 (one
  // 24-bit product), the farthest byte below 2^32.
  const int64_t esz = cache_dtype == yrb::kFP8E4M3 ? 1 : 2;
  const int64_t kLim24 = int64_t(1) << 24;
  if (n_sink + window > kLim24 || cache_strides[2] * esz >= kLim24 ||
      (n_sink + window - 1) * cache_strides[2] * esz + D * esz > int64_t(0xFFFFFFFF))
    return YRB_EINVAL;
  if (!strides_aligned(q_strides, 2, dtype) || !strides_aligned(o_strides, 2, dtype)) return YRB_EALIGN;
  if (!aligned16(q) || !aligned16(o) || !aligned16(k_cache) || !aligned16(v_cache) ||
      !aligned16(cos_sin))
    return YRB_EALIGN;
  if (n_table_rows < n_sink + window) return YRB_EINVAL;
  yrb::DecodeArgs a{};
  a.k_scale = k_scale;
  a.v_scale = v_scale;
  a.q = q;
  a.k = k_cache;
  a.v = v_cache;
  a.o = o;
  a.qs[0] = q_strides[0];
  a.qs[1] = q_strides[1];
  for (int i = 0; i < 3; ++i) a.cs[i] = cache_strides[i];
  a.os[0] = o_strides[0];
  a.os[1] = o_strides[1];
  a.B = B;
  a.Hq = Hq;
  a.Hkv = Hkv;
  a.n_sink = n_sink;
  a.window = window;
  a.cache_len = cache_len;
  a.ring_head = ring_head;
  a.cos_sin = cos_sin;
  a.softmax_scale = softmax_scale;
  return hip_status(
      yrb::launch_decode(cache_dtype, (int)D, interleaved, a, static_cast<hipStream_t>(stream)));
}

}  // namespace

int attn_decode_sink_window(const void* q, const void* k_cache, const void* v_cache, void* o,
                            int32_t dtype, int64_t B, int64_t Hq, int64_t Hkv, int64_t D,
                            int64_t n_sink, int64_t window, const int64_t q_strides[2],
                            const int64_t cache_strides[3], const int64_t o_strides[2],
                            const int32_t* cache_len, const int32_t* ring_head,
                            const float* cos_sin, int64_t n_table_rows, float softmax_scale,
                            void* stream) {
  if (dtype != YRB_BF16) return YRB_EUNSUPPORTED;
  return decode_common(yrb::kBF16, false, q, k_cache, v_cache, o, B, Hq, Hkv, D, n_sink, window,
                       q_strides, cache_strides, o_strides, cache_len, ring_head, nullptr,
                       nullptr, cos_sin, n_table_rows, softmax_scale, stream);
}

int attn_decode_sink_window_fp8(const void* q, const void* k_cache, const void* v_cache, void* o,
                                int64_t B, int64_t Hq, int64_t Hkv, int64_t D, int64_t n_sink,
                                int64_t window, const int64_t q_strides[2],
                                const int64_t cache_strides[3], const int64_t o_strides[2],
                                const int32_t* cache_len, const int32_t* ring_head,
                                const float* k_scale, const float* v_scale, const float* cos_sin,
                                int64_t n_table_rows, float softmax_scale, void* stream) {
  if ((k_scale && !aligned16(k_scale)) || (v_scale && !aligned16(v_scale))) return YRB_EALIGN;
  return decode_common(yrb::kFP8E4M3, false, q, k_cache, v_cache, o, B, Hq, Hkv, D, n_sink, window,
                       q_strides, cache_strides, o_strides, cache_len, ring_head, k_scale, v_scale,
                       cos_sin, n_table_rows, softmax_scale, stream);
}

int attn_decode_sink_window_ex(const void* q, const void* k_cache, const void* v_cache, void* o,
                               int32_t cache_dtype, int32_t layout, int64_t B, int64_t Hq,
                               int64_t Hkv, int64_t D, int64_t n_sink, int64_t window,
                               const int64_t q_strides[2], const int64_t cache_strides[3],
                               const int64_t o_strides[2], const int32_t* cache_len,
                               const int32_t* ring_head, const float* k_scale,
                               const float* v_scale, const float* cos_sin, int64_t n_table_rows,
                               float softmax_scale, void* stream) {
  if (layout != YRB_LAYOUT_HALF && layout != YRB_LAYOUT_INTERLEAVED) return YRB_EINVAL;
  if (cache_dtype != YRB_BF16 && cache_dtype != YRB_FP8_E4M3) return YRB_EUNSUPPORTED;
  const bool fp8 = cache_dtype == YRB_FP8_E4M3;
  if (fp8 && ((k_scale && !aligned16(k_scale)) || (v_scale && !aligned16(v_scale))))
    return YRB_EALIGN;
  return decode_common(fp8 ? yrb::kFP8E4M3 : yrb::kBF16, layout == YRB_LAYOUT_INTERLEAVED, q,
                       k_cache, v_cache, o, B, Hq, Hkv, D, n_sink, window, q_strides,
                       cache_strides, o_strides, cache_len, ring_head, fp8 ? k_scale : nullptr,
                       fp8 ? v_scale : nullptr, cos_sin, n_table_rows, softmax_scale, stream);
}

}  // extern "C"
