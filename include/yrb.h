/*
 * yrb.h -- C ABI of libyrb.so: RoPE under a context-extension rescale, fused
 * into exact blockwise causal attention, for AMD Instinct MI355X (gfx950).
 *
 * The calls of the path:
 *   rope_tables_build        frequencies theta'_i and fp32 cos/sin tables
 *   rope_apply               rotate half-split pairs of Q or K
 *   attn_prefill_blockwise   causal softmax attention with RoPE on load
 *   attn_prefill_sink_window the same under the sink+window mask, skipping tiles
 *   attn_block_accumulate    fold one external key/value block into a
 *                            query block's online-softmax state (one ring step)
 *   attn_decode_sink_window  one query per sequence over a sink + sliding
 *                            window cache, keys rotated on load
 *
 * Conventions shared by every call
 *  - Every device buffer is owned by the caller.  The library allocates no
 *    memory, never synchronises and keeps no mutable state between calls
 *    (one exception, attn_prefill_blockwise_noalloc, keeps its work-claim
 *    counter in a static per-GPU array; its declaration states the rule for
 *    overlapping calls): calls may be made from any thread, and calls
 *    queued on different streams may run at the same time, as long as they
 *    do not write the same buffers.  A workspace (below) counts as a written
 *    buffer.
 *  - Work is queued on `stream` (a hipStream_t; NULL = the default stream)
 *    and completes asynchronously.  A kernel fault surfaces at the caller's
 *    next synchronisation.
 *  - Arguments are validated on the host before anything is queued: a
 *    negative return means nothing was launched and nothing was written.
 *  - Tensors are token-major [batch][token][head][dim] with the dim stride
 *    equal to 1; the other strides are given in elements, each in
 *    [0, 2^31) (else YRB_EINVAL).  Base pointers must be 16-byte aligned and
 *    strides multiples of 16 bytes (else YRB_EALIGN).
 *  - Sizes are int64 and every check on them is free of overflow.  A call
 *    whose launch would exceed the dispatch limits returns YRB_EINVAL: a
 *    dispatch counts its work-items in 32 bits (at most 2^24 - 1
 *    workgroups of 256), so rope_tables_build needs n_pos * d/2 <= 2^32 -
 *    256, rope_apply S < 2^24 and H < 2^27, the bf16 prefill and
 *    accumulate ceil(S/256) * B * Hq < 2^24 (fp32: B and Hq <= 65535), and
 *    the decode B * Hkv < 2^24; positions stay below 2^31.  The decode
 *    addresses one (sequence, head)'s cache with 32-bit offsets: it needs
 *    n_sink + window <= 2^24, the entry stride below 2^24 bytes and
 *    (n_sink + window - 1) * entry stride + head_dim elements within 2^32
 *    bytes (else YRB_EINVAL).
 *  - dtype: YRB_BF16 (bfloat16 storage, fp32 arithmetic, bf16 MFMA for the
 *    products) or YRB_F32 (fp32 storage and arithmetic).
 *  - head_dim must be 64 or 128.
 *  - Cos/sin tables hold row r for position r (rows start at position 0),
 *    each row [head_dim/2][2] floats = (cos, sin) of pair i.  `n_table_rows`
 *    is the number of rows the caller allocated; every position a call uses
 *    must be below it.
 *
 * Sources (cited by page title and section):
 *  [T] "Context Window Scaling: YaRN, LongRoPE, and RingAttention
 *      Architectures" (tecvarsity)
 *  [C] "Context Length Extension" (14cs17 notes)
 *  [R] "Long-context extension: stretching attention past its training
 *      window" (root18d)
 *  [J] jovanaeducation guide a2-tli-4 (sections "YaRN: rescale the
 *      frequencies", "Attention sinks", "Ring attention")
 */
#ifndef YRB_H
#define YRB_H

#include <stdint.h>

/* The library is built with hidden visibility; these calls alone are
 * exported. */
#if defined(__GNUC__) || defined(__clang__)
#define YRB_API __attribute__((visibility("default")))
#else
#define YRB_API
#endif

#ifdef __cplusplus
extern "C" {
#endif

/* Status codes. */
#define YRB_OK            0
#define YRB_EINVAL       -1   /* bad size, pointer, flag or position range */
#define YRB_EUNSUPPORTED -2   /* head_dim or dtype the kernels do not build */
#define YRB_EALIGN       -3   /* base pointer or stride not 16-byte aligned */
#define YRB_EHIP         -4   /* the HIP runtime reported a launch error */

/* Rescale methods. */
#define YRB_ROPE_PLAIN 0      /* theta_i = base^(-2i/d)                 [T] Sec. 2 */
#define YRB_ROPE_PI    1      /* theta_i / s  (position m -> m/s)       [T] Sec. 2, [C] "Position Interpolation" */
#define YRB_ROPE_NTK   2      /* base -> base * s^(d/(d-2))             [C] "NTK-Aware Scaling" (formula not printed; this reading) */
#define YRB_ROPE_YARN  3      /* per-pair ramp between theta and theta/s, plus temperature  [R], [T] Sec. 3 */

/* Storage types. */
#define YRB_BF16     0
#define YRB_F32      1
#define YRB_FP8_E4M3 2        /* K/V cache codes of attn_decode_sink_window_ex */

/* Pair layouts of the rotation ([T] Sec. 2 pairs the d dimensions into d/2). */
#define YRB_LAYOUT_HALF        0   /* (x_i, x_{i+d/2}): every other call */
#define YRB_LAYOUT_INTERLEAVED 1   /* (x_{2i}, x_{2i+1}): the _ex calls    */

/* Bytes of the optional `workspace` of the prefill calls and
 * attn_block_accumulate: a device buffer, 16-byte aligned, that holds zeros
 * before its first use.  Given one, the last part of the launch's grid
 * (30 %; 15 % under the sink+window mask) takes its work items from a
 * counter there, so that the XCDs, which under
 * load run at clocks a few percent apart, finish together; each call leaves
 * the workspace as it found it (zero), so one workspace serves any number
 * of calls in sequence on a stream.  Calls that may run at the same time
 * need workspaces of their own.  With workspace = NULL every block takes a
 * fixed item; the results are the same bit for bit either way. */
#define YRB_WORKSPACE_BYTES 64

/* attn_block_accumulate flags. */
#define YRB_ACC_FIRST    1    /* ignore the incoming state: start from m=-inf, l=0, acc=0 */
#define YRB_ACC_FINALIZE 2    /* after folding the block, write o = acc / l */

typedef struct yrb_rope_config {
  int32_t kind;      /* YRB_ROPE_* */
  int32_t head_dim;  /* d: 64 or 128 */
  double  base;      /* b > 1 (10000 in the pages' examples) */
  double  scale;     /* s = L_target / L_train > 0 */
  int64_t orig_ctx;  /* L_train > 0; used by YaRN's ramp */
  double  alpha;     /* YaRN ramp: below alpha turns per training window -> full interpolation (1) */
  double  beta;      /* YaRN ramp: above beta turns -> untouched (32); alpha < beta */
} yrb_rope_config;

/*
 * rope_tables_build -- frequencies and cos/sin tables of one rescale.
 *
 * theta_i = base^(-2i/d) [T] Sec. 2; theta'_i per method:
 *   PLAIN theta; PI theta/s; NTK (base*s^(d/(d-2)))^(-2i/d);
 *   YARN  (1-g_i) theta_i/s + g_i theta_i with r_i = L_train*theta_i/(2 pi),
 *         g_i = clamp((r_i - alpha)/(beta - alpha), 0, 1)   [R], [T] Sec. 3.
 * attn_factor = (0.1 ln s + 1)^2 for YARN with s > 1, else 1 ([T] Sec. 3
 * temperature; the square because both q and k carry the factor).  The
 * caller folds it into softmax_scale = attn_factor / sqrt(d); the tables
 * themselves stay unit-norm.
 *
 *   cfg            host; validated (kind, head_dim in {64,128}, base > 1,
 *                  scale > 0, orig_ctx > 0, alpha < beta).
 *   pos0, n_pos    rows written are positions pos0 .. pos0+n_pos-1, row r
 *                  holding position pos0+r.  pos0 >= 0, n_pos >= 0.
 *   cos_sin        device [n_pos][d/2][2] fp32, cos then sin of pos*theta'_i,
 *                  with the angle formed and reduced in fp64.  May be NULL
 *                  only when n_pos == 0 (frequencies only, no launch).
 *   inv_freq_out   host [d/2] fp64 theta'_i, or NULL.
 *   attn_factor_out host fp64, or NULL.
 */
YRB_API int rope_tables_build(const yrb_rope_config* cfg, int64_t pos0, int64_t n_pos,
                      float* cos_sin, double* inv_freq_out, double* attn_factor_out,
                      void* stream);

/*
 * rope_tables_build_factors -- cos/sin tables from a per-pair rescale
 * vector: theta'_i = theta_i / lambda_i, theta_i = base^(-2i/d) ([T] Sec. 4:
 * a non-uniform scale for each dimension, found by search, in place of one
 * s or a ramp; the search itself is not here).  lambda_i = s for every i is
 * PI; a vector per layer is one call per layer.  No temperature: the caller
 * chooses softmax_scale.
 *
 *   head_dim       64 or 128 (else YRB_EUNSUPPORTED).
 *   base           b > 1, finite.
 *   factors        host [d/2] fp64, every lambda_i finite and > 0 (else
 *                  YRB_EINVAL; nothing is launched).
 *   pos0, n_pos, cos_sin, inv_freq_out   as for rope_tables_build.
 */
YRB_API int rope_tables_build_factors(int32_t head_dim, double base, const double* factors,
                              int64_t pos0, int64_t n_pos, float* cos_sin,
                              double* inv_freq_out, void* stream);

/*
 * rope_apply -- rotate every half-split pair (x_i, x_{i+d/2}) of x by the
 * angle of its token's position ([T] Sec. 2 rotation matrix
 * [[cos, -sin], [sin, cos]]):
 *   y_i = x_i c - x_{i+d/2} s,   y_{i+d/2} = x_i s + x_{i+d/2} c.
 *
 *   x, y           device [B][S][H][D] of dtype, strides x_strides / y_strides
 *                  (b, s, h; elements).  y may equal x (in place).
 *   cos_sin        device table (see conventions), n_table_rows rows.
 *   pos_ids        device int32 [B][S] (contiguous) giving each token's
 *                  position, or NULL: token s of every sequence sits at
 *                  pos_offset + s (then pos_offset + S <= n_table_rows is
 *                  checked on the host).  With pos_ids, a position outside
 *                  [0, n_table_rows) is not read: that token's output is NaN.
 * Arithmetic is fp32; bf16 results are rounded to nearest even.
 */
YRB_API int rope_apply(const void* x, void* y, int32_t dtype,
               int64_t B, int64_t S, int64_t H, int64_t D,
               const int64_t x_strides[3], const int64_t y_strides[3],
               const float* cos_sin, int64_t n_table_rows,
               int64_t pos_offset, const int32_t* pos_ids, void* stream);

/*
 * rope_apply_ex -- rope_apply with a choice of pair layout: YRB_LAYOUT_HALF
 * is rope_apply; YRB_LAYOUT_INTERLEAVED rotates adjacent pairs,
 *   y_{2i} = x_{2i} c - x_{2i+1} s,   y_{2i+1} = x_{2i} s + x_{2i+1} c,
 * with the same table (pair i's angle).  Any other layout: YRB_EINVAL.
 * A model in the interleaved layout rotates Q and K with this call and
 * passes cos_sin = NULL to attn_prefill_blockwise / attn_block_accumulate.
 */
YRB_API int rope_apply_ex(const void* x, void* y, int32_t dtype,
                  int64_t B, int64_t S, int64_t H, int64_t D,
                  const int64_t x_strides[3], const int64_t y_strides[3],
                  const float* cos_sin, int64_t n_table_rows,
                  int64_t pos_offset, const int32_t* pos_ids, int32_t layout, void* stream);

/*
 * attn_prefill_blockwise -- o = softmax(scale * Q' K'^T + causal mask) V per
 * (batch, query head), computed blockwise with a running row max and sum so
 * that the S x S score matrix never exists ([T] Sec. 1 MHSA relation;
 * [J] "Ring attention" / [C] "Ring Attention": the online softmax of
 * FlashAttention-style kernels).  Causal: key position <= query position
 * ([T] FAQ 2); key tiles wholly in a query tile's future are skipped.
 *
 *   q              device [B][S][Hq][D], strides[0] = (b, s, h) elements
 *   k, v           device [B][S][Hkv][D], strides[1], strides[2]
 *   o              device [B][S][Hq][D], strides[3]; written in dtype
 *   Hq % Hkv == 0; query head h reads key/value head h / (Hq/Hkv).
 *   cos_sin        NULL: q is already rotated.  Otherwise q is rotated on load
 *                  at positions 0..S-1 (S <= n_table_rows).  k must already
 *                  be rotated (rope_apply at the same positions): keys are
 *                  reused by every query tile, so they are rotated once, not
 *                  on every load.
 *   softmax_scale  multiplier of q.k (attn_factor / sqrt(d)); finite, > 0.
 *   causal         0 or 1.
 *   lse            device [B][Hq][S] fp32 or NULL: ln sum_j exp(scale q.k_j)
 *                  per row (-inf for a row that sees no key).
 *   workspace      NULL or YRB_WORKSPACE_BYTES of device memory (see there);
 *                  misaligned: YRB_EALIGN.
 * bf16: products on bf16 MFMA with fp32 accumulation; probabilities are
 * rounded to bf16 before the P V product; output rounded to nearest even.
 */
YRB_API int attn_prefill_blockwise(const void* q, const void* k, const void* v, void* o,
                           int32_t dtype, int64_t B, int64_t S, int64_t Hq, int64_t Hkv,
                           int64_t D, const int64_t strides[4][3],
                           const float* cos_sin, int64_t n_table_rows,
                           float softmax_scale, int32_t causal, float* lse,
                           void* workspace, void* stream);

/*
 * attn_prefill_blockwise_noalloc -- attn_prefill_blockwise without a
 * workspace argument, for callers that cannot allocate device memory (code
 * under HIP graph capture, tight serving loops, harnesses that forbid
 * allocation).  The work-claim counter comes from a static device array of
 * YRB_WORKSPACE_BYTES in the library, one copy per GPU, held until the
 * process ends; its address on a device is looked up on the first call
 * there.  It is the same size for every input, so no size is too large for
 * it.  Every call on a GPU shares that GPU's copy: calls that may overlap on
 * one GPU (two streams, or one captured graph replayed on two streams at
 * once) race on it and may skip or repeat work items; give such callers
 * attn_prefill_blockwise with workspaces of their own.  The counter needs
 * no clearing between calls: any value it holds claims every item once.
 * Arguments, results and errors otherwise as attn_prefill_blockwise; this
 * call allocates nothing and never synchronises.  YRB_EHIP if the array's
 * address cannot be found, YRB_EUNSUPPORTED past the 64th device.
 */
YRB_API int attn_prefill_blockwise_noalloc(const void* q, const void* k, const void* v, void* o,
                                   int32_t dtype, int64_t B, int64_t S, int64_t Hq, int64_t Hkv,
                                   int64_t D, const int64_t strides[4][3],
                                   const float* cos_sin, int64_t n_table_rows,
                                   float softmax_scale, int32_t causal, float* lse, void* stream);

/*
 * attn_prefill_sink_window -- attn_prefill_blockwise under the attention-sink
 * plus sliding-window mask, the prefill counterpart of the decode cache
 * ([C] "Sliding Window + Attention Sinks": the first s tokens and the last w
 * tokens; [J] "Attention sinks").  Key position n is visible to query
 * position t iff n <= t and (n < n_sink or n > t - window).  Key tiles that
 * no row of a query tile can see (between the sinks and the window) are
 * skipped, not masked, so the work per query tile is bounded by
 * n_sink + window + the tile, not by t.
 *
 * Arguments as attn_prefill_blockwise (workspace included), causal
 * implied, plus
 *   n_sink         >= 0; values above S act as S (every key a sink).
 *   window         >= 1; values above S act as S (plain causal).
 * dtype must be YRB_BF16 (YRB_EUNSUPPORTED otherwise); S < 2^30.
 */
YRB_API int attn_prefill_sink_window(const void* q, const void* k, const void* v, void* o,
                             int32_t dtype, int64_t B, int64_t S, int64_t Hq, int64_t Hkv,
                             int64_t D, const int64_t strides[4][3],
                             const float* cos_sin, int64_t n_table_rows,
                             float softmax_scale, int64_t n_sink, int64_t window,
                             float* lse, void* workspace, void* stream);

/*
 * attn_prefill_sink_window_chunk -- attn_prefill_sink_window for one chunk
 * of a longer sequence: the chunk's Sq queries against the sequence's first
 * Sk keys, under the same mask and with the same tile skipping, so a long
 * input can be prefilled chunk by chunk ([C] "Sliding Window + Attention
 * Sinks"; [J] "Attention sinks").  Positions are the sequence's own: query
 * s of the chunk sits at q_offset + s, key t at t; key t is visible to it
 * iff t <= q_offset + s and (t < n_sink or t > q_offset + s - window).
 * (A cache that evicts tokens and re-indexes positions is the decode's.)
 *
 *   q, o           device [B][Sq][Hq][D]   strides[0], strides[3]
 *   k, v           device [B][Sk][Hkv][D]  strides[1], strides[2]; k
 *                  already rotated at positions 0 .. Sk-1 (rope_apply).
 *                  Keys past a row's position are masked; the rows of the
 *                  chunk may see fewer keys when Sk < q_offset + Sq.
 *                  May be NULL when Sk = 0 (every row then sees no key:
 *                  output 0, lse -inf).
 *   q_offset       >= 0: position of the chunk's first query.
 *   cos_sin        NULL (q already rotated) or a table of n_table_rows >=
 *                  q_offset + Sq rows: q is rotated on load.
 *   lse            NULL or device [B][Hq][Sq] fp32.
 * Other arguments as attn_prefill_sink_window; n_sink values above Sk act
 * as Sk, windows above q_offset + Sq as q_offset + Sq.  dtype YRB_BF16
 * only; Sk < 2^30 and q_offset + Sq < 2^30.  q_offset = 0, Sq = Sk = S is
 * attn_prefill_sink_window.
 */
YRB_API int attn_prefill_sink_window_chunk(const void* q, const void* k, const void* v, void* o,
                                           int32_t dtype, int64_t B, int64_t Sq, int64_t Sk,
                                           int64_t Hq, int64_t Hkv, int64_t D,
                                           const int64_t strides[4][3], int64_t q_offset,
                                           const float* cos_sin, int64_t n_table_rows,
                                           float softmax_scale, int64_t n_sink, int64_t window,
                                           float* lse, void* workspace, void* stream);

/*
 * attn_block_accumulate -- one ring-attention step on one device: fold the
 * key/value block that just arrived into the local query block's state
 * ([J] "Ring attention": each device accumulates its block's contribution
 * as blocks rotate; [T] Sec. 5; [C] "Ring Attention": combined with online
 * softmax).
 *
 *   q              device [B][Sq][Hq][D]   strides[0], positions q_offset + s
 *   k_blk, v_blk   device [B][Sk][Hkv][D]  strides[1], strides[2],
 *                  positions k_offset + t
 *   k_blk must already be rotated at its positions (a ring device rotates
 *                  its own block once, before it travels around the ring).
 *   cos_sin        NULL (q already rotated) or a table covering q_offset+Sq
 *                  rows: q is then rotated on load.
 *   o_acc          device [B][Sq][Hq][D] fp32 contiguous: unnormalised sum of
 *                  exp(scaled logit - m) * v
 *   m, l           device [B][Hq][Sq] fp32 contiguous: running max of the
 *                  scaled logits and running sum of exp(logit - m) (natural
 *                  exp).  A row that has seen no key holds m = -inf, l = 0.
 *   flags          YRB_ACC_FIRST and/or YRB_ACC_FINALIZE.
 *   o_out          device [B][Sq][Hq][D] of dtype, o_strides; required iff
 *                  FINALIZE; rows with l = 0 are written as 0.
 *   workspace      NULL or YRB_WORKSPACE_BYTES of device memory, as for
 *                  attn_prefill_blockwise (bf16 only; fp32 ignores it).
 * With causal = 1 a block wholly in the future of every local query
 * (k_offset > q_offset + Sq - 1) contributes nothing ([T] FAQ 2); the call
 * still initialises (FIRST) and finalises (FINALIZE) as asked.  Folding the
 * blocks in any order gives the same result up to rounding.
 */
YRB_API int attn_block_accumulate(const void* q, const void* k_blk, const void* v_blk,
                          int32_t dtype, int64_t B, int64_t Sq, int64_t Sk,
                          int64_t Hq, int64_t Hkv, int64_t D,
                          const int64_t strides[3][3], int64_t q_offset, int64_t k_offset,
                          const float* cos_sin, int64_t n_table_rows,
                          float softmax_scale, int32_t causal,
                          float* o_acc, float* m, float* l, int32_t flags,
                          void* o_out, const int64_t o_strides[3], void* workspace,
                          void* stream);

/*
 * attn_decode_sink_window -- one new query per sequence against a cache of
 * n_sink attention-sink entries plus a sliding window of `window` entries
 * ([C] "Sliding Window + Attention Sinks": the cache is the first s tokens
 * and the last w tokens; [J] "Attention sinks").
 *
 *   q              device [B][Hq][D], q_strides (b, h)
 *   k_cache,
 *   v_cache        device [B][Hkv][C][D], C = n_sink + window, cache_strides
 *                  (b, h, slot); keys are stored un-rotated.
 *   o              device [B][Hq][D], o_strides (b, h)
 *   cache_len      device int32 [B]: entries present, 0 <= len <= C.
 *   ring_head      device int32 [B] or NULL (= 0): 0 <= head < window.
 * Entry e < len sits at position e (positions re-indexed inside the cache);
 * entry e < n_sink is in slot e, a window entry in slot
 * n_sink + (ring_head + e - n_sink) mod window.  The query sits at position
 * len - 1 (its own key/value were stored first) and sees every entry.
 * len = 0 gives o = 0; a len or ring_head out of range gives o = NaN for
 * that sequence (nothing out of range is read).  Needs n_table_rows >= C.
 */
YRB_API int attn_decode_sink_window(const void* q, const void* k_cache, const void* v_cache, void* o,
                            int32_t dtype, int64_t B, int64_t Hq, int64_t Hkv, int64_t D,
                            int64_t n_sink, int64_t window,
                            const int64_t q_strides[2], const int64_t cache_strides[3],
                            const int64_t o_strides[2],
                            const int32_t* cache_len, const int32_t* ring_head,
                            const float* cos_sin, int64_t n_table_rows,
                            float softmax_scale, void* stream);

/*
 * attn_decode_sink_window_fp8 -- attn_decode_sink_window over an FP8 K/V
 * cache, half the bytes of a bf16 one ([T] Sec. 7, FAQ 3: quantising the KV
 * cache to FP8).  The pages fix no format.  This reading takes OCP E4M3
 * codes (1 sign, 4 exponent bits with bias 7, 3 mantissa bits; no
 * infinities, S.1111.111 is NaN) and one fp32 dequantisation scale per
 * (sequence, key/value head) for K and one for V: a cached value is
 * scale * decode(code).  Everything else is as for attn_decode_sink_window.
 *
 *   q, o           device bf16 [B][Hq][D], q_strides / o_strides (b, h).
 *   k_cache,
 *   v_cache        device bytes [B][Hkv][C][D] of E4M3 codes, cache_strides
 *                  (b, h, slot) in bytes, each a multiple of 16; base
 *                  pointers 16-byte aligned (else YRB_EALIGN).
 *   k_scale,
 *   v_scale        device fp32 [B][Hkv] contiguous, or NULL (= 1).
 * A NaN code reaches the output as NaN.
 */
YRB_API int attn_decode_sink_window_fp8(const void* q, const void* k_cache, const void* v_cache, void* o,
                                int64_t B, int64_t Hq, int64_t Hkv, int64_t D,
                                int64_t n_sink, int64_t window,
                                const int64_t q_strides[2], const int64_t cache_strides[3],
                                const int64_t o_strides[2],
                                const int32_t* cache_len, const int32_t* ring_head,
                                const float* k_scale, const float* v_scale,
                                const float* cos_sin, int64_t n_table_rows,
                                float softmax_scale, void* stream);

/*
 * attn_decode_sink_window_ex -- the decode with both choices open: the cache
 * element type (YRB_BF16, or YRB_FP8_E4M3 as in attn_decode_sink_window_fp8,
 * with its scales) and the pair layout the keys and the query are rotated
 * in (YRB_LAYOUT_HALF or YRB_LAYOUT_INTERLEAVED).  Values are not rotated,
 * so the layout does not change how V or o are read and written.  Strides
 * and alignment follow the cache type as in the two calls above; scales are
 * ignored for bf16.
 */
YRB_API int attn_decode_sink_window_ex(const void* q, const void* k_cache, const void* v_cache, void* o,
                               int32_t cache_dtype, int32_t layout,
                               int64_t B, int64_t Hq, int64_t Hkv, int64_t D,
                               int64_t n_sink, int64_t window,
                               const int64_t q_strides[2], const int64_t cache_strides[3],
                               const int64_t o_strides[2],
                               const int32_t* cache_len, const int32_t* ring_head,
                               const float* k_scale, const float* v_scale,
                               const float* cos_sin, int64_t n_table_rows,
                               float softmax_scale, void* stream);

/* Human-readable name of a status code (static string). */
YRB_API const char* yrb_status_str(int status);

#ifdef __cplusplus
}
#endif

#endif /* YRB_H */
