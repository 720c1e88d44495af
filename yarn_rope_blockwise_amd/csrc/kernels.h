// Internal launch interface between the C-ABI layer (api.cpp) and the HIP
// kernels.  Arguments here are already validated.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace yrb {

enum DType { kBF16 = 0, kF32 = 1, kFP8E4M3 = 2 };

hipError_t launch_rope_tables(const double* theta, int half, int64_t pos0, int64_t n_pos,
                              float* cos_sin, hipStream_t stream);

struct RopeArgs {
  const void* x;
  void* y;
  int64_t xs[3];          // b, s, h strides (elements)
  int64_t ys[3];
  int64_t B, S, H;
  const float* cos_sin;
  int64_t n_rows;
  int64_t pos_offset;
  const int32_t* pos_ids; // [B][S] or null
};
hipError_t launch_rope_apply(int dtype, int D, bool interleaved, const RopeArgs& a, hipStream_t stream);

// One attention launch: prefill (no incoming state, finalize) or one ring
// step (optional incoming state, state out, optional finalize).
struct AttnArgs {
  const void* q;
  const void* k;
  const void* v;
  int64_t qs[3], ks[3], vs[3];   // b, s, h strides (elements)
  void* o;                       // finalized output (dtype) or null
  int64_t os[3];
  float* lse;                    // [B][Hq][Sq] natural log-sum-exp, or null
  float* o_acc;                  // state (accumulate mode) or null
  float* m;
  float* l;
  const float* cos_sin;          // rotate q on load when non-null
  int64_t B, Sq, Sk, Hq, Hkv;
  int64_t q_offset, k_offset;    // positions of q row 0 / k row 0
  float softmax_scale;
  int causal;
  int load_state;                // read (o_acc, m, l) first
  int store_state;               // write (o_acc, m, l) at the end
  int finalize;                  // write o (and lse) at the end
  // Sink+window mask (bf16 pipelined kernel only; window 0 = off): key
  // position n is visible to query position t iff n < n_sink or
  // n > t - window, on top of the causal rule.
  int n_sink;
  int window;
  // Work-claim counter in caller memory (bf16 pipelined kernel), or null:
  // every block then takes the work item of its index.
  unsigned* claims;
};
hipError_t launch_attention(int dtype, int D, const AttnArgs& a, hipStream_t stream);
// The software-pipelined bf16 kernel (attn_pp.hip); called by launch_attention.
hipError_t launch_attention_bf16_pp(int D, const AttnArgs& a, hipStream_t stream);

struct DecodeArgs {
  const void* q;
  const void* k;
  const void* v;
  void* o;
  int64_t qs[2];                 // b, h
  int64_t cs[3];                 // b, h, slot
  int64_t os[2];
  int64_t B, Hq, Hkv;
  int64_t n_sink, window;
  const int32_t* cache_len;
  const int32_t* ring_head;      // or null
  const float* cos_sin;
  float softmax_scale;
  const float* k_scale;          // fp8 caches: [B][Hkv] dequantisation scales, or null (1)
  const float* v_scale;
};
hipError_t launch_decode(int cache_dtype, int D, bool interleaved, const DecodeArgs& a,
                         hipStream_t stream);

}  // namespace yrb
