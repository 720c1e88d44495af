// Exact blockwise softmax attention: the launch dispatcher, and the kernel
// for fp32 storage.
//
// What both storage types compute (per batch b, query head h, query row i at
// position q_offset + i):
//   o_i = sum_j softmax_j(scale * q'_i . k'_j) v_j  over visible keys j,
// with causal visibility k_offset + j <= q_offset + i.  Keys are folded in
// tiles with a running row max m and row sum l ("Ring attention" in the
// jovanaeducation guide and "Ring Attention" in the 14cs17 notes: blocks are
// combined with the online softmax of FlashAttention-style kernels).  The
// same kernel serves a whole prefill (no incoming state; finalize) and one
// ring step (state read from / written to HBM).
//
// bf16 storage runs on the software-pipelined MFMA kernel (attn_pp.hip).
// fp32 storage, the small parity configuration, runs here: one query row
// per thread, scalar fp32 FMAs, key tiles of 32 staged in LDS, with the
// same visibility rules, state format and epilogue.
#include "common.h"
#include "kernels.h"

namespace yrb {

namespace {

template <int D>
__global__ __launch_bounds__(64) void attn_f32_kernel(AttnArgs a) {
  constexpr int BNF = 32;
  __shared__ float k_s[BNF][D];
  __shared__ float v_s[BNF][D];
  const int tid = threadIdx.x;
  const int64_t row0 = (int64_t)blockIdx.x * 64;
  const int64_t row = row0 + tid;
  const int h = blockIdx.y;
  const int64_t b = blockIdx.z;
  const int hk = h / (int)(a.Hq / a.Hkv);
  const int64_t Sq = a.Sq, Sk = a.Sk;
  const bool live = row < Sq;
  const int64_t rc = imin64(row, Sq - 1);
  const float scale_log2 = a.softmax_scale * kLog2e;

  float q[D];
  const float* qp = reinterpret_cast<const float*>(a.q) + b * a.qs[0] + rc * a.qs[1] + h * a.qs[2];
  for (int d = 0; d < D; ++d) q[d] = qp[d];
  if (a.cos_sin) {
    const float* cs = a.cos_sin + (a.q_offset + rc) * D;
    for (int i = 0; i < D / 2; ++i) {
      const float c = cs[2 * i], s = cs[2 * i + 1];
      const float x = q[i], z = q[i + D / 2];
      q[i] = x * c - z * s;
      q[i + D / 2] = x * s + z * c;
    }
  }
  float o[D];
  for (int d = 0; d < D; ++d) o[d] = 0.f;
  float m = -INFINITY, l = 0.f;
  const int64_t ml = (b * a.Hq + h) * Sq + rc;
  if (a.load_state && live) {
    const float m0 = a.m[ml];
    m = (m0 == -INFINITY) ? -INFINITY : m0 * kLog2e;
    l = a.l[ml];
    const float* op = a.o_acc + ((b * Sq + row) * a.Hq + h) * D;
    for (int d = 0; d < D; ++d) o[d] = op[d];
  }
  const int64_t qpos = a.q_offset + rc;
  const int64_t q_last = a.q_offset + imin64(Sq, row0 + 64) - 1;
  int64_t n_keys = Sk;
  if (a.causal) n_keys = imax64(0, imin64(Sk, q_last - a.k_offset + 1));
  const float* kb = reinterpret_cast<const float*>(a.k) + b * a.ks[0] + hk * a.ks[2];
  const float* vb = reinterpret_cast<const float*>(a.v) + b * a.vs[0] + hk * a.vs[2];
  for (int64_t k0 = 0; k0 < n_keys; k0 += BNF) {
    __syncthreads();
    for (int e = tid; e < BNF * D; e += 64) {
      const int r = e / D, d = e % D;
      const int64_t kr = imin64(k0 + r, Sk - 1);
      k_s[r][d] = kb[kr * a.ks[1] + d];
      v_s[r][d] = vb[kr * a.vs[1] + d];
    }
    __syncthreads();
    float s[BNF];
    float mx = -INFINITY;
    for (int j = 0; j < BNF; ++j) {
      float acc = 0.f;
      for (int d = 0; d < D; ++d) acc = __builtin_fmaf(q[d], k_s[j][d], acc);
      const bool bad = (k0 + j >= Sk) || (a.causal && a.k_offset + k0 + j > qpos);
      s[j] = bad ? -INFINITY : acc * scale_log2;
      mx = fmaxf(mx, s[j]);
    }
    const float mn = fmaxf(m, mx);
    if (mn == -INFINITY) continue;
    const float alpha = (m == -INFINITY) ? 0.f : fast_exp2(m - mn);
    l *= alpha;
    for (int d = 0; d < D; ++d) o[d] *= alpha;
    for (int j = 0; j < BNF; ++j) {
      const float p = fast_exp2(s[j] - mn);
      l += p;
      for (int d = 0; d < D; ++d) o[d] = __builtin_fmaf(p, v_s[j][d], o[d]);
    }
    m = mn;
  }
  if (!live) return;
  if (a.store_state) {
    a.m[ml] = (m == -INFINITY) ? -INFINITY : m * kLn2;
    a.l[ml] = l;
    float* op = a.o_acc + ((b * Sq + row) * a.Hq + h) * D;
    for (int d = 0; d < D; ++d) op[d] = o[d];
  }
  if (a.finalize) {
    const float inv = l > 0.f ? 1.0f / l : 0.f;
    float* op = reinterpret_cast<float*>(a.o) + b * a.os[0] + row * a.os[1] + h * a.os[2];
    for (int d = 0; d < D; ++d) op[d] = o[d] * inv;
    if (a.lse) a.lse[ml] = l > 0.f ? (m + __log2f(l)) * kLn2 : -INFINITY;
  }
}

template <int D>
hipError_t launch_f32(const AttnArgs& a, hipStream_t stream) {
  const int64_t nq = (a.Sq + 63) / 64;
  if (nq == 0 || a.B == 0 || a.Hq == 0) return hipSuccess;
  hipLaunchKernelGGL((attn_f32_kernel<D>), dim3((unsigned)nq, (unsigned)a.Hq, (unsigned)a.B),
                     dim3(64), 0, stream, a);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_attention(int dtype, int D, const AttnArgs& a, hipStream_t stream) {
  if (dtype == kBF16) return launch_attention_bf16_pp(D, a, stream);
  return D == 64 ? launch_f32<64>(a, stream) : launch_f32<128>(a, stream);
}

}  // namespace yrb
