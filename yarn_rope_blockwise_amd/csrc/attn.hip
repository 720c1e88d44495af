// Exact blockwise softmax attention with RoPE on the query load, for gfx950.
//
// What it computes (per batch b, query head h, query row i at position
// q_offset + i):
//   o_i = sum_j softmax_j(scale * q'_i . k'_j) v_j  over visible keys j,
// with causal visibility k_offset + j <= q_offset + i.  Keys are folded in
// tiles of 64 with a running row max m and row sum l ("Ring attention" in
// the jovanaeducation guide and "Ring Attention" in the 14cs17 notes: blocks
// are combined with the online softmax of FlashAttention-style kernels).
// The same kernel serves a whole prefill (no incoming state; finalize) and
// one ring step (state read from / written to HBM).
//
// gfx950 design (bf16):
//  * A workgroup is NW waves; each wave owns 32*NQT query rows of one head.
//    Q fragments stay in VGPRs for the whole launch, rotated on load in fp32
//    from the fp32 cos/sin table and rounded once to bf16.
//  * Scores are computed transposed, S^T = K Q^T, with
//    v_mfma_f32_32x32x16_bf16: the accumulator puts one query per lane
//    column, so row max/sum need only in-lane work plus one permlane32 swap,
//    and the same accumulator, packed to bf16, is directly the B operand of
//    O^T += V^T P^T (keys permuted consistently on both operands).
//  * K and V tiles go global -> LDS with global_load_lds_dwordx4 (no VGPR
//    staging), double-buffered, XOR-swizzled per row.  K feeds the MFMA A
//    operand with ds_read_b128; V is kept [key][d] and read transposed with
//    ds_read_b64_tr_b16.
//  * exp2 domain: scale*log2(e) folds into one FMA per score.  The running
//    max used for the exponentials is only moved when the true max exceeds
//    it by more than 8 (log2 units), so the O rescale is rare; the true max
//    is tracked exactly and restored before the state is stored.
//  * Causal: key tiles wholly in the future of the workgroup are never
//    loaded; waves skip tiles in their own future; only tiles that straddle
//    the diagonal (or the ragged end) are masked.
//  * Launch order: heaviest query tiles first; heads grouped per XCD so the
//    workgroups sharing a key/value head share an L2.
#include "attn_frag.h"
#include "common.h"
#include "kernels.h"

namespace yrb {

namespace {

template <int D, int BN, int NQT, int NW>
__global__ __launch_bounds__(NW * 64, 1) void attn_bf16_kernel(AttnArgs a, int64_t n_qtiles) {
  using T = Tile<D, BN>;
  constexpr int NDS = T::NDS;
  constexpr int QW = 32 * NQT;
  constexpr int BM = QW * NW;
  using TL = TileLoads<D, BN, NW>;

  // Double-buffered K and V tiles: [buf][K, V] (dynamic LDS, 4 * TILEB bytes).
  extern __shared__ __attribute__((aligned(1024))) char lds_raw[];
  YRB_LDS char* const K0 = (YRB_LDS char*)lds_raw;
  YRB_LDS char* const V0 = K0 + T::TILEB;
  YRB_LDS char* const K1 = K0 + 2 * T::TILEB;
  YRB_LDS char* const V1 = K0 + 3 * T::TILEB;

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);   // wave-uniform
  const int l32 = lane & 31;

  const WorkItem wi = work_item(a, n_qtiles);
  const int b = wi.b, h = wi.h, hk = wi.hk, qtile = wi.qtile;

  const int q0w = qtile * BM + wave * QW;                // first row of this wave
  const int Sq = (int)a.Sq, Sk = (int)a.Sk;
  const int q_offset = (int)a.q_offset, k_offset = (int)a.k_offset;

  bf16x8 qf[NQT][NDS];
  load_q<D, NQT>(a, b, h, q0w, lane, qf);
  WaveState<D, NQT> st;
  init_state<D, NQT>(a, b, h, q0w, lane, st);

  // Key tiles this workgroup needs.
  const int q_last_wg = q_offset + min(Sq, (qtile + 1) * BM) - 1;
  int n_keys = Sk;
  if (a.causal) n_keys = max(0, min(Sk, q_last_wg - k_offset + 1));
  const int n_tiles = (n_keys + BN - 1) / BN;
  const int qw_first = q_offset + q0w;
  const int qw_last = q_offset + min(Sq, q0w + QW) - 1;
  const bool wave_live = q0w < Sq;
  const float scale_log2 = a.softmax_scale * kLog2e;

  const __bf16* kbase = reinterpret_cast<const __bf16*>(a.k) + b * a.ks[0] + hk * a.ks[2];
  const __bf16* vbase = reinterpret_cast<const __bf16*>(a.v) + b * a.vs[0] + hk * a.vs[2];
  const int kstride = (int)a.ks[1], vstride = (int)a.vs[1];

  // Q, table and state loads are complete before the first tile is issued, so
  // no wait for them is left inside the tile loop.
  wait_vmcnt<0>();

  // One step: prefetch tile jt+1 into (kn, vn), fold tile jt from (kc, vc).
  auto step = [&](YRB_LDS char* kc, YRB_LDS char* vc, YRB_LDS char* kn, YRB_LDS char* vn,
                  int jt) {
    if (jt + 1 < n_tiles) {
      load_tile<D, BN, NW, false>(kn, kbase, kstride, (jt + 1) * BN, Sk, wave, lane);
      load_tile<D, BN, NW, true>(vn, vbase, vstride, (jt + 1) * BN, Sk, wave, lane);
      // all but the tile jt+1 loads this wave just issued (K and V)
      if (TL::EXTRA && wave < TL::EXTRA) wait_vmcnt<2 * (TL::LO + 1)>();
      else wait_vmcnt<2 * TL::LO>();
    } else {
      wait_vmcnt<0>();
    }
    // Tile jt has landed in LDS for this wave (vmcnt); the barrier makes it
    // so for all waves.  No fence: it would also wait for the prefetch.
    tile_barrier();
    const int k0 = jt * BN;
    const int kpos0 = k_offset + k0;
    const bool skip = !wave_live || (a.causal && kpos0 > qw_last);
    if (!skip) {
      const bool need_mask = (a.causal && kpos0 + BN - 1 > qw_first) || (k0 + BN > Sk);
      fold_tile<D, BN, NQT>(kc, vc, qf, st, need_mask, k0, Sk, kpos0, qw_first + l32,
                            a.causal != 0, scale_log2, lane);
    }
    // Every wave is done reading (kc, vc) before a later step refills them.
    tile_barrier();
  };

  if (n_tiles > 0) {
    load_tile<D, BN, NW, false>(K0, kbase, kstride, 0, Sk, wave, lane);
    load_tile<D, BN, NW, true>(V0, vbase, vstride, 0, Sk, wave, lane);
  }
  for (int jt = 0; jt < n_tiles; jt += 2) {
    step(K0, V0, K1, V1, jt);
    if (jt + 1 < n_tiles) step(K1, V1, K0, V0, jt + 1);
  }

  if (!wave_live) return;

  finish_rows<D, NQT>(a, b, h, q0w, lane, st);
}

// ---------------------------------------------------------------------------
// fp32 storage: one thread per query row, scalar fp32 FMAs, key tiles of 32
// staged in LDS.  Same visibility rules, state format and epilogue.
// ---------------------------------------------------------------------------
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

template <int D, int BN, int NQT, int NW>
hipError_t launch_bf16(const AttnArgs& a, hipStream_t stream) {
  constexpr int BM = 32 * NQT * NW;
  constexpr int LDS_BYTES = 4 * Tile<D, BN>::TILEB;
  const int64_t n_qtiles = (a.Sq + BM - 1) / BM;
  const int64_t blocks = n_qtiles * a.B * a.Hq;
  if (blocks == 0) return hipSuccess;
  if (LDS_BYTES > 65536) {   // above the default dynamic-LDS limit (gfx950 has 160 KiB)
    const hipError_t attr = hipFuncSetAttribute(
        reinterpret_cast<const void*>(&attn_bf16_kernel<D, BN, NQT, NW>),
        hipFuncAttributeMaxDynamicSharedMemorySize, LDS_BYTES);
    if (attr != hipSuccess) return attr;
  }
  hipLaunchKernelGGL((attn_bf16_kernel<D, BN, NQT, NW>), dim3((unsigned)blocks), dim3(NW * 64),
                     LDS_BYTES, stream, a, n_qtiles);
  return hipGetLastError();
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

// Keys per barrier step, query rows per wave (32 * NQT) and waves per
// workgroup of the bf16 kernel.
#ifndef YRB_PREFILL_BN
#define YRB_PREFILL_BN 64
#endif
#ifndef YRB_PREFILL_NQT
#define YRB_PREFILL_NQT 1
#endif
#ifndef YRB_PREFILL_NW
#define YRB_PREFILL_NW 8
#endif

#ifndef YRB_PREFILL_PIPELINED
#define YRB_PREFILL_PIPELINED 1
#endif

hipError_t launch_attention(int dtype, int D, const AttnArgs& a, hipStream_t stream) {
  constexpr int BN = YRB_PREFILL_BN, NQT = YRB_PREFILL_NQT, NW = YRB_PREFILL_NW;
  if (dtype == kBF16 && YRB_PREFILL_PIPELINED) return launch_attention_bf16_pp(D, a, stream);
  if (dtype == kBF16) return D == 64 ? launch_bf16<64, BN, NQT, NW>(a, stream)
                                     : launch_bf16<128, BN, NQT, NW>(a, stream);
  return D == 64 ? launch_f32<64>(a, stream) : launch_f32<128>(a, stream);
}

}  // namespace yrb
