// Exact blockwise softmax attention with RoPE on the query load, for gfx950:
// the software-pipelined bf16 kernel.  It computes the same thing as the
// kernel in attn.hip (per query row, softmax-weighted sum of the visible
// values, keys folded in with a running max and running sum; the update of
// "Ring attention" in the jovanaeducation guide and of "Ring Attention" in
// the 14cs17 notes), with a different mapping onto the CU:
//
//  * One wave per SIMD (4 waves, 256 query rows per workgroup), each wave
//    owning 64 rows as two 32-row query tiles.  Every K/V fragment read from
//    LDS then feeds twice the MFMA work it does with 32 rows per wave, which
//    halves LDS read traffic per flop; the wave holds up to 512 registers.
//  * With a single wave on the SIMD, MFMA and softmax VALU work overlap only
//    inside the wave.  The two query tiles are run half a step apart:
//        H1(q): MFMA  S1(q) = K(q) Q1^T,  O1 += V(q-1)^T P1(q-1)
//               VALU  softmax of S0(q) -> P0(q)
//        H2(q): MFMA  S0(q+1) = K(q+1) Q0^T,  O0 += V(q)^T P0(q)
//               VALU  softmax of S1(q) -> P1(q)
//    (q counts 32-key quarters), so the MFMAs of each half are independent
//    of the VALU work beside them.  The LDS reads of K(q+1) and V(q) are
//    issued in H1(q), a half step ahead of their use.
//  * The softmax of a quarter is branch-free: when the running max grows by
//    more than the lazy-rescale threshold, l and m move at once and the
//    O-accumulator rescale is applied at the boundary between half steps,
//    after the last product into that accumulator under the old max.
//  * Key tiles of 64 go global -> LDS with LDS-DMA into four buffers, two
//    tiles ahead, with one workgroup barrier per tile.  Tiles visible to
//    every row of the workgroup run through the pipeline; the few tiles on
//    the causal diagonal or at the ragged end of the keys are folded
//    afterwards, masked, by the plain per-quarter loop.
#include "attn_frag.h"
#include "common.h"
#include "kernels.h"

#include <type_traits>

namespace yrb {

namespace {

constexpr int kPPWaves = 4;    // one per SIMD
constexpr int kPPBN = 64;      // keys per tile (two quarters)
constexpr int kPPBufs = 4;     // LDS tile buffers (power of two)

// S^T of 32 keys against one 32-row query tile, accumulated onto `init`.
template <int D>
__device__ __forceinline__ f32x16 qk_tile(const bf16x8 (&kf)[D / 16], const bf16x8 (&q)[D / 16],
                                          const f32x16& init) {
  f32x16 s = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf[0], q[0], init, 0, 0, 0);
#pragma unroll
  for (int ds = 1; ds < D / 16; ++ds) s = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf[ds], q[ds], s, 0, 0, 0);
  return s;
}

// O^T += V^T P^T for 32 keys and query tile QT.
template <int D, int QT>
__device__ __forceinline__ void pv_tile(const bf16x8 (&vf)[2][D / 32], const bf16x8 (&pf)[2],
                                        WaveState<D, 2>& st) {
#pragma unroll
  for (int half = 0; half < 2; ++half)
#pragma unroll
    for (int dt = 0; dt < D / 32; ++dt)
      st.o[dt][QT] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vf[half][dt], pf[half], st.o[dt][QT], 0, 0, 0);
}

// IEEE maximum (v_maximum3_f32 on gfx950: no input canonicalisation).
__device__ __forceinline__ float vmax(float a, float b) { return __builtin_elementwise_maximum(a, b); }
__device__ __forceinline__ float pair_vmax(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return vmax(__uint_as_float(r[0]), __uint_as_float(r[1]));
}

// Sixteen copies of v, built as eight copies of a 64-bit pair (v_mov_b64).
__device__ __forceinline__ f32x16 splat16(float v) {
  typedef unsigned long long u64x8 __attribute__((ext_vector_type(8)));
  const unsigned long long u = __float_as_uint(v);
  const unsigned long long p = (u << 32) | u;
  const u64x8 r = {p, p, p, p, p, p, p, p};
  return __builtin_bit_cast(f32x16, r);
}

// Scores come out of the MFMA already in log2 units (Q is pre-multiplied by
// softmax_scale * log2(e)) and offset: each S chain starts from -base, base
// being the max the exponentials use (0 while a row has none).  Then, as
// long as no row max grows past that max by more than the threshold,
// P = exp2(S) needs no per-element subtraction.
struct Offsets {
  float base[2];       // the S chains of the tile start from -base
  float mu_tau[2];     // m_use + threshold
  float l_prev[2];     // row sum before the current quarter
};

template <int D>
__device__ __forceinline__ void offsets_from(const WaveState<D, 2>& st, Offsets& of) {
#pragma unroll
  for (int t = 0; t < 2; ++t) {
    const float mu = st.m_use[t];
    of.base[t] = mu == -INFINITY ? 0.f : mu;
    of.mu_tau[t] = mu + kTau;
    of.l_prev[t] = st.l[t];
  }
}

// Common case of the online-softmax update of query tile QT over 32 keys
// that are all visible: row max, exact running max, P = exp2(S) packed to
// bf16 as the B operand of O^T += V^T P^T, and the row sum taken over the
// bf16 values the product uses.  Returns whether the row max outgrew the
// threshold, in which case settle() redoes P with a new max.
template <int D, int QT>
__device__ __forceinline__ bool softmax_fast(const f32x16& s, WaveState<D, 2>& st, Offsets& of,
                                             bf16x8 (&pf)[2]) {
  float mx = vmax(s[0], s[1]);
#pragma unroll
  for (int j = 2; j < 16; ++j) mx = vmax(mx, s[j]);
  const float t1 = of.base[QT] + pair_vmax(mx);   // this quarter's row max
  st.m_true[QT] = vmax(st.m_true[QT], t1);
  const bool grow = t1 > of.mu_tau[QT];
  of.l_prev[QT] = st.l[QT];
  const bf16x2 ones = {(__bf16)1.0f, (__bf16)1.0f};
  float acc = st.l[QT];
#pragma unroll
  for (int half = 0; half < 2; ++half) {
    u32x4 w;
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int j = 8 * half + 2 * u;
      // The pair is packed into its own bf16x2 before the dot product: taking
      // it as an element of the u32x4 miscompiled (every dot2 read element 0).
      const bf16x2 pp = {(__bf16)fast_exp2(s[j]), (__bf16)fast_exp2(s[j + 1])};
      acc = __builtin_amdgcn_fdot2_f32_bf16(pp, ones, acc, false);
      w[u] = __builtin_bit_cast(unsigned, pp);
    }
    pf[half] = __builtin_bit_cast(bf16x8, w);
  }
  st.l[QT] = acc;
  return grow;
}

// Rare case, at the boundary after the last product into O of tile QT under
// the old max: rows that grew take their exact max as the new base, P and
// the row sum are redone against it, O is rescaled, and the S chains of the
// following quarters start from the new base.
template <int D, int QT>
__device__ __forceinline__ void settle(const f32x16& s, WaveState<D, 2>& st, Offsets& of, bool grow,
                                       bf16x8 (&pf)[2]) {
  if (__builtin_expect(__builtin_amdgcn_ballot_w64(grow) == 0, 1)) return;
  // A side effect, so the compiler keeps this block behind its branch rather
  // than computing it on every quarter and selecting.
  asm volatile("");
  const float mu_old = st.m_use[QT];
  const float mu_new = grow ? st.m_true[QT] : mu_old;
  const float shift = mu_new - of.base[QT];                          // 0 where kept
  const float alpha = grow ? fast_exp2(mu_old - mu_new) : 1.0f;      // 0 from an empty row
  const bf16x2 ones = {(__bf16)1.0f, (__bf16)1.0f};
  float acc = of.l_prev[QT] * alpha;
#pragma unroll
  for (int half = 0; half < 2; ++half) {
    u32x4 w;
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int j = 8 * half + 2 * u;
      const bf16x2 pp = {(__bf16)fast_exp2(s[j] - shift), (__bf16)fast_exp2(s[j + 1] - shift)};
      acc = __builtin_amdgcn_fdot2_f32_bf16(pp, ones, acc, false);
      w[u] = __builtin_bit_cast(unsigned, pp);
    }
    pf[half] = __builtin_bit_cast(bf16x8, w);
  }
  st.l[QT] = acc;
#pragma unroll
  for (int dt = 0; dt < D / 32; ++dt) st.o[dt][QT] *= alpha;
  st.m_use[QT] = mu_new;
  of.base[QT] = mu_new == -INFINITY ? 0.f : mu_new;
  of.mu_tau[QT] = mu_new + kTau;
}

// Keep the computation of P inside its half step (a use of its registers
// there, so nothing sinks it into the next block).
#ifndef YRB_PP_FAST_DMA
#define YRB_PP_FAST_DMA 1
#endif
__device__ __forceinline__ void keep(const bf16x8 (&pf)[2]) { asm volatile("" ::"v"(pf[0]), "v"(pf[1])); }

// Issue order of one half step: each MFMA followed by a few VALU
// instructions (and, in H1, the LDS reads for the next half step), so the
// VALU work and the reads go out while the matrix core is busy and no MFMA
// waits on the one before it.  Masks: 0x008 MFMA, 0x002 VALU, 0x100 DS read.
#ifndef YRB_PP_VALU_PER_MFMA
#define YRB_PP_VALU_PER_MFMA 4
#endif
#ifndef YRB_PP_INTERLEAVE
#define YRB_PP_INTERLEAVE 1
#endif
template <int NMFMA, int NDS_READ>
__device__ __forceinline__ void interleave() {
  if (!YRB_PP_INTERLEAVE) return;
#pragma unroll
  for (int i = 0; i < NMFMA; ++i) {
    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
    if (i < (NDS_READ + 1) / 2) __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
    __builtin_amdgcn_sched_group_barrier(0x002, YRB_PP_VALU_PER_MFMA, 0);
  }
}

template <int D>
__global__ __launch_bounds__(kPPWaves * 64, 1) void attn_bf16_pp_kernel(AttnArgs a, int64_t n_qtiles) {
  constexpr int NW = kPPWaves, BN = kPPBN, QW = 64, BM = NW * QW;
  constexpr int NDS = D / 16, NDT = D / 32;
  using T = Tile<D, BN>;
  using TL = TileLoads<D, BN, NW>;
  static_assert(TL::EXTRA == 0, "tile DMA must split evenly over the waves");
  constexpr int DMA = 2 * TL::LO;   // LDS-DMA instructions per wave per tile (K and V)

  // kPPBufs x [K tile, V tile] (dynamic LDS).
  extern __shared__ __attribute__((aligned(1024))) char lds_raw[];
  YRB_LDS char* const lds = (YRB_LDS char*)lds_raw;
  auto kbuf = [&](int t) -> YRB_LDS char* { return lds + (t & (kPPBufs - 1)) * 2 * T::TILEB; };
  auto vbuf = [&](int t) -> YRB_LDS char* { return kbuf(t) + T::TILEB; };

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int l32 = lane & 31;
  const WorkItem wi = work_item(a, n_qtiles);
  const int b = wi.b, h = wi.h, hk = wi.hk, qtile = wi.qtile;
  const int q0w = qtile * BM + wave * QW;
  const int Sq = (int)a.Sq, Sk = (int)a.Sk;
  const int q_offset = (int)a.q_offset, k_offset = (int)a.k_offset;

  // Q rotated and pre-multiplied by softmax_scale * log2(e): scores come out
  // of the MFMA in log2 units.
  bf16x8 qf[2][NDS];
  load_q<D, 2>(a, b, h, q0w, lane, qf, a.softmax_scale * kLog2e);
  // Q stays in AGPRs for the whole launch (an MFMA reads its A/B operands
  // from either register file); VGPRs hold O, S, P and the addresses.
#pragma unroll
  for (int t = 0; t < 2; ++t)
#pragma unroll
    for (int ds = 0; ds < NDS; ++ds) asm volatile("" : "+a"(qf[t][ds]));
  WaveState<D, 2> st;
  init_state<D, 2>(a, b, h, q0w, lane, st);

  // Key tiles: n_tiles reach the workgroup's last visible key; the first
  // n_full are visible to every row of the workgroup and hold no key past Sk.
  const int q_first_wg = q_offset + qtile * BM;
  const int q_last_wg = q_offset + min(Sq, (qtile + 1) * BM) - 1;
  int n_keys = Sk;
  if (a.causal) n_keys = max(0, min(Sk, q_last_wg - k_offset + 1));
  const int n_tiles = (n_keys + BN - 1) / BN;
  int n_full = min(n_tiles, Sk / BN);
  if (a.causal) n_full = min(n_full, max(0, q_first_wg - k_offset + 1) / BN);
  const int qw_first = q_offset + q0w;
  const int qw_last = q_offset + min(Sq, q0w + QW) - 1;
  const bool wave_live = q0w < Sq;

  const __bf16* kbase = reinterpret_cast<const __bf16*>(a.k) + b * a.ks[0] + hk * a.ks[2];
  const __bf16* vbase = reinterpret_cast<const __bf16*>(a.v) + b * a.vs[0] + hk * a.vs[2];
  const int kstride = (int)a.ks[1], vstride = (int)a.vs[1];

  // Q, table and state loads complete here, so the only vector-memory
  // operations in flight below are the tile DMAs.
  wait_vmcnt<0>();

  unsigned koff[TL::LO], voff[TL::LO];
  tile_offsets<D, BN, NW, false>(kstride, wave, lane, koff);
  tile_offsets<D, BN, NW, true>(vstride, wave, lane, voff);
  // Lane offsets of the fast DMA are 32-bit: (BN - 1) rows of stride plus a row.
  const bool fast_dma = (int64_t)max(kstride, vstride) * BN * 2 < ((int64_t)1 << 31);
  auto issue = [&](int t) {
    if (YRB_PP_FAST_DMA && fast_dma && (t + 1) * BN <= Sk) {
      load_tile_rows<D, BN, NW>(kbuf(t), kbase + (int64_t)t * BN * kstride, koff, wave);
      load_tile_rows<D, BN, NW>(vbuf(t), vbase + (int64_t)t * BN * vstride, voff, wave);
    } else {   // the ragged last tile: rows past the end read the last row
      load_tile<D, BN, NW, false>(kbuf(t), kbase, kstride, t * BN, Sk, wave, lane);
      load_tile<D, BN, NW, true>(vbuf(t), vbase, vstride, t * BN, Sk, wave, lane);
    }
  };
  // Before the first LDS read of tile t: this wave's DMA of tile t is done
  // (only tile t+1's may still be in flight), the barrier extends that to
  // every wave and certifies that every wave is past its reads of tile t-2,
  // whose buffer then takes tile t+2.
  auto arrive = [&](int t) {
    if (t + 1 < n_tiles) wait_vmcnt<DMA>();
    else wait_vmcnt<0>();
    tile_barrier();
    if (t + 2 < n_tiles) issue(t + 2);
  };
  if (n_tiles > 0) issue(0);
  if (n_tiles > 1) issue(1);

  if (n_full > 0) {
    bf16x8 kf[2][NDS];        // K(q) by quarter parity
    bf16x8 vf[2][2][NDT];     // V(q) by quarter parity
    bf16x8 p0[2], p1[2];
    f32x16 s0, s1;
    // The product of the quarter before the first is a no-op: P = V = 0.
#pragma unroll
    for (int half = 0; half < 2; ++half) {
      p1[half] = (bf16x8){};
#pragma unroll
      for (int dt = 0; dt < NDT; ++dt) vf[1][half][dt] = (bf16x8){};
    }
    Offsets of;
    offsets_from<D>(st, of);
    arrive(0);
    read_k_quarter<D>(kbuf(0), 0, lane, kf[0]);
    s0 = qk_tile<D>(kf[0], qf[0], splat16(-of.base[0]));

    // Quarters 2t and 2t+1 of tile t; LAST: no tile follows in the pipeline.
    auto tile = [&](int t, auto last_tag) {
      constexpr bool LAST = decltype(last_tag)::value;
      bool g;
      // H1(2t)
      read_k_quarter<D>(kbuf(t), 1, lane, kf[1]);
      read_v_quarter<D>(vbuf(t), 0, lane, vf[0]);
      s1 = qk_tile<D>(kf[0], qf[1], splat16(-of.base[1]));
      pv_tile<D, 1>(vf[1], p1, st);
      g = softmax_fast<D, 0>(s0, st, of, p0);
      keep(p0);
      interleave<4 * NDS / 2, NDS + 2 * NDT * 2>();
      settle<D, 0>(s0, st, of, g, p0);
      // H2(2t)
      s0 = qk_tile<D>(kf[1], qf[0], splat16(-of.base[0]));
      pv_tile<D, 0>(vf[0], p0, st);
      g = softmax_fast<D, 1>(s1, st, of, p1);
      keep(p1);
      interleave<4 * NDS / 2, 0>();
      settle<D, 1>(s1, st, of, g, p1);
      if constexpr (!LAST) arrive(t + 1);
      // H1(2t+1)
      if constexpr (!LAST) read_k_quarter<D>(kbuf(t + 1), 0, lane, kf[0]);
      read_v_quarter<D>(vbuf(t), 1, lane, vf[1]);
      s1 = qk_tile<D>(kf[1], qf[1], splat16(-of.base[1]));
      pv_tile<D, 1>(vf[0], p1, st);
      g = softmax_fast<D, 0>(s0, st, of, p0);
      keep(p0);
      interleave<4 * NDS / 2, (LAST ? 0 : NDS) + 2 * NDT * 2>();
      settle<D, 0>(s0, st, of, g, p0);
      // H2(2t+1)
      if constexpr (!LAST) s0 = qk_tile<D>(kf[0], qf[0], splat16(-of.base[0]));
      pv_tile<D, 0>(vf[1], p0, st);
      g = softmax_fast<D, 1>(s1, st, of, p1);
      keep(p1);
      interleave<(LAST ? 2 : 4) * NDS / 2, 0>();
      settle<D, 1>(s1, st, of, g, p1);
    };
    for (int t = 0; t + 1 < n_full; ++t) tile(t, std::false_type{});
    tile(n_full - 1, std::true_type{});
    pv_tile<D, 1>(vf[1], p1, st);
  }

  // Diagonal and ragged tiles: masked, per wave, skipping tiles wholly in
  // the wave's future (the barrier sequence stays the same for all waves).
  for (int t = n_full; t < n_tiles; ++t) {
    arrive(t);
    const int k0 = t * BN;
    const int kpos0 = k_offset + k0;
    const bool skip = !wave_live || (a.causal && kpos0 > qw_last);
    if (!skip) {
      const bool need_mask = (a.causal && kpos0 + BN - 1 > qw_first) || (k0 + BN > Sk);
      fold_tile<D, BN, 2>(kbuf(t), vbuf(t), qf, st, need_mask, k0, Sk, kpos0, qw_first + l32,
                          a.causal != 0, 1.0f, lane);   // Q carries the scale
    }
  }

  if (!wave_live) return;
  finish_rows<D, 2>(a, b, h, q0w, lane, st);
}

template <int D>
hipError_t launch_pp(const AttnArgs& a, hipStream_t stream) {
  constexpr int BM = kPPWaves * 64;
  constexpr int LDS_BYTES = kPPBufs * 2 * Tile<D, kPPBN>::TILEB;
  static_assert(LDS_BYTES <= 160 * 1024, "gfx950 LDS");
  const int64_t n_qtiles = (a.Sq + BM - 1) / BM;
  const int64_t blocks = n_qtiles * a.B * a.Hq;
  if (blocks == 0) return hipSuccess;
  if (LDS_BYTES > 65536) {   // above the default dynamic-LDS limit
    const hipError_t attr = hipFuncSetAttribute(reinterpret_cast<const void*>(&attn_bf16_pp_kernel<D>),
                                                hipFuncAttributeMaxDynamicSharedMemorySize, LDS_BYTES);
    if (attr != hipSuccess) return attr;
  }
  hipLaunchKernelGGL((attn_bf16_pp_kernel<D>), dim3((unsigned)blocks), dim3(kPPWaves * 64), LDS_BYTES,
                     stream, a, n_qtiles);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_attention_bf16_pp(int D, const AttnArgs& a, hipStream_t stream) {
  return D == 64 ? launch_pp<64>(a, stream) : launch_pp<128>(a, stream);
}

}  // namespace yrb
