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
#include "common.h"
#include "kernels.h"

namespace yrb {

namespace {

constexpr float kTau = 8.0f;   // lazy-rescale threshold (log2 units)

template <int D, int BN_>
struct Tile {
  static constexpr int BN = BN_;            // keys per barrier step (64 or 128)
  static constexpr int NKQ = BN / 32;       // 32-key quarters per step
  static constexpr int ROWB = D * 2;        // bytes per K/V row in LDS
  static constexpr int TILEB = BN * ROWB;   // bytes per K or V tile
  static constexpr int NDS = D / 16;        // k-steps of S^T = K Q^T
  static constexpr int NDT = D / 32;        // d tiles of O^T
};

// K tile: physical 16-byte chunk = logical chunk ^ ksw(row); makes the 16
// lanes of each ds_read_b128 quarter hit distinct banks.
template <int D>
__device__ __forceinline__ int ksw(int r) {
  return D == 128 ? (r & 15) : ((r >> 1) & 7);
}
// V tile: XOR on 64-byte blocks; the 4 rows of each transposed half-wave
// read land in distinct bank quarters.
template <int D>
__device__ __forceinline__ int vsw(int r) {
  return D == 128 ? ((r & 3) << 2) : (((r >> 1) & 1) << 2);
}

// s_waitcnt vmcnt(n) (gfx9 encoding), other counters untouched.
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
}

// Workgroup barrier that no memory access may cross in either direction at
// compile time (the LDS-DMA below is invisible to the compiler's model).
__device__ __forceinline__ void tile_barrier() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

// One tile (BN rows of K or V) global -> LDS.  The tile is TILEB/1024
// DMA instructions of 1 KiB; wave w issues instructions w, w+NW, ...  Rows
// past the end are clamped to the last row: finite data, masked out of the
// softmax.
template <int D, int BN, int NW>
struct TileLoads {
  static constexpr int INSTR = Tile<D, BN>::TILEB / 1024;
  static constexpr int LO = INSTR / NW;                // every wave issues at least LO
  static constexpr int EXTRA = INSTR % NW;             // waves < EXTRA issue LO + 1
};

template <int D, int BN, int NW, bool IS_V>
__device__ __forceinline__ void load_tile(YRB_LDS char* dst, const __bf16* src, int stride, int k0,
                                          int Sk, int wave, int lane) {
  using T = Tile<D, BN>;
  using TL = TileLoads<D, BN, NW>;
  constexpr int ROWB = T::ROWB;
#pragma unroll
  for (int n = 0; n < TL::LO + (TL::EXTRA ? 1 : 0); ++n) {
    const int idx = n * NW + wave;
    if (n >= TL::LO && idx >= TL::INSTR) break;   // wave-uniform
    const int base = idx * 1024;
    const int off = base + lane * 16;
    const int r = off / ROWB;
    const int p = (off % ROWB) >> 4;
    const int c = IS_V ? (p ^ vsw<D>(r)) : (p ^ ksw<D>(r));
    const int row = min(k0 + r, Sk - 1);
    const __bf16* g = src + (int64_t)row * stride + c * 8;
    // global_load_lds_dwordx4: lane i's 16 bytes land at M0 + 16*i.  Issued
    // from asm so the compiler does not add a vmcnt(0) before every LDS read
    // of the other buffer; ordering is by the explicit vmcnt waits and
    // barriers around fold_tile.  No register outputs.
    const unsigned m0v = (unsigned)(uintptr_t)(dst + base);
#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"   // m0 is reserved; nothing else here uses it
    asm volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, off"
                 :
                 : "v"(g), "s"(m0v)
                 : "memory", "m0");
#pragma clang diagnostic pop
  }
}

template <int D, int NQT>
struct WaveState {
  f32x16 o[D / 32][NQT];
  float m_use[NQT];    // max the exponentials are taken against (log2 units)
  float m_true[NQT];   // exact running max (log2 units)
  float l[NQT];        // per-lane partial row sum (this half's keys)
};

// K fragments (A operand of S^T = K Q^T) of quarter kq: lane holds key
// 32kq + l32, dims 16ds + 8hh .. +7.
template <int D>
__device__ __forceinline__ void read_k_quarter(const YRB_LDS char* kt_lds, int kq, int lane,
                                               bf16x8 (&kf)[D / 16]) {
  constexpr int ROWB = D * 2;
  const int hh = lane >> 5;
  const int r = kq * 32 + (lane & 31);
#pragma unroll
  for (int ds = 0; ds < D / 16; ++ds) {
    const int c = 2 * ds + hh;
    kf[ds] = *reinterpret_cast<const YRB_LDS bf16x8*>(kt_lds + r * ROWB + ((c ^ ksw<D>(r)) << 4));
  }
}

// S^T for 32 keys against the wave's queries:
// s[qt][j] = q(row qt*32 + l32) . k(key 32kq + 8(j/4) + 4hh + j%4).
template <int D, int NQT>
__device__ __forceinline__ void qk_mfma(const bf16x8 (&kf)[D / 16],
                                        const bf16x8 (&qf)[NQT][D / 16], f32x16 (&s)[NQT]) {
#pragma unroll
  for (int qt = 0; qt < NQT; ++qt) s[qt] = (f32x16){};
#pragma unroll
  for (int ds = 0; ds < D / 16; ++ds)
#pragma unroll
    for (int qt = 0; qt < NQT; ++qt)
      s[qt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf[ds], qf[qt][ds], s[qt], 0, 0, 0);
}

// V^T fragments (A operand of O^T += V^T P^T) of quarter kq.  Lane i
// supplies the address of V[row][d..d+3] with row = 16ks + 8*second +
// 4(i/32) + (i%16)/4 and d = 32dt + 16((i/16)%2) + 4(i%4);
// ds_read_b64_tr_b16 hands lane l the column d = 32dt + l%32 over keys
// 16ks + 8*second + 4(l/32) + 0..3, the key order the packed P uses.
template <int D>
__device__ __forceinline__ void read_v_quarter(const YRB_LDS char* vt_lds, int kq, int lane,
                                               bf16x8 (&vf)[2][D / 32]) {
  constexpr int ROWB = D * 2;
  const int g = lane >> 4;
  const int t4 = (lane & 15) >> 2;
  const int s4 = lane & 3;
#pragma unroll
  for (int half = 0; half < 2; ++half) {
    const int ks = 2 * kq + half;
    const int row1 = 16 * ks + 4 * (g >> 1) + t4;
    const int row2 = row1 + 8;
#pragma unroll
    for (int dt = 0; dt < D / 32; ++dt) {
      const int c = dt * 4 + 2 * (g & 1) + (s4 >> 1);
      const int boff = 8 * (s4 & 1);
      const YRB_LDS char* a1 = vt_lds + row1 * ROWB + ((c ^ vsw<D>(row1)) << 4) + boff;
      const YRB_LDS char* a2 = vt_lds + row2 * ROWB + ((c ^ vsw<D>(row2)) << 4) + boff;
      const i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((YRB_LDS i16x4*)a1);
      const i16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((YRB_LDS i16x4*)a2);
      const u32x2 lo2 = __builtin_bit_cast(u32x2, lo);
      const u32x2 hi2 = __builtin_bit_cast(u32x2, hi);
      const u32x4 vw = {lo2[0], lo2[1], hi2[0], hi2[1]};
      vf[half][dt] = __builtin_bit_cast(bf16x8, vw);
    }
  }
}

template <int D, int NQT>
__device__ __forceinline__ void pv_mfma(const bf16x8 (&vf)[2][D / 32], const bf16x8 (&pf)[2][NQT],
                                        WaveState<D, NQT>& st) {
#pragma unroll
  for (int half = 0; half < 2; ++half)
#pragma unroll
    for (int dt = 0; dt < D / 32; ++dt)
#pragma unroll
      for (int qt = 0; qt < NQT; ++qt)
        st.o[dt][qt] =
            __builtin_amdgcn_mfma_f32_32x32x16_bf16(vf[half][dt], pf[half][qt], st.o[dt][qt], 0, 0, 0);
}

// Online-softmax update for one quarter: mask, row max, (rare) rescale,
// P = exp2(s * scale_log2 - m_use) packed to bf16 as the B operand of
// O^T += V^T P^T (k-step 2kq + half takes j = 8*half .. 8*half+7).
template <int D, int NQT>
__device__ __forceinline__ void softmax_quarter(f32x16 (&s)[NQT], WaveState<D, NQT>& st,
                                                bool need_mask, int kk0, int Sk, int kpos_base,
                                                int qpos_lane0, bool causal, float scale_log2,
                                                int lane, bf16x8 (&pf)[2][NQT]) {
  const int hh = lane >> 5;
  if (need_mask) {
#pragma unroll
    for (int qt = 0; qt < NQT; ++qt) {
      const int qpos = qpos_lane0 + qt * 32;
#pragma unroll
      for (int j = 0; j < 16; ++j) {
        const int kk = kk0 + 8 * (j >> 2) + 4 * hh + (j & 3);   // key index in the block
        const bool bad = (kk >= Sk) || (causal && kpos_base + kk > qpos);
        if (bad) s[qt][j] = -INFINITY;
      }
    }
  }
  bool grow = false;
#pragma unroll
  for (int qt = 0; qt < NQT; ++qt) {
    float mx = s[qt][0];
#pragma unroll
    for (int j = 1; j < 16; ++j) mx = fmaxf(mx, s[qt][j]);
    mx = pair_max(mx) * scale_log2;     // scale > 0 commutes with max
    st.m_true[qt] = fmaxf(st.m_true[qt], mx);
    grow |= st.m_true[qt] > st.m_use[qt] + kTau;
  }
  if (__builtin_amdgcn_ballot_w64(grow)) {
#pragma unroll
    for (int qt = 0; qt < NQT; ++qt) {
      const float mn = st.m_true[qt];
      const float alpha = (st.m_use[qt] == -INFINITY) ? 0.f : fast_exp2(st.m_use[qt] - mn);
      if (mn != -INFINITY) {
        st.l[qt] *= alpha;
#pragma unroll
        for (int dt = 0; dt < D / 32; ++dt) st.o[dt][qt] *= alpha;
        st.m_use[qt] = mn;
      }
    }
  }
#pragma unroll
  for (int qt = 0; qt < NQT; ++qt) {
    const float mu = (st.m_use[qt] == -INFINITY) ? 0.f : st.m_use[qt];
    float acc = 0.f;
    float p[16];
#pragma unroll
    for (int j = 0; j < 16; ++j) {
      p[j] = fast_exp2(__builtin_fmaf(s[qt][j], scale_log2, -mu));
      acc += p[j];
    }
    st.l[qt] += acc;
#pragma unroll
    for (int half = 0; half < 2; ++half) {
      u32x4 w;
#pragma unroll
      for (int u = 0; u < 4; ++u) w[u] = pack_bf16x2(p[8 * half + 2 * u], p[8 * half + 2 * u + 1]);
      pf[half][qt] = __builtin_bit_cast(bf16x8, w);
    }
  }
}

// Fold one BN-key tile (already in LDS) into the wave's state, 32 keys
// (one quarter) at a time: S = K Q^T on the MFMA, the online-softmax update
// on the VALU, then O^T += V^T P^T.  With two waves per SIMD the matrix
// core of one wave's MFMAs overlaps the other wave's softmax.  (Explicitly
// pipelining quarters inside a wave measured no faster on gfx950.)
template <int D, int BN, int NQT>
__device__ __forceinline__ void fold_tile(const YRB_LDS char* kt_lds, const YRB_LDS char* vt_lds,
                                          const bf16x8 (&qf)[NQT][D / 16],
                                          WaveState<D, NQT>& st, bool need_mask, int k0, int Sk,
                                          int kpos0, int qpos_lane0, bool causal,
                                          float scale_log2, int lane) {
#pragma unroll
  for (int kq = 0; kq < BN / 32; ++kq) {
    bf16x8 kf[D / 16];
    f32x16 s[NQT];
    read_k_quarter<D>(kt_lds, kq, lane, kf);
    qk_mfma<D, NQT>(kf, qf, s);
    bf16x8 pf[2][NQT];
    softmax_quarter<D, NQT>(s, st, need_mask, k0 + 32 * kq, Sk, kpos0 - k0, qpos_lane0, causal,
                            scale_log2, lane, pf);
    bf16x8 vf[2][D / 32];
    read_v_quarter<D>(vt_lds, kq, lane, vf);
    pv_mfma<D, NQT>(vf, pf, st);
  }
}

template <int D, int BN, int NQT, int NW>
__global__ __launch_bounds__(NW * 64, 1) void attn_bf16_kernel(AttnArgs a, int64_t n_qtiles) {
  using T = Tile<D, BN>;
  constexpr int NDS = T::NDS;
  constexpr int NDT = T::NDT;
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
  const int hh = lane >> 5;
  const int l32 = lane & 31;

  // Work item: heaviest query tiles first; heads of one XCD contiguous.
  const int per = (int)(a.B * a.Hq);
  const int rank = (int)blockIdx.x / per;
  const int rem = (int)blockIdx.x - rank * per;
  const int b = rem / (int)a.Hq;
  const int Hq = (int)a.Hq;
  const int hp = rem - b * Hq;
  const int h = (Hq % 8 == 0) ? (hp & 7) * (Hq >> 3) + (hp >> 3) : hp;
  const int qtile = a.causal ? (int)(n_qtiles - 1 - rank) : rank;
  const int hk = h / (Hq / (int)a.Hkv);

  const int q0w = qtile * BM + wave * QW;                // first row of this wave
  const int Sq = (int)a.Sq, Sk = (int)a.Sk;
  const int q_offset = (int)a.q_offset, k_offset = (int)a.k_offset;

  // Q fragments (B operand of S^T = K Q^T): lane holds query row
  // q0w + qt*32 + l32, dims 16ds + 8hh .. +7.  Rotated here if asked.
  bf16x8 qf[NQT][NDS];
  const __bf16* qbase = reinterpret_cast<const __bf16*>(a.q) + b * a.qs[0] + h * a.qs[2];
#pragma unroll
  for (int qt = 0; qt < NQT; ++qt) {
    const int row = min(q0w + qt * 32 + l32, Sq - 1);
    const __bf16* qp = qbase + row * a.qs[1] + 8 * hh;
    u32x4 raw[NDS];
#pragma unroll
    for (int ds = 0; ds < NDS; ++ds) raw[ds] = *reinterpret_cast<const u32x4*>(qp + 16 * ds);
    if (a.cos_sin) {
      const float* cs = a.cos_sin + (int64_t)(q_offset + row) * D;
#pragma unroll
      for (int ds = 0; ds < NDS / 2; ++ds) {
        const int i0 = 16 * ds + 8 * hh;
        const f32x4* t = reinterpret_cast<const f32x4*>(cs + 2 * i0);
        float x[8], z[8], lo[8], hi[8];
        unpack8(raw[ds], x);
        unpack8(raw[ds + NDS / 2], z);
#pragma unroll
        for (int u2 = 0; u2 < 4; ++u2) {
          const f32x4 tt = t[u2];
          lo[2 * u2] = x[2 * u2] * tt[0] - z[2 * u2] * tt[1];
          hi[2 * u2] = x[2 * u2] * tt[1] + z[2 * u2] * tt[0];
          lo[2 * u2 + 1] = x[2 * u2 + 1] * tt[2] - z[2 * u2 + 1] * tt[3];
          hi[2 * u2 + 1] = x[2 * u2 + 1] * tt[3] + z[2 * u2 + 1] * tt[2];
        }
        raw[ds] = pack8(lo);
        raw[ds + NDS / 2] = pack8(hi);
      }
    }
#pragma unroll
    for (int ds = 0; ds < NDS; ++ds) qf[qt][ds] = __builtin_bit_cast(bf16x8, raw[ds]);
  }

  // State.
  WaveState<D, NQT> st;
#pragma unroll
  for (int qt = 0; qt < NQT; ++qt) {
    st.m_use[qt] = -INFINITY;
    st.m_true[qt] = -INFINITY;
    st.l[qt] = 0.f;
#pragma unroll
    for (int dt = 0; dt < NDT; ++dt) st.o[dt][qt] = (f32x16){};
  }
  if (a.load_state) {
#pragma unroll
    for (int qt = 0; qt < NQT; ++qt) {
      const int row = q0w + qt * 32 + l32;
      if (row < Sq) {
        const int64_t ml = ((int64_t)b * Hq + h) * Sq + row;
        const float m0 = a.m[ml];
        st.m_use[qt] = st.m_true[qt] = (m0 == -INFINITY) ? -INFINITY : m0 * kLog2e;
        st.l[qt] = hh == 0 ? a.l[ml] : 0.f;
        const float* op = a.o_acc + (((int64_t)b * Sq + row) * Hq + h) * D;
#pragma unroll
        for (int dt = 0; dt < NDT; ++dt)
#pragma unroll
          for (int q4 = 0; q4 < 4; ++q4) {
            const f32x4 v = *reinterpret_cast<const f32x4*>(op + dt * 32 + 8 * q4 + 4 * hh);
#pragma unroll
            for (int e = 0; e < 4; ++e) st.o[dt][qt][4 * q4 + e] = v[e];
          }
      }
    }
  }

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

  // Epilogue: restore the exact max, then store state and/or output.
#pragma unroll
  for (int qt = 0; qt < NQT; ++qt) {
    float lsum = pair_sum(st.l[qt]);
    const float mt = st.m_true[qt];
    if (mt != -INFINITY && st.m_use[qt] != mt) {
      const float alpha = fast_exp2(st.m_use[qt] - mt);
      lsum *= alpha;
#pragma unroll
      for (int dt = 0; dt < NDT; ++dt) st.o[dt][qt] *= alpha;
      st.m_use[qt] = mt;
    }
    const int row = q0w + qt * 32 + l32;
    if (row >= Sq) continue;
    const int64_t ml = ((int64_t)b * Hq + h) * Sq + row;
    if (a.store_state) {
      if (hh == 0) {
        a.m[ml] = (mt == -INFINITY) ? -INFINITY : mt * kLn2;
        a.l[ml] = lsum;
      }
      float* op = a.o_acc + (((int64_t)b * Sq + row) * Hq + h) * D;
#pragma unroll
      for (int dt = 0; dt < NDT; ++dt)
#pragma unroll
        for (int q4 = 0; q4 < 4; ++q4) {
          const f32x4 v = {st.o[dt][qt][4 * q4], st.o[dt][qt][4 * q4 + 1],
                           st.o[dt][qt][4 * q4 + 2], st.o[dt][qt][4 * q4 + 3]};
          *reinterpret_cast<f32x4*>(op + dt * 32 + 8 * q4 + 4 * hh) = v;
        }
    }
    if (a.finalize) {
      const float inv = lsum > 0.f ? 1.0f / lsum : 0.f;
      __bf16* op = reinterpret_cast<__bf16*>(a.o) + b * a.os[0] + row * a.os[1] + h * a.os[2];
#pragma unroll
      for (int dt = 0; dt < NDT; ++dt)
#pragma unroll
        for (int q4 = 0; q4 < 4; ++q4) {
          const u32x2 w = {pack_bf16x2(st.o[dt][qt][4 * q4] * inv, st.o[dt][qt][4 * q4 + 1] * inv),
                           pack_bf16x2(st.o[dt][qt][4 * q4 + 2] * inv,
                                       st.o[dt][qt][4 * q4 + 3] * inv)};
          *reinterpret_cast<u32x2*>(op + dt * 32 + 8 * q4 + 4 * hh) = w;
        }
      if (a.lse && hh == 0)
        a.lse[ml] = lsum > 0.f ? (mt + __log2f(lsum)) * kLn2 : -INFINITY;
    }
  }
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

hipError_t launch_attention(int dtype, int D, const AttnArgs& a, hipStream_t stream) {
  constexpr int BN = YRB_PREFILL_BN, NQT = YRB_PREFILL_NQT, NW = YRB_PREFILL_NW;
  if (dtype == kBF16) return D == 64 ? launch_bf16<64, BN, NQT, NW>(a, stream)
                                     : launch_bf16<128, BN, NQT, NW>(a, stream);
  return D == 64 ? launch_f32<64>(a, stream) : launch_f32<128>(a, stream);
}

}  // namespace yrb
