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
//    inside the wave, and the wave issues one instruction per four cycles:
//    the schedule is written out, one MFMA per issue step.  The two query
//    tiles run half a step apart (q counts 32-key quarters):
//        H1(q): MFMA  S1(q) = K(q) Q1^T,      O1 += V(q-1)^T P1(q-1)
//               VALU  softmax of S0(q) -> P0(q);  LDS  K(q+1)
//        H2(q): MFMA  S0(q+1) = K(q+1) Q0^T,  O0 += V(q)^T P0(q)
//               VALU  softmax of S1(q) -> P1(q);  LDS  V(q)
//    so the MFMAs of each half step are independent of the VALU work
//    beside them, the scores a softmax reads were finished half a step
//    earlier, and every LDS read lands eight MFMAs before its use.
//  * Scores come out of the MFMA in log2 units and offset by the running
//    max (Q is pre-multiplied by softmax_scale * log2(e), and each S chain
//    starts from minus that max), so the common softmax path is P = exp2(S).
//    When a row max outgrows the lazy-rescale threshold, a rarely taken
//    block at the half-step boundary redoes P against the new max and
//    rescales O, after the last product into O under the old max.
//  * O lives in AGPRs as the accumulator of the PV products, which are
//    issued as inline-asm MFMAs (AGPR C/D, VGPR A/B); VGPRs hold S, P, the
//    fragments and the offsets.  The compiler does not see those MFMAs, so
//    the few places where VALU code touches O or P next to them wait out
//    the MFMA hazards explicitly (xdl_drain, the s_nop after settle).
//  * Key tiles of 64 go global -> LDS with LDS-DMA into four buffers, two
//    tiles ahead, with one workgroup barrier per tile.  Both sit inside a
//    half step: the barrier after its first kArriveStep MFMAs, the tile's
//    DMA instructions one per issue step after it, so the matrix pipe runs
//    through them.  Tiles visible to every row of the workgroup run through
//    the pipeline as they are; the few on the causal diagonal or at the
//    ragged end of the keys run through it too, their scores masked to
//    -inf before the softmax.
//  * Set-up per workgroup: the first two key tiles, the query rows' table
//    rows (by LDS-DMA, coalesced, into buffers still free) and Q go out
//    together, and Q is rotated from the table in fp32.  Work items run
//    heaviest first; given a counter in caller memory, the last part of the
//    grid claims its items from it so that XCDs running at different clocks
//    finish together.
//  * A template flag adds the attention-sink plus sliding-window mask of
//    the 14cs17 notes ("Sliding Window + Attention Sinks") on top of the
//    causal rule: the pipeline walks the sink tiles, then only the tiles
//    some row of the workgroup sees in its window, from a phase shared by
//    neighbouring query tiles; the tiles between are never loaded.
#include "attn_frag.h"
#include "common.h"
#include "kernels.h"

#include <type_traits>

namespace yrb {

namespace {

constexpr int kPPWaves = 4;    // one per SIMD
constexpr int kPPBN = 64;      // keys per tile (two quarters)
constexpr int kPPBufs = 4;     // LDS tile buffers (the tile loop is unrolled by this)
// Issue step of the tile barrier in the arrival half step: the S-chain
// MFMAs of the steps before it need no LDS and run while the waves meet.
constexpr int kArriveStep = 2;

// Work items of the last part of the grid may be claimed at run time.
// Blocks go round robin over the 8 XCDs and each XCD runs its share at its
// own clock, which under load differs from XCD to XCD by a few percent: with
// a fixed item per block the slowest XCD finishes last while the others
// idle.  Given a counter in caller memory, a block from claim_from on takes
// the next ticket instead, so an XCD that runs ahead takes the heavier items
// (they come first).  Without a counter every block takes its own item.
constexpr int kClaimMinBlocks = 16;   // smaller grids take every item statically

// Source of the placeholder DMA when the fast path is off: 16 lane + n KiB
// stays inside it.
__device__ __attribute__((aligned(1024))) unsigned char g_dma_dummy[4096];

// The item of this block: blockIdx.x below claim_from, else claimed from
// the counter `ctr`.  The n = gridDim.x - claim_from claims of a launch take
// n consecutive tickets, and ticket c stands for item claim_from + c mod n:
// n consecutive integers cover every residue once, so every item is taken
// exactly once whatever the counter held.  The block whose ticket completes
// a multiple of n takes that multiple back off the counter, which keeps the
// residues of the tickets still to come and leaves the counter, once the
// launch's claims are made, at its starting value mod n: a counter that
// starts at zero ends at zero.
__device__ __forceinline__ int claim_item(int claim_from, unsigned* ctr, YRB_LDS int* cell) {
  if ((int)blockIdx.x < claim_from) return (int)blockIdx.x;
  if (threadIdx.x == 0) {
    const unsigned n = gridDim.x - (unsigned)claim_from;
    const unsigned c = __hip_atomic_fetch_add(ctr, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    const unsigned r = c % n;
    if (r == n - 1) __hip_atomic_fetch_sub(ctr, c + 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    *cell = claim_from + (int)r;
  }
  __syncthreads();
  return __builtin_amdgcn_readfirstlane(*cell);
}

// S^T of 32 keys against one 32-row query tile, accumulated onto `init`.
template <int D>
__device__ __forceinline__ f32x16 qk_tile(const bf16x8 (&kf)[D / 16], const bf16x8 (&q)[D / 16],
                                          const f32x16& init) {
  f32x16 s = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf[0], q[0], init, 0, 0, 0);
#pragma unroll
  for (int ds = 1; ds < D / 16; ++ds) s = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf[ds], q[ds], s, 0, 0, 0);
  return s;
}

// IEEE maximum (v_maximum3_f32 on gfx950: no input canonicalisation).
__device__ __forceinline__ float vmax(float a, float b) { return __builtin_elementwise_maximum(a, b); }
__device__ __forceinline__ float pair_vmax(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return vmax(__uint_as_float(r[0]), __uint_as_float(r[1]));
}

__device__ __forceinline__ f32x16 splat16(float v) {
  f32x16 r;
#pragma unroll
  for (int j = 0; j < 16; ++j) r[j] = v;
  return r;
}

// Offsets of the two query tiles: each S chain starts from negb = -base,
// base being the max the exponentials use (0 while a row has none).
struct Offsets {
  f32x16 negb[2];
  float base[2];
  float mu_tau[2];     // m_use + threshold
  float l_prev[2];     // row sum before the current quarter
  float thr[2];        // sum test: a quarter's P sum above this may hold a P above 2^threshold
};

// The sum test: with a reference in use, any P above 2^threshold makes the
// lane's quarter sum exceed 2^threshold; without one, any visible key does.
__device__ __forceinline__ float sum_threshold(float m_use) { return m_use == -INFINITY ? 0.f : exp2f(kTau); }

template <int D>
__device__ __forceinline__ void offsets_from(const WaveState<D, 2>& st, Offsets& of) {
#pragma unroll
  for (int t = 0; t < 2; ++t) {
    const float mu = st.m_use[t];
    of.base[t] = mu == -INFINITY ? 0.f : mu;
    of.mu_tau[t] = mu + kTau;
    of.negb[t] = splat16(-of.base[t]);
    of.l_prev[t] = st.l[t];
    of.thr[t] = sum_threshold(mu);
  }
}

// Per lane, for masking, all less 4(lane/32), the lane's row offset inside
// a quarter: the last key index inside the keys; for each query tile, the
// last key index visible to the lane's query row under the causal mask; the
// end of the sink keys and the window length (both unused without a
// window).  Wave-uniform, in key indices: the end of the sinks and the last
// key some row of the wave has outside its window (-1 if none).
struct MaskInfo {
  int key_last;
  int q_last[2];
  int sink_end;
  int window;
  bool causal;
  int sink_end_u;
  int w_lo_u;
};

// Mask of the quarter whose first key index is kbase, for query tile X:
// lane element j holds key row 8(j/4) + (j%4) of the quarter past
// 4(lane/32).  A key stays if it is inside the keys, not after the row
// (causal), and either a sink or inside the row's window; the others get
// -inf, so P = 0.
//
// With a window, whether some row's window starts past the quarter's first
// key and whether the quarter holds a sink key are wave-uniform, and each
// case takes its cheapest exact form: with no window start inside, every key
// is inside every row's window and the causal test alone decides (the
// diagonal, the ragged end, and sinks alike); a window start inside and no
// sink, one unsigned range test (e in (lo, hi]); both, the full test.
template <bool WIN>
__device__ __forceinline__ void mask_scores(f32x16& s, const MaskInfo& mi, int X, int kbase) {
  const int hi = (mi.causal ? min(mi.key_last, mi.q_last[X]) : mi.key_last) - kbase;
  const bool edge = WIN && kbase <= mi.w_lo_u;       // some row's window starts inside
  if (!edge) {
#pragma unroll
    for (int j = 0; j < 16; ++j) {
      const int e = 8 * (j >> 2) + (j & 3);
      s[j] = e <= hi ? s[j] : -INFINITY;
    }
    return;
  }
  const int lo = mi.q_last[X] - mi.window - kbase;   // window: keys after it
  const int se = mi.sink_end - kbase;                 // sinks: keys before it
  if (kbase >= mi.sink_end_u) {                      // no sink key
    const int lo1 = lo + 1;
    const unsigned width = (unsigned)max(hi - lo, 0);
#pragma unroll
    for (int j = 0; j < 16; ++j) {
      const int e = 8 * (j >> 2) + (j & 3);
      s[j] = (unsigned)(e - lo1) < width ? s[j] : -INFINITY;
    }
    return;
  }
#pragma unroll
  for (int j = 0; j < 16; ++j) {
    const int e = 8 * (j >> 2) + (j & 3);
    const bool keep = e <= hi && (e < se || e > lo);
    s[j] = keep ? s[j] : -INFINITY;
  }
}

// Rare case, at the boundary after the last product into O of tile QT under
// the old max: rows that grew take their exact max as the new base, P and
// the row sum are redone against it, O is rescaled, and the S chains of the
// following quarters start from the new base.
template <int D, int QT>
__device__ __forceinline__ void settle_rows(const f32x16& s, WaveState<D, 2>& st, Offsets& of, bool grow,
                                            bf16x8 (&pf)[2], float t_max) {
  const float mu_old = st.m_use[QT];
  const float mu_new = grow ? t_max : mu_old;
  // 0 where kept; 0 too for a row still empty (every score so far -inf),
  // whose P must come out 0, not exp2(-inf + inf)
  const float shift = mu_new == -INFINITY ? 0.f : mu_new - of.base[QT];
  const float alpha = grow ? fast_exp2(mu_old - mu_new) : 1.0f;      // 0 from an empty row
  float acc = of.l_prev[QT] * alpha;
#pragma unroll
  for (int half = 0; half < 2; ++half) {
    u32x4 w;
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int j = 8 * half + 2 * u;
      const float p0 = fast_exp2(s[j] - shift), p1 = fast_exp2(s[j + 1] - shift);
      acc += p0 + p1;
      const bf16x2 pp = {(__bf16)p0, (__bf16)p1};
      w[u] = __builtin_bit_cast(unsigned, pp);
    }
    pf[half] = __builtin_bit_cast(bf16x8, w);
  }
  st.l[QT] = acc;
#pragma unroll
  for (int dt = 0; dt < D / 32; ++dt) scale_o_agpr(st.o[dt][QT], alpha);
  st.m_use[QT] = mu_new;
  of.base[QT] = mu_new == -INFINITY ? 0.f : mu_new;
  of.mu_tau[QT] = mu_new + kTau;
  of.thr[QT] = sum_threshold(mu_new);
  of.negb[QT] = splat16(-of.base[QT]);
  // The next inline-asm MFMA may read this P at once.
  asm volatile("s_nop 4" ::: "memory");
}

// The boundary after a half step, one rarely taken branch for both rare
// cases: settle_rows when a row of tile QT grew, and the mask of the scores
// the next half step's softmax reads (s_next, query tile X_next, first key
// index kbase) when they come from a masked tile.  With EXACT the half step
// tracked the exact row max and `grow` is final; without, `grow` is the sum
// test's candidate and the exact max of the quarter is taken here.
template <int D, int QT, bool EXACT, bool WIN>
__device__ __forceinline__ void settle(const f32x16& s, WaveState<D, 2>& st, Offsets& of, bool grow, bool need,
                                       bf16x8 (&pf)[2], bool mask_next, f32x16& s_next, const MaskInfo& mi,
                                       int X_next, int kbase) {
  if (__builtin_expect(!need, 1)) return;
  const uint64_t grown = __builtin_amdgcn_ballot_w64(grow);
  if (grown != 0) {
    if constexpr (EXACT) {
      settle_rows<D, QT>(s, st, of, grow, pf, st.m_true[QT]);
    } else {
      float mx = s[0];
#pragma unroll
      for (int j = 1; j < 16; ++j) mx = vmax(mx, s[j]);
      const float t_max = of.base[QT] + pair_vmax(mx);   // this quarter's exact row max
      const bool g = t_max > of.mu_tau[QT];
      if (__builtin_amdgcn_ballot_w64(g) != 0) settle_rows<D, QT>(s, st, of, g, pf, t_max);
    }
  }
  if (mask_next) mask_scores<WIN>(s_next, mi, X_next, kbase);
}

// Pin a value to the current issue step: an empty volatile asm that reads
// and writes it, ordered with the step fences, so the value is computed
// within the step rather than wherever the instruction selector put it.
__device__ __forceinline__ void pin(float& x) { asm volatile("" : "+v"(x)); }
__device__ __forceinline__ void pin(unsigned& x) { asm volatile("" : "+v"(x)); }

__device__ __forceinline__ void pack_pair(const float (&p)[16], int u, unsigned (&w)[8]) {
  const bf16x2 pp = {(__bf16)p[2 * u], (__bf16)p[2 * u + 1]};
  w[u] = __builtin_bit_cast(unsigned, pp);
  pin(w[u]);
}
// Row sum of a pair, in fp32 adds: the bf16 dot instructions run on the
// matrix pipe on gfx950 and stall the MFMAs they sit between.
__device__ __forceinline__ void add_pair(const float (&p)[16], int u, float& acc) {
  acc += p[2 * u] + p[2 * u + 1];
  pin(acc);
}

// LDS layout of the pipeline: the kPPBufs K tiles, then the kPPBufs V tiles.
// Every fragment read is a per-lane base register (fixed for the launch)
// plus an immediate for buffer, quarter and k-step, so the reads need no
// address arithmetic.  The swizzles repeat every 16 rows, which keeps each
// lane's swizzle the same for every quarter and k-step.
template <int D>
struct LdsMap {
  static constexpr int TILEB = Tile<D, kPPBN>::TILEB;
  static constexpr int ROWB = Tile<D, kPPBN>::ROWB;
  static constexpr int VBASE = kPPBufs * TILEB;
  unsigned k[D / 16];   // K fragment ds: quarter 0 of buffer 0
  unsigned v[D / 32];   // V fragment dt: first transposed read, k-step 0 of buffer 0
};

template <int D>
__device__ __forceinline__ LdsMap<D> lds_map(int lane) {
  using M = LdsMap<D>;
  LdsMap<D> m;
  const int r = lane & 31, hh = lane >> 5;
#pragma unroll
  for (int ds = 0; ds < D / 16; ++ds) m.k[ds] = r * M::ROWB + (((2 * ds + hh) ^ ksw<D>(r)) << 4);
  const int g = lane >> 4, t4 = (lane & 15) >> 2, s4 = lane & 3;
  const int row = 4 * (g >> 1) + t4;
#pragma unroll
  for (int dt = 0; dt < D / 32; ++dt) {
    const int c = dt * 4 + 2 * (g & 1) + (s4 >> 1);
    m.v[dt] = M::VBASE + row * M::ROWB + ((c ^ vsw<D>(row)) << 4) + 8 * (s4 & 1);
  }
  return m;
}

template <int D, int B, int KQ>
__device__ __forceinline__ bf16x8 read_k_at(const YRB_LDS char* lds, const LdsMap<D>& m, int ds) {
  using M = LdsMap<D>;
  return *reinterpret_cast<const YRB_LDS bf16x8*>(lds + m.k[ds] + (B * M::TILEB + KQ * 32 * M::ROWB));
}

template <int D, int B, int KQ>
__device__ __forceinline__ bf16x8 read_v_at(const YRB_LDS char* lds, const LdsMap<D>& m, int half, int dt) {
  using M = LdsMap<D>;
  const YRB_LDS char* a1 = lds + m.v[dt] + (B * M::TILEB + (2 * KQ + half) * 16 * M::ROWB);
  const i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((YRB_LDS i16x4*)a1);
  const i16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((YRB_LDS i16x4*)(a1 + 8 * M::ROWB));
  const u32x2 lo2 = __builtin_bit_cast(u32x2, lo);
  const u32x2 hi2 = __builtin_bit_cast(u32x2, hi);
  const u32x4 vw = {lo2[0], lo2[1], hi2[0], hi2[1]};
  return __builtin_bit_cast(bf16x8, vw);
}

// One of the two transposed 64-bit reads of a V fragment (second: the
// k-step's keys 8..15).
template <int D, int B, int KQ>
__device__ __forceinline__ u32x2 read_v_part(const YRB_LDS char* lds, const LdsMap<D>& m, int half, int dt,
                                             int second) {
  using M = LdsMap<D>;
  const YRB_LDS char* a = lds + m.v[dt] + (B * M::TILEB + (2 * KQ + half) * 16 * M::ROWB + second * 8 * M::ROWB);
  return __builtin_bit_cast(u32x2, __builtin_amdgcn_ds_read_tr16_b64_v4i16((YRB_LDS i16x4*)a));
}

// The DMA of one tile, spread over the issue steps of a half step: source
// rows (SGPRs) and destination LDS addresses of K and V.  A tile that the
// fast path cannot load (past the keys the workgroup needs, ragged, or
// strides outside the fast path's range) still issues the same number of
// instructions, placeholders into a spare LDS region, so the vmcnt count
// per tile stays fixed; `slow` then asks for the clamped load of a ragged
// tile after the half step.
struct DmaPlan {
  const __bf16* k;
  const __bf16* v;
  unsigned k_m0, v_m0;
  bool slow;
};

// Plan of tile u, whose buffer is UB = u % kPPBufs (every argument
// wave-uniform): tiles below n_fast come from k_rows/v_rows (that tile's
// first key row) into buffer UB (k_m0/v_m0: buffer 0 plus this wave's
// LO KiB), the others are placeholders from kb/vb (the first key tile, or
// the dummy buffer when the fast path is off) into the spare region.
template <int D, int UB>
__device__ __forceinline__ DmaPlan dma_plan(int u, int n_fast, int n_tiles, const __bf16* k_rows,
                                            const __bf16* v_rows, const __bf16* kb, const __bf16* vb,
                                            unsigned k_m0, unsigned v_m0, unsigned spare_m0) {
  constexpr unsigned BOFF = UB * Tile<D, kPPBN>::TILEB;
  const bool real = u < n_fast;
  DmaPlan p;
  p.k = real ? k_rows : kb;
  p.v = real ? v_rows : vb;
  p.k_m0 = real ? k_m0 + BOFF : spare_m0;
  p.v_m0 = real ? v_m0 + BOFF : spare_m0;
  p.slow = !real && u < n_tiles;
  return p;
}

// Issue steps of a half step (NS = 2 * D/16), as compile-time functions.
// The scores the softmax reads come from the S chain in the first half of
// the previous half step, long finished, so the softmax starts at step 0.
// It ends three steps early: the row-max tail, then (step NS-2) the grow
// test and the boundary's branch condition run beside the last MFMAs, and
// the last step holds its MFMA alone.
template <int D>
struct Steps {
  static constexpr int NS = D / 8;
  static constexpr int SPAN = NS - 3;
  static constexpr int exp_at(int j) { return (j * SPAN) / 16; }
  static constexpr int max_at(int k) { return (k * SPAN) / 8; }
  static constexpr int pack_at(int u) { return exp_at(2 * u + 1) + 1; }
  static constexpr int dot_at(int u) { return pack_at(u); }
  static constexpr int final_at() { return NS - 3; }
  static constexpr int need_at() { return NS - 2; }
};

// One half step, kept in order by sched_barrier(0) between issue steps.
// Step i issues one MFMA (tile Y: the S chain on kf in steps 0 .. NDS-1,
// then the PV products on vf), LDS fragment reads (in H1 the next quarter's
// K, each fragment right after the S step that used the old one; in H2 the
// current quarter's V, a fragment per step in the first half, eight steps
// ahead of its PV product), and its share of tile X's softmax: exps, the
// max chain, packs of finished pairs and the row sum.  In the common case
// (no row max outgrew the threshold) tile X's softmax is then complete.
// Returns whether any row grew, for settle().
template <int D, int Y, int BV, int KQV, int BK, int KQK, bool READ_V, bool READ_K, bool EXACT, bool ARRIVE = false>
__device__ __forceinline__ bool half_step(WaveState<D, 2>& st, Offsets& of, const YRB_LDS char* lds,
                                          const LdsMap<D>& m, bf16x8 (&vf)[2][D / 32],
                                          const bf16x8 (&p_pv)[2], bf16x8 (&kf)[D / 16],
                                          const bf16x8 (&q_s)[D / 16], f32x16& s_y, const f32x16& s_x,
                                          bf16x8 (&p_x)[2], bool mask_next, bool& need,
                                          const DmaPlan* dp = nullptr,
                                          const unsigned* koff = nullptr, const unsigned* voff = nullptr,
                                          int wave = 0) {
  constexpr int X = 1 - Y;
  constexpr int NL = TileLoads<D, kPPBN, kPPWaves>::LO;   // DMA instructions per tile per wave, K or V
  constexpr int BS = ARRIVE ? kArriveStep : 0;              // barrier step; K reads and DMA follow it
  static_assert(!ARRIVE || BS + 2 * NL < D / 8, "the DMA pieces must fit the half step");
  static_assert(BS + D / 16 <= D / 8 - 2, "K reads end two steps before the next half step");
  auto dma_at = [&](auto i_tag) YRB_INLINE {   // DMA instruction of step i (1 .. 2 NL)
    constexpr int n = decltype(i_tag)::value - 1;
    if constexpr (n >= 0 && n < NL) dma_lds_m0<n * 1024, n == 0>(dp->k_m0, dp->k, koff[n]);
    else if constexpr (n >= NL && n < 2 * NL) dma_lds_m0<(n - NL) * 1024, n == NL>(dp->v_m0, dp->v, voff[n - NL]);
  };
  constexpr int NDS = D / 16, NDT = D / 32;
  using S = Steps<D>;
  constexpr int NS = S::NS;
  const float base_x = of.base[X];
  float acc = st.l[X];
  of.l_prev[X] = acc;
  float qs = 0.f;   // without EXACT: this quarter's P sum (set at its first pair)
  float p[16];
  unsigned w[8];
  float mx = 0.f;
  bool grow = false;
  // O stays in AGPRs (a no-op when the register allocator already has it there)
#pragma unroll
  for (int t = 0; t < 2; ++t)
#pragma unroll
    for (int dt = 0; dt < NDT; ++dt) asm volatile("" : "+a"(st.o[dt][t]));
  auto finish_max = [&]() YRB_INLINE {
    const float t1 = base_x + pair_vmax(mx);   // this quarter's row max
    st.m_true[X] = vmax(st.m_true[X], t1);
    grow = t1 > of.mu_tau[X];
    pin(st.m_true[X]);
  };
#pragma unroll
  for (int i = 0; i < NS; ++i) {
    // LDS waits of H2, three instead of one per MFMA: the K fragments (read
    // in H1) before the first S step, then the V fragments of this half
    // step in two halves, each half four or more steps after its reads.
    if (READ_V) {
      if (i == 0) wait_lgkmcnt<0>();
      if (i == NDS) wait_lgkmcnt<NDS>();
      if (i == NDS + NDS / 2) wait_lgkmcnt<0>();
    }
    // MFMA
    if (i < NDS) {
      s_y = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf[i], q_s[i], i == 0 ? of.negb[Y] : s_y, 0, 0, 0);
    } else {
      const int f = i - NDS;
      mfma_o(st.o[f % NDT][Y], vf[f / NDT][f % NDT], p_pv[f / NDT]);
    }
    // A PV MFMA issues first in its step: left free, the scheduler puts the
    // step's DMA and LDS reads ahead of it, and the MFMA pipe waits.
    if (i >= NDS) __builtin_amdgcn_sched_barrier(0);
    // Tile arrival (the MFMAs of the steps before run meanwhile): this
    // wave's DMA of the next tile is done, the barrier extends that to every
    // wave; then the DMA of the tile two ahead, one instruction per step.
    if (ARRIVE) {
      if (i == BS) {
        wait_vmcnt<2 * NL>();
        tile_barrier();
      } else if (i > BS) {
        static_for<2 * NL + 1>([&](auto j_tag) YRB_INLINE {
          if (decltype(j_tag)::value + BS == i) dma_at(j_tag);
        });
      }
    }
    // LDS fragment reads (K fragment j after the MFMA of step j that used it)
    if (READ_K && i >= 1 + BS && i <= NDS + BS) kf[i - 1 - BS] = read_k_at<D, BK, KQK>(lds, m, i - 1 - BS);
    if (READ_V && i < NDS) vf[i / NDT][i % NDT] = read_v_at<D, BV, KQV>(lds, m, i / NDT, i % NDT);
    // softmax of tile X
#pragma unroll
    for (int j = 0; j < 16; ++j)
      if (S::exp_at(j) == i) {
        p[j] = fast_exp2(s_x[j]);
        pin(p[j]);
      }
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      if (S::pack_at(u) == i) pack_pair(p, u, w);
      if (S::dot_at(u) == i) {
        if (!EXACT && u == 0) {   // the quarter sum starts at its first pair
          qs = p[0] + p[1];
          pin(qs);
        } else {
          add_pair(p, u, EXACT ? acc : qs);
        }
      }
    }
    if constexpr (EXACT) {
#pragma unroll
      for (int k = 0; k < 8; ++k) {
        if (S::max_at(k) != i) continue;
        if (k == 0) mx = vmax(vmax(s_x[0], s_x[1]), s_x[2]);
        else if (k < 7) mx = vmax(vmax(mx, s_x[2 * k + 1]), s_x[2 * k + 2]);
        else mx = vmax(mx, s_x[15]);
        pin(mx);
      }
      if (S::final_at() == i) finish_max();
    }
    // the boundary's branch condition, beside the last MFMA rather than
    // after it: any row may have grown, or the next scores need a mask
    if (i == S::need_at()) {
      if constexpr (!EXACT) {
        acc += qs;
        grow = qs > of.thr[X];
      }
      need = __builtin_amdgcn_ballot_w64(grow) != 0 || mask_next;
    }
    __builtin_amdgcn_sched_barrier(0);
  }
  // work that falls past the last step
  if (EXACT && S::final_at() >= NS) finish_max();
#pragma unroll
  for (int u = 0; u < 8; ++u) {
    if (S::pack_at(u) >= NS) pack_pair(p, u, w);
    if (S::dot_at(u) >= NS) add_pair(p, u, EXACT ? acc : qs);
  }
  st.l[X] = acc;
#pragma unroll
  for (int half = 0; half < 2; ++half) {
    const u32x4 v4 = {w[4 * half], w[4 * half + 1], w[4 * half + 2], w[4 * half + 3]};
    p_x[half] = __builtin_bit_cast(bf16x8, v4);
  }
  // keep P and the row sum in this block (nothing sinks them to the next)
  asm volatile("" ::"v"(p_x[0]), "v"(p_x[1]), "v"(acc));
  return grow;
}

// Final output of a prefill call (no state stored) through LDS: the wave's
// normalised 64 x D bf16 rows go into its own LDS region, 16-byte chunks
// XOR-swizzled by row so that the writes from the Oᵀ accumulator layout
// (a lane per row) spread over all banks, and come back a row per 16 (D=128)
// lanes, so each store writes whole rows.  Log-sum-exp as in finish_rows.
template <int D>
__device__ __forceinline__ void finish_rows_lds(const AttnArgs& a, int b, int h, int q0w, int lane,
                                                WaveState<D, 2>& st, YRB_LDS char* region) {
  constexpr int NDT = D / 32, CH = D / 8;   // 16-byte chunks per row
  const int hh = lane >> 5, l32 = lane & 31;
  const int Sq = (int)a.Sq, Hq = (int)a.Hq;
  auto swz = [](int r) YRB_INLINE { return r & (CH - 1); };
#pragma unroll
  for (int qt = 0; qt < 2; ++qt) {
    const float lsum = pair_sum(st.l[qt]);
    const float inv = lsum > 0.f ? 1.0f / lsum : 0.f;
    const int r = qt * 32 + l32;
#pragma unroll
    for (int dt = 0; dt < NDT; ++dt)
#pragma unroll
      for (int q4 = 0; q4 < 4; ++q4) {
        const int c = dt * 4 + q4;   // dims 8c .. 8c+7; this lane holds 8c + 4hh .. +3
        const u32x2 w = {pack_bf16x2(st.o[dt][qt][4 * q4] * inv, st.o[dt][qt][4 * q4 + 1] * inv),
                         pack_bf16x2(st.o[dt][qt][4 * q4 + 2] * inv, st.o[dt][qt][4 * q4 + 3] * inv)};
        *reinterpret_cast<YRB_LDS u32x2*>(region + r * (2 * D) + ((c ^ swz(r)) << 4) + 8 * hh) = w;
      }
    const int row = q0w + r;
    if (a.lse && hh == 0 && row < Sq)
      a.lse[((int64_t)b * Hq + h) * Sq + row] = lsum > 0.f ? (st.m_true[qt] + __log2f(lsum)) * kLn2 : -INFINITY;
  }
  // The region is this wave's alone: no barrier, only the wave's own writes.
  __builtin_amdgcn_s_waitcnt(15 | (3 << 14) | (7 << 4) | (0 << 8));   // lgkmcnt(0)
  constexpr int RPI = 64 / CH;   // rows per read instruction
#pragma unroll
  for (int i = 0; i < 64 / RPI; ++i) {
    const int r = i * RPI + lane / CH, c = lane % CH;
    const u32x4 v = *reinterpret_cast<const YRB_LDS u32x4*>(region + r * (2 * D) + ((c ^ swz(r)) << 4));
    const int row = q0w + r;
    if (row < Sq) {
      __bf16* op = reinterpret_cast<__bf16*>(a.o) + b * a.os[0] + row * a.os[1] + h * a.os[2];
      *reinterpret_cast<u32x4*>(op + 8 * c) = v;
    }
  }
}

// The table rows of one 32-row query tile (positions q_offset + row, rows
// clamped to the last query row) global -> LDS by DMA into the wave's
// region: 4D bytes a row, 1 KiB (256/D rows) per instruction, 16-byte chunk
// c of row r stored at position c ^ (r mod D/4) so that the lane reads below
// spread over the banks.
template <int D>
__device__ __forceinline__ void table_rows_to_lds(const AttnArgs& a, int row0, int lane, YRB_LDS char* region) {
  constexpr int CHT = D / 4;           // 16-byte chunks a table row
  constexpr int RPI = 64 / CHT;        // rows per DMA instruction
  const int Sq = (int)a.Sq;
  const unsigned m0 = __builtin_amdgcn_readfirstlane((unsigned)(uintptr_t)region);
  static_for<32 / RPI>([&](auto n_tag) YRB_INLINE {
    constexpr int n = decltype(n_tag)::value;
    const int r = n * RPI + lane / CHT;            // row inside the tile
    const int c = (lane % CHT) ^ (r & (CHT - 1));  // chunk this lane fetches
    const int row = min(row0 + r, Sq - 1);
    dma_lds_vaddr<n * 1024>(m0, a.cos_sin + (int64_t)((int)a.q_offset + row) * D + 4 * c);
  });
}

// The cos/sin a lane needs for query tile rows (row l32; chunks 8ds + 4hh + u2)
// from the wave's LDS region.
template <int D>
__device__ __forceinline__ void table_from_lds(const YRB_LDS char* region, int lane, f32x4 (&tab)[D / 32][4]) {
  constexpr int CHT = D / 4;
  const int r = lane & 31, hh = lane >> 5;
#pragma unroll
  for (int ds = 0; ds < D / 32; ++ds)
#pragma unroll
    for (int u2 = 0; u2 < 4; ++u2) {
      const int c = 8 * ds + 4 * hh + u2;
      tab[ds][u2] = *reinterpret_cast<const YRB_LDS f32x4*>(region + r * (4 * D) + ((c ^ (r & (CHT - 1))) << 4));
    }
}

// EXACT: track the exact running max (calls that store the state, whose m
// is that max); without it the grow test is the sum test and the output and
// log-sum-exp use the reference in use, which gives the same values.
template <int D, bool EXACT, bool WIN>
__global__ __launch_bounds__(kPPWaves * 64, 1) void attn_bf16_pp_kernel(AttnArgs a, int64_t n_qtiles,
                                                                         int claim_from) {
  constexpr int NW = kPPWaves, BN = kPPBN, QW = 64, BM = NW * QW;
  constexpr int NDS = D / 16, NDT = D / 32;
  using T = Tile<D, BN>;
  using TL = TileLoads<D, BN, NW>;
  static_assert(TL::EXTRA == 0, "tile DMA must split evenly over the waves");
  constexpr int DMA = 2 * TL::LO;   // LDS-DMA instructions per wave per tile (K and V)

  // kPPBufs K tiles, then kPPBufs V tiles (dynamic LDS).
  extern __shared__ __attribute__((aligned(1024))) char lds_raw[];
  YRB_LDS char* const lds = (YRB_LDS char*)lds_raw;
  auto kbuf = [&](int t) YRB_INLINE -> YRB_LDS char* { return lds + (t & (kPPBufs - 1)) * T::TILEB; };
  auto vbuf = [&](int t) YRB_INLINE -> YRB_LDS char* {
    return lds + LdsMap<D>::VBASE + (t & (kPPBufs - 1)) * T::TILEB;
  };

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int l32 = lane & 31;
  // The arguments the item's set-up reads go into SGPRs first, so their
  // loads go out together with the claim's rather than after it.
  asm volatile("" ::"s"(a.q), "s"(a.k), "s"(a.v), "s"(a.cos_sin), "s"(a.B), "s"(a.Sq), "s"(a.Sk), "s"(a.Hq),
               "s"(a.Hkv), "s"(a.qs[0]), "s"(a.ks[0]), "s"(a.vs[0]));
  // (The claim's LDS cell is in the spare region, which no DMA reaches
  // before the first tile's barrier.)
  const int item = claim_item(claim_from, a.claims, (YRB_LDS int*)(lds + 2 * kPPBufs * T::TILEB));
  const WorkItem wi = work_item_at(a, n_qtiles, item);
  const int b = wi.b, h = wi.h, hk = wi.hk, qtile = wi.qtile;
  const int q0w = qtile * BM + wave * QW;
  const int Sq = (int)a.Sq, Sk = (int)a.Sk;
  const int q_offset = (int)a.q_offset, k_offset = (int)a.k_offset;

  // Key tiles: n_tiles reach the workgroup's last visible key; the first
  // n_full are visible to every row of the workgroup and hold no key past Sk.
  const int q_first_wg = q_offset + qtile * BM;
  const int q_last_wg = q_offset + min(Sq, (qtile + 1) * BM) - 1;
  int n_keys = Sk;
  if (a.causal) n_keys = max(0, min(Sk, q_last_wg - k_offset + 1));
  const int n_key_tiles = (n_keys + BN - 1) / BN;
  int n_full = min(n_key_tiles, Sk / BN);
  if (a.causal) n_full = min(n_full, max(0, q_first_wg - k_offset + 1) / BN);
  // With a window the workgroup needs the sink tiles [0, n_sink_t) and the
  // window tiles [tw0, n_key_tiles): the pipeline walks the sink tiles
  // first (its tile t is key tile t below n_sink_t), then the window tiles
  // past them, skipping the gap between.
  // A key tile needs the mask unless it is below n_full and wholly among
  // the sinks (its last key before sink_end) or wholly inside the window of
  // the workgroup's last row (its first key after w_lo).  Without a window
  // sink_end = 0 and w_lo = -1, so only n_full decides.
  int n_sink_t = 0, gap = 0, sink_end = 0, w_lo = -1, n_win = 0, rot = 0;
  if constexpr (WIN) {
    sink_end = (int)max((int64_t)0, min((int64_t)a.n_sink - k_offset, (int64_t)n_key_tiles * BN));
    n_sink_t = (sink_end + BN - 1) / BN;
    const int tw0 = min(n_key_tiles, max(0, q_first_wg - k_offset - a.window + 1) / BN);
    gap = max(0, tw0 - n_sink_t);
    w_lo = max(-1, q_last_wg - k_offset - a.window);
    n_sink_t = __builtin_amdgcn_readfirstlane(n_sink_t);
    gap = __builtin_amdgcn_readfirstlane(gap);
    sink_end = __builtin_amdgcn_readfirstlane(sink_end);
    w_lo = __builtin_amdgcn_readfirstlane(w_lo);
    // The window tiles [wstart, n_key_tiles) start at a phase shared by the
    // 8 query tiles of an aligned group (the first window tile of the
    // group's last query tile) and wrap round to wstart: query tiles that
    // run side by side then read the same key tiles at about the same time.
    const int wstart = n_sink_t + gap;
    n_win = n_key_tiles - wstart;
    const int q_grp = q_offset + min((qtile | 7) * BM, (Sq - 1) / BM * BM);
    const int phase = max(0, q_grp - k_offset - a.window + 1) / BN;
    rot = max(0, min(phase - wstart, n_win - 1));
    n_win = __builtin_amdgcn_readfirstlane(n_win);
    rot = __builtin_amdgcn_readfirstlane(rot);
  }
  const int n_tiles = n_key_tiles - gap;   // pipeline tiles
  auto key_tile = [&](int t) YRB_INLINE {
    if constexpr (!WIN) return t;
    if (t < n_sink_t) return t;
    const int u = t - n_sink_t + rot;
    return n_sink_t + gap + (u >= n_win ? u - n_win : u);
  };
  const bool wave_live = q0w < Sq;

  const __bf16* kbase = reinterpret_cast<const __bf16*>(a.k) + b * a.ks[0] + hk * a.ks[2];
  const __bf16* vbase = reinterpret_cast<const __bf16*>(a.v) + b * a.vs[0] + hk * a.vs[2];
  const int kstride = (int)a.ks[1], vstride = (int)a.vs[1];
  const __bf16* const kbase_s = wave_uniform(kbase);
  const __bf16* const vbase_s = wave_uniform(vbase);

  // The fast DMA needs a whole first tile (its placeholders read it), and
  // token strides of at least a row whose BN rows fit the 32-bit lane
  // offsets.  Without it every tile takes the clamped load and the
  // placeholders read a dummy buffer.
  const bool fast_dma = Sk >= BN && min(kstride, vstride) >= D &&
                        (int64_t)max(kstride, vstride) * BN * 2 < ((int64_t)1 << 31);
  unsigned koff[TL::LO], voff[TL::LO];
  tile_offsets<D, BN, NW, false>(kstride, wave, lane, !fast_dma, koff);
  tile_offsets<D, BN, NW, true>(vstride, wave, lane, !fast_dma, voff);
  const __bf16* const ph_k = fast_dma ? kbase_s : reinterpret_cast<const __bf16*>(g_dma_dummy);
  const __bf16* const ph_v = fast_dma ? vbase_s : reinterpret_cast<const __bf16*>(g_dma_dummy);
  auto issue = [&](int t) YRB_INLINE {   // pipeline tile t into buffer t % kPPBufs
    const int kt = key_tile(t);
    if (fast_dma && (kt + 1) * BN <= Sk) {
      load_tile_rows<D, BN, NW>(kbuf(t), kbase_s + (int64_t)kt * BN * kstride, koff, wave);
      load_tile_rows<D, BN, NW>(vbuf(t), vbase_s + (int64_t)kt * BN * vstride, voff, wave);
    } else {   // the ragged last tile: rows past the end read the last row
      load_tile<D, BN, NW, false>(kbuf(t), kbase, kstride, kt * BN, Sk, wave, lane);
      load_tile<D, BN, NW, true>(vbuf(t), vbase, vstride, kt * BN, Sk, wave, lane);
    }
  };
  // Q rotated and pre-multiplied by softmax_scale * log2(e): scores come out
  // of the MFMA in log2 units.  Q and O stay in AGPRs for the whole launch.
  // Loads: the first two key tiles, the first query tile's table rows by
  // DMA into the wave's region of buffers 2/3 (free until the first tile
  // arrives), then Q; the second query tile's table rows follow through the
  // same region while the first query tile is rotated.
  bf16x8 qf[2][NDS];
  {
    YRB_LDS char* const region = lds + (wave < 2 ? 0 : LdsMap<D>::VBASE) + (2 + (wave & 1)) * T::TILEB;
    static_assert(32 * 4 * D <= T::TILEB, "a query tile's table rows fit one tile buffer");
    const float qscale = a.softmax_scale * kLog2e;
    QRaw<D, 2> qr;
    if (n_tiles > 0) issue(0);
    if (n_tiles > 1) issue(1);
    if (a.cos_sin) table_rows_to_lds<D>(a, q0w, lane, region);
    load_q_raw<D, 2, false>(a, b, h, q0w, lane, qr);   // Q only
    if (a.cos_sin) {
      // Q arrives with the table rows (waiting for both keeps the compiler's
      // own waits, which do not see the DMA, off the rotation below).  The
      // empty asm statements keep the LDS reads between the waits.
      wait_vmcnt<0>();
      asm volatile("" ::: "memory");
      table_from_lds<D>(region, lane, qr.tab[0]);
      wait_lgkmcnt<0>();   // the reads are done before the region is refilled
      asm volatile("" ::: "memory");
      table_rows_to_lds<D>(a, q0w + 32, lane, region);
      rotate_q_tile<D, 2, 0>(a, qr, qf, qscale);
      wait_vmcnt<0>();
      asm volatile("" ::: "memory");
      table_from_lds<D>(region, lane, qr.tab[1]);
      rotate_q_tile<D, 2, 1>(a, qr, qf, qscale);
    } else {
      rotate_q<D, 2>(a, qr, qf, qscale);
    }
  }
#pragma unroll
  for (int t = 0; t < 2; ++t)
#pragma unroll
    for (int ds = 0; ds < NDS; ++ds) asm volatile("" : "+a"(qf[t][ds]));
  WaveState<D, 2> st;
  init_state<D, 2>(a, b, h, q0w, lane, st);
  // O into the AGPRs the inline-asm MFMAs accumulate in.
#pragma unroll
  for (int t = 0; t < 2; ++t)
#pragma unroll
    for (int dt = 0; dt < NDT; ++dt) asm volatile("" : "+a"(st.o[dt][t]));
  asm volatile("s_nop 4" ::: "memory");

  // Q, table and state loads (and, being older, the first two tiles' DMA)
  // complete here, so the only vector-memory operations in flight below
  // are the tile DMAs.
  wait_vmcnt<0>();

  // The pipeline's DMA: every tile it asks for is one group of DMA
  // instructions (a placeholder when the tile is not a full one inside the
  // keys, plus the clamped load after the half step when it is ragged).
  // Pipeline tiles [0, n_fast) are full key tiles inside the keys the
  // workgroup needs and go by the fast path; the pipeline walks their first
  // rows tile by tile.  With a window the walk is not monotonic: a tile goes
  // by the fast path if it is a pipeline tile and a full key tile, and its
  // first row comes from its key tile.
  const int n_full_k = min(n_key_tiles, Sk / BN);
  const int n_fast = fast_dma ? min(n_tiles, Sk / BN) : 0;
  auto fast_bound = [&](int u) YRB_INLINE {   // dma_plan takes u as real iff u < fast_bound(u)
    if constexpr (!WIN) return n_fast;
    return (fast_dma && u < n_tiles && key_tile(u) < n_full_k) ? u + 1 : 0;
  };
  const int64_t kstep = fast_dma ? (int64_t)BN * kstride : 0, vstep = fast_dma ? (int64_t)BN * vstride : 0;
  const __bf16* k_rows = kbase_s + key_tile(2) * kstep;   // tile 2, then one tile further per pipeline tile
  const __bf16* v_rows = vbase_s + key_tile(2) * vstep;
  const unsigned k0_m0 = __builtin_amdgcn_readfirstlane((unsigned)(uintptr_t)lds + wave * TL::LO * 1024);
  const unsigned v0_m0 = k0_m0 + LdsMap<D>::VBASE;
  const unsigned spare_m0 = k0_m0 + 2 * kPPBufs * T::TILEB;

  if (n_tiles > 0) {
    const LdsMap<D> m = lds_map<D>(lane);
    MaskInfo mi;
    mi.key_last = Sk - 1 - 4 * (lane >> 5);
    mi.q_last[0] = q_offset + q0w + l32 - k_offset - 4 * (lane >> 5);
    mi.q_last[1] = mi.q_last[0] + 32;
    mi.sink_end = sink_end - 4 * (lane >> 5);
    mi.window = a.window;
    mi.causal = a.causal != 0;
    mi.sink_end_u = sink_end;
    mi.w_lo_u = -1;
    bf16x8 kf[NDS];           // K of the next S chain
    bf16x8 vf[2][NDT];        // V of the next PV products
    bf16x8 p0[2], p1[2];
    f32x16 s0, s1;
    // The product of the quarter before the first is a no-op: P = V = 0.
#pragma unroll
    for (int half = 0; half < 2; ++half) {
      p1[half] = (bf16x8){};
#pragma unroll
      for (int dt = 0; dt < NDT; ++dt) vf[half][dt] = (bf16x8){};
    }
    Offsets of;
    offsets_from<D>(st, of);
    {   // arrival of tile 0; tile 2 (or a placeholder) goes out at once
      if (n_tiles > 1) wait_vmcnt<DMA>();
      else wait_vmcnt<0>();
      tile_barrier();
      const DmaPlan dp = dma_plan<D, 2 % kPPBufs>(2, fast_bound(2), n_tiles, k_rows, v_rows, ph_k, ph_v, k0_m0,
                                                  v0_m0, spare_m0);
      static_for<TL::LO>([&](auto n_tag) YRB_INLINE {
        constexpr int n = decltype(n_tag)::value;
        dma_lds_m0<n * 1024, n == 0>(dp.k_m0, dp.k, koff[n]);
      });
      static_for<TL::LO>([&](auto n_tag) YRB_INLINE {
        constexpr int n = decltype(n_tag)::value;
        dma_lds_m0<n * 1024, n == 0>(dp.v_m0, dp.v, voff[n]);
      });
      if (dp.slow) issue(2);
    }
#pragma unroll
    for (int ds = 0; ds < NDS; ++ds) kf[ds] = read_k_at<D, 0, 0>(lds, m, ds);
    s0 = qk_tile<D>(kf, qf[0], of.negb[0]);
    // With a window the test is made per wave, for its own 64 rows: fewer
    // tiles on the diagonal and at the window's lower edge need the mask
    // than for the workgroup's 256 rows.
    int n_full_m = n_full, w_lo_m = w_lo;
    if constexpr (WIN) {
      const int qf_w = q_offset + q0w - k_offset, ql_w = q_offset + min(Sq, q0w + QW) - 1 - k_offset;
      n_full_m = min(min(n_key_tiles, Sk / BN), max(0, qf_w + 1) / BN);
      w_lo_m = max(-1, ql_w - a.window);
    }
    const int n_full_s = __builtin_amdgcn_readfirstlane(n_full_m);
    const int w_lo_s = __builtin_amdgcn_readfirstlane(w_lo_m);
    mi.w_lo_u = w_lo_s;
    auto masked = [&](int kt) YRB_INLINE {
      return kt >= n_full_s || (kt * BN + BN - 1 >= sink_end && kt * BN <= w_lo_s);
    };
    if (masked(key_tile(0))) mask_scores<WIN>(s0, mi, 0, BN * key_tile(0));

    // Tile t (buffer BT = t % 4, a compile-time constant here): quarters 2t
    // and 2t+1; tiles from n_full on (the causal diagonal, the ragged end)
    // have their scores masked at the boundary before their softmax.  After the last tile the S chain and the K
    // reads of the quarter that does not exist run on stale LDS data and go
    // unused.
    auto tile = [&](int t, auto bt_tag) YRB_INLINE {
      constexpr int BT = decltype(bt_tag)::value;
      constexpr int BT1 = (BT + 1) % kPPBufs;
      const int kb = BN * key_tile(t), kb1 = BN * key_tile(t + 1);   // first keys of tiles t, t+1
      const bool mk = masked(kb / BN), mk1 = masked(kb1 / BN);         // quarters 2t, 2t+1 / 2t+2 masked
      bool g, nd;
      // H1(2t): S1(2t), PV1(2t-1); softmax 0; read K(2t+1)
      g = half_step<D, 1, 0, 0, BT, 1, false, true, EXACT>(st, of, lds, m, vf, p1, kf, qf[1], s1, s0, p0, mk, nd);
      settle<D, 0, EXACT, WIN>(s0, st, of, g, nd, p0, mk, s1, mi, 1, kb);
      // H2(2t): S0(2t+1), PV0(2t); softmax 1; read V(2t)
      g = half_step<D, 0, BT, 0, 0, 0, true, false, EXACT>(st, of, lds, m, vf, p0, kf, qf[0], s0, s1, p1, mk, nd);
      settle<D, 1, EXACT, WIN>(s1, st, of, g, nd, p1, mk, s0, mi, 0, kb + 32);
      // H1(2t+1): S1(2t+1), PV1(2t); softmax 0; arrival of tile t+1, read
      // K(2t+2) from it, and the DMA of tile t+3 into the buffer of tile t-1
      if constexpr (WIN) {
        k_rows = kbase_s + key_tile(t + 3) * kstep;
        v_rows = vbase_s + key_tile(t + 3) * vstep;
      } else {
        k_rows += kstep;
        v_rows += vstep;
      }
      const DmaPlan dp = dma_plan<D, (BT + 3) % kPPBufs>(t + 3, fast_bound(t + 3), n_tiles, k_rows, v_rows, ph_k, ph_v,
                                                         k0_m0, v0_m0, spare_m0);
      g = half_step<D, 1, 0, 0, BT1, 0, false, true, EXACT, true>(st, of, lds, m, vf, p1, kf, qf[1], s1, s0, p0, mk,
                                                                  nd, &dp,
                                                           koff, voff, wave);
      settle<D, 0, EXACT, WIN>(s0, st, of, g, nd, p0, mk, s1, mi, 1, kb + 32);
      if (__builtin_expect(dp.slow, 0)) issue(t + 3);
      // H2(2t+1): S0(2t+2), PV0(2t+1); softmax 1; read V(2t+1)
      g = half_step<D, 0, BT, 1, 0, 0, true, false, EXACT>(st, of, lds, m, vf, p0, kf, qf[0], s0, s1, p1, mk1, nd);
      settle<D, 1, EXACT, WIN>(s1, st, of, g, nd, p1, mk1, s0, mi, 0, kb1);
    };
    for (int t = 0;;) {
      tile(t, std::integral_constant<int, 0>{});
      if (++t == n_tiles) break;
      tile(t, std::integral_constant<int, 1>{});
      if (++t == n_tiles) break;
      tile(t, std::integral_constant<int, 2>{});
      if (++t == n_tiles) break;
      tile(t, std::integral_constant<int, 3>{});
      if (++t == n_tiles) break;
    }
    // PV of the last quarter, tile 1; then let the asm MFMAs finish before
    // any VALU code reads O.
#pragma unroll
    for (int i = 0; i < NDS; ++i) mfma_o(st.o[i % NDT][1], vf[i / NDT][i % NDT], p1[i / NDT]);
    xdl_drain();
  }

  // no DMA (placeholders included) may land after the workgroup leaves
  wait_vmcnt<0>();
  xdl_drain();
  if constexpr (!EXACT) {   // the reference in use stands for the max
#pragma unroll
    for (int qt = 0; qt < 2; ++qt) st.m_true[qt] = st.m_use[qt];
  }
  if (a.finalize && !a.store_state) {
    // every wave is past its last tile reads and its DMA has landed: the LDS
    // is free for the output transpose (16 KiB per wave)
    tile_barrier();
    if (!wave_live) return;
    finish_rows_lds<D>(a, b, h, q0w, lane, st, lds + wave * (64 * 2 * D));
    return;
  }
  if (!wave_live) return;
  finish_rows<D, 2>(a, b, h, q0w, lane, st);
}

template <int D, bool EXACT, bool WIN>
hipError_t launch_pp_as(const AttnArgs& a, hipStream_t stream) {
  constexpr int BM = kPPWaves * 64;
  constexpr int LDS_BYTES = (kPPBufs * 2 + 1) * Tile<D, kPPBN>::TILEB;   // K, V tiles and a spare
  static_assert(LDS_BYTES <= 160 * 1024, "gfx950 LDS");
  const int64_t n_qtiles = (a.Sq + BM - 1) / BM;
  const int64_t blocks = n_qtiles * a.B * a.Hq;
  if (blocks == 0) return hipSuccess;
  if (LDS_BYTES > 65536) {   // above the default dynamic-LDS limit
    const hipError_t attr = hipFuncSetAttribute(reinterpret_cast<const void*>(&attn_bf16_pp_kernel<D, EXACT, WIN>),
                                                hipFuncAttributeMaxDynamicSharedMemorySize, LDS_BYTES);
    if (attr != hipSuccess) return attr;
  }
  // The grid's last 30 % claims its items; under the sink+window mask, whose
  // items are about equally long, the last 15 %, so that more blocks keep
  // their XCD's heads in L2 (A/B at 16k with w = 4096: 0.886 -> 0.873 ms;
  // the causal prefill is within 0.5 % from 5 to 30 %, and slower at 50 %).
  constexpr int kStaticPct = WIN ? 85 : 70;
  const int claim_from =
      (a.claims && blocks >= kClaimMinBlocks) ? (int)(blocks * kStaticPct / 100) : (int)blocks;
  hipLaunchKernelGGL((attn_bf16_pp_kernel<D, EXACT, WIN>), dim3((unsigned)blocks), dim3(kPPWaves * 64), LDS_BYTES,
                     stream, a, n_qtiles, claim_from);
  return hipGetLastError();
}

template <int D>
hipError_t launch_pp(const AttnArgs& a, hipStream_t stream) {
  // The sink+window mask comes only with a finalized output (the prefill).
  if (a.window > 0) return a.store_state ? hipErrorInvalidValue : launch_pp_as<D, false, true>(a, stream);
  return a.store_state ? launch_pp_as<D, true, false>(a, stream) : launch_pp_as<D, false, false>(a, stream);
}

}  // namespace

hipError_t launch_attention_bf16_pp(int D, const AttnArgs& a, hipStream_t stream) {
  return D == 64 ? launch_pp<64>(a, stream) : launch_pp<128>(a, stream);
}

}  // namespace yrb
