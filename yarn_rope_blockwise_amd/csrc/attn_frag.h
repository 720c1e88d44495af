// Building blocks of the pipelined bf16 attention kernel (gfx950): LDS tile
// geometry and swizzles, the LDS-DMA tile loaders, the per-wave state and
// its inline-asm product O^T += V^T P^T, the work order, the query load and
// rotation, and the state's set-up and epilogue.  Included by the kernel's
// translation unit; everything here has internal linkage.
#pragma once

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

// s_waitcnt lgkmcnt(n), other counters untouched.
template <int N>
__device__ __forceinline__ void wait_lgkmcnt() {
  static_assert(N >= 0 && N < 16, "lgkmcnt range");
  __builtin_amdgcn_s_waitcnt(15 | (3 << 14) | (7 << 4) | (N << 8));
}

// Workgroup barrier that no memory access may cross in either direction at
// compile time (the LDS-DMA below is invisible to the compiler's model).
__device__ __forceinline__ void tile_barrier() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

// One tile (BN rows of K or V) global -> LDS.  The tile is TILEB/1024
// DMA instructions of 1 KiB.  In the clamped load below wave w issues
// instructions w, w+NW, ...; rows past the end are clamped to the last row:
// finite data, masked out of the softmax.  (The fast path, tile_offsets and
// dma_lds_m0, gives each wave LO consecutive blocks instead.)
template <int D, int BN, int NW>
struct TileLoads {
  static constexpr int INSTR = Tile<D, BN>::TILEB / 1024;
  static constexpr int LO = INSTR / NW;                // every wave issues at least LO
  static constexpr int EXTRA = INSTR % NW;             // waves < EXTRA issue LO + 1
};

// global_load_lds_dwordx4 with a per-lane 64-bit address: lane i's 16
// bytes land at m0 + 16*i, with m0 = m0_base + IMM written inside the asm
// (used off the hot loop: the clamped tile load and the table rows).  The
// DMA is issued from asm so the compiler does not add a vmcnt(0) before
// every LDS read of another buffer: ordering is by explicit vmcnt waits and
// barriers.  No register outputs.
#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"   // m0 is reserved; nothing else here uses it
template <int IMM>
__device__ __forceinline__ void dma_lds_vaddr(unsigned m0_base, const void* g) {
  asm volatile("s_add_u32 m0, %1, %2\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, off"
               :
               : "v"(g), "s"(m0_base), "i"(IMM)
               : "memory", "m0", "scc");
}
#pragma clang diagnostic pop

// The fast tile DMA: SGPR base address, 32-bit per-lane byte offset, m0
// held by the compiler (one value per K or V group, set once and kept across
// the group's instructions).  The instruction offset IMM (below 4 KiB) moves
// both addresses: lane i reads rows + off + IMM and writes m0 + IMM + 16 i.
// FIRST: the group's first instruction, one wait state after the m0 write.
template <int IMM, bool FIRST>
__device__ __forceinline__ void dma_lds_m0(unsigned m0, const void* rows, unsigned off) {
  static_assert(IMM >= 0 && IMM < 4096, "global instruction offset range");
  if constexpr (FIRST)
    asm volatile("s_nop 0\n\tglobal_load_lds_dwordx4 %0, %1 offset:%2" : : "v"(off), "s"(rows), "i"(IMM), "{m0}"(m0)
                 : "memory");
  else
    asm volatile("global_load_lds_dwordx4 %0, %1 offset:%2" : : "v"(off), "s"(rows), "i"(IMM), "{m0}"(m0) : "memory");
}

template <int D, int BN, int NW, bool IS_V>
__device__ __forceinline__ void load_tile(YRB_LDS char* dst, const __bf16* src, int stride, int k0,
                                          int Sk, int wave, int lane) {
  using T = Tile<D, BN>;
  using TL = TileLoads<D, BN, NW>;
  constexpr int ROWB = T::ROWB;
  const unsigned m0w = __builtin_amdgcn_readfirstlane((unsigned)(uintptr_t)dst + wave * 1024);
  static_for<TL::LO + (TL::EXTRA ? 1 : 0)>([&](auto n_tag) YRB_INLINE {
    constexpr int n = decltype(n_tag)::value;
    const int idx = n * NW + wave;
    if (n >= TL::LO && idx >= TL::INSTR) return;   // wave-uniform
    const int off = idx * 1024 + lane * 16;
    const int r = off / ROWB;
    const int p = (off % ROWB) >> 4;
    const int c = IS_V ? (p ^ vsw<D>(r)) : (p ^ ksw<D>(r));
    const int row = min(k0 + r, Sk - 1);
    dma_lds_vaddr<n * NW * 1024>(m0w, src + (int64_t)row * stride + c * 8);
  });
}

// Tiles that need no row clamp (the fast path): wave w fills the tile's
// 1 KiB blocks w LO .. w LO + LO - 1, its n-th instruction with offset
// n KiB (dma_lds_m0).  Each lane's byte offsets of its 16-byte chunks,
// relative to the tile's first row and less that instruction offset, are
// fixed for the whole launch; the tile's row base then goes in SGPRs.
// The token stride must be at least D (then each offset is at least n KiB:
// a row is 2D bytes, which divides 1 KiB).  PLACEHOLDER: offsets 16 lane
// only, for instructions that read a small dummy buffer.
template <int D, int BN, int NW, bool IS_V>
__device__ __forceinline__ void tile_offsets(int stride, int wave, int lane, bool placeholder,
                                             unsigned (&off)[TileLoads<D, BN, NW>::LO]) {
  using TL = TileLoads<D, BN, NW>;
  static_assert(TL::EXTRA == 0, "tile DMA must split evenly over the waves");
  constexpr int ROWB = Tile<D, BN>::ROWB;
  static_assert(1024 % ROWB == 0, "rows tile the 1 KiB blocks");
#pragma unroll
  for (int n = 0; n < TL::LO; ++n) {
    const int o = (wave * TL::LO + n) * 1024 + lane * 16;
    const int r = o / ROWB;
    const int p = (o % ROWB) >> 4;
    const int c = IS_V ? (p ^ vsw<D>(r)) : (p ^ ksw<D>(r));
    off[n] = placeholder ? (unsigned)(lane * 16) : (unsigned)(r * stride + c * 8) * 2u - (unsigned)(n * 1024);
  }
}

// A pointer the caller knows to be the same in every lane, moved to SGPRs.
__device__ __forceinline__ const __bf16* wave_uniform(const __bf16* p) {
  // readfirstlane works on int: each half is taken back as unsigned before
  // widening, so the low half is zero-extended, not sign-extended.
  const uint64_t v = (uint64_t)(uintptr_t)p;
  const uint64_t lo = (unsigned)__builtin_amdgcn_readfirstlane((int)(unsigned)v);
  const uint64_t hi = (unsigned)__builtin_amdgcn_readfirstlane((int)(unsigned)(v >> 32));
  return reinterpret_cast<const __bf16*>((uintptr_t)(lo | (hi << 32)));
}

template <int D, int BN, int NW>
__device__ __forceinline__ void load_tile_rows(YRB_LDS char* dst, const __bf16* tile_rows,
                                               const unsigned (&off)[TileLoads<D, BN, NW>::LO],
                                               int wave) {
  using TL = TileLoads<D, BN, NW>;
  const __bf16* const rows = wave_uniform(tile_rows);
  const unsigned m0w = __builtin_amdgcn_readfirstlane((unsigned)(uintptr_t)dst + wave * TL::LO * 1024);
  static_for<TL::LO>([&](auto n_tag) YRB_INLINE {
    constexpr int n = decltype(n_tag)::value;
    dma_lds_m0<n * 1024, n == 0>(m0w, rows, off[n]);
  });
}

template <int D, int NQT>
struct WaveState {
  f32x16 o[D / 32][NQT];
  float m_use[NQT];    // max the exponentials are taken against (log2 units)
  float m_true[NQT];   // exact running max (log2 units)
  float l[NQT];        // per-lane partial row sum (this half's keys)
};

// O^T(AGPR) += V^T P^T for one 32x32x16 step, as inline asm so that the
// accumulator stays in AGPRs while the compiler keeps its own MFMAs in the
// VGPR form.  The compiler does not see this MFMA: VALU code that touches
// the accumulator next to it waits out the hazards itself (xdl_drain before
// reading it, s_nop after writing it).
__device__ __forceinline__ void mfma_o(f32x16& o, const bf16x8& v, const bf16x8& p) {
  asm("v_mfma_f32_32x32x16_bf16 %0, %1, %2, %0" : "+a"(o) : "v"(v), "v"(p));
}

// Wait states after the inline-asm MFMAs before VALU code reads or writes
// their accumulators (more than the longest MFMA-to-VALU requirement).
__device__ __forceinline__ void xdl_drain() { asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7" ::: "memory"); }

// O *= alpha on an accumulator that lives in AGPRs, between inline-asm MFMAs.
// Each element goes AGPR -> VGPR -> AGPR inside one asm statement, so the
// compiler never holds O in VGPRs (it would hoist such copies out of this
// rarely taken path into the hot one).
__device__ __forceinline__ void scale_o_agpr(f32x16& o, float alpha) {
  xdl_drain();
#pragma unroll
  for (int j = 0; j < 16; ++j) {
    float e = o[j];
    float tmp;
    asm volatile("v_accvgpr_read_b32 %1, %0\n\tv_mul_f32 %1, %1, %2\n\tv_accvgpr_write_b32 %0, %1"
                 : "+a"(e), "=&v"(tmp)
                 : "v"(alpha));
    o[j] = e;
  }
  asm volatile("" : "+a"(o));
  asm volatile("s_nop 4" ::: "memory");
}

// Work item of a workgroup: the heaviest (causal) query tiles are launched
// first, and consecutive workgroups take heads that are 8 apart, so the
// workgroups an XCD runs at once (blocks go round-robin over the 8 XCDs)
// share a few key/value heads in its L2.
struct WorkItem {
  int b, h, hk, qtile;
};

__device__ __forceinline__ WorkItem work_item_at(const AttnArgs& a, int64_t n_qtiles, int idx) {
  const int Hq = (int)a.Hq;
  const int per = (int)(a.B * a.Hq);
  const int rank = idx / per;
  const int rem = idx - rank * per;
  WorkItem w;
  w.b = rem / Hq;
  const int hp = rem - w.b * Hq;
  w.h = (Hq % 8 == 0) ? (hp & 7) * (Hq >> 3) + (hp >> 3) : hp;
  w.qtile = a.causal ? (int)(n_qtiles - 1 - rank) : rank;
  w.hk = w.h / (Hq / (int)a.Hkv);
  return w;
}
// Q fragments and their table rows as loaded, before the rotation.
template <int D, int NQT>
struct QRaw {
  u32x4 raw[NQT][D / 16];
  f32x4 tab[NQT][D / 32][4];
};

// Every load of Q and of its table rows goes out before any arithmetic:
// one memory round trip (issued per tile, the loads would wait on each
// other through register reuse).
template <int D, int NQT, bool TAB = true>
__device__ __forceinline__ void load_q_raw(const AttnArgs& a, int b, int h, int q0w, int lane,
                                           QRaw<D, NQT>& qr) {
  constexpr int NDS = D / 16;
  const int hh = lane >> 5;
  const int l32 = lane & 31;
  const int Sq = (int)a.Sq;
  const int q_offset = (int)a.q_offset;
  const __bf16* qbase = reinterpret_cast<const __bf16*>(a.q) + b * a.qs[0] + h * a.qs[2];
#pragma unroll
  for (int qt = 0; qt < NQT; ++qt) {
    const int row = min(q0w + qt * 32 + l32, Sq - 1);
    const __bf16* qp = qbase + row * a.qs[1] + 8 * hh;
#pragma unroll
    for (int ds = 0; ds < NDS; ++ds) qr.raw[qt][ds] = *reinterpret_cast<const u32x4*>(qp + 16 * ds);
    if (TAB && a.cos_sin) {
      const float* cs = a.cos_sin + (int64_t)(q_offset + row) * D;
#pragma unroll
      for (int ds = 0; ds < NDS / 2; ++ds)
#pragma unroll
        for (int u2 = 0; u2 < 4; ++u2)
          qr.tab[qt][ds][u2] = reinterpret_cast<const f32x4*>(cs + 2 * (16 * ds + 8 * hh))[u2];
    }
  }
}

// Rotation of query tile QT (pair (i, i + D/2) sits in fragments ds and
// ds + NDS/2), the qscale factor, and one rounding to bf16.
template <int D, int NQT, int QT>
__device__ __forceinline__ void rotate_q_tile(const AttnArgs& a, QRaw<D, NQT>& qr, bf16x8 (&qf)[NQT][D / 16],
                                              float qscale) {
  constexpr int NDS = D / 16;
  if (a.cos_sin) {
#pragma unroll
    for (int ds = 0; ds < NDS / 2; ++ds) {
      float x[8], z[8], lo[8], hi[8];
      unpack8(qr.raw[QT][ds], x);
      unpack8(qr.raw[QT][ds + NDS / 2], z);
#pragma unroll
      for (int u2 = 0; u2 < 4; ++u2) {
        const f32x4 tt = qr.tab[QT][ds][u2];
        lo[2 * u2] = (x[2 * u2] * tt[0] - z[2 * u2] * tt[1]) * qscale;
        hi[2 * u2] = (x[2 * u2] * tt[1] + z[2 * u2] * tt[0]) * qscale;
        lo[2 * u2 + 1] = (x[2 * u2 + 1] * tt[2] - z[2 * u2 + 1] * tt[3]) * qscale;
        hi[2 * u2 + 1] = (x[2 * u2 + 1] * tt[3] + z[2 * u2 + 1] * tt[2]) * qscale;
      }
      qr.raw[QT][ds] = pack8(lo);
      qr.raw[QT][ds + NDS / 2] = pack8(hi);
    }
  } else if (qscale != 1.0f) {
#pragma unroll
    for (int ds = 0; ds < NDS; ++ds) {
      float x[8];
      unpack8(qr.raw[QT][ds], x);
#pragma unroll
      for (int u = 0; u < 8; ++u) x[u] *= qscale;
      qr.raw[QT][ds] = pack8(x);
    }
  }
#pragma unroll
  for (int ds = 0; ds < NDS; ++ds) qf[QT][ds] = __builtin_bit_cast(bf16x8, qr.raw[QT][ds]);
}

template <int D, int NQT>
__device__ __forceinline__ void rotate_q(const AttnArgs& a, QRaw<D, NQT>& qr, bf16x8 (&qf)[NQT][D / 16],
                                         float qscale) {
  static_for<NQT>([&](auto qt_tag) YRB_INLINE {
    rotate_q_tile<D, NQT, decltype(qt_tag)::value>(a, qr, qf, qscale);
  });
}

// Running state of one wave: empty, or read from (o_acc, m, l) of an
// earlier step (m stored in natural-log units, kept here in log2 units).
template <int D, int NQT>
__device__ __forceinline__ void init_state(const AttnArgs& a, int b, int h, int q0w, int lane,
                                           WaveState<D, NQT>& st) {
  constexpr int NDT = D / 32;
  const int hh = lane >> 5;
  const int l32 = lane & 31;
  const int Sq = (int)a.Sq;
  const int Hq = (int)a.Hq;
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
}

// Epilogue of one wave: restore the exact running max, then store the state
// (ring step) and/or the normalised output and log-sum-exp (last step).
template <int D, int NQT>
__device__ __forceinline__ void finish_rows(const AttnArgs& a, int b, int h, int q0w, int lane,
                                            WaveState<D, NQT>& st) {
  constexpr int NDT = D / 32;
  const int hh = lane >> 5;
  const int l32 = lane & 31;
  const int Sq = (int)a.Sq;
  const int Hq = (int)a.Hq;
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

}  // namespace
}  // namespace yrb
