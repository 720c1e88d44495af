// One-query decode over an attention-sink + sliding-window KV cache, gfx950.
//
// The cache of a sequence holds its first n_sink tokens and its last
// `window` tokens ("Context Length Extension" (14cs17), section "Sliding
// Window + Attention Sinks": {x_1..x_s} U {x_{t-w+1}..x_t}; jovanaeducation
// guide, "Attention sinks").  Entries are re-indexed: entry e sits at
// position e, sinks in slots 0..n_sink-1, the window a ring buffer whose
// oldest entry is slot n_sink + ring_head.  Keys are stored un-rotated and
// rotated here at their cache position on every call; the query is rotated
// at position len - 1.
//
// gfx950 design: the call is HBM-bound (every cached K and V byte is read
// once, ~1 flop per byte), so the kernel is a streaming reduction.
//  * One workgroup (4 waves) per (sequence, 4 key/value heads): wave w owns
//    head 4g + w and the G query heads that share it.  All four waves walk
//    the same slots in memory order, so the cos/sin row of each slot's
//    position is fetched once per workgroup into LDS and shared (fetching
//    it per head costs as many bytes as K and V together).
//  * D/16 lanes share one key row: each lane reads the two 16-byte chunks
//    holding pairs (i, i + d/2) for its 8 pairs, so the rotation is
//    lane-local.  Each step a wave holds 4 rounds of K/V loads in flight,
//    and the next step's loads are issued before this step is reduced
//    (non-temporal: the cache is far larger than the L2/MALL).
//  * The score of a rotated key is  sum_i c_i (q_i k_i + q_j k_j) +
//    s_i (q_j k_i - q_i k_j), j = i + d/2.
//  * Online softmax per wave in the exp2 domain; lanes of one head then
//    combine their partial sums with cross-lane shuffles.
#include "common.h"
#include "kernels.h"

namespace yrb {

namespace {

constexpr int kWaves = 4;      // = key/value heads per workgroup

// Cache element: bf16 (two 16-byte chunks of 8 values per lane and key) or
// fp8 E4M3 (OCP; two 8-byte chunks).
template <bool FP8>
struct CacheType {
  using Chunk = u32x4;
  using Elem = __bf16;
  static constexpr int kRounds = 4;   // key rounds per wave per step
  __device__ static void unpack(const Chunk& w, float (&f)[8]) { unpack8(w, f); }
};
template <>
struct CacheType<true> {
  using Chunk = u32x2;
  using Elem = uint8_t;
  // Four rounds, as for bf16: six measured the same and eight lost a wave
  // per SIMD to registers (0.72 ms against 0.47 ms at 64 x 32 x 4100).
  static constexpr int kRounds = 4;
  // v_cvt_pk_f32_fp8 decodes two bytes of a dword; on gfx950 its fp8 is the
  // OCP E4M3 format (checked against a host decoder for all 256 codes).
  __device__ static void unpack(const Chunk& w, float (&f)[8]) {
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const f32x2 lo = __builtin_amdgcn_cvt_pk_f32_fp8((int)w[h], false);
      const f32x2 hi = __builtin_amdgcn_cvt_pk_f32_fp8((int)w[h], true);
      f[4 * h] = lo[0];
      f[4 * h + 1] = lo[1];
      f[4 * h + 2] = hi[0];
      f[4 * h + 3] = hi[1];
    }
  }
};

// Key rounds per wave per step: the cache type's, halved for a bf16 cache
// with 8 query heads per key head, whose per-head query and output
// registers leave too few for four rounds of 16-byte chunks (it spilled).
template <bool FP8, int G>
constexpr int rounds_of() { return (!FP8 && G >= 8) ? 2 : CacheType<FP8>::kRounds; }

// K/V of one step for one lane: R keys, two chunks each.
template <bool FP8, int R>
struct KVChunk {
  typename CacheType<FP8>::Chunk klo[R], khi[R], vlo[R], vhi[R];
  bool ok[R];
};

// The 8 pairs of one lane from its two chunks a, b (8 values each, at
// elements 8cc and d/2 + 8cc in either layout): half-split, pairs
// 8cc .. 8cc+7 with a the first elements and b their partners; interleaved
// (IL), a holds pairs 4cc .. 4cc+3 and b pairs d/4 + 4cc .. +3, each pair
// two adjacent values.
template <bool IL>
__device__ __forceinline__ void pairs_of(const float (&a)[8], const float (&b)[8], float (&x)[8],
                                         float (&z)[8]) {
#pragma unroll
  for (int u = 0; u < 8; ++u) {
    if constexpr (IL) {
      x[u] = u < 4 ? a[2 * u] : b[2 * u - 8];
      z[u] = u < 4 ? a[2 * u + 1] : b[2 * u - 7];
    } else {   // half-split
      x[u] = a[u];
      z[u] = b[u];
    }
  }
}

template <int D, int G, bool FP8, bool IL>
__global__ __launch_bounds__(kWaves * 64) void decode_bf16_kernel(DecodeArgs a) {
  using CT = CacheType<FP8>;
  using Chunk = typename CT::Chunk;
  using Elem = typename CT::Elem;
  constexpr int kRounds = rounds_of<FP8, G>();
  using KV = KVChunk<FP8, kRounds>;
  constexpr int TPK = D / 16;              // lanes per key row
  constexpr int KPW = 64 / TPK;            // keys per wave per round
  constexpr int KPS = KPW * kRounds;       // slots per step (shared by the 4 waves)
  constexpr int TROWB = 4 * D;             // bytes of one table row: D/2 pairs x (cos, sin)
  constexpr int TABB = KPS * TROWB;        // table bytes per step
  constexpr int TCH = TABB / 16 / (kWaves * 64);   // 16-byte table chunks per thread per step
  static_assert(TCH * 16 * kWaves * 64 == TABB, "table tile must split over the threads");
  __shared__ __attribute__((aligned(16))) char tab_raw[2 * TABB];
  YRB_LDS char* const tab0 = (YRB_LDS char*)tab_raw;
  YRB_LDS char* const tab1 = tab0 + TABB;

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int kg = lane / TPK;               // key within the round
  const int cc = lane % TPK;               // chunk: pairs 8cc .. 8cc+7
  const int n_groups = (int)((a.Hkv + kWaves - 1) / kWaves);
  const int64_t b = blockIdx.x / n_groups;
  const int hk_raw = (int)(blockIdx.x % n_groups) * kWaves + wave;
  const bool head_live = hk_raw < a.Hkv;
  const int hk = head_live ? hk_raw : (int)a.Hkv - 1;   // idle waves read a valid head
  const int C = (int)(a.n_sink + a.window);
  const int n_sink = (int)a.n_sink, window = (int)a.window;

  const int len_raw = a.cache_len[b];
  const int rh_raw = a.ring_head ? a.ring_head[b] : 0;
  const bool bad_seq = len_raw < 0 || len_raw > C || rh_raw < 0 || rh_raw >= window;
  const int len = bad_seq ? 0 : len_raw;
  const int rh = bad_seq ? 0 : rh_raw;

  // Position of the entry in `slot`, or -1 when the slot holds none.  A
  // window slot below C is less than `window` past n_sink and the head is
  // below `window`, so one conditional add takes the offset mod window, with
  // no integer division.
  auto position = [&](int slot) -> int {
    const int d = slot - n_sink - rh;
    const int e = slot < n_sink ? slot : n_sink + (d < 0 ? d + window : d);
    return (slot < C && e < len) ? e : -1;
  };

  // Rotated query (fp32) for each of the G heads: pairs 8cc..8cc+7.
  float qlo[G][8], qhi[G][8];
  {
    const int qpos = len > 0 ? len - 1 : 0;
    // (cos, sin) of the lane's pairs, two per f32x4 (see pairs_of)
    const float* trow = a.cos_sin + (int64_t)qpos * D;
    float c[8], s[8];
#pragma unroll
    for (int u2 = 0; u2 < 4; ++u2) {
      const int f = IL ? (u2 < 2 ? 8 * cc + 4 * u2 : D / 2 + 8 * cc + 4 * (u2 - 2)) : 16 * cc + 4 * u2;
      const f32x4 tt = *reinterpret_cast<const f32x4*>(trow + f);
      c[2 * u2] = tt[0]; s[2 * u2] = tt[1]; c[2 * u2 + 1] = tt[2]; s[2 * u2 + 1] = tt[3];
    }
#pragma unroll
    for (int g = 0; g < G; ++g) {
      const __bf16* qp = reinterpret_cast<const __bf16*>(a.q) + b * a.qs[0] +
                         (int64_t)(hk * G + g) * a.qs[1];
      float qa[8], qb[8], x[8], z[8];
      unpack8(*reinterpret_cast<const u32x4*>(qp + 8 * cc), qa);
      unpack8(*reinterpret_cast<const u32x4*>(qp + D / 2 + 8 * cc), qb);
      pairs_of<IL>(qa, qb, x, z);
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        qlo[g][u] = x[u] * c[u] - z[u] * s[u];
        qhi[g][u] = x[u] * s[u] + z[u] * c[u];
      }
    }
  }

  // fp8: per (sequence, kv head) dequantisation scales; K's folds into the
  // logit scale, V's into the final normalisation.
  const float k_deq = (FP8 && a.k_scale) ? a.k_scale[b * a.Hkv + hk] : 1.0f;
  const float v_deq = (FP8 && a.v_scale) ? a.v_scale[b * a.Hkv + hk] : 1.0f;
  const float scale_log2 = a.softmax_scale * kLog2e * k_deq;
  float m[G], l[G], o_lo[G][8], o_hi[G][8];
#pragma unroll
  for (int g = 0; g < G; ++g) {
    m[g] = -INFINITY;
    l[g] = 0.f;
#pragma unroll
    for (int u = 0; u < 8; ++u) o_lo[g][u] = o_hi[g][u] = 0.f;
  }

  const Elem* kb = reinterpret_cast<const Elem*>(a.k) + b * a.cs[0] + hk * a.cs[1];
  const Elem* vb = reinterpret_cast<const Elem*>(a.v) + b * a.cs[0] + hk * a.cs[1];
  const int n_slots = len <= n_sink ? len : C;   // slots worth scanning

  // Table rows of the step starting at `base`: thread t fetches TCH 16-byte
  // chunks; chunk k of the tile is row k / (TROWB/16), column k % (TROWB/16).
  auto load_tab = [&](int base, u32x4 (&tv)[TCH]) {
#pragma unroll
    for (int n = 0; n < TCH; ++n) {
      const int k = n * (kWaves * 64) + threadIdx.x;
      const int row = k / (TROWB / 16);
      const int col = k % (TROWB / 16);
      const int pos = position(base + row);
      tv[n] = *reinterpret_cast<const u32x4*>(a.cos_sin + (int64_t)(pos < 0 ? 0 : pos) * D +
                                               4 * col);
    }
  };
  auto store_tab = [&](YRB_LDS char* dst, const u32x4 (&tv)[TCH]) {
#pragma unroll
    for (int n = 0; n < TCH; ++n) {
      const int k = n * (kWaves * 64) + threadIdx.x;
      *reinterpret_cast<YRB_LDS u32x4*>(dst + 16 * k) = tv[n];
    }
  };
  // K/V loads of the step starting at `base`.
  auto load_kv = [&](int base, KV& ch) {
#pragma unroll
    for (int r = 0; r < kRounds; ++r) {
      const int slot = base + r * KPW + kg;
      ch.ok[r] = position(slot) >= 0 && head_live;
      const int sc = slot < C ? slot : C - 1;
      const Elem* kp = kb + (int64_t)sc * a.cs[2];
      const Elem* vp = vb + (int64_t)sc * a.cs[2];
      ch.klo[r] = __builtin_nontemporal_load(reinterpret_cast<const Chunk*>(kp + 8 * cc));
      ch.khi[r] = __builtin_nontemporal_load(reinterpret_cast<const Chunk*>(kp + D / 2 + 8 * cc));
      ch.vlo[r] = __builtin_nontemporal_load(reinterpret_cast<const Chunk*>(vp + 8 * cc));
      ch.vhi[r] = __builtin_nontemporal_load(reinterpret_cast<const Chunk*>(vp + D / 2 + 8 * cc));
    }
  };
  // Fold one step's keys into (m, l, o); (cos, sin) come from the LDS tile.
  auto fold = [&](const KV& ch, const YRB_LDS char* tl) {
    float sc_[G][kRounds];
#pragma unroll
    for (int r = 0; r < kRounds; ++r) {
      const YRB_LDS char* trow = tl + (r * KPW + kg) * TROWB;
      float c[8], s[8], ka[8], kb_[8], x[8], z[8];
#pragma unroll
      for (int u2 = 0; u2 < 4; ++u2) {
        const int off = IL ? (u2 < 2 ? 32 * cc + 16 * u2 : 2 * D + 32 * cc + 16 * (u2 - 2)) : 64 * cc + 16 * u2;
        const f32x4 tt = *reinterpret_cast<const YRB_LDS f32x4*>(trow + off);
        c[2 * u2] = tt[0]; s[2 * u2] = tt[1]; c[2 * u2 + 1] = tt[2]; s[2 * u2 + 1] = tt[3];
      }
      CT::unpack(ch.klo[r], ka);
      CT::unpack(ch.khi[r], kb_);
      pairs_of<IL>(ka, kb_, x, z);
#pragma unroll
      for (int g = 0; g < G; ++g) {
        float acc = 0.f;
#pragma unroll
        for (int u = 0; u < 8; ++u) {
          const float pc = qlo[g][u] * x[u] + qhi[g][u] * z[u];
          const float ps = qhi[g][u] * x[u] - qlo[g][u] * z[u];
          acc = __builtin_fmaf(c[u], pc, __builtin_fmaf(s[u], ps, acc));
        }
        // reduce over the TPK lanes of this key
#pragma unroll
        for (int off = 1; off < TPK; off <<= 1) acc += __shfl_xor(acc, off);
        sc_[g][r] = ch.ok[r] ? acc * scale_log2 : -INFINITY;
      }
    }
#pragma unroll
    for (int g = 0; g < G; ++g) {
      float mx = sc_[g][0];
#pragma unroll
      for (int r = 1; r < kRounds; ++r) mx = fmaxf(mx, sc_[g][r]);
#pragma unroll
      for (int off = TPK; off < 64; off <<= 1) mx = fmaxf(mx, __shfl_xor(mx, off));
      const float mn = fmaxf(m[g], mx);
      if (mn == -INFINITY) continue;
      const float alpha = m[g] == -INFINITY ? 0.f : fast_exp2(m[g] - mn);
      m[g] = mn;
      l[g] *= alpha;
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        o_lo[g][u] *= alpha;
        o_hi[g][u] *= alpha;
      }
#pragma unroll
      for (int r = 0; r < kRounds; ++r) {
        const float p = fast_exp2(sc_[g][r] - mn);   // 0 for a slot without an entry
        l[g] += p;
        // Such a slot's values are zeroed as raw words (whatever the cache
        // holds there, NaN codes included), so p * v adds 0.
        float v1[8], v2[8];
        CT::unpack(ch.ok[r] ? ch.vlo[r] : Chunk{}, v1);
        CT::unpack(ch.ok[r] ? ch.vhi[r] : Chunk{}, v2);
#pragma unroll
        for (int u = 0; u < 8; ++u) {
          o_lo[g][u] = __builtin_fmaf(p, v1[u], o_lo[g][u]);
          o_hi[g][u] = __builtin_fmaf(p, v2[u], o_hi[g][u]);
        }
      }
    }
  };
  // LDS-only barrier: the table writes are done (lgkmcnt), the K/V prefetch
  // in flight (vmcnt) is not waited for.
  auto lds_barrier = [&]() {
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_waitcnt(0xC07F);   // lgkmcnt(0); vmcnt, expcnt left at their maximum
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
  };

  // Step: tables and K/V of the next step are issued (tables first), this
  // step is reduced, then the next table tile is written to the other LDS
  // buffer.  One barrier per step: all waves are done with the current tile
  // before anyone overwrites the buffer it sits in.
  if (n_slots > 0) {
    u32x4 tv[TCH];
    load_tab(0, tv);
    store_tab(tab0, tv);
  }
  lds_barrier();
  KV c0, c1;
  if (n_slots > 0) load_kv(0, c0);
  auto step = [&](int base, KV& cur, KV& nxt, const YRB_LDS char* tl,
                  YRB_LDS char* tn) {
    const bool more = base + KPS < n_slots;
    u32x4 tv[TCH];
    if (more) {
      load_tab(base + KPS, tv);
      load_kv(base + KPS, nxt);
    }
    fold(cur, tl);
    if (more) store_tab(tn, tv);
    lds_barrier();
    return more;
  };
  for (int base = 0; base < n_slots; base += 2 * KPS) {
    if (!step(base, c0, c1, tab0, tab1)) break;
    if (!step(base + KPS, c1, c0, tab1, tab0)) break;
  }

  // Reduce across the key groups of the wave (lanes with equal cc), then
  // write the G output rows of this head.
#pragma unroll
  for (int g = 0; g < G; ++g) {
#pragma unroll
    for (int off = TPK; off < 64; off <<= 1) {
      l[g] += __shfl_xor(l[g], off);
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        o_lo[g][u] += __shfl_xor(o_lo[g][u], off);
        o_hi[g][u] += __shfl_xor(o_hi[g][u], off);
      }
    }
    if (head_live && kg == 0) {
      const float inv = l[g] > 0.f ? v_deq / l[g] : 0.f;
      float lo[8], hi[8];
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        lo[u] = bad_seq ? __builtin_nanf("") : o_lo[g][u] * inv;
        hi[u] = bad_seq ? __builtin_nanf("") : o_hi[g][u] * inv;
      }
      __bf16* op = reinterpret_cast<__bf16*>(a.o) + b * a.os[0] + (int64_t)(hk * G + g) * a.os[1];
      *reinterpret_cast<u32x4*>(op + 8 * cc) = pack8(lo);
      *reinterpret_cast<u32x4*>(op + D / 2 + 8 * cc) = pack8(hi);
    }
  }
}

template <int D, int G, bool FP8, bool IL>
hipError_t launch_dec(const DecodeArgs& a, hipStream_t stream) {
  const int64_t blocks = a.B * ((a.Hkv + kWaves - 1) / kWaves);
  if (blocks == 0) return hipSuccess;
  hipLaunchKernelGGL((decode_bf16_kernel<D, G, FP8, IL>), dim3((unsigned)blocks), dim3(kWaves * 64),
                     0, stream, a);
  return hipGetLastError();
}

template <int D, bool FP8, bool IL>
hipError_t launch_dec_g(const DecodeArgs& a, hipStream_t stream) {
  switch (a.Hq / a.Hkv) {
    case 1: return launch_dec<D, 1, FP8, IL>(a, stream);
    case 2: return launch_dec<D, 2, FP8, IL>(a, stream);
    case 4: return launch_dec<D, 4, FP8, IL>(a, stream);
    case 8: return launch_dec<D, 8, FP8, IL>(a, stream);
    default: return hipErrorInvalidValue;
  }
}

template <bool FP8, bool IL>
hipError_t launch_dec_d(int D, const DecodeArgs& a, hipStream_t stream) {
  return D == 64 ? launch_dec_g<64, FP8, IL>(a, stream) : launch_dec_g<128, FP8, IL>(a, stream);
}

}  // namespace

// Cache dtype kBF16 or kFP8E4M3 (query and output are bf16 either way);
// interleaved: keys and query paired (2i, 2i+1) instead of (i, i + d/2).
hipError_t launch_decode(int cache_dtype, int D, bool interleaved, const DecodeArgs& a,
                         hipStream_t stream) {
  if (cache_dtype == kBF16)
    return interleaved ? launch_dec_d<false, true>(D, a, stream) : launch_dec_d<false, false>(D, a, stream);
  if (cache_dtype == kFP8E4M3)
    return interleaved ? launch_dec_d<true, true>(D, a, stream) : launch_dec_d<true, false>(D, a, stream);
  return hipErrorInvalidValue;
}

}  // namespace yrb
