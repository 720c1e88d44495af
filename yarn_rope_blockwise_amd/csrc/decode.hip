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
//  * One workgroup (4 waves) per (sequence, key/value head), covering the G
//    query heads that share it.  Slots are walked in memory order.
//  * D/16 lanes share one key row: each lane reads the two 16-byte chunks
//    holding pairs (i, i + d/2) for its 8 pairs, so the rotation is
//    lane-local.  Per iteration a wave has 4 rounds of K and V loads in
//    flight (non-temporal: the cache is far larger than the L2/MALL).
//  * The score of a rotated key is  sum_i c_i (q_i k_i + q_j k_j) +
//    s_i (q_j k_i - q_i k_j), j = i + d/2, with (c, s) read from the fp32
//    table row of the entry's position (2 MiB for 4100 rows: L2-resident).
//  * Online softmax per wave (exp2 domain), then the 4 waves' (m, l, o) are
//    merged through LDS.
#include "common.h"
#include "kernels.h"

namespace yrb {

namespace {

constexpr int kWaves = 4;
// Key rounds per wave per iteration, and whether the next iteration's K/V
// loads are issued before the current one is reduced (register prefetch).
#ifndef YRB_DECODE_ROUNDS
#define YRB_DECODE_ROUNDS 4
#endif
#ifndef YRB_DECODE_PREFETCH
#define YRB_DECODE_PREFETCH 1
#endif
constexpr int kRounds = YRB_DECODE_ROUNDS;

// K/V of one iteration for one lane: kRounds keys, two 16-byte chunks each.
struct KVChunk {
  u32x4 klo[kRounds], khi[kRounds], vlo[kRounds], vhi[kRounds];
  int epos[kRounds];
  bool ok[kRounds];
};

template <int D, int G>
__global__ __launch_bounds__(kWaves * 64) void decode_bf16_kernel(DecodeArgs a) {
  constexpr int TPK = D / 16;              // lanes per key row
  constexpr int KPW = 64 / TPK;            // keys per wave per round
  constexpr int KPI = KPW * kRounds;       // keys per wave per iteration
  constexpr int KWG = KPI * kWaves;        // keys per workgroup per iteration
  __shared__ float red_m[kWaves][G];
  __shared__ float red_l[kWaves][G];
  __shared__ float red_o[kWaves][G][D];

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int kg = lane / TPK;               // key within the round
  const int cc = lane % TPK;               // chunk: pairs 8cc .. 8cc+7
  const int64_t b = blockIdx.x / a.Hkv;
  const int hk = (int)(blockIdx.x % a.Hkv);
  const int C = (int)(a.n_sink + a.window);
  const int n_sink = (int)a.n_sink, window = (int)a.window;

  const int len_raw = a.cache_len[b];
  const int rh_raw = a.ring_head ? a.ring_head[b] : 0;
  const bool bad_seq = len_raw < 0 || len_raw > C || rh_raw < 0 || rh_raw >= window;
  const int len = bad_seq ? 0 : len_raw;
  const int rh = bad_seq ? 0 : rh_raw;

  // Rotated query (fp32) for each of the G heads: pairs 8cc..8cc+7.
  float qlo[G][8], qhi[G][8];
  {
    const int qpos = len > 0 ? len - 1 : 0;
    const f32x4* t = reinterpret_cast<const f32x4*>(a.cos_sin + (int64_t)qpos * D + 16 * cc);
    float c[8], s[8];
#pragma unroll
    for (int u2 = 0; u2 < 4; ++u2) {
      const f32x4 tt = t[u2];
      c[2 * u2] = tt[0]; s[2 * u2] = tt[1]; c[2 * u2 + 1] = tt[2]; s[2 * u2 + 1] = tt[3];
    }
#pragma unroll
    for (int g = 0; g < G; ++g) {
      const __bf16* qp = reinterpret_cast<const __bf16*>(a.q) + b * a.qs[0] +
                         (int64_t)(hk * G + g) * a.qs[1];
      float x[8], z[8];
      unpack8(*reinterpret_cast<const u32x4*>(qp + 8 * cc), x);
      unpack8(*reinterpret_cast<const u32x4*>(qp + D / 2 + 8 * cc), z);
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        qlo[g][u] = x[u] * c[u] - z[u] * s[u];
        qhi[g][u] = x[u] * s[u] + z[u] * c[u];
      }
    }
  }

  const float scale_log2 = a.softmax_scale * kLog2e;
  float m[G], l[G], o_lo[G][8], o_hi[G][8];
#pragma unroll
  for (int g = 0; g < G; ++g) {
    m[g] = -INFINITY;
    l[g] = 0.f;
#pragma unroll
    for (int u = 0; u < 8; ++u) o_lo[g][u] = o_hi[g][u] = 0.f;
  }

  const __bf16* kb = reinterpret_cast<const __bf16*>(a.k) + b * a.cs[0] + hk * a.cs[1];
  const __bf16* vb = reinterpret_cast<const __bf16*>(a.v) + b * a.cs[0] + hk * a.cs[1];
  const int n_slots = len <= n_sink ? len : C;   // slots worth scanning

  // Issue the K/V loads of the iteration starting at slot `base`.
  auto load = [&](int base, KVChunk& ch) {
#pragma unroll
    for (int r = 0; r < kRounds; ++r) {
      const int slot = base + r * (KPW * kWaves) + wave * KPW + kg;
      int e;
      if (slot < n_sink) {
        e = slot;
      } else {
        int j = (slot - n_sink - rh) % window;
        if (j < 0) j += window;
        e = n_sink + j;
      }
      ch.ok[r] = slot < n_slots && e < len;
      ch.epos[r] = ch.ok[r] ? e : 0;
      const int sc = slot < C ? slot : C - 1;
      const __bf16* kp = kb + (int64_t)sc * a.cs[2];
      const __bf16* vp = vb + (int64_t)sc * a.cs[2];
      ch.klo[r] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(kp + 8 * cc));
      ch.khi[r] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(kp + D / 2 + 8 * cc));
      ch.vlo[r] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(vp + 8 * cc));
      ch.vhi[r] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(vp + D / 2 + 8 * cc));
    }
  };

  // Fold one iteration's keys into (m, l, o).
  auto fold = [&](const KVChunk& ch) {
    float sc_[G][kRounds];
#pragma unroll
    for (int r = 0; r < kRounds; ++r) {
      const f32x4* t = reinterpret_cast<const f32x4*>(a.cos_sin + (int64_t)ch.epos[r] * D + 16 * cc);
      float c[8], s[8], x[8], z[8];
#pragma unroll
      for (int u2 = 0; u2 < 4; ++u2) {
        const f32x4 tt = t[u2];
        c[2 * u2] = tt[0]; s[2 * u2] = tt[1]; c[2 * u2 + 1] = tt[2]; s[2 * u2 + 1] = tt[3];
      }
      unpack8(ch.klo[r], x);
      unpack8(ch.khi[r], z);
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
        const float p = fast_exp2(sc_[g][r] - mn);
        l[g] += p;
        float v1[8], v2[8];
        unpack8(ch.vlo[r], v1);
        unpack8(ch.vhi[r], v2);
#pragma unroll
        for (int u = 0; u < 8; ++u) {
          o_lo[g][u] = __builtin_fmaf(p, ch.ok[r] ? v1[u] : 0.f, o_lo[g][u]);
          o_hi[g][u] = __builtin_fmaf(p, ch.ok[r] ? v2[u] : 0.f, o_hi[g][u]);
        }
      }
    }
  };

#if YRB_DECODE_PREFETCH
  KVChunk c0, c1;
  if (n_slots > 0) load(0, c0);
  for (int base = 0; base < n_slots; base += 2 * KWG) {
    if (base + KWG < n_slots) load(base + KWG, c1);
    fold(c0);
    if (base + KWG >= n_slots) break;
    if (base + 2 * KWG < n_slots) load(base + 2 * KWG, c0);
    fold(c1);
  }
#else
  for (int base = 0; base < n_slots; base += KWG) {
    KVChunk c0;
    load(base, c0);
    fold(c0);
  }
#endif

  // Reduce across the key groups of the wave (lanes with equal cc).
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
    if (kg == 0) {
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        red_o[wave][g][8 * cc + u] = o_lo[g][u];
        red_o[wave][g][D / 2 + 8 * cc + u] = o_hi[g][u];
      }
      if (cc == 0) {
        red_m[wave][g] = m[g];
        red_l[wave][g] = l[g];
      }
    }
  }
  __syncthreads();
  // Merge the waves: thread t handles (g, d) pairs.
  for (int idx = threadIdx.x; idx < G * D; idx += kWaves * 64) {
    const int g = idx / D, d = idx % D;
    float mm = -INFINITY;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) mm = fmaxf(mm, red_m[w][g]);
    float lt = 0.f, ot = 0.f;
    if (mm != -INFINITY) {
#pragma unroll
      for (int w = 0; w < kWaves; ++w) {
        const float sw = red_m[w][g] == -INFINITY ? 0.f : fast_exp2(red_m[w][g] - mm);
        lt += sw * red_l[w][g];
        ot += sw * red_o[w][g][d];
      }
    }
    float res = lt > 0.f ? ot / lt : 0.f;
    if (bad_seq) res = __builtin_nanf("");
    __bf16* op = reinterpret_cast<__bf16*>(a.o) + b * a.os[0] + (int64_t)(hk * G + g) * a.os[1];
    op[d] = (__bf16)res;
  }
}

template <int D, int G>
hipError_t launch_dec(const DecodeArgs& a, hipStream_t stream) {
  const int64_t blocks = a.B * a.Hkv;
  if (blocks == 0) return hipSuccess;
  hipLaunchKernelGGL((decode_bf16_kernel<D, G>), dim3((unsigned)blocks), dim3(kWaves * 64), 0,
                     stream, a);
  return hipGetLastError();
}

template <int D>
hipError_t launch_dec_g(const DecodeArgs& a, hipStream_t stream) {
  switch (a.Hq / a.Hkv) {
    case 1: return launch_dec<D, 1>(a, stream);
    case 2: return launch_dec<D, 2>(a, stream);
    case 4: return launch_dec<D, 4>(a, stream);
    case 8: return launch_dec<D, 8>(a, stream);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace

hipError_t launch_decode(int dtype, int D, const DecodeArgs& a, hipStream_t stream) {
  if (dtype != kBF16) return hipErrorInvalidValue;
  return D == 64 ? launch_dec_g<64>(a, stream) : launch_dec_g<128>(a, stream);
}

}  // namespace yrb
