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
// once, about one flop per byte), so the kernel is a streaming reduction
// whose waves run independently.
//  * A wave owns one (sequence, key/value head) and a range of its cache
//    entries, walked by position in steps of 32 (entry e = A + j, A a
//    multiple of 32, j < 32), each step a few rounds of D/16-lane keys.  A
//    head's entries may be split over `parts` waves of one workgroup (the
//    host picks parts so that caches with few key/value heads still fill
//    the chip); the parts' (max, sum, output) merge through LDS at the end.
//  * D/16 lanes share one key and each holds 8 complete pairs, so the
//    rotation is lane-local: with a bf16 cache a lane reads the two chunks
//    holding pairs (i, i + d/2) (or, interleaved, adjacent pairs from the
//    same two chunks); an fp8 cache is read as below.  Loads are
//    non-temporal (the cache is far larger than L2 and MALL) and pipelined
//    by round: a ring of register sets keeps a step's worth of rounds in
//    flight, each set reloaded as soon as its round is folded.
//  * Rotation by angle addition: with e = 1024 a + 32 b + j,
//    R(e) = R(1024 a) R(32 b) R(j).  The 32 rows R(j) and the 32 rows
//    R(32 b) sit in LDS for the whole launch (read from the caller's table,
//    XOR-swizzled so that the lanes of a read hit distinct banks); R(1024 a)
//    comes from the table in global memory once every 32 steps.  With one
//    or two query heads per key head each step re-anchors the query
//    instead, q'.k' = (R(32 b)^T R(1024 a)^T q') . (R(j) k); with more, it
//    forms R(e) per key, once for all the key's heads.  Reading a table row
//    per key and head would move as many bytes as K and V together.
//  * An fp8 (E4M3) cache row is d bytes: each lane reads a 16-byte chunk
//    of it, so one load instruction covers whole rows (HBM serves
//    half-lines markedly slower), and for the half-split layout the lanes
//    of a key trade halves of their chunks so that each holds 8 complete
//    pairs.
//  * A lane addresses its head's cache with a 32-bit offset (one 24-bit
//    multiply) from a wave-uniform base; the host bounds the span.
//  * With 8 query heads per key head (bf16 cache, half-split pairs) the
//    logits of a round's keys come from MFMAs instead: the lanes write
//    their keys' rotated rows (bf16) into an LDS tile, one chain of
//    v_mfma_f32_16x16x32_bf16 multiplies it by the 8 heads' queries, and
//    the softmax keeps one reference per head for the whole wave; P returns
//    to the value lanes through LDS and PV stays on the VALU.  That path
//    reads each key's R(e) from the caller's table (L2-resident: the rows
//    are the same for every sequence and head) rather than composing it.
//  * Online softmax in the exp2 domain, the logit scale folded into the
//    query.  The running max is kept per key group (the lanes that share a
//    key agree on it), and a group moves its reference only when a key
//    beats it by more than 8: the same result in exact arithmetic, P <= 2^8,
//    and no cross-lane max per round.  The groups merge at the end with
//    DPP row rotations and the permlane swaps, which also do the per-key
//    sums; none of these goes through the LDS crossbar.
#include "common.h"
#include "kernels.h"

namespace yrb {

namespace {

constexpr int kWaves = 4;        // waves per workgroup
constexpr int kKPS = 32;         // cache positions per step
constexpr float kDecTau = 8.0f;  // lazy-rescale threshold (log2 units)

// Cache element: bf16 (a 16-byte chunk holds 8 values) or fp8 E4M3 (OCP; 8
// codes decode from one 8-byte half of a lane's 16-byte chunk).
template <bool FP8>
struct CacheType {
  using Chunk = u32x4;
  using Elem = __bf16;
  __device__ static void unpack(const Chunk& w, float (&f)[8]) { unpack8(w, f); }
};
template <>
struct CacheType<true> {
  using Chunk = u32x2;
  using Elem = uint8_t;
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

template <int D, int G, bool FP8 = false>
struct DecCfg {
  static constexpr int TPK = D / 16;                 // lanes per key (8 pairs each)
  static constexpr int KPW = 64 / TPK;               // keys per round
  static constexpr int ROUNDS = kKPS / KPW;          // rounds per step of 32 positions
  static constexpr int RPG = 16 / TPK;               // key rows per 16 lanes of an LDS read
  static constexpr int LOG_RPG = RPG == 2 ? 1 : 2;
  static constexpr int TROWB = 4 * D;                // bytes of an fp32 table row (d/2 pairs of (cos, sin))
  // LDS table: rows R(j) and R(32 j) (j < 32), then one row per wave for its
  // R(1024 a).
  static constexpr bool ANCHOR_Q = G <= 2;           // re-anchor the query, else compose R(e) per key
  static constexpr int ROW_32 = kKPS;                // row of R(32 j): ROW_32 + j
  static constexpr int ROW_W = ROW_32 + kKPS;        // row of wave w's R(1024 a): ROW_W + w
  static constexpr int TAB_BYTES = (ROW_W + kWaves) * TROWB;
  // Rounds of K/V loads in flight (register sets of the ring): a step's
  // worth, half of one when the per-head query and output registers leave
  // less room.
  static constexpr int PD = G <= 2 ? ROUNDS : (ROUNDS > 1 ? ROUNDS / 2 : 1);
  // Waves per SIMD the registers are sized for: an fp8 cache with one query
  // head per key head fits four (its key and value chunks are half the
  // size), whose latency hiding it needs: it has twice the arithmetic per
  // byte of a bf16 cache.
  static constexpr int WAVES_PER_EU = (FP8 && G == 1) ? 4 : G <= 4 ? 2 : 1;
  // Waves a launch aims at (the host splits heads into parts until it has
  // them): every SIMD's share at that occupancy, at least two per SIMD.
  static constexpr int64_t TARGET_WAVES = 1024 * (WAVES_PER_EU > 2 ? WAVES_PER_EU : 2);
  static_assert(ROUNDS * KPW == kKPS, "a step is whole rounds");
  static_assert(ROUNDS % PD == 0 || PD % ROUNDS == 0, "ring sets repeat within U steps");
  static constexpr int U = PD > ROUNDS ? PD / ROUNDS : 1;   // steps per pass of the loop
};

// Cross-lane reductions without the LDS crossbar (ds_bpermute, which a
// __shfl_xor becomes, costs an LDS round trip per step): DPP within rows of
// 16 lanes, and the gfx950 permlane swaps across rows and half-waves.
template <int CTRL>
__device__ __forceinline__ float dpp(float x) {
  return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), CTRL, 0xF, 0xF, false));
}
constexpr int kDppQuadXor1 = 0xB1;      // quad_perm [1, 0, 3, 2]
constexpr int kDppQuadXor2 = 0x4E;      // quad_perm [2, 3, 0, 1]
constexpr int kDppHalfMirror = 0x141;   // lane i <- 7 - i within 8 lanes
constexpr int kDppRowRor4 = 0x124;      // lane i <- (i + 4) mod 16 within a row
constexpr int kDppRowRor8 = 0x128;      // lane i <- (i + 8) mod 16 within a row

// Sum over the N lanes of an aligned group (N = 1, 2, 4 or 8).
template <int N>
__device__ __forceinline__ float group_sum(float x) {
  if constexpr (N >= 2) x += dpp<kDppQuadXor1>(x);
  if constexpr (N >= 4) x += dpp<kDppQuadXor2>(x);
  if constexpr (N >= 8) x += dpp<kDppHalfMirror>(x);   // the quads are uniform by now
  return x;
}
// op (symmetric) of x over the lanes l, l + N, l + 2N, ... (mod 64), i.e.
// over the aligned groups of N lanes (N = 4 or 8), for each position in a
// group: every lane ends with the combination for its position.  Row
// rotations by multiples of N keep the position; the permlane swaps pair
// lanes 16 and 32 apart.
template <int N, typename Op>
__device__ __forceinline__ float across_groups(float x, Op op) {
  static_assert(N == 4 || N == 8, "groups of 4 or 8 lanes");
  x = op(x, dpp<kDppRowRor8>(x));
  if constexpr (N == 4) x = op(x, dpp<kDppRowRor4>(x));
  {
    const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    x = op(__uint_as_float(r[0]), __uint_as_float(r[1]));
  }
  {
    const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    x = op(__uint_as_float(r[0]), __uint_as_float(r[1]));
  }
  return x;
}
struct MaxOp {
  __device__ float operator()(float a, float b) const { return fmaxf(a, b); }
};
struct AddOp {
  __device__ float operator()(float a, float b) const { return a + b; }
};

// 16-byte chunk k (2 pairs) of LDS table row j sits at chunk k ^ h(j, k):
// within each 16 lanes of a ds_read_b128 (RPG key rows, 16/RPG lanes each,
// every lane at its own chunk) the chunks land on 16 distinct bank groups.
template <int D>
__device__ __forceinline__ int tab_phys(int j, int k) {
  using C = DecCfg<D, 1>;
  return k ^ ((j & (C::RPG - 1)) | (((k >> 4) & 1) << C::LOG_RPG));
}

// Which 8 pairs lane cc (of the D/16 lanes that share a key) holds, and
// where its query and output chunks (8 elements each) sit.
//  * bf16 cache: the lane reads two 16-byte chunks per key, at elements 8cc
//    and d/2 + 8cc: half-split, pairs 8cc .. 8cc+7; interleaved, pairs
//    4cc .. 4cc+3 and d/4 + 4cc .. +3.  Each load instruction covers whole
//    128-byte halves of the key rows.
//  * fp8 cache: a row of codes is d bytes, so chunks at 8cc and d/2 + 8cc
//    would be 8 bytes each and a load instruction would cover half-lines,
//    which HBM serves markedly slower (a streaming probe of this cache
//    shape: 5.75-5.97 TB/s for half-lines against 6.75-6.94 for whole
//    rows).  So the lane reads the 16-byte chunk cc of the row: interleaved,
//    pairs 8cc .. 8cc+7 complete; half-split, the first TPK/2 lanes hold
//    first elements and the others their partners, in mirror order (lane
//    TPK-1-c holds the partners of lane c's), and the two trade halves so
//    that lane c takes pairs 16c .. 16c+7 and lane TPK-1-c pairs
//    16c+8 .. 16c+15.  Outputs: elements 16cc .. 16cc+15.
template <int D, bool FP8, bool IL>
struct LaneMap {
  static constexpr int TPK = D / 16;
  // pair index of the lane's u-th pair (u < 8)
  __device__ static int pair(int cc, int u) {
    if constexpr (!FP8) {
      if constexpr (!IL) return 8 * cc + u;
      return u < 4 ? 4 * cc + u : D / 4 + 4 * cc + (u - 4);
    } else {
      if constexpr (IL) return 8 * cc + u;
      return cc < TPK / 2 ? 16 * cc + u : 16 * (TPK - 1 - cc) + 8 + u;
    }
  }
  // 16-byte table chunk (2 pairs) of the lane's pairs 2w, 2w+1
  __device__ static int tchunk(int cc, int w) { return pair(cc, 2 * w) / 2; }
  // the lane's two query chunks (elements), read as pairs_of<IL> takes them
  __device__ static int q_a(int cc) { return FP8 ? (IL ? 16 * cc : pair(cc, 0)) : 8 * cc; }
  __device__ static int q_b(int cc) { return FP8 ? (IL ? 16 * cc + 8 : D / 2 + pair(cc, 0)) : D / 2 + 8 * cc; }
  // the elements of o_lo and o_hi (8 each)
  __device__ static int o_a(int cc) { return FP8 ? 16 * cc : 8 * cc; }
  __device__ static int o_b(int cc) { return FP8 ? 16 * cc + 8 : D / 2 + 8 * cc; }
};

// The 8 pairs of one lane from its two query chunks a, b (8 values each):
// half-split, a the first elements and b their partners; interleaved, a
// holds pairs 0..3 of the lane and b pairs 4..7, each pair two adjacent
// values.
template <bool IL>
__device__ __forceinline__ void pairs_of(const float (&a)[8], const float (&b)[8], float (&x)[8],
                                         float (&z)[8]) {
#pragma unroll
  for (int u = 0; u < 8; ++u) {
    if constexpr (IL) {
      x[u] = u < 4 ? a[2 * u] : b[2 * u - 8];
      z[u] = u < 4 ? a[2 * u + 1] : b[2 * u - 7];
    } else {
      x[u] = a[u];
      z[u] = b[u];
    }
  }
}

// (cos, sin) of the lane's 8 pairs: from a table row in global memory, or
// from LDS row j (swizzled).
template <class LM>
__device__ __forceinline__ void row_pairs(const float* row, int cc, float (&c)[8], float (&s)[8]) {
#pragma unroll
  for (int w = 0; w < 4; ++w) {
    const f32x4 t = *reinterpret_cast<const f32x4*>(row + 4 * LM::tchunk(cc, w));
    c[2 * w] = t[0];
    s[2 * w] = t[1];
    c[2 * w + 1] = t[2];
    s[2 * w + 1] = t[3];
  }
}
template <int D, class LM>
__device__ __forceinline__ void lds_pairs(const YRB_LDS char* tab, int j, int cc, float (&c)[8], float (&s)[8]) {
  const YRB_LDS char* row = tab + j * DecCfg<D, 1>::TROWB;
#pragma unroll
  for (int w = 0; w < 4; ++w) {
    const f32x4 t = *reinterpret_cast<const YRB_LDS f32x4*>(row + 16 * tab_phys<D>(j, LM::tchunk(cc, w)));
    c[2 * w] = t[0];
    s[2 * w] = t[1];
    c[2 * w + 1] = t[2];
    s[2 * w + 1] = t[3];
  }
}

// Pair rotations: by the angle (c, s), by its negative (the transpose), and
// the sum of two angles.
__device__ __forceinline__ void rot(float& x, float& z, float c, float s) {
  const float x0 = x;
  x = x0 * c - z * s;
  z = x0 * s + z * c;
}
__device__ __forceinline__ void rot_t(float& x, float& z, float c, float s) {
  const float x0 = x;
  x = x0 * c + z * s;
  z = z * c - x0 * s;
}
__device__ __forceinline__ void add_angle(float& c, float& s, float c2, float s2) {
  const float c0 = c;
  c = c0 * c2 - s * s2;
  s = s * c2 + c0 * s2;
}

// K/V chunks of one round for one lane, and whether its key counts: bf16,
// the two chunks of K and of V; fp8, one 16-byte chunk of each row.
template <bool FP8>
struct KVRound {
  u32x4 klo, khi, vlo, vhi;
  bool ok;
};
template <>
struct KVRound<true> {
  u32x4 k, v;
  bool ok;
};

// Mirror within the lanes of a key (lane c <-> TPK-1-c): row_half_mirror for
// 8 lanes, quad_perm [3, 2, 1, 0] for 4.
template <int TPK>
__device__ __forceinline__ unsigned key_mirror(unsigned x) {
  return (unsigned)__builtin_amdgcn_update_dpp(0, (int)x, TPK == 8 ? kDppHalfMirror : 0x1B, 0xF, 0xF, false);
}

template <int D, int G, bool FP8, bool IL>
__global__ __launch_bounds__(kWaves * 64) __attribute__((amdgpu_waves_per_eu(DecCfg<D, G, FP8>::WAVES_PER_EU)))
void decode_kernel(DecodeArgs a, int parts) {
  using CT = CacheType<FP8>;
  using Elem = typename CT::Elem;
  using Cfg = DecCfg<D, G, FP8>;
  constexpr int TPK = Cfg::TPK, KPW = Cfg::KPW, ROUNDS = Cfg::ROUNDS, PD = Cfg::PD;
  constexpr int MERGE_F = G * (D + 2);               // floats a wave leaves for the merge
  constexpr int U = Cfg::U;
  constexpr bool AQ = Cfg::ANCHOR_Q;
  // bf16 cache, half-split pairs, 8 query heads per key head: the logits of
  // a round's keys against all the heads come from one MFMA chain over the
  // rotated keys (bf16, through a per-wave LDS tile) instead of per-lane dot
  // products and cross-lane sums.  (At 4 heads the chain's latency, one round
  // at a time, costs more than the dot products it replaces.)
  constexpr bool MF = !FP8 && !IL && G >= 8;
  // MF: each key's R(e) is read from the caller's table (the rows of the
  // cache positions are the same for every sequence and head, so they stay
  // in L2) instead of composed from LDS rows.  This path is heavy on LDS
  // (the key tile, P), and without the composition it also holds no spill.
  // (The dot-product path measured slower with it: 0.181 -> 0.214 ms for
  // 32 query / 8 key heads; the 4 extra loads per round cost more than the
  // 40 VALU instructions they save.)
  constexpr bool TROW = MF;
  constexpr int KROWB = 2 * D + 16;                  // bytes of a key row in that tile (padded)
  using KV = KVRound<FP8>;
  using LM = LaneMap<D, FP8, IL>;

  __shared__ __attribute__((aligned(16))) char tab_raw[Cfg::TAB_BYTES];
  __shared__ __attribute__((aligned(16))) float merge[kWaves][MERGE_F];
  // AQ: each wave's query rotated to R(1024 a) (a the current 1024-entry
  // block), per head and lane chunk: the step reads it rather than hold it
  // in registers.
  __shared__ __attribute__((aligned(16))) float qrow[kWaves][AQ ? G * D : 1];
  // MF: the round's rotated keys, one bf16 row per key (the rows past the
  // round's keys are never written and their logits never used), and the
  // round's P by (key, head).
  __shared__ __attribute__((aligned(16))) char ktile_raw[kWaves][MF ? 16 * KROWB : 16];
  __shared__ __attribute__((aligned(16))) float ptile[kWaves][MF ? 16 * 16 : 4];
  YRB_LDS char* const tab = (YRB_LDS char*)tab_raw;

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int kg = lane / TPK;               // key within the round
  const int cc = lane % TPK;               // chunk: pairs 8cc .. 8cc+7
  const int heads_per_wg = kWaves / parts;
  const int n_groups = (int)((a.Hkv + heads_per_wg - 1) / heads_per_wg);
  const int64_t b = blockIdx.x / n_groups;
  const int hk_raw = (int)(blockIdx.x % n_groups) * heads_per_wg + wave / parts;
  const int part = wave % parts;
  const bool head_live = hk_raw < a.Hkv;
  const int hk = head_live ? hk_raw : (int)a.Hkv - 1;   // idle waves read a valid head
  const int C = (int)(a.n_sink + a.window);
  const int n_sink = (int)a.n_sink, window = (int)a.window;

  const int len_raw = a.cache_len[b];
  const int rh_raw = a.ring_head ? a.ring_head[b] : 0;
  const bool bad_seq = len_raw < 0 || len_raw > C || rh_raw < 0 || rh_raw >= window;
  const int len = bad_seq ? 0 : len_raw;
  const int rh = bad_seq ? 0 : rh_raw;

  // R(j) and R(32 j), j < 32, into LDS (rows past the cache are never used:
  // clamped).
  for (int idx = threadIdx.x; idx < (TROW ? 0 : Cfg::ROW_W * (D / 4)); idx += kWaves * 64) {
    const int row = idx / (D / 4), k = idx % (D / 4);
    const int pos = row < Cfg::ROW_32 ? row : kKPS * (row - Cfg::ROW_32);
    const f32x4 t = *reinterpret_cast<const f32x4*>(a.cos_sin + (int64_t)min(pos, C - 1) * D + 4 * k);
    *reinterpret_cast<YRB_LDS f32x4*>(tab + row * Cfg::TROWB + 16 * tab_phys<D>(row, k)) = t;
  }

  // This wave's steps: the head's ceil(len / 32) steps split over the parts.
  const int n_steps = (len + kKPS - 1) / kKPS;
  const int per_part = (n_steps + parts - 1) / parts;
  const int s_begin = head_live ? min(n_steps, part * per_part) : 0;
  const int s_end = head_live ? min(n_steps, s_begin + per_part) : 0;

  // fp8: per (sequence, kv head) dequantisation scales; K's folds into the
  // logit scale, V's into the final normalisation.
  const float k_deq = (FP8 && a.k_scale) ? a.k_scale[b * a.Hkv + hk] : 1.0f;
  const float v_deq = (FP8 && a.v_scale) ? a.v_scale[b * a.Hkv + hk] : 1.0f;
  const float scale_log2 = a.softmax_scale * kLog2e * k_deq;

  const __bf16* qhead = reinterpret_cast<const __bf16*>(a.q) + b * a.qs[0] + (int64_t)(hk * G) * a.qs[1];
  auto load_q = [&](int g, float (&x)[8], float (&z)[8]) {
    const __bf16* qp = qhead + (int64_t)g * a.qs[1];
    float qa[8], qb[8];
    unpack8(*reinterpret_cast<const u32x4*>(qp + LM::q_a(cc)), qa);
    unpack8(*reinterpret_cast<const u32x4*>(qp + LM::q_b(cc)), qb);
    pairs_of<IL>(qa, qb, x, z);
  };

  // Query of head g rotated at position `pos` and multiplied by the logit
  // scale (log2 units), as fp32 pairs.
  auto query_at = [&](int g, int pos, float (&x)[8], float (&z)[8]) {
    float c[8], s[8];
    row_pairs<LM>(a.cos_sin + (int64_t)pos * D, cc, c, s);
    load_q(g, x, z);
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      rot(x[u], z[u], c[u], s[u]);
      x[u] *= scale_log2;
      z[u] *= scale_log2;
    }
  };
  // Compose mode: the query at len - 1, held for the whole launch.
  float qx[(AQ || MF) ? 1 : G][8], qz[(AQ || MF) ? 1 : G][8];
  if constexpr (!AQ && !MF) {
#pragma unroll
    for (int g = 0; g < G; ++g) query_at(g, len > 0 ? len - 1 : 0, qx[g], qz[g]);
  }
  // MF: the query of head lane % 16 (zero past G) rotated at len - 1 and
  // scaled, as the B operand of v_mfma_f32_16x16x32_bf16: for k-step ks the
  // lane holds dimensions 32 ks + 8 (lane / 16) .. + 7.
  bf16x8 qb[MF ? D / 32 : 1];
  if constexpr (MF) {
    const int n = lane & 15;
    const int pos = len > 0 ? len - 1 : 0;
#pragma unroll
    for (int ks = 0; ks < D / 32; ++ks) {
      float f[8];
#pragma unroll
      for (int u = 0; u < 8; ++u) f[u] = 0.f;
      if (n < G) {
        const int d0 = 32 * ks + 8 * (lane >> 4);
        const bool first = d0 < D / 2;
        const int p0 = first ? d0 : d0 - D / 2;      // the 8 pairs p0 .. p0+7
        const __bf16* qp = qhead + (int64_t)n * a.qs[1];
        float xa[8], xb[8];
        unpack8(*reinterpret_cast<const u32x4*>(qp + p0), xa);
        unpack8(*reinterpret_cast<const u32x4*>(qp + D / 2 + p0), xb);
        const float* row = a.cos_sin + (int64_t)pos * D + 2 * p0;
#pragma unroll
        for (int w = 0; w < 4; ++w) {
          const f32x4 t = *reinterpret_cast<const f32x4*>(row + 4 * w);
#pragma unroll
          for (int h = 0; h < 2; ++h) {
            const int u = 2 * w + h;
            float x = xa[u], z = xb[u];
            rot(x, z, t[2 * h], t[2 * h + 1]);
            f[u] = (first ? x : z) * scale_log2;
          }
        }
      }
      qb[ks] = __builtin_bit_cast(bf16x8, pack8(f));
    }
  }

  // Running max, sum and output per head.  The max is kept per key group
  // (the TPK lanes that share a key hold the same one) and the groups merge
  // at the end, so no round needs a cross-lane max.
  float m[G], l[G], o_lo[G][8], o_hi[G][8];
#pragma unroll
  for (int g = 0; g < G; ++g) {
    m[g] = -INFINITY;
    l[g] = 0.f;
#pragma unroll
    for (int u = 0; u < 8; ++u) o_lo[g][u] = o_hi[g][u] = 0.f;
  }

  // The head's cache in bytes from a wave-uniform base; within it a lane's
  // chunk sits at a 32-bit offset (the host keeps an entry index and the
  // entry stride below 2^24 bytes, and their product below 2^32).
  const int64_t head_off = (b * a.cs[0] + hk * a.cs[1]) * (int64_t)sizeof(Elem);
  const uint8_t* kbase = reinterpret_cast<const uint8_t*>(a.k) + head_off;
  const uint8_t* vbase = reinterpret_cast<const uint8_t*>(a.v) + head_off;
  const unsigned row_bytes = (unsigned)(a.cs[2] * (int64_t)sizeof(Elem));
  // bf16: chunks at elements 8cc and d/2 + 8cc (16 bytes each); fp8: K's
  // chunk of the row (mirror order for the partners, half-split), V's chunk cc
  const unsigned lane_off = 16u * cc;
  const unsigned k_off = (FP8 && !IL && cc >= TPK / 2) ? D / 2 + 16u * (TPK - 1 - cc) : lane_off;
  constexpr unsigned HALF_OFF = D / 2 * sizeof(Elem);
  const int ring_shift = rh - n_sink;

  // Round t covers positions t KPW .. t KPW + KPW - 1; this lane's key is
  // entry e = t KPW + kg, in its slot: sinks first, then the ring buffer
  // (past the sinks, e - n_sink + ring_head lies in [0, 2 window), and the
  // unsigned min of it and of it less window is its value mod window).
  auto load_round = [&](int t, KV& kv) {
    const int e = t * KPW + kg;
    kv.ok = e < len;
    const int d = e + ring_shift;
    const unsigned dw = min((unsigned)d, (unsigned)(d - window));
    const int slot = !kv.ok ? 0 : e < n_sink ? e : n_sink + (int)dw;
    const unsigned off = __umul24((unsigned)slot, row_bytes);
    const unsigned vo = off + lane_off;
    if constexpr (FP8) {
      kv.k = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(kbase + (off + k_off)));
      kv.v = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(vbase + vo));
    } else {
      kv.klo = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(kbase + vo));
      kv.khi = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(kbase + vo + HALF_OFF));
      kv.vlo = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(vbase + vo));
      kv.vhi = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(vbase + vo + HALF_OFF));
    }
  };

  __syncthreads();   // the tables are in LDS

  if (s_begin < s_end) {
    const int t_begin = s_begin * ROUNDS, t_end = s_end * ROUNDS;
    KV ring[PD];
#pragma unroll
    for (int i = 0; i < PD; ++i)
      if (t_begin + i < t_end) load_round(t_begin + i, ring[i]);

    // Entry e = 1024 a2 + 32 b1 + j: R(e) = R(1024 a2) R(32 b1) R(j).  The
    // row of R(1024 a2) changes every 32 steps: it comes from global memory
    // into the wave's LDS row (the lanes of key group 0 writing it).
    int a_cur = -1;
    float rc[8], rs[8];              // compose: R(1024 a2 + 32 b1)
    // TROW: (cos, sin) of the lane's pairs at the key position of the next
    // round, loaded one round ahead from the caller's table (the same rows
    // for every sequence and head, so they stay in L2).
    // Two sets, by the parity of the round (a step is an even number of
    // rounds), so that no copy is needed.
    float tc[2][8], ts[2][8];
    auto load_trow = [&](int t, int set) {
      const int e = min(t * KPW + kg, C - 1);
      row_pairs<LM>(a.cos_sin + (int64_t)e * D, cc, tc[set], ts[set]);
    };
    static_assert(ROUNDS % 2 == 0, "rounds alternate the table sets");
    if constexpr (TROW) load_trow(t_begin, 0);

    // MASK: the step reaches past the last entry (its missing keys are
    // masked); the other steps skip the test.
    // U: the step's place in a pass of U steps, which picks the ring sets.
    auto step = [&](int s, auto u_tag, auto mask_tag) YRB_INLINE {
      constexpr int u = decltype(u_tag)::value;
      constexpr bool MASK = decltype(mask_tag)::value;
      const int A = s * kKPS;
      const int a2 = A >> 10, b1 = (A >> 5) & 31;
      const int jw = Cfg::ROW_W + wave;
      if (!TROW && a2 != a_cur) {
        // AQ: R(1024 a2)^T R(len - 1) q = R(len - 1 - 1024 a2) q, into the
        // wave's query rows; compose: R(1024 a2) into its table row.
        if constexpr (AQ) {
#pragma unroll
          for (int g = 0; g < G; ++g) {
            float x[8], z[8];
            query_at(g, len - 1 - (a2 << 10), x, z);
            if (kg == 0) {
              float* qr = &qrow[wave][(g * TPK + cc) * 16];
#pragma unroll
              for (int w = 0; w < 8; ++w) {
                qr[w] = x[w];
                qr[8 + w] = z[w];
              }
            }
          }
        } else {
          float c2[8], s2[8];
          row_pairs<LM>(a.cos_sin + (int64_t)(a2 << 10) * D, cc, c2, s2);
          if (kg == 0) {
            YRB_LDS char* row = tab + jw * Cfg::TROWB;
#pragma unroll
            for (int w = 0; w < 4; ++w) {
              const f32x4 t = {c2[2 * w], s2[2 * w], c2[2 * w + 1], s2[2 * w + 1]};
              *reinterpret_cast<YRB_LDS f32x4*>(row + 16 * tab_phys<D>(jw, LM::tchunk(cc, w))) = t;
            }
          }
        }
        a_cur = a2;
        // the lanes of key group 0 wrote what every lane reads next: keep
        // the compiler from moving those reads above the writes (a wave's
        // LDS accesses complete in order)
        __builtin_amdgcn_wave_barrier();
      }
      float c1[8], s1[8];
      if constexpr (!TROW) lds_pairs<D, LM>(tab, Cfg::ROW_32 + b1, cc, c1, s1);
      float qx_s[AQ ? G : 1][8], qz_s[AQ ? G : 1][8];   // AQ: the query this step's keys meet
      if constexpr (AQ) {
#pragma unroll
        for (int g = 0; g < G; ++g) {
          const float* qr = &qrow[wave][(g * TPK + cc) * 16];
#pragma unroll
          for (int w = 0; w < 8; ++w) {
            qx_s[g][w] = qr[w];
            qz_s[g][w] = qr[8 + w];
            rot_t(qx_s[g][w], qz_s[g][w], c1[w], s1[w]);
          }
        }
      } else if constexpr (!TROW) {
        float c2[8], s2[8];
        lds_pairs<D, LM>(tab, jw, cc, c2, s2);
#pragma unroll
        for (int w = 0; w < 8; ++w) {
          rc[w] = c2[w];
          rs[w] = s2[w];
          add_angle(rc[w], rs[w], c1[w], s1[w]);
        }
      }
#pragma unroll
      for (int r = 0; r < ROUNDS; ++r) {
        KV& kv = ring[(u * ROUNDS + r) % PD];
        const int t = s * ROUNDS + r;
        const int j = r * KPW + kg;
        // fp8: the lane's 8 pairs of codes.  Interleaved, its chunk as it
        // came; half-split, the first-element lanes keep their chunk's first
        // 8 codes and trade the last 8 for their mirror lane's first 8
        // partners, which keeps its last 8.
        u32x2 klo8, khi8;
        if constexpr (FP8) {
          if constexpr (IL) {
            klo8 = u32x2{kv.k[0], kv.k[1]};
            khi8 = u32x2{kv.k[2], kv.k[3]};
          } else {
            const bool first = cc < TPK / 2;
            const unsigned r0 = key_mirror<TPK>(first ? kv.k[2] : kv.k[0]);
            const unsigned r1 = key_mirror<TPK>(first ? kv.k[3] : kv.k[1]);
            klo8 = first ? u32x2{kv.k[0], kv.k[1]} : u32x2{r0, r1};
            khi8 = first ? u32x2{r0, r1} : u32x2{kv.k[2], kv.k[3]};
          }
        }
        float c[8], sn[8];
        if constexpr (TROW) {
#pragma unroll
          for (int w = 0; w < 8; ++w) {
            c[w] = tc[r & 1][w];
            sn[w] = ts[r & 1][w];
          }
        } else {
          lds_pairs<D, LM>(tab, j, cc, c, sn);
          if constexpr (!AQ) {
#pragma unroll
            for (int w = 0; w < 8; ++w) add_angle(c[w], sn[w], rc[w], rs[w]);
          }
        }
        float ka[8], kb2[8], x[8], z[8];
        if constexpr (FP8) {
          CT::unpack(klo8, ka);
          CT::unpack(khi8, kb2);
        } else {
          CT::unpack(kv.klo, ka);
          CT::unpack(kv.khi, kb2);
        }
        pairs_of<IL>(ka, kb2, x, z);
#pragma unroll
        for (int w = 0; w < 8; ++w) rot(x[w], z[w], c[w], sn[w]);
        // TROW: the next round's rows go out once this round's are used
        if constexpr (TROW)
          if (t + 1 < t_end) load_trow(t + 1, (r + 1) & 1);
        float p[G];
        if constexpr (MF) {
          // The key's rotated row into the tile; then S = K Q^T for the
          // round's keys (rows) and the heads (columns) by MFMA: the lane
          // holds rows 4 (lane / 16) + i, i < 4, of column lane % 16.
          YRB_LDS char* const kt = (YRB_LDS char*)ktile_raw[wave];
          const int p0 = LM::pair(cc, 0);
          *reinterpret_cast<YRB_LDS u32x4*>(kt + kg * KROWB + 2 * p0) = pack8(x);
          *reinterpret_cast<YRB_LDS u32x4*>(kt + kg * KROWB + D + 2 * p0) = pack8(z);
          f32x4 sacc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
          for (int ks = 0; ks < D / 32; ++ks) {
            const bf16x8 af =
                *reinterpret_cast<const YRB_LDS bf16x8*>(kt + (lane & 15) * KROWB + 64 * ks + 16 * (lane >> 4));
            sacc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(af, qb[ks], sacc, 0, 0, 0);
          }
          const int n = lane & 15;
          float sv[4], mx = -INFINITY;
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const int kr = 4 * (lane >> 4) + i;
            const bool ok = kr < KPW && (!MASK || t * KPW + kr < len);
            sv[i] = ok ? sacc[i] : -INFINITY;
            mx = fmaxf(mx, sv[i]);
          }
          // the round's max for the lane's head (the lanes 16 and 32 apart
          // hold the same head's other keys)
          {
            const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(mx), __float_as_uint(mx), false, false);
            mx = fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
          }
          if constexpr (KPW > 8) {
            const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(mx), __float_as_uint(mx), false, false);
            mx = fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
          }
          // One reference per head for the whole wave (lane g holds head
          // g's max): it moves when the round's max beats it by more than
          // the threshold.
          float ml = m[0];
#pragma unroll
          for (int g = 0; g < G; ++g) {
            const float tm = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(mx), g));
            if (tm > m[g] + kDecTau) {
              const float alpha = fast_exp2(m[g] - tm);   // 0 from the empty state
              m[g] = tm;
              l[g] *= alpha;
#pragma unroll
              for (int w = 0; w < 8; ++w) {
                o_lo[g][w] *= alpha;
                o_hi[g][w] *= alpha;
              }
            }
            ml = n == g ? m[g] : ml;
          }
          float* const pt = ptile[wave];
#pragma unroll
          for (int i = 0; i < 4; ++i)
            pt[(4 * (lane >> 4) + i) * 16 + n] = sv[i] == -INFINITY ? 0.f : fast_exp2(sv[i] - ml);
          // P of the lane's key for every head
#pragma unroll
          for (int g = 0; g < G; ++g) {
            p[g] = pt[kg * 16 + g];
            l[g] += p[g];
          }
        } else {
          // Logit of the lane's key with each head (log2 units), partial
          // over the lane's 8 pairs.
          float acc[G];
#pragma unroll
          for (int g = 0; g < G; ++g) {
            float sum = 0.f;
#pragma unroll
            for (int w = 0; w < 8; ++w) {
              const float qxw = AQ ? qx_s[AQ ? g : 0][w] : qx[AQ ? 0 : g][w];
              const float qzw = AQ ? qz_s[AQ ? g : 0][w] : qz[AQ ? 0 : g][w];
              sum = __builtin_fmaf(qxw, x[w], __builtin_fmaf(qzw, z[w], sum));
            }
            acc[g] = sum;
          }
#pragma unroll
          for (int g = 0; g < G; ++g) {
            float sc = group_sum<TPK>(acc[g]);
            sc = (!MASK || kv.ok) ? sc : -INFINITY;
            // a group's reference moves when its key beats it by more than
            // the threshold: rare once every group has seen a few keys
            const bool grow = sc > m[g] + kDecTau;
            if (__builtin_amdgcn_ballot_w64(grow) != 0) {
              const float alpha = grow ? fast_exp2(m[g] - sc) : 1.0f;   // 0 from the empty state
              m[g] = grow ? sc : m[g];
              l[g] *= alpha;
#pragma unroll
              for (int w = 0; w < 8; ++w) {
                o_lo[g][w] *= alpha;
                o_hi[g][w] *= alpha;
              }
            }
            // 0 for a slot without an entry (whose group may have no reference yet)
            p[g] = (!MASK || kv.ok) ? fast_exp2(sc - m[g]) : 0.f;
            l[g] += p[g];
          }
        }
        // P V (a slot without an entry adds 0: its raw words are zeroed,
        // whatever the cache holds there, NaN codes included)
        float v1[8], v2[8];
        if constexpr (FP8) {
          CT::unpack((!MASK || kv.ok) ? u32x2{kv.v[0], kv.v[1]} : u32x2{}, v1);
          CT::unpack((!MASK || kv.ok) ? u32x2{kv.v[2], kv.v[3]} : u32x2{}, v2);
        } else {
          CT::unpack((!MASK || kv.ok) ? kv.vlo : u32x4{}, v1);
          CT::unpack((!MASK || kv.ok) ? kv.vhi : u32x4{}, v2);
        }
#pragma unroll
        for (int g = 0; g < G; ++g)
#pragma unroll
          for (int w = 0; w < 8; ++w) {
            o_lo[g][w] = __builtin_fmaf(p[g], v1[w], o_lo[g][w]);
            o_hi[g][w] = __builtin_fmaf(p[g], v2[w], o_hi[g][w]);
          }
        // the set is free: the round PD ahead goes out into it
        if (t + PD < t_end) load_round(t + PD, kv);
      }
    };
    // Steps whose 32 entries all exist, then (the sequence's last step, if
    // partial) the masked one, in a loop of its own so that the two bodies
    // do not share registers.
    const int s_full = max(s_begin, min(s_end, len / kKPS));
    for (int s = s_begin; s < s_full; s += U) {
      static_for<U>([&](auto u_tag) YRB_INLINE {
        if (s + decltype(u_tag)::value < s_full) step(s + decltype(u_tag)::value, u_tag, std::false_type{});
      });
    }
    for (int s = s_full; s < s_end; ++s) {
      if constexpr (U == 1) {
        step(s, std::integral_constant<int, 0>{}, std::true_type{});
      } else {
        static_assert(U == 2, "two steps per pass at most");
        if ((s - s_begin) & 1) step(s, std::integral_constant<int, 1>{}, std::true_type{});
        else step(s, std::integral_constant<int, 0>{}, std::true_type{});
      }
    }
  }

  // Merge the key groups of the wave: each group's sums go to the wave's
  // max, then add over the groups (lanes with equal cc).
#pragma unroll
  for (int g = 0; g < G; ++g) {
    const float mw = across_groups<TPK>(m[g], MaxOp{});
    const float sc = m[g] == -INFINITY ? 0.f : fast_exp2(m[g] - mw);   // a group with no key: 0
    m[g] = mw;
    l[g] = across_groups<TPK>(l[g] * sc, AddOp{});
#pragma unroll
    for (int w = 0; w < 8; ++w) {
      o_lo[g][w] *= sc;
      o_hi[g][w] *= sc;
    }
#pragma unroll
    for (int w = 0; w < 8; ++w) {
      o_lo[g][w] = across_groups<TPK>(o_lo[g][w], AddOp{});
      o_hi[g][w] = across_groups<TPK>(o_hi[g][w], AddOp{});
    }
  }

  auto store = [&](int g, float lsum, const float (&lo)[8], const float (&hi)[8]) {
    const float inv = lsum > 0.f ? v_deq / lsum : 0.f;
    float ol[8], oh[8];
#pragma unroll
    for (int w = 0; w < 8; ++w) {
      ol[w] = bad_seq ? __builtin_nanf("") : lo[w] * inv;
      oh[w] = bad_seq ? __builtin_nanf("") : hi[w] * inv;
    }
    __bf16* op = reinterpret_cast<__bf16*>(a.o) + b * a.os[0] + (int64_t)(hk * G + g) * a.os[1];
    *reinterpret_cast<u32x4*>(op + LM::o_a(cc)) = pack8(ol);
    *reinterpret_cast<u32x4*>(op + LM::o_b(cc)) = pack8(oh);
  };

  if (parts == 1) {
    if (head_live && kg == 0)
#pragma unroll
      for (int g = 0; g < G; ++g) store(g, l[g], o_lo[g], o_hi[g]);
    return;
  }

  // Merge the parts of each head: every wave leaves (m, l, o) in LDS, then
  // the wave of part 0 rescales the parts to their common max and adds.
  // merge[wave]: per head, m and l, then o by element (the lane's o_lo and o_hi
  // elements as LaneMap places them).
  if (kg == 0) {
#pragma unroll
    for (int g = 0; g < G; ++g) {
      float* mg = &merge[wave][g * (D + 2)];
      if (cc == 0) {
        mg[0] = m[g];
        mg[1] = l[g];
      }
#pragma unroll
      for (int w = 0; w < 8; ++w) {
        mg[2 + LM::o_a(cc) + w] = o_lo[g][w];
        mg[2 + LM::o_b(cc) + w] = o_hi[g][w];
      }
    }
  }
  __syncthreads();
  if (part != 0 || !head_live || kg != 0) return;
#pragma unroll
  for (int g = 0; g < G; ++g) {
    float mt = -INFINITY;
    for (int p = 0; p < parts; ++p) mt = fmaxf(mt, merge[wave + p][g * (D + 2)]);
    float lsum = 0.f, lo[8], hi[8];
#pragma unroll
    for (int w = 0; w < 8; ++w) lo[w] = hi[w] = 0.f;
    for (int p = 0; p < parts; ++p) {
      const float* mg = &merge[wave + p][g * (D + 2)];
      const float wt = mg[0] == -INFINITY ? 0.f : fast_exp2(mg[0] - mt);
      lsum += wt * mg[1];
#pragma unroll
      for (int w = 0; w < 8; ++w) {
        lo[w] += wt * mg[2 + LM::o_a(cc) + w];
        hi[w] += wt * mg[2 + LM::o_b(cc) + w];
      }
    }
    store(g, lsum, lo, hi);
  }
}


template <int D, int G, bool FP8, bool IL>
hipError_t launch_dec(const DecodeArgs& a, hipStream_t stream) {
  // Waves that split one head's entries: enough (sequence, head, part)
  // units for the occupancy the kernel is built for, at most 4 parts.
  int parts = 1;
  while (parts < kWaves && a.B * a.Hkv * parts < DecCfg<D, G, FP8>::TARGET_WAVES) parts *= 2;
  const int heads_per_wg = kWaves / parts;
  const int64_t blocks = a.B * ((a.Hkv + heads_per_wg - 1) / heads_per_wg);
  if (blocks == 0) return hipSuccess;
  hipLaunchKernelGGL((decode_kernel<D, G, FP8, IL>), dim3((unsigned)blocks), dim3(kWaves * 64), 0, stream, a,
                     parts);
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
