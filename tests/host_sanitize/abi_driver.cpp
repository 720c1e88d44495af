// Host-only driver of the C ABI for the sanitizer build (AddressSanitizer +
// UndefinedBehaviorSanitizer, no recovery): fixed cases with their expected
// status, then a seeded sweep that calls every entry point with argument
// values drawn from the edges of their ranges (negative, zero, one, tile
// edges, 2^31 boundaries, int64 extremes, NULL and misaligned pointers).
// Device pointers are never dereferenced by the layer, so fake addresses
// stand in for them; host arrays (config, factors, strides, outputs) are
// real.  Checks: the documented status of the fixed cases, at most one
// launch per call, and no launch behind an error return.  Exit 0 on
// success; a sanitizer report or a failed check aborts.
#include <cmath>
#include <cstdint>
#include <cstdio>
#include <cstdlib>
#include <limits>

#include "../../include/yrb.h"

extern int g_launches;

namespace {

int failures = 0;
#define EXPECT(c)                                                                   \
  do {                                                                              \
    if (!(c)) {                                                                     \
      std::fprintf(stderr, "driver: %s failed (line %d)\n", #c, __LINE__);          \
      ++failures;                                                                   \
    }                                                                               \
  } while (0)

void* const DEV = reinterpret_cast<void*>(uintptr_t(0x100000));   // aligned fake device address
void* const MIS = reinterpret_cast<void*>(uintptr_t(0x100008));   // misaligned
float* const DEVF = static_cast<float*>(DEV);

// splitmix64
uint64_t rng_state = 0x9E3779B97F4A7C15ull;
uint64_t next() {
  uint64_t z = (rng_state += 0x9E3779B97F4A7C15ull);
  z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
  z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
  return z ^ (z >> 31);
}
template <typename T, size_t N>
T pick(const T (&v)[N]) { return v[next() % N]; }

const int64_t kMax = std::numeric_limits<int64_t>::max();
const int64_t kMin = std::numeric_limits<int64_t>::min();
const int64_t SIZES[] = {-1, 0, 1, 2, 63, 64, 65, 1000, 4100, (int64_t(1) << 30), (int64_t(1) << 31) - 1,
                         int64_t(1) << 31, int64_t(1) << 40, int64_t(1) << 62, kMax, kMin};
const int64_t STRIDES[] = {-8, 0, 8, 64, 128, 4096, (int64_t(1) << 31) - 8, int64_t(1) << 31, kMax, kMin, 12};
const int64_t DIMS[] = {64, 128, 80, 0, -64};
void* const PTRS[] = {DEV, DEV, DEV, nullptr, MIS};
const float SCALES[] = {0.1f, 1.0f, 0.0f, -1.0f, NAN, INFINITY};

// One call: at most one launch, none behind an error.
void account(int before, int rc) {
  const int launched = g_launches - before;
  EXPECT(launched == 0 || launched == 1);
  if (rc != YRB_OK) EXPECT(launched == 0);
  EXPECT(rc == YRB_OK || rc == YRB_EINVAL || rc == YRB_EUNSUPPORTED || rc == YRB_EALIGN || rc == YRB_EHIP);
}

void fixed_cases() {
  yrb_rope_config c = {YRB_ROPE_YARN, 128, 1e4, 4.0, 4096, 1.0, 32.0};
  double th[64], af = 0;
  int b = g_launches;
  EXPECT(rope_tables_build(&c, 0, 0, nullptr, th, &af, nullptr) == YRB_OK && g_launches == b);
  EXPECT(std::fabs(af - std::pow(0.1 * std::log(4.0) + 1.0, 2)) < 1e-15);
  EXPECT(rope_tables_build(&c, 0, 16, DEVF, th, &af, nullptr) == YRB_OK && g_launches == b + 1);
  EXPECT(rope_tables_build(nullptr, 0, 16, DEVF, nullptr, nullptr, nullptr) == YRB_EINVAL);
  c.head_dim = 80;
  EXPECT(rope_tables_build(&c, 0, 16, DEVF, nullptr, nullptr, nullptr) == YRB_EUNSUPPORTED);
  c.head_dim = 128;
  c.scale = NAN;
  EXPECT(rope_tables_build(&c, 0, 16, DEVF, nullptr, nullptr, nullptr) == YRB_EINVAL);
  c.scale = 4.0;
  c.alpha = 40.0;
  EXPECT(rope_tables_build(&c, 0, 16, DEVF, nullptr, nullptr, nullptr) == YRB_EINVAL);
  double f[64];
  for (double& x : f) x = 2.0;
  EXPECT(rope_tables_build_factors(128, 1e4, f, 0, 8, DEVF, th, nullptr) == YRB_OK);
  f[5] = -1.0;
  EXPECT(rope_tables_build_factors(128, 1e4, f, 0, 8, DEVF, th, nullptr) == YRB_EINVAL);
  const int64_t s3[3] = {64 * 4 * 128, 4 * 128, 128};
  EXPECT(rope_apply(DEV, DEV, YRB_BF16, 1, 64, 4, 128, s3, s3, DEVF, 64, 0, nullptr, nullptr) == YRB_OK);
  EXPECT(rope_apply(DEV, DEV, YRB_BF16, 1, 64, 4, 128, s3, s3, DEVF, 63, 0, nullptr, nullptr) == YRB_EINVAL);
  const int64_t s43[4][3] = {{64 * 4 * 128, 4 * 128, 128}, {64 * 2 * 128, 2 * 128, 128},
                             {64 * 2 * 128, 2 * 128, 128}, {64 * 4 * 128, 4 * 128, 128}};
  EXPECT(attn_prefill_blockwise(DEV, DEV, DEV, DEV, YRB_BF16, 1, 64, 4, 2, 128, s43, DEVF, 64, 0.1f, 1, nullptr,
                                nullptr, nullptr) == YRB_OK);
  EXPECT(attn_prefill_blockwise(DEV, DEV, DEV, DEV, YRB_BF16, 1, 64, 4, 2, 128, s43, DEVF, 64, 0.1f, 1, nullptr,
                                MIS, nullptr) == YRB_EALIGN);
  EXPECT(attn_prefill_sink_window(DEV, DEV, DEV, DEV, YRB_BF16, 1, 64, 4, 2, 128, s43, DEVF, 64, 0.1f, kMax, kMax,
                                  nullptr, nullptr, nullptr) == YRB_OK);
  EXPECT(attn_prefill_sink_window_chunk(DEV, DEV, DEV, DEV, YRB_BF16, 1, 64, 128, 4, 2, 128, s43, 64, DEVF, 128, 0.1f,
                                        4, 32, nullptr, nullptr, nullptr) == YRB_OK);
  EXPECT(attn_prefill_sink_window_chunk(DEV, DEV, DEV, DEV, YRB_BF16, 1, 64, 128, 4, 2, 128, s43, 64, DEVF, 127, 0.1f,
                                        4, 32, nullptr, nullptr, nullptr) == YRB_EINVAL);
  EXPECT(attn_prefill_sink_window_chunk(DEV, nullptr, nullptr, DEV, YRB_BF16, 1, 64, 0, 4, 2, 128, s43, 64, DEVF, 128,
                                        0.1f, kMax, kMax, nullptr, nullptr, nullptr) == YRB_OK);
  EXPECT(attn_prefill_sink_window_chunk(DEV, nullptr, DEV, DEV, YRB_BF16, 1, 64, 8, 4, 2, 128, s43, 64, DEVF, 128, 0.1f,
                                        4, 32, nullptr, nullptr, nullptr) == YRB_EINVAL);
  EXPECT(attn_prefill_sink_window_chunk(DEV, DEV, DEV, DEV, YRB_BF16, 1, 64, 128, 4, 2, 128, s43, -1, DEVF, 128, 0.1f,
                                        4, 32, nullptr, nullptr, nullptr) == YRB_EINVAL);
  const int64_t sq2[2] = {4 * 128, 128}, sc3[3] = {4 * 4100 * 128, 4100 * 128, 128};
  EXPECT(attn_decode_sink_window(DEV, DEV, DEV, DEV, YRB_BF16, 2, 4, 4, 128, 4, 4096, sq2, sc3, sq2,
                                 static_cast<int32_t*>(DEV), nullptr, DEVF, 4100, 0.1f, nullptr) == YRB_OK);
  EXPECT(attn_decode_sink_window(DEV, DEV, DEV, DEV, YRB_BF16, 2, 3, 1, 128, 4, 4096, sq2, sc3, sq2,
                                 static_cast<int32_t*>(DEV), nullptr, DEVF, 4100, 0.1f, nullptr) == YRB_EUNSUPPORTED);
  EXPECT(attn_decode_sink_window(DEV, DEV, DEV, DEV, YRB_BF16, 2, 4, 4, 128, kMax, kMax, sq2, sc3, sq2,
                                 static_cast<int32_t*>(DEV), nullptr, DEVF, 4100, 0.1f, nullptr) == YRB_EINVAL);
  for (int st = -6; st <= 1; ++st) EXPECT(yrb_status_str(st) != nullptr);
}

// Products of (possibly perturbed) sizes, saturating instead of overflowing.
int64_t mul(int64_t a, int64_t b) {
  int64_t r;
  return __builtin_mul_overflow(a, b, &r) ? kMax : r;
}
int64_t mul(int64_t a, int64_t b, int64_t c) { return mul(mul(a, b), c); }
int64_t add(int64_t a, int64_t b) {
  int64_t r;
  return __builtin_add_overflow(a, b, &r) ? kMax : r;
}

// A field of a valid argument set, replaced by an edge value with
// probability 1 / (2 + fields) per field: most calls stay near the valid
// set, so both sides of every check are reached.
struct Perturb {
  int n;
  bool hit() { return next() % (uint64_t)(2 + n) == 0; }
  int64_t size(int64_t v) { return hit() ? pick(SIZES) : v; }
  int64_t stride(int64_t v) { return hit() ? pick(STRIDES) : v; }
  void* ptr(void* v) { return hit() ? pick(PTRS) : v; }
  float scale(float v) { return hit() ? pick(SCALES) : v; }
  int32_t small(int32_t v, int lo, int hi) { return hit() ? lo + (int32_t)(next() % (uint64_t)(hi - lo + 1)) : v; }
};

void sweep(int iters) {
  for (int it = 0; it < iters; ++it) {
    const int before = g_launches;
    Perturb P{8};
    const int64_t D = P.hit() ? pick(DIMS) : ((next() & 1) ? 128 : 64);
    const int64_t Hkv = P.size(1 + (int64_t)(next() % 8));
    const int64_t G = 1 << (next() % 4);
    const int64_t Hq = P.size(mul(Hkv, G));
    const int64_t B = P.size(1 + (int64_t)(next() % 4)), S = P.size(1 + (int64_t)(next() % 3000));
    const int32_t dt = P.small(YRB_BF16, -1, 3);
    switch (next() % 7) {
      case 0: {
        yrb_rope_config c = {P.small(YRB_ROPE_YARN, -1, 4), (int32_t)D, P.hit() ? (double)pick(SIZES) : 1e4,
                             P.hit() ? (double)pick(SCALES) : 4.0, P.size(4096), 1.0, P.hit() ? 0.5 : 32.0};
        double th[64], af;
        account(before, rope_tables_build(P.hit() ? nullptr : &c, P.size(0), S,
                                          static_cast<float*>(P.ptr(DEV)), th, &af, nullptr));
        break;
      }
      case 1: {
        double f[64], th[64];
        for (double& x : f) x = (next() % 64) ? 1.0 + (double)(next() % 100) : (double)pick(SCALES);
        account(before, rope_tables_build_factors((int32_t)D, P.hit() ? (double)pick(SIZES) : 1e4, f, P.size(0), S,
                                                  static_cast<float*>(P.ptr(DEV)), th, nullptr));
        break;
      }
      case 2: {
        const int64_t xs[3] = {P.stride(mul(S, Hkv, D)), P.stride(mul(Hkv, D)), P.stride(D)};
        account(before, rope_apply_ex(P.ptr(DEV), P.ptr(DEV), dt, B, S, Hkv, D, xs, xs,
                                      static_cast<float*>(P.ptr(DEV)), P.size(add(S, (int64_t)(next() % 8))),
                                      P.size(0), (next() & 1) ? static_cast<int32_t*>(DEV) : nullptr,
                                      P.small(0, -1, 2), nullptr));
        break;
      }
      case 3: {
        const int64_t s[4][3] = {{P.stride(mul(S, Hq, D)), P.stride(mul(Hq, D)), P.stride(D)},
                                 {P.stride(mul(S, Hkv, D)), P.stride(mul(Hkv, D)), P.stride(D)},
                                 {P.stride(mul(S, Hkv, D)), P.stride(mul(Hkv, D)), P.stride(D)},
                                 {P.stride(mul(S, Hq, D)), P.stride(mul(Hq, D)), P.stride(D)}};
        const int64_t pick3 = (int64_t)(next() % 3);
        if (pick3 == 0)
          account(before, attn_prefill_sink_window(P.ptr(DEV), P.ptr(DEV), P.ptr(DEV), P.ptr(DEV), dt, B, S, Hq, Hkv, D,
                                                   s, static_cast<float*>(P.ptr(DEV)), P.size(S), P.scale(0.1f),
                                                   P.size(4), P.size(64), static_cast<float*>(P.ptr(nullptr)),
                                                   P.ptr(DEV), nullptr));
        else if (pick3 == 1) {
          const int64_t qo = P.size(mul(2, S)), Sk = P.size(add(qo, S));
          account(before, attn_prefill_sink_window_chunk(P.ptr(DEV), P.ptr(DEV), P.ptr(DEV), P.ptr(DEV), dt, B, S, Sk, Hq,
                                                         Hkv, D, s, qo, static_cast<float*>(P.ptr(DEV)),
                                                         P.size(add(qo, S)), P.scale(0.1f), P.size(4), P.size(64),
                                                         static_cast<float*>(P.ptr(nullptr)), P.ptr(DEV), nullptr));
        } else
          account(before, attn_prefill_blockwise(P.ptr(DEV), P.ptr(DEV), P.ptr(DEV), P.ptr(DEV), dt, B, S, Hq, Hkv, D,
                                                 s, static_cast<float*>(P.ptr(DEV)), P.size(S), P.scale(0.1f),
                                                 P.small(1, -1, 2), static_cast<float*>(P.ptr(nullptr)),
                                                 P.ptr(nullptr), nullptr));
        break;
      }
      case 4: {
        const int64_t s[3][3] = {{P.stride(mul(S, Hq, D)), P.stride(mul(Hq, D)), P.stride(D)},
                                 {P.stride(mul(S, Hkv, D)), P.stride(mul(Hkv, D)), P.stride(D)},
                                 {P.stride(mul(S, Hkv, D)), P.stride(mul(Hkv, D)), P.stride(D)}};
        const int64_t os[3] = {P.stride(mul(S, Hq, D)), P.stride(mul(Hq, D)), P.stride(D)};
        const int64_t qo = P.size(mul(3, S)), ko = P.size(S);
        const int32_t flags = P.small(3, -1, 4);
        account(before, attn_block_accumulate(P.ptr(DEV), P.ptr(DEV), P.ptr(DEV), dt, B, S, P.size(S), Hq, Hkv, D, s,
                                              qo, ko, static_cast<float*>(P.ptr(DEV)), P.size(mul(5, S)), P.scale(0.1f),
                                              P.small(1, -1, 2), DEVF, static_cast<float*>(P.ptr(DEV)), DEVF, flags,
                                              P.ptr(DEV), P.hit() ? nullptr : os, P.ptr(nullptr), nullptr));
        break;
      }
      default: {
        const int64_t C = add(S, 4);
        const int64_t qs[2] = {P.stride(mul(Hq, D)), P.stride(D)};
        const int64_t cs[3] = {P.stride(mul(Hkv, C, D)), P.stride(mul(C, D)), P.stride(D)};
        account(before, attn_decode_sink_window_ex(
                            P.ptr(DEV), P.ptr(DEV), P.ptr(DEV), P.ptr(DEV), P.small(YRB_BF16, -1, 3), P.small(0, -1, 2),
                            B, Hq, Hkv, D, P.size(4), P.size(S), qs, cs, qs, static_cast<int32_t*>(P.ptr(DEV)),
                            static_cast<int32_t*>(P.ptr(nullptr)), static_cast<float*>(P.ptr(nullptr)),
                            static_cast<float*>(P.ptr(nullptr)), static_cast<float*>(P.ptr(DEV)), P.size(C),
                            P.scale(0.1f), nullptr));
        break;
      }
    }
  }
}

}  // namespace

int main(int argc, char** argv) {
  const int iters = argc > 1 ? std::atoi(argv[1]) : 200000;
  fixed_cases();
  sweep(iters);
  std::printf("abi driver: %d launches, %d failures\n", g_launches, failures);
  return failures == 0 ? 0 : 1;
}
