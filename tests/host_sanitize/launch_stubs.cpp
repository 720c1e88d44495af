// Stand-ins for the kernel launchers, for the host-only sanitizer build of
// the C-ABI layer: each records the launch and checks that the arguments
// it receives are ones the validated layer may pass on (a failed check
// aborts, and the sanitizers report any bad access on the way).
#include <cstdio>
#include <cstdlib>

#include "kernels.h"

int g_launches = 0;

#define CHECK(c)                                                        \
  do {                                                                  \
    if (!(c)) {                                                         \
      std::fprintf(stderr, "launch stub: %s failed (%s:%d)\n", #c, __FILE__, __LINE__); \
      std::abort();                                                     \
    }                                                                   \
  } while (0)

namespace yrb {

hipError_t launch_rope_tables(const double* theta, int half, int64_t pos0, int64_t n_pos, float* cos_sin,
                              hipStream_t) {
  CHECK(theta && cos_sin && (half == 32 || half == 64) && pos0 >= 0 && n_pos > 0);
  for (int i = 0; i < half; ++i) CHECK(theta[i] > 0.0);
  ++g_launches;
  return hipSuccess;
}

hipError_t launch_rope_apply(int dtype, int D, bool, const RopeArgs& a, hipStream_t) {
  CHECK((dtype == kBF16 || dtype == kF32) && (D == 64 || D == 128));
  CHECK(a.x && a.y && a.cos_sin && a.B > 0 && a.S > 0 && a.H > 0);
  for (int i = 0; i < 3; ++i) CHECK(a.xs[i] >= 0 && a.ys[i] >= 0 && a.xs[i] < (int64_t(1) << 31));
  ++g_launches;
  return hipSuccess;
}

hipError_t launch_attention(int dtype, int D, const AttnArgs& a, hipStream_t) {
  CHECK((dtype == kBF16 || dtype == kF32) && (D == 64 || D == 128));
  CHECK(a.q && a.B > 0 && a.Sq > 0 && a.Sk >= 0 && a.Hq > 0 && a.Hkv > 0 && a.Hq % a.Hkv == 0);
  CHECK(a.Sk == 0 || (a.k && a.v));
  CHECK(a.q_offset + a.Sq < (int64_t(1) << 31) && a.k_offset + a.Sk < (int64_t(1) << 31));
  CHECK(!a.finalize || a.o);
  CHECK(!a.store_state || (a.o_acc && a.m && a.l));
  CHECK(a.softmax_scale > 0.f);
  ++g_launches;
  return hipSuccess;
}

hipError_t launch_attention_bf16_pp(int D, const AttnArgs& a, hipStream_t s) {
  CHECK(a.window > 0 && a.n_sink >= 0 && !a.store_state);
  return launch_attention(kBF16, D, a, s);
}

hipError_t launch_decode(int cache_dtype, int D, bool, const DecodeArgs& a, hipStream_t) {
  CHECK((cache_dtype == kBF16 || cache_dtype == kFP8E4M3) && (D == 64 || D == 128));
  CHECK(a.q && a.k && a.v && a.o && a.cache_len && a.cos_sin && a.B > 0);
  CHECK(a.Hq > 0 && a.Hkv > 0 && a.Hq % a.Hkv == 0 && a.window >= 1 && a.n_sink >= 0);
  CHECK(a.n_sink + a.window < (int64_t(1) << 31));
  ++g_launches;
  return hipSuccess;
}

}  // namespace yrb
