// attn_prefill_blockwise_noalloc: attn_prefill_blockwise for callers that
// cannot allocate device memory (code under HIP graph capture, tight
// serving loops, harnesses that forbid allocation).  The work-claim counter
// that attn_prefill_blockwise takes from a caller's workspace comes here
// from a file-scope device array, one copy per GPU, that lives until the
// process ends.
//
// The array's name in host code is a host-side stand-in, not a device
// address: its address on the current device is taken once per device with
// hipGetSymbolAddress, checked, and kept; launches receive that address.
// Nothing here allocates, frees or calls an allocating routine.
#include <hip/hip_runtime.h>

#include <mutex>

#include "../../include/yrb.h"

namespace {

// One workspace, whatever the input size: the claim counter needs no more.
static __device__ __align__(256) unsigned char scratch[YRB_WORKSPACE_BYTES];

constexpr int kMaxDevices = 64;
void* g_scratch[kMaxDevices] = {};
std::mutex g_scratch_mutex;

// The current device's copy of `scratch`, or an error status.
int scratch_of_current_device(void** out) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess) return YRB_EHIP;
  if (dev < 0 || dev >= kMaxDevices) return YRB_EUNSUPPORTED;
  std::lock_guard<std::mutex> lock(g_scratch_mutex);
  if (!g_scratch[dev]) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return YRB_EHIP;
    g_scratch[dev] = p;
  }
  *out = g_scratch[dev];
  return YRB_OK;
}

}  // namespace

extern "C" int attn_prefill_blockwise_noalloc(const void* q, const void* k, const void* v, void* o,
                                              int32_t dtype, int64_t B, int64_t S, int64_t Hq,
                                              int64_t Hkv, int64_t D, const int64_t strides[4][3],
                                              const float* cos_sin, int64_t n_table_rows,
                                              float softmax_scale, int32_t causal, float* lse,
                                              void* stream) {
  void* ws = nullptr;
  const int st = scratch_of_current_device(&ws);
  if (st != YRB_OK) return st;
  return attn_prefill_blockwise(q, k, v, o, dtype, B, S, Hq, Hkv, D, strides, cos_sin, n_table_rows,
                                softmax_scale, causal, lse, ws, stream);
}
