// RoPE cos/sin tables and the half-split pair rotation pass (gfx950).
//
// Tables: row r holds (cos, sin) of (pos0 + r) * theta'_i for each pair i
// ("Context Window Scaling ..." (tecvarsity), Section 2: the 2x2 rotation by
// m * theta_i).  Every 16th row's angle is formed and reduced in fp64 so
// that rows at positions ~2^18 keep fp32 accuracy; the rows between follow
// by angle addition in fp64; only the final values are rounded.
//
// Rotation: (x_i, x_{i+d/2}) -> (x_i c - x_{i+d/2} s, x_i s + x_{i+d/2} c),
// fp32 arithmetic, bf16 results rounded to nearest even.  HBM-bound: each
// thread moves two 16-byte halves of one row and reads its table slice
// (shared by all heads of a token, so it stays in L2).
#include <algorithm>
#include <cmath>
#include <cstdint>

#include "common.h"
#include "kernels.h"

namespace yrb {

struct ThetaPack {
  double t[64];   // theta'_i
  double c[64];   // cos(theta'_i)
  double s[64];   // sin(theta'_i)
};

// Rows a thread writes for its pair: the first from its own reduced angle,
// each further one by turning the row before by theta'_i.
constexpr int kTabRows = 16;

// half = d/2 is 32 or 64: pair index by mask, row group by shift.  Lanes
// take consecutive pairs, so each store of a wave writes whole rows.
__global__ __launch_bounds__(256) void rope_tables_kernel(ThetaPack th, int log2_half, int64_t pos0,
                                                          int64_t n_pos, float2* out) {
  const int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  const int i = (int)(idx & ((1 << log2_half) - 1));
  const int64_t r0 = (idx >> log2_half) * kTabRows;
  if (r0 >= n_pos) return;
  const double a = (double)(pos0 + r0) * th.t[i];
  // Reduce a modulo 2 pi in fp64 (Cody and Waite's two-constant
  // subtraction: 2 pi = P1 + P2, P1 with 33 significant bits so that k * P1
  // is exact for |k| < 2^20), then take sin/cos of the reduced angle in fp32.
  // The reduced angle keeps ~2^-45 absolute error in fp64 and ~2^-23 after
  // rounding to fp32, far inside the table tolerance.  Larger angles take
  // the fp64 library routine.
  constexpr double kP1 = 0x1.921fb544p+2;           // 2 pi rounded to 33 significant bits
  constexpr double kP2 = 0x1.0b4611a626331p-32;     // 2 pi - kP1 (rounded; 1.4e-26 left over)
  constexpr double kInv2Pi = 0x1.45f306dc9c883p-3;  // 1 / (2 pi)
  float s, c;
  const double k = __builtin_rint(a * kInv2Pi);
  if (__builtin_fabs(k) < 1048576.0) {
    double t = __builtin_fma(-k, kP1, a);
    t = __builtin_fma(-k, kP2, t);
    sincosf((float)t, &s, &c);
  } else {
    double sd, cd;
    sincos(a, &sd, &cd);
    s = (float)sd;
    c = (float)cd;
  }
  float2* o = out + (r0 << log2_half) + i;
  o[0] = make_float2(c, s);
  // The next rows by angle addition, (c, s) <- (c C - s S, s C + c S) with
  // C, S the cosine and sine of theta'_i, in fp64: a rotation keeps the
  // first row's error (one fp32 rounding) and adds ~2^-53 a step, so every
  // row stays within about 2^-23 of the exact value before its own
  // rounding.
  const int rows = (int)(n_pos - r0 < kTabRows ? n_pos - r0 : kTabRows);
  const double C = th.c[i], S = th.s[i];
  double cd = c, sd = s;
  for (int j = 1; j < rows; ++j) {
    const double cn = __builtin_fma(cd, C, -(sd * S));
    sd = __builtin_fma(sd, C, cd * S);
    cd = cn;
    o[(int64_t)j << log2_half] = make_float2((float)cd, (float)sd);
  }
}

hipError_t launch_rope_tables(const double* theta, int half, int64_t pos0, int64_t n_pos,
                              float* cos_sin, hipStream_t stream) {
  if (half != 32 && half != 64) return hipErrorInvalidValue;
  if (n_pos == 0) return hipSuccess;
  ThetaPack th = {};
  for (int i = 0; i < half; ++i) {
    th.t[i] = theta[i];
    th.c[i] = std::cos(theta[i]);
    th.s[i] = std::sin(theta[i]);
  }
  const int64_t threads = (n_pos + kTabRows - 1) / kTabRows * half;
  const int64_t blocks = (threads + 255) / 256;
  hipLaunchKernelGGL(rope_tables_kernel, dim3((unsigned)blocks), dim3(256), 0, stream, th, half == 64 ? 6 : 5,
                     pos0, n_pos, reinterpret_cast<float2*>(cos_sin));
  return hipGetLastError();
}

// 16-byte chunk of 8 bf16 or 4 fp32 values.
template <typename T>
struct Vec;
template <>
struct Vec<__bf16> {
  static constexpr int N = 8;
  __device__ static void load(const __bf16* p, float* f) {
    u32x4 w = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
    unpack8(w, f);
  }
  __device__ static void store(__bf16* p, const float* f) {
    *reinterpret_cast<u32x4*>(p) = pack8(f);
  }
};
template <>
struct Vec<float> {
  static constexpr int N = 4;
  __device__ static void load(const float* p, float* f) {
    f32x4 w = __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(p));
    for (int i = 0; i < 4; ++i) f[i] = w[i];
  }
  __device__ static void store(float* p, const float* f) {
    *reinterpret_cast<f32x4*>(p) = (f32x4){f[0], f[1], f[2], f[3]};
  }
};

// Grid: x = token s, y = groups of 256 (head, chunk) threads of that token,
// z = batch b (batch_base + blockIdx.z): no index divisions beyond the
// constant PER_ROW.  Thread c of a row moves the chunks at c N and
// D/2 + c N (coalesced the same way in both layouts).  Half-split, they hold
// pairs c N .. c N + N-1 (first elements, then partners); interleaved (IL),
// each chunk holds N/2 whole pairs (2p, 2p+1): pairs c N/2 .. and
// D/4 + c N/2 ..
template <typename T, int D, bool IL>
__global__ __launch_bounds__(256) void rope_apply_kernel(RopeArgs a, int64_t batch_base) {
  constexpr int N = Vec<T>::N;
  constexpr int PER_ROW = (D / 2) / N;  // threads per (b, s, h) row
  const int j = (int)blockIdx.y * 256 + (int)threadIdx.x;
  if (j >= (int)a.H * PER_ROW) return;
  const int c = j % PER_ROW;
  const int64_t h = j / PER_ROW;
  const int64_t s = blockIdx.x;
  const int64_t b = batch_base + blockIdx.z;
  const int64_t pos = a.pos_ids ? (int64_t)a.pos_ids[b * a.S + s] : a.pos_offset + s;
  const T* xr = reinterpret_cast<const T*>(a.x) + b * a.xs[0] + s * a.xs[1] + h * a.xs[2];
  T* yr = reinterpret_cast<T*>(a.y) + b * a.ys[0] + s * a.ys[1] + h * a.ys[2];
  const int i0 = c * N;
  float x[N], z[N], lo[N], hi[N];
  if constexpr (IL) {
    float wa[N], wb[N];
    Vec<T>::load(xr + i0, wa);
    Vec<T>::load(xr + D / 2 + i0, wb);
#pragma unroll
    for (int j = 0; j < N / 2; ++j) {
      x[j] = wa[2 * j];
      z[j] = wa[2 * j + 1];
      x[N / 2 + j] = wb[2 * j];
      z[N / 2 + j] = wb[2 * j + 1];
    }
  } else {
    Vec<T>::load(xr + i0, x);
    Vec<T>::load(xr + D / 2 + i0, z);
  }
  if (pos < 0 || pos >= a.n_rows) {
    const float nan = __builtin_nanf("");
    for (int j = 0; j < N; ++j) lo[j] = hi[j] = nan;
  } else {
    // (cos, sin) of this thread's pairs: i0 .. i0+N-1 (half-split), or
    // i0/2 .. and D/4 + i0/2 .. (interleaved), two pairs per f32x4
    const float* row = a.cos_sin + pos * (D / 2) * 2;
#pragma unroll
    for (int j = 0; j < N / 2; ++j) {
      const int pr = IL ? (2 * j < N / 2 ? i0 / 2 + 2 * j : D / 4 + i0 / 2 + 2 * j - N / 2) : i0 + 2 * j;
      f32x4 t = *reinterpret_cast<const f32x4*>(row + 2 * pr);  // pairs pr, pr+1
      lo[2 * j] = x[2 * j] * t[0] - z[2 * j] * t[1];
      hi[2 * j] = x[2 * j] * t[1] + z[2 * j] * t[0];
      lo[2 * j + 1] = x[2 * j + 1] * t[2] - z[2 * j + 1] * t[3];
      hi[2 * j + 1] = x[2 * j + 1] * t[3] + z[2 * j + 1] * t[2];
    }
  }
  if constexpr (IL) {
    float wa[N], wb[N];
#pragma unroll
    for (int j = 0; j < N / 2; ++j) {
      wa[2 * j] = lo[j];
      wa[2 * j + 1] = hi[j];
      wb[2 * j] = lo[N / 2 + j];
      wb[2 * j + 1] = hi[N / 2 + j];
    }
    Vec<T>::store(yr + i0, wa);
    Vec<T>::store(yr + D / 2 + i0, wb);
  } else {
    Vec<T>::store(yr + i0, lo);
    Vec<T>::store(yr + D / 2 + i0, hi);
  }
}

template <typename T, int D, bool IL>
static hipError_t launch_rope_t(const RopeArgs& a, hipStream_t stream) {
  constexpr int PER_ROW = (D / 2) / Vec<T>::N;
  if (a.B == 0 || a.S == 0 || a.H == 0) return hipSuccess;
  // a dispatch's x extent (blocks x 256 work-items) is a 32-bit count
  if (a.S > (int64_t)(UINT32_MAX / 256) || a.H * PER_ROW > INT32_MAX) return hipErrorInvalidValue;
  const unsigned groups = (unsigned)((a.H * PER_ROW + 255) / 256);
  constexpr int64_t kMaxZ = 65535;   // grid z limit: batches go in slices of it
  for (int64_t b0 = 0; b0 < a.B; b0 += kMaxZ) {
    const unsigned nb = (unsigned)std::min<int64_t>(kMaxZ, a.B - b0);
    hipLaunchKernelGGL((rope_apply_kernel<T, D, IL>), dim3((unsigned)a.S, groups, nb), dim3(256), 0, stream, a,
                       b0);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

template <bool IL>
static hipError_t launch_rope_l(int dtype, int D, const RopeArgs& a, hipStream_t stream) {
  if (dtype == kBF16) return D == 64 ? launch_rope_t<__bf16, 64, IL>(a, stream)
                                     : launch_rope_t<__bf16, 128, IL>(a, stream);
  return D == 64 ? launch_rope_t<float, 64, IL>(a, stream) : launch_rope_t<float, 128, IL>(a, stream);
}

hipError_t launch_rope_apply(int dtype, int D, bool interleaved, const RopeArgs& a, hipStream_t stream) {
  return interleaved ? launch_rope_l<true>(dtype, D, a, stream) : launch_rope_l<false>(dtype, D, a, stream);
}

}  // namespace yrb
