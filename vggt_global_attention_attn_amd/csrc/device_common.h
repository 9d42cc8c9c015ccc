// Helpers shared by the gfx950 kernels: vector types, bf16 conversions and the closed-form
// description of the kept set S and of the mean frames (integer code, also callable on the host).
#pragma once

#include <hip/hip_runtime.h>

#include <cstdint>
#include <utility>

#include "plan.h"

namespace vggt {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));

__device__ __forceinline__ float bf16_to_f32(uint16_t b) { return __uint_as_float(uint32_t(b) << 16); }

// Round-to-nearest-even (the hardware v_cvt_pk_bf16_f32 conversion).
__device__ __forceinline__ uint16_t f32_to_bf16(float x) { return __builtin_bit_cast(uint16_t, (__bf16)x); }

__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  return uint32_t(f32_to_bf16(lo)) | (uint32_t(f32_to_bf16(hi)) << 16);
}

// f16 score form: exponent e of the power-of-two key scale 2^-e of one head, from the bf16 bits
// of the largest |k| among its packed keys.  e puts that maximum in [128, 256), so every scaled
// key lies in f16's range and is exact there down to 2^-21 of the maximum; e is clamped to
// [-120, 120] so that 2^e and 2^-e are normal float32 values.
__device__ __forceinline__ int key_scale_exp(uint32_t kmax_bits) {
  if (kmax_bits == 0) return 0;
  const float km = __uint_as_float(kmax_bits << 16);
  const int e = __builtin_amdgcn_frexp_expf(km) - 8;  // km = m * 2^x, m in [0.5, 1): floor(log2 km) = x - 1
  return e < -120 ? -120 : (e > 120 ? 120 : e);
}

// t[i] for a run-time i, written as a chain of selects over compile-time indices (a fold
// expression, so every access has a constant index before any loop pass runs): indexing an
// array of the kernel-argument struct with a run-time value would make the compiler copy the
// whole struct to scratch memory.
template <typename V, int N, int... I>
__host__ __device__ __forceinline__ V pick_impl(const V (&t)[N], int i, std::integer_sequence<int, I...>) {
  V r = t[0];
  ((r = (i == I) ? t[I] : r), ...);
  return r;
}
template <typename V, int N>
__host__ __device__ __forceinline__ V pick(const V (&t)[N], int i) {
  return pick_impl(t, i, std::make_integer_sequence<int, N>{});
}

// Largest k < n with prefix[k] <= x, for a nondecreasing prefix with prefix[0] <= x: the
// number of j in [1, n) with prefix[j] <= x.
template <int N, int... I>
__host__ __device__ __forceinline__ int prefix_slot_impl(const int (&prefix)[N], int n, int x,
                                                         std::integer_sequence<int, I...>) {
  return ((int(I > 0 && I < n) & int(prefix[I] <= x)) + ...);
}
template <int N>
__host__ __device__ __forceinline__ int prefix_slot(const int (&prefix)[N], int n, int x) {
  return prefix_slot_impl(prefix, n, x, std::make_integer_sequence<int, N>{});
}

// Grid phase of frame f: f mod (s_h*s_w) with the phase-shifted grid, else 0.  Phase k has
// row offset k / s_w and column offset k % s_w ("RegimeVGGT" notes, 关键设计 3).
__host__ __device__ __forceinline__ int frame_phase(const IndexGeom& g, int64_t f) {
  return g.nphase > 1 ? int(f % g.nphase) : 0;
}

// Is patch (r, c) of a compressed frame of phase k kept?  "AVGGT" notes, 关键设计 2: the first
// patch of each s_h x s_w window, the windows starting at the phase's offsets.
__host__ __device__ __forceinline__ bool patch_kept(const IndexGeom& g, int k, int r, int c) {
  const int ro = k / g.s_w, co = k - ro * g.s_w;
  return (r % g.s_h) == ro && (c % g.s_w) == co;
}

// Is token t (global id) in S?  Specials always; every token of a dense frame; in a
// compressed frame the grid points of its phase.  Under G2M no token is.
__host__ __device__ __forceinline__ bool token_kept(const IndexGeom& g, int64_t t) {
  if (g.g2m) return false;
  if (!g.subsampled) return true;
  const int64_t f = t / g.L;
  const int j = int(t - f * g.L);
  if (j < g.n_special || (g.ref_dense && f == 0)) return true;
  const int p = j - g.n_special;
  const int r = p / g.grid_w, c = p - r * g.grid_w;
  return patch_kept(g, frame_phase(g, f), r, c);
}

// |D_f|: the tokens of frame f that feed its mean (dropped patches; every token under G2M).
__host__ __device__ __forceinline__ int frame_dropped(const IndexGeom& g, int64_t f) {
  if (g.g2m) return g.L;
  if (!g.subsampled || (g.ref_dense && f == 0)) return 0;
  const int k = frame_phase(g, f);
  return g.P - pick(g.rows_of, k / g.s_w) * pick(g.cols_of, k % g.s_w);
}

// The i-th element of S in ascending order (0 <= i < |S|), in closed form.  Compressed frames
// are counted as if frame 0 were compressed too ("virtual" index); one run of nphase frames
// holds cprefix[nphase] entries of S, and phase k starts at cprefix[k] within its run.
__host__ __device__ __forceinline__ int64_t token_of_kept_index(const IndexGeom& g, int64_t i) {
  if (!g.subsampled) return i;
  if (g.ref_dense) {
    if (i < g.L) return i;
    i -= g.L;
  }
  const int period = pick(g.cprefix, g.nphase);
  const int64_t v = i + int64_t(g.f0 / g.nphase) * period + pick(g.cprefix, g.f0 % g.nphase);
  const int64_t run = v / period;
  const int rem = int(v - run * period);
  const int k = prefix_slot(g.cprefix, g.nphase, rem);
  const int64_t f = run * g.nphase + k;
  const int j = rem - pick(g.cprefix, k);
  if (j < g.n_special) return f * g.L + j;
  const int ro = k / g.s_w, co = k - ro * g.s_w;
  const int nc = pick(g.cols_of, co);
  const int kp = j - g.n_special;
  const int kr = kp / nc, kc = kp - kr * nc;
  return f * g.L + g.n_special + int64_t(ro + kr * g.s_h) * g.grid_w + (co + kc * g.s_w);
}

// Frame of the m-th frame that feeds a mean (0 <= m < number of such frames): the compressed
// frames with a nonempty dropped set in ascending order (every frame under G2M).  One run of
// nphase frames holds mprefix[nphase] of them.
__host__ __device__ __forceinline__ int64_t mean_frame(const IndexGeom& g, int64_t m) {
  if (g.g2m) return m;
  const int per = pick(g.mprefix, g.nphase);
  const int64_t v = m + int64_t(g.f0 / g.nphase) * per + pick(g.mprefix, g.f0 % g.nphase);
  const int64_t run = v / per;
  const int rem = int(v - run * per);
  return run * g.nphase + prefix_slot(g.mprefix, g.nphase, rem);
}

}  // namespace vggt
