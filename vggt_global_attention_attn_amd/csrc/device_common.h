// Device-side helpers shared by the gfx950 kernels: vector types, bf16 conversions and the
// closed-form description of the kept set S.
#pragma once

#include <hip/hip_runtime.h>

#include <cstdint>

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

// Is token t (global id) in S?  "AVGGT" notes, 关键设计 2: specials always; every token of a
// dense frame; in a compressed frame the top-left patch of each s_h x s_w window.
__device__ __forceinline__ bool token_kept(const IndexGeom& g, int64_t t) {
  if (!g.subsampled) return true;
  const int f = int(t / g.L);
  const int j = int(t - int64_t(f) * g.L);
  if (j < g.n_special || (g.ref_dense && f == 0)) return true;
  const int p = j - g.n_special;
  const int r = p / g.grid_w, c = p - (p / g.grid_w) * g.grid_w;
  return (r % g.s_h) == 0 && (c % g.s_w) == 0;
}

// The i-th element of S in ascending order (0 <= i < |S|), in closed form.
__device__ __forceinline__ int64_t token_of_kept_index(const IndexGeom& g, int64_t i) {
  if (!g.subsampled) return i;
  const int64_t per = g.n_special + g.kept;  // S entries of one compressed frame
  int64_t f, j;
  if (g.ref_dense) {
    if (i < g.L) return i;
    const int64_t r = i - g.L;
    f = 1 + r / per;
    j = r - (f - 1) * per;
  } else {
    f = i / per;
    j = i - f * per;
  }
  int64_t slot;
  if (j < g.n_special) {
    slot = j;
  } else {
    const int kp = int(j - g.n_special);
    const int kr = kp / g.kw, kc = kp - (kp / g.kw) * g.kw;
    slot = g.n_special + int64_t(kr) * g.s_h * g.grid_w + int64_t(kc) * g.s_w;
  }
  return f * g.L + slot;
}

}  // namespace vggt
