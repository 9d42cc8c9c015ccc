// Gather/pack stage of subsampled global attention on gfx950.
//
// "AVGGT: Rethinking Global Attention for Accelerating VGGT" (papernotes.org CVPR 2026 notes),
// 关键设计 2: the keys and values of the global layer are restricted to S; 关键设计 3: mean keys
// and values stand in for the dropped patches; ablation table (G2M): one mean token replaces
// all keys and values.  "RegimeVGGT ..." notes, 关键设计 3: per-frame phase of the grid.  All
// kernels are HBM-bound streaming passes.
//
//   means_kernel         one work-group per (frame feeding a mean, head): float32 sums of the
//                        frame's dropped K and V rows (16-byte loads, 32 rows in flight per
//                        work-group).  Per-frame scope: divided by |D_f| and rounded to the
//                        input type.  Single mean (global scope, G2M): the float32 sums are
//                        kept for means_reduce_kernel.
//   means_reduce_kernel  one work-group per head: adds the per-frame sums in frame order,
//                        divides by the number of tokens and rounds.
//   pack_kernel          one work-group per (64-row key tile, head): copies the K/V rows of S
//                        (and the means, then zero padding) into packed tiles.  Keys stay
//                        row-major [row][d]; for bf16 the values are written as [d][64]
//                        key-minor tiles in the order the PV matrix-core step reads them, so
//                        the attention kernel loads every operand with contiguous 16-byte
//                        reads.  Head 0 also exports S, and work-group (0,0) exports |D_f|.
//   size_bias_kernel     size-aware keys ("RegimeVGGT" notes, 关键设计 2): the logit bias of
//                        every packed key row, log g of its token in raw-score units, and a
//                        copy of log g for the diagonal term.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>

#include "device_common.h"
#include "launch.h"

namespace vggt {
namespace {

struct MeansArgs {
  const void* k;
  const void* v;
  void* means;     // [H][M][2][64] input type (per-frame scope)
  float* partial;  // [H][F][2][64] float32 sums (single mean), else nullptr
  int64_t T;
  int M;           // mean keys
  int F;           // frames feeding a mean
  IndexGeom g;
};

template <typename E>
__device__ __forceinline__ void add_chunk(float* acc, const uint4& raw);

template <>
__device__ __forceinline__ void add_chunk<uint16_t>(float* acc, const uint4& raw) {
  const uint32_t w[4] = {raw.x, raw.y, raw.z, raw.w};
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    acc[2 * i] += __uint_as_float(w[i] << 16);
    acc[2 * i + 1] += __uint_as_float(w[i] & 0xffff0000u);
  }
}

template <>
__device__ __forceinline__ void add_chunk<float>(float* acc, const uint4& raw) {
  acc[0] += __uint_as_float(raw.x);
  acc[1] += __uint_as_float(raw.y);
  acc[2] += __uint_as_float(raw.z);
  acc[3] += __uint_as_float(raw.w);
}

__device__ __forceinline__ void store_elem(uint16_t* p, float x) { *p = f32_to_bf16(x); }
__device__ __forceinline__ void store_elem(float* p, float x) { *p = x; }

template <typename E>
__global__ __launch_bounds__(256) void means_kernel(MeansArgs a) {
  constexpr int CH = 16 / int(sizeof(E));  // channels per 16-byte chunk
  constexpr int CPR = kHeadDim / CH;       // chunks per row
  constexpr int RG = 256 / CPR;            // rows in flight
  const int m = blockIdx.x, h = blockIdx.y;
  const int64_t f = mean_frame(a.g, m);
  const int k = frame_phase(a.g, f);
  const int tid = threadIdx.x, chunk = tid % CPR, rg = tid / CPR;
  const size_t base = (size_t(h) * size_t(a.T) + size_t(f) * a.g.L) * kHeadDim + chunk * CH;
  const E* kb = static_cast<const E*>(a.k) + base;
  const E* vb = static_cast<const E*>(a.v) + base;
  float ks[CH], vs[CH];
#pragma unroll
  for (int i = 0; i < CH; ++i) ks[i] = vs[i] = 0.f;
  // Rows in batches of U per thread: every load of a batch is issued before the first add, so
  // 2*U 16-byte loads are in flight per thread (kept rows and rows past the frame load nothing).
  constexpr int U = 4;
  for (int j0 = rg; j0 < a.g.L; j0 += RG * U) {
    uint4 kr[U], vr[U];
    bool use[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int j = j0 + u * RG;
      bool dropped = j < a.g.L;
      if (!a.g.g2m && dropped) {
        if (j < a.g.n_special) {
          dropped = false;  // specials are always kept
        } else {
          const int p = j - a.g.n_special;
          const int r = p / a.g.grid_w, c = p - r * a.g.grid_w;
          dropped = !patch_kept(a.g, k, r, c);  // kept: not part of D_f
        }
      }
      use[u] = dropped;
      kr[u] = vr[u] = make_uint4(0, 0, 0, 0);
      if (dropped) {
        kr[u] = *reinterpret_cast<const uint4*>(kb + size_t(j) * kHeadDim);
        vr[u] = *reinterpret_cast<const uint4*>(vb + size_t(j) * kHeadDim);
      }
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      if (use[u]) {
        add_chunk<E>(ks, kr[u]);
        add_chunk<E>(vs, vr[u]);
      }
    }
  }
  __shared__ float red[RG][2][kHeadDim];
#pragma unroll
  for (int i = 0; i < CH; ++i) {
    red[rg][0][chunk * CH + i] = ks[i];
    red[rg][1][chunk * CH + i] = vs[i];
  }
  __syncthreads();
  if (tid < 2 * kHeadDim) {
    const int which = tid / kHeadDim, ch = tid % kHeadDim;
    float s = 0.f;
    for (int r = 0; r < RG; ++r) s += red[r][which][ch];
    if (a.partial) {
      a.partial[((size_t(h) * a.F + m) * 2 + which) * kHeadDim + ch] = s;
    } else {
      E* dst = static_cast<E*>(a.means) + ((size_t(h) * a.M + m) * 2 + which) * kHeadDim + ch;
      store_elem(dst, s / float(frame_dropped(a.g, f)));
    }
  }
}

struct ReduceArgs {
  const float* partial;  // [H][F][2][64]
  void* means;           // [H][1][2][64] input type
  int F;
  float count;           // tokens the mean stands for (exact: < 2^24)
};

template <typename E>
__global__ __launch_bounds__(128) void means_reduce_kernel(ReduceArgs a) {
  const int h = blockIdx.x, tid = threadIdx.x;  // tid = which * 64 + channel
  const float* src = a.partial + size_t(h) * a.F * 2 * kHeadDim + tid;
  float s = 0.f;
  for (int m = 0; m < a.F; ++m) s += src[size_t(m) * 2 * kHeadDim];
  store_elem(static_cast<E*>(a.means) + size_t(h) * 2 * kHeadDim + tid, s / a.count);
}

struct PackArgs {
  const void* k;
  const void* v;
  const void* means;  // [H][M][2][64]
  void* kpack;        // [H][rows][64]
  void* vpack;        // bf16: [H][rows/64][64][64] key-minor; fp32: [H][rows][64]
  int32_t* index;     // [|S|] or nullptr
  int32_t* dcount;    // [N]
  uint32_t* kmax;     // [H] bf16 bits of the largest packed |k| (f16 score form), else nullptr
  int64_t T;
  int64_t rows_per_head;
  int64_t nS;
  int M;
  int g2f;
  int segment_rows;
  int frames;
  IndexGeom g;
};

// Where packed row `row` of a head comes from: a token (>= 0), mean `-2 - m`, or padding (-1).
__device__ __forceinline__ int64_t packed_source(const PackArgs& a, int64_t row) {
  if (a.g2f) {
    const int64_t f = row / a.segment_rows, j = row - f * a.segment_rows;
    return j < a.g.L ? f * a.g.L + j : -1;
  }
  if (row < a.nS) return token_of_kept_index(a.g, row);
  if (row < a.nS + a.M) return -2 - (row - a.nS);
  return -1;
}

// Position p (0..63) of a packed value tile holds key key_at(p): within each half of 32 keys,
// positions g*8 + j hold keys g*4 + j (j < 4) and 16 + g*4 + (j - 4) (j >= 4).  This is the
// order in which a 16x16 score block leaves the matrix core (lane group g owns keys g*4..g*4+3
// of every 16-key block), so P can feed the PV product straight from registers.
__device__ __forceinline__ int key_at(int p) {
  const int half = p >> 5, g = (p >> 3) & 3, j = p & 7;
  return half * 32 + (j < 4 ? g * 4 + j : 16 + g * 4 + (j - 4));
}

template <typename E, bool TRANSPOSE_V>
__global__ __launch_bounds__(256) void pack_kernel(PackArgs a) {
  constexpr int CH = 16 / int(sizeof(E));
  constexpr int CPR = kHeadDim / CH;
  constexpr int CHUNKS = kTile * CPR;
  const int tile = blockIdx.x, h = blockIdx.y, tid = threadIdx.x;
  const E* K = static_cast<const E*>(a.k) + size_t(h) * size_t(a.T) * kHeadDim;
  const E* V = static_cast<const E*>(a.v) + size_t(h) * size_t(a.T) * kHeadDim;
  const E* MK = static_cast<const E*>(a.means) + size_t(h) * a.M * 2 * kHeadDim;
  E* KP = static_cast<E*>(a.kpack) + (size_t(h) * a.rows_per_head + size_t(tile) * kTile) * kHeadDim;
  E* VP = static_cast<E*>(a.vpack) + (size_t(h) * a.rows_per_head + size_t(tile) * kTile) * kHeadDim;
  // V rows of the tile, padded to 68 halves per row for conflict-light column reads.
  __shared__ uint16_t vt[TRANSPOSE_V ? kTile : 1][68];
  uint32_t kabs = 0;  // largest |k| seen by this thread, as bf16 bits (bf16 inputs)
  for (int e = tid; e < CHUNKS; e += 256) {
    const int row = e / CPR, ch = e % CPR;
    const int64_t prow = int64_t(tile) * kTile + row;
    const int64_t src = packed_source(a, prow);
    uint4 kv = make_uint4(0, 0, 0, 0), vv = make_uint4(0, 0, 0, 0);
    if (src >= 0) {
      kv = *reinterpret_cast<const uint4*>(K + size_t(src) * kHeadDim + ch * CH);
      vv = *reinterpret_cast<const uint4*>(V + size_t(src) * kHeadDim + ch * CH);
      if (a.index && h == 0 && ch == 0 && prow < a.nS) a.index[prow] = int32_t(src);
    } else if (src <= -2) {
      const int64_t m = -2 - src;
      kv = *reinterpret_cast<const uint4*>(MK + (size_t(m) * 2 + 0) * kHeadDim + ch * CH);
      vv = *reinterpret_cast<const uint4*>(MK + (size_t(m) * 2 + 1) * kHeadDim + ch * CH);
    }
    *reinterpret_cast<uint4*>(KP + size_t(row) * kHeadDim + ch * CH) = kv;
    if constexpr (TRANSPOSE_V) {
      const uint32_t w[4] = {kv.x, kv.y, kv.z, kv.w};
#pragma unroll
      for (int i = 0; i < 4; ++i) kabs = max(kabs, max(w[i] & 0x7fffu, (w[i] >> 16) & 0x7fffu));
    }
    if constexpr (TRANSPOSE_V) {
      uint2* dst = reinterpret_cast<uint2*>(&vt[row][ch * CH]);
      dst[0] = make_uint2(vv.x, vv.y);
      dst[1] = make_uint2(vv.z, vv.w);
    } else {
      *reinterpret_cast<uint4*>(VP + size_t(row) * kHeadDim + ch * CH) = vv;
    }
  }
  if (a.dcount && h == 0 && tile == 0) {
    for (int f = tid; f < a.frames; f += 256)
      a.dcount[f] = frame_dropped(a.g, f);
  }
  if constexpr (TRANSPOSE_V) {
    if (a.kmax) {  // (non-negative bf16 bits order like the values)
      // One atomic per work-group at most, and none once the head's maximum is at least this
      // tile's (the maximum only grows, so a stale read can only cause a redundant atomic).
      __shared__ uint32_t wmax[4];
#pragma unroll
      for (int off = 32; off > 0; off >>= 1) kabs = max(kabs, uint32_t(__shfl_xor(int(kabs), off)));
      if ((tid & 63) == 0) wmax[tid >> 6] = kabs;
      __syncthreads();
      if (tid == 0) {
        kabs = max(max(wmax[0], wmax[1]), max(wmax[2], wmax[3]));
        if (kabs > __hip_atomic_load(&a.kmax[h], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT))
          atomicMax(&a.kmax[h], kabs);
      }
    }
  }
  if constexpr (TRANSPOSE_V) {
    __syncthreads();
    // Output tile [64 d][64 positions]: thread writes 8 positions (16 bytes) of one d-row.
    for (int e = tid; e < kTile * 8; e += 256) {
      const int pc = e & 7, d = e >> 3;
      uint32_t w[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const uint32_t lo = vt[key_at(pc * 8 + 2 * i)][d];
        const uint32_t hi = vt[key_at(pc * 8 + 2 * i + 1)][d];
        w[i] = lo | (hi << 16);
      }
      *reinterpret_cast<uint4*>(reinterpret_cast<uint16_t*>(VP) + d * kTile + pc * 8) =
          make_uint4(w[0], w[1], w[2], w[3]);
    }
  }
}

// Index set and per-frame dropped counts alone, for plans whose attention reads K and V in
// place (dense and G2F: nothing to gather).
__global__ __launch_bounds__(256) void index_kernel(PackArgs a) {
  const int64_t stride = int64_t(gridDim.x) * 256;
  const int64_t first = int64_t(blockIdx.x) * 256 + threadIdx.x;
  if (a.index)
    for (int64_t i = first; i < a.nS; i += stride) a.index[i] = int32_t(token_of_kept_index(a.g, i));
  for (int64_t f = first; f < a.frames; f += stride) a.dcount[f] = frame_dropped(a.g, int(f));
}

// f16 score form, before the pack: the per-head maxima start at zero.
__global__ __launch_bounds__(256) void kmax_clear_kernel(uint32_t* kmax, int heads) {
  const int h = blockIdx.x * 256 + threadIdx.x;
  if (h < heads) kmax[h] = 0;
}

// f16 score form, after the pack: packed bf16 keys of head h -> f16(k * 2^-e_h) in place (an
// exact conversion for |k| above 2^-21 of the head's maximum, which sits in [128, 256)).  One
// thread per 16-byte chunk of 8 values.
__global__ __launch_bounds__(256) void kpack_f16_kernel(uint16_t* kpack, const uint32_t* kmax,
                                                        int64_t chunks_per_head, int64_t chunks) {
  const int64_t stride = int64_t(gridDim.x) * 256;
  for (int64_t i = int64_t(blockIdx.x) * 256 + threadIdx.x; i < chunks; i += stride) {
    const int h = int(i / chunks_per_head);
    const float scale = __builtin_amdgcn_ldexpf(1.f, -key_scale_exp(kmax[h]));
    uint4* p = reinterpret_cast<uint4*>(kpack) + i;
    const uint4 raw = *p;
    const uint32_t w[4] = {raw.x, raw.y, raw.z, raw.w};
    uint32_t o[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const _Float16 lo = (_Float16)(__uint_as_float(w[j] << 16) * scale);
      const _Float16 hi = (_Float16)(__uint_as_float(w[j] & 0xffff0000u) * scale);
      o[j] = uint32_t(__builtin_bit_cast(uint16_t, lo)) | (uint32_t(__builtin_bit_cast(uint16_t, hi)) << 16);
    }
    *p = make_uint4(o[0], o[1], o[2], o[3]);
  }
}

struct SizeBiasArgs {
  PackArgs pk;           // geometry of the packed rows (packed_source)
  const float* log_g;    // [T]
  float* kbias;          // [segments * segment_rows]
  float* logsize;        // [T]
  int64_t rows;          // segments * segment_rows
  float scale;           // sqrt(d) = 1 / tau: logit units -> raw-score units
};

__global__ __launch_bounds__(256) void size_bias_kernel(SizeBiasArgs a) {
  const int64_t stride = int64_t(gridDim.x) * 256;
  for (int64_t i = int64_t(blockIdx.x) * 256 + threadIdx.x; i < a.rows; i += stride) {
    const int64_t src = packed_source(a.pk, i);
    a.kbias[i] = src >= 0 ? a.log_g[src] * a.scale : 0.f;  // padding rows are masked later
  }
  for (int64_t t = int64_t(blockIdx.x) * 256 + threadIdx.x; t < a.pk.T; t += stride) a.logsize[t] = a.log_g[t];
}

}  // namespace

hipError_t launch_size_bias(const vggt_attn_plan_s& p, const float* log_g, void* ws, hipStream_t stream) {
  char* base = static_cast<char*>(ws);
  SizeBiasArgs a{};
  a.pk.T = p.T;
  a.pk.nS = p.nS;
  a.pk.M = int(p.M);
  a.pk.g2f = p.g2f ? 1 : 0;
  a.pk.segment_rows = int(p.segment_rows);
  a.pk.g = p.geom;
  a.log_g = log_g;
  a.kbias = reinterpret_cast<float*>(base + p.layout.off_kbias);
  a.logsize = reinterpret_cast<float*>(base + p.layout.off_logsize);
  a.rows = p.rows_per_head;
  a.scale = float(std::sqrt(double(p.head_dim)));
  const int64_t work = a.rows > p.T ? a.rows : p.T;
  const unsigned blocks = unsigned(std::min<int64_t>((work + 255) / 256, 4096));
  hipLaunchKernelGGL(size_bias_kernel, dim3(blocks), dim3(256), 0, stream, a);
  return hipGetLastError();
}

hipError_t launch_means(const vggt_attn_plan_s& p, const void* k, const void* v, void* ws,
                        hipStream_t stream) {
  if (p.M == 0) return hipSuccess;
  const bool single = p.mean_global || p.g2m;
  char* base = static_cast<char*>(ws);
  MeansArgs a{};
  a.k = k;
  a.v = v;
  a.means = base + p.layout.off_means;
  a.partial = single ? reinterpret_cast<float*>(base + p.layout.off_partial) : nullptr;
  a.T = p.T;
  a.M = int(p.M);
  a.F = int(p.M_frames);
  a.g = p.geom;
  const dim3 grid(unsigned(p.M_frames), unsigned(p.heads));
  const bool bf16 = p.in_dtype == VGGT_ATTN_BF16;
  if (bf16)
    hipLaunchKernelGGL(means_kernel<uint16_t>, grid, dim3(256), 0, stream, a);
  else
    hipLaunchKernelGGL(means_kernel<float>, grid, dim3(256), 0, stream, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || !single) return e;
  ReduceArgs r{};
  r.partial = a.partial;
  r.means = a.means;
  r.F = a.F;
  r.count = float(p.dropped_total);
  if (bf16)
    hipLaunchKernelGGL(means_reduce_kernel<uint16_t>, dim3(unsigned(p.heads)), dim3(128), 0, stream, r);
  else
    hipLaunchKernelGGL(means_reduce_kernel<float>, dim3(unsigned(p.heads)), dim3(128), 0, stream, r);
  return hipGetLastError();
}

hipError_t launch_pack(const vggt_attn_plan_s& p, const void* k, const void* v, void* ws,
                       hipStream_t stream) {
  char* base = static_cast<char*>(ws);
  PackArgs a{};
  a.k = k;
  a.v = v;
  a.means = base + p.layout.off_means;
  a.kpack = base + p.layout.off_kpack;
  a.vpack = base + p.layout.off_vpack;
  a.index = p.g2f ? nullptr : reinterpret_cast<int32_t*>(base + p.layout.off_index);
  a.dcount = reinterpret_cast<int32_t*>(base + p.layout.off_dcount);
  a.T = p.T;
  a.rows_per_head = p.rows_per_head;
  a.nS = p.nS;
  a.M = int(p.M);
  a.g2f = p.g2f ? 1 : 0;
  a.segment_rows = int(p.segment_rows);
  a.frames = p.frames;
  a.g = p.geom;
  a.kmax = p.prescale_q ? reinterpret_cast<uint32_t*>(base + p.layout.off_kmax) : nullptr;
  if (p.inplace) {
    const int64_t work = std::max<int64_t>(a.index ? p.nS : 0, p.frames);
    const unsigned blocks = unsigned(std::min<int64_t>((work + 255) / 256, 4096));
    hipLaunchKernelGGL(index_kernel, dim3(blocks), dim3(256), 0, stream, a);
    return hipGetLastError();
  }
  if (a.kmax) {
    hipLaunchKernelGGL(kmax_clear_kernel, dim3(unsigned((p.heads + 255) / 256)), dim3(256), 0, stream, a.kmax, p.heads);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  const dim3 grid(unsigned(p.rows_per_head / kTile), unsigned(p.heads));
  if (p.in_dtype == VGGT_ATTN_BF16)
    hipLaunchKernelGGL((pack_kernel<uint16_t, true>), grid, dim3(256), 0, stream, a);
  else
    hipLaunchKernelGGL((pack_kernel<float, false>), grid, dim3(256), 0, stream, a);
  if (!a.kmax) return hipGetLastError();
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const int64_t per_head = p.rows_per_head * kHeadDim / 8;
  const int64_t chunks = per_head * p.heads;
  const unsigned blocks = unsigned(std::min<int64_t>((chunks + 255) / 256, 8192));
  hipLaunchKernelGGL(kpack_f16_kernel, dim3(blocks), dim3(256), 0, stream, static_cast<uint16_t*>(a.kpack),
                     static_cast<const uint32_t*>(a.kmax), per_head, chunks);
  return hipGetLastError();
}

}  // namespace vggt
