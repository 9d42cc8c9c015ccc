// Attention stage on gfx950: out = softmax(Q K^T / sqrt(d)) V over packed keys, with the
// diagonal self term and the mean keys folded into the same running max and sum.
//
// Operation: "AVGGT: Rethinking Global Attention for Accelerating VGGT" (papernotes.org CVPR
// 2026 notes), 关键设计 2 (the attention equation over the kept set S), 关键设计 3 (diagonal
// self term and mean K/V share one softmax normalisation), 关键设计 1 (Global-to-Frame: keys of
// a query are the tokens of its own frame); "RegimeVGGT ..." (papernotes.org NeurIPS 2026
// notes), 关键设计 2 (a key standing for g tokens carries +ln g on its logit -- used for the
// COUNT weighting of the mean keys).
//
// attn_bf16_kernel: flash-style forward on the bf16 matrix cores (v_mfma_f32_16x16x32_bf16,
// float32 accumulation).  A work-group of 4 waves owns BM = 4*16*QB query rows of one head and
// streams the key segment in 64-key tiles through double-buffered LDS.  Scores are formed
// transposed, S^T = K Q^T, so each lane holds 4 keys x 1 query per 16x16 block: the row max
// is a 16-value in-lane max plus two cross-lane steps, the row sum stays lane-local until the
// epilogue, and the bf16 probabilities are already laid out as the B operand of
// O^T = V^T P^T (the packed value tiles store keys in the matching order).
//
// attn_f32_kernel: float32 path (fp32 inputs and outputs), one lane per query, keys through LDS.
#include <hip/hip_runtime.h>

#include <cmath>

#include "device_common.h"
#include "launch.h"

namespace vggt {
namespace {

struct AttnArgs {
  const void* q;
  const void* k;
  const void* v;
  const void* kpack;
  const void* vpack;
  void* out;
  int64_t T;
  int64_t rows_per_head;
  int segment_rows;
  int nkeys;       // valid keys per segment
  int n_plain;     // keys before the mean keys
  int nktiles;     // ceil(nkeys / 64)
  int slow_from;   // first tile that holds a mean key or padding
  float bias_s;    // added to the raw score q.k of a mean key (COUNT weighting), else 0
  float c_log2;    // tau * log2(e)
  int qtiles;      // query tiles per head
  int g2f;
  int qtiles_per_frame;
  int diag;
  IndexGeom g;
};

__device__ __forceinline__ float wave_max_across_groups(float x) {
  // Lanes l, l^16, l^32, l^48 hold the same query; combine them.
  x = fmaxf(x, __shfl_xor(x, 16));
  x = fmaxf(x, __shfl_xor(x, 32));
  return x;
}

__device__ __forceinline__ float wave_sum_across_groups(float x) {
  x += __shfl_xor(x, 16);
  x += __shfl_xor(x, 32);
  return x;
}

template <int QB, bool OUT_BF16>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(1, 1)))
void attn_bf16_kernel(AttnArgs a) {
  constexpr int WQ = 16 * QB;  // query rows per wave
  constexpr int BM = 4 * WQ;   // query rows per work-group
  // [buffer][0 = K tile, 1 = V tile][64 rows x 128 bytes], 16-byte chunks XOR-swizzled by row.
  __shared__ __attribute__((aligned(16))) uint8_t smem[2][2][kTile * 128];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int l16 = lane & 15, grp = lane >> 4;
  const int h = blockIdx.x / a.qtiles, qt = blockIdx.x - h * a.qtiles;

  int64_t row0, row_end, seg;
  if (a.g2f) {
    const int f = qt / a.qtiles_per_frame, qf = qt - f * a.qtiles_per_frame;
    row0 = int64_t(f) * a.g.L + int64_t(qf) * BM;
    row_end = int64_t(f + 1) * a.g.L;
    seg = f;
  } else {
    row0 = int64_t(qt) * BM;
    row_end = a.T;
    seg = 0;
  }
  const int64_t wrow0 = row0 + int64_t(wave) * WQ;

  const uint16_t* Q = static_cast<const uint16_t*>(a.q) + size_t(h) * size_t(a.T) * kHeadDim;
  const uint16_t* Kin = static_cast<const uint16_t*>(a.k) + size_t(h) * size_t(a.T) * kHeadDim;
  const uint16_t* Vin = static_cast<const uint16_t*>(a.v) + size_t(h) * size_t(a.T) * kHeadDim;
  const size_t seg_off = (size_t(h) * a.rows_per_head + size_t(seg) * a.segment_rows) * kHeadDim;
  const uint16_t* kseg = static_cast<const uint16_t*>(a.kpack) + seg_off;
  const uint16_t* vseg = static_cast<const uint16_t*>(a.vpack) + seg_off;

  // Q as the B operand of S^T = K Q^T: lane (l16, grp) holds query l16 of its block and
  // channels c*32 + grp*8 .. +7 for c = 0, 1.
  bf16x8_t qf[QB][2];
  float m_run[QB], l_run[QB];
  f32x4_t o[QB][4];
  const float c = a.c_log2;
#pragma unroll
  for (int qb = 0; qb < QB; ++qb) {
    const int64_t t = wrow0 + qb * 16 + l16;
    const bool valid = t < row_end;
#pragma unroll
    for (int cc = 0; cc < 2; ++cc) {
      uint4 raw = make_uint4(0, 0, 0, 0);
      if (valid) raw = *reinterpret_cast<const uint4*>(Q + size_t(t) * kHeadDim + cc * 32 + grp * 8);
      qf[qb][cc] = __builtin_bit_cast(bf16x8_t, raw);
    }
    // Diagonal prologue: a query whose own token is not in S starts with its self term,
    // m = tau*log2(e)*q.k_self, l = 1, O = v_self.
    const bool self = a.diag && valid && !token_kept(a.g, t);
    float dot = 0.f;
    uint4 kr[2] = {make_uint4(0, 0, 0, 0), make_uint4(0, 0, 0, 0)};
    if (self) {
      kr[0] = *reinterpret_cast<const uint4*>(Kin + size_t(t) * kHeadDim + grp * 8);
      kr[1] = *reinterpret_cast<const uint4*>(Kin + size_t(t) * kHeadDim + 32 + grp * 8);
    }
#pragma unroll
    for (int cc = 0; cc < 2; ++cc) {
      const uint4 qraw = __builtin_bit_cast(uint4, qf[qb][cc]);
      const uint32_t qw[4] = {qraw.x, qraw.y, qraw.z, qraw.w};
      const uint32_t kw[4] = {kr[cc].x, kr[cc].y, kr[cc].z, kr[cc].w};
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        dot = fmaf(__uint_as_float(qw[i] << 16), __uint_as_float(kw[i] << 16), dot);
        dot = fmaf(__uint_as_float(qw[i] & 0xffff0000u), __uint_as_float(kw[i] & 0xffff0000u), dot);
      }
    }
    dot = wave_sum_across_groups(dot);
    m_run[qb] = self ? dot * c : -INFINITY;
    l_run[qb] = (self && grp == 0) ? 1.f : 0.f;
#pragma unroll
    for (int db = 0; db < 4; ++db) {
      f32x4_t init = {0.f, 0.f, 0.f, 0.f};
      if (self) {
        const uint2 vr = *reinterpret_cast<const uint2*>(Vin + size_t(t) * kHeadDim + db * 16 + grp * 4);
        init[0] = __uint_as_float(vr.x << 16);
        init[1] = __uint_as_float(vr.x & 0xffff0000u);
        init[2] = __uint_as_float(vr.y << 16);
        init[3] = __uint_as_float(vr.y & 0xffff0000u);
      }
      o[qb][db] = init;
    }
  }

  // Global -> LDS staging of one tile: 512 chunks of 16 bytes per tensor, 2 per thread.
  auto load_tile = [&](int j, uint4 (&kr)[2], uint4 (&vr)[2]) {
    const uint16_t* kt = kseg + size_t(j) * kTile * kHeadDim;
    const uint16_t* vt = vseg + size_t(j) * kTile * kHeadDim;
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int e = tid + 256 * i;
      kr[i] = *reinterpret_cast<const uint4*>(kt + e * 8);
      vr[i] = *reinterpret_cast<const uint4*>(vt + e * 8);
    }
  };
  auto store_tile = [&](int b, const uint4 (&kr)[2], const uint4 (&vr)[2]) {
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int e = tid + 256 * i;
      const int row = e >> 3, ch = e & 7;
      const int off = row * 128 + ((ch ^ (row & 7)) << 4);
      *reinterpret_cast<uint4*>(&smem[b][0][off]) = kr[i];
      *reinterpret_cast<uint4*>(&smem[b][1][off]) = vr[i];
    }
  };

  const int nkt = a.nktiles;
  {
    uint4 kr[2], vr[2];
    load_tile(0, kr, vr);
    store_tile(0, kr, vr);
  }
  __syncthreads();

  for (int j = 0; j < nkt; ++j) {
    const int b = j & 1;
    uint4 kr[2], vr[2];
    const bool more = j + 1 < nkt;
    if (more) load_tile(j + 1, kr, vr);

    // ---- S^T = K Q^T for 64 keys x WQ queries ----
    f32x4_t s[QB][4];
#pragma unroll
    for (int kb = 0; kb < 4; ++kb) {
      const int row = kb * 16 + l16;
      const bf16x8_t k0 = *reinterpret_cast<const bf16x8_t*>(&smem[b][0][row * 128 + (((0 + grp) ^ (row & 7)) << 4)]);
      const bf16x8_t k1 = *reinterpret_cast<const bf16x8_t*>(&smem[b][0][row * 128 + (((4 + grp) ^ (row & 7)) << 4)]);
#pragma unroll
      for (int qb = 0; qb < QB; ++qb) {
        f32x4_t acc = {0.f, 0.f, 0.f, 0.f};
        acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(k0, qf[qb][0], acc, 0, 0, 0);
        acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(k1, qf[qb][1], acc, 0, 0, 0);
        s[qb][kb] = acc;
      }
    }

    // ---- mean-key bias and padding mask (only the last few tiles) ----
    if (j >= a.slow_from) {
#pragma unroll
      for (int kb = 0; kb < 4; ++kb) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int key = j * kTile + kb * 16 + grp * 4 + i;
          const float add = key >= a.nkeys ? -INFINITY : (key >= a.n_plain ? a.bias_s : 0.f);
#pragma unroll
          for (int qb = 0; qb < QB; ++qb) s[qb][kb][i] += add;
        }
      }
    }

    // ---- online softmax ----
    bf16x8_t pf[QB][2];
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) {
      float mx = s[qb][0][0];
#pragma unroll
      for (int kb = 0; kb < 4; ++kb)
#pragma unroll
        for (int i = 0; i < 4; ++i) mx = fmaxf(mx, s[qb][kb][i]);
      mx = wave_max_across_groups(mx);
      const float m_new = fmaxf(m_run[qb], mx * c);
      const float alpha = __builtin_amdgcn_exp2f(m_run[qb] - m_new);
      m_run[qb] = m_new;
      float lsum = 0.f;
      float p[4][4];
#pragma unroll
      for (int kb = 0; kb < 4; ++kb)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          p[kb][i] = __builtin_amdgcn_exp2f(fmaf(s[qb][kb][i], c, -m_new));
          lsum += p[kb][i];
        }
      l_run[qb] = l_run[qb] * alpha + lsum;
#pragma unroll
      for (int db = 0; db < 4; ++db) o[qb][db] *= alpha;
#pragma unroll
      for (int h2 = 0; h2 < 2; ++h2) {
        const uint4 w = make_uint4(pack_bf16x2(p[2 * h2][0], p[2 * h2][1]), pack_bf16x2(p[2 * h2][2], p[2 * h2][3]),
                                   pack_bf16x2(p[2 * h2 + 1][0], p[2 * h2 + 1][1]),
                                   pack_bf16x2(p[2 * h2 + 1][2], p[2 * h2 + 1][3]));
        pf[qb][h2] = __builtin_bit_cast(bf16x8_t, w);
      }
    }

    // ---- O^T += V^T P^T ----
#pragma unroll
    for (int db = 0; db < 4; ++db) {
      const int row = db * 16 + l16;
      const bf16x8_t v0 = *reinterpret_cast<const bf16x8_t*>(&smem[b][1][row * 128 + (((0 + grp) ^ (row & 7)) << 4)]);
      const bf16x8_t v1 = *reinterpret_cast<const bf16x8_t*>(&smem[b][1][row * 128 + (((4 + grp) ^ (row & 7)) << 4)]);
#pragma unroll
      for (int qb = 0; qb < QB; ++qb) {
        o[qb][db] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(v0, pf[qb][0], o[qb][db], 0, 0, 0);
        o[qb][db] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(v1, pf[qb][1], o[qb][db], 0, 0, 0);
      }
    }

    if (more) store_tile(b ^ 1, kr, vr);
    __syncthreads();
  }

  // ---- epilogue: O / l ----
#pragma unroll
  for (int qb = 0; qb < QB; ++qb) {
    const float l = wave_sum_across_groups(l_run[qb]);
    const float inv = 1.f / l;
    const int64_t t = wrow0 + qb * 16 + l16;
    if (t >= row_end) continue;
#pragma unroll
    for (int db = 0; db < 4; ++db) {
      const size_t off = (size_t(h) * size_t(a.T) + size_t(t)) * kHeadDim + db * 16 + grp * 4;
      const f32x4_t r = o[qb][db] * inv;
      if constexpr (OUT_BF16) {
        *reinterpret_cast<uint2*>(static_cast<uint16_t*>(a.out) + off) =
            make_uint2(pack_bf16x2(r[0], r[1]), pack_bf16x2(r[2], r[3]));
      } else {
        *reinterpret_cast<f32x4_t*>(static_cast<float*>(a.out) + off) = r;
      }
    }
  }
}

// float32 path: one wave per work-group, one lane per query row, keys and values through LDS
// (every lane reads the same key row, an LDS broadcast).
__global__ __launch_bounds__(64) void attn_f32_kernel(AttnArgs a) {
  constexpr int BM = 64;
  __shared__ float ks[kTile][kHeadDim];
  __shared__ float vs[kTile][kHeadDim];
  const int lane = threadIdx.x;
  const int h = blockIdx.x / a.qtiles, qt = blockIdx.x - h * a.qtiles;
  int64_t row0, row_end, seg;
  if (a.g2f) {
    const int f = qt / a.qtiles_per_frame, qf = qt - f * a.qtiles_per_frame;
    row0 = int64_t(f) * a.g.L + int64_t(qf) * BM;
    row_end = int64_t(f + 1) * a.g.L;
    seg = f;
  } else {
    row0 = int64_t(qt) * BM;
    row_end = a.T;
    seg = 0;
  }
  const int64_t t = row0 + lane;
  const bool valid = t < row_end;
  const float* Q = static_cast<const float*>(a.q) + size_t(h) * size_t(a.T) * kHeadDim;
  const float* Kin = static_cast<const float*>(a.k) + size_t(h) * size_t(a.T) * kHeadDim;
  const float* Vin = static_cast<const float*>(a.v) + size_t(h) * size_t(a.T) * kHeadDim;
  const size_t seg_off = (size_t(h) * a.rows_per_head + size_t(seg) * a.segment_rows) * kHeadDim;
  const float* kseg = static_cast<const float*>(a.kpack) + seg_off;
  const float* vseg = static_cast<const float*>(a.vpack) + seg_off;

  float q[kHeadDim], o[kHeadDim];
#pragma unroll
  for (int d = 0; d < kHeadDim; ++d) q[d] = valid ? Q[size_t(t) * kHeadDim + d] : 0.f;
  const float c = a.c_log2;
  float m_run = -INFINITY, l_run = 0.f;
  const bool self = a.diag && valid && !token_kept(a.g, t);
  if (self) {
    float dot = 0.f;
#pragma unroll
    for (int d = 0; d < kHeadDim; ++d) dot = fmaf(q[d], Kin[size_t(t) * kHeadDim + d], dot);
    m_run = dot * c;
    l_run = 1.f;
  }
#pragma unroll
  for (int d = 0; d < kHeadDim; ++d) o[d] = self ? Vin[size_t(t) * kHeadDim + d] : 0.f;

  for (int j = 0; j < a.nktiles; ++j) {
    __syncthreads();
    const float4* ksrc = reinterpret_cast<const float4*>(kseg + size_t(j) * kTile * kHeadDim);
    const float4* vsrc = reinterpret_cast<const float4*>(vseg + size_t(j) * kTile * kHeadDim);
    for (int e = lane; e < kTile * kHeadDim / 4; e += 64) {
      reinterpret_cast<float4*>(&ks[0][0])[e] = ksrc[e];
      reinterpret_cast<float4*>(&vs[0][0])[e] = vsrc[e];
    }
    __syncthreads();
    float sc[kTile];
    float mx = -INFINITY;
#pragma unroll
    for (int kk = 0; kk < kTile; ++kk) {
      float dot = 0.f;
#pragma unroll
      for (int d = 0; d < kHeadDim; ++d) dot = fmaf(q[d], ks[kk][d], dot);
      const int key = j * kTile + kk;
      if (key >= a.nkeys) dot = -INFINITY;
      else if (key >= a.n_plain) dot += a.bias_s;
      sc[kk] = dot;
      mx = fmaxf(mx, dot);
    }
    const float m_new = fmaxf(m_run, mx * c);
    const float alpha = __builtin_amdgcn_exp2f(m_run - m_new);
    m_run = m_new;
    l_run *= alpha;
#pragma unroll
    for (int d = 0; d < kHeadDim; ++d) o[d] *= alpha;
#pragma unroll
    for (int kk = 0; kk < kTile; ++kk) {
      const float p = __builtin_amdgcn_exp2f(fmaf(sc[kk], c, -m_new));
      l_run += p;
#pragma unroll
      for (int d = 0; d < kHeadDim; ++d) o[d] = fmaf(p, vs[kk][d], o[d]);
    }
  }
  if (valid) {
    const float inv = 1.f / l_run;
    float* out = static_cast<float*>(a.out) + (size_t(h) * size_t(a.T) + size_t(t)) * kHeadDim;
#pragma unroll
    for (int d = 0; d < kHeadDim; d += 4)
      *reinterpret_cast<float4*>(out + d) = make_float4(o[d] * inv, o[d + 1] * inv, o[d + 2] * inv, o[d + 3] * inv);
  }
}

}  // namespace

hipError_t launch_attend(const vggt_attn_plan_s& p, const void* q, const void* k, const void* v,
                         void* out, const void* ws, hipStream_t stream) {
  const char* base = static_cast<const char*>(ws);
  AttnArgs a{};
  a.q = q;
  a.k = k;
  a.v = v;
  a.kpack = base + p.layout.off_kpack;
  a.vpack = base + p.layout.off_vpack;
  a.out = out;
  a.T = p.T;
  a.rows_per_head = p.rows_per_head;
  a.segment_rows = int(p.segment_rows);
  a.nkeys = int(p.keys_per_segment);
  a.n_plain = int(p.n_plain);
  a.nktiles = int(p.segment_rows / kTile);
  a.slow_from = int(p.n_plain / kTile);
  const double tau = 1.0 / std::sqrt(double(p.head_dim));
  // COUNT: logit += ln|D_f|  <=>  raw score q.k += ln|D_f| / tau.
  a.bias_s = (p.mean_count && p.M > 0) ? float(std::log(double(p.dropped)) / tau) : 0.f;
  a.c_log2 = float(tau * 1.4426950408889634);
  a.g2f = p.g2f ? 1 : 0;
  a.diag = p.diag ? 1 : 0;
  a.g = p.geom;

  if (p.in_dtype == VGGT_ATTN_FP32) {
    constexpr int BM = 64;
    if (p.g2f) {
      a.qtiles_per_frame = int((p.L + BM - 1) / BM);
      a.qtiles = a.qtiles_per_frame * p.frames;
    } else {
      a.qtiles = int((p.T + BM - 1) / BM);
    }
    const unsigned blocks = unsigned(int64_t(a.qtiles) * p.heads);
    hipLaunchKernelGGL(attn_f32_kernel, dim3(blocks), dim3(64), 0, stream, a);
    return hipGetLastError();
  }

  // bf16: 64 queries per wave for the global forms (K/V traffic halves against 32), 32 per
  // wave under G2F (1374-token frames pad to 1408 instead of 1536 query rows).
  const bool small = p.g2f;
  const int BM = small ? 128 : 256;
  if (p.g2f) {
    a.qtiles_per_frame = int((p.L + BM - 1) / BM);
    a.qtiles = a.qtiles_per_frame * p.frames;
  } else {
    a.qtiles = int((p.T + BM - 1) / BM);
  }
  const unsigned blocks = unsigned(int64_t(a.qtiles) * p.heads);
  const bool ob = p.out_dtype == VGGT_ATTN_BF16;
  if (small) {
    if (ob) hipLaunchKernelGGL((attn_bf16_kernel<2, true>), dim3(blocks), dim3(256), 0, stream, a);
    else hipLaunchKernelGGL((attn_bf16_kernel<2, false>), dim3(blocks), dim3(256), 0, stream, a);
  } else {
    if (ob) hipLaunchKernelGGL((attn_bf16_kernel<4, true>), dim3(blocks), dim3(256), 0, stream, a);
    else hipLaunchKernelGGL((attn_bf16_kernel<4, false>), dim3(blocks), dim3(256), 0, stream, a);
  }
  return hipGetLastError();
}

}  // namespace vggt
