// Attention stage on gfx950: out = softmax(Q K^T / sqrt(d)) V over packed keys, with the
// diagonal self term and the mean keys folded into the same running max and sum.
//
// Operation: "AVGGT: Rethinking Global Attention for Accelerating VGGT" (papernotes.org CVPR
// 2026 notes), 关键设计 2 (the attention equation over the kept set S), 关键设计 3 (diagonal
// self term and mean K/V share one softmax normalisation), 关键设计 1 (Global-to-Frame: keys of
// a query are the tokens of its own frame), ablation table (G2M: a single mean key); "RegimeVGGT
// ..." (papernotes.org NeurIPS 2026 notes), 关键设计 2 (a key standing for g tokens carries +ln g
// on its logit -- used for the COUNT weighting of the mean keys), 关键设计 3 (per-frame phase of
// the sampling grid, which sets |D_f| and so the bias of each frame's mean key).
//
// attn_bf16_kernel: flash-style forward on the bf16 matrix cores (v_mfma_f32_16x16x32_bf16,
// float32 accumulation; in the opt-in f16 score form Q K^T runs on v_mfma_f32_16x16x32_f16 with
// the softmax scale folded into Q).  A work-group of 4 waves owns BM = 4*16*QB query rows of one head and
// streams the key segment -- the packed workspace, or under G2F the frame's own rows of K and
// V read in place -- in 64-key tiles through LDS filled by direct global->LDS buffer loads.
// Work items are numbered XCD by XCD, so that neighbouring items share an L2.  Scores are
// formed transposed, S^T = K Q^T, so each lane holds 4 keys x 1 query per 16x16 block: the row
// max is a 16-value in-lane max plus two cross-lane steps, the row sum stays lane-local until
// the epilogue, and the bf16 probabilities are already laid out as the B operand of
// O^T = V^T P^T (packed value tiles store keys in the matching order; in-place value tiles are
// read transposed out of LDS in that order).
//
// attn_f32_kernel: float32 path (fp32 inputs and outputs), one lane per query, keys through LDS.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <type_traits>

#include "device_common.h"
#include "launch.h"


// Row-sum method of the bf16 kernel: 0 = matrix cores in the exact-scale forms without key
// biases, VALU dot2 in the others (the default), 1 = matrix cores everywhere, 2 = VALU dot2
// everywhere (for timing comparisons).
#ifndef VGGT_SUM_MODE
#define VGGT_SUM_MODE 0
#endif

namespace vggt {
namespace {

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef _Float16 f16x8_t __attribute__((ext_vector_type(8)));
typedef short i16x4_t __attribute__((ext_vector_type(4)));
typedef short i16x8_t __attribute__((ext_vector_type(8)));
// s_waitcnt immediate for vmcnt(0) with expcnt and lgkmcnt left at their maxima (gfx9 encoding).
constexpr int kWaitVmcnt0 = 0x0F70;
constexpr bf16x2_t kOnes2 = {(__bf16)1.0f, (__bf16)1.0f};
// Word 3 of a raw buffer descriptor on gfx9-family parts (gfx950 included): 32-bit data format,
// no swizzle, so that offsets are plain byte offsets range-checked against num_records.
constexpr int kBufferWord3 = 0x00020000;

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
  // COUNT bias of mean key m: slot s = (m + mean_off) % mean_run indexes the mean frames of one
  // run of grid phases (per-frame scope under the phase shift; otherwise one slot).
  int mean_off, mean_run;
  float mean_bias_s[kMaxPhases];     // raw-score units, ln(n)/tau (0 for UNIT weighting)
  float mean_bias_log2[kMaxPhases];  // the same in log2 units, log2(n) (PRESCALE_Q path)
  float c_log2;    // tau * log2(e)
  float weight_shift, weight_scale;  // weights are 2^-weight_shift (= weight_scale) smaller
  const uint32_t* kmax;  // f16 score form: bf16 bits of each head's largest packed |k|
  const float* kbias;    // size-aware keys: bias of each packed key row (raw-score units), else null
  const float* logsize;  // size-aware keys: log g per token (for the diagonal term), else null
  float size_scale;      // sqrt(d): log g -> raw-score units
  int64_t split_from;    // first work item of the split last round
  int nsplit;            // key-range pieces per split item (1: none)
  float* part;           // [split items * nsplit][BM][kPartRow] partial states of the pieces
  int qtiles;      // query tiles per head
  int g2f;
  int qtiles_per_frame;
  int diag;
  IndexGeom g;
};

// Query rows [row0, row_end) of a work item of BM rows, its head and its key segment.
struct ItemRows {
  int h;
  int64_t row0, row_end, seg;
};
__device__ __forceinline__ ItemRows item_rows(const AttnArgs& a, int64_t item, int BM) {
  ItemRows r;
  r.h = int(item / a.qtiles);
  const int qt = int(item - int64_t(r.h) * a.qtiles);
  if (a.g2f) {
    const int f = qt / a.qtiles_per_frame, qf = qt - f * a.qtiles_per_frame;
    r.row0 = int64_t(f) * a.g.L + int64_t(qf) * BM;
    r.row_end = int64_t(f + 1) * a.g.L;
    r.seg = f;
  } else {
    r.row0 = int64_t(qt) * BM;
    r.row_end = a.T;
    r.seg = 0;
  }
  return r;
}

// Work item of block b of nb: block b runs on XCD b % kXcds, so renumbering the blocks of
// XCD x to a contiguous range of items (the first nb % kXcds XCDs take one item more) keeps
// items that are adjacent in item order -- the query tiles of one frame under G2F, which read
// the same key segment -- on one XCD, where they share one L2 copy of that segment (5% less
// time at 200 frames).  The global forms, where every work-group streams its head's segment,
// measured within 0.5% either way.
__device__ __forceinline__ int64_t xcd_item(unsigned b, unsigned nb) {
  const unsigned x = b % kXcds, i = b / kXcds, q = nb / kXcds, r = nb % kXcds;
  return x < r ? int64_t(x) * (q + 1) + i : int64_t(r) * (q + 1) + int64_t(x - r) * q + i;
}

// Logit bias of mean key m (0 <= m < M): it depends only on the grid phase of the frame the
// key stands for, i.e. on the key's slot within a run of phases.
__device__ __forceinline__ float mean_bias(const AttnArgs& a, const float (&tab)[kMaxPhases], int m) {
  return a.mean_run > 1 ? pick(tab, (m + a.mean_off) % a.mean_run) : tab[0];
}

// This file is compiled with -fno-honor-nans (scores are never NaN; infinities are honoured),
// so fmaxf lowers to plain v_max_f32 and chains of it fuse into v_max3_f32.
__device__ __forceinline__ float vmax(float a, float b) { return fmaxf(a, b); }

// Lanes l, l^16, l^32 and l^48 hold the same query.  v_permlane16_swap(x, x) leaves each
// lane holding its own value and its xor-16 partner's in the two results; v_permlane32_swap
// does the same for the xor-32 partner.  Pure VALU, no LDS round trip.
__device__ __forceinline__ float group_max(float x) {
  const auto p = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  x = vmax(__uint_as_float(p[0]), __uint_as_float(p[1]));
  const auto q = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return vmax(__uint_as_float(q[0]), __uint_as_float(q[1]));
}
__device__ __forceinline__ float group_sum(float x) {
  const auto p = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  x = __uint_as_float(p[0]) + __uint_as_float(p[1]);
  const auto q = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(q[0]) + __uint_as_float(q[1]);
}

// SPLIT: the blocks run key-range pieces of the split last round of work items and store
// partial softmax states (merge_pieces_kernel finishes them); otherwise one block = one item.
// INPLACE (G2F): the keys of a frame are its tokens, so K and V tiles are copied from the input
// tensors instead of the packed workspace, and V is read transposed out of LDS.
template <int QB, int WPE, bool OUT_BF16, bool PRESCALE_Q, bool LOGSIZE, bool SPLIT, bool INPLACE>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(WPE, WPE)))
void attn_bf16_kernel(AttnArgs a) {
  static_assert(!(LOGSIZE && PRESCALE_Q), "size-aware keys use the exact scale");
  static_assert(!(SPLIT && LOGSIZE), "split pieces have no key biases");
  static_assert(!(INPLACE && PRESCALE_Q), "the f16 score form reads f16 keys from the packed workspace");
  constexpr bool kExactScale = !PRESCALE_Q;
  constexpr int WQ = 16 * QB;  // query rows per wave
  constexpr int BM = 4 * WQ;   // query rows per work-group
  // Two K tiles and two V tiles of 64 rows x 128 bytes; 16-byte chunks XOR-swizzled by row so
  // that the 16-byte operand reads of 8 consecutive lanes hit distinct banks.  The K stream runs
  // one tile ahead of the V stream: step j reads K tile j+1 (scores of the next tile) and V tile
  // j (output of the current tile).
  // Four separate LDS objects (not one array), so that the copy into one buffer is known not
  // to alias reads of the others and no wait is placed in front of those reads.
  __shared__ __attribute__((aligned(16))) uint8_t kbuf0[kTile * 128];
  __shared__ __attribute__((aligned(16))) uint8_t kbuf1[kTile * 128];
  __shared__ __attribute__((aligned(16))) uint8_t vbuf0[kTile * 128];
  __shared__ __attribute__((aligned(16))) uint8_t vbuf1[kTile * 128];
  // Size-aware keys: the 64 key biases of a K tile travel with it (same schedule, same parity).
  __shared__ __attribute__((aligned(16))) float bbuf0[kTile];
  __shared__ __attribute__((aligned(16))) float bbuf1[kTile];
  auto kbuf = [&](auto par) -> uint8_t* { if constexpr (decltype(par)::value == 0) return kbuf0; else return kbuf1; };
  auto vbuf = [&](auto par) -> uint8_t* { if constexpr (decltype(par)::value == 0) return vbuf0; else return vbuf1; };
  auto bbuf = [&](auto par) -> float* { if constexpr (decltype(par)::value == 0) return bbuf0; else return bbuf1; };

  // The wave index is uniform: keeping it in a scalar register makes every LDS destination of
  // the tile copies a scalar (m0) value.
  const int tid = threadIdx.x, lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int l16 = lane & 15, grp = lane >> 4;
  // Key tiles [tb, tb + nkt) of the segment: all of them, or one piece of a split item.  (The
  // whole-item form keeps the bound a kernel argument: a computed bound costs registers.)
  // A piece sees its tiles as 0 .. nkt-1: the segment pointers move to its first tile and the
  // tile/key bounds are rebased once (the tile offset itself never enters the loop).
  int64_t item = SPLIT ? 0 : xcd_item(blockIdx.x, gridDim.x);
  int piece = 0, tb = 0, nkt = a.nktiles;
  int slow_from = a.slow_from, nkeys = a.nkeys, n_plain = a.n_plain;
  if constexpr (SPLIT) {
    item = a.split_from + blockIdx.x / a.nsplit;
    piece = int(blockIdx.x % a.nsplit);
    tb = int(int64_t(piece) * a.nktiles / a.nsplit);
    nkt = int(int64_t(piece + 1) * a.nktiles / a.nsplit) - tb;
    slow_from -= tb;
    nkeys -= tb * kTile;
    n_plain -= tb * kTile;
  }
  const ItemRows ir = item_rows(a, item, BM);
  const int h = ir.h;
  const int64_t row0 = ir.row0, row_end = ir.row_end, seg = ir.seg;
  const int64_t wrow0 = row0 + int64_t(wave) * WQ;

  const uint16_t* Q = static_cast<const uint16_t*>(a.q) + size_t(h) * size_t(a.T) * kHeadDim;
  const uint16_t* Kin = static_cast<const uint16_t*>(a.k) + size_t(h) * size_t(a.T) * kHeadDim;
  const uint16_t* Vin = static_cast<const uint16_t*>(a.v) + size_t(h) * size_t(a.T) * kHeadDim;
  // Key rows of this item from kseg/vseg on: the packed segment, or (INPLACE) the tokens from
  // the first key of the item's range, of which kv_rows remain in the head's tensor (a tile
  // that runs past them is cut by its copy's range check, which lands zeros; they are masked).
  const uint16_t* kseg;
  const uint16_t* vseg;
  int64_t kv_rows;
  if constexpr (INPLACE) {
    const int64_t first = (a.g2f ? seg * a.g.L : 0) + int64_t(tb) * kTile;
    kseg = Kin + size_t(first) * kHeadDim;
    vseg = Vin + size_t(first) * kHeadDim;
    kv_rows = a.T - first;
  } else {
    const size_t seg_off = (size_t(h) * a.rows_per_head + size_t(seg) * a.segment_rows + size_t(tb) * kTile) * kHeadDim;
    kseg = static_cast<const uint16_t*>(a.kpack) + seg_off;
    vseg = static_cast<const uint16_t*>(a.vpack) + seg_off;
    kv_rows = int64_t(a.nktiles) * kTile;
  }
  const float* bseg = LOGSIZE ? a.kbias + size_t(seg) * a.segment_rows + size_t(tb) * kTile : nullptr;

  // Q as the B operand of S^T = K Q^T: lane (l16, grp) holds query l16 of its block and
  // channels cc*32 + grp*8 .. +7 for cc = 0, 1.
  bf16x8_t qf[QB][2];
  // Running max and lane-partial row sum.  From tile 0 on, the running max m is kept as the
  // exp2 offset -(m + w) in log2 units (m c for raw scores s, plus the weight shift w below): the
  // exact form adds it to c s in the exp argument, the f16 score form starts its QK^T chains
  // from it.  Before tile 0 the slot holds the diagonal term's logit (raw or log2 units).
  float m_run[QB];
  f32x4_t o[QB][4];
  // Row sums, two ways.  kMfmaSum: on the matrix cores, l^T += 1 P^T with an all-ones A operand,
  // two 16x16x32 products per block beside the 8 of PV, so every lane holds its query's whole
  // sum (4 equal copies).  Else: VALU dot2 instructions into a lane-partial sum (summed over the
  // lane group at the end).  The dot2 instructions run on the matrix pipe of gfx950 -- each one
  // waits for the MFMA in flight to drain -- so the products win where the registers allow them:
  // the exact scale at 800 frames (830 -> 818 ms in one session, 800 -> 789 in another) and
  // dense (7.24 -> 6.95 ms).  The f16 score form (its chain-start tuples stay live) and the
  // size-aware keys (bias tiles) spill into their loops with the 12 extra registers and keep
  // dot2 (787 against 811 ms and 877 against 890 ms at 800 frames).
  constexpr bool kMfmaSum = VGGT_SUM_MODE == 1 || (VGGT_SUM_MODE == 0 && !PRESCALE_Q && !LOGSIZE);
  f32x4_t l_acc[QB];
  float l_run[QB];
  const bf16x8_t ones8 = {(__bf16)1.0f, (__bf16)1.0f, (__bf16)1.0f, (__bf16)1.0f,
                          (__bf16)1.0f, (__bf16)1.0f, (__bf16)1.0f, (__bf16)1.0f};
  // Two ways to reach log2 units.  Exact (default): Q is used as given, scores are in units of
  // q.k, and the exp2 argument is c s plus the offset, c = tau*log2(e).
  // f16 score form (PRESCALE_Q plan flag): the packed keys of head h are f16(k * 2^-e_h) and Q
  // is scaled by c * 2^e_h once and rounded to f16, so that the f16 matrix cores deliver scores
  // in log2 units and the running max enters their accumulator: no multiply per score.  The
  // rounding of Q perturbs each logit term by a relative 2^-11 at most.
  const float c = a.c_log2;
  const int kexp = PRESCALE_Q ? key_scale_exp(a.kmax[h]) : 0;
  const float qscale = kExactScale ? 1.f : __builtin_amdgcn_ldexpf(c, kexp);  // applied to Q at load
  const float kscale = kExactScale ? 1.f : __builtin_amdgcn_ldexpf(1.f, -kexp);  // of the packed keys
  const float sc = kExactScale ? c : 1.f;       // applied to scores at the exp
  // Weight shift w (from the plan): every weight is taken 2^w times smaller,
  // p = 2^(c (s - m) - w), a common factor that cancels in O / l (bf16 and fp32 keep the same
  // relative rounding while p stays far above 2^-126).  It moves the overflow test below from
  // one octave above the running max to w + 1 octaves, so the max that the first tile sets is
  // almost never raised.
  const float shift = a.weight_shift;
  const float shift_scale = a.weight_scale;  // 2^-w
  // Raw Q fragments of every query block, as straight-line range-checked buffer loads (rows
  // past the head's T read as zero; rows past the item's end are computed but never stored), so
  // that they are in flight together with the first tile copies issued below.
  const auto qrsrc = __builtin_amdgcn_make_buffer_rsrc(const_cast<uint16_t*>(Q), 0, int(a.T * 128), kBufferWord3);
  uint4 qraw[QB][2];
#pragma unroll
  for (int qb = 0; qb < QB; ++qb)
#pragma unroll
    for (int cc = 0; cc < 2; ++cc)
      qraw[qb][cc] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(
          qrsrc, int(wrow0 + qb * 16 + l16) * 128 + cc * 64 + grp * 16, 0, 0));

  // Global -> LDS copy of one 64x128-byte tile with buffer_load_dwordx4 ... lds: lane L of a wave
  // instruction writes the 16 bytes at LDS base + 16*L, so each lane fetches the global chunk
  // that belongs at that position of the swizzled layout.  8 wave instructions per tile (2 per
  // wave); no registers are used and completion is awaited (vmcnt) before the step's barrier.
  // The tile's address lives in a buffer descriptor (scalar registers, advanced per tile); the
  // lane's byte offset within the tile is the same for every tile, so a copy costs no vector ALU
  // work.  Instruction i fills KB i*4 + wave of the tile: rows blk*8 + (lane >> 3), whose low
  // three bits are lane >> 3, so both instructions use the same chunk swizzle.  K tiles (and
  // packed V tiles) swizzle 16-byte chunks by row & 7; row-major V tiles of the INPLACE form by
  // row & 6, which spreads their transposed reads over the banks.
  const int k_off = (wave * 8 + (lane >> 3)) * 128 + (((lane & 7) ^ (lane >> 3)) << 4);
  const int v_off = INPLACE ? (wave * 8 + (lane >> 3)) * 128 + (((lane & 7) ^ ((lane >> 3) & 6)) << 4) : k_off;
  auto async_tile = [&](const uint16_t* base, int j, uint8_t* buf, int v_tile) {
    const int lane_off = INPLACE && v_tile ? v_off : k_off;
    const int rows = INPLACE ? int(min(kv_rows - int64_t(j) * kTile, int64_t(kTile))) : kTile;
    const auto rsrc = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<uint16_t*>(base + size_t(j) * kTile * kHeadDim), 0, rows * 128, kBufferWord3);
#pragma unroll
    for (int i = 0; i < 2; ++i)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(
          rsrc, (__attribute__((address_space(3))) void*)(buf + (i * 4 + wave) * 1024), 16,
          lane_off + i * 4096, 0, 0, 0);
  };
  // Key biases of tile j: wave 0 copies the 64 floats with 4-byte loads (lane L lands at LDS
  // base + 4*L).
  auto async_bias = [&](int j, float* buf) {
    if constexpr (LOGSIZE) {
      if (wave == 0) {
        const auto rsrc = __builtin_amdgcn_make_buffer_rsrc(
            const_cast<float*>(bseg + size_t(j) * kTile), 0, kTile * 4, kBufferWord3);
        __builtin_amdgcn_raw_ptr_buffer_load_lds(rsrc, (__attribute__((address_space(3))) void*)buf, 4,
                                                 lane * 4, 0, 0, 0);
      }
    }
  };
  auto wait_tiles = [&]() { __builtin_amdgcn_s_waitcnt(kWaitVmcnt0); };
  // 16-byte operand read of LDS row `row`, chunk `ch` (undoing the swizzle).
  auto lds_frag = [&](const uint8_t* buf, int row, int ch) {
    return *reinterpret_cast<const bf16x8_t*>(&buf[row * 128 + ((ch ^ (row & 7)) << 4)]);
  };

  // K (or packed V) operand fragments of a tile: read once per step, shared by every query block.
  auto k_frags = [&](const uint8_t* kb, bf16x8_t (&kf)[4][2]) {
#pragma unroll
    for (int k4 = 0; k4 < 4; ++k4) {
      kf[k4][0] = lds_frag(kb, k4 * 16 + l16, grp);
      kf[k4][1] = lds_frag(kb, k4 * 16 + l16, 4 + grp);
    }
  };
  // V^T operand fragments from a row-major V tile (INPLACE) with ds_read_b64_tr_b16.  Within
  // each 16-lane group, lane j of the instruction reads 4 consecutive values of its own address
  // (row j of a 16 x 4 block) and lane i receives column i & 3 of rows 4r + (i >> 2), r = 0..3.
  // Lane j = (l16 of this lane) therefore addresses key 4*grp + (j >> 2) (+ 16u + 32h) and the
  // channels db*16 + 4*(j & 3) .. +3, so that lane i ends up with channel db*16 + i of keys
  // 4*grp + r, the order in which P leaves the score blocks; u = 1 gives the keys 16 further on.
  const int vt_row = 4 * grp + (l16 >> 2);
  int vt_addr[4];
#pragma unroll
  for (int db = 0; db < 4; ++db)
    vt_addr[db] = vt_row * 128 + (((2 * db + ((l16 >> 1) & 1)) ^ (vt_row & 6)) << 4) + 8 * (l16 & 1);
  auto v_frags = [&](const uint8_t* vb, bf16x8_t (&vf)[4][2]) {
    if constexpr (!INPLACE) {
      k_frags(vb, vf);
    } else {
#pragma unroll
      for (int db = 0; db < 4; ++db) {
#pragma unroll
        for (int hh = 0; hh < 2; ++hh) {
          const uint8_t* p0 = vb + vt_addr[db] + hh * 4096;
          const i16x4_t lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
              (__attribute__((address_space(3))) i16x4_t*)(p0));
          const i16x4_t hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
              (__attribute__((address_space(3))) i16x4_t*)(p0 + 2048));
          vf[db][hh] = __builtin_bit_cast(bf16x8_t, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
        }
      }
    }
  };
  // S^T = K Q^T for 64 keys x the 16 queries of block qb: s[k4][i] is key k4*16 + grp*4 + i.
  // Exact mode starts each two-MFMA chain from a zero accumulator (an inline constant, so the
  // first MFMA reads no accumulator registers and the second takes its input straight from the
  // first); the running max is applied in the exp argument.  The f16 score form starts it from
  // `from` = -(m + w), so the scores leave the matrix core already shifted.
  // Size-aware keys start the chain from the keys' biases instead (read from LDS).
  auto scores_qb = [&](const bf16x8_t (&kf)[4][2], const float* bb, int qb, f32x4_t (&s)[4], float from) {
#pragma unroll
    for (int k4 = 0; k4 < 4; ++k4) {
      f32x4_t acc = {0.f, 0.f, 0.f, 0.f};
      if constexpr (PRESCALE_Q) {
        acc = f32x4_t{from, from, from, from};
        acc = __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8_t, kf[k4][0]),
                                                     __builtin_bit_cast(f16x8_t, qf[qb][0]), acc, 0, 0, 0);
        s[k4] = __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8_t, kf[k4][1]),
                                                       __builtin_bit_cast(f16x8_t, qf[qb][1]), acc, 0, 0, 0);
      } else {
        if constexpr (LOGSIZE) acc = *reinterpret_cast<const f32x4_t*>(bb + k4 * 16 + grp * 4);
        acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kf[k4][0], qf[qb][0], acc, 0, 0, 0);
        s[k4] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kf[k4][1], qf[qb][1], acc, 0, 0, 0);
      }
    }
  };
  // Mean-key bias and padding mask, only for the last tiles of the segment.
  auto bias_mask = [&](int j, f32x4_t (&s)[QB][4]) {
    if (j < slow_from) return;
#pragma unroll
    for (int k4 = 0; k4 < 4; ++k4) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int key = j * kTile + k4 * 16 + grp * 4 + i;
        float bias = 0.f;
        if (!INPLACE && key >= n_plain) {  // (a G2F segment has no mean keys)
          if constexpr (PRESCALE_Q) bias = mean_bias(a, a.mean_bias_log2, key - n_plain);
          else bias = mean_bias(a, a.mean_bias_s, key - n_plain);
        }
        const float add = key >= nkeys ? -INFINITY : bias;
#pragma unroll
        for (int qb = 0; qb < QB; ++qb) s[qb][k4][i] += add;
      }
    }
  };
  // In-lane max as two independent max3 chains, then the lane-group exchange.
  auto row_max = [&](const f32x4_t (&s)[4]) {
    float x = fmaxf(fmaxf(s[0][0], s[0][1]), s[0][2]);
    float y = fmaxf(fmaxf(s[2][0], s[2][1]), s[2][2]);
    x = fmaxf(fmaxf(x, s[0][3]), s[1][0]);
    y = fmaxf(fmaxf(y, s[2][3]), s[3][0]);
    x = fmaxf(fmaxf(x, s[1][1]), s[1][2]);
    y = fmaxf(fmaxf(y, s[3][1]), s[3][2]);
    return group_max(fmaxf(fmaxf(x, s[1][3]), fmaxf(y, s[3][3])));
  };
  // p = 2^(c s - c m - w) (exact) or 2^s' (f16 score form, s' already offset) rounded to bf16,
  // already in the B-operand layout of the PV product (the row sum is taken there too, on the
  // same rounded weights).
  // Returns the OR of the packed bf16 words: every p >= 0, so some p >= 2 (a score more than
  // w + 1 octaves above the running max) exactly when bit 14 of some half is set.
  auto probs_qb = [&](int qb, const f32x4_t (&s)[4], bf16x8_t (&pf)[2]) {
    const float off = m_run[qb];
    auto e = [&](float x) { return (__bf16)__builtin_amdgcn_exp2f(PRESCALE_Q ? x : fmaf(x, c, off)); };
    uint32_t bits = 0;
    float l = l_run[qb];
#pragma unroll
    for (int h2 = 0; h2 < 2; ++h2) {
      const f32x4_t& s0 = s[2 * h2];
      const f32x4_t& s1 = s[2 * h2 + 1];
      const bf16x8_t pv = {e(s0[0]), e(s0[1]), e(s0[2]), e(s0[3]), e(s1[0]), e(s1[1]), e(s1[2]), e(s1[3])};
      pf[h2] = pv;
      const uint4 w = __builtin_bit_cast(uint4, pv);
      bits |= w.x | w.y | w.z | w.w;
      if constexpr (!kMfmaSum) {
        l = __builtin_amdgcn_fdot2_f32_bf16(__builtin_shufflevector(pv, pv, 0, 1), kOnes2, l, false);
        l = __builtin_amdgcn_fdot2_f32_bf16(__builtin_shufflevector(pv, pv, 2, 3), kOnes2, l, false);
        l = __builtin_amdgcn_fdot2_f32_bf16(__builtin_shufflevector(pv, pv, 4, 5), kOnes2, l, false);
        l = __builtin_amdgcn_fdot2_f32_bf16(__builtin_shufflevector(pv, pv, 6, 7), kOnes2, l, false);
      }
    }
    if constexpr (!kMfmaSum) l_run[qb] = l;
    return bits;
  };
  auto accumulate_qb = [&](const bf16x8_t (&vf)[4][2], int qb, const bf16x8_t (&pf)[2]) {
#pragma unroll
    for (int db = 0; db < 4; ++db) {
      o[qb][db] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(vf[db][0], pf[0], o[qb][db], 0, 0, 0);
      o[qb][db] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(vf[db][1], pf[1], o[qb][db], 0, 0, 0);
    }
    if constexpr (kMfmaSum) {
      l_acc[qb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ones8, pf[0], l_acc[qb], 0, 0, 0);
      l_acc[qb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ones8, pf[1], l_acc[qb], 0, 0, 0);
    }
  };
  // Softmax of query block qb of the tile in hand, with the block's next-tile scores formed on
  // the matrix cores in the same stretch of code.  Lazy running max: weights are taken against
  // the current m; only if some weight reaches 2 is m raised exactly to the row max (O and l
  // rescaled) and the block redone, so in the steady state no per-score max and no rescale run.
  auto block = [&](const bf16x8_t (&kf)[4][2], const float* bb, int qb, f32x4_t (&s_cur)[4],
                   f32x4_t (&s_next)[4], bf16x8_t (&pf)[2], bool next) {
    if (next) scores_qb(kf, bb, qb, s_next, m_run[qb]);
    const float l_prev = l_run[qb];
    const uint32_t bits = probs_qb(qb, s_cur, pf);
    // (expected false: the rescale is laid out of line, so the common path runs straight on)
    if (__builtin_expect(__builtin_amdgcn_ballot_w64((bits & 0x40004000u) != 0) != 0, 0)) {
      asm volatile("; rare rescale" ::);  // keeps this branch from being speculated into every tile
      // Exact mode: scores are absolute (q.k); the offset drops to -(c mx + w) for the row max
      // mx.  f16 score form: scores are relative to m + w (log2 units), so the offset drops by
      // the raise d of m, and the current and already formed next-tile scores shift with it.
      const float mx = row_max(s_cur);
      const float d = PRESCALE_Q ? vmax(mx + shift, 0.f) : vmax(m_run[qb] - fmaf(-mx, c, -shift), 0.f);
      const float alpha = __builtin_amdgcn_exp2f(-d);
      m_run[qb] -= d;
      if constexpr (kMfmaSum) l_acc[qb] *= alpha;  // (this block's weights are added after the check)
      else l_run[qb] = l_prev * alpha;
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        o[qb][k] *= alpha;
        if constexpr (PRESCALE_Q) {
          s_cur[k] -= d;
          if (next) s_next[k] -= d;
        }
      }
      probs_qb(qb, s_cur, pf);
    }
  };

  async_tile(kseg, 0, kbuf0, 0);
  async_bias(0, bbuf0);
  async_tile(vseg, 0, vbuf0, 1);
  // K tile 1 unconditionally (tile 0 again when it is the only one), so that the number of
  // copies in flight after K tile 0 is the same on every path.
  async_tile(kseg, min(1, nkt - 1), kbuf1, 0);
  async_bias(min(1, nkt - 1), bbuf1);
  // Q in the B-operand layout, and the diagonal term's initial state.
#pragma unroll
  for (int qb = 0; qb < QB; ++qb) {
    const int64_t t = wrow0 + qb * 16 + l16;
    const bool valid = t < row_end;
    float dot = 0.f;
    // The diagonal term belongs to one piece of a split item only.
    const bool self = !INPLACE && a.diag && valid && piece == 0 && !token_kept(a.g, t);  // (no G2F row has one)
#pragma unroll
    for (int cc = 0; cc < 2; ++cc) {
      const uint4 raw = qraw[qb][cc];
      uint4 kraw = make_uint4(0, 0, 0, 0);
      if (self) kraw = *reinterpret_cast<const uint4*>(Kin + size_t(t) * kHeadDim + cc * 32 + grp * 8);
      const uint32_t qw[4] = {raw.x, raw.y, raw.z, raw.w};
      const uint32_t kw[4] = {kraw.x, kraw.y, kraw.z, kraw.w};
      if constexpr (PRESCALE_Q) {
        f16x8_t v;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          // (saturated at the f16 maximum: only logit terms beyond 2^22 octaves reach it)
          const float q0 = __builtin_amdgcn_fmed3f(__uint_as_float(qw[i] << 16) * qscale, -65504.f, 65504.f);
          const float q1 = __builtin_amdgcn_fmed3f(__uint_as_float(qw[i] & 0xffff0000u) * qscale, -65504.f, 65504.f);
          v[2 * i] = (_Float16)q0;
          v[2 * i + 1] = (_Float16)q1;
          // Diagonal self logit from the same rounded query the matrix core uses (its key is
          // scaled below, exactly as the packed keys are).
          dot = fmaf(float(v[2 * i]), __uint_as_float(kw[i] << 16), dot);
          dot = fmaf(float(v[2 * i + 1]), __uint_as_float(kw[i] & 0xffff0000u), dot);
        }
        qf[qb][cc] = __builtin_bit_cast(bf16x8_t, v);
      } else {
#pragma unroll
        for (int i = 0; i < 4; ++i) {  // diagonal self logit, q.k in float32
          dot = fmaf(__uint_as_float(qw[i] << 16), __uint_as_float(kw[i] << 16), dot);
          dot = fmaf(__uint_as_float(qw[i] & 0xffff0000u), __uint_as_float(kw[i] & 0xffff0000u), dot);
        }
        qf[qb][cc] = __builtin_bit_cast(bf16x8_t, raw);
      }
    }
    // Diagonal term: a query whose own token is not in S starts with its self term
    // (m = self logit, weight 2^-w in l and O); the others start empty.
    dot = group_sum(dot) * kscale;
    if constexpr (LOGSIZE) {
      if (self) dot += a.logsize[t] * a.size_scale;
    }
    m_run[qb] = self ? dot : -INFINITY;
    if constexpr (kMfmaSum)
      l_acc[qb] = self ? f32x4_t{shift_scale, shift_scale, shift_scale, shift_scale} : f32x4_t{0.f, 0.f, 0.f, 0.f};
    else
      l_run[qb] = (self && grp == 0) ? shift_scale : 0.f;
#pragma unroll
    for (int db = 0; db < 4; ++db) {
      f32x4_t init = {0.f, 0.f, 0.f, 0.f};
      if (self) {
        const uint2 vr = *reinterpret_cast<const uint2*>(Vin + size_t(t) * kHeadDim + db * 16 + grp * 4);
        init[0] = __uint_as_float(vr.x << 16) * shift_scale;
        init[1] = __uint_as_float(vr.x & 0xffff0000u) * shift_scale;
        init[2] = __uint_as_float(vr.y << 16) * shift_scale;
        init[3] = __uint_as_float(vr.y & 0xffff0000u) * shift_scale;
      }
      o[qb][db] = init;
    }
  }
  // Only K tile 0 (and its biases) is needed for the first scores: wait for the copies before the
  // ones issued after it (V tile 0, K tile 1 and its biases: 2 + 2 loads per wave, one more for
  // wave 0 under size-aware keys; vector-memory loads complete in issue order), so that those
  // land while tile 0 is scored.  A bare barrier, since __syncthreads' release fence would wait
  // for every copy; the memory clobber keeps LDS reads below it.
  if (LOGSIZE && wave == 0) __builtin_amdgcn_s_waitcnt(kWaitVmcnt0 | 5);
  else __builtin_amdgcn_s_waitcnt(kWaitVmcnt0 | 4);
  asm volatile("s_barrier" ::: "memory");

  // A wave with no query row in range (in the last, partial work item of a frame or a head)
  // computes nothing: it only copies its share of every tile and meets every barrier of the
  // steps below (one after tile 0, one per step), leaving its SIMD to the other work-group's
  // wave.  (Wave 0 always has rows, so the bias copies of wave 0 never take this path.)
  if (wrow0 >= row_end) {
    wait_tiles();
    __syncthreads();
    for (int jj = 0; jj + 1 < nkt; ++jj) {
      const bool odd = jj & 1;
      async_tile(kseg, min(jj + 2, nkt - 1), odd ? kbuf1 : kbuf0, 0);
      async_bias(min(jj + 2, nkt - 1), odd ? bbuf1 : bbuf0);
      async_tile(vseg, jj + 1, odd ? vbuf0 : vbuf1, 1);
      wait_tiles();
      __syncthreads();
    }
    return;
  }

  // One pipelined step: finish tile j (scores s_cur) while the scores of tile j+1 are formed,
  // query block by query block so that every stretch of code mixes matrix-core and VALU work.
  // P = j & 1 is a compile-time constant, so every LDS buffer is static.  MASK = tile j+1 may
  // hold mean keys or padding (kept out of the steady-state loop, where the compiler would
  // otherwise if-convert the bias into every tile).
  auto step = [&](auto parity, auto mask_tag, int j, f32x4_t (&s_cur)[QB][4], f32x4_t (&s_next)[QB][4]) {
    constexpr int P = decltype(parity)::value;
    using same_t = std::integral_constant<int, P>;
    using other_t = std::integral_constant<int, P ^ 1>;
    async_tile(kseg, min(j + 2, nkt - 1), kbuf(same_t{}), 0);
    async_bias(min(j + 2, nkt - 1), bbuf(same_t{}));
    async_tile(vseg, j + 1, vbuf(other_t{}), 1);
    bf16x8_t kf[4][2], vf[4][2];
    k_frags(kbuf(other_t{}), kf);
    v_frags(vbuf(same_t{}), vf);
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) {
      bf16x8_t pf[2];
      block(kf, bbuf(other_t{}), qb, s_cur[qb], s_next[qb], pf, true);
      accumulate_qb(vf, qb, pf);
    }
    if constexpr (decltype(mask_tag)::value) bias_mask(j + 1, s_next);
    wait_tiles();
    __syncthreads();
  };
  auto last = [&](auto parity, f32x4_t (&s_cur)[QB][4]) {
    bf16x8_t kf[4][2], vf[4][2];
    v_frags(vbuf(parity), vf);
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) {
      bf16x8_t pf[2];
      block(kf, nullptr, qb, s_cur[qb], s_cur[qb], pf, false);
      accumulate_qb(vf, qb, pf);
    }
  };
  using plain_t = std::integral_constant<bool, false>;
  using masked_t = std::integral_constant<bool, true>;
  using even_t = std::integral_constant<int, 0>;
  using odd_t = std::integral_constant<int, 1>;

  // Tile 0 sets the running max exactly (from the diagonal term, if any, and the tile).
  f32x4_t sa[QB][4], sb[QB][4];
  {
    bf16x8_t kf[4][2];
    k_frags(kbuf0, kf);
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) scores_qb(kf, bbuf0, qb, sa[qb], 0.f);
  }
  bias_mask(0, sa);
#pragma unroll
  for (int qb = 0; qb < QB; ++qb) {
    const float m_new = vmax(m_run[qb], row_max(sa[qb]));  // finite: tile 0 holds a valid key
    if constexpr (!INPLACE) {  // (without a diagonal term l and O are still zero)
      const float alpha = __builtin_amdgcn_exp2f((m_run[qb] - m_new) * sc);
      if constexpr (kMfmaSum) l_acc[qb] *= alpha;
      else l_run[qb] *= alpha;
#pragma unroll
      for (int k = 0; k < 4; ++k) o[qb][k] *= alpha;
    }
    m_run[qb] = PRESCALE_Q ? -(m_new + shift) : fmaf(-m_new, c, -shift);
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      if constexpr (PRESCALE_Q) sa[qb][k] -= m_new + shift;
    }
  }
  // V tile 0 and K tile 1 for the first step.
  wait_tiles();
  __syncthreads();
  int j = 0;  // always even at the top of these loops
  for (; j + 2 < nkt && j + 2 < slow_from; j += 2) {
    step(even_t{}, plain_t{}, j, sa, sb);
    step(odd_t{}, plain_t{}, j + 1, sb, sa);
  }
  for (; j + 2 < nkt; j += 2) {
    step(even_t{}, masked_t{}, j, sa, sb);
    step(odd_t{}, masked_t{}, j + 1, sb, sa);
  }
  if (j + 1 < nkt) {
    step(even_t{}, masked_t{}, j, sa, sb);
    last(odd_t{}, sb);
  } else {
    last(even_t{}, sa);
  }

  // ---- epilogue: O / l, or the unnormalised state of a piece ----
  if constexpr (SPLIT) {
    float* dst = a.part + size_t(blockIdx.x) * BM * kPartRow;
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) {
      const float l = kMfmaSum ? l_acc[qb][0] : group_sum(l_run[qb]);
      float* row = dst + size_t(wave * WQ + qb * 16 + l16) * kPartRow;
#pragma unroll
      for (int db = 0; db < 4; ++db) *reinterpret_cast<f32x4_t*>(row + db * 16 + grp * 4) = o[qb][db];
      if (grp == 0) {
        row[64] = -m_run[qb];  // m + w in log2 units
        row[65] = l;
      }
    }
    return;
  }
#pragma unroll
  for (int qb = 0; qb < QB; ++qb) {
    const float l = kMfmaSum ? l_acc[qb][0] : group_sum(l_run[qb]);
    const float inv = __builtin_amdgcn_rcpf(l);
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

// Merge of the pieces of split work items: for each query row, the pieces' running maxima,
// sums and unnormalised outputs combine exactly as the online softmax would have across the
// whole key range.  One thread per (row, 4 channels); rows past the segment end are skipped.
template <bool OUT_BF16>
__global__ __launch_bounds__(256) void merge_pieces_kernel(AttnArgs a, int BM) {
  const int64_t gid = int64_t(blockIdx.x) * 256 + threadIdx.x;
  const int64_t rr = gid >> 4;  // row over all split items
  const int chunk = int(gid & 15);
  const int64_t k = rr / BM;
  const int r = int(rr - k * BM);
  const ItemRows ir = item_rows(a, a.split_from + k, BM);
  const int64_t t = ir.row0 + r;
  if (t >= ir.row_end) return;
  const float* base = a.part + (size_t(k) * a.nsplit * BM + r) * kPartRow;
  const size_t piece_stride = size_t(BM) * kPartRow;
  float mx = -INFINITY;
  for (int p = 0; p < a.nsplit; ++p) mx = fmaxf(mx, base[p * piece_stride + 64]);
  float l = 0.f;
  f32x4_t acc = {0.f, 0.f, 0.f, 0.f};
  for (int p = 0; p < a.nsplit; ++p) {
    const float* row = base + p * piece_stride;
    const float e = __builtin_amdgcn_exp2f(row[64] - mx);  // maxima in log2 units
    l = fmaf(row[65], e, l);
    acc += *reinterpret_cast<const f32x4_t*>(row + chunk * 4) * e;
  }
  const f32x4_t res = acc * (1.f / l);
  const size_t off = (size_t(ir.h) * size_t(a.T) + size_t(t)) * kHeadDim + chunk * 4;
  if constexpr (OUT_BF16) {
    *reinterpret_cast<uint2*>(static_cast<uint16_t*>(a.out) + off) =
        make_uint2(pack_bf16x2(res[0], res[1]), pack_bf16x2(res[2], res[3]));
  } else {
    *reinterpret_cast<f32x4_t*>(static_cast<float*>(a.out) + off) = res;
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
  const float* bseg = a.kbias ? a.kbias + size_t(seg) * a.segment_rows : nullptr;

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
    if (a.logsize) dot += a.logsize[t] * a.size_scale;
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
      else if (key >= a.n_plain) dot += mean_bias(a, a.mean_bias_s, key - a.n_plain);
      else if (bseg) dot += bseg[key];
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

// G2M: every query attends to the one mean key, so its softmax weight is exactly 1 and each
// output row is the mean value itself -- what the general kernel computes too (p = 2^0 = 1,
// O = 1 * v, l = 1), bit for bit.  So the output is a broadcast of v-bar[h] to every row of head
// h: each thread writes 16-byte chunks of one fixed column range (the grid stride is a multiple
// of the chunks per row), and the kernel is bound by the output writes.
template <typename E, bool OUT_BF16>
__global__ __launch_bounds__(256) void g2m_broadcast_kernel(const E* means, void* out, int64_t T) {
  constexpr int PER = OUT_BF16 ? 8 : 4;    // output elements per 16-byte chunk
  constexpr int CPR = kHeadDim / PER;      // chunks per row
  static_assert(256 % CPR == 0, "the grid stride must keep each thread on one column range");
  const int h = blockIdx.y;
  const E* vbar = means + (size_t(h) * 2 + 1) * kHeadDim;  // means[h][0][1][:]
  const int64_t total = T * CPR;
  const int64_t stride = int64_t(gridDim.x) * 256;
  int64_t i = int64_t(blockIdx.x) * 256 + threadIdx.x;
  const int col = int(i % CPR) * PER;
  uint4 chunk;
  if constexpr (OUT_BF16) {
    static_assert(sizeof(E) == 2, "bf16 output comes from bf16 input");
    chunk = *reinterpret_cast<const uint4*>(vbar + col);
  } else {
    float f[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      if constexpr (sizeof(E) == 2) f[j] = __uint_as_float(uint32_t(vbar[col + j]) << 16);
      else f[j] = vbar[col + j];
    }
    chunk = make_uint4(__float_as_uint(f[0]), __float_as_uint(f[1]), __float_as_uint(f[2]), __float_as_uint(f[3]));
  }
  uint4* dst = reinterpret_cast<uint4*>(static_cast<char*>(out) + size_t(h) * size_t(T) * kHeadDim * (OUT_BF16 ? 2 : 4));
  for (; i < total; i += stride) dst[i] = chunk;
}

}  // namespace

hipError_t launch_attend(const vggt_attn_plan_s& p, const void* q, const void* k, const void* v,
                         void* out, void* ws, hipStream_t stream) {
  char* base = static_cast<char*>(ws);
  if (p.g2m) {
    const bool ob = p.out_dtype == VGGT_ATTN_BF16;
    const int64_t total = p.T * (ob ? kHeadDim / 8 : kHeadDim / 4);
    const dim3 grid(unsigned(std::min<int64_t>((total + 255) / 256, 1024)), unsigned(p.heads));
    const void* means = base + p.layout.off_means;
    if (p.in_dtype == VGGT_ATTN_FP32)
      hipLaunchKernelGGL((g2m_broadcast_kernel<float, false>), grid, dim3(256), 0, stream, static_cast<const float*>(means), out, p.T);
    else if (ob)
      hipLaunchKernelGGL((g2m_broadcast_kernel<uint16_t, true>), grid, dim3(256), 0, stream, static_cast<const uint16_t*>(means), out, p.T);
    else
      hipLaunchKernelGGL((g2m_broadcast_kernel<uint16_t, false>), grid, dim3(256), 0, stream, static_cast<const uint16_t*>(means), out, p.T);
    return hipGetLastError();
  }
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
  // COUNT: logit += ln(n)  <=>  raw score q.k += ln(n) / tau, n = tokens behind the mean key.
  // Per-frame means under the phase shift: the mean frames of one run of nphase frames are the
  // phases with a nonempty dropped set, in phase order; mean key 0 is frame f0's slot.
  a.mean_off = 0;
  a.mean_run = 1;
  const IndexGeom& g = p.geom;
  const bool per_slot = p.M > 0 && !p.mean_global && !p.g2m && g.nphase > 1;
  int slot_phase[kMaxPhases] = {0};
  if (per_slot) {
    a.mean_run = g.mprefix[g.nphase];
    a.mean_off = g.mprefix[g.f0 % g.nphase];
    for (int k = 0; k < g.nphase; ++k)
      if (g.mprefix[k + 1] > g.mprefix[k]) slot_phase[g.mprefix[k]] = k;
  }
  for (int s = 0; s < kMaxPhases; ++s) {
    const double b = p.mean_bias_s[per_slot ? slot_phase[s] : 0];
    a.mean_bias_s[s] = float(b);
    a.mean_bias_log2[s] = float(b * tau * 1.4426950408889634);
  }
  a.c_log2 = float(tau * 1.4426950408889634);
  // Global-to-Frame segments are one frame (22 tiles at 1374 tokens), so the first tile's max
  // is often beaten later and each raise costs a rescale and a redone block; weights shifted
  // 32 octaves down make those raises almost never needed (11% less time at 200 frames).  The
  // global forms keep w = 0: with 800 frames the shifted weights ran the same instruction count
  // at a lower sustained clock (4-5% slower), for reasons not pinned down.
  a.weight_shift = p.g2f ? 32.f : 0.f;
  a.weight_scale = p.g2f ? 0x1p-32f : 1.f;
  if (p.log_size) {
    a.kbias = reinterpret_cast<const float*>(base + p.layout.off_kbias);
    a.logsize = reinterpret_cast<const float*>(base + p.layout.off_logsize);
    a.size_scale = float(std::sqrt(double(p.head_dim)));
  }
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

  // bf16: QB blocks of 16 query rows per wave, 4 waves per work-group, WPE work-groups'
  // waves per SIMD (occupancy), so that the matrix-core phase of one work-group overlaps the
  // softmax phase of another on the same CU.
  const bool inplace = p.inplace;
  const int qbn = p.g2f ? VGGT_G2F_QB : VGGT_GLOBAL_QB;
  const int BM = 64 * qbn;
  if (p.g2f) {
    a.qtiles_per_frame = int((p.L + BM - 1) / BM);
    a.qtiles = a.qtiles_per_frame * p.frames;
  } else {
    a.qtiles = int((p.T + BM - 1) / BM);
  }
  a.split_from = p.split_from;
  a.nsplit = p.nsplit;
  a.part = p.nsplit > 1 ? reinterpret_cast<float*>(base + p.layout.off_part) : nullptr;
  a.kmax = p.prescale_q ? reinterpret_cast<const uint32_t*>(base + p.layout.off_kmax) : nullptr;
  const unsigned blocks = unsigned(p.split_from);
  const unsigned pblocks = unsigned(p.split_items * p.nsplit);
  const bool ob = p.out_dtype == VGGT_ATTN_BF16;
  const bool pre = p.prescale_q;  // never set together with log_size, never in place
  const bool sz = p.log_size;
  if (pre && (sz || inplace)) return hipErrorInvalidValue;  // (the plan never combines them)
  // One instantiation per (tiling, output type, score form, split, in-place) actually used.
  auto go = [&](auto qb_, auto wpe_, auto ob_, auto pre_, auto sz_, auto ip_) {
    constexpr int QB_ = decltype(qb_)::value, WPE_ = decltype(wpe_)::value;
    constexpr bool OB = decltype(ob_)::value, PRE = decltype(pre_)::value, SZ = decltype(sz_)::value;
    constexpr bool IP = decltype(ip_)::value;
    if constexpr (!(PRE && (SZ || IP))) {
      if (blocks > 0)
        hipLaunchKernelGGL((attn_bf16_kernel<QB_, WPE_, OB, PRE, SZ, false, IP>), dim3(blocks), dim3(256), 0, stream, a);
      if constexpr (!SZ) {
        if (pblocks > 0)
          hipLaunchKernelGGL((attn_bf16_kernel<QB_, WPE_, OB, PRE, false, true, IP>), dim3(pblocks), dim3(256), 0, stream, a);
      }
    }
  };
  using T_ = std::true_type;
  using F_ = std::false_type;
  auto by_form = [&](auto qb_, auto wpe_, auto ip_) {
    if (ob) {
      if (sz) go(qb_, wpe_, T_{}, F_{}, T_{}, ip_);
      else if (pre) go(qb_, wpe_, T_{}, T_{}, F_{}, ip_);
      else go(qb_, wpe_, T_{}, F_{}, F_{}, ip_);
    } else {
      if (sz) go(qb_, wpe_, F_{}, F_{}, T_{}, ip_);
      else if (pre) go(qb_, wpe_, F_{}, T_{}, F_{}, ip_);
      else go(qb_, wpe_, F_{}, F_{}, F_{}, ip_);
    }
  };
  using QBg = std::integral_constant<int, VGGT_GLOBAL_QB>;
  using WPEg = std::integral_constant<int, VGGT_GLOBAL_WPE>;
  using QBf = std::integral_constant<int, VGGT_G2F_QB>;
  using WPEf = std::integral_constant<int, VGGT_G2F_WPE>;
  // bf16 G2F plans read K/V in place, except in the f16 score form (packed f16 keys).
  if (p.g2f && inplace) by_form(QBf{}, WPEf{}, T_{});
  else if (p.g2f) by_form(QBf{}, WPEf{}, F_{});
  else by_form(QBg{}, WPEg{}, F_{});
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || p.nsplit <= 1) return e;
  const int64_t threads = p.split_items * BM * 16;
  const unsigned mblocks = unsigned((threads + 255) / 256);
  if (ob) hipLaunchKernelGGL((merge_pieces_kernel<true>), dim3(mblocks), dim3(256), 0, stream, a, BM);
  else hipLaunchKernelGGL((merge_pieces_kernel<false>), dim3(mblocks), dim3(256), 0, stream, a, BM);
  return hipGetLastError();
}

}  // namespace vggt
