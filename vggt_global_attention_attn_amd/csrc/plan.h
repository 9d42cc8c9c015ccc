// Host-side plan of one VGGT global-attention call: validated geometry, the sizes of the kept
// set S, the mean keys and the diagonal terms, and the workspace layout.  Pure integer code;
// it makes no HIP call, so plans can be built and tested without a GPU.
#pragma once

#include <cstddef>
#include <cstdint>
#include <string>

#include "vggt_attn.h"

namespace vggt {

constexpr int kHeadDim = 64;   // the only head size the library implements
constexpr int kTile = 64;      // packed key rows per tile (attention key-tile height)
constexpr int64_t kMaxTokens = 8000000;
constexpr int kMaxHeads = 4096;
constexpr int64_t kMaxPackedRows = 16000000;  // per head, keeps row*64 within int32

constexpr int kMaxPhases = 9;  // s_h * s_w for the largest window (3 x 3)

// Tiling of the bf16 attention kernel: 16-row query blocks per wave (QB), waves of one work-group
// per SIMD (WPE).  A work-group has 4 waves and owns 64*QB query rows.
#ifndef VGGT_GLOBAL_QB
#define VGGT_GLOBAL_QB 3
#endif
#ifndef VGGT_GLOBAL_WPE
#define VGGT_GLOBAL_WPE 2
#endif
#ifndef VGGT_G2F_QB
#define VGGT_G2F_QB 3
#endif
#ifndef VGGT_G2F_WPE
#define VGGT_G2F_WPE 2
#endif
// Work-groups resident at once on a 256-CU gfx950 part (MI355X): one per SIMD set per unit of
// WPE.  Used only to size the last round of work-groups (see kMaxSplit); correctness does not
// depend on it.
constexpr int kComputeUnits = 256;
// A last round of work-groups that would fill at most half of the resident slots is split
// along the key range into up to this many pieces, merged afterwards.
constexpr int kMaxSplit = 8;
// gfx950 (MI355X) dispatches the work-groups of a launch to its 8 XCDs round-robin; each XCD
// has its own L2.  Used only to order work items; correctness does not depend on it.
constexpr int kXcds = 8;
constexpr int kPartRow = 68;  // floats per query row of a piece: O[64], m, l, 2 unused
// Size of the static device workspace of vggt_attn_forward_noalloc (one copy per GPU).
constexpr size_t kScratchBytes = size_t(256) << 20;

// Geometry the device code needs to enumerate S and the mean frames and to test membership in
// closed form.  Compressed frame f has grid phase k = f mod nphase (nphase = s_h*s_w with the
// phase-shifted grid, else 1), row offset k / s_w and column offset k % s_w; every quantity of
// a compressed frame depends on f only through k.
struct IndexGeom {
  int L;           // tokens per frame
  int P;           // patches per frame
  int n_special;   // camera/register tokens per frame (slots 0 .. n_special-1)
  int grid_w;      // patch columns
  int s_h, s_w;    // window (row stride, column stride)
  int ref_dense;   // frame 0 dense
  int subsampled;  // sigma > 1
  int g2m;         // every token feeds one mean, none is kept
  int f0;          // first compressed frame (1 with a dense frame 0, else 0)
  int nphase;      // grid phases (1 without the phase shift)
  int rows_of[3];  // kept rows for row offset ro: ceil((grid_h - ro) / s_h)
  int cols_of[3];  // kept columns for column offset co: ceil((grid_w - co) / s_w)
  int cprefix[kMaxPhases + 1];  // S entries of compressed frames of phases 0..k-1 (one each)
  int mprefix[kMaxPhases + 1];  // phases 0..k-1 whose frames have a nonempty dropped set
};

}  // namespace vggt

struct vggt_attn_plan_s {
  // as given
  int frames, grid_h, grid_w, n_special, heads, head_dim, sigma;
  unsigned flags;
  int in_dtype, out_dtype;
  // derived
  bool g2f, ref_dense, diag, mean, mean_count, subsampled, prescale_q;
  bool phase, mean_global, g2m, log_size;
  int s_h, s_w, L, P;
  int64_t T;
  int64_t dropped_of_phase[vggt::kMaxPhases];  // |D_f| of a compressed frame of phase k
  int64_t n_dense_frames, n_compressed_frames;
  int64_t dropped_total;  // sum of |D_f| over all frames (G2M: T)
  int64_t nS, M, n_diag;
  int64_t M_frames;       // frames feeding a mean (nonempty dropped set; G2M: every frame)
  double mean_bias_s[vggt::kMaxPhases];  // per phase (per-frame scope) or [0] (single mean):
                                         // COUNT bias in raw-score units, ln(n) / tau
  int64_t segments, segment_rows, keys_per_segment, n_plain, rows_per_head;
  // bf16 G2F plans read K and V where they lie (the keys of a frame are its tokens, in order):
  // no packed copy; the pack stage writes only the per-frame counts.  (Dense plans could do the
  // same, but there the transposed V reads cost more attention time than the O(T) pack.)  The
  // f16 score form (prescale_q) packs G2F keys too: they are converted to f16.
  bool inplace;
  // bf16 attention work split: work items (query tile x head) below split_from run whole; the
  // split_items after them run as nsplit key-range pieces each, merged by a second kernel.
  int64_t work_items, split_from, split_items;
  int nsplit, block_rows;
  double flops;
  size_t elem_bytes;
  vggt_attn_layout_t layout;
  vggt::IndexGeom geom;
};

namespace vggt {

// Fills *plan from the arguments; returns a vggt_attn_status and a message on failure.
int build_plan(vggt_attn_plan_s* plan, int frames, int grid_h, int grid_w, int n_special,
               int heads, int head_dim, int sigma, unsigned flags, int in_dtype, int out_dtype,
               std::string* err);

}  // namespace vggt
