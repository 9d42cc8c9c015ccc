// Host-side plan of one VGGT global-attention call: validated geometry, the sizes of the kept
// set S, the mean keys and the diagonal terms, and the workspace layout.  Pure integer code;
// it makes no HIP call, so plans can be built and tested without a GPU.
#pragma once

#include <cstddef>
#include <cstdint>
#include <string>

#include "vggt_attn.h"

namespace vggt {

constexpr int kHeadDim = 64;   // the only head size this build implements
constexpr int kTile = 64;      // packed key rows per tile (attention key-tile height)
constexpr int64_t kMaxTokens = 8000000;
constexpr int kMaxHeads = 4096;
constexpr int64_t kMaxPackedRows = 16000000;  // per head, keeps row*64 within int32

// Geometry the device code needs to enumerate S and to test membership in closed form.
struct IndexGeom {
  int L;           // tokens per frame
  int P;           // patches per frame
  int n_special;   // camera/register tokens per frame (slots 0 .. n_special-1)
  int grid_w;      // patch columns
  int s_h, s_w;    // window (row stride, column stride)
  int kw;          // kept columns per compressed frame = ceil(grid_w / s_w)
  int kept;        // kept patches per compressed frame = ceil(grid_h/s_h)*ceil(grid_w/s_w)
  int ref_dense;   // frame 0 dense
  int subsampled;  // sigma > 1
};

}  // namespace vggt

struct vggt_attn_plan_s {
  // as given
  int frames, grid_h, grid_w, n_special, heads, head_dim, sigma;
  unsigned flags;
  int in_dtype, out_dtype;
  // derived
  bool g2f, ref_dense, diag, mean, mean_count, subsampled, prescale_q;
  int s_h, s_w, L, P, kh, kw, kept;
  int64_t T;
  int64_t dropped;        // |D_f| of a compressed frame
  int64_t n_dense_frames, n_compressed_frames;
  int64_t nS, M, n_diag;
  int64_t segments, segment_rows, keys_per_segment, n_plain, rows_per_head;
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
