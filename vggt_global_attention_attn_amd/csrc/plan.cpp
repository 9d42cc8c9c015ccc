// Plan construction: validation, window shape, sizes of S / means / diagonal terms, FLOPs and
// the workspace layout.
//
// Sources: "AVGGT: Rethinking Global Attention for Accelerating VGGT" (papernotes.org CVPR 2026
// notes), 关键设计 1 (Global-to-Frame keeps the per-frame layout), 关键设计 2 (sigma = s_h*s_w
// with 2->(1,2), 4->(2,2), 6->(2,3), 9->(3,3); the first patch of each window, all queries and
// all special tokens kept; frame 0 uncompressed for VGGT, every frame compressed for pi^3),
// 关键设计 3 (diagonal and mean terms), ablation table (G2M: K/V replaced by one mean token);
// "RegimeVGGT ..." (papernotes.org NeurIPS 2026 notes), 核心机制 (L = T + 5 tokens per frame),
// 关键设计 3 (per-frame phase of the sampling grid).
#include "plan.h"

#include <algorithm>
#include <cmath>
#include <cstdio>

namespace vggt {
namespace {

int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }
int64_t align256(int64_t x) { return (x + 255) & ~int64_t(255); }

bool window_of(int sigma, int* s_h, int* s_w) {
  switch (sigma) {
    case 1: *s_h = 1; *s_w = 1; return true;
    case 2: *s_h = 1; *s_w = 2; return true;
    case 4: *s_h = 2; *s_w = 2; return true;
    case 6: *s_h = 2; *s_w = 3; return true;
    case 9: *s_h = 3; *s_w = 3; return true;
    default: return false;
  }
}

int fail(std::string* err, int code, const char* fmt, long long a = 0, long long b = 0) {
  char buf[256];
  std::snprintf(buf, sizeof buf, fmt, a, b);
  if (err) *err = buf;
  return code;
}

}  // namespace

int build_plan(vggt_attn_plan_s* p, int frames, int grid_h, int grid_w, int n_special, int heads,
               int head_dim, int sigma, unsigned flags, int in_dtype, int out_dtype,
               std::string* err) {
  if (frames < 1 || grid_h < 1 || grid_w < 1 || heads < 1 || n_special < 0)
    return fail(err, VGGT_ATTN_EINVAL, "frames, grid_h, grid_w, heads must be >= 1 and n_special >= 0");
  if (heads > kMaxHeads) return fail(err, VGGT_ATTN_EINVAL, "heads %lld exceeds %lld", heads, kMaxHeads);
  if (head_dim != kHeadDim)
    return fail(err, VGGT_ATTN_EUNSUPPORTED, "head_dim %lld not supported (only %lld)", head_dim, kHeadDim);
  int s_h, s_w;
  if (!window_of(sigma, &s_h, &s_w))
    return fail(err, VGGT_ATTN_EINVAL, "sigma %lld not in {1, 2, 4, 6, 9}", sigma);
  const unsigned known = VGGT_ATTN_G2F | VGGT_ATTN_REF_DENSE | VGGT_ATTN_DIAG | VGGT_ATTN_MEAN |
                         VGGT_ATTN_MEAN_COUNT | VGGT_ATTN_PRESCALE_Q | VGGT_ATTN_PHASE_SHIFT |
                         VGGT_ATTN_MEAN_GLOBAL | VGGT_ATTN_G2M | VGGT_ATTN_LOG_SIZE;
  if (flags & ~known) return fail(err, VGGT_ATTN_EINVAL, "unknown flag bits 0x%llx", flags & ~known);
  const bool g2f = flags & VGGT_ATTN_G2F;
  const bool g2m = flags & VGGT_ATTN_G2M;
  const unsigned refine = VGGT_ATTN_DIAG | VGGT_ATTN_MEAN | VGGT_ATTN_MEAN_GLOBAL | VGGT_ATTN_PHASE_SHIFT;
  if (g2f && (sigma != 1 || (flags & (refine | VGGT_ATTN_G2M))))
    return fail(err, VGGT_ATTN_EINVAL, "G2F takes sigma == 1 and none of DIAG/MEAN/MEAN_GLOBAL/PHASE_SHIFT/G2M");
  if (g2m && (sigma != 1 || (flags & refine)))
    return fail(err, VGGT_ATTN_EINVAL, "G2M takes sigma == 1 and none of DIAG/MEAN/MEAN_GLOBAL/PHASE_SHIFT");
  if ((flags & VGGT_ATTN_MEAN_GLOBAL) && !(flags & VGGT_ATTN_MEAN))
    return fail(err, VGGT_ATTN_EINVAL, "MEAN_GLOBAL requires MEAN");
  if ((flags & VGGT_ATTN_LOG_SIZE) && (flags & (VGGT_ATTN_MEAN | VGGT_ATTN_G2M)))
    return fail(err, VGGT_ATTN_EINVAL, "LOG_SIZE is not combined with MEAN or G2M");
  const bool dtype_ok = (in_dtype == VGGT_ATTN_BF16 && (out_dtype == VGGT_ATTN_FP32 || out_dtype == VGGT_ATTN_BF16)) ||
                        (in_dtype == VGGT_ATTN_FP32 && out_dtype == VGGT_ATTN_FP32);
  if (!dtype_ok)
    return fail(err, VGGT_ATTN_EINVAL, "dtype pair (%lld, %lld) not supported", in_dtype, out_dtype);

  const int64_t P = int64_t(grid_h) * grid_w;
  const int64_t L = P + n_special;
  const int64_t T = L * frames;
  if (P > (1 << 24) || T > kMaxTokens)
    return fail(err, VGGT_ATTN_EINVAL, "T = %lld tokens exceeds the limit %lld", T, kMaxTokens);

  *p = vggt_attn_plan_s{};
  p->frames = frames; p->grid_h = grid_h; p->grid_w = grid_w; p->n_special = n_special;
  p->heads = heads; p->head_dim = head_dim; p->sigma = sigma; p->flags = flags;
  p->in_dtype = in_dtype; p->out_dtype = out_dtype;
  p->g2f = g2f;
  p->g2m = g2m;
  p->subsampled = sigma > 1;
  p->ref_dense = flags & VGGT_ATTN_REF_DENSE;
  p->diag = (flags & VGGT_ATTN_DIAG) && p->subsampled;
  p->mean = (flags & VGGT_ATTN_MEAN) && p->subsampled;
  p->mean_global = (flags & VGGT_ATTN_MEAN_GLOBAL) && p->mean;
  p->mean_count = flags & VGGT_ATTN_MEAN_COUNT;
  p->log_size = flags & VGGT_ATTN_LOG_SIZE;
  p->prescale_q = (flags & VGGT_ATTN_PRESCALE_Q) && !p->log_size && in_dtype == VGGT_ATTN_BF16;
  p->phase = (flags & VGGT_ATTN_PHASE_SHIFT) && p->subsampled;
  p->s_h = s_h; p->s_w = s_w;
  p->L = int(L); p->P = int(P); p->T = T;

  // Grid phases of the compressed frames (RegimeVGGT notes, 关键设计 3): phase k = f mod
  // (s_h*s_w) has row offset k / s_w and column offset k % s_w; without the shift every frame
  // has phase 0.  Partial windows at the grid edge count (ceil).
  IndexGeom& g = p->geom;
  g.L = p->L; g.P = p->P; g.n_special = n_special; g.grid_w = grid_w;
  g.s_h = s_h; g.s_w = s_w;
  g.ref_dense = p->ref_dense ? 1 : 0; g.subsampled = p->subsampled ? 1 : 0; g.g2m = g2m ? 1 : 0;
  g.f0 = (p->subsampled && p->ref_dense) ? 1 : 0;
  g.nphase = p->phase ? s_h * s_w : 1;
  for (int ro = 0; ro < s_h; ++ro) g.rows_of[ro] = int(ceil_div(std::max<int64_t>(grid_h - ro, 0), s_h));
  for (int co = 0; co < s_w; ++co) g.cols_of[co] = int(ceil_div(std::max<int64_t>(grid_w - co, 0), s_w));
  g.cprefix[0] = 0;
  g.mprefix[0] = 0;
  for (int k = 0; k < g.nphase; ++k) {
    const int64_t kept = int64_t(g.rows_of[k / s_w]) * g.cols_of[k % s_w];
    p->dropped_of_phase[k] = P - kept;
    g.cprefix[k + 1] = g.cprefix[k] + n_special + int(kept);
    g.mprefix[k + 1] = g.mprefix[k] + (P - kept > 0 ? 1 : 0);
  }

  const double tau = 1.0 / std::sqrt(double(head_dim));
  if (g2m) {
    // Every token feeds one mean; nothing is kept.
    p->n_dense_frames = 0;
    p->n_compressed_frames = 0;
    p->nS = 0;
    p->dropped_total = T;
    p->M_frames = frames;
    p->M = 1;
  } else if (!p->subsampled) {
    p->n_dense_frames = frames;
    p->n_compressed_frames = 0;
    p->nS = T;
  } else {
    p->n_dense_frames = p->ref_dense ? 1 : 0;
    p->n_compressed_frames = frames - p->n_dense_frames;
    // Compressed frames f in [f0, N) of each phase k.
    auto below = [&](int64_t n, int k) { return n / g.nphase + (n % g.nphase > k ? 1 : 0); };
    int64_t kept_total = 0;
    for (int k = 0; k < g.nphase; ++k) {
      const int64_t cnt = below(frames, k) - below(g.f0, k);
      kept_total += cnt * (P - p->dropped_of_phase[k]);
      p->dropped_total += cnt * p->dropped_of_phase[k];
      if (p->dropped_of_phase[k] > 0) p->M_frames += cnt;
    }
    // |S| = specials of every frame + every patch of dense frames + kept grid points elsewhere.
    p->nS = int64_t(frames) * n_special + p->n_dense_frames * P + kept_total;
    if (p->mean) p->M = p->mean_global ? (p->dropped_total > 0 ? 1 : 0) : p->M_frames;
    if (!p->mean) p->M_frames = 0;
    if (p->mean_count && p->M > 0) {
      if (p->mean_global) {
        p->mean_bias_s[0] = std::log(double(p->dropped_total)) / tau;
      } else {
        for (int k = 0; k < g.nphase; ++k)
          if (p->dropped_of_phase[k] > 0) p->mean_bias_s[k] = std::log(double(p->dropped_of_phase[k])) / tau;
      }
    }
  }
  p->n_diag = p->diag ? p->dropped_total : 0;

  const double d4H = 4.0 * head_dim * heads;
  if (g2f) {
    p->segments = frames;
    p->keys_per_segment = L;
    p->n_plain = L;
    p->flops = d4H * double(frames) * double(L) * double(L);
  } else {
    p->segments = 1;
    p->keys_per_segment = p->nS + p->M;
    p->n_plain = p->nS;
    p->flops = d4H * (double(T) * double(p->nS + p->M) + double(p->n_diag));
  }
  p->segment_rows = ceil_div(p->keys_per_segment, kTile) * kTile;
  p->rows_per_head = p->segments * p->segment_rows;
  if (p->rows_per_head > kMaxPackedRows)
    return fail(err, VGGT_ATTN_EINVAL, "packed rows per head %lld exceed %lld", p->rows_per_head, kMaxPackedRows);

  // bf16 work items and the split of a sparse last round (float32 inputs: one item per 64 rows,
  // never split; nor is the LOG_SIZE form).
  const int qb = g2f ? VGGT_G2F_QB : VGGT_GLOBAL_QB;
  const int wpe = g2f ? VGGT_G2F_WPE : VGGT_GLOBAL_WPE;
  p->block_rows = in_dtype == VGGT_ATTN_BF16 ? 64 * qb : 64;
  const int64_t qtiles = g2f ? ceil_div(L, p->block_rows) * frames : ceil_div(T, p->block_rows);
  p->work_items = qtiles * heads;
  p->split_from = p->work_items;
  p->split_items = 0;
  p->nsplit = 1;
  if (in_dtype == VGGT_ATTN_BF16 && !p->log_size) {
    const int64_t slots = int64_t(kComputeUnits) * wpe;
    const int64_t tail = p->work_items % slots;
    const int64_t nkt = p->segment_rows / kTile;
    const int64_t pieces = std::min<int64_t>({tail > 0 ? slots / tail : 0, nkt / 4, kMaxSplit});
    if (tail > 0 && 2 * tail <= slots && pieces >= 2) {
      p->nsplit = int(pieces);
      p->split_items = tail;
      p->split_from = p->work_items - tail;
    }
  }

  // bf16 G2F reads K and V in place, unless the f16 score form needs K converted and packed.
  p->inplace = in_dtype == VGGT_ATTN_BF16 && g2f && !p->prescale_q;
  p->elem_bytes = in_dtype == VGGT_ATTN_BF16 ? 2 : 4;
  vggt_attn_layout_t& lay = p->layout;
  lay.segments = p->segments;
  lay.segment_rows = p->segment_rows;
  lay.keys_per_segment = p->keys_per_segment;
  int64_t off = 0;
  lay.off_index = off;  off = align256(off + (g2f ? 0 : p->nS) * 4);
  lay.off_dcount = off; off = align256(off + int64_t(frames) * 4);
  lay.off_means = off;  off = align256(off + int64_t(heads) * p->M * 2 * head_dim * int64_t(p->elem_bytes));
  const int64_t partials = (p->mean_global || p->g2m) ? p->M_frames : 0;
  lay.off_partial = off; off = align256(off + int64_t(heads) * partials * 2 * head_dim * 4);
  lay.off_kbias = off;  off = align256(off + (p->log_size ? p->rows_per_head * 4 : 0));
  lay.off_logsize = off; off = align256(off + (p->log_size ? T * 4 : 0));
  lay.off_part = off;   off = align256(off + p->split_items * p->nsplit * p->block_rows * kPartRow * 4 * (p->nsplit > 1));
  lay.split_pieces = p->nsplit > 1 ? p->nsplit : 0;
  lay.off_kmax = off;   off = align256(off + (p->prescale_q ? int64_t(heads) * 4 : 0));
  const int64_t packed = p->inplace ? 0 : int64_t(heads) * p->rows_per_head * head_dim * int64_t(p->elem_bytes);
  lay.off_kpack = off;  off = align256(off + packed);
  lay.off_vpack = off;  off = align256(off + packed);
  lay.total_bytes = off;
  return VGGT_ATTN_OK;
}

}  // namespace vggt
