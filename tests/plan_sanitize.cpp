// Host-side plan construction under AddressSanitizer and UndefinedBehaviorSanitizer: every
// combination of a grid of descriptors (valid, degenerate and out of range), each checked for
// the workspace-layout invariants the C ABI documents.  Built with g++ by
// tests/test_plan_sanitize.py; prints one line and exits non-zero on the first violation.
#include <cstdio>
#include <string>

#include "plan.h"

namespace {

int failures = 0;

void expect(bool ok, const char* what, int frames, int gh, int gw, int ns, int heads, int sigma, unsigned flags) {
  if (ok) return;
  if (failures < 10)
    std::printf("violation: %s (frames %d grid %dx%d specials %d heads %d sigma %d flags 0x%x)\n", what, frames, gh, gw,
                ns, heads, sigma, flags);
  ++failures;
}

}  // namespace

int main() {
  const int frames_list[] = {-1, 0, 1, 2, 7, 200, 800, 5822, 5823, 100000};
  const int grids[][2] = {{1, 1}, {0, 5}, {2, 65}, {13, 11}, {37, 37}, {4097, 4097}};
  const int specials[] = {-1, 0, 5, 7};
  const int heads_list[] = {0, 1, 16, 4096, 4097};
  const int sigmas[] = {0, 1, 2, 3, 4, 6, 9};
  const unsigned flag_sets[] = {
      0u,
      VGGT_ATTN_REF_DENSE,
      VGGT_ATTN_REF_DENSE | VGGT_ATTN_DIAG | VGGT_ATTN_MEAN,
      VGGT_ATTN_REF_DENSE | VGGT_ATTN_DIAG | VGGT_ATTN_MEAN | VGGT_ATTN_MEAN_COUNT | VGGT_ATTN_PHASE_SHIFT,
      VGGT_ATTN_DIAG | VGGT_ATTN_MEAN | VGGT_ATTN_MEAN_GLOBAL | VGGT_ATTN_MEAN_COUNT,
      VGGT_ATTN_MEAN_GLOBAL,
      VGGT_ATTN_G2F,
      VGGT_ATTN_G2F | VGGT_ATTN_PRESCALE_Q,
      VGGT_ATTN_G2F | VGGT_ATTN_DIAG,
      VGGT_ATTN_G2M,
      VGGT_ATTN_G2M | VGGT_ATTN_G2F,
      VGGT_ATTN_REF_DENSE | VGGT_ATTN_DIAG | VGGT_ATTN_LOG_SIZE | VGGT_ATTN_PRESCALE_Q,
      VGGT_ATTN_LOG_SIZE | VGGT_ATTN_MEAN,
      VGGT_ATTN_REF_DENSE | VGGT_ATTN_DIAG | VGGT_ATTN_MEAN | VGGT_ATTN_PRESCALE_Q,
      1u << 12,
  };
  const int dtypes[][2] = {{VGGT_ATTN_BF16, VGGT_ATTN_FP32}, {VGGT_ATTN_BF16, VGGT_ATTN_BF16},
                           {VGGT_ATTN_FP32, VGGT_ATTN_FP32}, {VGGT_ATTN_FP32, VGGT_ATTN_BF16}};
  long plans = 0, accepted = 0;
  for (int frames : frames_list)
    for (const auto& g : grids)
      for (int ns : specials)
        for (int heads : heads_list)
          for (int sigma : sigmas)
            for (unsigned flags : flag_sets)
              for (const auto& dt : dtypes)
                for (int hd : {64, 128}) {
                  vggt_attn_plan_s p;
                  std::string err;
                  const int rc = vggt::build_plan(&p, frames, g[0], g[1], ns, heads, hd, sigma, flags, dt[0], dt[1], &err);
                  ++plans;
                  if (rc != VGGT_ATTN_OK) {
                    expect(!err.empty(), "a rejected plan carries a message", frames, g[0], g[1], ns, heads, sigma, flags);
                    continue;
                  }
                  ++accepted;
                  const vggt_attn_layout_t& l = p.layout;
                  auto E = [&](bool ok, const char* what) { expect(ok, what, frames, g[0], g[1], ns, heads, sigma, flags); };
                  E(p.T == int64_t(frames) * (ns + int64_t(g[0]) * g[1]) && p.T <= vggt::kMaxTokens, "T");
                  E(p.nS >= 0 && p.nS <= p.T && p.M >= 0 && p.n_diag >= 0 && p.n_diag <= p.T, "counts in range");
                  E(p.nS + p.dropped_total == (p.g2m ? 0 : p.T) + (p.g2m ? p.T : 0) || p.g2f || !p.subsampled,
                    "kept plus dropped tokens make T");
                  E(p.segment_rows % vggt::kTile == 0 && p.segment_rows >= p.keys_per_segment, "segment rows");
                  E(p.rows_per_head <= vggt::kMaxPackedRows, "packed rows per head");
                  const int64_t offs[] = {l.off_index, l.off_dcount, l.off_means, l.off_partial, l.off_kbias,
                                          l.off_logsize, l.off_part, l.off_kmax, l.off_kpack, l.off_vpack, l.total_bytes};
                  for (int i = 0; i < 11; ++i) E(offs[i] % 256 == 0 && offs[i] >= 0, "part offsets 256-byte aligned");
                  for (int i = 1; i < 11; ++i) E(offs[i] >= offs[i - 1], "parts in order");
                  E(l.off_dcount - l.off_index >= (p.g2f ? 0 : 4 * p.nS), "index part size");
                  E(l.off_means - l.off_dcount >= 4 * int64_t(frames), "count part size");
                  E(l.off_partial - l.off_means >= int64_t(heads) * p.M * 2 * hd * int64_t(p.elem_bytes), "means part");
                  E(l.off_kmax - l.off_part >= (p.nsplit > 1 ? p.split_items * p.nsplit * p.block_rows * vggt::kPartRow * 4 : 0),
                    "split part size");
                  E(l.off_kpack - l.off_kmax >= (p.prescale_q ? 4 * int64_t(heads) : 0), "key maxima part");
                  const int64_t packed = p.inplace ? 0 : int64_t(heads) * p.rows_per_head * hd * int64_t(p.elem_bytes);
                  E(l.off_vpack - l.off_kpack >= packed && l.total_bytes - l.off_vpack >= packed, "packed parts");
                  E(!p.prescale_q || dt[0] == VGGT_ATTN_BF16, "f16 score form only for bf16 inputs");
                  E(!(p.prescale_q && p.inplace), "f16 score form packs its keys");
                  E(p.split_from + p.split_items == p.work_items && p.split_from >= 0, "work split");
                  E(p.flops >= 0.0, "flops");
                }
  std::printf("plans %ld accepted %ld violations %d\n", plans, accepted, failures);
  return failures ? 1 : 0;
}
