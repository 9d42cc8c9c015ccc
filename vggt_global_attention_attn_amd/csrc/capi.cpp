// C ABI entry points: argument checks, then kernel launches on the caller's stream.
#include <hip/hip_runtime_api.h>

#include <cstdint>
#include <cstdio>
#include <new>
#include <string>

#include "launch.h"
#include "plan.h"
#include "vggt_attn.h"

namespace {

thread_local std::string g_last_error;

int set_error(int code, const std::string& msg) {
  g_last_error = msg;
  return code;
}

int ok() {
  g_last_error.clear();
  return VGGT_ATTN_OK;
}

int hip_error(hipError_t e, const char* what) {
  return set_error(VGGT_ATTN_EHIP, std::string(what) + ": " + hipGetErrorString(e));
}

bool misaligned(const void* ptr) { return (reinterpret_cast<uintptr_t>(ptr) & 15u) != 0; }

bool overlaps(const void* a, size_t na, const void* b, size_t nb) {
  const uintptr_t x = reinterpret_cast<uintptr_t>(a), y = reinterpret_cast<uintptr_t>(b);
  return na && nb && x < y + nb && y < x + na;
}

size_t tensor_bytes(const vggt_attn_plan_s& p, int dtype) {
  return size_t(p.heads) * size_t(p.T) * size_t(p.head_dim) * (dtype == VGGT_ATTN_BF16 ? 2 : 4);
}

int check_workspace(const vggt_attn_plan_s& p, const void* ws, size_t ws_bytes) {
  if (!ws) return set_error(VGGT_ATTN_EINVAL, "workspace is NULL");
  if (misaligned(ws)) return set_error(VGGT_ATTN_EALIGN, "workspace is not 16-byte aligned");
  if (ws_bytes < size_t(p.layout.total_bytes))
    return set_error(VGGT_ATTN_ENOSPC, "workspace has " + std::to_string(ws_bytes) + " bytes, needs " +
                                           std::to_string(p.layout.total_bytes));
  return VGGT_ATTN_OK;
}

int check_tensors(const vggt_attn_plan_s& p, const void* q, const void* k, const void* v,
                  const void* out, bool need_q_out) {
  if (!k || !v || (need_q_out && (!q || !out))) return set_error(VGGT_ATTN_EINVAL, "NULL tensor pointer");
  if (misaligned(k) || misaligned(v) || (need_q_out && (misaligned(q) || misaligned(out))))
    return set_error(VGGT_ATTN_EALIGN, "tensor pointer is not 16-byte aligned");
  return VGGT_ATTN_OK;
}

int check_out_alias(const vggt_attn_plan_s& p, const void* q, const void* k, const void* v,
                    const void* out, const void* ws, size_t ws_bytes) {
  const size_t nin = tensor_bytes(p, p.in_dtype), nout = tensor_bytes(p, p.out_dtype);
  if (overlaps(out, nout, q, nin) || overlaps(out, nout, k, nin) || overlaps(out, nout, v, nin) ||
      overlaps(out, nout, ws, ws_bytes))
    return set_error(VGGT_ATTN_EALIAS, "out overlaps q, k, v or the workspace");
  return VGGT_ATTN_OK;
}

int do_pack(const vggt_attn_plan_s& p, const void* k, const void* v, const float* log_g, void* ws,
            hipStream_t s) {
  hipError_t e = vggt::launch_means(p, k, v, ws, s);
  if (e != hipSuccess) return hip_error(e, "means kernel launch");
  e = vggt::launch_pack(p, k, v, ws, s);
  if (e != hipSuccess) return hip_error(e, "pack kernel launch");
  if (p.log_size) {
    e = vggt::launch_size_bias(p, log_g, ws, s);
    if (e != hipSuccess) return hip_error(e, "size bias kernel launch");
  }
  return VGGT_ATTN_OK;
}

// log_g of a LOG_SIZE plan: present, 4-byte aligned, not overlapping `out` or the workspace.
int check_log_g(const vggt_attn_plan_s& p, const float* log_g, const void* out, const void* ws,
                size_t ws_bytes) {
  if (!p.log_size) return set_error(VGGT_ATTN_EINVAL, "plan has no LOG_SIZE flag: use the plain entry points");
  if (!log_g) return set_error(VGGT_ATTN_EINVAL, "log_g is NULL");
  if (reinterpret_cast<uintptr_t>(log_g) & 3u) return set_error(VGGT_ATTN_EALIGN, "log_g is not 4-byte aligned");
  const size_t n = size_t(p.T) * 4;
  if (overlaps(log_g, n, ws, ws_bytes) || (out && overlaps(log_g, n, out, tensor_bytes(p, p.out_dtype))))
    return set_error(VGGT_ATTN_EALIAS, "log_g overlaps out or the workspace");
  return VGGT_ATTN_OK;
}

int no_log_size(const vggt_attn_plan_s& p) {
  if (p.log_size) return set_error(VGGT_ATTN_EINVAL, "plan has LOG_SIZE: use the *_sized entry points");
  return VGGT_ATTN_OK;
}

int pack_impl(const vggt_attn_plan_s& p, const void* k, const void* v, const float* log_g, void* workspace,
              size_t workspace_bytes, void* stream) {
  int rc = check_tensors(p, nullptr, k, v, nullptr, false);
  if (rc) return rc;
  if ((rc = check_workspace(p, workspace, workspace_bytes))) return rc;
  const size_t nin = tensor_bytes(p, p.in_dtype);
  if (overlaps(workspace, workspace_bytes, k, nin) || overlaps(workspace, workspace_bytes, v, nin))
    return set_error(VGGT_ATTN_EALIAS, "workspace overlaps k or v");
  if ((rc = do_pack(p, k, v, log_g, workspace, static_cast<hipStream_t>(stream)))) return rc;
  return ok();
}

int forward_impl(const vggt_attn_plan_s& p, const void* q, const void* k, const void* v, const float* log_g,
                 void* out, void* workspace, size_t workspace_bytes, void* stream) {
  int rc = check_tensors(p, q, k, v, out, true);
  if (rc) return rc;
  if ((rc = check_workspace(p, workspace, workspace_bytes))) return rc;
  if ((rc = check_out_alias(p, q, k, v, out, workspace, workspace_bytes))) return rc;
  const size_t nin = tensor_bytes(p, p.in_dtype);
  if (overlaps(workspace, workspace_bytes, k, nin) || overlaps(workspace, workspace_bytes, v, nin) ||
      overlaps(workspace, workspace_bytes, q, nin))
    return set_error(VGGT_ATTN_EALIAS, "workspace overlaps q, k or v");
  const hipStream_t s = static_cast<hipStream_t>(stream);
  if ((rc = do_pack(p, k, v, log_g, workspace, s))) return rc;
  hipError_t e = vggt::launch_attend(p, q, k, v, out, workspace, s);
  if (e != hipSuccess) return hip_error(e, "attention kernel launch");
  return ok();
}

}  // namespace

extern "C" {

int vggt_attn_plan(vggt_attn_plan_t** out, int frames, int grid_h, int grid_w, int n_special,
                   int heads, int head_dim, int sigma, unsigned flags, int in_dtype,
                   int out_dtype) {
  if (!out) return set_error(VGGT_ATTN_EINVAL, "plan output pointer is NULL");
  *out = nullptr;
  auto* p = new (std::nothrow) vggt_attn_plan_s();
  if (!p) return set_error(VGGT_ATTN_EINVAL, "out of host memory");
  std::string err;
  const int rc = vggt::build_plan(p, frames, grid_h, grid_w, n_special, heads, head_dim, sigma,
                                  flags, in_dtype, out_dtype, &err);
  if (rc != VGGT_ATTN_OK) {
    delete p;
    return set_error(rc, err);
  }
  *out = p;
  return ok();
}

void vggt_attn_plan_destroy(vggt_attn_plan_t* plan) { delete plan; }

size_t vggt_attn_workspace_bytes(const vggt_attn_plan_t* plan) {
  return plan ? size_t(plan->layout.total_bytes) : 0;
}

int vggt_attn_counts(const vggt_attn_plan_t* plan, int64_t* n_kv, int64_t* n_mean,
                     int64_t* n_diag, double* flops) {
  if (!plan) return set_error(VGGT_ATTN_EINVAL, "plan is NULL");
  if (n_kv) *n_kv = plan->g2f ? plan->L : plan->nS;
  if (n_mean) *n_mean = plan->M;
  if (n_diag) *n_diag = plan->n_diag;
  if (flops) *flops = plan->flops;
  return ok();
}

int vggt_attn_layout(const vggt_attn_plan_t* plan, vggt_attn_layout_t* out) {
  if (!plan || !out) return set_error(VGGT_ATTN_EINVAL, "NULL argument");
  *out = plan->layout;
  return ok();
}

int vggt_attn_pack(const vggt_attn_plan_t* plan, const void* k, const void* v, void* workspace,
                   size_t workspace_bytes, void* stream) {
  if (!plan) return set_error(VGGT_ATTN_EINVAL, "plan is NULL");
  if (int rc = no_log_size(*plan)) return rc;
  return pack_impl(*plan, k, v, nullptr, workspace, workspace_bytes, stream);
}

int vggt_attn_pack_sized(const vggt_attn_plan_t* plan, const void* k, const void* v, const float* log_g,
                         void* workspace, size_t workspace_bytes, void* stream) {
  if (!plan) return set_error(VGGT_ATTN_EINVAL, "plan is NULL");
  if (int rc = check_log_g(*plan, log_g, nullptr, workspace, workspace_bytes)) return rc;
  return pack_impl(*plan, k, v, log_g, workspace, workspace_bytes, stream);
}

int vggt_attn_attend(const vggt_attn_plan_t* plan, const void* q, const void* k, const void* v,
                     void* out, void* workspace, size_t workspace_bytes, void* stream) {
  if (!plan) return set_error(VGGT_ATTN_EINVAL, "plan is NULL");
  int rc = check_tensors(*plan, q, k, v, out, true);
  if (rc) return rc;
  if ((rc = check_workspace(*plan, workspace, workspace_bytes))) return rc;
  if ((rc = check_out_alias(*plan, q, k, v, out, workspace, workspace_bytes))) return rc;
  // (the attention stage writes the split pieces' partial states into the workspace)
  const size_t nin = tensor_bytes(*plan, plan->in_dtype);
  if (overlaps(workspace, workspace_bytes, k, nin) || overlaps(workspace, workspace_bytes, v, nin) ||
      overlaps(workspace, workspace_bytes, q, nin))
    return set_error(VGGT_ATTN_EALIAS, "workspace overlaps q, k or v");
  hipError_t e = vggt::launch_attend(*plan, q, k, v, out, workspace, static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return hip_error(e, "attention kernel launch");
  return ok();
}

int vggt_attn_forward(const vggt_attn_plan_t* plan, const void* q, const void* k, const void* v,
                      void* out, void* workspace, size_t workspace_bytes, void* stream) {
  if (!plan) return set_error(VGGT_ATTN_EINVAL, "plan is NULL");
  if (int rc = no_log_size(*plan)) return rc;
  return forward_impl(*plan, q, k, v, nullptr, out, workspace, workspace_bytes, stream);
}

int vggt_attn_forward_sized(const vggt_attn_plan_t* plan, const void* q, const void* k, const void* v,
                            const float* log_g, void* out, void* workspace, size_t workspace_bytes,
                            void* stream) {
  if (!plan) return set_error(VGGT_ATTN_EINVAL, "plan is NULL");
  if (int rc = check_log_g(*plan, log_g, out, workspace, workspace_bytes)) return rc;
  return forward_impl(*plan, q, k, v, log_g, out, workspace, workspace_bytes, stream);
}

int vggt_attn_forward_noalloc(const vggt_attn_plan_t* plan, const void* q, const void* k, const void* v,
                              void* out, void* stream) {
  if (!plan) return set_error(VGGT_ATTN_EINVAL, "plan is NULL");
  if (int rc = no_log_size(*plan)) return rc;
  if (size_t(plan->layout.total_bytes) > vggt::kScratchBytes)
    return set_error(VGGT_ATTN_ENOSPC, "plan needs " + std::to_string(plan->layout.total_bytes) +
                                           " bytes of workspace; the no-allocation entry point has " +
                                           std::to_string(vggt::kScratchBytes) + " (use vggt_attn_forward)");
  void* ws = nullptr;
  const hipError_t e = vggt::scratch_address(&ws);
  if (e != hipSuccess) return hip_error(e, "static workspace address");
  return forward_impl(*plan, q, k, v, nullptr, out, ws, vggt::kScratchBytes, stream);
}

int vggt_attn_layer_schedule(int model, int layer, int sigma, int* out_sigma, unsigned* out_flags) {
  // AVGGT notes, 整体框架: t_early = 9 (VGGT) or 10 (pi^3); ablation row AVGGT(2)-: late = 20..23.
  constexpr int kGlobalLayers = 24, kLateFrom = 20;
  int t_early;
  if (model == VGGT_ATTN_MODEL_VGGT) t_early = 9;
  else if (model == VGGT_ATTN_MODEL_PI3) t_early = 10;
  else return set_error(VGGT_ATTN_EINVAL, "model must be VGGT_ATTN_MODEL_VGGT or VGGT_ATTN_MODEL_PI3");
  if (layer < 0 || layer >= kGlobalLayers)
    return set_error(VGGT_ATTN_EINVAL, "layer " + std::to_string(layer) + " not in [0, 24)");
  if (sigma != 1 && sigma != 2 && sigma != 4 && sigma != 6 && sigma != 9)
    return set_error(VGGT_ATTN_EINVAL, "sigma " + std::to_string(sigma) + " not in {1, 2, 4, 6, 9}");
  int s = 1;
  unsigned f = 0;
  if (layer < t_early) {
    f = VGGT_ATTN_G2F;
  } else if (layer < kLateFrom) {
    s = sigma;
    if (sigma > 1) f = VGGT_ATTN_DIAG | VGGT_ATTN_MEAN | (model == VGGT_ATTN_MODEL_VGGT ? VGGT_ATTN_REF_DENSE : 0u);
  }
  if (out_sigma) *out_sigma = s;
  if (out_flags) *out_flags = f;
  return ok();
}

int vggt_attn_copy_index_set(const vggt_attn_plan_t* plan, const void* workspace,
                             int32_t* host_idx, int32_t* host_dcount, void* stream) {
  if (!plan || !workspace) return set_error(VGGT_ATTN_EINVAL, "NULL argument");
  const hipStream_t s = static_cast<hipStream_t>(stream);
  const char* base = static_cast<const char*>(workspace);
  hipError_t e;
  if (host_idx && !plan->g2f && plan->nS > 0) {
    e = hipMemcpyAsync(host_idx, base + plan->layout.off_index, size_t(plan->nS) * 4,
                       hipMemcpyDeviceToHost, s);
    if (e != hipSuccess) return hip_error(e, "index copy");
  }
  if (host_dcount) {
    e = hipMemcpyAsync(host_dcount, base + plan->layout.off_dcount, size_t(plan->frames) * 4,
                       hipMemcpyDeviceToHost, s);
    if (e != hipSuccess) return hip_error(e, "dcount copy");
  }
  e = hipStreamSynchronize(s);
  if (e != hipSuccess) return hip_error(e, "stream synchronize");
  return ok();
}

const char* vggt_attn_last_error(void) { return g_last_error.c_str(); }

}  // extern "C"
