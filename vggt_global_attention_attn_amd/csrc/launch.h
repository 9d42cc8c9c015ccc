// Kernel launchers (defined in the .hip files) used by the C ABI.  Each enqueues on `stream`
// and returns the hipError_t of the launch.
#pragma once

#include <hip/hip_runtime_api.h>

#include "plan.h"

namespace vggt {

// Mean key/value of the dropped patches of every compressed frame -> workspace means area.
hipError_t launch_means(const vggt_attn_plan_s& p, const void* k, const void* v, void* ws,
                        hipStream_t stream);

// S, |D_f|, and the packed key/value tiles -> workspace.  Runs after launch_means.
hipError_t launch_pack(const vggt_attn_plan_s& p, const void* k, const void* v, void* ws,
                       hipStream_t stream);

// LOG_SIZE plans: packed per-key logit bias and a copy of log_g -> workspace.
hipError_t launch_size_bias(const vggt_attn_plan_s& p, const float* log_g, void* ws, hipStream_t stream);

// Attention over the packed keys (bf16 inputs: MFMA kernel; fp32 inputs: fp32 kernel).
hipError_t launch_attend(const vggt_attn_plan_s& p, const void* q, const void* k, const void* v,
                         void* out, void* ws, hipStream_t stream);

// Device address, on the current device, of the static workspace of the no-allocation entry
// point (kScratchBytes bytes); looked up once per device.
hipError_t scratch_address(void** out);

}  // namespace vggt
