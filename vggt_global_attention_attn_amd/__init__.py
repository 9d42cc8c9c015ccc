"""MI355X-native forward pass of VGGT global attention: dense, AVGGT subsampled (SGA, with an
optional phase-shifted grid), enhanced SGA (diagonal + per-frame or global mean K/V),
Global-to-Frame and Global-to-Mean, with optional size-aware keys, behind a C ABI (include/vggt_attn.h) implemented by
hand-written gfx950 HIP kernels."""
from .binding import (BF16, DIAG, EXPORTS, FP32, G2F, G2M, GLOBAL_LAYERS, LIB_PATH, LOG_SIZE, MEAN, MEAN_COUNT,
                      MEAN_GLOBAL, MODELS, PHASE_SHIFT, PRESCALE_Q, REF_DENSE, Plan, ScheduledLayers, VggtAttnError,
                      attention, layer_schedule, lib)

__all__ = ["BF16", "DIAG", "EXPORTS", "FP32", "G2F", "G2M", "GLOBAL_LAYERS", "LIB_PATH", "LOG_SIZE", "MEAN",
           "MEAN_COUNT", "MEAN_GLOBAL", "MODELS", "PHASE_SHIFT", "PRESCALE_Q", "REF_DENSE", "Plan", "ScheduledLayers",
           "VggtAttnError", "attention", "layer_schedule", "lib"]
