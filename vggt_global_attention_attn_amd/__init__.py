"""MI355X-native forward pass of VGGT global attention: dense, AVGGT subsampled (SGA),
enhanced SGA (diagonal + per-frame mean K/V) and Global-to-Frame, behind a C ABI
(include/vggt_attn.h) implemented by hand-written gfx950 HIP kernels."""
from .binding import (BF16, DIAG, EXPORTS, FP32, G2F, LIB_PATH, MEAN, MEAN_COUNT, PRESCALE_Q, REF_DENSE,
                      Plan, VggtAttnError, attention, lib)

__all__ = ["BF16", "DIAG", "EXPORTS", "FP32", "G2F", "LIB_PATH", "MEAN", "MEAN_COUNT", "PRESCALE_Q", "REF_DENSE", "Plan",
           "VggtAttnError", "attention", "lib"]
