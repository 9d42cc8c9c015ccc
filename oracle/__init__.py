"""CPU float64 oracle for VGGT global attention (test infrastructure only).

Only the test suite, the smoke check and the benchmark's CPU-baseline leg may import this
package; the HIP library never does."""
from .attention import (SIGMA_WINDOWS, Desc, as_f64, attention, attention_bruteforce, counts,
                        dropped_counts, frame_is_dense, frame_means, index_set, kept_mask,
                        kept_mask_by_sets, mean_frames)

__all__ = ["SIGMA_WINDOWS", "Desc", "as_f64", "attention", "attention_bruteforce", "counts",
           "dropped_counts", "frame_is_dense", "frame_means", "index_set", "kept_mask",
           "kept_mask_by_sets", "mean_frames"]
