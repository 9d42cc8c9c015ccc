"""Helpers for the GPU tests: upload seeded inputs, compare with the oracle."""
import numpy as np

from synth import make_qkv

BF16_MAX_ABS = 2e-2
BF16_REL_L2 = 5e-3
FP32_MAX_ABS = 1e-5
FP32_REL_L2 = 1e-5


def to_device(x, device="cuda"):
    import torch
    if x.dtype == np.uint16:
        return torch.from_numpy(np.ascontiguousarray(x).view(np.int16)).view(torch.bfloat16).to(device)
    return torch.from_numpy(np.ascontiguousarray(x)).to(device)


def errors(got, ref):
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    diff = got - ref
    max_abs = float(np.max(np.abs(diff))) if diff.size else 0.0
    rel = float(np.linalg.norm(diff) / max(np.linalg.norm(ref), 1e-300)) if diff.size else 0.0
    return max_abs, rel


def assert_close(got, ref, fp32: bool, label: str = ""):
    max_abs, rel = errors(got, ref)
    lim_abs, lim_rel = (FP32_MAX_ABS, FP32_REL_L2) if fp32 else (BF16_MAX_ABS, BF16_REL_L2)
    assert np.all(np.isfinite(got)), f"{label}: non-finite output"
    assert max_abs <= lim_abs and rel <= lim_rel, f"{label}: max-abs {max_abs:.3e} (<= {lim_abs}), rel-L2 {rel:.3e} (<= {lim_rel})"
    return max_abs, rel


def inputs_for(desc, dtype, seed=0):
    return make_qkv(desc.frames, desc.grid_h, desc.grid_w, desc.n_special, desc.heads, desc.head_dim,
                    dtype=dtype, seed=seed)


def plan_kwargs(desc, in_dtype="bf16", out_dtype="fp32"):
    return dict(frames=desc.frames, grid_h=desc.grid_h, grid_w=desc.grid_w, heads=desc.heads,
                head_dim=desc.head_dim, n_special=desc.n_special, sigma=desc.sigma, ref_dense=desc.ref_dense,
                diag=desc.diag, mean=desc.mean, mean_count=desc.mean_count, g2f=desc.g2f,
                phase_shift=desc.phase_shift, mean_global=desc.mean_global, g2m=desc.g2m, log_size=desc.log_size,
                in_dtype=in_dtype, out_dtype=out_dtype)
