"""Seeded synthetic inputs for VGGT global attention: test and benchmark infrastructure.

This module is shared by the CPU oracle side and the GPU side.  It draws random numbers, mixes
them into the shared-position recipe below, and rounds to bfloat16.  It contains no attention
arithmetic at all (no index sets, no softmax, no means).

Token geometry (AVGGT page, "整体框架" and design 1; RegimeVGGT page, "核心机制"): a sequence
has N frames of L = n_special + gh*gw tokens each, T = N*L tokens in all.  Within a frame the
n_special camera/register tokens come first and the gh x gw patch tokens follow in row-major
order.  Tensors are laid out [H][T][d] (heads, tokens, channels), frame-major along T.

Value recipe, for each of Q, K, V independently:
    x[h, f*L + j, :] = 0.7 * u[h, j, :] + 0.7 * noise_f[h, j, :]
u is one standard-normal draw per in-frame slot (specials included) shared by every frame, and
noise_f is a fresh standard-normal draw per frame; the sum is formed in float32 and rounded to
bfloat16 with round-to-nearest-even (or kept as float32 for fp32 workloads).  The shared term
makes the same grid position correlate across frames, the structure that global attention in
VGGT matches across views.

Random stream: one numpy Generator(PCG64(seed)), drawn in this order: for X in (Q, K, V), first
u_X as one (H, L, d) float32 standard-normal array, then the noise of frame 0, 1, ..., N-1, each
one (H, L, d) float32 array.  The draws are sequential; combining and rounding run on all host
cores beside them.  `per_frame_streams=True` swaps in independent streams instead (PCG64 from
SeedSequence(entropy=seed, spawn_key=(tensor, 0)) for u and (tensor, 1, frame) for each frame's
noise, tensor 0/1/2 = Q/K/V), which draw in parallel: used only for the largest edge-case
geometry, whose billions of values one stream draws too slowly.
"""
from __future__ import annotations

import os
from concurrent.futures import ThreadPoolExecutor

import numpy as np

__all__ = [
    "tokens_per_frame",
    "f32_to_bf16_bits",
    "bf16_bits_to_f32",
    "make_qkv",
    "sample_rows",
    "host_threads",
    "make_log_sizes",
]


def host_threads() -> int:
    """Number of host threads this process may use (its CPU affinity set, capped at 16)."""
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:  # pragma: no cover
        n = os.cpu_count() or 1
    return max(1, min(16, n))


def tokens_per_frame(grid_h: int, grid_w: int, n_special: int) -> int:
    return n_special + grid_h * grid_w


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 values to bfloat16 (IEEE round-to-nearest-even); returns the uint16 bits.

    Inputs are finite by construction; NaN handling is not needed here."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    bias = np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1))
    return ((u + bias) >> np.uint32(16)).astype(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    """Exact widening of bfloat16 bits (uint16) to float32."""
    return (np.ascontiguousarray(b, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


def _rng(seed: int, *key: int) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence(entropy=seed, spawn_key=key)))


def make_qkv(frames: int, grid_h: int, grid_w: int, n_special: int, heads: int, head_dim: int,
             dtype: str = "bf16", seed: int = 0, workers: int | None = None,
             shared: float = 0.7, noise: float = 0.7, tie_qk: bool = False,
             per_frame_streams: bool = False):
    """Draw Q, K, V of shape [heads][frames*L][head_dim].

    dtype "bf16" returns uint16 arrays of bfloat16 bits; "fp32" returns float32 arrays.
    The same (geometry, seed, per_frame_streams) always gives the same bytes, whatever the
    worker count.  tie_qk: K takes Q's per-position component u_Q (a stress input: a query's
    logits then peak at its own slot in every frame); u_K is still drawn, so the noise draws
    keep their places in the stream."""
    if dtype not in ("bf16", "fp32"):
        raise ValueError(f"dtype must be 'bf16' or 'fp32', got {dtype!r}")
    L = tokens_per_frame(grid_h, grid_w, n_special)
    T = frames * L
    out_dtype = np.uint16 if dtype == "bf16" else np.float32
    workers = workers or host_threads()
    shape = (heads, L, head_dim)
    rng = np.random.Generator(np.random.PCG64(seed))
    result = {}
    u_q = None
    with ThreadPoolExecutor(max_workers=workers) as pool:
        for ti, name in enumerate(("q", "k", "v")):
            if per_frame_streams:
                u = _rng(seed, 0 if (tie_qk and name == "k") else ti, 0).standard_normal(shape, dtype=np.float32)
            else:
                u = rng.standard_normal(shape, dtype=np.float32)
                if name == "q":
                    u_q = u.copy()
                elif tie_qk and name == "k":
                    u = u_q.copy()
            u *= np.float32(shared)
            x = np.empty((heads, T, head_dim), dtype=out_dtype)

            def finish(f: int, nz: np.ndarray, u=u, x=x):
                nz *= np.float32(noise)
                nz += u
                x[:, f * L:(f + 1) * L, :] = f32_to_bf16_bits(nz) if dtype == "bf16" else nz

            if per_frame_streams:
                def fill(f: int, ti=ti):
                    finish(f, _rng(seed, ti, 1, f).standard_normal(shape, dtype=np.float32))

                list(pool.map(fill, range(frames)))
            else:
                # the draws stay in stream order; at most 2 * workers frames wait to be finished
                pending = []
                for f in range(frames):
                    pending.append(pool.submit(finish, f, rng.standard_normal(shape, dtype=np.float32)))
                    if len(pending) >= 2 * workers:
                        pending.pop(0).result()
                for fut in pending:
                    fut.result()
            result[name] = x
    return result["q"], result["k"], result["v"]


def sample_rows(frames: int, grid_h: int, grid_w: int, n_special: int, count: int = 4096,
                seed: int = 1) -> np.ndarray:
    """Seeded query rows for sampled parity checks at full size.

    A forced set first: for frames {0, 1, N//2, N-1}, every special slot, the four grid corners,
    the patches next to the first corner, and a 3x3 block of interior patches (which holds both
    a kept and a dropped position for every window shape up to 3x3).  The rest are drawn
    uniformly without replacement with PCG64(seed).  Returns sorted unique token ids (int64)."""
    L = tokens_per_frame(grid_h, grid_w, n_special)
    T = frames * L
    if count >= T:
        return np.arange(T, dtype=np.int64)
    forced = []
    cells = {(0, 0), (0, 1), (1, 0), (0, grid_w - 1), (grid_h - 1, 0), (grid_h - 1, grid_w - 1)}
    r0, c0 = grid_h // 2, grid_w // 2
    for dr in range(3):
        for dc in range(3):
            cells.add((min(r0 + dr, grid_h - 1), min(c0 + dc, grid_w - 1)))
    for f in sorted({0, min(1, frames - 1), frames // 2, frames - 1}):
        base = f * L
        forced.extend(base + j for j in range(n_special))
        forced.extend(base + n_special + r * grid_w + c for (r, c) in sorted(cells))
    forced = np.unique(np.asarray(forced, dtype=np.int64))
    rest = max(0, count - forced.size)
    pool = np.setdiff1d(np.arange(T, dtype=np.int64), forced, assume_unique=True)
    draw = np.random.Generator(np.random.PCG64(seed)).choice(pool, size=min(rest, pool.size), replace=False)
    return np.unique(np.concatenate([forced, draw.astype(np.int64)]))


def make_log_sizes(frames: int, grid_h: int, grid_w: int, n_special: int, seed: int = 0, max_size: int = 4):
    """Per-token group sizes g (int64, uniform in 1..max_size) and their natural logs as float32,
    the form in which a caller hands sizes to the library: synthetic stand-ins for the token
    counts behind merged tokens.  One PCG64 stream, spawn_key=(3, 0)."""
    T = frames * tokens_per_frame(grid_h, grid_w, n_special)
    g = _rng(seed, 3, 0).integers(1, max_size + 1, size=T, dtype=np.int64)
    return g, np.log(g.astype(np.float64)).astype(np.float32)
