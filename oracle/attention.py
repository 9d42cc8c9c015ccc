"""CPU float64 oracle for VGGT global attention in its dense, SGA, enhanced-SGA and G2F forms.

TEST INFRASTRUCTURE ONLY.  Nothing on the product path may import or call this module: only the
test suite, the smoke check and the benchmark's CPU-baseline leg use it.  It shares no code with
the HIP library; the only thing both sides share is the seeded input generator in synth/.

Sources (the pages are web notes on the methods; cited by page title and section):
  [AVGGT-zh]  "AVGGT: Rethinking Global Attention for Accelerating VGGT", papernotes.org CVPR 2026
              notes: 整体框架 (layout, layer roles), 关键设计 1 (Global-to-Frame),
              关键设计 2 (SGA: sigma -> window map, first patch per window, all queries and all
              special tokens kept, frame 0 uncompressed for VGGT, the attention equation),
              关键设计 3 (diagonal self term + mean K/V, one shared softmax).
  [AVGGT-de]  gist.science summary of the same paper, "Technische Zusammenfassung" 2.B
              (one kept token per s_h x s_w window; queries and camera/register tokens kept;
              diagonal kept; dropped tokens approximated by a mean token).
  [Regime]    "RegimeVGGT: Layer-Wise Spatially Preserving Redundancy Removal ...", papernotes.org
              NeurIPS 2026 notes: 核心机制 (L = T + 5 tokens per frame), 关键设计 2 (a key that
              stands for g tokens gets +log g on its logit), 关键设计 3 (the K/V sampling grid of
              frame f is shifted by row (f div t) mod t and column f mod t; frame 0 and the
              camera/register tokens stay at full density).
  [AVGGT-abl] the AVGGT notes' ablation table (VGGT on RealEstate10K, row VGGT(G2M)) and 关键发现:
              G2M replaces the K/V of a global layer by one mean token.

Readings taken where the pages are silent (each one is a stated choice, listed in the design
notes of the repository):
  R1  in-frame order: the 5 special tokens first, then patches row-major.
  R2  sigma in {1,2,4,6,9}; sigma = 1 is dense (1x1 windows).
  R3  the window pair is (s_h, s_w): rows stride s_h, columns stride s_w.
  R4  partial windows at the grid edge count (their top-left patch is kept).
  R5  S is ordered by ascending global token id.
  R7  the softmax scale is 1/sqrt(head_dim) applied to Q.K^T; inputs are not pre-scaled.
  R8  the diagonal term is added only for a query whose own token is not in S (the three
      components are disjoint).
  R9  one mean K/V per compressed frame (frames with a nonempty dropped set), keys and values
      averaged independently over that frame's dropped patches.
  R10 mean weight: UNIT (plain token, bias 0) by default; COUNT adds ln|D_f| to its logit.
  R11 the means are per-frame constants (a dropped query's own key stays inside its mean).
  R12 the same S for every head.
  R13 means are taken of the K/V given to the op (after any upstream position encoding).
  R14 layout [H][T][d], batch 1.
  R19 phase-shifted grid ([Regime] 关键设计 3) for a window (s_h, s_w): the tile size t of the page
      becomes s_h for rows and s_w for columns, so compressed frame f keeps the patches with
      row % s_h == (f div s_w) mod s_h and column % s_w == f mod s_w.  For square windows
      (sigma 4, 9) this is the page's formula with t = s_h = s_w; for every window the offsets
      of s_h*s_w consecutive frames run through all s_h*s_w residues, so their kept sets
      partition the grid.  Frame 0 (with the reference flag) and the specials stay dense.
  R20 global mean scope: one mean K/V over the union of the dropped sets of all frames (the
      literal "single mean" of [AVGGT-zh] 关键设计 3); COUNT adds ln(sum_f |D_f|).
  R21 G2M ([AVGGT-abl]): the keys/values of every query are one token, the mean of K and of V
      over all T tokens (specials included); the output of every query is that mean value.
  R22 a frame whose dropped set is empty (possible under the phase shift on one-patch-wide
      grids) contributes no mean term.
  R23 size-aware keys ([Regime] 关键设计 2): the caller gives log g_t per token (natural log,
      finite, shared by all heads); the logit of every token key -- S, the diagonal self term,
      G2F's frame keys -- gets + log g_t.  Not combined with a mean term or G2M (the pages do not
      say how sizes enter a mean).

Parity: these functions are pinned by tests against torch's scaled-dot-product attention on
explicitly built key lists, closed-form counts, hand-enumerated index sets and exact identities.
The three-component formula of the enhanced SGA itself is printed only in the paper's
supplement, which the pages do not contain: for DIAG/MEAN the oracle follows readings R8-R11,
not the authors' unpublished code.
"""
from __future__ import annotations

from concurrent.futures import ThreadPoolExecutor
from dataclasses import dataclass

import numpy as np

# [AVGGT-zh] 关键设计 2: total factor sigma = s_h * s_w with the four listed window shapes; sigma = 1
# is plain global attention (reading R2).
SIGMA_WINDOWS = {1: (1, 1), 2: (1, 2), 4: (2, 2), 6: (2, 3), 9: (3, 3)}


@dataclass(frozen=True)
class Desc:
    """One global-attention call: geometry, heads and the accelerated form to compute."""
    frames: int
    grid_h: int
    grid_w: int
    heads: int
    head_dim: int = 64
    n_special: int = 5
    sigma: int = 1
    ref_dense: bool = True     # frame 0 uncompressed (VGGT); False = every frame compressed (pi^3)
    diag: bool = False         # diagonal self term for queries whose token is not kept
    mean: bool = False         # per-frame mean K/V of the dropped patches
    mean_count: bool = False   # mean logit += ln|D_f| (else unit weight)
    g2f: bool = False          # Global-to-Frame: each frame attends only to itself
    phase_shift: bool = False  # per-frame offset of the sampling grid (reading R19)
    mean_global: bool = False  # one mean over all dropped patches instead of one per frame (R20)
    g2m: bool = False          # K/V = one mean token over all tokens (R21)
    log_size: bool = False     # token keys carry a caller-supplied log-size bias (R23)

    def __post_init__(self):
        if self.sigma not in SIGMA_WINDOWS:
            raise ValueError(f"sigma must be one of {sorted(SIGMA_WINDOWS)}, got {self.sigma}")
        if self.g2f and (self.sigma != 1 or self.diag or self.mean):
            raise ValueError("Global-to-Frame takes no subsampling, diagonal or mean term")
        if self.g2m and (self.sigma != 1 or self.diag or self.mean or self.g2f):
            raise ValueError("G2M takes no subsampling, diagonal, per-frame mean or G2F")
        if self.mean_global and not self.mean:
            raise ValueError("mean_global selects the scope of the mean term; it needs mean=True")
        if self.log_size and (self.mean or self.g2m):
            raise ValueError("log-size keys are not combined with a mean term or G2M")
        if min(self.frames, self.grid_h, self.grid_w, self.heads, self.head_dim) < 1 or self.n_special < 0:
            raise ValueError("sizes must be positive")

    @property
    def P(self) -> int:
        return self.grid_h * self.grid_w

    @property
    def L(self) -> int:
        return self.n_special + self.P

    @property
    def T(self) -> int:
        return self.frames * self.L

    @property
    def tau(self) -> float:
        return 1.0 / np.sqrt(self.head_dim)

    @property
    def window(self) -> tuple[int, int]:
        return SIGMA_WINDOWS[self.sigma]


def as_f64(x: np.ndarray) -> np.ndarray:
    """float64 view of an input: uint16 arrays are bfloat16 bit patterns, others are floats."""
    x = np.asarray(x)
    if x.dtype == np.uint16:
        return (x.astype(np.uint32) << np.uint32(16)).view(np.float32).astype(np.float64)
    return x.astype(np.float64)


# ----------------------------------------------------------------------------------------------
# The kept set S and the dropped sets D_f
# ----------------------------------------------------------------------------------------------

def frame_is_dense(desc: Desc, f: int) -> bool:
    """[AVGGT-zh] 关键设计 2: with subsampling, VGGT keeps frame 0 as the uncompressed reference
    view while pi^3 compresses every frame; sigma = 1 compresses nothing."""
    return desc.sigma == 1 or (desc.ref_dense and f == 0)


def grid_phase(desc: Desc, f: int) -> tuple[int, int]:
    """(row offset, column offset) of the sampling grid of frame f: (0, 0) without the phase
    shift; with it, [Regime] 关键设计 3 read for an s_h x s_w window (reading R19)."""
    if not desc.phase_shift:
        return 0, 0
    s_h, s_w = desc.window
    return (f // s_w) % s_h, f % s_w


def kept_mask(desc: Desc) -> np.ndarray:
    """Boolean [T]: token t is in S.

    Token t = f*L + j; slot j < n_special is a camera/register token, always kept ([AVGGT-zh]
    关键设计 2, [AVGGT-de] 2.B).  Patch slot j >= n_special is patch p = j - n_special at row
    p // gw, column p % gw; in a compressed frame it is kept iff it is the first (top-left) patch
    of its s_h x s_w window, i.e. row % s_h == 0 and column % s_w == 0 (readings R3, R4); with
    the phase shift the windows start at the frame's offsets instead (R19).  G2M keeps no
    token (R21)."""
    s_h, s_w = desc.window
    keep = np.zeros(desc.T, dtype=bool)
    if desc.g2m:
        return keep
    for f in range(desc.frames):
        base = f * desc.L
        keep[base:base + desc.n_special] = True
        if frame_is_dense(desc, f):
            keep[base:base + desc.L] = True
            continue
        ro, co = grid_phase(desc, f)
        for p in range(desc.P):
            r, c = divmod(p, desc.grid_w)
            if r % s_h == ro and c % s_w == co:
                keep[base + desc.n_special + p] = True
    return keep


def index_set(desc: Desc) -> np.ndarray:
    """S as ascending int32 global token ids (reading R5)."""
    return np.flatnonzero(kept_mask(desc)).astype(np.int32)


def dropped_counts(desc: Desc) -> np.ndarray:
    """|D_f| per frame: the tokens of frame f that are not in S -- its dropped patches (0 for
    dense frames); under G2M every token of the frame feeds the one mean (R21)."""
    keep = kept_mask(desc).reshape(desc.frames, desc.L)
    return (~keep).sum(axis=1).astype(np.int64)


def mean_frames(desc: Desc) -> np.ndarray:
    """Frames that contribute to a mean K/V term (readings R9, R22): those with a nonempty
    dropped set, in ascending order; empty unless the MEAN form (or G2M) is on."""
    if not (desc.mean or desc.g2m) or desc.g2f:
        return np.zeros(0, dtype=np.int64)
    return np.flatnonzero(dropped_counts(desc) > 0).astype(np.int64)


def counts(desc: Desc) -> dict:
    """Sizes of one call: |S|, number of mean keys M, number of queries with a diagonal term."""
    if desc.g2f:
        return {"n_kv": desc.L, "n_mean": 0, "n_diag": 0}
    keep = kept_mask(desc)
    nm = int(mean_frames(desc).size)
    if desc.mean_global or desc.g2m:
        nm = min(nm, 1)
    return {
        "n_kv": int(keep.sum()),
        "n_mean": nm,
        "n_diag": int((~keep).sum()) if desc.diag else 0,
    }


def frame_means(k: np.ndarray, v: np.ndarray, desc: Desc):
    """Mean keys and values over the dropped tokens ([AVGGT-zh] 关键设计 3 (iii); readings
    R9, R11, R13): one per frame with a nonempty dropped set, or -- global scope (R20) and G2M
    (R21) -- a single one over the union of those sets.  Returns (kbar [H][M][d], vbar [H][M][d],
    frames [M] (the first contributing frame for a single mean), sizes [M]) in float64."""
    frames = mean_frames(desc)
    keep = kept_mask(desc)
    H, d = k.shape[0], k.shape[2]
    groups = []
    for f in frames:
        tok = np.arange(f * desc.L, (f + 1) * desc.L)
        groups.append(tok[~keep[tok]])
    if (desc.mean_global or desc.g2m) and groups:
        groups = [np.concatenate(groups)]
        frames = frames[:1]
    kbar = np.zeros((H, len(groups), d))
    vbar = np.zeros((H, len(groups), d))
    sizes = np.zeros(len(groups), dtype=np.int64)
    for m, dropped in enumerate(groups):
        sizes[m] = dropped.size
        kbar[:, m, :] = as_f64(k[:, dropped, :]).mean(axis=1)
        vbar[:, m, :] = as_f64(v[:, dropped, :]).mean(axis=1)
    return kbar, vbar, frames, sizes


# ----------------------------------------------------------------------------------------------
# Attention, gather formulation
# ----------------------------------------------------------------------------------------------

def _log_sizes(desc: Desc, log_g):
    """float64 [T] per-token log sizes: the given ones (R23), zeros without the size option."""
    if not desc.log_size:
        if log_g is not None:
            raise ValueError("log_g given for a descriptor without log_size")
        return np.zeros(desc.T)
    if log_g is None or np.shape(log_g) != (desc.T,):
        raise ValueError("log_size needs log_g of shape [T]")
    return np.asarray(log_g, dtype=np.float64)


def attention(q, k, v, desc: Desc, rows=None, workers: int = 1, chunk: int = 256, log_g=None) -> np.ndarray:
    """out[h, i, :] for query token rows[i] (all tokens if rows is None), float64 [H][R][d].

    GLOBAL form ([AVGGT-zh] 关键设计 2, the attention equation; reading R7): for query q of
    token t_q, the logits are tau*<q, k_t> for t in S, plus
      - DIAG: tau*<q, k_{t_q}> with value v_{t_q}, only if t_q is not in S (R8);
      - MEAN: tau*<q, kbar_f> + beta_f with value vbar_f for every compressed frame f, beta_f = 0
        (UNIT) or ln|D_f| (COUNT, [Regime] 关键设计 2) (R9, R10); global scope: one such term
        over the union of the dropped sets (R20);
    and the output is the softmax-weighted sum of the values under one joint normalisation.
    G2F form ([AVGGT-zh] 关键设计 1): the keys of a query are the L tokens of its own frame.
    G2M form (R21): a softmax over one key, so every output row is the mean value.
    sigma = 1 gives S = every token: plain global attention.
    With log_size, the logit of token key t also gets + log_g[t] ([Regime] 关键设计 2, R23)."""
    H, T, d = q.shape
    if T != desc.T or H != desc.heads or d != desc.head_dim:
        raise ValueError("q shape does not match the descriptor")
    rows = np.arange(T, dtype=np.int64) if rows is None else np.asarray(rows, dtype=np.int64)
    out = np.empty((H, rows.size, d))
    tau = desc.tau
    lg_size = _log_sizes(desc, log_g)

    if desc.g2m:
        vbar = frame_means(k, v, desc)[1]

        def run_head(h):
            out[h] = vbar[h, 0][None, :]
    elif desc.g2f:
        frame_of = rows // desc.L

        def run_head(h):
            for f in np.unique(frame_of):
                sel = np.flatnonzero(frame_of == f)
                kf = as_f64(k[h, f * desc.L:(f + 1) * desc.L])
                vf = as_f64(v[h, f * desc.L:(f + 1) * desc.L])
                bias = lg_size[f * desc.L:(f + 1) * desc.L]
                for c0 in range(0, sel.size, chunk):
                    s = sel[c0:c0 + chunk]
                    lg = tau * (as_f64(q[h, rows[s]]) @ kf.T) + bias[None, :]
                    out[h, s] = _joint_softmax([(lg, vf)])
    else:
        S = index_set(desc)
        keep = kept_mask(desc)
        kbar, vbar, _, sizes = frame_means(k, v, desc)
        beta = np.log(sizes.astype(np.float64)) if desc.mean_count else np.zeros(sizes.size)

        def run_head(h):
            kS, vS = as_f64(k[h, S]), as_f64(v[h, S])
            for c0 in range(0, rows.size, chunk):
                r = rows[c0:c0 + chunk]
                qr = as_f64(q[h, r])
                parts = [(tau * (qr @ kS.T) + lg_size[S][None, :], vS)]
                if kbar.shape[1]:
                    parts.append((tau * (qr @ kbar[h].T) + beta[None, :], vbar[h]))
                if desc.diag:
                    own_k, own_v = as_f64(k[h, r]), as_f64(v[h, r])
                    ls = np.where(keep[r], -np.inf, tau * np.einsum("rd,rd->r", qr, own_k) + lg_size[r])
                    parts.append((ls[:, None], own_v[:, None, :]))
                out[h, c0:c0 + r.size] = _joint_softmax(parts)

    if workers > 1:
        with ThreadPoolExecutor(max_workers=workers) as pool:
            list(pool.map(run_head, range(H)))
    else:
        for h in range(H):
            run_head(h)
    return out


def _joint_softmax(parts) -> np.ndarray:
    """Joint softmax over logit blocks.  parts: (logits [R][n], values) with values either a
    shared [n][d] block or a per-row [R][n][d] block.  Rows whose every logit of a block is -inf
    get zero weight from that block."""
    m = np.max(np.concatenate([lg for lg, _ in parts], axis=1), axis=1, keepdims=True)
    z = np.zeros_like(m)
    acc = 0.0
    for lg, val in parts:
        e = np.exp(lg - m)
        z = z + e.sum(axis=1, keepdims=True)
        acc = acc + (np.einsum("rn,rnd->rd", e, val) if val.ndim == 3 else e @ val)
    return acc / z


# ----------------------------------------------------------------------------------------------
# Attention, brute-force formulation over the full token set (small inputs only)
# ----------------------------------------------------------------------------------------------

def kept_mask_by_sets(desc: Desc) -> np.ndarray:
    """S built a second way, as a union of sets: all specials, all tokens of dense frames, and
    the grid points {(r, c): r in range(r0, gh, s_h), c in range(c0, gw, s_w)} of every other
    frame, (r0, c0) = (0, 0) or the frame's phase offsets."""
    s_h, s_w = desc.window
    keep = np.zeros(desc.T, dtype=bool)
    if desc.g2m:
        return keep
    frames = np.arange(desc.frames)
    keep[(frames[:, None] * desc.L + np.arange(desc.n_special)[None, :]).ravel()] = True
    dense = [f for f in frames if frame_is_dense(desc, int(f))]
    for f in dense:
        keep[f * desc.L:(f + 1) * desc.L] = True
    for f in frames:
        r0, c0 = ((f // s_w) % s_h, f % s_w) if desc.phase_shift else (0, 0)
        rr, cc = np.meshgrid(np.arange(r0, desc.grid_h, s_h), np.arange(c0, desc.grid_w, s_w), indexing="ij")
        keep[f * desc.L + desc.n_special + (rr * desc.grid_w + cc).ravel()] = True
    return keep


def attention_bruteforce(q, k, v, desc: Desc, log_g=None) -> np.ndarray:
    """Same operation as attention(), written as one masked softmax over T + N columns.

    Columns 0..T-1 are the tokens; column T+f is frame f's mean K/V, built with an averaging
    matrix A[f, t] = 1/|D_f| for t in D_f.  A token column is open for a query row if the token
    is in S, or (DIAG) it is the row's own token and that token is not in S; under G2F a token
    column is open iff it lies in the row's frame.  A mean column is open when MEAN is on and
    |D_f| > 0, with bias ln|D_f| under COUNT.  Global mean scope and G2M use one mean column
    whose row of A averages every token outside S.  Token column t carries + log_g[t] under the
    size option.  Meant for T up to a few thousand."""
    H, T, d = q.shape
    q64, k64, v64 = as_f64(q), as_f64(k), as_f64(v)
    N, L = desc.frames, desc.L
    lg_size = _log_sizes(desc, log_g)
    frame = np.arange(T) // L
    if desc.g2f:
        open_tok = frame[:, None] == frame[None, :]
        open_mean = np.zeros((T, N), dtype=bool)
        A = np.zeros((N, T))
        bias = np.zeros(N)
    else:
        keep = kept_mask_by_sets(desc)
        open_tok = np.broadcast_to(keep[None, :], (T, T)).copy()
        if desc.diag:
            own = np.arange(T)
            open_tok[own[~keep], own[~keep]] = True
        dropped = ~keep
        A = np.zeros((N, T))
        if desc.mean_global or desc.g2m:
            A[0, np.flatnonzero(dropped)] = 1.0
        else:
            A[frame[dropped], np.flatnonzero(dropped)] = 1.0
        size = A.sum(axis=1)
        with np.errstate(divide="ignore", invalid="ignore"):
            A = np.where(size[:, None] > 0, A / np.maximum(size, 1)[:, None], 0.0)
            bias = np.log(np.maximum(size, 1)) if desc.mean_count else np.zeros(N)
        open_mean = np.broadcast_to((size > 0) & (desc.mean or desc.g2m), (T, N)).copy()
    mask = np.concatenate([open_tok, open_mean], axis=1)
    out = np.empty((H, T, d))
    for h in range(H):
        keys = np.concatenate([k64[h], A @ k64[h]], axis=0)
        vals = np.concatenate([v64[h], A @ v64[h]], axis=0)
        lg = desc.tau * (q64[h] @ keys.T)
        lg[:, T:] += bias[None, :]
        lg[:, :T] += lg_size[None, :]
        lg = np.where(mask, lg, -np.inf)
        w = np.exp(lg - lg.max(axis=1, keepdims=True))
        w /= w.sum(axis=1, keepdims=True)
        out[h] = w @ vals
    return out
