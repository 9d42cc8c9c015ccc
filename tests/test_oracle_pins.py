"""Pins for the CPU oracle: checks against things other than the oracle itself.

Each check ties the oracle to a fact the pages fix or to an independent route:
  * hand-enumerated index sets (tests/golden, derived from the first-patch-per-window rule of
    the AVGGT notes, 关键设计 2) and closed-form set sizes;
  * torch's scaled_dot_product_attention (float64, CPU) on explicitly built key/value lists --
    a library routine standing in for the plain attention equation of 关键设计 2;
  * exact identities: a COUNT-weighted mean equals |D_f| copies of the mean token (RegimeVGGT
    notes, 关键设计 2, the log g bias); identical dropped rows make enhanced SGA collapse to dense
    attention; shift invariance in K; linearity in V; V = 1 gives 1;
  * the oracle's own brute-force (full-mask) formulation, on small and odd grids;
  * for the phase-shifted grid (RegimeVGGT notes, 关键设计 3): a hand-enumerated index set, the
    page's offset formula for square windows, and the coverage the page states (consecutive
    frames' grids together cover every patch);
  * for the global mean scope and G2M: explicit key lists through torch SDPA, and the collapse
    identity (identical keys give uniform weights, so attention returns the mean value);
  * for size-aware keys (RegimeVGGT notes, 关键设计 2): a key standing for g tokens equals g
    copies of it in a plain attention (integer g, through torch SDPA).
"""
import math
import os

import numpy as np
import pytest
import torch

import oracle
from oracle import Desc
from synth import bf16_bits_to_f32, f32_to_bf16_bits, make_log_sizes, make_qkv, sample_rows

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def load_golden(name):
    vals = []
    with open(os.path.join(GOLDEN, name)) as fh:
        for line in fh:
            line = line.split("#", 1)[0].strip()
            if line:
                vals.extend(int(x) for x in line.split())
    return np.asarray(vals, dtype=np.int64)


def f64(x):
    return bf16_bits_to_f32(x).astype(np.float64) if x.dtype == np.uint16 else x.astype(np.float64)


def sdpa(q, k, v):
    """torch SDPA, float64 on the CPU; q [.., R, d], k/v [.., n, d]."""
    with torch.no_grad():
        return torch.nn.functional.scaled_dot_product_attention(
            torch.from_numpy(np.ascontiguousarray(q)), torch.from_numpy(np.ascontiguousarray(k)),
            torch.from_numpy(np.ascontiguousarray(v))).numpy()


def inputs(desc, dtype="bf16", seed=0):
    return make_qkv(desc.frames, desc.grid_h, desc.grid_w, desc.n_special, desc.heads, desc.head_dim,
                    dtype=dtype, seed=seed)


GOLD_DESC = dict(frames=3, grid_h=5, grid_w=7, heads=2, sigma=6, ref_dense=True)


def hand_S():
    return load_golden("index_set_3f_5x7_sigma6.txt")


def hand_dropped(frame):
    """Dropped patches of a compressed frame of the 3 x (5x7) golden geometry: every patch token
    of the frame that the hand-enumerated S does not list."""
    L = 40
    S = set(hand_S().tolist())
    return np.asarray([t for t in range(frame * L + 5, (frame + 1) * L) if t not in S])


# ------------------------------------------------------------------------------------------
# Index set
# ------------------------------------------------------------------------------------------

def test_sigma_windows_as_listed_on_the_page():
    # AVGGT notes 关键设计 2: 2 -> (1,2), 4 -> (2,2), 6 -> (2,3), 9 -> (3,3); sigma = s_h * s_w.
    assert oracle.SIGMA_WINDOWS[2] == (1, 2)
    assert oracle.SIGMA_WINDOWS[4] == (2, 2)
    assert oracle.SIGMA_WINDOWS[6] == (2, 3)
    assert oracle.SIGMA_WINDOWS[9] == (3, 3)
    for s, (a, b) in oracle.SIGMA_WINDOWS.items():
        assert a * b == s


def test_index_set_hand_enumerated_nonsquare_grid():
    d = Desc(**GOLD_DESC)
    assert np.array_equal(oracle.index_set(d), hand_S())
    assert np.array_equal(np.flatnonzero(oracle.kept_mask_by_sets(d)), hand_S())
    assert list(oracle.dropped_counts(d)) == [0, 26, 26]


def test_index_set_hand_enumerated_pi3():
    d = Desc(frames=4, grid_h=8, grid_w=8, heads=2, sigma=4, ref_dense=False, diag=True, mean=True)
    gold = load_golden("index_set_tiny_pi3.txt")
    assert np.array_equal(oracle.index_set(d), gold)
    c = oracle.counts(d)
    assert (c["n_kv"], c["n_mean"], c["n_diag"]) == (84, 4, 192)


@pytest.mark.parametrize("N,gh,gw,sigma,ref,expect", [
    (4, 8, 8, 4, True, 132),            # tiny workload
    (32, 37, 37, 1, True, 43968),       # dense, every token
    (100, 37, 37, 4, True, 37608),
    (200, 37, 37, 9, True, 36000),
    (800, 37, 37, 6, True, 202722),     # "about 203k K/V tokens" at 800 frames, sigma 6
    (3, 5, 7, 2, True, 40 + 2 * (5 + 5 * 4)),
    (3, 5, 7, 2, False, 3 * (5 + 5 * 4)),
])
def test_index_set_size_closed_form(N, gh, gw, sigma, ref, expect):
    s_h, s_w = oracle.SIGMA_WINDOWS[sigma]
    ref = ref and sigma > 1
    closed = N * 5 + gh * gw * int(ref or sigma == 1) + (N - int(ref)) * math.ceil(gh / s_h) * math.ceil(gw / s_w) \
        if sigma > 1 else N * (5 + gh * gw)
    assert closed == expect
    d = Desc(frames=N, grid_h=gh, grid_w=gw, heads=1, sigma=sigma, ref_dense=ref)
    if N * (5 + gh * gw) <= 400_000:
        assert int(oracle.kept_mask(d).sum()) == expect
        assert np.array_equal(oracle.kept_mask(d), oracle.kept_mask_by_sets(d))
    else:  # counts only at full size: the per-patch loop runs once per frame
        assert oracle.counts(d)["n_kv"] == expect
    # about 203k K/V tokens including the means at 800 frames
    if N == 800:
        dm = Desc(frames=N, grid_h=gh, grid_w=gw, heads=1, sigma=sigma, diag=True, mean=True)
        c = oracle.counts(dm)
        assert c["n_mean"] == 799 and c["n_diag"] == 799 * 1122
        assert 202_000 < c["n_kv"] + c["n_mean"] < 204_000


# ------------------------------------------------------------------------------------------
# Attention against torch SDPA on explicit key lists
# ------------------------------------------------------------------------------------------

@pytest.mark.parametrize("flags", [dict(), dict(diag=True, mean=True), dict(diag=True, mean=True, mean_count=True)])
def test_sigma1_is_plain_attention(flags):
    d = Desc(frames=3, grid_h=4, grid_w=5, heads=2, sigma=1, **flags)
    q, k, v = inputs(d)
    ref = sdpa(f64(q), f64(k), f64(v))
    np.testing.assert_allclose(oracle.attention(q, k, v, d), ref, rtol=0, atol=1e-12)


def test_g2f_is_per_frame_attention():
    d = Desc(frames=4, grid_h=3, grid_w=5, heads=3, g2f=True)
    q, k, v = inputs(d)
    H, T, D = q.shape
    shape = (H, d.frames, d.L, D)
    ref = sdpa(f64(q).reshape(shape), f64(k).reshape(shape), f64(v).reshape(shape)).reshape(H, T, D)
    np.testing.assert_allclose(oracle.attention(q, k, v, d), ref, rtol=0, atol=1e-12)


def test_sga_plain_is_attention_over_hand_set():
    d = Desc(**GOLD_DESC)
    q, k, v = inputs(d, seed=3)
    S = hand_S()
    ref = sdpa(f64(q), f64(k)[:, S], f64(v)[:, S])
    np.testing.assert_allclose(oracle.attention(q, k, v, d), ref, rtol=0, atol=1e-12)


def test_diag_adds_own_token_only_when_dropped():
    d = Desc(**GOLD_DESC, diag=True)
    q, k, v = inputs(d, seed=4)
    S = hand_S()
    Sset = set(S.tolist())
    qf, kf, vf = f64(q), f64(k), f64(v)
    out = oracle.attention(q, k, v, d)
    for r in range(d.T):
        keys = S if r in Sset else np.append(S, r)
        ref = sdpa(qf[:, r:r + 1], kf[:, keys], vf[:, keys])[:, 0]
        np.testing.assert_allclose(out[:, r], ref, rtol=0, atol=1e-12)


def _mean_lists(kf, vf, reps):
    ks, vs = [], []
    for f in (1, 2):
        D = hand_dropped(f)
        assert D.size == 26
        km, vm = kf[:, D].mean(axis=1, keepdims=True), vf[:, D].mean(axis=1, keepdims=True)
        n = D.size if reps == "count" else 1
        ks.append(np.repeat(km, n, axis=1))
        vs.append(np.repeat(vm, n, axis=1))
    return ks, vs


@pytest.mark.parametrize("weight", ["unit", "count"])
def test_mean_term_is_extra_tokens(weight):
    """UNIT: each compressed frame adds one mean token.  COUNT: the log|D_f| bias equals |D_f|
    copies of the mean token (RegimeVGGT notes, 关键设计 2)."""
    d = Desc(**GOLD_DESC, mean=True, mean_count=(weight == "count"))
    q, k, v = inputs(d, seed=5)
    qf, kf, vf = f64(q), f64(k), f64(v)
    S = hand_S()
    ks, vs = _mean_lists(kf, vf, weight)
    ref = sdpa(qf, np.concatenate([kf[:, S]] + ks, axis=1), np.concatenate([vf[:, S]] + vs, axis=1))
    np.testing.assert_allclose(oracle.attention(q, k, v, d), ref, rtol=0, atol=1e-12)


def test_enhanced_sga_diag_plus_mean_against_explicit_lists():
    d = Desc(**GOLD_DESC, diag=True, mean=True)
    q, k, v = inputs(d, seed=6)
    qf, kf, vf = f64(q), f64(k), f64(v)
    S = hand_S()
    Sset = set(S.tolist())
    ks, vs = _mean_lists(kf, vf, "unit")
    out = oracle.attention(q, k, v, d)
    for r in range(0, d.T, 3):
        extra_k = [kf[:, r:r + 1]] if r not in Sset else []
        extra_v = [vf[:, r:r + 1]] if r not in Sset else []
        keys = np.concatenate([kf[:, S]] + ks + extra_k, axis=1)
        vals = np.concatenate([vf[:, S]] + vs + extra_v, axis=1)
        ref = sdpa(qf[:, r:r + 1], keys, vals)[:, 0]
        np.testing.assert_allclose(out[:, r], ref, rtol=0, atol=1e-12)


@pytest.mark.parametrize("ref_dense", [True, False])
def test_collapse_identity_count_mean_equals_dense(ref_dense):
    """If every dropped K/V row of a frame is the same row, a COUNT-weighted mean stands in for
    exactly those rows, so enhanced SGA (mean, no diagonal) equals plain dense attention."""
    d = Desc(frames=3, grid_h=6, grid_w=7, heads=2, sigma=6, ref_dense=ref_dense, mean=True, mean_count=True)
    q, k, v = inputs(d, dtype="fp32", seed=7)
    keep = oracle.kept_mask_by_sets(d)
    rng = np.random.default_rng(0)
    for f in range(d.frames):
        tok = np.arange(f * d.L, (f + 1) * d.L)
        drop = tok[~keep[tok]]
        if drop.size:
            k[:, drop] = rng.standard_normal((d.heads, 1, d.head_dim)).astype(np.float32)
            v[:, drop] = rng.standard_normal((d.heads, 1, d.head_dim)).astype(np.float32)
    ref = sdpa(f64(q), f64(k), f64(v))
    np.testing.assert_allclose(oracle.attention(q, k, v, d), ref, rtol=0, atol=1e-12)


# ------------------------------------------------------------------------------------------
# Identities and the brute-force formulation
# ------------------------------------------------------------------------------------------

FORMS = [
    dict(sigma=1),
    dict(g2f=True),
    dict(sigma=2),
    dict(sigma=4, diag=True, mean=True),
    dict(sigma=6, diag=True, mean=True, mean_count=True),
    dict(sigma=9, diag=True, mean=True, ref_dense=False),
    dict(sigma=6, diag=True),
    dict(sigma=9, mean=True, mean_count=True, ref_dense=False),
    dict(sigma=6, diag=True, mean=True, mean_count=True, phase_shift=True),
    dict(sigma=4, diag=True, mean=True, mean_global=True),
    dict(sigma=9, mean=True, mean_count=True, mean_global=True, phase_shift=True, ref_dense=False),
    dict(g2m=True),
]


@pytest.mark.parametrize("flags", FORMS)
@pytest.mark.parametrize("geom", [(4, 8, 8), (3, 5, 7), (2, 7, 4), (1, 3, 3)])
def test_bruteforce_matches_gather(flags, geom):
    N, gh, gw = geom
    d = Desc(frames=N, grid_h=gh, grid_w=gw, heads=2, **flags)
    q, k, v = inputs(d, seed=N * 100 + gh)
    np.testing.assert_allclose(oracle.attention(q, k, v, d), oracle.attention_bruteforce(q, k, v, d),
                               rtol=0, atol=1e-12)


@pytest.mark.parametrize("flags", FORMS)
def test_v_ones_gives_ones(flags):
    """The weights over S, the diagonal and the means sum to one (one joint normalisation)."""
    d = Desc(frames=3, grid_h=5, grid_w=7, heads=2, **flags)
    q, k, _ = inputs(d, seed=8)
    v = np.ones((d.heads, d.T, d.head_dim), dtype=np.float32)
    np.testing.assert_allclose(oracle.attention(q, k, v, d), 1.0, rtol=0, atol=1e-13)


@pytest.mark.parametrize("flags", FORMS)
def test_shift_invariance_in_k(flags):
    """Adding one vector c to every key moves every logit of a row (means and self included) by
    tau*<q, c>, which the softmax cancels."""
    d = Desc(frames=3, grid_h=5, grid_w=7, heads=2, **flags)
    q, k, v = inputs(d, dtype="fp32", seed=9)
    c = np.random.default_rng(1).standard_normal((d.heads, 1, d.head_dim))
    k2 = k.astype(np.float64) + c
    np.testing.assert_allclose(oracle.attention(q, k2, v, d), oracle.attention(q, k, v, d), rtol=0, atol=1e-11)


@pytest.mark.parametrize("flags", FORMS)
def test_linearity_in_v(flags):
    d = Desc(frames=3, grid_h=5, grid_w=7, heads=2, **flags)
    q, k, v1 = inputs(d, dtype="fp32", seed=10)
    _, _, v2 = inputs(d, dtype="fp32", seed=11)
    a = oracle.attention(q, k, v1.astype(np.float64) + v2, d)
    b = oracle.attention(q, k, v1, d) + oracle.attention(q, k, v2, d)
    np.testing.assert_allclose(a, b, rtol=0, atol=1e-12)


def test_sampled_rows_match_full_rows():
    d = Desc(frames=5, grid_h=6, grid_w=6, heads=2, sigma=4, diag=True, mean=True)
    q, k, v = inputs(d, seed=12)
    rows = sample_rows(d.frames, d.grid_h, d.grid_w, d.n_special, count=60, seed=1)
    full = oracle.attention(q, k, v, d)
    part = oracle.attention(q, k, v, d, rows=rows, workers=2, chunk=7)
    np.testing.assert_allclose(part, full[:, rows], rtol=0, atol=1e-14)


def test_invalid_descriptors_rejected():
    with pytest.raises(ValueError):
        Desc(frames=2, grid_h=4, grid_w=4, heads=1, sigma=3)
    with pytest.raises(ValueError):
        Desc(frames=2, grid_h=4, grid_w=4, heads=1, sigma=4, g2f=True)
    with pytest.raises(ValueError):
        Desc(frames=2, grid_h=4, grid_w=4, heads=1, g2f=True, mean=True)
    with pytest.raises(ValueError):
        Desc(frames=2, grid_h=4, grid_w=4, heads=1, sigma=4, g2m=True)
    with pytest.raises(ValueError):
        Desc(frames=2, grid_h=4, grid_w=4, heads=1, g2m=True, diag=True)
    with pytest.raises(ValueError):
        Desc(frames=2, grid_h=4, grid_w=4, heads=1, sigma=4, mean_global=True)


# ------------------------------------------------------------------------------------------
# Phase-shifted sampling grid (RegimeVGGT notes, 关键设计 3)
# ------------------------------------------------------------------------------------------

PHASE_DESC = dict(frames=7, grid_h=5, grid_w=7, heads=2, sigma=6, ref_dense=True, phase_shift=True)


def phase_S():
    return load_golden("index_set_7f_5x7_sigma6_phase.txt")


def test_phase_shift_index_set_hand_enumerated():
    d = Desc(**PHASE_DESC)
    assert np.array_equal(oracle.index_set(d), phase_S())
    assert np.array_equal(np.flatnonzero(oracle.kept_mask_by_sets(d)), phase_S())
    assert list(oracle.dropped_counts(d)) == [0, 29, 29, 29, 31, 31, 26]
    c = oracle.counts(Desc(**PHASE_DESC, diag=True, mean=True))
    assert (c["n_kv"], c["n_mean"], c["n_diag"]) == (105, 6, 175)


@pytest.mark.parametrize("sigma,t", [(4, 2), (9, 3)])
def test_phase_shift_square_windows_follow_the_page_formula(sigma, t):
    """Square t x t windows: frame f's grid starts at row (f div t) mod t, column f mod t."""
    d = Desc(frames=20, grid_h=9, grid_w=9, heads=1, sigma=sigma, ref_dense=False, phase_shift=True)
    keep = oracle.kept_mask(d).reshape(d.frames, d.L)[:, d.n_special:].reshape(d.frames, 9, 9)
    for f in range(d.frames):
        rows, cols = np.nonzero(keep[f])
        assert set((rows % t).tolist()) == {(f // t) % t} and set((cols % t).tolist()) == {f % t}
        assert rows.min() == (f // t) % t and cols.min() == f % t
        assert rows.size == len(range((f // t) % t, 9, t)) * len(range(f % t, 9, t))


@pytest.mark.parametrize("sigma", [2, 4, 6, 9])
@pytest.mark.parametrize("geom", [(5, 7), (37, 37), (4, 4), (1, 5), (6, 1)])
def test_phase_shift_consecutive_frames_cover_the_grid(sigma, geom):
    """The page shifts the grid so that the union over frames covers the whole space: here any
    s_h*s_w consecutive compressed frames keep every patch position exactly once."""
    gh, gw = geom
    s_h, s_w = oracle.SIGMA_WINDOWS[sigma]
    n = s_h * s_w
    for start in (0, 1, 5):
        d = Desc(frames=start + n, grid_h=gh, grid_w=gw, heads=1, n_special=2, sigma=sigma,
                 ref_dense=False, phase_shift=True)
        keep = oracle.kept_mask(d).reshape(d.frames, d.L)[start:, d.n_special:]
        assert np.array_equal(keep.sum(axis=0), np.ones(gh * gw, dtype=np.int64))


def test_phase_shift_size_at_800_frames():
    # 37 x 37 grid, 2 x 3 windows: phase (row, col) keeps 19|18 rows x 13|12|12 columns; one
    # period of 6 phases keeps 247+228+228+234+216+216 = 1369 = every patch once.  Frames
    # 1..798 are 133 full periods and frame 799 has phase 1 (228 patches).
    expect = 800 * 5 + 1369 + 133 * 1369 + 228
    assert expect == 187_674
    d = Desc(frames=800, grid_h=37, grid_w=37, heads=1, sigma=6, phase_shift=True)
    assert oracle.counts(d)["n_kv"] == expect


def test_phase_shift_sga_is_attention_over_hand_set():
    d = Desc(**PHASE_DESC)
    q, k, v = inputs(d, seed=21)
    S = phase_S()
    ref = sdpa(f64(q), f64(k)[:, S], f64(v)[:, S])
    np.testing.assert_allclose(oracle.attention(q, k, v, d), ref, rtol=0, atol=1e-12)


@pytest.mark.parametrize("weight", ["unit", "count"])
def test_phase_shift_means_with_unequal_dropped_sets(weight):
    """Per-frame means over dropped sets of different sizes (29, 31, 26 patches): COUNT equals
    |D_f| copies of each frame's mean token."""
    d = Desc(**PHASE_DESC, mean=True, mean_count=(weight == "count"))
    q, k, v = inputs(d, seed=22)
    qf, kf, vf = f64(q), f64(k), f64(v)
    S = phase_S()
    Sset = set(S.tolist())
    ks, vs = [kf[:, S]], [vf[:, S]]
    for f in range(1, d.frames):
        D = np.asarray([t for t in range(f * 40 + 5, (f + 1) * 40) if t not in Sset])
        assert D.size == [29, 29, 29, 31, 31, 26][f - 1]
        n = D.size if weight == "count" else 1
        ks.append(np.repeat(kf[:, D].mean(axis=1, keepdims=True), n, axis=1))
        vs.append(np.repeat(vf[:, D].mean(axis=1, keepdims=True), n, axis=1))
    ref = sdpa(qf, np.concatenate(ks, axis=1), np.concatenate(vs, axis=1))
    np.testing.assert_allclose(oracle.attention(q, k, v, d), ref, rtol=0, atol=1e-12)


@pytest.mark.parametrize("flags", [dict(diag=True, mean=True), dict(diag=True, mean=True, mean_count=True),
                                   dict(mean=True, mean_global=True, mean_count=True)])
def test_phase_shift_one_wide_grid_with_empty_dropped_sets(flags):
    """A 6 x 1 grid with 1 x 2 windows: even frames keep their whole column, odd frames keep
    nothing, so only odd frames have a mean term (reading R22)."""
    d = Desc(frames=5, grid_h=6, grid_w=1, heads=2, sigma=2, ref_dense=False, phase_shift=True, **flags)
    assert list(oracle.dropped_counts(d)) == [0, 6, 0, 6, 0]
    c = oracle.counts(d)
    assert c["n_kv"] == 5 * 5 + 3 * 6
    assert c["n_mean"] == (1 if d.mean_global else 2)
    q, k, v = inputs(d, seed=23)
    np.testing.assert_allclose(oracle.attention(q, k, v, d), oracle.attention_bruteforce(q, k, v, d),
                               rtol=0, atol=1e-12)


# ------------------------------------------------------------------------------------------
# Global mean scope and G2M
# ------------------------------------------------------------------------------------------

@pytest.mark.parametrize("weight", ["unit", "count"])
def test_global_mean_is_one_token_over_all_dropped(weight):
    """One mean over D_1 and D_2 together (52 patches): UNIT adds one token, COUNT adds 52
    copies of it."""
    d = Desc(**GOLD_DESC, mean=True, mean_global=True, mean_count=(weight == "count"))
    q, k, v = inputs(d, seed=24)
    qf, kf, vf = f64(q), f64(k), f64(v)
    S = hand_S()
    D = np.concatenate([hand_dropped(1), hand_dropped(2)])
    n = D.size if weight == "count" else 1
    keys = np.concatenate([kf[:, S], np.repeat(kf[:, D].mean(axis=1, keepdims=True), n, axis=1)], axis=1)
    vals = np.concatenate([vf[:, S], np.repeat(vf[:, D].mean(axis=1, keepdims=True), n, axis=1)], axis=1)
    np.testing.assert_allclose(oracle.attention(q, k, v, d), sdpa(qf, keys, vals), rtol=0, atol=1e-12)
    assert oracle.counts(d)["n_mean"] == 1


@pytest.mark.parametrize("phase", [False, True])
def test_collapse_identity_global_mean(phase):
    """If every dropped K/V row of every frame is the same row, the COUNT-weighted global mean
    stands in for exactly those rows: SGA + global mean equals dense attention."""
    d = Desc(frames=4, grid_h=6, grid_w=7, heads=2, sigma=6, mean=True, mean_global=True, mean_count=True,
             phase_shift=phase)
    q, k, v = inputs(d, dtype="fp32", seed=25)
    drop = np.flatnonzero(~oracle.kept_mask_by_sets(d))
    rng = np.random.default_rng(2)
    k[:, drop] = rng.standard_normal((d.heads, 1, d.head_dim)).astype(np.float32)
    v[:, drop] = rng.standard_normal((d.heads, 1, d.head_dim)).astype(np.float32)
    np.testing.assert_allclose(oracle.attention(q, k, v, d), sdpa(f64(q), f64(k), f64(v)), rtol=0, atol=1e-12)


def test_g2m_equals_attention_over_identical_keys():
    """With every key equal, attention weights are uniform and the output of every query is
    the mean value over all tokens -- which is what G2M computes for any keys."""
    d = Desc(frames=3, grid_h=4, grid_w=5, heads=2, g2m=True)
    q, k, v = inputs(d, dtype="fp32", seed=26)
    out = oracle.attention(q, k, v, d)
    k_same = np.broadcast_to(f64(k)[:, :1], k.shape)
    np.testing.assert_allclose(out, sdpa(f64(q), k_same, f64(v)), rtol=0, atol=1e-12)
    c = oracle.counts(d)
    assert (c["n_kv"], c["n_mean"], c["n_diag"]) == (0, 1, 0)
    assert list(oracle.dropped_counts(d)) == [d.L] * d.frames


# ------------------------------------------------------------------------------------------
# The shared input generator
# ------------------------------------------------------------------------------------------

def test_bf16_rounding_is_nearest_even():
    x = np.array([1.0, 1.0 + 2.0 ** -8, 1.0 + 3 * 2.0 ** -8, 1.0 + 2.0 ** -9, -2.5, 3.0e-3,
                  1.0 + 2.0 ** -8 + 2.0 ** -20], dtype=np.float32)
    want = np.array([1.0, 1.0, 1.0 + 2.0 ** -6, 1.0, -2.5, None, 1.0 + 2.0 ** -7], dtype=object)
    got = bf16_bits_to_f32(f32_to_bf16_bits(x))
    for g, w in zip(got, want):
        if w is not None:
            assert g == np.float32(w)
    # the rounded value is always the nearer of the two bf16 neighbours
    r = np.random.default_rng(0).standard_normal(10000).astype(np.float32)
    b = bf16_bits_to_f32(f32_to_bf16_bits(r))
    ulp = np.abs(b) * 2.0 ** -7
    assert np.all(np.abs(b - r) <= ulp / 2 * (1 + 1e-6))


def test_generator_reproducible_and_worker_independent():
    a = make_qkv(3, 4, 5, 5, 2, 64, "bf16", seed=3, workers=1)
    b = make_qkv(3, 4, 5, 5, 2, 64, "bf16", seed=3, workers=4)
    for x, y in zip(a, b):
        assert x.dtype == np.uint16 and np.array_equal(x, y)
    c = make_qkv(3, 4, 5, 5, 2, 64, "bf16", seed=4)
    assert not np.array_equal(a[0], c[0])
    p1 = make_qkv(3, 4, 5, 5, 2, 64, "bf16", seed=3, workers=1, per_frame_streams=True)
    p4 = make_qkv(3, 4, 5, 5, 2, 64, "bf16", seed=3, workers=4, per_frame_streams=True)
    for x, y in zip(p1, p4):
        assert np.array_equal(x, y)


def test_generator_single_stream_order():
    """One PCG64(seed) stream: u_Q, Q's per-frame noise, then u_K, K's noise, then V's; each value
    0.7 u + 0.7 noise in float32, rounded to bf16; tie_qk gives K the same u as Q."""
    frames, gh, gw, ns, H, d = 3, 4, 5, 5, 2, 64
    L = ns + gh * gw
    got = make_qkv(frames, gh, gw, ns, H, d, "bf16", seed=3)
    tied = make_qkv(frames, gh, gw, ns, H, d, "bf16", seed=3, tie_qk=True)
    rng = np.random.Generator(np.random.PCG64(3))
    us = []
    for x, xt in zip(got, tied):
        u = rng.standard_normal((H, L, d), np.float32)
        us.append(u)
        for f in range(frames):
            nz = rng.standard_normal((H, L, d), np.float32)
            assert np.array_equal(x[:, f * L:(f + 1) * L], f32_to_bf16_bits(np.float32(0.7) * u + np.float32(0.7) * nz))
            ut = us[0] if len(us) == 2 else u
            assert np.array_equal(xt[:, f * L:(f + 1) * L],
                                  f32_to_bf16_bits(np.float32(0.7) * ut + np.float32(0.7) * nz))


def test_generator_shared_position_structure():
    q, k, v = make_qkv(40, 4, 4, 5, 1, 64, "fp32", seed=0)
    L = 21
    x = k[0].reshape(40, L, 64)
    # same slot across frames: correlation 0.49/(0.49+0.49) = 0.5; different slots ~0
    same = np.mean([np.corrcoef(x[0, j], x[f, j])[0, 1] for j in range(L) for f in range(1, 40)])
    diff = np.mean([np.corrcoef(x[0, j], x[f, (j + 1) % L])[0, 1] for j in range(L) for f in range(1, 40)])
    assert 0.4 < same < 0.6 and abs(diff) < 0.1


def test_sample_rows_forced_and_seeded():
    r1 = sample_rows(100, 37, 37, 5, count=4096, seed=1)
    r2 = sample_rows(100, 37, 37, 5, count=4096, seed=1)
    assert np.array_equal(r1, r2) and r1.size == 4096 and np.all(np.diff(r1) > 0)
    L = 1374
    for f in (0, 1, 50, 99):
        for j in range(5):
            assert f * L + j in set(r1.tolist())
        assert f * L + 5 + 36 * 37 + 36 in set(r1.tolist())  # last patch of the frame


# ------------------------------------------------------------------------------------------
# Size-aware keys: + log g on the logit (RegimeVGGT notes, 关键设计 2)
# ------------------------------------------------------------------------------------------

def _sizes(d, seed=0):
    g, _ = make_log_sizes(d.frames, d.grid_h, d.grid_w, d.n_special, seed=seed)
    return g, np.log(g.astype(np.float64))


def test_log_size_dense_is_replicated_keys():
    """Dense attention where key t carries + ln g_t equals plain attention over a key list in
    which token t appears g_t times."""
    d = Desc(frames=3, grid_h=4, grid_w=5, heads=2, sigma=1, log_size=True)
    q, k, v = inputs(d, seed=31)
    g, lg = _sizes(d, seed=1)
    assert set(np.unique(g).tolist()) == {1, 2, 3, 4}
    rep = np.repeat(np.arange(d.T), g)
    ref = sdpa(f64(q), f64(k)[:, rep], f64(v)[:, rep])
    np.testing.assert_allclose(oracle.attention(q, k, v, d, log_g=lg), ref, rtol=0, atol=1e-12)


def test_log_size_sga_with_diag_is_replicated_keys():
    """SGA with the diagonal term: every key of S and the self term of a dropped query stand for
    their g copies."""
    d = Desc(**GOLD_DESC, diag=True, log_size=True)
    q, k, v = inputs(d, seed=32)
    g, lg = _sizes(d, seed=2)
    S = hand_S()
    Sset = set(S.tolist())
    qf, kf, vf = f64(q), f64(k), f64(v)
    out = oracle.attention(q, k, v, d, log_g=lg)
    for r in range(0, d.T, 2):
        keys = S if r in Sset else np.append(S, r)
        rep = np.repeat(keys, g[keys])
        ref = sdpa(qf[:, r:r + 1], kf[:, rep], vf[:, rep])[:, 0]
        np.testing.assert_allclose(out[:, r], ref, rtol=0, atol=1e-12)


def test_log_size_g2f_is_replicated_keys_per_frame():
    d = Desc(frames=3, grid_h=3, grid_w=5, heads=2, g2f=True, log_size=True)
    q, k, v = inputs(d, seed=33)
    g, lg = _sizes(d, seed=3)
    out = oracle.attention(q, k, v, d, log_g=lg)
    for f in range(d.frames):
        tok = np.arange(f * d.L, (f + 1) * d.L)
        rep = np.repeat(tok, g[tok])
        ref = sdpa(f64(q)[:, tok], f64(k)[:, rep], f64(v)[:, rep])
        np.testing.assert_allclose(out[:, tok], ref, rtol=0, atol=1e-12)


@pytest.mark.parametrize("flags", [dict(sigma=1), dict(g2f=True), dict(sigma=6, diag=True),
                                   dict(sigma=9, diag=True, ref_dense=False, phase_shift=True)])
@pytest.mark.parametrize("geom", [(3, 5, 7), (2, 7, 4)])
def test_log_size_bruteforce_matches_gather(flags, geom):
    N, gh, gw = geom
    d = Desc(frames=N, grid_h=gh, grid_w=gw, heads=2, log_size=True, **flags)
    q, k, v = inputs(d, seed=34)
    _, lg = _sizes(d, seed=4)
    np.testing.assert_allclose(oracle.attention(q, k, v, d, log_g=lg),
                               oracle.attention_bruteforce(q, k, v, d, log_g=lg), rtol=0, atol=1e-12)


def test_log_size_unit_sizes_change_nothing():
    d = Desc(frames=3, grid_h=5, grid_w=7, heads=2, sigma=4, diag=True, log_size=True)
    q, k, v = inputs(d, seed=35)
    plain = Desc(frames=3, grid_h=5, grid_w=7, heads=2, sigma=4, diag=True)
    np.testing.assert_allclose(oracle.attention(q, k, v, d, log_g=np.zeros(d.T)), oracle.attention(q, k, v, plain),
                               rtol=0, atol=1e-14)


def test_log_size_descriptor_rules():
    with pytest.raises(ValueError):
        Desc(frames=2, grid_h=4, grid_w=4, heads=1, sigma=4, mean=True, log_size=True)
    with pytest.raises(ValueError):
        Desc(frames=2, grid_h=4, grid_w=4, heads=1, g2m=True, log_size=True)
    d = Desc(frames=2, grid_h=4, grid_w=4, heads=1, sigma=4, log_size=True)
    q, k, v = inputs(d)
    with pytest.raises(ValueError):
        oracle.attention(q, k, v, d)  # sizes missing
