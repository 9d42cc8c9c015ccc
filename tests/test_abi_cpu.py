"""CPU-side checks of the C ABI: the library loads, exports every function the header declares,
and its host plan agrees with the oracle's counts (no device call is made)."""
import os
import re

import pytest

import oracle
from oracle import Desc

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def ensure_built():
    import vggt_global_attention_attn_amd as va
    if not os.path.exists(va.LIB_PATH):
        from vggt_global_attention_attn_amd.build import build
        build()
    return va


@pytest.fixture(scope="module")
def va():
    return ensure_built()


def declared_functions():
    names = set()
    inc = os.path.join(ROOT, "include")
    for fn in os.listdir(inc):
        if fn.endswith(".h"):
            text = open(os.path.join(inc, fn)).read()
            text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
            names.update(re.findall(r"\b(vggt_attn_[a-z_]+)\s*\(", text))
    return names


def test_library_exports_every_declared_symbol(va):
    names = declared_functions()
    assert {"vggt_attn_plan", "vggt_attn_forward"} <= names
    lib = va.lib()
    for n in sorted(names):
        assert hasattr(lib, n), f"{n} not exported"
    assert set(va.EXPORTS) == names


CONFIGS = [
    Desc(4, 8, 8, 2, sigma=4, diag=True, mean=True),
    Desc(4, 8, 8, 2, sigma=4, diag=True, mean=True, ref_dense=False),
    Desc(32, 37, 37, 16, sigma=1),
    Desc(100, 37, 37, 16, sigma=4, diag=True, mean=True),
    Desc(200, 37, 37, 16, g2f=True),
    Desc(200, 37, 37, 16, sigma=9, diag=True, mean=True),
    Desc(800, 37, 37, 16, sigma=6, diag=True, mean=True),
    Desc(3, 5, 7, 2, sigma=2, mean=True, mean_count=True),
    Desc(3, 1, 1, 2, sigma=9, diag=True, mean=True),  # every window is a single patch: nothing dropped
    Desc(2, 2, 1, 1, sigma=2, diag=True, mean=True),  # one column: (1,2) windows keep everything
    Desc(7, 5, 7, 2, sigma=6, diag=True, mean=True, mean_count=True, phase_shift=True),
    Desc(800, 37, 37, 16, sigma=6, diag=True, mean=True, phase_shift=True),
    Desc(200, 37, 37, 16, sigma=9, diag=True, mean=True, mean_global=True, phase_shift=True, ref_dense=False),
    Desc(100, 37, 37, 16, sigma=4, mean=True, mean_global=True, mean_count=True),
    Desc(5, 6, 1, 2, sigma=2, diag=True, mean=True, phase_shift=True, ref_dense=False),  # empty dropped sets
    Desc(32, 37, 37, 16, g2m=True),
    Desc(32, 37, 37, 16, sigma=1, log_size=True),
    Desc(200, 37, 37, 16, g2f=True, log_size=True),
    Desc(100, 37, 37, 16, sigma=4, diag=True, log_size=True, phase_shift=True),
]


@pytest.mark.parametrize("desc", CONFIGS, ids=lambda d: f"{d.frames}x{d.grid_h}x{d.grid_w}-s{d.sigma}-g2f{int(d.g2f)}"
                         f"-ph{int(d.phase_shift)}-mg{int(d.mean_global)}-g2m{int(d.g2m)}")
def test_plan_counts_match_oracle(va, desc):
    p = va.Plan(desc.frames, desc.grid_h, desc.grid_w, desc.heads, sigma=desc.sigma, ref_dense=desc.ref_dense,
                diag=desc.diag, mean=desc.mean, mean_count=desc.mean_count, g2f=desc.g2f,
                phase_shift=desc.phase_shift, mean_global=desc.mean_global, g2m=desc.g2m, log_size=desc.log_size)
    c = p.counts()
    o = oracle.counts(desc)
    assert (c["n_kv"], c["n_mean"], c["n_diag"]) == (o["n_kv"], o["n_mean"], o["n_diag"])
    d4H = 4 * desc.head_dim * desc.heads
    if desc.g2f:
        flops = d4H * desc.frames * desc.L ** 2
    else:
        flops = d4H * (desc.T * (o["n_kv"] + o["n_mean"]) + o["n_diag"])
    assert c["flops"] == pytest.approx(flops, rel=1e-12)
    lay = p.layout()
    assert lay["segment_rows"] % 64 == 0 and lay["segment_rows"] >= lay["keys_per_segment"]
    for key in ("off_index", "off_dcount", "off_means", "off_partial", "off_kbias", "off_logsize", "off_kmax",
                "off_kpack", "off_vpack", "total_bytes"):
        assert lay[key] % 256 == 0
    if desc.log_size:
        assert lay["off_logsize"] - lay["off_kbias"] >= 4 * lay["segments"] * lay["segment_rows"]
        assert lay["off_kmax"] - lay["off_logsize"] >= 4 * desc.T
    assert lay["total_bytes"] == p.workspace_bytes
    # The packed parts hold H x padded rows x d values, except for bf16 G2F plans, whose keys
    # (each frame's own tokens) are read in place.
    inplace = desc.g2f
    rows = lay["segments"] * lay["segment_rows"]
    kbytes = lay["off_vpack"] - lay["off_kpack"]
    if inplace:
        assert kbytes == 0 and lay["total_bytes"] == lay["off_vpack"]
    else:
        assert kbytes >= desc.heads * rows * desc.head_dim * 2
        assert lay["total_bytes"] - lay["off_vpack"] >= desc.heads * rows * desc.head_dim * 2


def test_config5_sizes(va):
    p = va.Plan(800, 37, 37, 16, sigma=6, diag=True, mean=True)
    c = p.counts()
    assert c["n_kv"] == 202722 and c["n_mean"] == 799 and c["n_diag"] == 896478
    assert c["flops"] == pytest.approx(916.32e12, rel=1e-4)
    lay = p.layout()
    assert lay["segment_rows"] == 203584 and lay["keys_per_segment"] == 203521


@pytest.mark.parametrize("kwargs,code", [
    (dict(sigma=3), "EINVAL"),
    (dict(sigma=0), "EINVAL"),
    (dict(head_dim=128), "EUNSUPPORTED"),
    (dict(g2f=True, sigma=4), "EINVAL"),
    (dict(g2f=True, mean=True), "EINVAL"),
    (dict(in_dtype="fp32", out_dtype="bf16"), "EINVAL"),
    (dict(flags=1 << 10), "EINVAL"),
    (dict(flags=1 << 12), "EINVAL"),
    (dict(g2m=True, sigma=4), "EINVAL"),
    (dict(g2m=True, diag=True), "EINVAL"),
    (dict(g2m=True, g2f=True), "EINVAL"),
    (dict(g2f=True, phase_shift=True), "EINVAL"),
    (dict(sigma=4, mean_global=True), "EINVAL"),  # MEAN_GLOBAL without MEAN
    (dict(sigma=4, mean=True, log_size=True), "EINVAL"),
    (dict(g2m=True, log_size=True), "EINVAL"),
    (dict(frames=0), "EINVAL"),
    (dict(heads=0), "EINVAL"),
    (dict(frames=6000, grid_h=37, grid_w=37), "EINVAL"),  # 8.2M tokens > limit
])
def test_plan_rejects(va, kwargs, code):
    base = dict(frames=4, grid_h=8, grid_w=8, heads=2)
    base.update(kwargs)
    with pytest.raises(va.VggtAttnError) as ei:
        va.Plan(**base)
    assert ei.value.status == code
    assert va.lib().vggt_attn_last_error()


def test_null_arguments(va):
    import ctypes
    L = va.lib()
    assert L.vggt_attn_plan(None, 1, 1, 1, 5, 1, 64, 1, 0, 0, 0) == -1
    assert L.vggt_attn_workspace_bytes(None) == 0
    assert L.vggt_attn_counts(None, None, None, None, None) == -1
    p = va.Plan(4, 8, 8, 2)
    assert L.vggt_attn_forward(p.handle, None, None, None, None, None, 0, None) == -1
    assert L.vggt_attn_pack(p.handle, None, None, None, 0, None) == -1
    L.vggt_attn_plan_destroy(None)
    assert L.vggt_attn_counts(p.handle, None, None, None, None) == 0


def test_sized_entry_points_match_the_plan(va):
    """A LOG_SIZE plan refuses the plain forward/pack and a plain plan refuses the sized ones;
    both checks come before any pointer is used, so they run without a GPU."""
    L = va.lib()
    sized = va.Plan(4, 8, 8, 2, sigma=4, diag=True, log_size=True)
    plain = va.Plan(4, 8, 8, 2, sigma=4, diag=True)
    assert L.vggt_attn_forward(sized.handle, None, None, None, None, None, 0, None) == -1
    assert b"_sized" in L.vggt_attn_last_error()
    assert L.vggt_attn_pack(sized.handle, None, None, None, 0, None) == -1
    assert L.vggt_attn_forward_sized(plain.handle, None, None, None, None, None, None, 0, None) == -1
    assert b"LOG_SIZE" in L.vggt_attn_last_error()
    assert L.vggt_attn_pack_sized(sized.handle, None, None, None, None, 0, None) == -1  # log_g NULL
    assert L.vggt_attn_pack_sized(sized.handle, None, None, 2, None, 0, None) == -4  # misaligned log_g


def test_token_limit_is_exact(va):
    """T = frames * 1374 may reach 8,000,000: 5822 frames (7,999,428 tokens) plan, 5823 do not."""
    p = va.Plan(5822, 37, 37, 6, g2f=True)
    assert p.T == 7_999_428 and p.counts()["n_kv"] == 1374
    with pytest.raises(va.VggtAttnError) as ei:
        va.Plan(5823, 37, 37, 6, g2f=True)
    assert ei.value.status == "EINVAL"


def test_split_cases_split(va):
    """The GPU cases meant to exercise split work items do split: dense 3x37x37 (44 items on 512
    slots: 8 pieces each) and G2F 4x37x37 (64 items: 5 pieces of 22 tiles); the 800-frame
    workload (91,600 items) does not."""
    assert va.Plan(3, 37, 37, 2, sigma=1).layout()["split_pieces"] == 8
    assert va.Plan(4, 37, 37, 2, g2f=True).layout()["split_pieces"] == 5
    assert va.Plan(800, 37, 37, 16, sigma=6, diag=True, mean=True).layout()["split_pieces"] == 0
    assert va.Plan(3, 37, 37, 2, sigma=1, prescale_q=True).layout()["split_pieces"] == 8


def test_f16_score_form_layout(va):
    """PRESCALE_Q (f16 score form): a uint32 key maximum per head, and G2F plans keep a packed
    copy (their f16 keys cannot be read in place); fp32 plans ignore the flag."""
    for kw in (dict(sigma=6, diag=True, mean=True), dict(sigma=1), dict(g2f=True)):
        lay = va.Plan(4, 13, 11, 3, prescale_q=True, **kw).layout()
        rows = lay["segments"] * lay["segment_rows"]
        assert lay["off_kmax"] % 256 == 0 and lay["off_kpack"] - lay["off_kmax"] >= 3 * 4
        assert lay["off_vpack"] - lay["off_kpack"] >= 3 * rows * 64 * 2
        plain = va.Plan(4, 13, 11, 3, **kw).layout()
        assert plain["off_kpack"] == plain["off_kmax"]
    lay = va.Plan(4, 13, 11, 3, sigma=4, prescale_q=True, in_dtype="fp32").layout()
    assert lay["off_kpack"] == lay["off_kmax"]


def test_noalloc_refuses_large_plans_before_any_device_call(va):
    """vggt_attn_forward_noalloc checks the plan's workspace against its static 256 MiB before it
    looks at a device: the 800-frame workload (about 800 MiB) gets ENOSPC with the sizes named,
    and LOG_SIZE plans get EINVAL (no tensor pointer is needed to reach either answer)."""
    L = va.lib()
    assert L.vggt_attn_forward_noalloc(None, None, None, None, None, None) == -1
    big = va.Plan(800, 37, 37, 16, sigma=6, diag=True, mean=True)
    assert big.workspace_bytes > 256 << 20
    assert L.vggt_attn_forward_noalloc(big.handle, None, None, None, None, None) == -3
    msg = L.vggt_attn_last_error().decode()
    assert str(big.workspace_bytes) in msg and str(256 << 20) in msg
    sized = va.Plan(4, 8, 8, 2, sigma=4, diag=True, log_size=True)
    assert L.vggt_attn_forward_noalloc(sized.handle, None, None, None, None, None) == -1


def test_alias_checks_come_before_any_device_call(va):
    """Overlaps between out, the workspace and the inputs are refused (EALIAS) by forward, pack
    and attend from the addresses alone, so fake (never dereferenced) addresses serve here.
    Host-only: where a GPU is visible it is skipped, so that a regression in these checks could
    never launch kernels on the fake addresses."""
    import torch
    if torch.cuda.is_available():
        pytest.skip("fake device addresses: run on a host without a GPU")
    L = va.lib()
    p = va.Plan(4, 8, 8, 2, sigma=4, diag=True, mean=True)
    nin = 2 * p.T * 64 * 2  # bf16 q/k/v bytes
    nws = p.workspace_bytes
    base = 1 << 40
    q, k, v, out, ws = (base + i * (1 << 24) for i in range(5))
    for call in ("forward", "attend"):
        f = getattr(L, f"vggt_attn_{call}")
        assert f(p.handle, q, k, v, k + 4096, ws, nws, None) == -5          # out inside k
        assert f(p.handle, q, k, v, out, k + nin - 16, nws, None) == -5    # workspace over k's tail
        assert f(p.handle, q, k, v, out, q, nws, None) == -5               # workspace on q
        assert f(p.handle, q, k, v, ws + nws - 16, ws, nws, None) == -5    # out over the workspace's tail
        assert b"overlaps" in L.vggt_attn_last_error()
    assert L.vggt_attn_pack(p.handle, k, v, v + 16, nws, None) == -5


def test_layer_schedule_follows_avggt(va):
    """AVGGT notes, 整体框架: the 24 global layers are numbered 0-23; indices below t_early (9 for
    VGGT, i.e. layers 0-8; 10 for pi^3) become Global-to-Frame, the middle layers keep global
    attention with K/V subsampled by sigma (with the diagonal and mean terms of 关键设计 3, the
    flowchart's SGA branch), and the late layers stay unchanged; the ablation table's row
    AVGGT(2)- ("late layers (20-23) also to frame attention") fixes the late part as 20-23.
    VGGT keeps frame 0 dense, pi^3 compresses every frame (关键设计 2)."""
    for model, t_early, ref in (("vggt", 9, True), ("pi3", 10, False)):
        for sigma in (2, 4, 6, 9):
            s = va.layer_schedule(model, sigma)
            assert len(s) == 24
            for layer, kw in enumerate(s):
                if layer < t_early:
                    assert kw == dict(sigma=1, g2f=True, ref_dense=False, diag=False, mean=False), (model, layer)
                elif layer < 20:
                    assert kw == dict(sigma=sigma, g2f=False, ref_dense=ref, diag=True, mean=True), (model, layer)
                else:
                    assert kw == dict(sigma=1, g2f=False, ref_dense=False, diag=False, mean=False), (model, layer)
    # sigma 1 keeps the middle layers dense
    assert all(kw["sigma"] == 1 and not kw["diag"] for kw in va.layer_schedule("vggt", 1)[9:])
    L = va.lib()
    import ctypes
    for model, layer, sigma in ((2, 0, 9), (0, 24, 9), (0, -1, 9), (1, 5, 3)):
        assert L.vggt_attn_layer_schedule(model, layer, sigma, None, None) == -1
    s, f = ctypes.c_int(), ctypes.c_uint()
    assert L.vggt_attn_layer_schedule(0, 8, 6, ctypes.byref(s), ctypes.byref(f)) == 0 and f.value == va.G2F
    assert L.vggt_attn_layer_schedule(0, 9, 6, ctypes.byref(s), ctypes.byref(f)) == 0 and s.value == 6
    assert f.value == va.DIAG | va.MEAN | va.REF_DENSE


def test_scheduled_layers_share_plans(va):
    """The scheduled driver builds one plan per distinct form (G2F, SGA, dense) and reports the
    pass's FLOPs as the sum over the 24 layers of each layer's plan."""
    sl = va.ScheduledLayers(6, 13, 11, 2, model="vggt", sigma=4, device="cpu")
    assert len(sl.plans) == 3
    assert sl.index[:9] == [sl.index[0]] * 9 and len(set(sl.index[9:20])) == 1 and len(set(sl.index[20:])) == 1
    per = [p.counts()["flops"] for p in sl.plans]
    assert sl.flops() == 9 * per[sl.index[0]] + 11 * per[sl.index[9]] + 4 * per[sl.index[20]]
