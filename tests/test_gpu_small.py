"""GPU parity at sizes the oracle finishes in seconds: several key and query tiles, ragged
tails, every form (dense, SGA sigma 2/4/6/9, enhanced SGA with UNIT and COUNT means, pi^3
without a dense frame, the phase-shifted grid, the global mean scope, G2F, G2M), both output
types, the exact and the f16 score form, plus the bit-exact index set and packed rows (and the
f16 packed keys), V = 1, determinism, a NaN-poisoned workspace, the rising-logit, spike and
tied-Q/K stress inputs, the collapse identity (identical dropped rows under COUNT means equal
dense attention), G2F's in-place reads stopping at the tensors' end, degenerate shapes (one
token, one frame, nothing dropped, no specials), 160 seeded random configurations on the bf16
path and 40 on the float32 path, and the C ABI's error codes.  Every call goes
through the C ABI of libvggt_attn.so."""
import ctypes
import zlib

import numpy as np
import pytest

import oracle
from oracle import Desc
from synth import make_qkv
from tests.gpu_util import assert_close, errors, inputs_for, plan_kwargs, to_device

pytestmark = pytest.mark.gpu

CASES = [
    # frames, gh, gw, heads, flags                               (label)
    (Desc(3, 5, 7, 2, sigma=1), "dense-tiny-ragged"),
    (Desc(3, 5, 7, 2, sigma=6, diag=True, mean=True), "sga6-enh-tiny"),
    (Desc(6, 13, 11, 2, sigma=2), "sga2-plain"),
    (Desc(6, 13, 11, 2, sigma=4, diag=True, mean=True), "sga4-enh"),
    (Desc(6, 13, 11, 2, sigma=6, diag=True, mean=True, mean_count=True), "sga6-enh-count"),
    (Desc(6, 13, 11, 2, sigma=9, diag=True, mean=True, ref_dense=False), "sga9-enh-pi3"),
    (Desc(5, 13, 11, 3, g2f=True), "g2f-small"),
    (Desc(7, 37, 37, 2, sigma=4, diag=True, mean=True), "sga4-enh-37x37"),
    (Desc(3, 37, 37, 2, sigma=1), "dense-37x37"),
    (Desc(4, 37, 37, 2, g2f=True), "g2f-37x37"),
    (Desc(9, 37, 37, 1, sigma=9, diag=True, mean=True, mean_count=True), "sga9-enh-count-37x37"),
    # phase-shifted grid (per-frame |D_f| and COUNT bias), global mean scope, G2M
    (Desc(7, 5, 7, 2, sigma=6, diag=True, mean=True, mean_count=True, phase_shift=True), "sga6-phase-count-tiny"),
    (Desc(8, 13, 11, 2, sigma=6, diag=True, mean=True, mean_count=True, phase_shift=True), "sga6-phase-count"),
    (Desc(10, 37, 37, 1, sigma=9, diag=True, mean=True, mean_count=True, phase_shift=True, ref_dense=False),
     "sga9-phase-pi3-37x37"),
    (Desc(6, 13, 11, 2, sigma=4, diag=True, mean=True, mean_global=True), "sga4-global"),
    (Desc(6, 13, 11, 2, sigma=4, diag=True, mean=True, mean_global=True, mean_count=True, phase_shift=True),
     "sga4-global-count-phase"),
    (Desc(5, 6, 1, 2, sigma=2, diag=True, mean=True, mean_count=True, phase_shift=True, ref_dense=False),
     "sga2-phase-empty-sets"),
    (Desc(4, 13, 11, 2, g2m=True), "g2m"),
    # G2F frame lengths around the first-half-only last key tile (<= 32 keys in range): L = 70
    # (two tiles, 6 keys in the last), 96 (32: the boundary), 97 (33: the whole tile), 203 (four
    # tiles, 11 keys)
    (Desc(5, 5, 13, 3, g2f=True), "g2f-L70"),
    (Desc(4, 7, 13, 2, g2f=True), "g2f-L96"),
    (Desc(4, 2, 46, 2, g2f=True), "g2f-L97"),
    (Desc(3, 9, 22, 2, g2f=True), "g2f-L203"),
]
NEW = {c[1]: c for c in CASES[11:]}


@pytest.fixture(scope="module")
def lib():
    import vggt_global_attention_attn_amd as va
    return va


def run(va, desc, q, k, v, out_dtype="fp32", in_dtype="bf16", prescale_q=False):
    import torch
    plan = va.Plan(**plan_kwargs(desc, in_dtype, out_dtype), prescale_q=prescale_q)
    qd, kd, vd = to_device(q), to_device(k), to_device(v)
    out = plan.new_output()
    ws = plan.new_workspace()
    plan.forward(qd, kd, vd, out, ws)
    torch.cuda.synchronize()
    return plan, out.float().cpu().numpy(), ws, (qd, kd, vd)


@pytest.mark.parametrize("desc,label", CASES, ids=[c[1] for c in CASES])
def test_parity_bf16(lib, desc, label):
    print(f"[parity] {label} {desc}", flush=True)
    q, k, v = inputs_for(desc, "bf16", seed=zlib.crc32(label.encode()) % 1000)
    _, got, _, _ = run(lib, desc, q, k, v)
    ref = oracle.attention(q, k, v, desc, workers=4)
    print(label, "max-abs %.3e rel-L2 %.3e" % errors(got, ref))
    assert_close(got, ref, fp32=False, label=label)


# bf16 output on every kernel form: the general kernel, split work items merged by the merge kernel
# (dense-37x37: 44 items on 512 slots), G2F read in place (g2f-37x37, also split) and G2M.
BF16_OUT = CASES[:6] + [CASES[8], CASES[9], NEW["g2m"]]


@pytest.mark.parametrize("desc,label", BF16_OUT, ids=[c[1] for c in BF16_OUT])
def test_parity_bf16_out(lib, desc, label):
    q, k, v = inputs_for(desc, "bf16", seed=3)
    _, got, _, _ = run(lib, desc, q, k, v, out_dtype="bf16")
    ref = oracle.attention(q, k, v, desc)
    assert_close(got, ref, fp32=False, label=label + "/bf16-out")


FP32_CASES = [
    (Desc(4, 8, 8, 2, sigma=4, diag=True, mean=True), "tiny-workload"),
    (Desc(4, 8, 8, 2, sigma=4, diag=True, mean=True, ref_dense=False), "tiny-pi3"),
    (Desc(4, 8, 8, 2, sigma=4, diag=True, mean=True, mean_count=True), "tiny-count"),
    (Desc(3, 5, 7, 2, sigma=1), "fp32-dense"),
    (Desc(3, 9, 9, 2, g2f=True), "fp32-g2f"),
    (Desc(3, 6, 7, 2, sigma=9, diag=True, mean=True), "fp32-sga9"),
    (Desc(7, 5, 7, 2, sigma=6, diag=True, mean=True, mean_count=True, phase_shift=True), "fp32-phase-count"),
    (Desc(4, 8, 8, 2, sigma=4, diag=True, mean=True, mean_global=True, mean_count=True), "fp32-global-count"),
    (Desc(3, 5, 7, 2, g2m=True), "fp32-g2m"),
]


@pytest.mark.parametrize("desc,label", FP32_CASES, ids=[c[1] for c in FP32_CASES])
def test_parity_fp32(lib, desc, label):
    q, k, v = inputs_for(desc, "fp32", seed=0)
    _, got, _, _ = run(lib, desc, q, k, v, out_dtype="fp32", in_dtype="fp32")
    ref = oracle.attention(q, k, v, desc)
    print(label, "max-abs %.3e rel-L2 %.3e" % errors(got, ref))
    assert_close(got, ref, fp32=True, label=label)


@pytest.mark.parametrize("desc,label", [c for c in CASES if not c[0].g2f], ids=[c[1] for c in CASES if not c[0].g2f])
def test_index_set_bit_exact(lib, desc, label):
    q, k, v = inputs_for(desc, "bf16", seed=1)
    plan, _, ws, _ = run(lib, desc, q, k, v)
    idx, dcount = plan.index_set(ws)
    assert np.array_equal(idx, oracle.index_set(desc))
    assert np.array_equal(dcount, oracle.dropped_counts(desc).astype(np.int32))


def key_at(p):
    """Packed value-tile position -> key within the 64-key tile (the documented layout)."""
    half, g, j = p >> 5, (p >> 3) & 3, p & 7
    return half * 32 + (g * 4 + j if j < 4 else 16 + g * 4 + (j - 4))


# Plans with a packed copy (bf16 G2F plans read K/V in place and have none).
PACKED = [CASES[3], CASES[5], CASES[7], NEW["sga6-phase-count"], NEW["sga4-global-count-phase"],
          NEW["sga2-phase-empty-sets"], NEW["g2m"]]


@pytest.mark.parametrize("desc,label", PACKED, ids=[c[1] for c in PACKED])
def test_packed_rows(lib, desc, label):
    """Rows of S are bit-exact copies; the means are within one bf16 step of the fp64 means;
    padding is zero; values sit in the key-minor tile order."""
    import torch
    q, k, v = inputs_for(desc, "bf16", seed=2)
    plan, _, ws, _ = run(lib, desc, q, k, v)
    lay = plan.layout()
    H, d = desc.heads, desc.head_dim
    rows = lay["segments"] * lay["segment_rows"]
    kp = ws[lay["off_kpack"]:lay["off_kpack"] + H * rows * d * 2].view(torch.int16).cpu().numpy().view(np.uint16)
    vp = ws[lay["off_vpack"]:lay["off_vpack"] + H * rows * d * 2].view(torch.int16).cpu().numpy().view(np.uint16)
    kp = kp.reshape(H, rows, d)
    perm = np.array([key_at(p) for p in range(64)])
    vt = vp.reshape(H, rows // 64, d, 64)
    vrows = np.zeros((H, rows // 64, 64, d), dtype=np.uint16)
    vrows[:, :, perm, :] = vt.transpose(0, 1, 3, 2)
    vrows = vrows.reshape(H, rows, d)
    S = oracle.index_set(desc)
    nS = S.size
    assert np.array_equal(kp[:, :nS], k[:, S]) and np.array_equal(vrows[:, :nS], v[:, S])
    kbar, vbar, _, _ = oracle.frame_means(k, v, desc)
    M = kbar.shape[1]
    from synth import bf16_bits_to_f32
    for got, ref in ((kp[:, nS:nS + M], kbar), (vrows[:, nS:nS + M], vbar)):
        g = bf16_bits_to_f32(got).astype(np.float64)
        assert np.all(np.abs(g - ref) <= np.abs(ref) * 2.0 ** -7 + 1e-6)
    assert not kp[:, nS + M:].any() and not vrows[:, nS + M:].any()


VONES = [CASES[4], CASES[5], CASES[6], NEW["sga6-phase-count"], NEW["sga4-global-count-phase"], NEW["g2m"]]


@pytest.mark.parametrize("desc,label", VONES, ids=[c[1] for c in VONES])
def test_v_ones_gives_ones(lib, desc, label):
    q, k, _ = inputs_for(desc, "bf16", seed=5)
    v = np.full(q.shape, 0x3F80, dtype=np.uint16)  # bf16 1.0
    _, got, _, _ = run(lib, desc, q, k, v)
    assert np.max(np.abs(got - 1.0)) <= 4e-3


def test_deterministic_and_poisoned_workspace(lib):
    import torch
    desc = CASES[7][0]
    q, k, v = inputs_for(desc, "bf16", seed=6)
    plan = lib.Plan(**plan_kwargs(desc))
    qd, kd, vd = to_device(q), to_device(k), to_device(v)
    ws = plan.new_workspace()
    o1, o2, o3 = plan.new_output(), plan.new_output(), plan.new_output()
    ws.zero_()
    plan.forward(qd, kd, vd, o1, ws)
    plan.forward(qd, kd, vd, o2, ws)
    ws.fill_(0xFF)  # every bf16 lane becomes NaN
    plan.forward(qd, kd, vd, o3, ws)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(o1, o3)


def test_pack_then_attend_equals_forward(lib):
    import torch
    desc = CASES[4][0]
    q, k, v = inputs_for(desc, "bf16", seed=7)
    plan = lib.Plan(**plan_kwargs(desc))
    qd, kd, vd = to_device(q), to_device(k), to_device(v)
    ws = plan.new_workspace()
    o1, o2 = plan.new_output(), plan.new_output()
    plan.forward(qd, kd, vd, o1, ws)
    plan.pack(kd, vd, ws)
    plan.attend(qd, kd, vd, o2, ws)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2)


def test_error_codes(lib):
    import torch
    L = lib.lib()
    desc = CASES[3][0]
    plan = lib.Plan(**plan_kwargs(desc))
    q, k, v = (to_device(x) for x in inputs_for(desc, "bf16", seed=8))
    out = plan.new_output()
    ws = plan.new_workspace()
    nbytes = plan.workspace_bytes
    stream = torch.cuda.current_stream().cuda_stream
    h = plan.handle
    P = lambda t, off=0: ctypes.c_void_p(t.data_ptr() + off)
    assert L.vggt_attn_forward(h, P(q), P(k), P(v), P(out), P(ws), nbytes - 1, stream) == -3
    assert L.vggt_attn_forward(h, P(q), P(k), P(v), P(out), None, nbytes, stream) == -1
    assert L.vggt_attn_forward(h, None, P(k), P(v), P(out), P(ws), nbytes, stream) == -1
    assert L.vggt_attn_forward(h, P(q, 2), P(k), P(v), P(out), P(ws), nbytes, stream) == -4
    assert L.vggt_attn_forward(h, P(q), P(k), P(v), P(ws, 4096), P(ws), nbytes, stream) == -5
    assert L.vggt_attn_forward(h, P(q), P(k), P(v), P(k), P(ws), nbytes, stream) == -5
    assert b"overlaps" in L.vggt_attn_last_error()
    assert L.vggt_attn_forward(None, P(q), P(k), P(v), P(out), P(ws), nbytes, stream) == -1
    assert L.vggt_attn_forward(h, P(q), P(k), P(v), P(out), P(ws), nbytes, stream) == 0
    assert L.vggt_attn_last_error() == b""
    torch.cuda.synchronize()


def _rising(desc, seed, spike=None):
    """bf16 inputs whose logits grow along the key sequence (every later tile raises the running
    max), optionally with one key scaled up to a logit far above everything else."""
    from synth import bf16_bits_to_f32, f32_to_bf16_bits
    q, k, v = inputs_for(desc, "bf16", seed=seed)
    kf = bf16_bits_to_f32(k)
    ramp = np.linspace(0.2, 4.0, desc.T, dtype=np.float32)[None, :, None]
    kf = kf * ramp
    if spike is not None:
        t, factor = spike
        kf[:, t, :] = bf16_bits_to_f32(q)[:, 0, :] * factor  # aligned with query 0: huge logit for row 0
    return q, f32_to_bf16_bits(kf), v


@pytest.mark.parametrize("desc,label", [
    (Desc(6, 13, 11, 2, sigma=1), "dense"),
    (Desc(6, 13, 11, 2, sigma=4, diag=True, mean=True), "sga4-enh"),
    (Desc(4, 37, 37, 2, g2f=True), "g2f"),
], ids=["dense", "sga4-enh", "g2f"])
@pytest.mark.parametrize("prescale_q", [False, True], ids=["exact", "f16"])
def test_running_max_catch_up(lib, desc, label, prescale_q):
    """Logits that keep rising along the keys force the rare exact catch-up of the running max
    (a score more than an octave above it) in many tiles; a spiked key drives exp2 past the
    float range before the catch-up.  Both must still match the oracle, in the exact and the
    f16 score form."""
    q, k, v = _rising(desc, seed=11)
    _, got, _, _ = run(lib, desc, q, k, v, prescale_q=prescale_q)
    ref = oracle.attention(q, k, v, desc, workers=4)
    print(label, prescale_q, "rising max-abs %.3e rel-L2 %.3e" % errors(got, ref))
    assert_close(got, ref, fp32=False, label=label + "/rising")
    last_frame_token = desc.T - 3
    q, k, v = _rising(desc, seed=12, spike=(last_frame_token, 40.0))
    _, got, _, _ = run(lib, desc, q, k, v, prescale_q=prescale_q)
    ref = oracle.attention(q, k, v, desc, workers=4)
    print(label, prescale_q, "spike max-abs %.3e rel-L2 %.3e" % errors(got, ref))
    if not prescale_q:
        assert_close(got, ref, fp32=False, label=label + "/spike")
    else:
        # The f16 score form rounds Q * tau * log2(e) * 2^e_h to f16 once: each logit term moves
        # by up to 2^-11 of itself, so the error of a weight grows with its logit.  The spiked key
        # lifts the logits of the queries correlated with query 0 to hundreds of octaves, where
        # that is a few percent of the few weights that dominate those rows: 1.4e-2 and 2.1e-2
        # max-abs on two input draws (the exact form: 2e-3).  The rel-L2 bar is unchanged; the
        # max-abs bar for this input in this opt-in form is 5e-2.
        e_abs, e_rel = errors(got, ref)
        assert np.all(np.isfinite(got)) and e_abs <= 5e-2 and e_rel <= 5e-3, (label, e_abs, e_rel)


# f16 score form (PRESCALE_Q): plain SGA, enhanced SGA (UNIT and COUNT means, pi^3), dense with
# split work items (dense-37x37), G2F on packed f16 keys (g2f-37x37, also split), the phase
# shift and the global mean, and G2M (one mean key).
PRESCALED = [CASES[i] for i in (0, 1, 2, 4, 5, 6, 7, 8, 9)] + [NEW["sga6-phase-count"], NEW["sga4-global-count-phase"],
                                                               NEW["sga2-phase-empty-sets"], NEW["g2m"]]


@pytest.mark.parametrize("desc,label", PRESCALED, ids=[c[1] for c in PRESCALED])
@pytest.mark.parametrize("out_dtype", ["fp32", "bf16"])
def test_parity_prescaled_q(lib, desc, label, out_dtype):
    """The f16 score form: packed keys f16(k * 2^-e_h), Q * tau * log2(e) * 2^e_h rounded to
    f16 once, on the seeded workload inputs."""
    q, k, v = inputs_for(desc, "bf16", seed=13)
    _, got, _, _ = run(lib, desc, q, k, v, out_dtype=out_dtype, prescale_q=True)
    ref = oracle.attention(q, k, v, desc, workers=4)
    print(label, out_dtype, "f16 form max-abs %.3e rel-L2 %.3e" % errors(got, ref))
    assert_close(got, ref, fp32=False, label=label + "/f16-" + out_dtype)


def _key_exp(kmax_bits):
    """The documented key-scale exponent: 2^-e puts the largest |k| in [128, 256)."""
    if kmax_bits == 0:
        return 0
    km = np.array([kmax_bits << 16], dtype=np.uint32).view(np.float32)[0]
    e = int(np.frexp(np.float64(km))[1]) - 8
    return min(max(e, -120), 120)


F16_PACKED = [CASES[5], CASES[8], CASES[9], NEW["sga4-global-count-phase"], NEW["g2m"]]


@pytest.mark.parametrize("desc,label", F16_PACKED, ids=[c[1] for c in F16_PACKED])
@pytest.mark.parametrize("scale", [1.0, 2.0 ** 20, 2.0 ** -30], ids=["k", "k*2^20", "k*2^-30"])
def test_f16_packed_keys(lib, desc, label, scale):
    """f16 score form: the per-head maximum is the largest |k| among the packed keys (S and the
    means), and every packed key row is f16(k * 2^-e_h) exactly, e_h from that maximum; keys
    scaled far from 1 (with Q scaled inversely, so the logits stay put) still match the oracle."""
    import torch
    from synth import bf16_bits_to_f32, f32_to_bf16_bits
    q, k, v = inputs_for(desc, "bf16", seed=14)
    if scale != 1.0:
        k = f32_to_bf16_bits(bf16_bits_to_f32(k) * np.float32(scale))
        q = f32_to_bf16_bits(bf16_bits_to_f32(q) / np.float32(scale))
    plan, got, ws, _ = run(lib, desc, q, k, v, prescale_q=True)
    lay = plan.layout()
    H, d = desc.heads, desc.head_dim
    rows = lay["segments"] * lay["segment_rows"]
    kmax = ws[lay["off_kmax"]:lay["off_kmax"] + 4 * H].view(torch.int32).cpu().numpy().view(np.uint32)
    kp = ws[lay["off_kpack"]:lay["off_kpack"] + H * rows * d * 2].view(torch.int16).cpu().numpy().view(np.uint16)
    kp = kp.reshape(H, rows, d)
    if desc.g2f:
        src = [np.arange(f * desc.L, (f + 1) * desc.L) for f in range(desc.frames)]
        seg = lay["segment_rows"]
        packed_bf16 = np.zeros((H, rows, d), dtype=np.uint16)
        for f, s_ in enumerate(src):
            packed_bf16[:, f * seg:f * seg + s_.size] = k[:, s_]
    else:
        S = oracle.index_set(desc)
        nS, M = S.size, lay["keys_per_segment"] - S.size
        means = ws[lay["off_means"]:lay["off_means"] + H * M * 2 * d * 2].view(torch.int16).cpu().numpy()
        means = means.view(np.uint16).reshape(H, M, 2, d)
        packed_bf16 = np.zeros((H, rows, d), dtype=np.uint16)
        packed_bf16[:, :nS] = k[:, S]
        packed_bf16[:, nS:nS + M] = means[:, :, 0]
    for h in range(H):
        assert kmax[h] == int((packed_bf16[h] & 0x7FFF).max())
        e = _key_exp(int(kmax[h]))
        want = (bf16_bits_to_f32(packed_bf16[h]).astype(np.float64) * 2.0 ** -e).astype(np.float16).view(np.uint16)
        assert np.array_equal(kp[h], want)
    ref = oracle.attention(q, k, v, desc, workers=4)
    assert_close(got, ref, fp32=False, label=f"{label}/f16-keys-x{scale:g}")


SIZED = [
    (Desc(3, 5, 7, 2, sigma=1, log_size=True), "dense-tiny-sized"),
    (Desc(6, 13, 11, 2, sigma=6, diag=True, log_size=True), "sga6-diag-sized"),
    (Desc(5, 13, 11, 3, g2f=True, log_size=True), "g2f-sized"),
    (Desc(7, 37, 37, 2, sigma=4, diag=True, phase_shift=True, log_size=True), "sga4-phase-diag-sized-37x37"),
    (Desc(3, 37, 37, 2, sigma=1, log_size=True), "dense-sized-37x37"),
]


def run_sized(va, desc, q, k, v, log_g, out_dtype="fp32", in_dtype="bf16"):
    import torch
    plan = va.Plan(**plan_kwargs(desc, in_dtype, out_dtype))
    out = plan.new_output()
    plan.forward_sized(to_device(q), to_device(k), to_device(v), torch.from_numpy(log_g).cuda(), out,
                       plan.new_workspace())
    torch.cuda.synchronize()
    return out.float().cpu().numpy()


@pytest.mark.parametrize("desc,label", SIZED, ids=[c[1] for c in SIZED])
@pytest.mark.parametrize("out_dtype", ["fp32", "bf16"])
def test_parity_log_size(lib, desc, label, out_dtype):
    """Size-aware keys (+ log g on each token key's logit) with seeded group sizes 1..4."""
    from synth import make_log_sizes
    print(f"[sized] {label} {out_dtype}", flush=True)
    q, k, v = inputs_for(desc, "bf16", seed=zlib.crc32(label.encode()) % 1000)
    _, lg = make_log_sizes(desc.frames, desc.grid_h, desc.grid_w, desc.n_special, seed=5)
    got = run_sized(lib, desc, q, k, v, lg, out_dtype=out_dtype)
    ref = oracle.attention(q, k, v, desc, workers=4, log_g=lg)
    assert_close(got, ref, fp32=False, label=label + "/" + out_dtype)


@pytest.mark.parametrize("desc,label", [(Desc(4, 8, 8, 2, sigma=4, diag=True, log_size=True), "fp32-sga4-sized"),
                                        (Desc(3, 9, 9, 2, g2f=True, log_size=True), "fp32-g2f-sized")],
                         ids=["fp32-sga4-sized", "fp32-g2f-sized"])
def test_parity_log_size_fp32(lib, desc, label):
    from synth import make_log_sizes
    q, k, v = inputs_for(desc, "fp32", seed=9)
    _, lg = make_log_sizes(desc.frames, desc.grid_h, desc.grid_w, desc.n_special, seed=6)
    got = run_sized(lib, desc, q, k, v, lg, in_dtype="fp32")
    ref = oracle.attention(q, k, v, desc, log_g=lg)
    assert_close(got, ref, fp32=True, label=label)


@pytest.mark.parametrize("desc,label", [(Desc(6, 13, 11, 2, sigma=4, diag=True, log_size=True), "sga4-sized-extreme"),
                                        (Desc(5, 37, 37, 2, sigma=6, diag=True, log_size=True), "sga6-sized-extreme-37x37"),
                                        (Desc(3, 37, 37, 2, g2f=True, log_size=True), "g2f-sized-extreme-37x37")],
                         ids=["sga4", "sga6-37x37", "g2f-37x37"])
def test_log_size_extreme(lib, desc, label):
    """Sizes far outside 1..4: a few tokens late in the key range stand for up to e^25 tokens
    (each pulls its row's running max up by tens of octaves mid-stream, through the rescale
    path), one group of tokens is fractional (ln g = -20), the rest stay small."""
    from synth import make_log_sizes
    q, k, v = inputs_for(desc, "bf16", seed=41)
    _, lg = make_log_sizes(desc.frames, desc.grid_h, desc.grid_w, desc.n_special, seed=7)
    rng = np.random.default_rng(41)
    late = rng.choice(np.arange(desc.T // 2, desc.T), size=6, replace=False)
    lg[late] = np.array([25.0, 12.5, 7.0, 18.0, 3.0, 21.0], dtype=np.float32)
    lg[rng.choice(desc.T // 2, size=4, replace=False)] = -20.0
    got = run_sized(lib, desc, q, k, v, lg)
    ref = oracle.attention(q, k, v, desc, workers=4, log_g=lg)
    assert_close(got, ref, fp32=False, label=label)


def test_log_size_zero_sizes_equal_plain_path(lib):
    """log g = 0 everywhere: the size-aware kernel gives the plain kernel's weights bit for bit;
    the outputs then differ only by the order of the float32 row sums (the plain kernel sums P
    on the matrix cores, the size-aware one with VALU dot2 instructions), a few ulp at most."""
    desc = Desc(6, 13, 11, 2, sigma=6, diag=True, log_size=True)
    plain = Desc(6, 13, 11, 2, sigma=6, diag=True)
    q, k, v = inputs_for(desc, "bf16", seed=10)
    got = run_sized(lib, desc, q, k, v, np.zeros(desc.T, dtype=np.float32))
    _, ref, _, _ = run(lib, plain, q, k, v)
    assert np.all(np.abs(got - ref) <= 4e-7 * np.abs(ref) + 1e-9), float(np.max(np.abs(got - ref)))


TIED = [(Desc(6, 13, 11, 2, sigma=6, diag=True, mean=True), "sga6-enh"),
        (Desc(7, 37, 37, 2, sigma=4, diag=True, mean=True, mean_count=True), "sga4-enh-count-37x37"),
        (Desc(4, 37, 37, 2, g2f=True), "g2f-37x37"),
        (Desc(3, 37, 37, 2, sigma=1), "dense-37x37")]


@pytest.mark.parametrize("desc,label", TIED, ids=[c[1] for c in TIED])
@pytest.mark.parametrize("prescale_q", [False, True], ids=["exact", "f16"])
def test_parity_tied_qk(lib, desc, label, prescale_q):
    """Stress input: K carries Q's per-position component, so a query's logits peak at its own
    patch position in every frame (about tau * 0.49 * 64 = 3.9 above the rest), far from the
    first tile's keys, which moves the running max."""
    print(f"[tied] {label} {prescale_q}", flush=True)
    q, k, v = make_qkv(desc.frames, desc.grid_h, desc.grid_w, desc.n_special, desc.heads, desc.head_dim,
                       dtype="bf16", seed=21, tie_qk=True)
    _, got, _, _ = run(lib, desc, q, k, v, prescale_q=prescale_q)
    ref = oracle.attention(q, k, v, desc, workers=4)
    print(label, "tied max-abs %.3e rel-L2 %.3e" % errors(got, ref))
    assert_close(got, ref, fp32=False, label=label + "/tied")


def test_collapse_identity(lib):
    """Collapse identity: when every dropped K/V row of a frame is the same row, SGA with COUNT
    means and no diagonal term equals dense attention (a mean key with bias ln|D_f| stands for
    |D_f| copies of that key).  GPU SGA against the oracle's dense attention."""
    desc = Desc(5, 13, 11, 2, sigma=6, mean=True, mean_count=True)
    dense = Desc(5, 13, 11, 2, sigma=1)
    q, k, v = inputs_for(desc, "bf16", seed=22)
    kept = set(oracle.index_set(desc).tolist())
    for f in range(desc.frames):
        dropped = [t for t in range(f * desc.L, (f + 1) * desc.L) if t not in kept]
        if dropped:
            k[:, dropped] = k[:, dropped[:1]]
            v[:, dropped] = v[:, dropped[:1]]
    _, got, _, _ = run(lib, desc, q, k, v)
    ref = oracle.attention(q, k, v, dense, workers=4)
    assert_close(got, ref, fp32=False, label="collapse")


def test_g2f_reads_stop_at_tensor_end(lib):
    """bf16 G2F reads K and V in place; the last frame's last key tile runs past the end of the
    tensors and must be cut there by the copies' range check: NaN right after both tensors
    leaves the output finite and equal to the oracle's."""
    import torch
    desc = Desc(3, 13, 11, 2, g2f=True)  # L = 145: the last tile of a frame holds 17 keys
    q, k, v = inputs_for(desc, "bf16", seed=23)
    plan = lib.Plan(**plan_kwargs(desc))

    def poisoned(x):
        n = x.size
        big = torch.full((n + 64 * 64 * 4,), float("nan"), dtype=torch.bfloat16, device="cuda")
        big[:n] = to_device(x).reshape(-1)
        return big[:n].view(x.shape)

    kd, vd = poisoned(k), poisoned(v)
    out = plan.new_output()
    ws = plan.new_workspace()
    plan.forward(to_device(q), kd, vd, out, ws)
    torch.cuda.synchronize()
    got = out.float().cpu().numpy()
    assert_close(got, oracle.attention(q, k, v, desc), fp32=False, label="g2f-poisoned-tail")


EDGE = [
    (Desc(1, 1, 1, 1, n_special=0, sigma=1), "one-token"),
    (Desc(1, 1, 1, 2, n_special=0, g2f=True), "one-token-g2f"),
    (Desc(1, 4, 5, 2, sigma=6, diag=True, mean=True), "one-frame-sga6"),      # frame 0 dense: every key kept
    (Desc(2, 1, 1, 1, n_special=0, sigma=4, diag=True, mean=True), "one-patch-frames"),  # nothing dropped
    (Desc(3, 9, 8, 1, n_special=0, sigma=9, diag=True, mean=True, mean_count=True), "no-specials-sga9"),
    (Desc(2, 2, 65, 1, n_special=0, sigma=2, diag=True, mean=True, ref_dense=False), "wide-grid-pi3"),
    (Desc(3, 13, 11, 1, n_special=7, sigma=6, diag=True, mean=True, phase_shift=True), "seven-specials-phase"),
    (Desc(2, 2, 2, 4096, n_special=1, sigma=4, diag=True, mean=True), "max-heads"),  # the largest head count
    (Desc(2, 2, 3, 4096, n_special=1, g2f=True), "max-heads-g2f"),
]


@pytest.mark.parametrize("desc,label", EDGE, ids=[c[1] for c in EDGE])
@pytest.mark.parametrize("prescale_q", [False, True], ids=["exact", "f16"])
def test_edge_shapes(lib, desc, label, prescale_q):
    """Degenerate geometries: a single token (softmax over one key: out = v), a single frame
    (everything dense), one-patch frames (no dropped patch, so no diagonal or mean term), no
    special tokens, a grid one row high, more specials than usual, the largest head count a plan
    accepts (4096); exact and f16 score forms."""
    q, k, v = inputs_for(desc, "bf16", seed=31)
    _, got, _, _ = run(lib, desc, q, k, v, prescale_q=prescale_q)
    ref = oracle.attention(q, k, v, desc, workers=4)
    assert_close(got, ref, fp32=False, label=f"{label}/{'f16' if prescale_q else 'exact'}")
    if desc.T == 1:
        from synth import bf16_bits_to_f32
        assert np.array_equal(got, bf16_bits_to_f32(v).astype(np.float32))  # one key: weight exactly 1


def _random_desc(rng):
    """A seeded random valid descriptor: geometry, form and options."""
    frames = int(rng.integers(1, 10))
    gh, gw = int(rng.integers(1, 21)), int(rng.integers(1, 21))
    ns = int(rng.integers(0, 8))
    heads = int(rng.integers(1, 4))
    form = rng.choice(["dense", "sga", "g2f", "g2m"], p=[0.15, 0.65, 0.12, 0.08])
    if form == "g2f":
        return Desc(frames, gh, gw, heads, n_special=ns, g2f=True, log_size=bool(rng.random() < 0.3))
    if form == "g2m":
        return Desc(frames, gh, gw, heads, n_special=ns, g2m=True)
    sigma = 1 if form == "dense" else int(rng.choice([2, 4, 6, 9]))
    log_size = bool(rng.random() < 0.2)
    mean = (not log_size) and bool(rng.random() < 0.7)
    return Desc(frames, gh, gw, heads, n_special=ns, sigma=sigma, ref_dense=bool(rng.random() < 0.7),
                diag=bool(rng.random() < 0.7), mean=mean, mean_count=mean and bool(rng.random() < 0.5),
                phase_shift=bool(rng.random() < 0.4), mean_global=mean and bool(rng.random() < 0.3),
                log_size=log_size)


@pytest.mark.parametrize("case", range(160))
def test_random_configs(lib, case):
    """Seeded random geometries (1-9 frames, grids up to 20 x 20, 0-7 specials, 1-3 heads) and
    forms with random options, in both score forms and both output types, against the oracle."""
    import torch
    from synth import make_log_sizes
    rng = np.random.default_rng(1000 + case)
    desc = _random_desc(rng)
    prescale_q = bool(rng.random() < 0.5)
    out_dtype = "bf16" if rng.random() < 0.3 else "fp32"
    print(f"[random {case}] {desc} prescale_q={prescale_q} out={out_dtype}", flush=True)
    q, k, v = inputs_for(desc, "bf16", seed=case)
    plan = lib.Plan(**plan_kwargs(desc, "bf16", out_dtype), prescale_q=prescale_q)
    out, ws = plan.new_output(), plan.new_workspace()
    log_g = None
    if desc.log_size:
        _, log_g = make_log_sizes(desc.frames, desc.grid_h, desc.grid_w, desc.n_special, seed=case)
        plan.forward_sized(to_device(q), to_device(k), to_device(v), torch.from_numpy(log_g).cuda(), out, ws)
    else:
        plan.forward(to_device(q), to_device(k), to_device(v), out, ws)
    torch.cuda.synchronize()
    ref = oracle.attention(q, k, v, desc, workers=4, log_g=log_g)
    assert_close(out.float().cpu().numpy(), ref, fp32=False, label=f"random-{case}")


@pytest.mark.parametrize("case", range(40))
def test_random_configs_fp32(lib, case):
    """The float32 path (float32 in and out) on seeded random geometries and forms, at the
    float32 bar."""
    import torch
    from synth import make_log_sizes
    rng = np.random.default_rng(7000 + case)  # (this seed range draws every form)
    desc = _random_desc(rng)
    print(f"[random fp32 {case}] {desc}", flush=True)
    q, k, v = inputs_for(desc, "fp32", seed=500 + case)
    plan = lib.Plan(**plan_kwargs(desc, "fp32", "fp32"))
    out, ws = plan.new_output(), plan.new_workspace()
    log_g = None
    if desc.log_size:
        _, log_g = make_log_sizes(desc.frames, desc.grid_h, desc.grid_w, desc.n_special, seed=500 + case)
        plan.forward_sized(to_device(q), to_device(k), to_device(v), torch.from_numpy(log_g).cuda(), out, ws)
    else:
        plan.forward(to_device(q), to_device(k), to_device(v), out, ws)
    torch.cuda.synchronize()
    ref = oracle.attention(q, k, v, desc, workers=4, log_g=log_g)
    assert_close(out.cpu().numpy(), ref, fp32=True, label=f"random-fp32-{case}")


@pytest.mark.parametrize("model", ["vggt", "pi3"])
def test_scheduled_layers_match_oracle(lib, model):
    """The 24 global layers of VGGT (pi^3) under AVGGT's schedule (sigma 4) on one set of inputs,
    run by the scheduled driver: each layer's output equals the oracle's for that layer's form
    (G2F for 0-8 (0-9), enhanced SGA for 9-19 (10-19) with frame 0 dense for VGGT only, dense for
    20-23), and layers of one form give identical bits."""
    import torch
    import vggt_global_attention_attn_amd as va
    d0 = Desc(6, 13, 11, 2, sigma=4, diag=True, mean=True)
    q, k, v = inputs_for(d0, "bf16", seed=41)
    qd, kd, vd = to_device(q), to_device(k), to_device(v)
    sl = va.ScheduledLayers(6, 13, 11, 2, model=model, sigma=4)
    outs = []
    for layer in range(24):
        out = sl.plan(layer).new_output().fill_(float("nan"))
        sl.forward(layer, qd, kd, vd, out)
        outs.append(out)
    torch.cuda.synchronize()
    refs = {}
    for layer, kw in enumerate(va.layer_schedule(model, 4)):
        desc = Desc(6, 13, 11, 2, sigma=kw["sigma"], g2f=kw["g2f"], ref_dense=kw["ref_dense"], diag=kw["diag"],
                    mean=kw["mean"])
        key = (kw["sigma"], kw["g2f"], kw["diag"])
        if key not in refs:
            refs[key] = (oracle.attention(q, k, v, desc), outs[layer])
        ref, first = refs[key]
        got = outs[layer].double().cpu().numpy()
        assert_close(got, ref, fp32=False, label=f"layer {layer}")
        assert torch.equal(outs[layer], first)
    assert len(refs) == 3


# Guard-padded buffers: the output and the workspace sit inside larger allocations whose
# 4 KiB borders hold a byte pattern, and the inputs are compared before and after; a write
# outside [out, out + size) or [ws, ws + workspace_bytes), or into Q/K/V, changes one of them.
# One case per kernel path: global forms with the diagonal and means (exact and f16 score
# form, bf16 output), split pieces and their merge, G2F read in place (first-half last tile,
# two-tile frames), G2M, size-aware keys, and the fp32 path.
GUARDED = [
    (Desc(3, 5, 7, 2, sigma=6, diag=True, mean=True), "sga6-enh", "bf16", "fp32", False),
    (Desc(6, 13, 11, 2, sigma=4, diag=True, mean=True, mean_count=True), "sga4-f16", "bf16", "bf16", True),
    (Desc(3, 37, 37, 2, sigma=1), "dense-split", "bf16", "fp32", False),
    (Desc(4, 37, 37, 2, g2f=True), "g2f-37x37", "bf16", "bf16", False),
    (Desc(5, 5, 13, 3, g2f=True), "g2f-L70", "bf16", "fp32", False),
    (Desc(4, 13, 11, 2, g2m=True), "g2m", "bf16", "fp32", False),
    (Desc(5, 13, 11, 3, sigma=4, diag=True, log_size=True), "sga4-sized", "bf16", "fp32", False),
    (Desc(4, 8, 8, 2, sigma=4, diag=True, mean=True), "fp32-tiny", "fp32", "fp32", False),
]


@pytest.mark.parametrize("desc,label,in_dtype,out_dtype,prescale_q", GUARDED, ids=[c[1] for c in GUARDED])
def test_guard_padded_buffers(lib, desc, label, in_dtype, out_dtype, prescale_q):
    import torch
    from synth import make_log_sizes
    print(f"[guard] {label}", flush=True)
    q, k, v = inputs_for(desc, in_dtype, seed=17)
    qd, kd, vd = to_device(q), to_device(k), to_device(v)
    before = [x.clone() for x in (qd, kd, vd)]
    plan = lib.Plan(**plan_kwargs(desc, in_dtype, out_dtype), prescale_q=prescale_q)
    G = 4096
    out_dt = torch.bfloat16 if out_dtype == "bf16" else torch.float32
    out_bytes = desc.heads * plan.T * desc.head_dim * (2 if out_dtype == "bf16" else 4)
    ws_bytes = max(1, plan.workspace_bytes)
    raw_out = torch.full((G + out_bytes + G,), 0xA5, dtype=torch.uint8, device="cuda")
    raw_ws = torch.full((G + ws_bytes + G,), 0x5A, dtype=torch.uint8, device="cuda")
    out = raw_out[G:G + out_bytes].view(out_dt).view(desc.heads, plan.T, desc.head_dim)
    ws = raw_ws[G:G + ws_bytes]
    lg = None
    if desc.log_size:
        _, lg = make_log_sizes(desc.frames, desc.grid_h, desc.grid_w, desc.n_special, seed=5)
        plan.forward_sized(qd, kd, vd, torch.from_numpy(lg).cuda(), out, ws)
    else:
        plan.forward(qd, kd, vd, out, ws)
    torch.cuda.synchronize()
    for raw, lo, hi, pat in ((raw_out, G, G + out_bytes, 0xA5), (raw_ws, G, G + ws_bytes, 0x5A)):
        assert bool((raw[:lo] == pat).all()) and bool((raw[hi:] == pat).all()), f"{label}: write outside a buffer"
    for a, b in zip(before, (qd, kd, vd)):
        assert torch.equal(a, b), f"{label}: an input changed"
    ref = oracle.attention(q, k, v, desc, workers=4, log_g=lg)
    got = out.float().cpu().numpy()
    if prescale_q:  # the f16 score form on ordinary inputs: the usual bars
        assert_close(got, ref, fp32=False, label=label)
    else:
        assert_close(got, ref, fp32=(in_dtype == "fp32"), label=label)
