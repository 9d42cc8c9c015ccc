"""GPU parity at the workloads' full sizes, in the launch configuration the benchmark times
(pack + attend through the C ABI), on 4096 seeded query rows per workload (all heads), which
the oracle computes one by one; plus the bit-exact index set and |D_f| at full size.

Workloads: dense 32 frames (and G2M on the same tensors); SGA sigma 4 at 100 frames (UNIT and
COUNT means); G2F, SGA sigma 9, and sigma 9 with the phase-shifted grid and a global COUNT
mean on the same 200-frame tensors; SGA sigma 6 at 800 frames, with and without the phase
shift.  All use 37x37 patches + 5 special tokens per frame, 16 heads, d = 64, bf16 inputs and
fp32 output.  One gives every token a seeded group size of 1..4 (size-aware keys); the last two
run G2F and enhanced SGA sigma 9 at the largest token count a plan accepts.  Names ending in -f16 run the f16 score form
(PRESCALE_Q: packed keys f16(k * 2^-e_h), Q * tau * log2(e) * 2^e_h rounded to f16 once).  A separate test runs the 800-frame sigma 6
workload on the tied-Q/K stress input with bf16 output."""
import numpy as np
import pytest

import oracle
from oracle import Desc
from synth import host_threads, make_qkv, sample_rows
from tests.gpu_util import assert_close, errors, plan_kwargs

pytestmark = pytest.mark.gpu

FULL = [
    ("dense-32f", Desc(32, 37, 37, 16, sigma=1)),
    ("dense-32f-f16", Desc(32, 37, 37, 16, sigma=1)),
    ("g2m-32f", Desc(32, 37, 37, 16, g2m=True)),
    ("sga4-100f", Desc(100, 37, 37, 16, sigma=4, diag=True, mean=True)),
    ("sga4-100f-count", Desc(100, 37, 37, 16, sigma=4, diag=True, mean=True, mean_count=True)),
    ("g2f-200f", Desc(200, 37, 37, 16, g2f=True)),
    ("g2f-200f-f16", Desc(200, 37, 37, 16, g2f=True)),
    ("sga9-200f", Desc(200, 37, 37, 16, sigma=9, diag=True, mean=True)),
    ("sga9-200f-phase-global-count", Desc(200, 37, 37, 16, sigma=9, diag=True, mean=True, mean_count=True,
                                          phase_shift=True, mean_global=True)),
    ("sga6-800f", Desc(800, 37, 37, 16, sigma=6, diag=True, mean=True)),
    ("sga6-800f-f16", Desc(800, 37, 37, 16, sigma=6, diag=True, mean=True)),
    ("sga6-800f-phase", Desc(800, 37, 37, 16, sigma=6, diag=True, mean=True, phase_shift=True)),
    ("sga6-800f-sized", Desc(800, 37, 37, 16, sigma=6, diag=True, log_size=True)),
    # the largest plan the library accepts: T = 7,999,428 tokens (limit 8,000,000); with 6 heads
    # an [H][T][64] tensor holds 3.07e9 elements, so every offset needs 64 bits
    ("g2f-5822f-max", Desc(5822, 37, 37, 6, g2f=True)),
    # the global path at the same size (same tensors): 1,014,228 + 5,821 packed keys, 249,984
    # work items whose sparse last round runs as 4 key-range pieces and the merge
    ("sga9-5822f-max", Desc(5822, 37, 37, 6, sigma=9, diag=True, mean=True)),
]
# sampled rows per workload (4096 unless listed: each of these rows attends to a million keys)
ROWS = {"sga9-5822f-max": 512}

_cache = {}
_refs = {}  # oracle rows of the last workload, shared by its exact and f16 score-form cases


def device_inputs(desc):
    """Host and device copies of the seeded inputs of a geometry (one geometry cached)."""
    import torch
    key = (desc.frames, desc.grid_h, desc.grid_w, desc.heads)
    if key not in _cache:
        _cache.clear()
        # (the largest geometry, 9.2e9 values, draws on independent per-frame streams in parallel)
        q, k, v = make_qkv(desc.frames, desc.grid_h, desc.grid_w, desc.n_special, desc.heads, desc.head_dim,
                           "bf16", seed=0, per_frame_streams=desc.frames > 1000)
        up = lambda x: torch.from_numpy(x.view(np.int16)).view(torch.bfloat16).cuda()
        _cache[key] = ((q, k, v), (up(q), up(k), up(v)))
    return _cache[key]


@pytest.mark.timeout(900)
@pytest.mark.parametrize("name,desc", FULL, ids=[n for n, _ in FULL])
def test_full_size_sampled_rows(name, desc):
    import torch
    import vggt_global_attention_attn_amd as va
    print(f"[full] {name}: drawing inputs", flush=True)
    (q, k, v), (qd, kd, vd) = device_inputs(desc)
    # "-f16": the f16 score form (PRESCALE_Q)
    plan = va.Plan(**plan_kwargs(desc), prescale_q=name.endswith("-f16"))
    out = plan.new_output()
    ws = plan.new_workspace()
    print(f"[full] {name}: pack + attend", flush=True)
    log_g = None
    if desc.log_size:
        from synth import make_log_sizes
        _, log_g = make_log_sizes(desc.frames, desc.grid_h, desc.grid_w, desc.n_special, seed=5)
        plan.pack_sized(kd, vd, torch.from_numpy(log_g).cuda(), ws)
    else:
        plan.pack(kd, vd, ws)
    plan.attend(qd, kd, vd, out, ws)
    torch.cuda.synchronize()
    assert bool(torch.isfinite(out).all())
    if not desc.g2f:
        idx, dcount = plan.index_set(ws)
        assert np.array_equal(idx, oracle.index_set(desc))
        assert np.array_equal(dcount, oracle.dropped_counts(desc).astype(np.int32))
    rows = sample_rows(desc.frames, desc.grid_h, desc.grid_w, desc.n_special, count=ROWS.get(name, 4096), seed=1)
    got = out[:, torch.from_numpy(rows).cuda()].double().cpu().numpy()
    del out, ws
    base = name[:-len("-f16")] if name.endswith("-f16") else name
    if base not in _refs:
        print(f"[full] {name}: oracle on {rows.size} rows", flush=True)
        _refs.clear()
        _refs[base] = oracle.attention(q, k, v, desc, rows=rows, workers=host_threads(), log_g=log_g)
    ref = _refs[base]
    print(f"[full] {name}: max-abs %.3e rel-L2 %.3e" % errors(got, ref), flush=True)
    assert_close(got, ref, fp32=False, label=name)


@pytest.mark.timeout(900)
def test_full_size_tied_qk_bf16_out():
    """The 800-frame sigma 6 workload on the tied-Q/K stress input (K carries Q's per-position
    component, so every query's logits peak at its own slot in all 800 frames and the running max
    moves across the whole key range), with bf16 output, on the 4096 sampled rows."""
    import torch
    import vggt_global_attention_attn_amd as va
    desc = Desc(800, 37, 37, 16, sigma=6, diag=True, mean=True)
    _cache.clear()
    print("[full] tied-qk: drawing inputs", flush=True)
    q, k, v = make_qkv(desc.frames, desc.grid_h, desc.grid_w, desc.n_special, desc.heads, desc.head_dim,
                       "bf16", seed=0, tie_qk=True)
    up = lambda x: torch.from_numpy(x.view(np.int16)).view(torch.bfloat16).cuda()
    plan = va.Plan(**plan_kwargs(desc, out_dtype="bf16"))
    out = plan.new_output()
    ws = plan.new_workspace()
    print("[full] tied-qk: pack + attend", flush=True)
    plan.forward(up(q), up(k), up(v), out, ws)
    torch.cuda.synchronize()
    assert bool(torch.isfinite(out.float()).all())
    rows = sample_rows(desc.frames, desc.grid_h, desc.grid_w, desc.n_special, count=4096, seed=1)
    got = out[:, torch.from_numpy(rows).cuda()].double().cpu().numpy()
    del out, ws
    print(f"[full] tied-qk: oracle on {rows.size} rows", flush=True)
    ref = oracle.attention(q, k, v, desc, rows=rows, workers=host_threads())
    print("[full] tied-qk: max-abs %.3e rel-L2 %.3e" % errors(got, ref), flush=True)
    assert_close(got, ref, fp32=False, label="tied-qk-800f-bf16-out")
