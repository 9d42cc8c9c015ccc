"""Streams and graphs through the C ABI.  Forwards enqueued on two non-default streams at once
(one plan with two workspaces, and a second plan) give the same bits as the same forwards run
one after another on the current stream; a forward captured into a HIP graph and replayed, with
the inputs rewritten, the output and workspace poisoned and other eager work between replays,
gives the eager bits on every replay.  The kernels are deterministic (no order-dependent float
atomics; the f16 key maximum is an integer max), so equality is exact."""
import numpy as np
import pytest

from oracle import Desc
from tests.gpu_util import inputs_for, plan_kwargs, to_device

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def va():
    import vggt_global_attention_attn_amd as va
    return va


def _inputs(desc, seed):
    return [to_device(x) for x in inputs_for(desc, "bf16", seed=seed)]


def test_two_streams_match_sequential(va):
    import torch
    d1 = Desc(7, 37, 37, 2, sigma=4, diag=True, mean=True)
    d2 = Desc(4, 37, 37, 2, g2f=True)
    p1, p2 = va.Plan(**plan_kwargs(d1)), va.Plan(**plan_kwargs(d2))
    xa, xb, xc = _inputs(d1, 21), _inputs(d1, 23), _inputs(d2, 22)
    jobs = [(p1, xa), (p1, xb), (p2, xc)]
    ref = []
    for plan, (q, k, v) in jobs:
        o, ws = plan.new_output(), plan.new_workspace()
        plan.forward(q, k, v, o, ws)
        ref.append(o)
    torch.cuda.synchronize()

    s1, s2 = torch.cuda.Stream(), torch.cuda.Stream()  # default priority
    outs = [plan.new_output().fill_(float("nan")) for plan, _ in jobs]
    wss = [plan.new_workspace() for plan, _ in jobs]
    for s in (s1, s2):
        s.wait_stream(torch.cuda.current_stream())
    streams = [s1, s2, s1]
    for _ in range(3):  # enqueued back to back, no synchronisation between them
        for i, (plan, (q, k, v)) in enumerate(jobs):
            plan.forward(q, k, v, outs[i], wss[i], stream=streams[i])
    torch.cuda.synchronize()
    for i in range(len(jobs)):
        assert torch.equal(outs[i], ref[i]), f"job {i} differs from its sequential result"


GRAPH_CASES = [
    (Desc(6, 13, 11, 2, sigma=4, diag=True, mean=True, mean_count=True), False, "sga4-enh-count"),
    (Desc(6, 13, 11, 2, sigma=6, diag=True, mean=True), True, "sga6-enh-f16"),  # key-max clear + atomics
    (Desc(3, 37, 37, 2, sigma=1), False, "dense-split"),  # key-range pieces + merge kernel
    (Desc(4, 37, 37, 2, g2f=True), False, "g2f-in-place"),
    (Desc(4, 13, 11, 2, g2m=True), False, "g2m"),
]


@pytest.mark.parametrize("desc,prescale_q,label", GRAPH_CASES, ids=[c[2] for c in GRAPH_CASES])
def test_graph_replays_match_eager(va, desc, prescale_q, label):
    import torch
    plan = va.Plan(**plan_kwargs(desc), prescale_q=prescale_q)
    ins = [_inputs(desc, s) for s in (31, 32, 33)]
    ws_e = plan.new_workspace()
    eager = []
    for q, k, v in ins:
        o = plan.new_output()
        plan.forward(q, k, v, o, ws_e)
        eager.append(o)
    torch.cuda.synchronize()
    assert not torch.equal(eager[0], eager[1])

    sq, sk, sv = (t.clone() for t in ins[0])
    out, ws = plan.new_output(), plan.new_workspace()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):  # warm-up off the capture, as torch's capture recipe asks
        plan.forward(sq, sk, sv, out, ws)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()

    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        plan.forward(sq, sk, sv, out, ws)
    torch.cuda.synchronize()
    for r in range(6):
        q, k, v = ins[r % 3]
        sq.copy_(q)
        sk.copy_(k)
        sv.copy_(v)
        out.fill_(float("nan"))
        ws.fill_(0xFF)
        torch.cuda.synchronize()
        g.replay()
        junk = torch.randn(1 << 18, device="cuda").sum()  # eager work between replays
        torch.cuda.synchronize()
        assert np.isfinite(junk.item())
        assert torch.equal(out, eager[r % 3]), f"{label}: replay {r} differs from the eager result"
