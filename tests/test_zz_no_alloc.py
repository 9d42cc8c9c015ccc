"""The no-allocation entry point, vggt_attn_forward_noalloc, through the C ABI: its output equals
that of vggt_attn_forward (caller workspace) bit for bit -- both run the same kernels on the same
inputs, and the kernels are deterministic -- on calls in a row on one GPU, each smaller than the
one before and the last of another dtype pair, so that every call after the first runs on the
static workspace the previous one left filled.  The reference workspaces are NaN-poisoned and
every output starts as NaN, so a part of either path that read memory it had not written would
show."""
import pytest

from oracle import Desc
from tests.gpu_util import inputs_for, plan_kwargs, to_device

pytestmark = pytest.mark.gpu

# Enhanced SGA, sigma 4, 12 frames x 1374 tokens, 4 heads; dense 3 x 1374 tokens, 2 heads (its
# last round of work-groups runs as key-range pieces, merged through the workspace); a sigma 6
# plan with the log-count mean bias on a non-square grid, float32.
CALLS = [
    (Desc(12, 37, 37, 4, sigma=4, diag=True, mean=True), "bf16", "fp32", 31),
    (Desc(3, 37, 37, 2, sigma=1), "bf16", "bf16", 32),
    (Desc(3, 13, 11, 2, sigma=6, diag=True, mean=True, mean_count=True), "fp32", "fp32", 33),
]


def test_noalloc_matches_forward_in_a_row():
    import torch
    import vggt_global_attention_attn_amd as va
    sizes = []
    for desc, in_dtype, out_dtype, seed in CALLS:
        q, k, v = (to_device(x) for x in inputs_for(desc, in_dtype, seed=seed))
        plan = va.Plan(**plan_kwargs(desc, in_dtype, out_dtype))
        ws = plan.new_workspace()
        ws.view(torch.uint8).fill_(0xFF)  # NaN in every float view of it
        ref = plan.new_output().fill_(float("nan"))
        plan.forward(q, k, v, ref, ws)
        got = plan.new_output().fill_(float("nan"))
        plan.forward_noalloc(q, k, v, got)
        torch.cuda.synchronize()
        assert torch.isfinite(ref).all()
        assert torch.equal(got, ref), f"{desc}: no-allocation output differs from vggt_attn_forward"
        sizes.append(plan.T * plan.heads)
    assert sizes == sorted(sizes, reverse=True) and len(set(sizes)) == len(sizes)
