"""The allocation-free tensor-product backward (cgtp_tp_backward_noalloc) against
the workspace entry point (cgtp_tp_backward) and the oracle.

Shared weights keep per-row grad_w partials in the library's device scratch:
two calls in a row, the first over 100,000 rows (several 256-row-aligned passes
through the scratch), the second over a smaller ragged batch, each bitwise equal
to the workspace entry point; the second also against the oracle. A row of
weights too wide for one 256-row pass is refused with WORKSPACE before any
launch, and a narrower batch of the same plan that fits runs.
"""

import numpy as np
import pytest

from oracle import tp as otp
from oracle.irreps import Layout
from clebsch_gordan_tensor_amd import synth
from tests.gpu_util import assert_close, host, w_blocks, x_blocks, y_blocks

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
if not torch.cuda.is_available():
    pytest.skip("no GPU", allow_module_level=True)
cgtp = pytest.importorskip("clebsch_gordan_tensor_amd.cgtp")


def device_inputs(plan, B, seed):
    gen = torch.Generator(device="cuda")
    gen.manual_seed(seed)
    x = torch.randn((B, plan.dim_x), generator=gen, device="cuda")
    y = torch.randn((B, plan.dim_y), generator=gen, device="cuda")
    w = torch.randn((plan.w_numel,), generator=gen, device="cuda")
    g = torch.randn((B, plan.dim_out), generator=gen, device="cuda")
    return x, y, w, g


def test_noalloc_matches_workspace_backward_twice():
    c = synth.CONFIGS["tp_small"]
    ix, iy, io = c["irreps_x"], c["irreps_y"], c["irreps_out"]
    plan = cgtp.Plan(ix, iy, io, wkind="shared")
    for B, seed in ((100000, 0), (4133, 1)):
        print("noalloc backward: tp_small irreps, shared weights, B =", B, flush=True)
        x, y, w, g = device_inputs(plan, B, seed)
        ref = plan.tp_backward(x, y, w, g)
        got = plan.tp_backward_noalloc(x, y, w, g)
        torch.cuda.synchronize()
        for a, b, what in zip(got, ref, ("grad_x", "grad_y", "grad_w")):
            assert torch.equal(a, b), "%s differs from the workspace entry point at B = %d" % (what, B)
    L = Layout(ix, iy, io)
    rdx, rdy, rdw = otp.backward(L, host(x), host(y), host(w), host(g))
    assert_close(host(got[0]), rdx, x_blocks(L), "f32", "noalloc grad_x")
    assert_close(host(got[1]), rdy, y_blocks(L), "f32", "noalloc grad_y")
    assert_close(host(got[2]), rdw, w_blocks(L), "f32", "noalloc grad_w")


def test_noalloc_size_limit():
    # 16384 channels x 5 paths = 81,920 shared weights: 320 KB of fp32 partials
    # per row, so about 204 rows fit the 64 MiB scratch in one pass and a batch
    # that needs a 256-row pass is refused
    ix, iy, io = "16384x0e", "0e+1o+2e+3o+4e", "0e+1o+2e+3o+4e"
    plan = cgtp.Plan(ix, iy, io, wkind="shared")
    assert plan.w_numel == 81920
    print("noalloc size limit: W =", plan.w_numel, flush=True)
    x, y, w, g = device_inputs(plan, 300, 2)
    with pytest.raises(cgtp.CgtpError) as e:
        plan.tp_backward_noalloc(x, y, w, g)
    assert e.value.status == 5 and "scratch" in str(e.value)
    xs, ys, gs = x[:200].contiguous(), y[:200].contiguous(), g[:200].contiguous()
    got = plan.tp_backward_noalloc(xs, ys, w, gs)
    ref = plan.tp_backward(xs, ys, w, gs)
    torch.cuda.synchronize()
    for a, b in zip(got, ref):
        assert torch.equal(a, b)


def test_noalloc_empty_and_per_row():
    c = synth.CONFIGS["tp_small"]
    plan = cgtp.Plan(c["irreps_x"], c["irreps_y"], c["irreps_out"], wkind="shared")
    x, y, w, g = device_inputs(plan, 0, 3)
    dw = torch.full((plan.w_numel,), 7.0, device="cuda")
    plan.tp_backward_noalloc(x, y, w, g, need=(False, False, True), out=(None, None, dw))
    torch.cuda.synchronize()
    assert float(dw.abs().max()) == 0.0
    pr = cgtp.Plan(c["irreps_x"], c["irreps_y"], c["irreps_out"], wkind="per_row")
    gen = torch.Generator(device="cuda")
    gen.manual_seed(4)
    B = 777
    x = torch.randn((B, pr.dim_x), generator=gen, device="cuda")
    y = torch.randn((B, pr.dim_y), generator=gen, device="cuda")
    w = torch.randn((B, pr.w_numel), generator=gen, device="cuda")
    g = torch.randn((B, pr.dim_out), generator=gen, device="cuda")
    for a, b in zip(pr.tp_backward_noalloc(x, y, w, g), pr.tp_backward(x, y, w, g)):
        assert torch.equal(a, b)
