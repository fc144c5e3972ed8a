"""GPU parity of the convolution with outputs collapsed by (l3, p3), against the oracle.

The collapsed comparison setting of the E3J paper (appendix B.3: 2048 nodes,
45 neighbours per node on average, 128 channels per degree, L = 3 and 4) runs
the collapsed fused forward at x degrees l1 = 0..L with L = 3 and 4; these
tests run exactly those irreps:

* on a small radius graph in full (every receiver, forward and backward), in
  fp32, bf16 and fp64, so every kernel instantiation the benchmark times is
  compared with the oracle, including the L = 4 slot tables that split one x
  block's output types over several waves;
* at full size (2048 nodes) on sampled receivers and senders, in the
  benchmark's launch configuration;
* with y irreps whose parities are not (-1)^l (a y block '2o' beside '0e', or
  '1e' among even harmonics): the slots of one x block that share (l2 mod 2,
  l3) then feed different output types, so these plans must not share an
  accumulator (the planner sends them to the general kernel);
* the double backward of a collapsed plan at the L = 4 irreps.
"""

import math

import numpy as np
import pytest

from oracle import conv as oconv
from oracle import sh as osh
from oracle.irreps import Layout
from clebsch_gordan_tensor_amd import synth
from tests.gpu_util import assert_close, block_errors, dev, host, out_blocks, w_blocks, x_blocks, y_blocks

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
if not torch.cuda.is_available():
    pytest.skip("no GPU", allow_module_level=True)
cgtp = pytest.importorskip("clebsch_gordan_tensor_amd.cgtp")

from tests.test_gpu_conv import Case, check_sampled  # noqa: E402


def small_case(n=30, box=6.0, r_cut=2.5, seed=13):
    return Case(synth.uniform_box(n, box, seed), box, r_cut)


def full_check(ix, iy, io, dtype, case, Y_host, seed=0, collapse=True, scale=0.29):
    L = Layout(ix, iy, io, "all", collapse)
    plan = cgtp.Plan(ix, iy, io, dtype=dtype, collapse=collapse)
    x = dev(synth.gaussian((case.N, L.dim_x), seed, synth.S_X), dtype)
    Y = dev(Y_host, dtype)
    w = dev(synth.gaussian((case.E, L.w_numel), seed, synth.S_W), dtype)
    g = dev(synth.gaussian((case.N, L.dim_out), seed, synth.S_G), dtype)
    out = plan.conv_forward(case.graph, x, Y, w, scale)
    dx, dY, dw = plan.conv_backward(case.graph, x, Y, w, scale, g)
    torch.cuda.synchronize()
    hx, hY, hw, hg = host(x), host(Y), host(w), host(g)
    tag = "%s | %s collapse=%s %s" % (ix, iy, collapse, dtype)
    assert_close(host(out), oconv.forward(L, case.h_row, case.h_src, hx, hY, hw, scale), out_blocks(L), dtype,
                 "forward " + tag)
    rdx, rdY, rdw = oconv.backward(L, case.h_row, case.h_src, hx, hY, hw, scale, hg)
    assert_close(host(dx), rdx, x_blocks(L), dtype, "grad_x " + tag)
    assert_close(host(dY), rdY, y_blocks(L), dtype, "grad_sh " + tag)
    assert_close(host(dw), rdw, w_blocks(L), dtype, "grad_w " + tag)


@pytest.mark.parametrize("dtype", ["f32", "bf16", "f64"])
@pytest.mark.parametrize("name", ["conv_collapsed_l3", "conv_collapsed_l4"])
def test_benchmark_irreps_small_graph_full(name, dtype):
    c = synth.CONFIGS[name]
    case = small_case()
    assert case.E > 200
    full_check(c["irreps_x"], c["irreps_y"], c["irreps_out"], dtype, case, osh.real_sh(c["L"], case.vec))


@pytest.mark.parametrize("name", ["conv_collapsed_l3", "conv_collapsed_l4"])
def test_benchmark_workload_full_size_sampled(name):
    """The 2048-node comparison graph at full size, as the benchmark launches it."""
    c = synth.CONFIGS[name]
    L = Layout(c["irreps_x"], c["irreps_y"], c["irreps_out"], "all", True)
    case = Case(synth.positions_for(c, 0), c["box"], c["r_cut"])
    plan = cgtp.Plan(c["irreps_x"], c["irreps_y"], c["irreps_out"], collapse=True)
    Y = dev(osh.real_sh(c["L"], case.vec), "f32")
    W1, W2 = synth.mlp_params(8, 64, L.w_numel, 0)
    r = torch.from_numpy(np.linalg.norm(case.vec, axis=1)).float().cuda()
    w = synth.radial_weights_torch(r, c["r_cut"], torch.from_numpy(W1).float().cuda(),
                                   torch.from_numpy(W2).float().cuda()).contiguous()
    gen = torch.Generator(device="cuda")
    gen.manual_seed(0)
    x = torch.randn((case.N, L.dim_x), generator=gen, device="cuda")
    check_sampled(L, case, plan, x, Y, w, 1.0 / math.sqrt(case.E / case.N), "f32", backward=True, n_nodes=40)


@pytest.mark.parametrize("dtype", ["f32", "f64"])
@pytest.mark.parametrize("ix,iy,io", [
    ("8x2e", "0e+2o", "2e+2o"),                                   # (l2=0, l3=2) -> 2e, (l2=2, l3=2) -> 2o
    ("8x0e+8x1o+8x2e", "0e+1e+2e", "0e+0o+1e+1o+2e+2o"),          # a '1e' among even harmonics
    ("8x1o+8x2e", "0o+1e+2o", "0e+0o+1e+1o+2e+2o+3e+3o"),         # every y parity flipped: fused kernel still valid
])
def test_y_parities_other_than_harmonics(ix, iy, io, dtype):
    case = small_case(n=36, seed=12)
    L = Layout(ix, iy, io, "all", True)
    Y = synth.gaussian((case.E, L.dim_y), 3, synth.S_Y)
    full_check(ix, iy, io, dtype, case, Y, seed=3)
    full_check(ix, iy, io, dtype, case, Y, seed=3, collapse=False)


def test_collapsed_double_backward_l4():
    c = synth.CONFIGS["conv_collapsed_l4"]
    ix, iy, io = c["irreps_x"], c["irreps_y"], c["irreps_out"]
    L = Layout(ix, iy, io, "all", True)
    case = small_case(n=24, seed=14)
    plan = cgtp.Plan(ix, iy, io, collapse=True)
    x = dev(synth.gaussian((case.N, L.dim_x), 4, synth.S_X), "f32")
    Y = dev(osh.real_sh(4, case.vec), "f32")
    w = dev(synth.gaussian((case.E, L.w_numel), 4, synth.S_W), "f32")
    g = dev(synth.gaussian((case.N, L.dim_out), 4, synth.S_G), "f32")
    ggx = dev(synth.gaussian((case.N, L.dim_x), 5, synth.S_X), "f32")
    ggY = dev(synth.gaussian((case.E, L.dim_y), 5, synth.S_Y), "f32")
    ggw = dev(synth.gaussian((case.E, L.w_numel), 5, synth.S_W), "f32")
    sc = 0.31
    res = plan.conv_double_backward(case.graph, x, Y, w, sc, g, gg=(ggx, ggY, ggw))
    torch.cuda.synchronize()
    ref = oconv.double_backward(L, case.h_row, case.h_src, host(x), host(Y), host(w), sc, host(g),
                                host(ggx), host(ggY), host(ggw))
    for got, want, blocks, what in zip(res, ref, (x_blocks(L), y_blocks(L), w_blocks(L), out_blocks(L)),
                                       ("x", "sh", "w", "grad_out")):
        assert_close(host(got), want, blocks, "f32", "collapsed double backward " + what)


@pytest.mark.parametrize("general", [False, True])
@pytest.mark.parametrize("name", ["conv_collapsed_l3", "conv_collapsed_l4"])
def test_bf16_collapsed_running_sum_in_fp32(name, general):
    """bf16 storage with a workspace: the x blocks add into an fp32 running sum
    that is rounded to bf16 once, so the output is bitwise the fp32 plan's
    output (same kernels and order on the same bf16-representable inputs)
    rounded to bf16. Without the workspace the running sum is rounded after
    every x block (within the bf16 tolerance of the oracle), or by the general
    kernel after every path. general: misaligned weights send both plans to
    the general (per-path) kernel."""
    c = synth.CONFIGS[name]
    ix, iy, io = c["irreps_x"], c["irreps_y"], c["irreps_out"]
    L = Layout(ix, iy, io, "all", True)
    case = small_case(n=40, seed=21)
    pb = cgtp.Plan(ix, iy, io, dtype="bf16", collapse=True)
    pf = cgtp.Plan(ix, iy, io, dtype="f32", collapse=True)
    assert pb.workspace_size(cgtp.OP_CONV_FORWARD, graph=case.graph) == case.N * L.dim_out * 4
    assert pf.workspace_size(cgtp.OP_CONV_FORWARD, graph=case.graph) == 0
    x = dev(synth.gaussian((case.N, L.dim_x), 6, synth.S_X), "bf16")
    Y = dev(osh.real_sh(c["L"], case.vec), "bf16")
    w = dev(synth.gaussian((case.E, L.w_numel), 6, synth.S_W), "bf16")

    def maybe_misalign(t):
        if not general:
            return t
        buf = torch.empty(t.numel() + 1, dtype=t.dtype, device="cuda")
        v = buf[1:].view(t.shape)
        v.copy_(t)
        return v

    xf, Yf, wf = x.float(), Y.float(), maybe_misalign(w.float())
    wb = maybe_misalign(w)
    sc = 0.37
    once = pb.conv_forward(case.graph, x, Y, wb, sc)
    per_block = pb.conv_forward(case.graph, x, Y, wb, sc, fp32_running_sum=False)
    ref32 = pf.conv_forward(case.graph, xf, Yf, wf, sc)
    torch.cuda.synchronize()
    assert torch.equal(once, ref32.to(torch.bfloat16))
    want = oconv.forward(L, case.h_row, case.h_src, host(x), host(Y), host(w), sc)
    e_once = assert_close(host(once), want, out_blocks(L), "bf16", "fp32 running sum")
    if general:
        # the general kernel adds path by path: without the workspace the sum is
        # rounded once per path (65 at L = 4), which can exceed the tolerance
        assert e_once <= max(block_errors(host(per_block), want, out_blocks(L)))
    else:
        assert_close(host(per_block), want, out_blocks(L), "bf16", "running sum rounded per x block")


def test_conv_forward_ws_errors_and_ignored_workspace():
    """cgtp_conv_forward_ws: a workspace smaller than the size query is refused
    (WORKSPACE) and a misaligned one too (INVALID_ARG), before any launch; plans
    that need none (fp32 storage, uncollapsed bf16) ignore one and give the
    results of cgtp_conv_forward bit for bit."""
    c = synth.CONFIGS["conv_collapsed_l3"]
    ix, iy, io = c["irreps_x"], c["irreps_y"], c["irreps_out"]
    L = Layout(ix, iy, io, "all", True)
    case = small_case(n=30, seed=22)
    pb = cgtp.Plan(ix, iy, io, dtype="bf16", collapse=True)
    x = dev(synth.gaussian((case.N, L.dim_x), 8, synth.S_X), "bf16")
    Y = dev(osh.real_sh(c["L"], case.vec), "bf16")
    w = dev(synth.gaussian((case.E, L.w_numel), 8, synth.S_W), "bf16")
    nws = pb.workspace_size(cgtp.OP_CONV_FORWARD, graph=case.graph)
    with pytest.raises(cgtp.CgtpError) as e:
        pb.conv_forward(case.graph, x, Y, w, 0.5, ws=torch.empty(nws - 16, dtype=torch.uint8, device="cuda"))
    assert e.value.status == 5
    buf = torch.empty(nws + 16, dtype=torch.uint8, device="cuda")
    with pytest.raises(cgtp.CgtpError) as e:
        pb.conv_forward(case.graph, x, Y, w, 0.5, ws=buf[4:4 + nws])
    assert e.value.status == 1
    del e
    for dtype, collapse in (("f32", True), ("bf16", False)):
        Lp = Layout(ix, iy, io, "all", collapse)
        p = cgtp.Plan(ix, iy, io, dtype=dtype, collapse=collapse)
        assert p.workspace_size(cgtp.OP_CONV_FORWARD, graph=case.graph) == 0
        xx = dev(synth.gaussian((case.N, Lp.dim_x), 9, synth.S_X), dtype)
        YY = dev(osh.real_sh(c["L"], case.vec), dtype)
        ww = dev(synth.gaussian((case.E, Lp.w_numel), 9, synth.S_W), dtype)
        a = p.conv_forward(case.graph, xx, YY, ww, 0.5, ws=torch.empty(64, dtype=torch.uint8, device="cuda"))
        b = p.conv_forward(case.graph, xx, YY, ww, 0.5, fp32_running_sum=False)
        torch.cuda.synchronize()
        assert torch.equal(a, b), (dtype, collapse)
