"""GPU parity of the parity-selected and collapsed tensor-product plans against the oracle.

Symmetric / skew path selections and outputs collapsed by (l3, p3), forward and
backward, fp32 / bf16 / fp64, per-row and shared weights, at ragged batches; the
L = 4 irreps of the 100k-point workload; the unaligned (one channel per lane)
route; groups of different multiplicities; the full-size tp_large batch on
sampled rows; x blocks no path reads (zero gradient); and the convolution with
every path selection and collapsed outputs (fused and general kernels).
"""

import numpy as np
import pytest

from oracle import conv as oconv
from oracle import graph as ograph
from oracle import tp as otp
from oracle import sh as osh
from oracle.irreps import Layout
from clebsch_gordan_tensor_amd import synth
from tests.gpu_util import TOL, assert_close, dev, host, out_blocks, w_blocks, x_blocks, y_blocks

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
if not torch.cuda.is_available():
    pytest.skip("no GPU", allow_module_level=True)
cgtp = pytest.importorskip("clebsch_gordan_tensor_amd.cgtp")

TPL = synth.CONFIGS["tp_large"]


def inputs(L, B, seed, shared, dtype):
    x = synth.gaussian((B, L.dim_x), seed, synth.S_X)
    y = synth.gaussian((B, L.dim_y), seed, synth.S_Y)
    w = synth.gaussian((L.w_numel,) if shared else (B, L.w_numel), seed, synth.S_W)
    g = synth.gaussian((B, L.dim_out), seed, synth.S_G)
    d = [dev(a, dtype) for a in (x, y, w, g)]
    return d, [host(t) for t in d]


def run(ix, iy, io, B, dtype, select, collapse, shared=False, seed=0):
    L = Layout(ix, iy, io, select, collapse)
    plan = cgtp.Plan(ix, iy, io, dtype=dtype, wkind="shared" if shared else "per_row", select=select,
                     collapse=collapse)
    (x, y, w, g), (hx, hy, hw, hg) = inputs(L, B, seed, shared, dtype)
    tag = "%s %s collapse=%s B=%d %s" % (ix, select, collapse, B, dtype)
    out = plan.tp_forward(x, y, w)
    torch.cuda.synchronize()
    assert_close(host(out), otp.forward(L, hx, hy, hw), out_blocks(L), dtype, "forward " + tag)
    dx, dy, dw = plan.tp_backward(x, y, w, g)
    torch.cuda.synchronize()
    rdx, rdy, rdw = otp.backward(L, hx, hy, hw, hg)
    assert_close(host(dx), rdx, x_blocks(L), dtype, "grad_x " + tag)
    assert_close(host(dy), rdy, y_blocks(L), dtype, "grad_y " + tag)
    assert_close(host(dw), rdw, w_blocks(L), dtype, "grad_w " + tag)


@pytest.mark.parametrize("dtype", ["f32", "bf16", "f64"])
@pytest.mark.parametrize("collapse", [False, True])
@pytest.mark.parametrize("select", ["all", "symmetric", "skew"])
def test_tp_large_irreps_variants(select, collapse, dtype):
    run(TPL["irreps_x"], TPL["irreps_y"], TPL["irreps_out"], 1037, dtype, select, collapse)


@pytest.mark.parametrize("select", ["all", "symmetric"])
def test_shared_weights_collapsed(select):
    c = synth.CONFIGS["tp_small"]
    run(c["irreps_x"], c["irreps_y"], c["irreps_out"], 3000, "f32", select, True, shared=True)


@pytest.mark.parametrize("dtype", ["f32", "f64"])
def test_lmax4_collapsed(dtype):
    c = synth.CONFIGS["conv_uniform100k"]
    run(c["irreps_x"], c["irreps_y"], c["irreps_out"], 333, dtype, "all", True)


@pytest.mark.parametrize("ix,iy,io", [
    ("4x0e+6x1e", "0e", "1e+0e"),                    # groups of different multiplicity, one channel per lane
    ("8x1o+8x0e+8x2o", "0e+1o+2e", "0e+1o+1e+2e+2o"),
    ("264x0e+264x1o", "0e+1o", "0e+1o+1e"),           # more channel groups than lanes per row
])
def test_irregular_collapsed(ix, iy, io):
    run(ix, iy, io, 257, "f32", "all", True)


@pytest.mark.parametrize("shared", [False, True])
def test_unread_x_block_gets_zero_gradient(shared):
    # the 4x1o block reaches no output: its gradient is zero, not left unwritten
    run("4x1o+8x0e", "0e", "0e", 300, "f32", "all", False, shared=shared)


def test_unaligned_collapsed_forward():
    ix, iy, io = TPL["irreps_x"], TPL["irreps_y"], TPL["irreps_out"]
    L = Layout(ix, iy, io, "all", True)
    plan = cgtp.Plan(ix, iy, io, collapse=True)
    (x, y, w, g), (hx, hy, hw, hg) = inputs(L, 70, 4, False, "f32")
    xb = torch.empty(70 * L.dim_x + 1, device="cuda")
    xv = xb[1:].view(70, L.dim_x)  # 4-byte offset: the one-channel-per-lane route
    xv.copy_(x)
    out = plan.tp_forward(xv, y, w)
    torch.cuda.synchronize()
    assert_close(host(out), otp.forward(L, hx, hy, hw), out_blocks(L), "f32", "unaligned collapsed forward")


def test_collapsed_determinism_and_empty():
    ix, iy, io = TPL["irreps_x"], TPL["irreps_y"], TPL["irreps_out"]
    L = Layout(ix, iy, io, "all", True)
    plan = cgtp.Plan(ix, iy, io, collapse=True)
    (x, y, w, g), _ = inputs(L, 2000, 5, False, "f32")
    a = [t.clone() for t in (plan.tp_forward(x, y, w),) + plan.tp_backward(x, y, w, g)]
    b = [t.clone() for t in (plan.tp_forward(x, y, w),) + plan.tp_backward(x, y, w, g)]
    for u, v in zip(a, b):
        assert torch.equal(u, v)
    e = plan.tp_forward(x[:0], y[:0], w[:0])
    torch.cuda.synchronize()
    assert e.shape == (0, L.dim_out)


def test_tp_large_collapsed_full_size_sampled():
    """tp_large at its full batch with collapsed outputs (8 blocks of 128 channels)."""
    ix, iy, io = TPL["irreps_x"], TPL["irreps_y"], TPL["irreps_out"]
    L = Layout(ix, iy, io, "all", True)
    plan = cgtp.Plan(ix, iy, io, collapse=True)
    B = TPL["B"]
    gen = torch.Generator(device="cuda")
    gen.manual_seed(0)
    x = torch.randn((B, L.dim_x), generator=gen, device="cuda")
    w = torch.randn((B, L.w_numel), generator=gen, device="cuda")
    y = dev(osh.real_sh(3, synth.unit_vectors(B, 0)), "f32")
    g = torch.randn((B, L.dim_out), generator=gen, device="cuda")
    out = plan.tp_forward(x, y, w)
    dx, dy, dw = plan.tp_backward(x, y, w, g)
    torch.cuda.synchronize()
    rows = np.sort(np.random.default_rng(1).choice(B, 256, replace=False))
    rows[-1] = B - 1
    ri = torch.from_numpy(rows).cuda()
    hx, hy, hw, hg = host(x[ri]), host(y[ri]), host(w[ri]), host(g[ri])
    assert_close(host(out[ri]), otp.forward(L, hx, hy, hw), out_blocks(L), "f32", "full-size collapsed forward")
    rdx, rdy, rdw = otp.backward(L, hx, hy, hw, hg)
    assert_close(host(dx[ri]), rdx, x_blocks(L), "f32", "full-size collapsed grad_x")
    assert_close(host(dy[ri]), rdy, y_blocks(L), "f32", "full-size collapsed grad_y")
    assert_close(host(dw[ri]), rdw, w_blocks(L), "f32", "full-size collapsed grad_w")


def small_graph(seed=0):
    pos = synth.uniform_box(60, 6.0, seed)
    src, dst, vec = synth.radius_graph(pos, 6.0, 2.5)
    row_ptr, src_s, perm = ograph.csr_from_coo(60, src, dst)
    return 60, row_ptr, src_s, vec[perm]


CONV_PLANS = [
    ("16x0e+16x1o+16x2e", "0e+1o+2e", "0e+0o+1e+1o+2e+2o", 2),          # fused kernels
    ("8x0e+8x1o", "0e+1o+2e+3o", "0e+0o+1e+1o+2e+2o+3e+3o", 3),        # fused, L > l1
    ("68x0e+68x2e", "0e+1o+2e", "0e+1o+2e+3o+4e", 2),                   # two channel chunks
    ("3x1o+3x0e", "1o+1e", "0e+1o+1e+2e", -1),                          # general kernel (repeated degree)
]


@pytest.mark.parametrize("select", ["all", "symmetric", "skew"])
@pytest.mark.parametrize("collapse", [False, True])
@pytest.mark.parametrize("ix,iy,io,lmax", CONV_PLANS)
@pytest.mark.parametrize("dtype", ["f32", "bf16", "f64"])
def test_conv_variants(ix, iy, io, lmax, select, collapse, dtype):
    """Convolution with selected paths and collapsed outputs (skew: the 0e block
    reaches no output, 0 + l2 + l2 being even, so its grad_x is zero)."""
    try:
        L = Layout(ix, iy, io, select, collapse)
    except ValueError:
        pytest.skip("collapsed outputs fed by different multiplicities")
    if not L.paths:
        pytest.skip("no path in this selection")
    N, row_ptr, src, vec = small_graph(3)
    E = len(src)
    plan = cgtp.Plan(ix, iy, io, dtype=dtype, select=select, collapse=collapse)
    graph = cgtp.Graph(N, torch.from_numpy(row_ptr.astype(np.int32)).cuda(),
                       torch.from_numpy(src.astype(np.int32)).cuda())
    x = synth.gaussian((N, L.dim_x), 7, synth.S_X)
    Y = osh.real_sh(lmax, vec) if lmax >= 0 else synth.gaussian((E, L.dim_y), 7, synth.S_Y)
    w = synth.gaussian((E, L.w_numel), 7, synth.S_W)
    g = synth.gaussian((N, L.dim_out), 7, synth.S_G)
    dx_, dY_, dw_, dg_ = (dev(a, dtype) for a in (x, Y, w, g))
    hx, hY, hw, hg = (host(t) for t in (dx_, dY_, dw_, dg_))
    scale = 0.37
    tag = "%s %s collapse=%s %s" % (ix, select, collapse, dtype)
    out = plan.conv_forward(graph, dx_, dY_, dw_, scale)
    gx, gY, gw = plan.conv_backward(graph, dx_, dY_, dw_, scale, dg_)
    torch.cuda.synchronize()
    assert_close(host(out), oconv.forward(L, row_ptr, src, hx, hY, hw, scale), out_blocks(L), dtype,
                 "conv " + tag)
    rdx, rdY, rdw = oconv.backward(L, row_ptr, src, hx, hY, hw, scale, hg)
    assert_close(host(gx), rdx, x_blocks(L), dtype, "conv grad_x " + tag)
    assert_close(host(gY), rdY, y_blocks(L), dtype, "conv grad_Y " + tag)
    assert_close(host(gw), rdw, w_blocks(L), dtype, "conv grad_w " + tag)
