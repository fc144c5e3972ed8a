"""GPU parity of the double backward (reverse mode of the backward) against the oracle.

Tensor product: fp32 / bf16 / fp64, per-row and shared weights, collapsed
outputs, missing cotangents and skipped outputs, ragged batches. Convolution:
fused and general kernels, collapsed outputs, on a small radius graph, and the
1000-molecule water box at full size (the force-training shape: cotangents on
grad_sh and grad_w only) on sampled nodes and edges.
"""

import numpy as np
import pytest

from oracle import conv as oconv
from oracle import graph as ograph
from oracle import tp as otp
from oracle import sh as osh
from oracle.irreps import Layout
from clebsch_gordan_tensor_amd import synth
from tests.gpu_util import assert_close, dev, host, out_blocks, w_blocks, x_blocks, y_blocks

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
if not torch.cuda.is_available():
    pytest.skip("no GPU", allow_module_level=True)
cgtp = pytest.importorskip("clebsch_gordan_tensor_amd.cgtp")

TPL = synth.CONFIGS["tp_large"]


def tp_case(ix, iy, io, B, dtype, shared=False, collapse=False, drop=(), skip=(), seed=0):
    L = Layout(ix, iy, io, "all", collapse)
    plan = cgtp.Plan(ix, iy, io, dtype=dtype, wkind="shared" if shared else "per_row", collapse=collapse)
    wshape = (L.w_numel,) if shared else (B, L.w_numel)
    h = [synth.gaussian((B, L.dim_x), seed, synth.S_X), synth.gaussian((B, L.dim_y), seed, synth.S_Y),
         synth.gaussian(wshape, seed, synth.S_W), synth.gaussian((B, L.dim_out), seed, synth.S_G)]
    gg = [synth.gaussian((B, L.dim_x), seed + 50, synth.S_X), synth.gaussian((B, L.dim_y), seed + 50, synth.S_Y),
          synth.gaussian(wshape, seed + 50, synth.S_W)]
    d = [dev(a, dtype) for a in h]
    dg = [None if k in drop else dev(a, dtype) for k, a in enumerate(gg)]
    hd = [host(t) for t in d]
    hg = [None if t is None else host(t) for t in dg]
    need = tuple(k not in skip for k in range(4))
    outs = plan.tp_double_backward(*d, gg=tuple(dg), need=need)
    torch.cuda.synchronize()
    ref = otp.double_backward(L, *hd, *hg)
    tag = "%s B=%d %s shared=%s collapse=%s drop=%s" % (ix, B, dtype, shared, collapse, drop)
    blocks = [x_blocks(L), y_blocks(L), w_blocks(L), out_blocks(L)]
    for k, (o, r) in enumerate(zip(outs, ref)):
        if k in skip:
            assert o is None
            continue
        hr = host(o)
        if k == 2 and shared:
            hr, r = hr[None], r[None]
        assert_close(hr, r, blocks[k], dtype, "%s of %s" % (("ddx", "ddy", "ddw", "ddg")[k], tag))


@pytest.mark.parametrize("dtype", ["f32", "bf16", "f64"])
def test_tp_large_irreps(dtype):
    tp_case(TPL["irreps_x"], TPL["irreps_y"], TPL["irreps_out"], 517, dtype)


@pytest.mark.parametrize("shared", [False, True])
@pytest.mark.parametrize("collapse", [False, True])
def test_tp_weights_and_collapse(shared, collapse):
    c = synth.CONFIGS["tp_small"]
    tp_case(c["irreps_x"], c["irreps_y"], c["irreps_out"], 1300, "f32", shared=shared, collapse=collapse)


@pytest.mark.parametrize("drop", [(0,), (1,), (2,), (0, 2), (0, 1, 2)])
def test_tp_missing_cotangents(drop):
    c = synth.CONFIGS["tp_small"]
    tp_case(c["irreps_x"], c["irreps_y"], c["irreps_out"], 300, "f32", drop=drop)


def test_tp_skipped_outputs():
    c = synth.CONFIGS["tp_small"]
    tp_case(c["irreps_x"], c["irreps_y"], c["irreps_out"], 300, "f32", skip=(0, 3))
    tp_case(c["irreps_x"], c["irreps_y"], c["irreps_out"], 300, "f32", skip=(1, 2))


def small_graph(seed=0):
    pos = synth.uniform_box(60, 6.0, seed)
    src, dst, vec = synth.radius_graph(pos, 6.0, 2.5)
    row_ptr, src_s, perm = ograph.csr_from_coo(60, src, dst)
    return 60, row_ptr, src_s, vec[perm]


CONV_PLANS = [
    ("16x0e+16x1o+16x2e", "0e+1o+2e", "0e+0o+1e+1o+2e+2o", 2),          # fused kernels
    ("3x1o+3x0e", "1o+1e", "0e+1o+1e+2e", -1),                          # general kernel
]


@pytest.mark.parametrize("collapse", [False, True])
@pytest.mark.parametrize("ix,iy,io,lmax", CONV_PLANS)
@pytest.mark.parametrize("dtype", ["f32", "f64", "bf16"])
def test_conv_small_graph(ix, iy, io, lmax, collapse, dtype):
    L = Layout(ix, iy, io, "all", collapse)
    N, row_ptr, src, vec = small_graph(4)
    E = len(src)
    plan = cgtp.Plan(ix, iy, io, dtype=dtype, collapse=collapse)
    graph = cgtp.Graph(N, torch.from_numpy(row_ptr.astype(np.int32)).cuda(),
                       torch.from_numpy(src.astype(np.int32)).cuda())
    Y = osh.real_sh(lmax, vec) if lmax >= 0 else synth.gaussian((E, L.dim_y), 8, synth.S_Y)
    h = [synth.gaussian((N, L.dim_x), 8, synth.S_X), Y, synth.gaussian((E, L.w_numel), 8, synth.S_W),
         synth.gaussian((N, L.dim_out), 8, synth.S_G)]
    gg = [synth.gaussian((N, L.dim_x), 9, synth.S_X), synth.gaussian((E, L.dim_y), 9, synth.S_Y),
          synth.gaussian((E, L.w_numel), 9, synth.S_W)]
    d = [dev(a, dtype) for a in h]
    dg = [dev(a, dtype) for a in gg]
    hd, hg = [host(t) for t in d], [host(t) for t in dg]
    sc = 0.43
    outs = plan.conv_double_backward(graph, d[0], d[1], d[2], sc, d[3], gg=tuple(dg))
    torch.cuda.synchronize()
    ref = oconv.double_backward(L, row_ptr, src, hd[0], hd[1], hd[2], sc, hd[3], *hg)
    blocks = [x_blocks(L), y_blocks(L), w_blocks(L), out_blocks(L)]
    for k in range(4):
        assert_close(host(outs[k]), ref[k], blocks[k], dtype,
                     "conv %s of %s collapse=%s %s" % (("ddx", "ddsh", "ddw", "ddg")[k], ix, collapse, dtype))


def test_conv_water1k_force_training_sampled():
    """Full-size water1k (E = 156,076): cotangents on grad_sh and grad_w only (the
    shape of training on forces, whose gradient reaches the conv through the
    harmonics and the radial weights); sampled nodes and edges against the oracle."""
    c = synth.CONFIGS["conv_water1k"]
    L = Layout(c["irreps_x"], c["irreps_y"], c["irreps_out"])
    plan = cgtp.Plan(c["irreps_x"], c["irreps_y"], c["irreps_out"])
    pos = synth.positions_for(c, 0)
    src, dst, vec = synth.radius_graph(pos, c["box"], c["r_cut"])
    N = pos.shape[0]
    row_ptr, s, perm = ograph.csr_from_coo(N, src, dst)
    E = len(s)
    graph = cgtp.Graph(N, torch.from_numpy(row_ptr.astype(np.int32)).cuda(), torch.from_numpy(s.astype(np.int32)).cuda())
    Y = dev(osh.real_sh(c["L"], vec[perm]), "f32")
    gen = torch.Generator(device="cuda")
    gen.manual_seed(2)
    x = torch.randn((N, L.dim_x), generator=gen, device="cuda")
    w = torch.randn((E, L.w_numel), generator=gen, device="cuda")
    g = torch.randn((N, L.dim_out), generator=gen, device="cuda")
    gY = torch.randn((E, L.dim_y), generator=gen, device="cuda")
    gw = torch.randn((E, L.w_numel), generator=gen, device="cuda")
    sc = oconv.avg_neighbors_scale(N, E)
    ddx, ddY, ddw, ddg = plan.conv_double_backward(graph, x, Y, w, sc, g, gg=(None, gY, gw))
    torch.cuda.synchronize()
    # oracle on the subgraph of the sampled receivers' edges (their ddg, ddY, ddw are exact there)
    rng = np.random.default_rng(3)
    nodes = np.sort(rng.choice(N, 24, replace=False))
    eidx = np.concatenate([np.arange(row_ptr[n], row_ptr[n + 1]) for n in nodes])
    sub_rp = np.zeros(len(nodes) + 1, np.int64)
    sub_rp[1:] = np.cumsum([row_ptr[n + 1] - row_ptr[n] for n in nodes])
    hx = host(x)
    he = lambda t: host(t[torch.from_numpy(eidx).cuda()])
    _, rY, rw, rg = oconv.double_backward(L, sub_rp, s[eidx], hx, he(Y), he(w), sc,
                                          host(g[torch.from_numpy(nodes).cuda()]), None, he(gY), he(gw))
    assert_close(host(ddg[torch.from_numpy(nodes).cuda()]), rg, out_blocks(L), "f32", "water1k ddg")
    assert_close(he(ddY), rY, y_blocks(L), "f32", "water1k ddsh")
    assert_close(he(ddw), rw, w_blocks(L), "f32", "water1k ddw")
    # ddx through the adjoint identity <ddx, x> = <gY, dY> with the backward's dY
    # (ddx has the terms back(x, gY, w, g).dx + back(x, Y, gw, g).dx, each linear in x)
    _, dY, dw = plan.conv_backward(graph, x, Y, w, sc, g, need=(False, True, True))
    torch.cuda.synchronize()
    lhs = torch.sum(ddx.double() * x.double()).item()
    rhs = torch.sum(gY.double() * dY.double()).item() + torch.sum(gw.double() * dw.double()).item()
    scale = torch.sum((gY.double() * dY.double()).abs()).item() + torch.sum((gw.double() * dw.double()).abs()).item()
    assert abs(lhs - rhs) <= 1e-5 * scale


def test_empty_batch_and_edgeless_graph():
    """B = 0: a shared-weight plan still gets a zero cotangent for w; a graph
    without edges gives zero cotangents for x and grad_out (outputs are
    pre-filled with NaN so an unwritten one fails)."""
    c = synth.CONFIGS["tp_small"]
    plan = cgtp.Plan(c["irreps_x"], c["irreps_y"], c["irreps_out"], wkind="shared")
    z = lambda *s: torch.zeros(s, device="cuda")
    nan = lambda *s: torch.full(s, float("nan"), device="cuda")
    x, y, g = z(0, plan.dim_x), z(0, plan.dim_y), z(0, plan.dim_out)
    w = torch.randn(plan.w_numel, device="cuda")
    gw = torch.randn(plan.w_numel, device="cuda")
    ddw = nan(plan.w_numel)
    outs = plan.tp_double_backward(x, y, w, g, gg=(None, None, gw),
                                   out=(None, None, ddw, None))
    torch.cuda.synchronize()
    assert outs[2] is ddw and float(ddw.abs().max()) == 0.0
    assert outs[0].shape == (0, plan.dim_x) and outs[3].shape == (0, plan.dim_out)

    cp = synth.CONFIGS["conv_water1k"]
    plan = cgtp.Plan(cp["irreps_x"], cp["irreps_y"], cp["irreps_out"])
    N = 5
    graph = cgtp.Graph(N, torch.zeros(N + 1, dtype=torch.int32, device="cuda"),
                       torch.zeros(0, dtype=torch.int32, device="cuda"))
    x, g = torch.randn(N, plan.dim_x, device="cuda"), torch.randn(N, plan.dim_out, device="cuda")
    sh, w = z(0, plan.dim_y), z(0, plan.w_numel)
    gx = torch.randn(N, plan.dim_x, device="cuda")
    ddx, ddg = nan(N, plan.dim_x), nan(N, plan.dim_out)
    outs = plan.conv_double_backward(graph, x, sh, w, 0.5, g, gg=(gx, z(0, plan.dim_y), z(0, plan.w_numel)),
                                     out=(ddx, None, None, ddg))
    torch.cuda.synchronize()
    assert float(ddx.abs().max()) == 0.0 and float(ddg.abs().max()) == 0.0
    assert outs[1].shape == (0, plan.dim_y) and outs[2].shape == (0, plan.w_numel)
