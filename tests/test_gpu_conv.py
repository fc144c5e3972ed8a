"""GPU parity of the message-passing convolution (forward and backward).

Small graphs are compared in full; the three convolution workloads (water box
of 1000 molecules, water box of 8000, 100,000 uniform points) run at full size
in the benchmark's launch configuration and are checked on sampled receivers
(forward, grad_sh, grad_w) and sampled senders (grad_x) against the oracle.
Also: empty edge lists, isolated nodes, the general (non-fused) kernel, bitwise
determinism and rotation equivariance of the GPU output, and the force chain
(gradient with respect to the edge vectors: the library's harmonics backward of
grad_sh plus the radial network's chain of grad_w, which the caller owns).
"""

import math

import numpy as np
import pytest

from oracle import conv as oconv
from oracle import graph as ograph
from oracle import sh as osh
from oracle import tp as otp
from oracle import wigner
from oracle.irreps import Layout
from clebsch_gordan_tensor_amd import synth
from tests.gpu_util import TOL, assert_close, dev, host, out_blocks, rel_err, w_blocks, x_blocks, y_blocks

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
if not torch.cuda.is_available():
    pytest.skip("no GPU", allow_module_level=True)
cgtp = pytest.importorskip("clebsch_gordan_tensor_amd.cgtp")


def i32(a):
    return torch.from_numpy(np.ascontiguousarray(a, np.int32)).cuda()


class Case:
    """A graph on the device plus the oracle's view of it."""

    def __init__(self, pos, box, r_cut):
        src, dst, vec = synth.radius_graph(pos, box, r_cut)
        self.N, self.E = pos.shape[0], src.shape[0]
        self.row_ptr, self.src, perm = cgtp.csr_from_coo(self.N, i32(src), i32(dst))
        self.h_row, self.h_src, h_perm = ograph.csr_from_coo(self.N, src, dst)
        self.graph = cgtp.Graph(self.N, self.row_ptr, self.src)
        self.vec = vec[h_perm]  # CSR order
        self.h_dst = ograph.dst_of_csr(self.h_row)
        self.col_ptr, self.eid = ograph.csr_transpose(self.N, self.h_row, self.h_src)
        self.r_cut = r_cut


def small_inputs(L, case, seed, dtype, lmax):
    x = dev(synth.gaussian((case.N, L.dim_x), seed, synth.S_X), dtype)
    Y = dev(osh.real_sh(lmax, case.vec), dtype)
    W1, W2 = synth.mlp_params(8, 16, L.w_numel, seed)
    w = dev(synth.radial_weights_np(np.linalg.norm(case.vec, axis=1), case.r_cut, W1, W2), dtype)
    g = dev(synth.gaussian((case.N, L.dim_out), seed, synth.S_G), dtype)
    return x, Y, w, g


PLANS = [
    ("4x0e+4x1o+4x2e", "0e+1o+2e", "0e+0o+1e+1o+2e+2o", 2),                    # fused
    ("8x0e+8x1o", "0e+1o+2e+3o", "0e+0o+1e+1o+2e+2o+3e+3o", 3),               # fused, L > l1
    ("12x1o+4x2e", "0e+1o+2e", "0e+1o+2e", 2),                                 # fused, parity-filtered slots
    ("3x1o+5x0e", "1o+1e", "0e+1o+1e+2e", 1),                                  # general (repeated degree in y)
    ("68x0e+68x2e", "0e+1o+2e", "0e+1o+2e+3o+4e", 2),                          # two channel chunks
]


@pytest.mark.parametrize("ix,iy,io,lmax", PLANS)
@pytest.mark.parametrize("dtype", ["f32", "f64", "bf16"])
def test_small_graphs_full(ix, iy, io, lmax, dtype):
    L = Layout(ix, iy, io)
    case = Case(synth.uniform_box(90, 7.0, 1), 7.0, 2.6)
    plan = cgtp.Plan(ix, iy, io, dtype=dtype)
    if L.dim_y != (lmax + 1) ** 2:
        Y = dev(synth.gaussian((case.E, L.dim_y), 0, synth.S_Y), dtype)
        x, _, w, g = small_inputs(L, case, 0, dtype, 0)
    else:
        x, Y, w, g = small_inputs(L, case, 0, dtype, lmax)
    sc = oconv.avg_neighbors_scale(case.N, case.E)
    out = plan.conv_forward(case.graph, x, Y, w, sc)
    dx, dY, dw = plan.conv_backward(case.graph, x, Y, w, sc, g)
    torch.cuda.synchronize()
    hx, hY, hw, hg = host(x), host(Y), host(w), host(g)
    assert_close(host(out), oconv.forward(L, case.h_row, case.h_src, hx, hY, hw, sc), out_blocks(L), dtype,
                 "conv forward")
    rdx, rdY, rdw = oconv.backward(L, case.h_row, case.h_src, hx, hY, hw, sc, hg)
    assert_close(host(dx), rdx, x_blocks(L), dtype, "conv grad_x")
    assert_close(host(dY), rdY, y_blocks(L), dtype, "conv grad_sh")
    assert_close(host(dw), rdw, w_blocks(L), dtype, "conv grad_w")


def test_empty_edges_and_isolated_nodes():
    ix, iy, io = "4x0e+4x1o", "0e+1o", "0e+1o+1e"
    L = Layout(ix, iy, io)
    plan = cgtp.Plan(ix, iy, io)
    N = 6
    g0 = cgtp.Graph(N, i32(np.zeros(N + 1)), i32(np.zeros(0)))
    x = torch.randn((N, L.dim_x), device="cuda")
    out = torch.full((N, L.dim_out), 3.0, device="cuda")
    plan.conv_forward(g0, x, torch.zeros((0, L.dim_y), device="cuda"), torch.zeros((0, L.w_numel), device="cuda"),
                      1.0, out=out)
    dx = torch.full((N, L.dim_x), 3.0, device="cuda")
    plan.conv_backward(g0, x, torch.zeros((0, L.dim_y), device="cuda"), torch.zeros((0, L.w_numel), device="cuda"),
                       1.0, torch.randn((N, L.dim_out), device="cuda"), need=(True, True, True),
                       out=(dx, None, None))
    torch.cuda.synchronize()
    assert float(out.abs().max()) == 0.0 and float(dx.abs().max()) == 0.0
    # edges 0->2 and 5->2 only: every other row is zero
    row_ptr, s, perm = cgtp.csr_from_coo(N, i32([0, 5]), i32([2, 2]))
    g1 = cgtp.Graph(N, row_ptr, s)
    Y = dev(osh.real_sh(1, np.array([[0.1, 0.2, 0.3], [-0.5, 0.2, 0.1]])), "f32")
    w = torch.randn((2, L.w_numel), device="cuda")
    out = plan.conv_forward(g1, x, Y, w, 1.0)
    dx, _, _ = plan.conv_backward(g1, x, Y, w, 1.0, torch.randn((N, L.dim_out), device="cuda"))
    torch.cuda.synchronize()
    o = host(out)
    assert np.all(o[[0, 1, 3, 4, 5]] == 0.0) and np.abs(o[2]).max() > 0
    d = host(dx)
    assert np.all(d[[1, 2, 3, 4]] == 0.0) and np.abs(d[0]).max() > 0 and np.abs(d[5]).max() > 0


def test_determinism_and_equivariance():
    ix, iy, io = "16x0e+16x1o+16x2e", "0e+1o+2e", "0e+0o+1e+1o+2e+2o"
    L = Layout(ix, iy, io)
    plan = cgtp.Plan(ix, iy, io)
    pos = synth.uniform_box(150, 8.0, 5)
    case = Case(pos, 8.0, 2.5)
    x, Y, w, g = small_inputs(L, case, 5, "f32", 2)
    sc = 0.3
    a = [plan.conv_forward(case.graph, x, Y, w, sc)] + list(plan.conv_backward(case.graph, x, Y, w, sc, g))
    b = [plan.conv_forward(case.graph, x, Y, w, sc)] + list(plan.conv_backward(case.graph, x, Y, w, sc, g))
    for u, v in zip(a, b):
        assert torch.equal(u, v)
    # rotate the system: harmonics of rotated edge vectors, rotated x -> rotated output
    ang = wigner.random_euler(np.random.default_rng(0))
    R = wigner.euler_to_matrix(*ang)
    Yr = dev(osh.real_sh(2, case.vec @ R.T), "f32")
    hx = host(x)
    xr = hx.copy()
    for (mul, l, _), o in zip(L.X, L.x_off):
        D = wigner.wigner_D_real(l, *ang)
        blk = hx[:, o:o + mul * (2 * l + 1)].reshape(-1, 2 * l + 1, mul)
        xr[:, o:o + mul * (2 * l + 1)] = np.einsum("ab,zbu->zau", D, blk).reshape(case.N, -1)
    out_r = host(plan.conv_forward(case.graph, dev(xr, "f32"), Yr, w, sc))
    out = host(a[0])
    rot = out.copy()
    for p in L.paths:
        D = wigner.wigner_D_real(p["l3"], *ang)
        blk = L.out_block(out, p)
        L.out_block(rot, p)[...] = np.einsum("ab,zbu->zau", D, blk)
    assert rel_err(out_r, rot) < 1e-5


def workload(name, dtype, seed=0):
    """A full-size convolution workload on the device, as the benchmark builds it."""
    c = synth.CONFIGS[name]
    L = Layout(c["irreps_x"], c["irreps_y"], c["irreps_out"])
    case = Case(synth.positions_for(c, seed), c["box"], c["r_cut"])
    td = {"f32": torch.float32, "f64": torch.float64}[dtype]
    Y = dev(osh.real_sh(c["L"], case.vec), dtype)
    W1, W2 = synth.mlp_params(8, 64, L.w_numel, seed)
    W1 = torch.from_numpy(W1).to(td).cuda()
    W2 = torch.from_numpy(W2).to(td).cuda()
    r = torch.from_numpy(np.linalg.norm(case.vec, axis=1)).to(td).cuda()
    w = torch.empty((case.E, L.w_numel), dtype=td, device="cuda")
    for a in range(0, case.E, 1 << 19):
        w[a:a + (1 << 19)] = synth.radial_weights_torch(r[a:a + (1 << 19)], c["r_cut"], W1, W2)
    gen = torch.Generator(device="cuda")
    gen.manual_seed(seed)
    x = torch.randn((case.N, L.dim_x), generator=gen, device="cuda", dtype=td)
    return c, L, case, x, Y, w


def check_sampled(L, case, plan, x, Y, w, sc, dtype, backward, n_nodes=48):
    rng = np.random.default_rng(1)
    nodes = np.sort(rng.choice(case.N, n_nodes, replace=False))
    out = plan.conv_forward(case.graph, x, Y, w, sc)
    torch.cuda.synchronize()
    hx = host(x)
    # forward on sampled receivers: their CSR segments only
    segs = [np.arange(case.h_row[n], case.h_row[n + 1]) for n in nodes]
    sub_row = np.concatenate([[0], np.cumsum([len(s) for s in segs])])
    eidx = np.concatenate(segs)
    ei = torch.from_numpy(eidx).cuda()
    hY, hw = host(Y[ei]), host(w[ei])
    ref = oconv.forward(L, sub_row, case.h_src[eidx], hx, hY, hw, sc)
    assert_close(host(out[torch.from_numpy(nodes).cuda()]), ref, out_blocks(L), dtype, "sampled forward")
    del out
    if not backward:
        return
    gen = torch.Generator(device="cuda")
    gen.manual_seed(7)
    g = torch.randn((case.N, L.dim_out), generator=gen, device="cuda", dtype=x.dtype)
    dx, dY, dw = plan.conv_backward(case.graph, x, Y, w, sc, g)
    torch.cuda.synchronize()
    hg = host(g)
    # grad_sh and grad_w on the sampled receivers' edges
    _, rdY, rdw = otp.backward(L, hx[case.h_src[eidx]], hY, hw, sc * hg[case.h_dst[eidx]])
    assert_close(host(dY[ei]), rdY, y_blocks(L), dtype, "sampled grad_sh")
    assert_close(host(dw[ei]), rdw, w_blocks(L), dtype, "sampled grad_w")
    # grad_x on sampled senders: all their outgoing edges
    sidx = np.concatenate([case.eid[case.col_ptr[n]:case.col_ptr[n + 1]] for n in nodes])
    si = torch.from_numpy(sidx).cuda()
    rdxe, _, _ = otp.backward(L, hx[case.h_src[sidx]], host(Y[si]), host(w[si]), sc * hg[case.h_dst[sidx]])
    rdx = np.zeros((n_nodes, L.dim_x))
    pos_of = {n: k for k, n in enumerate(nodes)}
    for row, e in enumerate(sidx):
        rdx[pos_of[case.h_src[e]]] += rdxe[row]
    assert_close(host(dx[torch.from_numpy(nodes).cuda()]), rdx, x_blocks(L), dtype, "sampled grad_x")


def test_conv_water1k_full_size():
    c, L, case, x, Y, w = workload("conv_water1k", "f32")
    plan = cgtp.Plan(c["irreps_x"], c["irreps_y"], c["irreps_out"])
    check_sampled(L, case, plan, x, Y, w, 1.0 / math.sqrt(case.E / case.N), "f32", backward=True, n_nodes=300)


def test_conv_water8k_full_size():
    c, L, case, x, Y, w = workload("conv_water8k", "f32")
    plan = cgtp.Plan(c["irreps_x"], c["irreps_y"], c["irreps_out"])
    check_sampled(L, case, plan, x, Y, w, 1.0 / math.sqrt(case.E / case.N), "f32", backward=True)


def test_conv_uniform100k_full_size_f32():
    c, L, case, x, Y, w = workload("conv_uniform100k", "f32")
    plan = cgtp.Plan(c["irreps_x"], c["irreps_y"], c["irreps_out"])
    check_sampled(L, case, plan, x, Y, w, 1.0 / math.sqrt(case.E / case.N), "f32", backward=True)
    del x, Y, w
    torch.cuda.empty_cache()


def test_conv_uniform100k_full_size_f64_forward():
    c, L, case, x, Y, w = workload("conv_uniform100k", "f64")
    plan = cgtp.Plan(c["irreps_x"], c["irreps_y"], c["irreps_out"], dtype="f64")
    check_sampled(L, case, plan, x, Y, w, 1.0 / math.sqrt(case.E / case.N), "f64", backward=False)
    del x, Y, w
    torch.cuda.empty_cache()


def test_wide_channels_and_fallback_paths():
    """320 channels: the fused forward uses two channel chunks per receiver and the
    backward takes the row-parallel fallback (more than 64 lanes per edge)."""
    ix, iy, io = "320x0e+320x1o", "0e+1o+2e", "0e+1o+1e+2e"
    L = Layout(ix, iy, io)
    case = Case(synth.uniform_box(60, 6.0, 3), 6.0, 2.5)
    plan = cgtp.Plan(ix, iy, io)
    x, Y, w, g = small_inputs(L, case, 3, "f32", 2)
    sc = 0.21
    out = plan.conv_forward(case.graph, x, Y, w, sc)
    dx, dY, dw = plan.conv_backward(case.graph, x, Y, w, sc, g)
    torch.cuda.synchronize()
    hx, hY, hw, hg = host(x), host(Y), host(w), host(g)
    assert_close(host(out), oconv.forward(L, case.h_row, case.h_src, hx, hY, hw, sc), out_blocks(L), "f32", "fwd")
    rdx, rdY, rdw = oconv.backward(L, case.h_row, case.h_src, hx, hY, hw, sc, hg)
    assert_close(host(dx), rdx, x_blocks(L), "f32", "grad_x")
    assert_close(host(dY), rdY, y_blocks(L), "f32", "grad_sh")
    assert_close(host(dw), rdw, w_blocks(L), "f32", "grad_w")


def test_misaligned_tensors_take_general_kernels():
    ix, iy, io = "8x0e+8x1o+8x2e", "0e+1o+2e", "0e+0o+1e+1o+2e+2o"
    L = Layout(ix, iy, io)
    case = Case(synth.uniform_box(50, 6.0, 4), 6.0, 2.5)
    plan = cgtp.Plan(ix, iy, io)
    x, Y, w, g = small_inputs(L, case, 4, "f32", 2)
    wb = torch.empty(case.E * L.w_numel + 1, device="cuda")
    wv = wb[1:].view(case.E, L.w_numel)  # 4-byte offset
    wv.copy_(w)
    out = plan.conv_forward(case.graph, x, Y, wv, 1.0)
    dx, dY, dw = plan.conv_backward(case.graph, x, Y, wv, 1.0, g)
    torch.cuda.synchronize()
    hx, hY, hw, hg = host(x), host(Y), host(w), host(g)
    assert_close(host(out), oconv.forward(L, case.h_row, case.h_src, hx, hY, hw, 1.0), out_blocks(L), "f32", "fwd")
    rdx, rdY, rdw = oconv.backward(L, case.h_row, case.h_src, hx, hY, hw, 1.0, hg)
    assert_close(host(dx), rdx, x_blocks(L), "f32", "grad_x")
    assert_close(host(dw), rdw, w_blocks(L), "f32", "grad_w")


def test_conv_error_paths():
    ix, iy, io = "4x0e+4x1o", "0e+1o", "0e+1o+1e"
    L = Layout(ix, iy, io)
    case = Case(synth.uniform_box(30, 5.0, 5), 5.0, 2.0)
    shared = cgtp.Plan(ix, iy, io, wkind="shared")
    x = torch.zeros((case.N, L.dim_x), device="cuda")
    Y = torch.zeros((case.E, L.dim_y), device="cuda")
    w = torch.zeros((case.E, L.w_numel), device="cuda")
    with pytest.raises(cgtp.CgtpError) as e:
        shared.conv_forward(case.graph, x, Y, w, 1.0)
    assert e.value.status == 3
    plan = cgtp.Plan(ix, iy, io)
    small_ws = torch.empty(16, dtype=torch.uint8, device="cuda")
    with pytest.raises(cgtp.CgtpError) as e:
        plan.conv_backward(case.graph, x, Y, w, 1.0, torch.zeros((case.N, L.dim_out), device="cuda"), ws=small_ws)
    assert e.value.status == 5
    # the workspace size is the per-edge grad_x partials in the accumulation
    # type (256-byte aligned), then one grad_sh copy per x block
    nws = plan.workspace_size(cgtp.OP_CONV_BACKWARD, graph=case.graph)
    assert nws == -(-case.E * L.dim_x * 4 // 256) * 256 + 2 * case.E * L.dim_y * 4
    g = torch.zeros((case.N, L.dim_out), device="cuda")
    # a host workspace is refused before any launch; a workspace of another
    # dtype counts in bytes
    with pytest.raises(ValueError):
        plan.conv_backward(case.graph, x, Y, w, 1.0, g, ws=torch.empty(nws, dtype=torch.uint8))
    dx, _, _ = plan.conv_backward(case.graph, x, Y, w, 1.0, g,
                                  ws=torch.empty(nws // 4, dtype=torch.float32, device="cuda"))
    torch.cuda.synchronize()
    assert float(dx.abs().max()) == 0.0


def radial_chain(vec_d, r_cut, W1, W2, dw, chunk=1 << 18):
    """Caller-side radial network: d/dvec of sum(dw * w(|vec|)) by torch autograd."""
    out = torch.empty_like(vec_d)
    for a in range(0, vec_d.shape[0], chunk):
        v = vec_d[a:a + chunk].detach().requires_grad_(True)
        wv = synth.radial_weights_torch(v.norm(dim=1), r_cut, W1, W2)
        (gv,) = torch.autograd.grad(wv, v, dw[a:a + chunk])
        out[a:a + chunk] = gv
    return out


def force_chain_case(name, small=None, seed=0):
    """Harmonics from the edge vectors by the library, weights by the radial network,
    convolution forward and backward, then the edge-vector gradient."""
    if small is None:
        c = synth.CONFIGS[name]
        ix, iy, io, lmax, rc = c["irreps_x"], c["irreps_y"], c["irreps_out"], c["L"], c["r_cut"]
        case = Case(synth.positions_for(c, seed), c["box"], rc)
        hidden = 64
    else:
        (ix, iy, io, lmax), (n, box, rc) = small
        case = Case(synth.uniform_box(n, box, seed), box, rc)
        hidden = 16
    L = Layout(ix, iy, io)
    plan = cgtp.Plan(ix, iy, io)
    vec32 = case.vec.astype(np.float32)
    vd = torch.from_numpy(vec32).cuda()
    W1, W2 = synth.mlp_params(8, hidden, L.w_numel, seed)
    tW1, tW2 = torch.from_numpy(W1).float().cuda(), torch.from_numpy(W2).float().cuda()
    Y = cgtp.sh_forward(lmax, vd)
    w = torch.empty((case.E, L.w_numel), device="cuda")
    with torch.no_grad():
        for a in range(0, case.E, 1 << 19):
            w[a:a + (1 << 19)] = synth.radial_weights_torch(vd[a:a + (1 << 19)].norm(dim=1), rc, tW1, tW2)
    gen = torch.Generator(device="cuda")
    gen.manual_seed(seed)
    x = torch.randn((case.N, L.dim_x), generator=gen, device="cuda")
    g = torch.randn((case.N, L.dim_out), generator=gen, device="cuda")
    sc = oconv.avg_neighbors_scale(case.N, case.E)
    out = plan.conv_forward(case.graph, x, Y, w, sc)
    dx, dY, dw = plan.conv_backward(case.graph, x, Y, w, sc, g)
    gvec = cgtp.sh_backward(lmax, vd, dY) + radial_chain(vd, rc, tW1, tW2, dw)
    torch.cuda.synchronize()
    return L, case, lmax, rc, W1, W2, sc, vec32, x, w, g, out, dx, gvec


def oracle_force_chain(L, lmax, rc, W1, W2, vec, hw, hg_e, src_x):
    """Oracle side for a set of edges: harmonics from the vectors, TP backward,
    radial chain in fp64, then the edge-vector gradient."""
    hv = np.asarray(vec, np.float64)
    hY = osh.real_sh(lmax, hv)
    _, rdY, rdw = otp.backward(L, src_x, hY, hw, hg_e)
    gr = synth.radial_weights_backward_np(np.linalg.norm(hv, axis=1), rc, W1, W2, rdw)
    return hY, oconv.edge_vector_grad(lmax, hv, rdY, gr)


def test_force_chain_small_graph_full():
    small = (("4x0e+4x1o+4x2e", "0e+1o+2e", "0e+0o+1e+1o+2e+2o", 2), (40, 9.0, 3.2))
    L, case, lmax, rc, W1, W2, sc, vec32, x, w, g, out, dx, gvec = force_chain_case(None, small, seed=3)
    assert case.E > 100
    hx, hw, hg = host(x), host(w), host(g)
    hY, ref = oracle_force_chain(L, lmax, rc, W1, W2, vec32, hw, sc * hg[case.h_dst], hx[case.h_src])
    assert_close(host(out), oconv.forward(L, case.h_row, case.h_src, hx, hY, hw, sc), out_blocks(L), "f32",
                 "forward with library harmonics")
    rdx, _, _ = oconv.backward(L, case.h_row, case.h_src, hx, hY, hw, sc, hg)
    assert_close(host(dx), rdx, x_blocks(L), "f32", "grad_x")
    assert_close(host(gvec), ref, [(0, 3)], "f32", "edge-vector gradient")


def test_conv_water8k_forces_full_size():
    """The 8000-molecule water box with forces, at full size, on sampled receivers' edges."""
    L, case, lmax, rc, W1, W2, sc, vec32, x, w, g, out, dx, gvec = force_chain_case("conv_water8k")
    rng = np.random.default_rng(2)
    nodes = np.sort(rng.choice(case.N, 32, replace=False))
    eidx = np.concatenate([np.arange(case.h_row[n], case.h_row[n + 1]) for n in nodes])
    ei = torch.from_numpy(eidx).cuda()
    hx, hg = host(x), host(g)
    hY, ref = oracle_force_chain(L, lmax, rc, W1, W2, vec32[eidx], host(w[ei]),
                                 sc * hg[case.h_dst[eidx]], hx[case.h_src[eidx]])
    assert_close(host(gvec[ei]), ref, [(0, 3)], "f32", "sampled edge-vector gradient")
    sub_row = np.concatenate([[0], np.cumsum(case.h_row[nodes + 1] - case.h_row[nodes])])
    rout = oconv.forward(L, sub_row, case.h_src[eidx], hx, hY, host(w[ei]), sc)
    assert_close(host(out[torch.from_numpy(nodes).cuda()]), rout, out_blocks(L), "f32", "sampled forward")
    del w, out, dx, gvec
    torch.cuda.empty_cache()


@pytest.mark.parametrize("dtype", ["f32", "f64", "bf16"])
def test_conv_backward_blocks_side_by_side(dtype):
    """The x blocks' backward launches run side by side when the workspace holds
    a grad_sh copy per block; with room for the grad_x partials only they
    accumulate grad_sh in place in block order. Same sums in the same order:
    fp32 and fp64 results are bitwise equal; bf16 rounds grad_sh once instead
    of once per block (both within tolerance of the oracle)."""
    ix, iy, io = "8x0e+8x1o+8x2e", "0e+1o+2e+3o", "0e+0o+1e+1o+2e+2o+3e+3o"
    L = Layout(ix, iy, io)
    case = Case(synth.uniform_box(200, 8.0, 11), 8.0, 3.0)
    plan = cgtp.Plan(ix, iy, io, dtype=dtype, wkind="per_row")
    x, Y, w, g = small_inputs(L, case, 3, dtype, 3)
    es = 8 if dtype == "f64" else 4
    part = -(-case.E * L.dim_x * es // 256) * 256
    nws = plan.workspace_size(cgtp.OP_CONV_BACKWARD, graph=case.graph)
    assert nws == part + 3 * case.E * L.dim_y * es
    full = plan.conv_backward(case.graph, x, Y, w, 0.7, g)
    serial = plan.conv_backward(case.graph, x, Y, w, 0.7, g,
                                ws=torch.empty(part, dtype=torch.uint8, device="cuda"))
    # without grad_x and without a workspace the launches also run in place
    _, dy_nows, dw_nows = plan.conv_backward(case.graph, x, Y, w, 0.7, g, need=(False, True, True),
                                             ws=torch.empty(0, dtype=torch.uint8, device="cuda"))
    torch.cuda.synchronize()
    rdx, rdY, rdw = oconv.backward(L, case.h_row, case.h_src, host(x), host(Y), host(w), 0.7, host(g))
    for name, (a, b) in zip(("grad_x", "grad_sh", "grad_w"), zip(full, serial)):
        if dtype != "bf16" or name != "grad_sh":
            assert torch.equal(a, b), name
    assert torch.equal(serial[1], dy_nows) and torch.equal(serial[2], dw_nows)
    for res in (full, serial):
        assert_close(host(res[0]), rdx, x_blocks(L), dtype, "grad_x")
        assert_close(host(res[1]), rdY, y_blocks(L), dtype, "grad_sh")
        assert_close(host(res[2]), rdw, w_blocks(L), dtype, "grad_w")
