"""GPU parity of the convolution with the radial network's last layer joined
(cgtp_conv_forward_radial / cgtp_conv_backward_radial) against the oracle
(oracle/radial.py): w = h W2 formed inside the forward on the matrix cores.

Small radius graphs in full (several irreps, 16 to 128 channels, L = 2..4,
more edges per receiver than one 16-edge batch, a padding node, an empty edge
list), and the 8000-molecule water box at full size on sampled receivers and
senders, with h the hidden activations of the benchmark's radial network.
"""

import math

import numpy as np
import pytest

from oracle import radial as orad
from oracle import sh as osh
from oracle.irreps import Layout
from clebsch_gordan_tensor_amd import synth
from tests.gpu_util import assert_close, dev, host, out_blocks, w_blocks, x_blocks, y_blocks

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
if not torch.cuda.is_available():
    pytest.skip("no GPU", allow_module_level=True)
cgtp = pytest.importorskip("clebsch_gordan_tensor_amd.cgtp")

from tests.test_gpu_conv import Case  # noqa: E402


def hidden(vec, r_cut, H, seed):
    """Hidden activations of the benchmark's radial network (SiLU of the
    Bessel-envelope basis times W1) and its last layer W2."""
    W1, _ = synth.mlp_params(8, H, 4, seed)
    pre = synth.bessel_envelope(np.linalg.norm(vec, axis=1), r_cut) @ W1
    return pre / (1.0 + np.exp(-pre))


PLANS = [
    ("16x0e+16x1o+16x2e", "0e+1o+2e", "0e+0o+1e+1o+2e+2o", 2, 16),
    ("128x0e+128x1o", "0e+1o+2e+3o", "0e+0o+1e+1o+2e+2o+3e+3o", 3, 64),
    ("64x0e+64x1o+64x2e+64x3o+64x4e", "0e+1o+2e+3o+4e", "0e+1o+2e+3o+4e+0o+1e+2o+3e+4o", 4, 32),
    ("32x1o+64x2e", "0e+1o+2e", "0e+1o+2e+3o", 2, 8),
]


@pytest.mark.parametrize("ix,iy,io,lmax,H", PLANS)
def test_small_graph_full(ix, iy, io, lmax, H):
    L = Layout(ix, iy, io)
    case = Case(synth.uniform_box(40, 6.0, 21), 6.0, 2.9)
    assert case.E / case.N > 16  # receivers with more than one 16-edge batch
    plan = cgtp.Plan(ix, iy, io)
    x = dev(synth.gaussian((case.N, L.dim_x), 1, synth.S_X), "f32")
    Y = dev(osh.real_sh(lmax, case.vec), "f32")
    h = dev(hidden(case.vec, 2.9, H, 1), "f32")
    W2 = dev(synth.gaussian((H, L.w_numel), 1, synth.S_MLP2) / math.sqrt(H), "f32")
    g = dev(synth.gaussian((case.N, L.dim_out), 1, synth.S_G), "f32")
    sc = 0.27
    out = plan.conv_forward_radial(case.graph, x, Y, h, W2, sc)
    dx, dY, dh, dW2 = plan.conv_backward_radial(case.graph, x, Y, h, W2, sc, g)
    torch.cuda.synchronize()
    hx, hY, hh, hW2, hg = host(x), host(Y), host(h), host(W2), host(g)
    tag = "%s H=%d" % (ix, H)
    assert_close(host(out), orad.forward(L, case.h_row, case.h_src, hx, hY, hh, hW2, sc), out_blocks(L), "f32",
                 "radial forward " + tag)
    rdx, rdY, rdh, rdW2 = orad.backward(L, case.h_row, case.h_src, hx, hY, hh, hW2, sc, hg)
    assert_close(host(dx), rdx, x_blocks(L), "f32", "radial grad_x " + tag)
    assert_close(host(dY), rdY, y_blocks(L), "f32", "radial grad_sh " + tag)
    assert_close(host(dh), rdh, [(0, H)], "f32", "radial grad_h " + tag)
    assert_close(host(dW2).reshape(H, -1), rdW2, [(o, n) for o, n in w_blocks(L)], "f32", "radial grad_W2 " + tag)
    # bitwise repeatable
    again = plan.conv_forward_radial(case.graph, x, Y, h, W2, sc)
    torch.cuda.synchronize()
    assert torch.equal(again, out)


def test_padding_node_and_empty_edges():
    ix, iy, io = "32x0e+32x1o", "0e+1o+2e", "0e+1o+1e+2e"
    L = Layout(ix, iy, io)
    N0 = 30
    pos = synth.uniform_box(N0, 6.0, 22)
    src, dst, vec = synth.radius_graph(pos, 6.0, 2.5)
    npad = len(src) // 3
    src = np.concatenate([src, np.full(npad, N0)])
    dst = np.concatenate([dst, np.full(npad, N0)])
    vec = np.concatenate([vec, np.random.default_rng(0).standard_normal((npad, 3)) + 1.0])
    N = N0 + 1
    i32 = lambda a: torch.from_numpy(np.ascontiguousarray(a, np.int32)).cuda()
    row_ptr, s, perm = cgtp.csr_from_coo(N, i32(src), i32(dst))
    graph = cgtp.Graph(N, row_ptr, s, pad_node=N0)
    p = perm.cpu().numpy()
    plan = cgtp.Plan(ix, iy, io)
    H = 16
    x = dev(synth.gaussian((N, L.dim_x), 2, synth.S_X), "f32")
    Y = dev(osh.real_sh(2, vec[p]), "f32")
    h = dev(synth.gaussian((len(src), H), 2, synth.S_MLP1), "f32")
    W2 = dev(synth.gaussian((H, L.w_numel), 2, synth.S_MLP2) / 4.0, "f32")
    g = dev(synth.gaussian((N, L.dim_out), 2, synth.S_G), "f32")
    out = plan.conv_forward_radial(graph, x, Y, h, W2, 0.5)
    dx, dY, dh, dW2 = plan.conv_backward_radial(graph, x, Y, h, W2, 0.5, g)
    torch.cuda.synchronize()
    hr = row_ptr.cpu().numpy()
    hs = s.cpu().numpy()
    args = (L, hr, hs, host(x), host(Y), host(h), host(W2), 0.5)
    assert_close(host(out), orad.forward(*args, pad_node=N0), out_blocks(L), "f32", "padded radial forward")
    rdx, rdY, rdh, rdW2 = orad.backward(*args, host(g), pad_node=N0)
    assert_close(host(dx), rdx, x_blocks(L), "f32", "padded grad_x")
    assert_close(host(dh), rdh, [(0, H)], "f32", "padded grad_h")
    assert_close(host(dW2), rdW2, [(0, L.w_numel)], "f32", "padded grad_W2")
    # no edges at all: zero output, zero grad_x and grad_W2
    g0 = cgtp.Graph(N, i32(np.zeros(N + 1)), i32(np.zeros(0)))
    e = lambda *shape: torch.zeros(shape, device="cuda")
    out0 = torch.full((N, L.dim_out), 3.0, device="cuda")
    plan.conv_forward_radial(g0, x, e(0, L.dim_y), e(0, H), W2, 1.0, out=out0)
    d0 = plan.conv_backward_radial(g0, x, e(0, L.dim_y), e(0, H), W2, 1.0, g)
    torch.cuda.synchronize()
    assert float(out0.abs().max()) == 0.0 and float(d0[0].abs().max()) == 0.0 and float(d0[3].abs().max()) == 0.0


def test_water8k_full_size_sampled():
    """The 8000-molecule water box (128x(0e+1o+2e), L = 3, 24 paths) with the
    benchmark's radial network's hidden layer (64 wide) at full size."""
    c = synth.CONFIGS["conv_water8k"]
    L = Layout(c["irreps_x"], c["irreps_y"], c["irreps_out"])
    case = Case(synth.positions_for(c, 0), c["box"], c["r_cut"])
    plan = cgtp.Plan(c["irreps_x"], c["irreps_y"], c["irreps_out"])
    Y = dev(osh.real_sh(3, case.vec), "f32")
    W1, W2 = synth.mlp_params(8, 64, L.w_numel, 0)
    r = torch.from_numpy(np.linalg.norm(case.vec, axis=1)).float().cuda()
    W1d, eye = torch.from_numpy(W1).float().cuda(), torch.eye(64, device="cuda")
    h = torch.empty((case.E, 64), device="cuda")
    for a in range(0, case.E, 1 << 19):  # the network up to its hidden layer (last layer = identity)
        h[a:a + (1 << 19)] = synth.radial_weights_torch(r[a:a + (1 << 19)], c["r_cut"], W1d, eye)
    W2d = torch.from_numpy(W2).float().cuda()
    gen = torch.Generator(device="cuda")
    gen.manual_seed(0)
    x = torch.randn((case.N, L.dim_x), generator=gen, device="cuda")
    sc = 1.0 / math.sqrt(case.E / case.N)
    out = plan.conv_forward_radial(case.graph, x, Y, h, W2d, sc)
    torch.cuda.synchronize()
    nodes = np.sort(np.random.default_rng(1).choice(case.N, 32, replace=False))
    segs = [np.arange(case.h_row[n], case.h_row[n + 1]) for n in nodes]
    sub_row = np.concatenate([[0], np.cumsum([len(s) for s in segs])])
    eidx = np.concatenate(segs)
    ei = torch.from_numpy(eidx).cuda()
    ref = orad.forward(L, sub_row, case.h_src[eidx], host(x), host(Y[ei]), host(h[ei]), host(W2d), sc)
    assert_close(host(out[torch.from_numpy(nodes).cuda()]), ref, out_blocks(L), "f32", "water8k radial forward")
    del out
    gen.manual_seed(7)
    g = torch.randn((case.N, L.dim_out), generator=gen, device="cuda")
    dx, dY, dh, dW2 = plan.conv_backward_radial(case.graph, x, Y, h, W2d, sc, g)
    torch.cuda.synchronize()
    hg, hx = host(g), host(x)
    w_e = host(h[ei]) @ host(W2d)
    from oracle import tp as otp
    _, rdY, rdw = otp.backward(L, hx[case.h_src[eidx]], host(Y[ei]), w_e, sc * hg[case.h_dst[eidx]])
    assert_close(host(dY[ei]), rdY, y_blocks(L), "f32", "water8k radial grad_sh")
    assert_close(host(dh[ei]), rdw @ host(W2d).T, [(0, 64)], "f32", "water8k radial grad_h")


@pytest.mark.parametrize("ix,iy,io", [
    ("256x0e+256x1o", "0e+1o+2e", "0e+1o+2e"),                # chunks of 1-2 slots: tiles fit the LDS
    ("256x1o", "0e+1o+2e", "0e+0o+1e+1o+2e+2o"),              # a chunk of several slots may exceed it
])
def test_256_channel_blocks(ix, iy, io):
    """Blocks of 256 channels: either parity with the oracle or a clean
    UNSUPPORTED when a slot chunk's two weight tiles and partial sums exceed the
    device's LDS (the call then writes nothing and raises)."""
    L = Layout(ix, iy, io)
    case = Case(synth.uniform_box(24, 5.0, 23), 5.0, 2.4)
    plan = cgtp.Plan(ix, iy, io)
    H = 64
    x = dev(synth.gaussian((case.N, L.dim_x), 3, synth.S_X), "f32")
    Y = dev(osh.real_sh(2, case.vec), "f32")
    h = dev(synth.gaussian((case.E, H), 3, synth.S_MLP1), "f32")
    W2 = dev(synth.gaussian((H, L.w_numel), 3, synth.S_MLP2) / 8.0, "f32")
    try:
        out = plan.conv_forward_radial(case.graph, x, Y, h, W2, 0.5)
    except cgtp.CgtpError as e:
        assert e.status == 3 and "LDS" in str(e)  # CGTP_ERR_UNSUPPORTED
        return
    torch.cuda.synchronize()
    ref = orad.forward(L, case.h_row, case.h_src, host(x), host(Y), host(h), host(W2), 0.5)
    assert_close(host(out), ref, out_blocks(L), "f32", "radial forward, 256 channels " + ix)
