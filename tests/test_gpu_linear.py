"""GPU parity of the equivariant linear map (MFMA kernels) against the oracle.

Full comparisons on small and ragged shapes (rows not a multiple of the
64-row tile, channel counts not multiples of 16, several row chunks for
grad_W, unreached output blocks), fp32 and bf16; B = 0; bitwise determinism;
the fully connected ("uvw") tensor product as the linear map after the
unit-weight uvu product; and, at the full size of the tensor-product workload
(2^20 rows of 128x(0e+1o+2e+3o)), sampled rows of the forward and grad_x
against the oracle plus the adjoint identities <g, f(x, W)> = <grad_x, x> =
<grad_W, W> for grad_W.
"""

import numpy as np
import pytest

from oracle import linear as olin
from oracle import tp as otp
from oracle.irreps import Layout
from clebsch_gordan_tensor_amd import synth
from tests.gpu_util import TOL, assert_close, dev, host

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
if not torch.cuda.is_available():
    pytest.skip("no GPU", allow_module_level=True)
cgtp = pytest.importorskip("clebsch_gordan_tensor_amd.cgtp")


def in_blocks(LL):
    return [(o, mul * (2 * l + 1)) for (mul, l, _), o in zip(LL.I, LL.in_off)]


def out_blocks(LL):
    return [(o, mul * (2 * l + 1)) for (mul, l, _), o in zip(LL.O, LL.out_off)]


def w_blocks(LL):
    return [(p["w_off"], p["mu"] * p["mv"]) for p in LL.paths]


CASES = [
    ("2x1o+3x1o+1x0e+2x2e", "4x1o+2x0e+1x2o+3x2e", 1000),      # mixing, unreached block, ragged rows
    ("16x0e+16x1o", "32x0e+8x1o", 64),
    ("5x1o+17x0e", "3x1o+19x0e+2x1o", 130),                   # channels not multiples of 16
    ("160x0e+32x2e", "144x0e+40x2e", 200),                    # more than 128 columns: column runs
    ("128x0e+128x1o+128x2e+128x3o", "128x0e+128x1o+128x2e+128x3o", 3000),
    ("8x0e+8x1o", "8x0e+8x1o", 5000),                         # several grad_W row chunks
]


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("ii,io,B", CASES)
def test_linear_full(ii, io, B, dtype):
    LL = olin.LinearLayout(ii, io)
    lin = cgtp.Linear(ii, io, dtype=dtype)
    x = dev(synth.gaussian((B, LL.dim_in), 1, synth.S_X), dtype)
    w = dev(synth.gaussian((LL.w_numel,), 1, synth.S_W), dtype)
    g = dev(synth.gaussian((B, LL.dim_out), 1, synth.S_G), dtype)
    out = lin.forward(x, w)
    dx, dw = lin.backward(x, w, g)
    torch.cuda.synchronize()
    hx, hw, hg = host(x), host(w), host(g)
    assert_close(host(out), olin.forward(LL, hx, hw), out_blocks(LL), dtype, "forward")
    rdx, rdw = olin.backward(LL, hx, hw, hg)
    assert_close(host(dx), rdx, in_blocks(LL), dtype, "grad_x")
    assert_close(host(dw)[None], rdw[None], w_blocks(LL), dtype, "grad_w")


def test_linear_empty_and_determinism():
    lin = cgtp.Linear("8x0e+8x1o", "4x0e+4x1o")
    x = torch.empty((0, lin.dim_in), device="cuda")
    w = torch.randn(lin.w_numel, device="cuda")
    g = torch.empty((0, lin.dim_out), device="cuda")
    assert lin.forward(x, w).shape == (0, lin.dim_out)
    dx, dw = lin.backward(x, w, g)
    torch.cuda.synchronize()
    assert dx.shape == (0, lin.dim_in) and torch.all(dw == 0)
    gen = torch.Generator(device="cuda")
    gen.manual_seed(3)
    x = torch.randn((9000, lin.dim_in), generator=gen, device="cuda")
    g = torch.randn((9000, lin.dim_out), generator=gen, device="cuda")
    a = [lin.forward(x, w), *lin.backward(x, w, g)]
    b = [lin.forward(x, w), *lin.backward(x, w, g)]
    for u, v in zip(a, b):
        assert torch.equal(u, v)


def test_fully_connected_tp_on_the_device():
    """uvw with y of multiplicity 1 = linear map after the unit-weight uvu product."""
    ix, iy, io = "16x0e+16x1o", "0e+1o+2e", "8x0e+8x1o+8x1e+8x2e"
    L = Layout(ix, iy, "0e+0o+1e+1o+2e+2o+3e+3o")
    B = 700
    plan = cgtp.Plan(ix, iy, "0e+0o+1e+1o+2e+2o+3e+3o", wkind="shared")
    t_irreps = "+".join("%dx%d%s" % (p["mul"], p["l3"], "e" if p["p3"] > 0 else "o") for p in L.paths)
    lin = cgtp.Linear(t_irreps, io)
    LL = olin.LinearLayout(t_irreps, io)
    x = dev(synth.gaussian((B, L.dim_x), 2, synth.S_X), "f32")
    y = dev(synth.gaussian((B, L.dim_y), 2, synth.S_Y), "f32")
    W = dev(synth.gaussian((LL.w_numel,), 2, synth.S_W), "f32")
    t = plan.tp_forward(x, y, torch.ones(L.w_numel, device="cuda"))
    out = lin.forward(t, W)
    torch.cuda.synchronize()
    ref = olin.forward(LL, otp.forward(L, host(x), host(y), np.ones(L.w_numel)), host(W))
    assert_close(host(out), ref, out_blocks(LL), "f32", "uvw forward")


def test_linear_full_size_tp_shapes():
    irreps = "128x0e+128x1o+128x2e+128x3o"
    LL = olin.LinearLayout(irreps, irreps)
    lin = cgtp.Linear(irreps, irreps)
    B = 1 << 20
    gen = torch.Generator(device="cuda")
    gen.manual_seed(0)
    x = torch.randn((B, LL.dim_in), generator=gen, device="cuda")
    w = torch.randn(LL.w_numel, generator=gen, device="cuda") / np.sqrt(128.0)
    g = torch.randn((B, LL.dim_out), generator=gen, device="cuda")
    out = lin.forward(x, w)
    dx, dw = lin.backward(x, w, g)
    torch.cuda.synchronize()
    rows = torch.from_numpy(np.sort(np.random.default_rng(5).choice(B, 64, replace=False))).cuda()
    hx, hw = host(x[rows]), host(w)
    assert_close(host(out[rows]), olin.forward(LL, hx, hw), out_blocks(LL), "f32", "sampled forward")
    rdx, _ = olin.backward(LL, hx, hw, host(g[rows]))
    assert_close(host(dx[rows]), rdx, in_blocks(LL), "f32", "sampled grad_x")
    # grad_w through the adjoint identities (fp64 inner products of the device results)
    f = torch.sum(g.double() * out.double()).item()
    fx = torch.sum(dx.double() * x.double()).item()
    fw = torch.sum(dw.double() * w.double()).item()
    scale = torch.sum((g.double() * out.double()).abs()).item()
    assert abs(fx - f) <= TOL["f32"] * scale and abs(fw - f) <= TOL["f32"] * scale
    del x, g, out, dx
    torch.cuda.empty_cache()
