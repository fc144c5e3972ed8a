"""GPU parity of the connection modes against the oracle (oracle/modes.py).

* uvw (fully connected, shared weights [u][w] per path): the fused forward
  (CG path outputs on the vector ALUs into LDS, channel mixing on the matrix
  cores) and the composed backward, fp32 and bf16, with and without collapsed
  outputs, path selections, ragged batches, output multiplicities other than
  x's, more than 128 output channels (two column tiles) and more than 128 x
  channels (two LDS chunks); the tp_large irreps with every output at 128
  channels, at full size on sampled rows (the benchmark's shape).
* uvu with y of multiplicity v > 1 (weights [u][v] per path), shared and per
  row, fp32 / fp64 / bf16.
"""

import numpy as np
import pytest

from oracle import modes
from oracle import sh as osh
from clebsch_gordan_tensor_amd import synth
from tests.gpu_util import assert_close, dev, host

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
if not torch.cuda.is_available():
    pytest.skip("no GPU", allow_module_level=True)
cgtp = pytest.importorskip("clebsch_gordan_tensor_amd.cgtp")


def out_blocks(ML):
    return [(g["out_off"], g["mul"] * (2 * g["l3"] + 1)) for g in ML.groups]


def x_blocks(ML):
    return [(o, mul * (2 * l + 1)) for (mul, l, _), o in zip(ML.X, ML.x_off)]


def y_blocks(ML):
    return [(o, v * (2 * l + 1)) for (v, l, _), o in zip(ML.Y, ML.y_off)]


def w_blocks(ML):
    return [(p["w_off"], p["w_len"]) for p in ML.paths]


def run(ix, iy, io, mode, B, dtype, wkind, collapse=False, select="all", seed=0, wscale=1.0):
    ML = modes.ModeLayout(ix, iy, io, mode, select, collapse)
    plan = cgtp.Plan(ix, iy, io, mode=mode, dtype=dtype, wkind=wkind, select=select, collapse=collapse)
    assert (plan.dim_out, plan.w_numel) == (ML.dim_out, ML.w_numel)
    shared = wkind == "shared"
    x = dev(synth.gaussian((B, ML.dim_x), seed, synth.S_X), dtype)
    y = dev(synth.gaussian((B, ML.dim_y), seed, synth.S_Y), dtype)
    w = dev(wscale * synth.gaussian((ML.w_numel,) if shared else (B, ML.w_numel), seed, synth.S_W), dtype)
    g = dev(synth.gaussian((B, ML.dim_out), seed, synth.S_G), dtype)
    tag = "%s %s | %s -> %s B=%d %s %s collapse=%s" % (mode, ix, iy, io, B, dtype, wkind, collapse)
    print(tag, flush=True)
    out = plan.tp_forward(x, y, w)
    torch.cuda.synchronize()
    hx, hy, hw, hg = host(x), host(y), host(w), host(g)
    assert_close(host(out), modes.forward(ML, hx, hy, hw), out_blocks(ML), dtype, "forward " + tag)
    dx, dy, dw = plan.tp_backward(x, y, w, g)
    torch.cuda.synchronize()
    rdx, rdy, rdw = modes.backward(ML, hx, hy, hw, hg)
    assert_close(host(dx), rdx, x_blocks(ML), dtype, "grad_x " + tag)
    assert_close(host(dy), rdy, y_blocks(ML), dtype, "grad_y " + tag)
    assert_close(host(dw), rdw, w_blocks(ML), dtype, "grad_w " + tag)
    return plan, (x, y, w, g), out


UVW = [
    ("8x0e+8x1o+8x2e", "0e+1o+2e", "8x0e+8x0o+8x1e+8x1o+8x2e+8x2o"),
    ("4x0e+12x1o+8x2e", "0e+1o+2e", "16x0e+4x0o+12x1e+8x1o+20x2e+4x2o+8x3e"),   # w != u
    ("32x0e+32x1o+32x2e+32x3o+32x4e", "0e+1o+2e+3o+4e", "12x0e+8x1o+16x2e+4x3o+8x4e"),  # L = 4
    ("16x0e+16x1o", "0e+1o", "160x0e+136x1o+144x1e"),                          # two output column tiles
    ("200x0e+132x1o", "0e+1o", "8x0e+16x1o+12x1e"),                            # two x-channel chunks
]


@pytest.mark.parametrize("collapse", [False, True])
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("ix,iy,io", UVW)
def test_uvw(ix, iy, io, dtype, collapse):
    run(ix, iy, io, "uvw", 37, dtype, "shared", collapse=collapse, wscale=0.3)


@pytest.mark.parametrize("select", ["symmetric", "skew"])
def test_uvw_selected_paths(select):
    run("8x0e+8x1o+8x2e", "0e+1o+2e", "8x0e+8x0o+8x1e+8x1o+8x2e+8x2o", "uvw", 300, "f32", "shared",
        collapse=True, select=select)


def test_uvw_harmonics_ragged_and_deterministic():
    ix, iy, io = "16x0e+16x1o+16x2e", "0e+1o+2e", "16x0e+16x0o+16x1e+16x1o+16x2e+16x2o"
    plan, (x, y, w, g), out = run(ix, iy, io, "uvw", 1000 + 9, "f32", "shared", collapse=True)
    y2 = dev(osh.real_sh(2, synth.unit_vectors(x.shape[0], 3)), "f32")
    a = [plan.tp_forward(x, y2, w)] + list(plan.tp_backward(x, y2, w, g))
    b = [plan.tp_forward(x, y2, w)] + list(plan.tp_backward(x, y2, w, g))
    torch.cuda.synchronize()
    for u, v in zip(a, b):
        assert torch.equal(u, v)
    e = plan.tp_forward(x[:0], y2[:0], w)
    ex, ey, ew = plan.tp_backward(x[:0], y2[:0], w, g[:0])
    torch.cuda.synchronize()
    assert e.shape[0] == 0 and float(ew.abs().max()) == 0.0


@pytest.mark.parametrize("collapse", [False, True])
def test_uvw_tp_large_full_size_sampled(collapse):
    """2^20 rows of 128x(0e+1o+2e+3o) with harmonics L = 3, every output type at
    128 channels, shared 128 x 128 weights per path, on sampled rows."""
    c = synth.CONFIGS["tp_large"]
    ix, iy = c["irreps_x"], c["irreps_y"]
    io = "+".join("128x%d%s" % (l, p) for l in range(4) for p in "eo")
    ML = modes.ModeLayout(ix, iy, io, "uvw", "all", collapse)
    plan = cgtp.Plan(ix, iy, io, mode="uvw", wkind="shared", collapse=collapse)
    B = c["B"]
    gen = torch.Generator(device="cuda")
    gen.manual_seed(0)
    x = torch.randn((B, ML.dim_x), generator=gen, device="cuda")
    y = dev(osh.real_sh(3, synth.unit_vectors(B, 0)), "f32")
    w = torch.randn((ML.w_numel,), generator=gen, device="cuda") / 16.0
    out = plan.tp_forward(x, y, w)
    torch.cuda.synchronize()
    rows = np.sort(np.random.default_rng(1).choice(B, 16, replace=False))  # the oracle takes ~0.6 s a row
    rows[-1] = B - 1
    ri = torch.from_numpy(rows).cuda()
    assert_close(host(out[ri]), modes.forward(ML, host(x[ri]), host(y[ri]), host(w)), out_blocks(ML), "f32",
                 "full-size uvw forward")


@pytest.mark.parametrize("wkind", ["per_row", "shared"])
@pytest.mark.parametrize("dtype", ["f32", "f64", "bf16"])
def test_uvu_y_multiplicity(dtype, wkind):
    run("6x0e+6x1o+4x2e", "3x0e+2x1o+2x2e", "0e+0o+1e+1o+2e+2o", "uvu", 301, dtype, wkind, seed=2)


def test_uvu_y_multiplicity_l4_and_unread_block():
    # the 5x3e block reaches no output here (3e x 0e -> 3e, 3e x 1o -> 2o, 3o, 4o): zero gradient
    run("8x1o+5x3e+4x4e", "4x0e+3x1o", "0e+1e+1o+4e", "uvu", 257, "f32", "per_row", seed=3)
