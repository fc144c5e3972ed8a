"""GPU parity of the uvu tensor product (forward and backward) against the oracle.

Every call goes through the C ABI (ctypes binding). Sizes span several
workgroups and a ragged tail; the full-size tp_large case is checked on
sampled rows in the launch configuration the benchmark times.
"""

import numpy as np
import pytest

from oracle import sh as osh
from oracle import tp as otp
from oracle.irreps import Layout
from clebsch_gordan_tensor_amd import synth
from tests.gpu_util import (TOL, assert_close, dev, host, out_blocks, rel_err, torch_dtype, w_blocks,
                            x_blocks, y_blocks)

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
if not torch.cuda.is_available():
    pytest.skip("no GPU", allow_module_level=True)
cgtp = pytest.importorskip("clebsch_gordan_tensor_amd.cgtp")


def host_inputs(L, B, seed, shared, dtype):
    x = synth.gaussian((B, L.dim_x), seed, synth.S_X)
    y = osh.real_sh(max(l for _, l, _ in L.Y), synth.unit_vectors(B, seed))
    if y.shape[1] != L.dim_y:  # y irreps that are not SH(0..L): plain Gaussian rows
        y = synth.gaussian((B, L.dim_y), seed, synth.S_Y)
    w = synth.gaussian((L.w_numel,) if shared else (B, L.w_numel), seed, synth.S_W)
    g = synth.gaussian((B, L.dim_out), seed, synth.S_G)
    d = [dev(a, dtype) for a in (x, y, w, g)]
    h = [host(t) for t in d]  # the exact device values
    return d, h


def run_case(ix, iy, io, B, dtype, shared, seed=0, check_bwd=True):
    L = Layout(ix, iy, io)
    plan = cgtp.Plan(ix, iy, io, dtype=dtype, wkind="shared" if shared else "per_row")
    (x, y, w, g), (hx, hy, hw, hg) = host_inputs(L, B, seed, shared, dtype)
    out = plan.tp_forward(x, y, w)
    torch.cuda.synchronize()
    ref = otp.forward(L, hx, hy, hw)
    e = assert_close(host(out), ref, out_blocks(L), dtype, "forward %s B=%d %s" % (ix, B, dtype))
    if not check_bwd:
        return e
    dx, dy, dw = plan.tp_backward(x, y, w, g)
    torch.cuda.synchronize()
    rdx, rdy, rdw = otp.backward(L, hx, hy, hw, hg)
    assert_close(host(dx), rdx, x_blocks(L), dtype, "grad_x")
    assert_close(host(dy), rdy, y_blocks(L), dtype, "grad_y")
    assert_close(host(dw), rdw, w_blocks(L), dtype, "grad_w")
    return e


def test_tp_small_full():
    """tp_small workload (32x(0e+1o+2e), SH L=2, 15 paths, shared weights, 4096 rows, fp32)."""
    c = synth.CONFIGS["tp_small"]
    run_case(c["irreps_x"], c["irreps_y"], c["irreps_out"], c["B"], "f32", shared=True)


@pytest.mark.parametrize("dtype", ["f32", "bf16", "f64"])
def test_tp_large_shape_ragged(dtype):
    """tp_large irreps (34 paths, per-row weights) at a ragged batch."""
    c = synth.CONFIGS["tp_large"]
    run_case(c["irreps_x"], c["irreps_y"], c["irreps_out"], 1037, dtype, shared=False)


@pytest.mark.parametrize("dtype", ["f32", "f64"])
def test_lmax4_all_paths(dtype):
    c = synth.CONFIGS["conv_uniform100k"]
    run_case(c["irreps_x"], c["irreps_y"], c["irreps_out"], 300, dtype, shared=False)


@pytest.mark.parametrize("ix,iy,io", [
    ("8x1o+4x0e+3x2o", "1o+0e", "0e+1o+2e"),           # mixed multiplicities: one channel per lane
    ("5x2e", "1o+1e", "1e+1o+2e+3o+3e"),               # repeated degree in y
    ("2x1o", "2e", "1o+3o+2e"),
    ("512x0e+264x1o", "0e+1o", "0e+1o+1e"),            # more channel groups than lanes
    ("4x4e+4x3o", "4e+3o+2e", "0e+1o+2e+3o+4e+1e+2o+3e+4o"),
])
@pytest.mark.parametrize("shared", [False, True])
def test_irregular_plans(ix, iy, io, shared):
    run_case(ix, iy, io, 77, "f32", shared=shared)


@pytest.mark.parametrize("dtype", ["f32", "bf16", "f64"])
@pytest.mark.parametrize("ix,iy,io", [
    ("8x3o+8x1e", "0e+1o+2e", "0e+1o+1e+2e+2o"),  # an x degree above the largest y/output degree
    ("16x0e+16x1o", "0e+1o", "0e+1o+1e"),           # x degrees within it
])
def test_backward_x_degree_bound(ix, iy, io, dtype):
    """The one-launch backward is compiled for x degrees up to the plan's largest
    y/output degree when no x block goes beyond it, and for every degree
    otherwise: both kinds, in every storage type, with vectorised channels."""
    run_case(ix, iy, io, 133, dtype, shared=False)


def test_empty_and_single_row():
    c = synth.CONFIGS["tp_large"]
    plan = cgtp.Plan(c["irreps_x"], c["irreps_y"], c["irreps_out"])
    z = torch.zeros((0, plan.dim_x), device="cuda")
    out = plan.tp_forward(z, torch.zeros((0, plan.dim_y), device="cuda"),
                          torch.zeros((0, plan.w_numel), device="cuda"))
    assert out.shape == (0, plan.dim_out)
    run_case(c["irreps_x"], c["irreps_y"], c["irreps_out"], 1, "f32", shared=False)
    ps = cgtp.Plan(c["irreps_x"], c["irreps_y"], c["irreps_out"], wkind="shared")
    dw = torch.full((ps.w_numel,), 7.0, device="cuda")
    ps.tp_backward(z, torch.zeros((0, ps.dim_y), device="cuda"), torch.zeros(ps.w_numel, device="cuda"),
                   torch.zeros((0, ps.dim_out), device="cuda"), need=(False, False, True), out=(None, None, dw))
    torch.cuda.synchronize()
    assert float(dw.abs().max()) == 0.0


def test_misaligned_views_use_scalar_path():
    c = synth.CONFIGS["tp_small"]
    L = Layout(c["irreps_x"], c["irreps_y"], c["irreps_out"])
    plan = cgtp.Plan(c["irreps_x"], c["irreps_y"], c["irreps_out"])
    (x, y, w, g), (hx, hy, hw, hg) = host_inputs(L, 50, 3, False, "f32")
    xb = torch.empty(50 * L.dim_x + 1, device="cuda")
    xv = xb[1:].view(50, L.dim_x)  # 4-byte offset: not 16-byte aligned
    xv.copy_(x)
    out = plan.tp_forward(xv, y, w)
    torch.cuda.synchronize()
    assert_close(host(out), otp.forward(L, hx, hy, hw), out_blocks(L), "f32", "misaligned forward")


def test_determinism_bitwise():
    c = synth.CONFIGS["tp_small"]
    L = Layout(c["irreps_x"], c["irreps_y"], c["irreps_out"])
    plan = cgtp.Plan(c["irreps_x"], c["irreps_y"], c["irreps_out"], wkind="shared")
    (x, y, w, g), _ = host_inputs(L, 4096, 1, True, "f32")
    a = [t.clone() for t in (plan.tp_forward(x, y, w),) + plan.tp_backward(x, y, w, g)]
    b = [t.clone() for t in (plan.tp_forward(x, y, w),) + plan.tp_backward(x, y, w, g)]
    for u, v in zip(a, b):
        assert torch.equal(u, v)


def test_tp_large_full_size_sampled():
    """tp_large at its full batch (1,048,576 rows, fp32) in the benchmark's launch
    configuration; 512 sampled rows checked against the oracle."""
    c = synth.CONFIGS["tp_large"]
    L = Layout(c["irreps_x"], c["irreps_y"], c["irreps_out"])
    plan = cgtp.Plan(c["irreps_x"], c["irreps_y"], c["irreps_out"])
    B = c["B"]
    gen = torch.Generator(device="cuda")
    gen.manual_seed(0)
    x = torch.randn((B, L.dim_x), generator=gen, device="cuda")
    w = torch.randn((B, L.w_numel), generator=gen, device="cuda")
    y = dev(osh.real_sh(3, synth.unit_vectors(B, 0)), "f32")
    out = plan.tp_forward(x, y, w)
    rows = np.sort(np.random.default_rng(0).choice(B, 512, replace=False))
    rows[-1] = B - 1
    ri = torch.from_numpy(rows).cuda()
    hx, hy, hw = host(x[ri]), host(y[ri]), host(w[ri])
    assert_close(host(out[ri]), otp.forward(L, hx, hy, hw), out_blocks(L), "f32", "full-size forward")
    del out
    g = torch.randn((B, L.dim_out), generator=gen, device="cuda")
    dx, dy, dw = plan.tp_backward(x, y, w, g)
    rdx, rdy, rdw = otp.backward(L, hx, hy, hw, host(g[ri]))
    assert_close(host(dx[ri]), rdx, x_blocks(L), "f32", "full-size grad_x")
    assert_close(host(dy[ri]), rdy, y_blocks(L), "f32", "full-size grad_y")
    assert_close(host(dw[ri]), rdw, w_blocks(L), "f32", "full-size grad_w")
    del x, y, w, g, dx, dy, dw
    torch.cuda.empty_cache()


def test_many_repeated_y_blocks_lds_limit():
    """130 harmonic components (y blocks repeated): the backward's per-lane grad_y
    columns take 130 KB of LDS in fp32, so the vectorised kernels (plus grad_x
    rows) would exceed the device limit and the one-channel kernel runs; in fp64
    the columns alone exceed it and the call is refused, not launched."""
    props = torch.cuda.get_device_properties(0)
    print("LDS per workgroup reported by the device:", getattr(props, "shared_memory_per_block", "n/a"), flush=True)
    ix, iy, io = "8x0e+8x4e", "+".join(["0e+1o+2e+3o+4e"] * 5 + ["0e"] * 5), "0e+4e"
    run_case(ix, iy, io, 300, "f32", shared=False)
    L = Layout(ix, iy, io)
    assert L.dim_y == 130
    plan = cgtp.Plan(ix, iy, io, dtype="f64")
    (x, y, w, g), _ = host_inputs(L, 64, 1, False, "f64")
    with pytest.raises(cgtp.CgtpError) as e:
        plan.tp_backward(x, y, w, g)
    assert e.value.status == 3
