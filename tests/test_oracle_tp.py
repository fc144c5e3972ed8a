"""Pins of the oracle's uvu tensor product (CPU only).

Sparse loops vs a dense einsum ([COURSE] 03b), bilinearity, O(3) equivariance
with the parity rule p3 = p1 p2 ([COURSE] 03a), l = 0 paths as channel scaling,
1 x 1 against dot/cross products, the adjoint identities of the trilinear form
<g, TP(x, y, w)> ([E3J] E.1) and central finite differences.
"""

import math

import numpy as np
import pytest

from oracle import sh, tp, wigner
from oracle.irreps import Layout, parse_irreps, paths_uvu
from clebsch_gordan_tensor_amd import synth


def make_inputs(L, B, seed, shared=False):
    x = synth.gaussian((B, L.dim_x), seed, synth.S_X)
    y = synth.gaussian((B, L.dim_y), seed, synth.S_Y)
    w = synth.gaussian((L.w_numel,) if shared else (B, L.w_numel), seed, synth.S_W)
    return x, y, w


def test_parse_irreps():
    assert parse_irreps(" 16x0e + 8x1o+2e ") == [(16, 0, 1), (8, 1, -1), (1, 2, 1)]
    assert parse_irreps("") == []
    for bad in ["3x", "x1e", "1q", "0x1e", "1e++2o"]:
        with pytest.raises(ValueError):
            parse_irreps(bad)


def test_path_counts_of_the_workloads():
    # All (l3, p) with l3 <= L are allowed; counts follow from the triangle rule.
    want = {"tp_small": 15, "tp_large": 34, "conv_water1k": 13, "conv_water8k": 24, "conv_uniform100k": 65}
    for name, n in want.items():
        c = synth.CONFIGS[name]
        assert len(paths_uvu(c["irreps_x"], c["irreps_y"], c["irreps_out"])) == n
    L = Layout(synth.CONFIGS["tp_large"]["irreps_x"], synth.CONFIGS["tp_large"]["irreps_y"],
               synth.CONFIGS["tp_large"]["irreps_out"])
    assert (L.dim_x, L.dim_y, L.dim_out, L.w_numel) == (2048, 16, 19968, 4352)


def test_parity_filter():
    # natural-parity outputs only: 1o x 1o -> 1e is dropped, 0e and 2e kept
    ps = paths_uvu("1o", "1o", "0e+1o+2e")
    assert [(p["l3"], p["p3"]) for p in ps] == [(0, 1), (2, 1)]
    ps = paths_uvu("1o", "1o", "1e")
    assert [(p["l3"], p["p3"]) for p in ps] == [(1, 1)]


@pytest.mark.parametrize("shared", [False, True])
def test_sparse_equals_dense(shared):
    L = Layout("3x0e+3x1o+3x2e+3x3o", "0e+1o+2e+3o", "0e+0o+1e+1o+2e+2o+3e+3o")
    x, y, w = make_inputs(L, 5, 0, shared)
    assert np.abs(tp.forward(L, x, y, w) - tp.forward_dense(L, x, y, w)).max() < 1e-12


def test_bilinear():
    L = Layout("4x0e+4x1o+4x2e", "0e+1o+2e", "0e+0o+1e+1o+2e+2o")
    x, y, w = make_inputs(L, 3, 1)
    x2, y2, _ = make_inputs(L, 3, 2)
    f = lambda a, b: tp.forward(L, a, b, w)
    assert np.abs(f(x + 2.5 * x2, y) - f(x, y) - 2.5 * f(x2, y)).max() < 1e-11
    assert np.abs(f(x, y - 0.5 * y2) - f(x, y) + 0.5 * f(x, y2)).max() < 1e-11


def _rotate_rows(L_irreps, rows, ang, inv, offs):
    out = rows.copy()
    for (mul, l, p), o in zip(L_irreps, offs):
        D = wigner.wigner_D_real(l, *ang) * (p if inv else 1)
        blk = rows[:, o:o + mul * (2 * l + 1)].reshape(-1, 2 * l + 1, mul)
        out[:, o:o + mul * (2 * l + 1)] = np.einsum("ab,zbu->zau", D, blk).reshape(rows.shape[0], -1)
    return out


@pytest.mark.parametrize("inv", [False, True])
def test_o3_equivariance(inv):
    ix, iy, io = "2x0e+2x1o+2x2e+2x1e", "0e+1o+2e", "0e+0o+1e+1o+2e+2o+3e+3o"
    L = Layout(ix, iy, io)
    x, y, w = make_inputs(L, 4, 3)
    ang = wigner.random_euler(np.random.default_rng(9))
    out = tp.forward(L, x, y, w)
    xr = _rotate_rows(L.X, x, ang, inv, L.x_off)
    yr = _rotate_rows(L.Y, y, ang, inv, L.y_off)
    out_r = tp.forward(L, xr, yr, w)
    O = [(p["mul"], p["l3"], p["p3"]) for p in L.paths]
    assert np.abs(out_r - _rotate_rows(O, out, ang, inv, [p["out_off"] for p in L.paths])).max() < 1e-11


def test_scalar_paths_scale_channels():
    L = Layout("3x0e+3x2e", "0e", "0e+2e")
    x, y, w = make_inputs(L, 4, 4)
    out = tp.forward(L, x, y, w)
    for p in L.paths:
        ref = L.x_block(x, p["i1"]) * y[:, :1, None] * L.w_block(w, p)[:, None, :]
        assert np.abs(L.out_block(out, p) - ref).max() < 1e-14


def test_1x1_single_channel():
    L = Layout("1x1o", "1x1o", "0e+1e+2e")
    rng = np.random.default_rng(11)
    a, b = rng.standard_normal(3), rng.standard_normal(3)
    x = np.array([[a[1], a[2], a[0]]])
    y = np.array([[b[1], b[2], b[0]]])
    out = tp.forward(L, x, y, np.ones((1, 3)))
    assert out[0, 0] == pytest.approx(a @ b / math.sqrt(3), abs=1e-14)
    c = np.cross(a, b) / math.sqrt(2)
    assert np.abs(out[0, 1:4] - [c[1], c[2], c[0]]).max() < 1e-14


def test_harmonic_inputs_layout():
    # y built from harmonics of random directions: blocks of y line up with the irreps
    L = Layout("2x1o", "0e+1o+2e", "1o")
    v = synth.unit_vectors(3, 0)
    Y = sh.real_sh(2, v)
    assert Y.shape == (3, L.dim_y)


@pytest.mark.parametrize("shared", [False, True])
def test_backward_adjoint_identities(shared):
    L = Layout("3x0e+3x1o+3x2e+3x3o", "0e+1o+2e+3o", "0e+0o+1e+1o+2e+2o+3e+3o")
    x, y, w = make_inputs(L, 4, 5, shared)
    g = synth.gaussian((4, L.dim_out), 5, synth.S_G)
    dx, dy, dw = tp.backward(L, x, y, w, g)
    f = np.sum(g * tp.forward(L, x, y, w))
    for d, v in ((dx, x), (dy, y), (dw, w)):
        assert np.sum(d * v) == pytest.approx(f, rel=1e-12)


def test_backward_finite_differences():
    L = Layout("2x0e+2x1o+2x2e", "0e+1o+2e", "0e+0o+1e+1o+2e+2o")
    x, y, w = make_inputs(L, 2, 6)
    g = synth.gaussian((2, L.dim_out), 6, synth.S_G)
    dx, dy, dw = tp.backward(L, x, y, w, g)
    f = lambda a, b, c: np.sum(g * tp.forward(L, a, b, c))
    h = 1e-6
    rng = np.random.default_rng(0)
    for d, which in ((dx, 0), (dy, 1), (dw, 2)):
        args = [x, y, w]
        for _ in range(6):
            idx = tuple(rng.integers(0, s) for s in args[which].shape)
            ap, am = [a.copy() for a in args], [a.copy() for a in args]
            ap[which][idx] += h
            am[which][idx] -= h
            assert d[idx] == pytest.approx((f(*ap) - f(*am)) / (2 * h), abs=1e-7)
