"""Pins of the connection-mode oracle (oracle/modes.py: uvu with y multiplicity
v >= 1, and uvw, [COURSE] 03b) against what the pages and the mathematics fix.

* uvu with v = 1 is the channel-wise product of oracle/tp.py (itself pinned);
* uvu with v > 1 is linear in y: summing, over the y channels b, the v = 1
  product of y's channel b with the weight column w[:, b] gives it;
* uvw with v = 1 is, path by path, the equivariant linear map (oracle/linear.py,
  pinned on its own) applied to the unit-weight uvu path outputs; collapsed
  uvw is that linear map from all path outputs to the collapsed blocks;
* 1o x 1o in uvw mode from the dot and cross products in closed form (the CG
  blocks 1 x 1 -> 0 and -> 1 are dot/sqrt3 and cross/sqrt2, [COURSE] 03a);
* O(3) equivariance (Wigner-D on every block, parity included);
* weight counts sum u v (uvu) and sum u v w (uvw) ([COURSE] 03b counts weights);
* the backward: the adjoint identities of the trilinear form and central
  differences;
* planted mistakes (transposed uvw weights, a dropped y-channel sum, the output
  multiplicity taken from x) are caught.
"""

import math

import numpy as np
import pytest

from oracle import linear as olin
from oracle import modes
from oracle import tp
from oracle import wigner
from oracle.irreps import Layout
from clebsch_gordan_tensor_amd import synth


def inputs(ML, B, seed, shared=False):
    x = synth.gaussian((B, ML.dim_x), seed, synth.S_X)
    y = synth.gaussian((B, ML.dim_y), seed, synth.S_Y)
    w = synth.gaussian((ML.w_numel,) if shared else (B, ML.w_numel), seed, synth.S_W)
    return x, y, w


@pytest.mark.parametrize("shared", [False, True])
def test_uvu_v1_is_the_channelwise_product(shared):
    ix, iy, io = "3x0e+3x1o+3x2e", "0e+1o+2e", "0e+0o+1e+1o+2e+2o"
    ML, L = modes.ModeLayout(ix, iy, io, "uvu"), Layout(ix, iy, io)
    x, y, w = inputs(ML, 5, 1, shared)
    assert ML.w_numel == L.w_numel and ML.dim_out == L.dim_out
    assert np.abs(modes.forward(ML, x, y, w) - tp.forward(L, x, y, w)).max() < 1e-13
    g = synth.gaussian((5, ML.dim_out), 1, synth.S_G)
    for a, b in zip(modes.backward(ML, x, y, w, g), tp.backward(L, x, y, w, g)):
        assert np.abs(a - b).max() < 1e-12


def uvu_v_pin(collapse):
    """(oracle output, sum over y channels of v = 1 products) for uvu with v = 3."""
    ix, iy, io, v = "4x0e+4x1o+4x2e", "3x0e+3x1o+3x2e", "0e+0o+1e+1o+2e+2o", 3
    ML = modes.ModeLayout(ix, iy, io, "uvu", collapse=collapse)
    L1 = Layout(ix, "0e+1o+2e", io, "all", collapse)
    x, y, w = inputs(ML, 4, 2)
    out = modes.forward(ML, x, y, w)
    ref = np.zeros_like(out)
    for b in range(v):
        yb = np.concatenate([y[:, o:o + v * (2 * l + 1)].reshape(4, 2 * l + 1, v)[:, :, b]
                             for (_, l, _), o in zip(ML.Y, ML.y_off)], axis=1)
        wb = np.concatenate([w[:, p["w_off"]:p["w_off"] + p["w_len"]].reshape(4, p["u"], v)[:, :, b]
                             for p in ML.paths], axis=1)
        ref += tp.forward(L1, x, yb, wb)
    return out, ref


@pytest.mark.parametrize("collapse", [False, True])
def test_uvu_v_channels_sum_of_v1_products(collapse):
    out, ref = uvu_v_pin(collapse)
    assert np.abs(out - ref).max() < 1e-12


def uvw_linear_pin(collapse):
    """(oracle output, per-path linear map of the unit-weight uvu path outputs)."""
    ix, iy = "3x0e+2x1o+3x2e", "0e+1o+2e"
    io = "4x0e+5x0o+2x1e+3x1o+4x2e+2x2o"
    ML = modes.ModeLayout(ix, iy, io, "uvw", collapse=collapse)
    L = Layout(ix, iy, io)
    B = 6
    x, y, W = inputs(ML, B, 3, shared=True)
    T = tp.forward(L, x, y, np.ones(L.w_numel))  # unit-weight path outputs, [B, sum_p u_p (2l3+1)]
    out = modes.forward(ML, x, y, W)
    ref = np.zeros_like(out)
    for p, q in zip(ML.paths, L.paths):
        Tp = L.out_block(T, q).reshape(B, -1)
        LL = olin.LinearLayout([(p["u"], p["l3"], p["p3"])], [(p["mul"], p["l3"], p["p3"])])
        Wp = W[p["w_off"]:p["w_off"] + p["w_len"]]  # [u][1][w] = [u][w]
        ML.out_block(ref, p)[...] += olin.forward(LL, Tp, Wp).reshape(B, 2 * p["l3"] + 1, p["mul"])
    return out, ref


@pytest.mark.parametrize("collapse", [False, True])
def test_uvw_v1_is_linear_after_unit_uvu(collapse):
    out, ref = uvw_linear_pin(collapse)
    assert np.abs(out - ref).max() < 1e-12


def test_uvw_1o_x_1o_dot_and_cross():
    ML = modes.ModeLayout("2x1o", "1x1o", "3x0e+2x1e", "uvw")
    rng = np.random.default_rng(7)
    a = rng.standard_normal((2, 3))  # two x channels, Cartesian
    b = rng.standard_normal(3)
    x = np.array([[a[c, k] for k in (1, 2, 0) for c in range(2)]])  # [m][channel], m = (y, z, x)
    y = np.array([[b[1], b[2], b[0]]])
    W = rng.standard_normal(ML.w_numel)
    W0 = W[:6].reshape(2, 1, 3)[:, 0, :]    # path 1o x 1o -> 0e: [u][w]
    W1 = W[6:10].reshape(2, 1, 2)[:, 0, :]  # path 1o x 1o -> 1e
    out = modes.forward(ML, x, y, W)[0]
    dots = a @ b / math.sqrt(3)
    assert np.abs(out[:3] - dots @ W0).max() < 1e-13
    cr = np.cross(a, b) / math.sqrt(2)             # [u][xyz]
    mixed = cr.T @ W1                               # [xyz][w]
    assert np.abs(out[3:].reshape(3, 2) - mixed[[1, 2, 0]]).max() < 1e-13


def _rotate(irreps, offs, rows, ang, inv):
    out = rows.copy()
    for (mul, l, p), o in zip(irreps, offs):
        D = wigner.wigner_D_real(l, *ang) * (p if inv else 1)
        blk = rows[:, o:o + mul * (2 * l + 1)].reshape(-1, 2 * l + 1, mul)
        out[:, o:o + mul * (2 * l + 1)] = np.einsum("ab,zbu->zau", D, blk).reshape(rows.shape[0], -1)
    return out


@pytest.mark.parametrize("mode,inv", [("uvu", False), ("uvu", True), ("uvw", False), ("uvw", True)])
def test_o3_equivariance(mode, inv):
    ix, iy, io = "2x0e+2x1o+2x2e", "2x0e+2x1o+2x2e", "3x0e+3x0o+3x1e+2x1o+2x2e+2x2o+3x3e+3x3o"
    ML = modes.ModeLayout(ix, iy, io, mode)
    x, y, w = inputs(ML, 3, 4)
    ang = wigner.random_euler(np.random.default_rng(5))
    out = modes.forward(ML, x, y, w)
    out_r = modes.forward(ML, _rotate(ML.X, ML.x_off, x, ang, inv), _rotate(ML.Y, ML.y_off, y, ang, inv), w)
    O = [(g["mul"], g["l3"], g["p3"]) for g in ML.groups]
    assert np.abs(out_r - _rotate(O, [g["out_off"] for g in ML.groups], out, ang, inv)).max() < 1e-11


def test_weight_counts():
    ML = modes.ModeLayout("3x0e+2x1o", "4x0e+1x1o", "5x0e+6x1o+7x1e", "uvw")
    # 0e x 0e -> 0e; 0e x 1o -> 1o; 1o x 0e -> 1o; 1o x 1o -> 0e, 1e
    assert ML.w_numel == 3 * 4 * 5 + 3 * 1 * 6 + 2 * 4 * 6 + 2 * 1 * 5 + 2 * 1 * 7
    MU = modes.ModeLayout("3x0e+2x1o", "4x0e+1x1o", "5x0e+6x1o+7x1e", "uvu")
    assert MU.w_numel == 3 * 4 + 3 * 1 + 2 * 4 + 2 * 1 + 2 * 1
    assert MU.dim_out == 3 + 3 * 3 + 2 * 3 + 2 + 2 * 3


@pytest.mark.parametrize("mode,shared,collapse", [("uvu", False, False), ("uvu", True, True),
                                                  ("uvw", True, False), ("uvw", False, True)])
def test_backward_adjoint_identities(mode, shared, collapse):
    ML = modes.ModeLayout("2x0e+2x1o+2x2e", "2x0e+1x1o+2x2e", "2x0e+2x0o+2x1e+2x1o+2x2e+2x2o", mode,
                          collapse=collapse)
    x, y, w = inputs(ML, 3, 6, shared)
    g = synth.gaussian((3, ML.dim_out), 6, synth.S_G)
    f = np.sum(g * modes.forward(ML, x, y, w))
    for d, v in zip(modes.backward(ML, x, y, w, g), (x, y, w)):
        assert np.sum(d * v) == pytest.approx(f, rel=1e-12)


@pytest.mark.parametrize("mode", ["uvu", "uvw"])
def test_backward_finite_differences(mode):
    ML = modes.ModeLayout("2x0e+2x1o", "2x0e+2x1o", "2x0e+2x1o+2x1e", mode)
    x, y, w = inputs(ML, 2, 8)
    g = synth.gaussian((2, ML.dim_out), 8, synth.S_G)
    grads = modes.backward(ML, x, y, w, g)
    f = lambda a, b, c: np.sum(g * modes.forward(ML, a, b, c))
    h = 1e-6
    rng = np.random.default_rng(1)
    for which in range(3):
        for _ in range(6):
            args = [x, y, w]
            idx = tuple(rng.integers(0, s) for s in args[which].shape)
            ap, am = [a.copy() for a in args], [a.copy() for a in args]
            ap[which][idx] += h
            am[which][idx] -= h
            assert grads[which][idx] == pytest.approx((f(*ap) - f(*am)) / (2 * h), abs=1e-7)


def test_planted_mistakes_are_caught(monkeypatch):
    """Each plausible slip planted in the oracle's arithmetic fails the pin above
    that guards it."""
    real_einsum = np.einsum

    def planted(spec_from, fn):
        def einsum(spec, *ops):
            return fn(*ops) if spec == spec_from else real_einsum(spec, *ops)
        return einsum

    # uvw weights read as W_p[k, b, a] (flat order reversed) instead of W_p[a, b, k]
    monkeypatch.setattr(modes.np, "einsum", planted(
        "ijk,zia,zjb,zabc->zkc",
        lambda C, xb, yb, wb: real_einsum("ijk,zia,zjb,zcba->zkc", C, xb, yb,
                                          wb.reshape(wb.shape[0], wb.shape[3], wb.shape[2], wb.shape[1]))))
    for collapse in (False, True):
        out, ref = uvw_linear_pin(collapse)
        assert np.abs(out - ref).max() > 1e-3
    # uvu: the sum over the y channels b dropped (only b = 0 kept)
    monkeypatch.setattr(modes.np, "einsum", planted(
        "ijk,zia,zjb,zab->zka",
        lambda C, xb, yb, wb: real_einsum("ijk,zia,zj,za->zka", C, xb, yb[:, :, 0], wb[:, :, 0])))
    out, ref = uvu_v_pin(False)
    assert np.abs(out - ref).max() > 1e-3
    monkeypatch.setattr(modes.np, "einsum", real_einsum)
    # the uvw output multiplicity taken from x (u) instead of irreps_out: the
    # weight count would be sum u v u, not the closed form of test_weight_counts
    ML = modes.ModeLayout("3x0e+2x1o", "4x0e+1x1o", "5x0e+6x1o+7x1e", "uvw")
    assert sum(p["u"] * p["v"] * p["u"] for p in ML.paths) != 3 * 4 * 5 + 3 * 1 * 6 + 2 * 4 * 6 + 2 * 1 * 5 + 2 * 1 * 7
    # the uvw backward with dx's weight contraction transposed: the adjoint identity fails
    monkeypatch.setattr(modes.np, "einsum", planted(
        "ijk,zjb,zkc,zabc->zia",
        lambda C, yb, gb, wb: real_einsum("ijk,zjb,zka,zcba->zia", C, yb, gb[:, :, :wb.shape[1]],
                                          wb[:, :, :, :wb.shape[1]].transpose(0, 3, 2, 1))))
    MA = modes.ModeLayout("2x0e+2x1o", "1x0e+1x1o", "2x0e+2x1o+2x1e", "uvw")
    x, y, w = inputs(MA, 3, 11, True)
    g = synth.gaussian((3, MA.dim_out), 11, synth.S_G)
    dx, _, _ = modes.backward(MA, x, y, w, g)
    monkeypatch.setattr(modes.np, "einsum", real_einsum)
    f = np.sum(g * modes.forward(MA, x, y, w))
    assert abs(np.sum(dx * x) - f) > 1e-6 * abs(f)
