"""Pins of the oracle's parity-selected and collapsed tensor-product variants (CPU only).

[E3J] B.1: the Gaunt product covers the symmetric paths (l1 + l2 + l3 even),
the vector signal product the skew-symmetric ones, and e3j selects the matching
paths by parity and collapses outputs by degree; [E3J] B.3: collapsing sums the
isomorphic copies of each irreducible output space.

Pinned by: 1o x 1o splitting into dot and symmetric-traceless (symmetric) and
cross product (skew); the skew paths vanishing on harmonics of one direction
(the product of two functions on the sphere, which is what the Gaunt product
computes, only has l1 + l2 + l3 even parts); the symmetric and skew path sets
partitioning all paths; collapsed blocks equal to the sums of the uncollapsed
path blocks; O(3) equivariance of the collapsed blocks; adjoint identities and
central differences of the collapsed backward; and planted mistakes.
"""

import math

import numpy as np
import pytest

from oracle import sh, tp, wigner
from oracle.irreps import Layout, paths_uvu
from clebsch_gordan_tensor_amd import synth

IX, IY, IO = "2x0e+2x1o+2x2e+2x3o", "0e+1o+2e+3o", "0e+0o+1e+1o+2e+2o+3e+3o"


def inputs(L, B, seed, shared=False):
    x = synth.gaussian((B, L.dim_x), seed, synth.S_X)
    y = synth.gaussian((B, L.dim_y), seed, synth.S_Y)
    w = synth.gaussian((L.w_numel,) if shared else (B, L.w_numel), seed, synth.S_W)
    return x, y, w


def test_selection_partitions_the_paths():
    key = lambda p: (p["i1"], p["i2"], p["l3"])
    full = [key(p) for p in paths_uvu(IX, IY, IO)]
    sym = [key(p) for p in paths_uvu(IX, IY, IO, "symmetric")]
    skew = [key(p) for p in paths_uvu(IX, IY, IO, "skew")]
    assert sorted(sym + skew) == sorted(full) and not set(sym) & set(skew)
    assert all((p["l1"] + p["l2"] + p["l3"]) % 2 == 0 for p in paths_uvu(IX, IY, IO, "symmetric"))
    with pytest.raises(ValueError):
        paths_uvu(IX, IY, IO, "other")


def test_1x1_symmetric_and_skew():
    rng = np.random.default_rng(21)
    a, b = rng.standard_normal(3), rng.standard_normal(3)
    x = np.array([[a[1], a[2], a[0]]])       # real l = 1 order (y, z, x)
    y = np.array([[b[1], b[2], b[0]]])
    sym = Layout("1o", "1o", "0e+1e+2e", "symmetric", collapse=True)
    skew = Layout("1o", "1o", "0e+1e+2e", "skew", collapse=True)
    assert [(g["l3"], g["p3"]) for g in sym.groups] == [(0, 1), (2, 1)]
    assert [(g["l3"], g["p3"]) for g in skew.groups] == [(1, 1)]
    os_ = tp.forward(sym, x, y, np.ones((1, sym.w_numel)))
    ok = tp.forward(skew, x, y, np.ones((1, skew.w_numel)))
    assert os_[0, 0] == pytest.approx(a @ b / math.sqrt(3), abs=1e-14)
    c = np.cross(a, b) / math.sqrt(2)
    assert np.abs(ok[0] - [c[1], c[2], c[0]]).max() < 1e-14
    # the symmetric l = 2 part is the traceless symmetric matrix: its norm is
    # |a|^2 |b|^2 / 2 + (a.b)^2 / 2 - (a.b)^2 / 3 (squared Frobenius norm of
    # (ab^T + ba^T)/2 - a.b I/3, orthonormal CG blocks preserve it)
    ab = a @ b
    want = (a @ a) * (b @ b) / 2 + ab * ab / 2 - ab * ab / 3
    assert np.sum(os_[0, 1:] ** 2) == pytest.approx(want, rel=1e-12)


def test_skew_paths_vanish_on_one_direction():
    v = synth.unit_vectors(6, 3)
    Yv = sh.real_sh(3, v)
    ix = "0e+1o+2e+3o"                       # x = the harmonics themselves, one channel per degree
    L = Layout(ix, IY, IO, "skew", collapse=True)
    Ls = Layout(ix, IY, IO, "symmetric", collapse=True)
    La = Layout(ix, IY, IO, "all", collapse=True)
    ones = lambda L_: np.ones((6, L_.w_numel))
    assert np.abs(tp.forward(L, Yv, Yv, ones(L))).max() < 1e-13
    out_s, out_a = tp.forward(Ls, Yv, Yv, ones(Ls)), tp.forward(La, Yv, Yv, ones(La))
    for g in La.groups:
        o = g["out_off"]
        n = g["mul"] * (2 * g["l3"] + 1)
        hit = [h for h in Ls.groups if (h["l3"], h["p3"]) == (g["l3"], g["p3"])]
        ref = out_s[:, hit[0]["out_off"]:hit[0]["out_off"] + n] if hit else 0.0
        assert np.abs(out_a[:, o:o + n] - ref).max() < 1e-13


@pytest.mark.parametrize("select", ["all", "symmetric", "skew"])
def test_collapsed_is_the_sum_of_path_blocks(select):
    Lc = Layout(IX, IY, IO, select, collapse=True)
    Lf = Layout(IX, IY, IO, select, collapse=False)
    assert Lc.w_numel == Lf.w_numel and len(Lc.paths) == len(Lf.paths)
    x, y, w = inputs(Lf, 3, 22)
    full, col = tp.forward(Lf, x, y, w), tp.forward(Lc, x, y, w)
    ref = np.zeros_like(col)
    for pf, pc in zip(Lf.paths, Lc.paths):
        n = pf["mul"] * (2 * pf["l3"] + 1)
        ref[:, pc["out_off"]:pc["out_off"] + n] += full[:, pf["out_off"]:pf["out_off"] + n]
    assert np.abs(col - ref).max() < 1e-13
    # one block per (l3, p3) reached, in irreps_out order, multiplicity 2
    reached = {(p["l3"], p["p3"]) for p in Lf.paths}
    want = [(l, q) for l in range(4) for q in (1, -1) if (l, q) in reached]
    assert [(g["l3"], g["p3"]) for g in Lc.groups] == want
    assert Lc.dim_out == sum(2 * (2 * l + 1) for l, _ in want)


@pytest.mark.parametrize("inv", [False, True])
def test_collapsed_equivariance(inv):
    L = Layout(IX, IY, IO, "all", collapse=True)
    x, y, w = inputs(L, 3, 23)
    ang = wigner.random_euler(np.random.default_rng(24))

    def rot(blocks, rows):
        res = rows.copy()
        for mul, l, p, o in blocks:
            D = wigner.wigner_D_real(l, *ang) * (p if inv else 1)
            blk = rows[:, o:o + mul * (2 * l + 1)].reshape(-1, 2 * l + 1, mul)
            res[:, o:o + mul * (2 * l + 1)] = np.einsum("ab,zbu->zau", D, blk).reshape(rows.shape[0], -1)
        return res

    xb = [(m, l, p, o) for (m, l, p), o in zip(L.X, L.x_off)]
    yb = [(1, l, p, o) for (_, l, p), o in zip(L.Y, L.y_off)]
    ob = [(g["mul"], g["l3"], g["p3"], g["out_off"]) for g in L.groups]
    out_r = tp.forward(L, rot(xb, x), rot(yb, y), w)
    assert np.abs(out_r - rot(ob, tp.forward(L, x, y, w))).max() < 1e-11


@pytest.mark.parametrize("shared", [False, True])
def test_collapsed_backward(shared):
    L = Layout(IX, IY, IO, "all", collapse=True)
    x, y, w = inputs(L, 3, 25, shared)
    g = synth.gaussian((3, L.dim_out), 25, synth.S_G)
    dx, dy, dw = tp.backward(L, x, y, w, g)
    f = np.sum(g * tp.forward(L, x, y, w))
    for d, v in ((dx, x), (dy, y), (dw, w)):
        assert np.sum(d * v) == pytest.approx(f, rel=1e-12)
    h = 1e-6
    rng = np.random.default_rng(26)
    args = [x, y, w]
    for d, k in ((dx, 0), (dy, 1), (dw, 2)):
        for _ in range(4):
            idx = tuple(rng.integers(0, s) for s in args[k].shape)
            ap = [a.copy() for a in args]
            am = [a.copy() for a in args]
            ap[k][idx] += h
            am[k][idx] -= h
            fd = (np.sum(g * tp.forward(L, *ap)) - np.sum(g * tp.forward(L, *am))) / (2 * h)
            assert d[idx] == pytest.approx(fd, abs=1e-7)


def test_collapse_needs_equal_multiplicities():
    with pytest.raises(ValueError):
        Layout("2x0e+3x1o", "0e+1o", "0e+1o", collapse=True)   # 1o is fed by the 2x0e and 3x1o blocks
    L = Layout("2x0e+3x1e", "0e", "0e+1e", collapse=True)       # separate outputs: fine
    assert [g["mul"] for g in L.groups] == [2, 3]


def _fails(check):
    try:
        check()
    except (AssertionError, ValueError, IndexError):
        return True
    return False


def test_planted_mistakes_are_caught(monkeypatch):
    import oracle.irreps as irr
    orig = irr.paths_uvu

    # symmetric and skew exchanged
    def swapped(ix, iy, io, select="all"):
        return orig(ix, iy, io, {"symmetric": "skew", "skew": "symmetric"}.get(select, select))
    with monkeypatch.context() as m:
        m.setattr(irr, "paths_uvu", swapped)
        assert _fails(test_1x1_symmetric_and_skew)
        assert _fails(test_skew_paths_vanish_on_one_direction)

    # collapsed blocks overwritten instead of summed
    orig_fwd = tp.forward

    def overwrite(L, x, y, w):
        out = np.zeros((x.shape[0], L.dim_out))
        for p in L.paths:
            one = Layout.__new__(Layout)
            one.__dict__.update(L.__dict__)
            one.paths = [p]
            blk = orig_fwd(one, x, y, w)
            o, n = p["out_off"], p["mul"] * (2 * p["l3"] + 1)
            out[:, o:o + n] = blk[:, o:o + n]
        return out
    with monkeypatch.context() as m:
        m.setattr(tp, "forward", overwrite)
        assert _fails(lambda: test_collapsed_is_the_sum_of_path_blocks("all"))
