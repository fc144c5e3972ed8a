"""Pins of the oracle's spherical harmonics and Wigner-D matrices (CPU only).

Closed forms of the textbook real harmonics for l <= 3 (tabulated Cartesian
polynomials, times sqrt(4 pi) for component normalisation), the m = +-l form
c_l (x +- iy)^l of [E3J] G.1, component normalisation ([V2106]), equivariance
and parity ([COURSE] 02b), Wigner-D homomorphism ([COURSE] 01b) and central
finite differences for the gradient.
"""

import math

import numpy as np
import pytest

from oracle import sh, wigner


def textbook_real_sh(v):
    """Component-normalised real harmonics l = 0..3 written out per (l, m)."""
    x, y, z = v.T
    s = math.sqrt
    Y = [np.ones_like(x),
         s(3) * y, s(3) * z, s(3) * x,
         s(15) * x * y, s(15) * y * z, s(5) / 2 * (3 * z * z - 1), s(15) * x * z, s(15) / 2 * (x * x - y * y),
         s(35 / 8) * y * (3 * x * x - y * y), s(105) * x * y * z, s(21 / 8) * y * (5 * z * z - 1),
         s(7) / 2 * z * (5 * z * z - 3),
         s(21 / 8) * x * (5 * z * z - 1), s(105) / 2 * z * (x * x - y * y), s(35 / 8) * x * (x * x - 3 * y * y)]
    return np.stack(Y, axis=1)


def rand_units(n, seed):
    v = np.random.default_rng(seed).standard_normal((n, 3))
    return v / np.linalg.norm(v, axis=1, keepdims=True)


def test_closed_forms_l_le_3():
    v = rand_units(50, 0)
    assert np.abs(sh.real_sh(3, v) - textbook_real_sh(v)).max() < 1e-13


def test_unnormalised_input_and_zero_vector():
    v = rand_units(10, 1)
    Y = sh.real_sh(4, v)
    assert np.abs(sh.real_sh(4, 3.7 * v) - Y).max() < 1e-13
    Z = sh.real_sh(4, np.zeros((1, 3)))
    assert Z[0, 0] == 1.0 and np.all(Z[0, 1:] == 0.0)


def test_component_normalisation():
    v = rand_units(40, 2)
    Y = sh.real_sh(6, v)
    for l in range(7):
        assert np.abs((Y[:, l * l:(l + 1) ** 2] ** 2).sum(1) - (2 * l + 1)).max() < 1e-12


def test_top_weight_is_power_of_x_plus_iy():
    # m = +-l is proportional to Re/Im (x + iy)^l with one constant per l
    v = rand_units(30, 3)
    w = v[:, 0] + 1j * v[:, 1]
    Y = sh.real_sh(6, v)
    for l in range(1, 7):
        re, im = (w ** l).real, (w ** l).imag
        cp = Y[:, l * l + 2 * l] / re
        cm = Y[:, l * l] / im
        assert np.ptp(cp) < 1e-9 * abs(cp[0]) and np.ptp(cm) < 1e-9 * abs(cm[0])
        assert cp[0] == pytest.approx(cm[0], rel=1e-12)


@pytest.mark.parametrize("l", range(7))
def test_equivariance_and_parity(l):
    rng = np.random.default_rng(10 + l)
    ang = wigner.random_euler(rng)
    R = wigner.euler_to_matrix(*ang)
    D = wigner.wigner_D_real(l, *ang)
    v = rand_units(20, 20 + l)
    blk = lambda Y: Y[:, l * l:(l + 1) ** 2]
    assert np.abs(blk(sh.real_sh(l, v @ R.T)) - blk(sh.real_sh(l, v)) @ D.T).max() < 1e-12
    assert np.abs(blk(sh.real_sh(l, -v)) - (-1) ** l * blk(sh.real_sh(l, v))).max() < 1e-13


def test_wigner_l1_and_homomorphism():
    rng = np.random.default_rng(5)
    P = np.array([[0, 1, 0], [0, 0, 1], [1, 0, 0]], dtype=float)  # (x,y,z) -> (y,z,x)
    for _ in range(5):
        a1 = wigner.random_euler(rng)
        a2 = wigner.random_euler(rng)
        R1, R2 = wigner.euler_to_matrix(*a1), wigner.euler_to_matrix(*a2)
        assert np.abs(wigner.wigner_D_real(1, *a1) - P @ R1 @ P.T).max() < 1e-14
        a12 = wigner.matrix_to_euler(R1 @ R2)
        assert np.abs(wigner.euler_to_matrix(*a12) - R1 @ R2).max() < 1e-12
        for l in range(5):
            D12 = wigner.wigner_D_real(l, *a12)
            D1, D2 = wigner.wigner_D_real(l, *a1), wigner.wigner_D_real(l, *a2)
            assert np.abs(D12 - D1 @ D2).max() < 1e-11
            assert np.abs(D1 @ D1.T - np.eye(2 * l + 1)).max() < 1e-12


@pytest.mark.parametrize("lmax", [1, 3, 4])
def test_gradient_central_differences(lmax):
    rng = np.random.default_rng(40 + lmax)
    v = rng.standard_normal((8, 3)) * 2.0
    g = rng.standard_normal((8, (lmax + 1) ** 2))
    an = sh.real_sh_grad(lmax, v, g)
    h = 1e-6
    fd = np.zeros_like(v)
    for k in range(3):
        e = np.zeros(3)
        e[k] = h
        fd[:, k] = ((sh.real_sh(lmax, v + e) - sh.real_sh(lmax, v - e)) * g).sum(1) / (2 * h)
    assert np.abs(an - fd).max() < 1e-8 * max(1.0, np.abs(fd).max())
    assert np.all(sh.real_sh_grad(lmax, np.zeros((1, 3)), g[:1]) == 0.0)
