"""Real spherical harmonics, component-normalised (oracle; test infrastructure).

[COURSE] lesson 02b: Y^(l)(R r) = D^(l)(R) Y^(l)(r), parity (-1)^l, several
normalisation conventions; [V2106] uses component-normalised harmonics
(sum_m Y_lm^2 = 2l+1 on the unit sphere); [E3J] G.1: the m = +-l harmonic is
c_l (x +- i y)^l and the longitude dependence is e^{i m phi}.

Reading taken (the pages fix no axis or ordering): z is the polar axis, m runs
-l ... l inside a block, blocks are l-major; no Condon-Shortley sign. In
Cartesian form, for a unit vector (x, y, z):

  Y_lm = sqrt(2l+1) sqrt((l-|m|)!/(l+|m|)!) P_l^{(|m|)}(z) T_m(x, y)
  T_0 = 1,  T_m = sqrt2 Re (x+iy)^m (m > 0),  T_m = sqrt2 Im (x+iy)^|m| (m < 0)

with P_l^{(k)} the k-th derivative of the Legendre polynomial P_l. This gives
Y_0 = 1 and Y_1 = sqrt3 (y, z, x). Inputs are normalised first; the zero vector
maps to Y_0 = 1 and zeros elsewhere.
"""

import math

import numpy as np
from numpy.polynomial import legendre as npleg


def _legendre_deriv(l, k, z):
    c = np.zeros(l + 1)
    c[l] = 1.0
    if k > 0:
        c = npleg.legder(c, k) if k <= l else np.zeros(1)
    return npleg.legval(z, c)


def _norm(l, am):
    return math.sqrt(2 * l + 1) * math.sqrt(math.factorial(l - am) / math.factorial(l + am))


def real_sh(lmax, vec):
    """Y_l(vec/|vec|) for l = 0..lmax; vec [n, 3] -> [n, (lmax+1)^2] fp64."""
    vec = np.asarray(vec, dtype=np.float64)
    n = vec.shape[0]
    r = np.linalg.norm(vec, axis=1)
    zero = r == 0.0
    rs = np.where(zero, 1.0, r)
    x, y, z = vec[:, 0] / rs, vec[:, 1] / rs, vec[:, 2] / rs
    w = x + 1j * y
    out = np.zeros((n, (lmax + 1) ** 2))
    for l in range(lmax + 1):
        for m in range(-l, l + 1):
            am = abs(m)
            p = _legendre_deriv(l, am, z)
            if m == 0:
                t = np.ones(n)
            elif m > 0:
                t = math.sqrt(2.0) * (w ** am).real
            else:
                t = math.sqrt(2.0) * (w ** am).imag
            out[:, l * l + l + m] = _norm(l, am) * p * t
    out[zero, :] = 0.0
    out[zero, 0] = 1.0
    return out


def real_sh_grad(lmax, vec, grad_sh):
    """Vector-Jacobian product: d/dvec of sum(grad_sh * real_sh(lmax, vec)).

    Y depends on vec only through rhat = vec/|vec|, so
    d/dvec = (I - rhat rhat^T) / |vec| . grad_P(rhat), where P is the Cartesian
    polynomial of the module docstring (any smooth extension of Y off the
    sphere gives the same tangential part). Zero vectors get a zero gradient.
    """
    vec = np.asarray(vec, dtype=np.float64)
    grad_sh = np.asarray(grad_sh, dtype=np.float64)
    n = vec.shape[0]
    r = np.linalg.norm(vec, axis=1)
    zero = r == 0.0
    rs = np.where(zero, 1.0, r)
    rh = vec / rs[:, None]
    x, y, z = rh[:, 0], rh[:, 1], rh[:, 2]
    w = x + 1j * y
    gP = np.zeros((n, 3))
    for l in range(lmax + 1):
        for m in range(-l, l + 1):
            am = abs(m)
            g = grad_sh[:, l * l + l + m]
            c = _norm(l, am)
            p = _legendre_deriv(l, am, z)
            dp = _legendre_deriv(l, am + 1, z)
            if m == 0:
                t, tx, ty = np.ones(n), np.zeros(n), np.zeros(n)
            else:
                wm = w ** am
                wm1 = w ** (am - 1)
                s2 = math.sqrt(2.0)
                if m > 0:
                    t = s2 * wm.real
                    tx = s2 * am * wm1.real
                    ty = -s2 * am * wm1.imag
                else:
                    t = s2 * wm.imag
                    tx = s2 * am * wm1.imag
                    ty = s2 * am * wm1.real
            gP[:, 0] += g * c * p * tx
            gP[:, 1] += g * c * p * ty
            gP[:, 2] += g * c * dp * t
    radial = np.einsum("ni,ni->n", rh, gP)
    out = (gP - rh * radial[:, None]) / rs[:, None]
    out[zero, :] = 0.0
    return out
