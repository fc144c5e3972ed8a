"""Real Wigner-D matrices (oracle test tool; test infrastructure).

[COURSE] lesson 01b: representations satisfy D(g1 g2) = D(g1) D(g2); the irreps
of SO(3) are labelled by l with dimension 2l+1 (``o3.wigner_D``). Built here
independently of the harmonics and of the CG tables, from Euler angles:

  R = Rz(alpha) Ry(beta) Rz(gamma)
  D^l_{m'm}(R) = e^{-i m' alpha} d^l_{m'm}(beta) e^{-i m gamma}      (complex basis)
  d^l_{m'm}(beta) = sum_s (-1)^{m'-m+s} sqrt((l+m')!(l-m')!(l+m)!(l-m)!)
                    / ((l+m-s)! s! (m'-m+s)! (l-m'-s)!)
                    cos(beta/2)^{2l+m-m'-2s} sin(beta/2)^{m'-m+2s}

The complex harmonics obey Y(R r) = conj(D(R)) Y(r), so in the real basis
(``cg.real_basis``) D_real(R) = U conj(D(R)) U^H, which is real orthogonal.
"""

import math

import numpy as np

from .cg import real_basis


def rot_z(a):
    c, s = math.cos(a), math.sin(a)
    return np.array([[c, -s, 0.0], [s, c, 0.0], [0.0, 0.0, 1.0]])


def rot_y(b):
    c, s = math.cos(b), math.sin(b)
    return np.array([[c, 0.0, s], [0.0, 1.0, 0.0], [-s, 0.0, c]])


def euler_to_matrix(alpha, beta, gamma):
    return rot_z(alpha) @ rot_y(beta) @ rot_z(gamma)


def random_euler(rng):
    """Haar-random rotation as zyz Euler angles."""
    alpha = rng.uniform(0.0, 2.0 * math.pi)
    gamma = rng.uniform(0.0, 2.0 * math.pi)
    beta = math.acos(rng.uniform(-1.0, 1.0))
    return alpha, beta, gamma


def small_d(l, beta):
    f = math.factorial
    c, s = math.cos(beta / 2.0), math.sin(beta / 2.0)
    d = np.zeros((2 * l + 1, 2 * l + 1))
    for mp in range(-l, l + 1):
        for m in range(-l, l + 1):
            tot = 0.0
            pre = math.sqrt(f(l + mp) * f(l - mp) * f(l + m) * f(l - m))
            for k in range(0, 2 * l + 1):
                a1, a2, a3, a4 = l + m - k, k, mp - m + k, l - mp - k
                if min(a1, a2, a3, a4) < 0:
                    continue
                tot += ((-1) ** (mp - m + k) * pre / (f(a1) * f(a2) * f(a3) * f(a4))
                        * c ** (2 * l + m - mp - 2 * k) * s ** (mp - m + 2 * k))
            d[mp + l, m + l] = tot
    return d


def wigner_D_complex(l, alpha, beta, gamma):
    ms = np.arange(-l, l + 1)
    d = small_d(l, beta)
    return np.exp(-1j * ms[:, None] * alpha) * d * np.exp(-1j * ms[None, :] * gamma)


def wigner_D_real(l, alpha, beta, gamma):
    """Real-basis D^l for R = Rz(alpha) Ry(beta) Rz(gamma): Y_l(R r) = D Y_l(r)."""
    U = real_basis(l)
    D = U @ np.conj(wigner_D_complex(l, alpha, beta, gamma)) @ U.conj().T
    if np.abs(D.imag).max() > 1e-12:
        raise AssertionError("real Wigner-D has an imaginary part")
    return D.real.copy()


def matrix_to_euler(R):
    """zyz Euler angles of a rotation matrix (generic case sin(beta) != 0)."""
    beta = math.acos(max(-1.0, min(1.0, R[2, 2])))
    alpha = math.atan2(R[1, 2], R[0, 2])
    gamma = math.atan2(R[2, 1], -R[2, 0])
    return alpha, beta, gamma
