"""Clebsch-Gordan coefficients (oracle; test infrastructure).

The complex coefficients come from Racah's closed formula, evaluated exactly in
rational arithmetic (``fractions.Fraction``) and converted to fp64 only at the
end: each coefficient is +-sqrt(q) with q rational. This is deliberately a
different derivation from the ladder/eigen-equation construction that [E3J]
appendix G.2 describes (the HIP library's planner uses that one), so the two
can be checked against each other.

The real blocks follow [COURSE] 03a (Clebsch-Gordan decomposition of l1 x l2 in
the real basis of the spherical harmonics of lesson 02b):

  C_real[m1, m2, m3] = sum_{M1, M2, M3} conj(U1[m1, M1]) conj(U2[m2, M2])
                        U3[m3, M3] <l1 M1 l2 M2 | l3 M3>

where U_l maps complex harmonics (Condon-Shortley phase) to real ones,
Y_real = U_l Y_complex (see ``real_basis``). The result is purely real or purely
imaginary; its nonzero part is the real block. Each block is orthonormal,
sum_{m1 m2} C[m1,m2,m3] C[m1,m2,m3'] = delta(m3, m3').

Sign reading (the pages fix none; any per-path sign is equally equivariant):
for an even path (l1+l2+l3 even) the block is flipped so that C[0,0,0] > 0;
for an odd path, so that its first entry with |C| > 1e-9 in lexicographic
(m1, m2, m3) order, each m ascending from -l, is positive.
"""

from fractions import Fraction
from functools import lru_cache
import math

import numpy as np


def _fact(n):
    return math.factorial(n)


def cg_complex_exact(j1, m1, j2, m2, J, M):
    """<j1 m1 j2 m2 | J M> as (sign, Fraction q) with value sign*sqrt(q).

    Racah's formula for integer angular momenta:
      delta(M, m1+m2) * sqrt[(2J+1)(J+j1-j2)!(J-j1+j2)!(j1+j2-J)! / (j1+j2+J+1)!]
        * sqrt[(J+M)!(J-M)!(j1-m1)!(j1+m1)!(j2-m2)!(j2+m2)!]
        * sum_k (-1)^k / [k!(j1+j2-J-k)!(j1-m1-k)!(j2+m2-k)!(J-j2+m1+k)!(J-j1-m2+k)!]
    where k runs over every integer making all factorial arguments >= 0.
    """
    if M != m1 + m2:
        return 0, Fraction(0)
    if not (abs(j1 - j2) <= J <= j1 + j2):
        return 0, Fraction(0)
    if abs(m1) > j1 or abs(m2) > j2 or abs(M) > J:
        return 0, Fraction(0)
    pref = Fraction((2 * J + 1) * _fact(J + j1 - j2) * _fact(J - j1 + j2) * _fact(j1 + j2 - J),
                    _fact(j1 + j2 + J + 1))
    pref *= (_fact(J + M) * _fact(J - M) * _fact(j1 - m1) * _fact(j1 + m1)
             * _fact(j2 - m2) * _fact(j2 + m2))
    s = Fraction(0)
    for k in range(0, j1 + j2 - J + 1):
        args = [k, j1 + j2 - J - k, j1 - m1 - k, j2 + m2 - k, J - j2 + m1 + k, J - j1 - m2 + k]
        if min(args) < 0:
            continue
        den = 1
        for a in args:
            den *= _fact(a)
        s += Fraction((-1) ** k, den)
    if s == 0:
        return 0, Fraction(0)
    sign = 1 if s > 0 else -1
    return sign, s * s * pref


def cg_complex(j1, m1, j2, m2, J, M):
    """fp64 value of <j1 m1 j2 m2 | J M> (correctly rounded sqrt of an exact rational)."""
    sign, q = cg_complex_exact(j1, m1, j2, m2, J, M)
    if sign == 0:
        return 0.0
    return sign * math.sqrt(float(q))


def real_basis(l):
    """U_l, complex (2l+1)x(2l+1): rows = real m, columns = complex m, both -l..l.

    Real harmonics in terms of complex ones (Condon-Shortley phase in Y^m):
      m > 0:  (Y^{-m} + (-1)^m Y^{m}) / sqrt2
      m = 0:  Y^0
      m < 0:  i (Y^{m} - (-1)^m Y^{-m}) / sqrt2
    so that Y_real[l, m] is sqrt2 * (-1)^m Re Y^m (m > 0) and
    sqrt2 * (-1)^m Im Y^{|m|} (m < 0): cos(m phi) and sin(|m| phi) types
    without a Condon-Shortley sign, matching ``sh.real_sh``.
    """
    n = 2 * l + 1
    U = np.zeros((n, n), dtype=np.complex128)
    r2 = 1.0 / math.sqrt(2.0)
    for m in range(-l, l + 1):
        if m > 0:
            U[m + l, -m + l] = r2
            U[m + l, m + l] = (-1) ** m * r2
        elif m == 0:
            U[l, l] = 1.0
        else:
            U[m + l, m + l] = 1j * r2
            U[m + l, -m + l] = -1j * (-1) ** m * r2
    return U


@lru_cache(maxsize=None)
def _cg_complex_block(l1, l2, l3):
    C = np.zeros((2 * l1 + 1, 2 * l2 + 1, 2 * l3 + 1))
    for m1 in range(-l1, l1 + 1):
        for m2 in range(-l2, l2 + 1):
            m3 = m1 + m2
            if abs(m3) <= l3:
                C[m1 + l1, m2 + l2, m3 + l3] = cg_complex(l1, m1, l2, m2, l3, m3)
    return C


def cg_complex_block(l1, l2, l3):
    """Dense complex-basis block [2l1+1, 2l2+1, 2l3+1] (copy)."""
    return _cg_complex_block(l1, l2, l3).copy()


def apply_sign_rule(C, l1, l2, l3):
    """Fix the per-path sign as documented in the module docstring."""
    if (l1 + l2 + l3) % 2 == 0:
        ref = C[l1, l2, l3]
        if ref == 0.0:
            raise AssertionError("even path with C[0,0,0] == 0")
        return C if ref > 0 else -C
    for v in C.reshape(-1):  # C-order == lexicographic (m1, m2, m3)
        if abs(v) > 1e-9:
            return C if v > 0 else -C
    raise AssertionError("empty CG block")


@lru_cache(maxsize=None)
def _cg_real(l1, l2, l3):
    if not (abs(l1 - l2) <= l3 <= l1 + l2):
        raise ValueError("triangle rule violated: %d %d %d" % (l1, l2, l3))
    Cc = _cg_complex_block(l1, l2, l3)
    U1, U2, U3 = real_basis(l1), real_basis(l2), real_basis(l3)
    X = np.einsum("aA,bB,cC,ABC->abc", U1.conj(), U2.conj(), U3, Cc)
    re, im = np.abs(X.real).max(), np.abs(X.imag).max()
    if re >= im:
        if im > 1e-13:
            raise AssertionError("real CG block not purely real")
        C = X.real.copy()
    else:
        if re > 1e-13:
            raise AssertionError("real CG block not purely imaginary")
        C = X.imag.copy()
    C[np.abs(C) < 1e-15] = 0.0
    C = apply_sign_rule(C, l1, l2, l3)
    # orthonormal columns: sum over (m1, m2) of C[.,.,m3] C[.,.,m3'] = delta
    G = np.einsum("abc,abd->cd", C, C)
    if np.abs(G - np.eye(2 * l3 + 1)).max() > 1e-12:
        raise AssertionError("real CG block not orthonormal")
    return C


def cg_real(l1, l2, l3):
    """Real-basis CG block [2l1+1, 2l2+1, 2l3+1], fp64, with the sign rule."""
    return _cg_real(l1, l2, l3).copy()
