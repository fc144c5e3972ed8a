"""Pins of the oracle's Clebsch-Gordan coefficients (CPU only).

Nothing here re-types the oracle's formulas: the checks are textbook tables,
independent closed forms (stretched states, J = 0, the m = 0 3j symbol),
orthonormality/completeness, the 1 x 1 = dot / cross / symmetric-traceless
decomposition ([COURSE] 03a), equivariance under independently built Wigner-D
matrices ([COURSE] 01b), the harmonic product rule and a null-space derivation.
"""

import math
import os

import numpy as np
import pytest

from oracle import cg, sh, wigner

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "cg_complex_textbook.txt")
LMAX = 4


def all_triples(lmax=LMAX):
    for l1 in range(lmax + 1):
        for l2 in range(lmax + 1):
            for l3 in range(abs(l1 - l2), l1 + l2 + 1):
                yield l1, l2, l3


def test_textbook_table():
    n = 0
    for line in open(GOLDEN):
        if line.startswith("#") or not line.strip():
            continue
        j1, m1, j2, m2, J, M, s, num, den = map(int, line.split())
        assert cg.cg_complex(j1, m1, j2, m2, J, M) == pytest.approx(s * math.sqrt(num / den), abs=1e-15)
        n += 1
    assert n == 33


def _binom(n, k):
    return math.comb(n, k)


def test_stretched_closed_form():
    # <j1 m1 j2 m2 | j1+j2, m1+m2> = sqrt(C(2j1, j1+m1) C(2j2, j2+m2) / C(2J, J+M))
    for j1 in range(5):
        for j2 in range(5):
            J = j1 + j2
            for m1 in range(-j1, j1 + 1):
                for m2 in range(-j2, j2 + 1):
                    M = m1 + m2
                    ref = math.sqrt(_binom(2 * j1, j1 + m1) * _binom(2 * j2, j2 + m2) / _binom(2 * J, J + M))
                    assert abs(cg.cg_complex(j1, m1, j2, m2, J, M) - ref) < 1e-14


def test_singlet_closed_form():
    # <j m j -m | 0 0> = (-1)^(j-m) / sqrt(2j+1)
    for j in range(6):
        for m in range(-j, j + 1):
            ref = (-1) ** (j - m) / math.sqrt(2 * j + 1)
            assert abs(cg.cg_complex(j, m, j, -m, 0, 0) - ref) < 1e-14


def threej_000(l1, l2, l3):
    """(l1 l2 l3; 0 0 0) closed form for even l1+l2+l3 = 2g."""
    g2 = l1 + l2 + l3
    if g2 % 2:
        return 0.0
    g = g2 // 2
    f = math.factorial
    return ((-1) ** g * math.sqrt(f(2 * g - 2 * l1) * f(2 * g - 2 * l2) * f(2 * g - 2 * l3) / f(2 * g + 1))
            * f(g) / (f(g - l1) * f(g - l2) * f(g - l3)))


def test_m0_closed_form():
    # <l1 0 l2 0 | l3 0> = (-1)^(l1-l2) sqrt(2 l3 + 1) (l1 l2 l3; 0 0 0)
    for l1, l2, l3 in all_triples(6):
        ref = (-1) ** (l1 - l2) * math.sqrt(2 * l3 + 1) * threej_000(l1, l2, l3)
        assert abs(cg.cg_complex(l1, 0, l2, 0, l3, 0) - ref) < 1e-14


@pytest.mark.parametrize("l1,l2,l3", list(all_triples()))
def test_real_block_orthonormal_and_sign(l1, l2, l3):
    C = cg.cg_real(l1, l2, l3)
    G = np.einsum("abc,abd->cd", C, C)
    assert np.abs(G - np.eye(2 * l3 + 1)).max() < 1e-13
    if (l1 + l2 + l3) % 2 == 0:
        assert C[l1, l2, l3] > 0
    else:
        first = C.reshape(-1)[np.abs(C.reshape(-1)) > 1e-9][0]
        assert first > 0


def test_real_blocks_complete():
    # Over all l3 the blocks form an orthogonal change of basis of l1 (x) l2.
    for l1 in range(LMAX + 1):
        for l2 in range(LMAX + 1):
            n = (2 * l1 + 1) * (2 * l2 + 1)
            Q = np.concatenate([cg.cg_real(l1, l2, l3).reshape(n, -1)
                                for l3 in range(abs(l1 - l2), l1 + l2 + 1)], axis=1)
            assert Q.shape == (n, n)
            assert np.abs(Q @ Q.T - np.eye(n)).max() < 1e-13


def _yzx(v):
    """Real l = 1 components (m = -1, 0, 1) of a Cartesian vector: (y, z, x)."""
    return np.array([v[1], v[2], v[0]])


def test_1x1_dot_cross_symmetric_traceless():
    rng = np.random.default_rng(1)
    a, b = rng.standard_normal(3), rng.standard_normal(3)
    A, B = _yzx(a), _yzx(b)
    out0 = np.einsum("abc,a,b->c", cg.cg_real(1, 1, 0), A, B)
    out1 = np.einsum("abc,a,b->c", cg.cg_real(1, 1, 1), A, B)
    out2 = np.einsum("abc,a,b->c", cg.cg_real(1, 1, 2), A, B)
    assert out0[0] == pytest.approx(a @ b / math.sqrt(3), abs=1e-14)
    assert np.abs(out1 - _yzx(np.cross(a, b)) / math.sqrt(2)).max() < 1e-14
    S = 0.5 * (np.outer(a, b) + np.outer(b, a))
    S -= np.trace(S) / 3 * np.eye(3)
    # orthonormal symmetric-traceless basis in the m = -2..2 order of the harmonics
    ref = np.array([math.sqrt(2) * S[0, 1], math.sqrt(2) * S[1, 2],
                    (2 * S[2, 2] - S[0, 0] - S[1, 1]) / math.sqrt(6),
                    math.sqrt(2) * S[0, 2], (S[0, 0] - S[1, 1]) / math.sqrt(2)])
    assert np.abs(out2 - ref).max() < 1e-14
    assert np.linalg.norm(out2) == pytest.approx(np.linalg.norm(S), abs=1e-14)


def test_scalar_paths_are_identities():
    for l in range(LMAX + 1):
        n = 2 * l + 1
        assert np.abs(cg.cg_real(0, l, l)[0] - np.eye(n)).max() < 1e-15
        assert np.abs(cg.cg_real(l, 0, l)[:, 0, :] - np.eye(n)).max() < 1e-15


@pytest.mark.parametrize("l1,l2,l3", list(all_triples()))
def test_equivariance_wigner(l1, l2, l3):
    rng = np.random.default_rng(100 + 25 * l1 + 5 * l2 + l3)
    ang = wigner.random_euler(rng)
    D1, D2, D3 = (wigner.wigner_D_real(l, *ang) for l in (l1, l2, l3))
    C = cg.cg_real(l1, l2, l3)
    a, b = rng.standard_normal(2 * l1 + 1), rng.standard_normal(2 * l2 + 1)
    lhs = np.einsum("abc,a,b->c", C, D1 @ a, D2 @ b)
    rhs = D3 @ np.einsum("abc,a,b->c", C, a, b)
    assert np.abs(lhs - rhs).max() < 1e-12


@pytest.mark.parametrize("l1,l2,l3", list(all_triples()))
def test_harmonic_product_rule(l1, l2, l3):
    # (Y_l1 (x) Y_l2)_l3 = sqrt((2l1+1)(2l2+1)/(2l3+1)) |<l1 0 l2 0|l3 0>| Y_l3 on even
    # paths; odd paths vanish (an equivariant polynomial of parity (-1)^(l1+l2)
    # cannot transform as Y_l3 when l1+l2+l3 is odd).
    rng = np.random.default_rng(7)
    v = rng.standard_normal((6, 3))
    L = max(l1, l2, l3)
    Y = sh.real_sh(L, v)
    blk = lambda l: Y[:, l * l:(l + 1) ** 2]
    prod = np.einsum("abc,na,nb->nc", cg.cg_real(l1, l2, l3), blk(l1), blk(l2))
    if (l1 + l2 + l3) % 2:
        assert np.abs(prod).max() < 1e-12
    else:
        k = math.sqrt((2 * l1 + 1) * (2 * l2 + 1) / (2 * l3 + 1)) * abs(
            math.sqrt(2 * l3 + 1) * threej_000(l1, l2, l3))
        assert np.abs(prod - k * blk(l3)).max() < 1e-12


@pytest.mark.parametrize("l1,l2,l3", [(1, 1, 1), (2, 1, 2), (2, 2, 2), (3, 2, 1), (3, 3, 3), (4, 2, 3)])
def test_nullspace_derivation(l1, l2, l3):
    # Third derivation: the equivariant maps l1 x l2 -> l3 are the null space of
    # (D1 (x) D2 (x) D3 - I) over a few random rotations (Schur: dimension one).
    rng = np.random.default_rng(3)
    n = (2 * l1 + 1) * (2 * l2 + 1) * (2 * l3 + 1)
    rows = []
    for _ in range(3):
        ang = wigner.random_euler(rng)
        D = [wigner.wigner_D_real(l, *ang) for l in (l1, l2, l3)]
        rows.append(np.kron(np.kron(D[0], D[1]), D[2]) - np.eye(n))
    _, s, Vt = np.linalg.svd(np.concatenate(rows))
    assert s[-1] < 1e-10 and s[-2] > 1e-3
    v = Vt[-1].reshape(2 * l1 + 1, 2 * l2 + 1, 2 * l3 + 1)
    C = cg.cg_real(l1, l2, l3)
    v *= math.sqrt(2 * l3 + 1) / np.linalg.norm(v)
    v *= np.sign(np.sum(v * C))
    assert np.abs(v - C).max() < 1e-10
