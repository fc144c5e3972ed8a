"""Planted mistakes in the oracle must be caught by its pins (CPU only).

Each case patches one plausible error into the oracle (a dropped term, a wrong
sign, a transposed operand, a wrong index) and checks that at least one pin
test fails. Mistakes are planted in the oracle only, on the CPU.
"""

import contextlib

import numpy as np
import pytest

import oracle.cg as cg
import oracle.sh as sh
import oracle.tp as tp
import tests.test_oracle_cg as tcg
import tests.test_oracle_sh as tsh
import tests.test_oracle_tp as ttp


@contextlib.contextmanager
def patched(obj, name, value):
    old = getattr(obj, name)
    setattr(obj, name, value)
    cg._cg_real.cache_clear()
    cg._cg_complex_block.cache_clear()
    try:
        yield
    finally:
        setattr(obj, name, old)
        cg._cg_real.cache_clear()
        cg._cg_complex_block.cache_clear()


def fails(*checks):
    for c in checks:
        try:
            c()
        except AssertionError:
            return True
    return False


CG_PINS = (tcg.test_textbook_table, tcg.test_stretched_closed_form, tcg.test_m0_closed_form,
           tcg.test_1x1_dot_cross_symmetric_traceless, tcg.test_real_blocks_complete,
           lambda: [tcg.test_equivariance_wigner(*t) for t in [(1, 1, 1), (2, 1, 2), (2, 2, 3), (3, 2, 2)]],
           lambda: [tcg.test_harmonic_product_rule(*t) for t in [(1, 1, 2), (2, 2, 2), (3, 1, 2)]])


def test_dropped_racah_term_is_caught():
    orig = cg.cg_complex_exact

    def bad(j1, m1, j2, m2, J, M):
        s, q = orig(j1, m1, j2, m2, J, M)
        if j1 >= 1 and j2 >= 1 and m1 == 0:
            q = q * 0.9  # as if one term of the sum went missing
        return s, q

    with patched(cg, "cg_complex_exact", bad):
        assert fails(*CG_PINS)


def test_wrong_real_basis_sign_is_caught():
    orig = cg.real_basis

    def bad(l):
        U = orig(l)
        if l >= 1:
            U[0] = -U[0]
        return U

    with patched(cg, "real_basis", bad):
        assert fails(*CG_PINS)


def test_transposed_cg_operands_are_caught():
    orig = cg._cg_real.__wrapped__

    def bad(l1, l2, l3):
        if l1 == l2:
            return orig(l1, l2, l3).transpose(1, 0, 2).copy()
        return orig(l1, l2, l3)

    with patched(cg, "cg_real", lambda a, b, c: bad(a, b, c)):
        assert fails(tcg.test_1x1_dot_cross_symmetric_traceless)


def test_sh_sign_error_is_caught():
    orig = sh._norm

    def bad(l, am):
        return -orig(l, am) if (l == 3 and am == 1) else orig(l, am)

    with patched(sh, "_norm", bad):
        assert fails(tsh.test_closed_forms_l_le_3, lambda: tsh.test_equivariance_and_parity(3))


def test_tp_swapped_m_indices_are_caught():
    orig = tp.forward

    def bad(L, x, y, w):
        x = np.asarray(x, np.float64)
        out = orig(L, x, y, w)
        # plant: output components of the first l3 = 2 block reversed in m3
        for p in L.paths:
            if p["l3"] == 2:
                b = L.out_block(out, p)
                b[...] = b[:, ::-1, :].copy()
                break
        return out

    with patched(tp, "forward", bad):
        assert fails(lambda: ttp.test_sparse_equals_dense(False), lambda: ttp.test_o3_equivariance(False))


def test_tp_backward_dropped_path_is_caught():
    orig = tp.backward

    def bad(L, x, y, w, g):
        dx, dy, dw = orig(L, x, y, w, g)
        return dx, dy * 0.999, dw

    with patched(tp, "backward", bad):
        assert fails(lambda: ttp.test_backward_adjoint_identities(False))
