"""Host-side checks of libcgtp (CPU only, no compute calls).

* the library loads and exports every function include/cgtp.h declares;
* the planner's CG blocks (ladder construction) equal the oracle's (Racah);
* path tables and row sizes equal the oracle's enumeration;
* malformed or unsupported plans return the documented status codes;
* parity-selected and collapsed plans list the oracle's paths and output blocks.
"""

import os
import re

import numpy as np
import pytest

from oracle import cg as ocg
from oracle.irreps import Layout

cgtp = pytest.importorskip("clebsch_gordan_tensor_amd.cgtp")

HEADER = os.path.join(os.path.dirname(os.path.dirname(__file__)), "include", "cgtp.h")


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(cgtp_[a-z_]+)\s*\(", text)))


def test_every_declared_symbol_is_exported():
    names = declared_functions()
    assert len(names) == 35
    for n in names:
        assert hasattr(cgtp._lib, n), n
    assert sorted(cgtp.EXPORTED) == names


def all_triples(lmax=4):
    for l1 in range(lmax + 1):
        for l2 in range(lmax + 1):
            for l3 in range(abs(l1 - l2), l1 + l2 + 1):
                if l3 <= lmax:
                    yield l1, l2, l3


@pytest.mark.parametrize("l1,l2,l3", list(all_triples()))
def test_planner_cg_equals_oracle(l1, l2, l3):
    par = lambda l: "e" if l % 2 == 0 else "o"
    p3 = "e" if (l1 + l2) % 2 == 0 else "o"
    plan = cgtp.Plan("1x%d%s" % (l1, par(l1)), "1x%d%s" % (l2, par(l2)), "%d%s" % (l3, p3))
    assert plan.num_paths == 1
    assert np.abs(plan.cg(0) - ocg.cg_real(l1, l2, l3)).max() < 1e-13


CASES = [
    ("32x0e+32x1o+32x2e", "0e+1o+2e", "0e+0o+1e+1o+2e+2o"),
    ("128x0e+128x1o+128x2e+128x3o", "0e+1o+2e+3o", "0e+0o+1e+1o+2e+2o+3e+3o"),
    ("64x0e+64x1o+64x2e+64x3o+64x4e", "0e+1o+2e+3o+4e", "0e+0o+1e+1o+2e+2o+3e+3o+4e+4o"),
    ("8x1o+4x0e+3x2o", "1o+0e", "0e+1o+2e"),          # mixed multiplicities, natural parity only
    ("5x2e", "1o+1e", "1e+1o+2e+3o+3e"),                # repeated degree in y
    ("2x1o", "2e", "1o+3o+2e"),
]


@pytest.mark.parametrize("ix,iy,io", CASES)
def test_paths_and_sizes_equal_oracle(ix, iy, io):
    L = Layout(ix, iy, io)
    plan = cgtp.Plan(ix, iy, io)
    assert (plan.dim_x, plan.dim_y, plan.dim_out, plan.num_paths, plan.w_numel) == (
        L.dim_x, L.dim_y, L.dim_out, len(L.paths), L.w_numel)
    ref = np.array([[p["i1"], p["i2"], p["l1"], p["l2"], p["l3"], p["p3"]] for p in L.paths])
    assert np.array_equal(plan.paths(), ref)
    for k, p in enumerate(L.paths):
        assert np.abs(plan.cg(k) - ocg.cg_real(p["l1"], p["l2"], p["l3"])).max() < 1e-13


def status_of(fn):
    with pytest.raises(cgtp.CgtpError) as e:
        fn()
    return e.value.status


def test_error_codes():
    ERR_INVALID, ERR_PARSE, ERR_UNSUPPORTED = 1, 2, 3
    assert status_of(lambda: cgtp.Plan("3x", "0e", "0e")) == ERR_PARSE
    assert status_of(lambda: cgtp.Plan("1x1q", "0e", "0e")) == ERR_PARSE
    assert status_of(lambda: cgtp.Plan("1e++1o", "0e", "0e")) == ERR_PARSE
    assert status_of(lambda: cgtp.Plan("0x1e", "0e", "1e")) == ERR_PARSE
    assert status_of(lambda: cgtp.Plan("4x1o", "1o", "4x0e", mode="uvw")) == ERR_UNSUPPORTED  # per-row uvw
    assert status_of(lambda: cgtp.Plan("1x1o", "1o", "0e", mode="uvx")) == ERR_UNSUPPORTED
    assert status_of(lambda: cgtp.Plan("1x5o", "0e", "5o")) == ERR_UNSUPPORTED
    assert status_of(lambda: cgtp.Plan("1x1o", "2x1o", "0e", collapse=True)) == ERR_UNSUPPORTED
    assert status_of(lambda: cgtp.Plan("1x1o", "1o", "1o")) == ERR_UNSUPPORTED  # no path survives
    p = cgtp.Plan("1x1o", "1o", "0e")
    buf = np.zeros(27)
    assert cgtp._lib.cgtp_plan_cg(p._h, 5, buf.ctypes.data_as(cgtp.ctypes.POINTER(cgtp.ctypes.c_double))) == ERR_INVALID
    assert cgtp._lib.cgtp_plan_create(None, None, None, None, 0, 0, None) == ERR_INVALID
    assert cgtp._lib.cgtp_tp_forward(None, 1, None, None, None, None, None) == ERR_INVALID
    assert cgtp._lib.cgtp_sh_forward(5, 0, 1, None, None, None) == ERR_UNSUPPORTED
    assert cgtp._lib.cgtp_sh_forward(2, 7, 1, None, None, None) == ERR_INVALID
    assert cgtp._lib.cgtp_sh_forward(5, 0, 1, None, None, None) == ERR_UNSUPPORTED
    assert "lmax" in cgtp._lib.cgtp_last_error().decode()


def test_workspace_sizes():
    ps = cgtp.Plan("32x0e+32x1o+32x2e", "0e+1o+2e", "0e+0o+1e+1o+2e+2o", wkind="shared")
    pr = cgtp.Plan("32x0e+32x1o+32x2e", "0e+1o+2e", "0e+0o+1e+1o+2e+2o", wkind="per_row")
    assert pr.workspace_size(cgtp.OP_TP_BACKWARD, 4096) == 0
    # per-row partials + one partial per 256-row chunk, fp32
    assert ps.workspace_size(cgtp.OP_TP_BACKWARD, 4096) == (4096 + 16) * 480 * 4
    assert ps.workspace_size(cgtp.OP_TP_BACKWARD, 0) == 0


# ------------------------------------------------------------ linear map plans

@pytest.mark.parametrize("ii,io", [("2x1o+3x1o+1x0e+2x2e", "4x1o+2x0e+1x2o+3x2e"),
                                   ("128x0e+128x1o+128x2e+128x3o", "128x0e+128x1o+128x2e+128x3o"),
                                   ("7x0e", "3x0o")])
def test_linear_paths_equal_oracle(ii, io):
    from oracle.linear import LinearLayout
    lin = cgtp.Linear(ii, io)
    LL = LinearLayout(ii, io)
    assert (lin.dim_in, lin.dim_out, lin.num_paths, lin.w_numel) == (LL.dim_in, LL.dim_out, len(LL.paths), LL.w_numel)
    want = [[p["i"], p["o"], p["l"], p["mu"], p["mv"]] for p in LL.paths]
    assert lin.paths().tolist() == want


def test_linear_errors():
    ERR_INVALID, ERR_PARSE, ERR_UNSUPPORTED = 1, 2, 3
    assert status_of(lambda: cgtp.Linear("2x1q", "1x1o")) == ERR_PARSE
    assert status_of(lambda: cgtp.Linear("2x1o", "1x1o", dtype="f64")) == ERR_UNSUPPORTED
    assert cgtp._lib.cgtp_linear_create(None, None, 0, None) == ERR_INVALID
    lin = cgtp.Linear("4x0e+2x1o", "3x0e")
    assert lin.workspace_size(0) == 0
    assert lin.workspace_size(1000) == 12 * 4          # one row chunk of partials
    assert lin.workspace_size(10 ** 6) > 0


@pytest.mark.parametrize("select", ["all", "symmetric", "skew"])
@pytest.mark.parametrize("collapse", [False, True])
@pytest.mark.parametrize("ix,iy,io", [
    ("2x0e+2x1o+2x2e+2x3o", "0e+1o+2e+3o", "0e+0o+1e+1o+2e+2o+3e+3o"),
    ("64x0e+64x1o+64x2e+64x3o+64x4e", "0e+1o+2e+3o+4e", "0e+0o+1e+1o+2e+2o+3e+3o+4e+4o"),
    ("4x0e+6x1e", "0e", "1e+0e"),                                  # groups in irreps_out order
])
def test_variant_plans_equal_oracle(ix, iy, io, select, collapse):
    L = Layout(ix, iy, io, select, collapse)
    if not L.paths:
        with pytest.raises(cgtp.CgtpError):
            cgtp.Plan(ix, iy, io, select=select, collapse=collapse)
        return
    plan = cgtp.Plan(ix, iy, io, select=select, collapse=collapse)
    assert (plan.dim_out, plan.num_paths, plan.w_numel) == (L.dim_out, len(L.paths), L.w_numel)
    want = [(p["i1"], p["i2"], p["l1"], p["l2"], p["l3"], p["p3"]) for p in L.paths]
    assert [tuple(r) for r in plan.paths()] == want
    assert [tuple(r) for r in plan.outputs()] == [(g["l3"], g["p3"], g["mul"], g["out_off"]) for g in L.groups]


def test_variant_plan_errors():
    bad = ctypes_plan_ex("2x0e+3x1o", "0e+1o", "0e+1o", 0, 1)      # 0e fed by 2x and 3x blocks
    assert bad == 3
    assert ctypes_plan_ex("2x0e", "0e", "0e", 7, 0) == 1              # no such selection
    assert ctypes_plan_ex("2x1o", "1o", "1e", 1, 0) == 3              # the only path is skew
    assert ctypes_plan_ex("2x1o", "1o", "1e", 2, 1) == 0


def ctypes_plan_ex(ix, iy, io, select, collapse):
    import ctypes
    h = ctypes.c_void_p()
    st = cgtp._lib.cgtp_plan_create_ex(ix.encode(), iy.encode(), io.encode(), b"uvu", 0, 1, select, collapse,
                                       ctypes.byref(h))
    if st == 0:
        cgtp._lib.cgtp_plan_destroy(h)
    return st


# ------------------------------------------------------- connection modes

@pytest.mark.parametrize("ix,iy,io,mode,wkind,collapse", [
    ("4x0e+4x1o+8x2e", "0e+1o+2e", "8x0e+4x0o+12x1e+4x1o+8x2e+4x2o", "uvw", "shared", False),
    ("4x0e+4x1o+8x2e", "0e+1o+2e", "8x0e+4x0o+12x1e+4x1o+8x2e+4x2o", "uvw", "shared", True),
    ("128x0e+128x1o+128x2e+128x3o", "0e+1o+2e+3o", "128x0e+128x0o+128x1e+128x1o+128x2e+128x2o+128x3e+128x3o",
     "uvw", "shared", True),
    ("3x0e+5x1o+2x2e", "2x0e+3x1o+1x2e", "0e+0o+1e+1o+2e+2o", "uvu", "per_row", False),
    ("3x0e+5x1o+2x2e", "2x0e+3x1o+1x2e", "0e+0o+1e+1o+2e+2o", "uvu", "shared", False),
])
def test_mode_plans_equal_oracle(ix, iy, io, mode, wkind, collapse):
    from oracle.modes import ModeLayout
    p = cgtp.Plan(ix, iy, io, mode=mode, wkind=wkind, collapse=collapse)
    ML = ModeLayout(ix, iy, io, mode, collapse=collapse)
    assert (p.dim_x, p.dim_y, p.dim_out, p.num_paths, p.w_numel) == (ML.dim_x, ML.dim_y, ML.dim_out, len(ML.paths),
                                                                      ML.w_numel)
    assert p.paths().tolist() == [[q["i1"], q["i2"], q["l1"], q["l2"], q["l3"], q["p3"]] for q in ML.paths]
    assert p.outputs().tolist() == [[g["l3"], g["p3"], g["mul"], g["out_off"]] for g in ML.groups]


def test_mode_errors():
    ERR_UNSUPPORTED, ERR_WORKSPACE = 3, 5
    full = ("4x0e+4x1o", "0e+1o", "4x0e+4x1o+4x1e")
    assert status_of(lambda: cgtp.Plan(*full, mode="uvw", wkind="shared", dtype="f64")) == ERR_UNSUPPORTED
    assert status_of(lambda: cgtp.Plan("4x0e", "2x0e", "4x0e", mode="uvw", wkind="shared")) == ERR_UNSUPPORTED
    assert status_of(lambda: cgtp.Plan("3x0e", "0e", "4x0e", mode="uvw", wkind="shared")) == ERR_UNSUPPORTED
    assert status_of(lambda: cgtp.Plan("4x0e", "0e", "3x0e", mode="uvw", wkind="shared")) == ERR_UNSUPPORTED
    # uvw and y multiplicities > 1 run the tensor product only: the convolution,
    # the double backward and the allocation-free backward refuse them
    pw = cgtp.Plan(*full, mode="uvw", wkind="shared")
    pv = cgtp.Plan("4x0e+4x1o", "2x0e+2x1o", "0e+1o+1e", wkind="per_row")
    for p in (pw, pv):
        assert cgtp._lib.cgtp_conv_forward(p._h, None, None, None, None, 1.0, None, None) in (1, ERR_UNSUPPORTED)
        assert cgtp._lib.cgtp_tp_double_backward(p._h, 0, *([None] * 12), 0, None) == ERR_UNSUPPORTED
        assert cgtp._lib.cgtp_tp_backward_noalloc(p._h, 1, *([None] * 8)) in (1, ERR_UNSUPPORTED)
    # workspaces: uvw holds the path outputs and their cotangent (plus grad_W
    # partials); uvu with v > 1 the per-path grad of the mixed y
    assert pw.workspace_size(cgtp.OP_TP_BACKWARD, 1000) >= 2 * 1000 * (4 * 1 + 4 * 3 + 4 * 3 + 4 * 1 + 4 * 3) * 4
    assert pv.workspace_size(cgtp.OP_TP_BACKWARD, 100) >= 100 * (4 * 1 + 4 * 3 + 4 * 3 + 4 * 1 + 4 * 3) * 4
