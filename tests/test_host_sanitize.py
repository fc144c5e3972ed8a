"""The host planner built with AddressSanitizer and UndefinedBehaviorSanitizer
(CPU only, no device).

tests/host/plan_sanitize.cpp links the planner (csrc/plan.cpp) into a small
driver built with g++ -fsanitize=address,undefined; each case builds a plan in
every dtype and weight kind from an irreps triple, and the run must end with
no sanitizer report. Valid plans must give the oracle's row sizes and path
count (oracle/modes.py ModeLayout); malformed or unsupported requests the
status codes include/cgtp.h documents.
"""

import os
import shutil
import subprocess

import pytest

from oracle.modes import ModeLayout

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "clebsch_gordan_tensor_amd", "csrc")
ROCM = os.environ.get("ROCM_PATH", "/opt/rocm")

F32, F64, BF16 = 0, 1, 2
SHARED, PER_ROW = 0, 1
PARSE, UNSUPPORTED, INVALID_ARG = 2, 3, 1
SEL = {"all": 0, "symmetric": 1, "skew": 2}


@pytest.fixture(scope="module")
def driver(tmp_path_factory):
    gxx = shutil.which("g++")
    if gxx is None or not os.path.exists(os.path.join(ROCM, "include", "hip", "hip_runtime_api.h")):
        pytest.skip("g++ or the ROCm headers are missing")
    exe = str(tmp_path_factory.mktemp("asan") / "plan_sanitize")
    cmd = [gxx, "-std=c++17", "-O1", "-g", "-fno-omit-frame-pointer", "-fsanitize=address,undefined",
           "-fno-sanitize-recover=undefined", "-D__HIP_PLATFORM_AMD__", "-I" + os.path.join(ROCM, "include"),
           "-I" + os.path.join(ROOT, "include"), "-I" + CSRC, os.path.join(CSRC, "plan.cpp"),
           os.path.join(ROOT, "tests", "host", "plan_sanitize.cpp"), "-L" + os.path.join(ROCM, "lib"),
           "-lamdhip64", "-Wl,-rpath," + os.path.join(ROCM, "lib"), "-o", exe]
    r = subprocess.run(cmd, capture_output=True, text=True, timeout=300)
    assert r.returncode == 0, r.stderr[-4000:]
    return exe


def run(exe, cases):
    """Run the driver over (x, y, out, mode, select, collapse) cases; returns
    one list of 6 result lines (3 dtypes x 2 weight kinds) per case."""
    args = []
    for x, y, o, mode, sel, col in cases:
        args += [x, y, o, "%s/%d/%d" % (mode, SEL.get(sel, sel), int(col))]
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=0:exitcode=23",
               UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1")
    r = subprocess.run([exe] + args, capture_output=True, text=True, timeout=300, env=env)
    assert r.returncode == 0, (r.returncode, r.stderr[-4000:])
    assert "Sanitizer" not in r.stderr and "runtime error" not in r.stderr, r.stderr[-4000:]
    lines = r.stdout.split("\n")[:-1]
    assert len(lines) == 6 * len(cases)
    return [lines[6 * i:6 * i + 6] for i in range(len(cases))]


def expect_ok(line, dt, wk, L):
    assert line == "ok %d %d %d %d %d %d %d" % (dt, wk, L.dim_x, L.dim_y, L.dim_out, L.w_numel, len(L.paths))


VALID_UVU = [
    ("128x0e+128x1o+128x2e+128x3o", "0e+1o+2e+3o", "0e+0o+1e+1o+2e+2o+3e+3o", "all", False),
    ("64x0e+64x1o+64x2e+64x3o+64x4e", "0e+1o+2e+3o+4e", "0e+1o+2e+3o+4e+0o+1e+2o+3e+4o", "skew", True),
    ("64x0e+64x1o+64x2e+64x3o+64x4e", "0e+1o+2e+3o+4e", "0e+1o+2e+3o+4e+0o+1e+2o+3e+4o", "symmetric", False),
    ("32x0e+32x1o", "4x0e+4x1o+4x2e", "0e+1o+2e", "all", False),            # y multiplicity 4
    ("  2x1o + 3x0e ", "1o", "1e+0e+2e", "all", False),                       # whitespace, default multiplicity
    ("1x0e", "0e", "0e", "all", True),
    ("65536x0e", "0e+1o", "0e+1o+1e", "all", False),                          # wide channel block
    ("16x1o+16x1o+8x2e", "1o+1o", "0e+1e+2e+3e+1o+2o", "all", True),          # repeated blocks summed
]


def test_valid_uvu_plans_match_the_oracle_layout(driver):
    cases = [(x, y, o, "uvu", s, c) for x, y, o, s, c in VALID_UVU]
    for (x, y, o, _, s, c), lines in zip(cases, run(driver, cases)):
        L = ModeLayout(x, y, o, "uvu", s, c)
        assert L.paths
        i = 0
        for dt in (F32, F64, BF16):
            for wk in (SHARED, PER_ROW):
                expect_ok(lines[i], dt, wk, L)
                i += 1


def test_uvw_plans_within_and_outside_their_limits(driver):
    cases = [
        ("128x0e+128x1o", "0e+1o+2e+3o", "128x0e+128x0o+128x1e+128x1o", "uvw", "symmetric", True),
        ("16x0e+16x1o", "0e+1o+2e", "32x0e+32x1o+16x2e", "uvw", "all", False),
        ("6x0e", "0e", "4x0e", "uvw", "all", False),               # multiplicity not a multiple of 4
        ("16x0e", "2x0e", "16x0e", "uvw", "all", False),           # y multiplicity 2
    ]
    res = run(driver, cases)
    for case, lines in zip(cases[:2], res[:2]):
        L = ModeLayout(*case)
        # shared weights, fp32 or bf16 storage only
        expect_ok(lines[0], F32, SHARED, L)
        expect_ok(lines[4], BF16, SHARED, L)
        assert [lines[j] for j in (1, 2, 3, 5)] == ["err 0 1 3", "err 1 0 3", "err 1 1 3", "err 2 1 3"]
    for lines in res[2:]:
        assert all(ln.startswith("err ") and ln.endswith(" 3") for ln in lines)


ERRORS = [
    # (x, y, out, mode, select, collapse, status)
    ("bad", "0e", "0e", "uvu", "all", False, PARSE),
    ("2x", "0e+1o", "0e+1o+1e", "uvu", "all", False, PARSE),
    ("x0e", "0e+1o", "0e+1o+1e", "uvu", "all", False, PARSE),
    ("0q", "0e+1o", "0e+1o+1e", "uvu", "all", False, PARSE),
    ("1e+", "0e+1o", "0e+1o+1e", "uvu", "all", False, PARSE),
    ("+", "0e+1o", "0e+1o+1e", "uvu", "all", False, PARSE),
    ("3x-1e", "0e+1o", "0e+1o+1e", "uvu", "all", False, PARSE),
    ("0e++1o", "0e+1o", "0e+1o+1e", "uvu", "all", False, PARSE),
    ("0x0e", "0e+1o", "0e+1o+1e", "uvu", "all", False, PARSE),
    ("-2x1o", "0e+1o", "0e+1o+1e", "uvu", "all", False, PARSE),
    ("1.5x0e", "0e+1o", "0e+1o+1e", "uvu", "all", False, PARSE),
    ("2x1o2", "0e+1o", "0e+1o+1e", "uvu", "all", False, PARSE),
    ("1xe", "0e+1o", "0e+1o+1e", "uvu", "all", False, PARSE),
    ("2147483648x0e", "0e+1o", "0e+1o+1e", "uvu", "all", False, PARSE),   # multiplicity past int32
    ("99999999999999999999x0e", "0e", "0e", "uvu", "all", False, PARSE),
    ("0e", "0e", "1e+" * 5000 + "1e", "uvu", "all", False, UNSUPPORTED),    # long string, no path
    ("1x5e", "0e", "5e", "uvu", "all", False, UNSUPPORTED),                 # l above the compiled maximum
    ("10e", "0e+1o", "0e+1o+1e", "uvu", "all", False, UNSUPPORTED),
    ("", "", "", "uvu", "all", False, UNSUPPORTED),                         # no path at all
    ("0e", "0e", "1o", "uvu", "skew", False, UNSUPPORTED),
    ("1o", "1e+0e+2e", "1o", "uvx", "all", False, UNSUPPORTED),             # unknown mode
    ("2x0e", "0e", "0e", "uvu", 7, False, INVALID_ARG),                     # bad selection
    ("16x0e+32x1o", "0e+1o", "0e+1o", "uvu", "all", True, UNSUPPORTED),     # collapse over unequal multiplicities
    ("32x0e+32x1o", "4x0e+4x1o", "0e+1o", "uvu", "all", True, UNSUPPORTED),  # collapse with y multiplicity 4
]


def test_malformed_and_unsupported_requests(driver):
    cases = [c[:6] for c in ERRORS]
    for c, lines in zip(ERRORS, run(driver, cases)):
        want = ["err %d %d %d" % (dt, wk, c[6]) for dt in (F32, F64, BF16) for wk in (SHARED, PER_ROW)]
        assert lines == want, c
    with pytest.raises(ValueError):  # the oracle refuses the unequal collapse too
        ModeLayout("16x0e+32x1o", "0e+1o", "0e+1o", "uvu", "all", True)
