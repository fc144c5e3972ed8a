"""GPU parity of the harmonics kernels and the graph preparation.

Harmonics: values and vector-Jacobian products against the oracle, fp32/fp64/
bf16, lmax 0..4, including the zero vector and unnormalised inputs.
Graph: CSR by destination and its transpose must equal the oracle's stable
lexicographic sorts bit for bit; invalid arrays return CGTP_ERR_INDEX.
"""

import numpy as np
import pytest

from oracle import graph as ograph
from oracle import sh as osh
from clebsch_gordan_tensor_amd import synth
from tests.gpu_util import TOL, dev, host, rel_err

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
if not torch.cuda.is_available():
    pytest.skip("no GPU", allow_module_level=True)
cgtp = pytest.importorskip("clebsch_gordan_tensor_amd.cgtp")


@pytest.mark.parametrize("dtype", ["f32", "f64", "bf16"])
@pytest.mark.parametrize("lmax", [0, 1, 2, 3, 4])
def test_sh_forward_backward(dtype, lmax):
    rng = np.random.default_rng(lmax)
    v = rng.standard_normal((5003, 3)) * rng.uniform(0.1, 7.0, (5003, 1))
    v[17] = 0.0
    vd = dev(v, dtype)
    hv = host(vd)
    Y = cgtp.sh_forward(lmax, vd)
    g = dev(rng.standard_normal((5003, (lmax + 1) ** 2)), dtype)
    gv = cgtp.sh_backward(lmax, vd, g)
    torch.cuda.synchronize()
    refY = osh.real_sh(lmax, hv)
    refg = osh.real_sh_grad(lmax, hv, host(g))
    for l in range(lmax + 1):
        assert rel_err(host(Y)[:, l * l:(l + 1) ** 2], refY[:, l * l:(l + 1) ** 2]) <= TOL[dtype]
    # The gradient scales like 1/|v|; times |v| it is the gradient on the unit
    # sphere, compared like every other tensor (max error over max value).
    r = np.linalg.norm(hv, axis=1, keepdims=True)
    assert rel_err(host(gv) * r, refg * r) <= TOL[dtype]
    assert float(host(Y)[17, 0]) == 1.0 and np.all(host(Y)[17, 1:] == 0) and np.all(host(gv)[17] == 0)


def to_dev_i32(a):
    return torch.from_numpy(np.ascontiguousarray(a, np.int32)).cuda()


@pytest.mark.parametrize("N,E,seed", [(1, 5, 0), (500, 10000, 1), (3, 0, 2), (7000, 200000, 3)])
def test_csr_from_coo_bit_exact(N, E, seed):
    rng = np.random.default_rng(seed)
    src = rng.integers(0, N, E)
    dst = rng.integers(0, N, E)  # duplicates and self-loops included: ties keep input order
    row_ptr, s, perm = cgtp.csr_from_coo(N, to_dev_i32(src), to_dev_i32(dst))
    r_row, r_s, r_perm = ograph.csr_from_coo(N, src, dst)
    assert np.array_equal(row_ptr.cpu().numpy(), r_row)
    assert np.array_equal(s.cpu().numpy(), r_s)
    assert np.array_equal(perm.cpu().numpy(), r_perm)
    g = cgtp.Graph(N, row_ptr, s)
    col_ptr, eid = g.transpose()
    r_col, r_eid = ograph.csr_transpose(N, r_row, r_s)
    assert np.array_equal(col_ptr.cpu().numpy(), r_col)
    assert np.array_equal(eid.cpu().numpy(), r_eid)


@pytest.mark.parametrize("N,E,big,seed", [(60, 300000, 200000, 4), (9, 70000, 69000, 5), (3000, 12345, 700, 6)])
def test_csr_with_one_large_segment(N, E, big, seed):
    """A padding-like receiver with most of the edges and a source with many
    outgoing edges: segments far longer than one sorting run (merge passes)."""
    rng = np.random.default_rng(seed)
    src = rng.integers(0, N, E)
    dst = rng.integers(0, N, E)
    dst[rng.choice(E, big, replace=False)] = N // 3
    src[rng.choice(E, big // 2, replace=False)] = N - 1
    row_ptr, s, perm = cgtp.csr_from_coo(N, to_dev_i32(src), to_dev_i32(dst))
    r_row, r_s, r_perm = ograph.csr_from_coo(N, src, dst)
    assert np.array_equal(row_ptr.cpu().numpy(), r_row)
    assert np.array_equal(s.cpu().numpy(), r_s)
    assert np.array_equal(perm.cpu().numpy(), r_perm)
    for pad in (None, N // 3):
        g = cgtp.Graph(N, row_ptr, s, pad_node=pad)
        col_ptr, eid = g.transpose()
        keep = np.ones(E, bool)
        if pad is not None:
            keep[r_row[pad]:r_row[pad + 1]] = False
        # reference transpose of the kept edges (CSR positions grouped by source, ascending)
        pos = np.nonzero(keep)[0]
        order = np.lexsort((pos, r_s[pos]))
        r_col = np.concatenate([[0], np.cumsum(np.bincount(r_s[pos], minlength=N))])
        assert np.array_equal(col_ptr.cpu().numpy(), r_col)
        assert np.array_equal(eid.cpu().numpy(), pos[order])


def test_radius_graph_csr_bit_exact():
    c = synth.CONFIGS["conv_water1k"]
    pos = synth.positions_for(c, 0)
    src, dst, _ = synth.radius_graph(pos, c["box"], c["r_cut"])
    p = np.random.default_rng(0).permutation(len(src))  # shuffled input order
    row_ptr, s, perm = cgtp.csr_from_coo(pos.shape[0], to_dev_i32(src[p]), to_dev_i32(dst[p]))
    r_row, r_s, r_perm = ograph.csr_from_coo(pos.shape[0], src[p], dst[p])
    assert np.array_equal(row_ptr.cpu().numpy(), r_row)
    assert np.array_equal(s.cpu().numpy(), r_s)
    assert np.array_equal(perm.cpu().numpy(), r_perm)


def test_invalid_graphs_are_rejected():
    with pytest.raises(cgtp.CgtpError) as e:
        cgtp.csr_from_coo(4, to_dev_i32([0, 1, 4]), to_dev_i32([1, 2, 3]))
    assert e.value.status == 4
    with pytest.raises(cgtp.CgtpError) as e:
        cgtp.csr_from_coo(4, to_dev_i32([0, 1, 2]), to_dev_i32([1, -1, 3]))
    assert e.value.status == 4
    bad = [
        ([0, 2, 1, 3], [0, 1, 2]),   # decreasing row_ptr
        ([1, 2, 3, 3], [0, 1, 2]),   # row_ptr[0] != 0
        ([0, 1, 2, 2], [0, 1, 2]),   # row_ptr[N] != E
        ([0, 1, 2, 3], [0, 3, 2]),   # src out of range
    ]
    for rp, s in bad:
        with pytest.raises(cgtp.CgtpError) as e:
            cgtp.Graph(3, to_dev_i32(rp), to_dev_i32(s))
        assert e.value.status == 4
    g = cgtp.Graph(3, to_dev_i32([0, 0, 0, 0]), to_dev_i32(np.zeros(0)))
    assert g.E == 0
