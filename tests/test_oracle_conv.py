"""Pins of the oracle's graph layouts and convolution (CPU only).

Cell-list radius graph vs O(N^2) brute force, CSR and its transpose vs direct
definitions, the convolution by explicit loops vs gather + scatter-add, and the
[V2106] test matrix: edge-order invariance, empty edges, isolated nodes,
rotation/inversion equivariance, translation invariance, node relabelling;
backward by adjoint identities and finite differences.
"""

import numpy as np
import pytest

from oracle import conv, graph, sh, wigner
from oracle.irreps import Layout
from clebsch_gordan_tensor_amd import synth

IX, IY, IO = "2x0e+2x1o+2x2e", "0e+1o+2e", "0e+0o+1e+1o+2e+2o"


def small_system(seed=0, n=12, box=6.0, r_cut=2.4):
    pos = synth.uniform_box(n, box, seed)
    src, dst, vec = synth.radius_graph(pos, box, r_cut)
    return pos, box, r_cut, src, dst, vec


def test_radius_graph_matches_bruteforce():
    for seed in range(3):
        pos = synth.uniform_box(60, 7.0, seed)
        a = synth.radius_graph(pos, 7.0, 2.2)
        b = graph.radius_graph_bruteforce(pos, 7.0, 2.2)
        assert np.array_equal(a[0], b[0]) and np.array_equal(a[1], b[1])
        assert np.abs(a[2] - b[2]).max() < 1e-12
    pos = synth.water_box(40, 11.0, 3)
    a = synth.radius_graph(pos, 11.0, 5.0)
    b = graph.radius_graph_bruteforce(pos, 11.0, 5.0)
    assert np.array_equal(a[0], b[0]) and np.array_equal(a[1], b[1])


def test_radius_graph_symmetric_and_loop_free():
    _, _, _, src, dst, vec = small_system(1, n=40, box=8.0, r_cut=3.0)
    fwd = set(zip(src.tolist(), dst.tolist()))
    assert fwd == set(zip(dst.tolist(), src.tolist()))
    assert np.all(src != dst)


def test_water_box_geometry():
    pos = synth.water_box(50, 12.0, 0)
    m = pos.reshape(50, 3, 3)
    d1 = graph.min_image(m[:, 1] - m[:, 0], 12.0)
    d2 = graph.min_image(m[:, 2] - m[:, 0], 12.0)
    assert np.abs(np.linalg.norm(d1, axis=1) - 0.96).max() < 1e-12
    cosang = np.einsum("ij,ij->i", d1, d2) / (0.96 ** 2)
    assert np.abs(np.degrees(np.arccos(cosang)) - 104.5).max() < 1e-9
    o = m[:, 0]
    dd = graph.min_image(o[:, None] - o[None], 12.0)
    r = np.linalg.norm(dd, axis=2) + np.eye(50) * 99
    assert r.min() >= 2.5
    assert pos.min() >= 0.0 and pos.max() < 12.0


def test_csr_and_transpose_definitions():
    rng = np.random.default_rng(2)
    N, E = 9, 40
    src = rng.integers(0, N, E)
    dst = rng.integers(0, N, E)
    row_ptr, s, perm = graph.csr_from_coo(N, src, dst)
    assert np.array_equal(s, src[perm]) and np.array_equal(dst[perm], graph.dst_of_csr(row_ptr))
    keys = list(zip(dst[perm].tolist(), s.tolist(), perm.tolist()))
    assert keys == sorted(keys)  # (dst, src) order, ties by input index
    col_ptr, eid = graph.csr_transpose(N, row_ptr, s)
    for n in range(N):
        seg = eid[col_ptr[n]:col_ptr[n + 1]]
        assert np.all(s[seg] == n) and np.all(np.diff(seg) > 0)
    assert sorted(eid.tolist()) == list(range(E))


def make_conv_inputs(L, N, vec, seed, r_cut):
    x = synth.gaussian((N, L.dim_x), seed, synth.S_X)
    Y = sh.real_sh(2, vec)
    W1, W2 = synth.mlp_params(8, 16, L.w_numel, seed)
    w = synth.radial_weights_np(np.linalg.norm(vec, axis=1), r_cut, W1, W2)
    return x, Y, w


def test_loops_equal_scatter():
    L = Layout(IX, IY, IO)
    pos, box, rc, src, dst, vec = small_system(0)
    N = pos.shape[0]
    row_ptr, s, perm = graph.csr_from_coo(N, src, dst)
    x, Y, w = make_conv_inputs(L, N, vec[perm], 0, rc)
    sc = conv.avg_neighbors_scale(N, len(src))
    a = conv.forward_loops(L, row_ptr, s, x, Y, w, sc)
    b = conv.forward(L, row_ptr, s, x, Y, w, sc)
    assert np.abs(a - b).max() < 1e-12


def test_edge_order_invariance_and_relabelling():
    L = Layout(IX, IY, IO)
    pos, box, rc, src, dst, vec = small_system(1)
    N = pos.shape[0]
    rng = np.random.default_rng(0)
    sh_perm = rng.permutation(len(src))
    outs = []
    for order in (np.arange(len(src)), sh_perm):
        row_ptr, s, perm = graph.csr_from_coo(N, src[order], dst[order])
        x, Y, w = make_conv_inputs(L, N, vec[order][perm], 1, rc)
        outs.append(conv.forward(L, row_ptr, s, x, Y, w, 1.0))
    assert np.array_equal(outs[0], outs[1])
    # relabel nodes: out permutes with the labels
    lab = rng.permutation(N)  # new id of old node i is lab[i]
    row_ptr, s, perm = graph.csr_from_coo(N, lab[src], lab[dst])
    x, Y, w = make_conv_inputs(L, N, vec[perm], 1, rc)
    x_new = np.empty_like(x)
    x_new[lab] = x
    out_new = conv.forward(L, row_ptr, s, x_new, Y, w, 1.0)
    assert np.abs(out_new[lab] - outs[0]).max() < 1e-12


def test_empty_edges_and_isolated_nodes():
    L = Layout(IX, IY, IO)
    N = 5
    row_ptr, s, _ = graph.csr_from_coo(N, np.zeros(0, int), np.zeros(0, int))
    x = synth.gaussian((N, L.dim_x), 0, synth.S_X)
    out = conv.forward(L, row_ptr, s, x, np.zeros((0, L.dim_y)), np.zeros((0, L.w_numel)), 1.0)
    assert out.shape == (N, L.dim_out) and np.all(out == 0.0)
    # one edge 0 -> 1: every node but 1 gets a zero row
    row_ptr, s, _ = graph.csr_from_coo(N, np.array([0]), np.array([1]))
    Y = sh.real_sh(2, np.array([[0.3, -0.2, 0.9]]))
    w = synth.gaussian((1, L.w_numel), 0, synth.S_W)
    out = conv.forward(L, row_ptr, s, x, Y, w, 1.0)
    assert np.all(out[[0, 2, 3, 4]] == 0.0) and np.abs(out[1]).max() > 0


@pytest.mark.parametrize("inv", [False, True])
def test_rotation_inversion_translation(inv):
    L = Layout(IX, IY, IO)
    pos, box, rc, src, dst, vec = small_system(2)
    N = pos.shape[0]
    row_ptr, s, perm = graph.csr_from_coo(N, src, dst)
    vec = vec[perm]
    x, Y, w = make_conv_inputs(L, N, vec, 2, rc)
    out = conv.forward(L, row_ptr, s, x, Y, w, 1.0)
    ang = wigner.random_euler(np.random.default_rng(4))
    R = wigner.euler_to_matrix(*ang) * (-1.0 if inv else 1.0)

    def rot(irreps, rows, offs):
        res = rows.copy()
        for (mul, l, p), o in zip(irreps, offs):
            D = wigner.wigner_D_real(l, *ang) * (p if inv else 1)
            blk = rows[:, o:o + mul * (2 * l + 1)].reshape(-1, 2 * l + 1, mul)
            res[:, o:o + mul * (2 * l + 1)] = np.einsum("ab,zbu->zau", D, blk).reshape(rows.shape[0], -1)
        return res

    xr = rot(L.X, x, L.x_off)
    Yr = sh.real_sh(2, vec @ R.T)  # edge vectors of the rotated (inverted) system
    out_r = conv.forward(L, row_ptr, s, xr, Yr, w, 1.0)
    O = [(p["mul"], p["l3"], p["p3"]) for p in L.paths]
    assert np.abs(out_r - rot(O, out, [p["out_off"] for p in L.paths])).max() < 1e-11
    # translation: the graph built from shifted positions gives the same edges and vectors
    src2, dst2, vec2 = synth.radius_graph(pos + np.array([1.3, -0.7, 2.9]), box, rc)
    assert np.array_equal(src2, src) and np.array_equal(dst2, dst)


def test_backward_adjoint_and_fd():
    L = Layout(IX, IY, IO)
    pos, box, rc, src, dst, vec = small_system(3)
    N = pos.shape[0]
    row_ptr, s, perm = graph.csr_from_coo(N, src, dst)
    x, Y, w = make_conv_inputs(L, N, vec[perm], 3, rc)
    sc = 0.7
    g = synth.gaussian((N, L.dim_out), 3, synth.S_G)
    dx, dY, dw = conv.backward(L, row_ptr, s, x, Y, w, sc, g)
    f = np.sum(g * conv.forward(L, row_ptr, s, x, Y, w, sc))
    for d, v in ((dx, x), (dY, Y), (dw, w)):
        assert np.sum(d * v) == pytest.approx(f, rel=1e-11)
    h = 1e-6
    rng = np.random.default_rng(1)
    for _ in range(5):
        n, k = rng.integers(0, N), rng.integers(0, L.dim_x)
        xp, xm = x.copy(), x.copy()
        xp[n, k] += h
        xm[n, k] -= h
        fd = (np.sum(g * conv.forward(L, row_ptr, s, xp, Y, w, sc))
              - np.sum(g * conv.forward(L, row_ptr, s, xm, Y, w, sc))) / (2 * h)
        assert dx[n, k] == pytest.approx(fd, abs=1e-7)


def test_radial_backward_matches_fd():
    r = np.linspace(0.8, 4.9, 7)
    W1, W2 = synth.mlp_params(8, 16, 5, 0)
    dw = np.random.default_rng(0).standard_normal((7, 5))
    an = synth.radial_weights_backward_np(r, 5.0, W1, W2, dw)
    h = 1e-6
    fd = ((synth.radial_weights_np(r + h, 5.0, W1, W2) - synth.radial_weights_np(r - h, 5.0, W1, W2)) * dw).sum(1) / (2 * h)
    assert np.abs(an - fd).max() < 1e-7


def test_force_chain_matches_fd():
    """Edge-vector gradient (harmonics + radial network) vs central differences of
    f(vec) = <g, conv(x, Y(vec), w(|vec|))>."""
    L = Layout(IX, IY, IO)
    pos, box, rc, src, dst, vec = small_system(5)
    N = pos.shape[0]
    row_ptr, s, perm = graph.csr_from_coo(N, src, dst)
    vec = vec[perm]
    x = synth.gaussian((N, L.dim_x), 5, synth.S_X)
    g = synth.gaussian((N, L.dim_out), 5, synth.S_G)
    W1, W2 = synth.mlp_params(8, 16, L.w_numel, 5)
    sc = 0.6

    def f(v):
        r = np.linalg.norm(v, axis=1)
        return np.sum(g * conv.forward(L, row_ptr, s, x, sh.real_sh(2, v), synth.radial_weights_np(r, rc, W1, W2), sc))

    r = np.linalg.norm(vec, axis=1)
    w = synth.radial_weights_np(r, rc, W1, W2)
    _, dY, dw = conv.backward(L, row_ptr, s, x, sh.real_sh(2, vec), w, sc, g)
    gv = conv.edge_vector_grad(2, vec, dY, synth.radial_weights_backward_np(r, rc, W1, W2, dw))
    h = 1e-6
    rng = np.random.default_rng(2)
    for _ in range(8):
        e, k = rng.integers(0, vec.shape[0]), rng.integers(0, 3)
        vp, vm = vec.copy(), vec.copy()
        vp[e, k] += h
        vm[e, k] -= h
        fd = (f(vp) - f(vm)) / (2 * h)
        assert gv[e, k] == pytest.approx(fd, rel=1e-6, abs=1e-7)


def test_padding_edges_equal_the_graph_without_them():
    """Edges into a padding node add nothing ([E3J] 3.1.2, 3.2): forward, backward
    and double backward equal those of the graph with the padding edges removed
    (built again from the remaining edge list), with zero rows for the padding."""
    from oracle import graph as og
    L = Layout("2x0e+2x1o+2x2e", "0e+1o+2e", "0e+0o+1e+1o+2e+2o")
    rng = np.random.default_rng(41)
    N, pad = 12, 11
    src = rng.integers(0, N - 1, 40)
    dst = rng.integers(0, N - 1, 40)
    src = np.concatenate([src, np.full(15, pad), rng.integers(0, N - 1, 3)])   # padding edges, and 3 more into pad
    dst = np.concatenate([dst, np.full(15, pad), np.full(3, pad)])
    row_ptr, s, perm = og.csr_from_coo(N, src, dst)
    E = len(s)
    x = synth.gaussian((N, L.dim_x), 42, synth.S_X)
    Y = synth.gaussian((E, L.dim_y), 42, synth.S_Y)
    w = synth.gaussian((E, L.w_numel), 42, synth.S_W)
    g = synth.gaussian((N, L.dim_out), 42, synth.S_G)
    keep = np.ones(E, bool)
    keep[row_ptr[pad]:row_ptr[pad + 1]] = False
    d = og.dst_of_csr(row_ptr)
    rp2, s2, perm2 = og.csr_from_coo(N, s[keep], d[keep])
    Yk, wk = Y[keep][perm2], w[keep][perm2]
    out = conv.forward(L, row_ptr, s, x, Y, w, 0.6, pad_node=pad)
    ref = conv.forward(L, rp2, s2, x, Yk, wk, 0.6)
    assert np.abs(out - ref).max() < 1e-13 and np.all(out[pad] == 0)
    dx, dY, dw = conv.backward(L, row_ptr, s, x, Y, w, 0.6, g, pad_node=pad)
    rdx, rdY, rdw = conv.backward(L, rp2, s2, x, Yk, wk, 0.6, g)
    assert np.abs(dx - rdx).max() < 1e-13
    kept_pos = np.nonzero(keep)[0][perm2]          # CSR position (full graph) of each edge of the reduced graph
    assert np.abs(dY[kept_pos] - rdY).max() < 1e-13 and np.abs(dw[kept_pos] - rdw).max() < 1e-13
    assert np.all(dY[~keep] == 0) and np.all(dw[~keep] == 0)
    gY = synth.gaussian((E, L.dim_y), 43, synth.S_Y)
    gw = synth.gaussian((E, L.w_numel), 43, synth.S_W)
    dd = conv.double_backward(L, row_ptr, s, x, Y, w, 0.6, g, None, gY, gw, pad_node=pad)
    rd = conv.double_backward(L, rp2, s2, x, Yk, wk, 0.6, g, None, gY[keep][perm2], gw[keep][perm2])
    assert np.abs(dd[0] - rd[0]).max() < 1e-12 and np.abs(dd[3] - rd[3]).max() < 1e-12
    assert np.abs(dd[1][kept_pos] - rd[1]).max() < 1e-12 and np.all(dd[2][~keep] == 0)
