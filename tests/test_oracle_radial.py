"""Pins of the radial-last-layer convolution oracle (oracle/radial.py).

* an identity last layer (H = W, W2 = I) gives the convolution with w = h;
* a last layer of rank one (W2 = a b^T) gives the convolution with per-edge
  weights (h a) b^T, formed entry by entry;
* the radial network of the benchmark (Bessel basis, envelope, Linear -> SiLU
  -> Linear) split at its last layer: w from synth's network equals h W2 with
  h its hidden activations;
* the output is linear in each of x, Y, h and W2 separately: the adjoint
  identities <g, out> = <dx, x> = <dY, Y> = <dh, h> = <dW2, W2> hold;
* central differences of <g, out> for every input;
* planted mistakes (W2 transposed in dh, dW2 missing the sum over edges) fail.
"""

import numpy as np
import pytest

from oracle import conv, graph, radial, sh
from oracle.irreps import Layout
from clebsch_gordan_tensor_amd import synth

IX, IY, IO = "2x0e+2x1o+2x2e", "0e+1o+2e", "0e+0o+1e+1o+2e+2o"


def system(seed=0, n=14, box=6.0, r_cut=2.6, H=6):
    pos = synth.uniform_box(n, box, seed)
    src, dst, vec = synth.radius_graph(pos, box, r_cut)
    row, s, perm = graph.csr_from_coo(n, src, dst)
    L = Layout(IX, IY, IO)
    E = len(src)
    x = synth.gaussian((n, L.dim_x), seed, synth.S_X)
    Y = sh.real_sh(2, vec[perm])
    h = synth.gaussian((E, H), seed, synth.S_MLP1)
    W2 = synth.gaussian((H, L.w_numel), seed, synth.S_MLP2)
    g = synth.gaussian((n, L.dim_out), seed, synth.S_G)
    return L, row, s, x, Y, h, W2, g, vec[perm]


def test_identity_last_layer_is_the_convolution():
    L, row, s, x, Y, h, _, _, _ = system(1)
    E = len(s)
    hw = synth.gaussian((E, L.w_numel), 1, synth.S_W)
    out = radial.forward(L, row, s, x, Y, hw, np.eye(L.w_numel), 0.4)
    assert np.abs(out - conv.forward(L, row, s, x, Y, hw, 0.4)).max() < 1e-13


def test_rank_one_last_layer():
    L, row, s, x, Y, h, _, _, _ = system(2)
    rng = np.random.default_rng(3)
    a, b = rng.standard_normal(h.shape[1]), rng.standard_normal(L.w_numel)
    w = np.empty((len(s), L.w_numel))
    for e in range(len(s)):
        he = sum(h[e, j] * a[j] for j in range(h.shape[1]))
        for k in range(L.w_numel):
            w[e, k] = he * b[k]
    out = radial.forward(L, row, s, x, Y, h, np.outer(a, b), 0.7)
    assert np.abs(out - conv.forward(L, row, s, x, Y, w, 0.7)).max() < 1e-12


def test_benchmark_radial_network_split_at_its_last_layer():
    L, row, s, x, Y, _, _, _, vec = system(3)
    W1, W2 = synth.mlp_params(8, 16, L.w_numel, 3)
    r = np.linalg.norm(vec, axis=1)
    w = synth.radial_weights_np(r, 2.6, W1, W2)
    pre = synth.bessel_envelope(r, 2.6) @ W1
    h = pre / (1.0 + np.exp(-pre))  # SiLU
    assert np.abs(radial.edge_weights(h, W2) - w).max() < 1e-12
    assert np.abs(radial.forward(L, row, s, x, Y, h, W2, 0.3) - conv.forward(L, row, s, x, Y, w, 0.3)).max() < 1e-12


def test_adjoint_identities():
    L, row, s, x, Y, h, W2, g, _ = system(4)
    f = np.sum(g * radial.forward(L, row, s, x, Y, h, W2, 0.6))
    grads = radial.backward(L, row, s, x, Y, h, W2, 0.6, g)
    for d, v in zip(grads, (x, Y, h, W2)):
        assert np.sum(d * v) == pytest.approx(f, rel=1e-12)


def test_finite_differences():
    L, row, s, x, Y, h, W2, g, _ = system(5, n=10)
    grads = radial.backward(L, row, s, x, Y, h, W2, 0.6, g)
    f = lambda *a: np.sum(g * radial.forward(L, row, s, *a, 0.6))
    rng = np.random.default_rng(6)
    hstep = 1e-6
    args = [x, Y, h, W2]
    for which in range(4):
        for _ in range(5):
            idx = tuple(rng.integers(0, n) for n in args[which].shape)
            ap, am = [a.copy() for a in args], [a.copy() for a in args]
            ap[which][idx] += hstep
            am[which][idx] -= hstep
            assert grads[which][idx] == pytest.approx((f(*ap) - f(*am)) / (2 * hstep), abs=1e-7)


def test_planted_mistakes_are_caught(monkeypatch):
    L, row, s, x, Y, h, W2, g, _ = system(7)
    f = np.sum(g * radial.forward(L, row, s, x, Y, h, W2, 0.6))
    real = radial.backward

    def dh_transposed(*a):  # dh from W2 read transposed in the wrong order (row-major reshape)
        dx, dY, dh, dW2 = real(*a)
        _, _, dw = conv.backward(L, row, s, x, Y, radial.edge_weights(h, W2), 0.6, g)
        return dx, dY, dw @ W2.reshape(W2.shape[1], W2.shape[0]), dW2

    def dW2_one_edge(*a):  # the sum over edges dropped (first edge only)
        dx, dY, dh, dW2 = real(*a)
        _, _, dw = conv.backward(L, row, s, x, Y, radial.edge_weights(h, W2), 0.6, g)
        return dx, dY, dh, np.outer(h[0], dw[0])

    for bad, k, v in ((dh_transposed, 2, h), (dW2_one_edge, 3, W2)):
        monkeypatch.setattr(radial, "backward", bad)
        d = radial.backward(L, row, s, x, Y, h, W2, 0.6, g)[k]
        monkeypatch.setattr(radial, "backward", real)
        assert abs(np.sum(d * v) - f) > 1e-6 * abs(f)
