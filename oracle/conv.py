"""Tensor-field-network convolution, forward and backward (oracle; test infrastructure).

[COURSE] lesson 06a: m_ij = (R(|r_ij|) Y(rhat_ij)) (x)_w h_j aggregated at the
receiver i; [V2106] Convolution(edge_src, edge_dst, radial) with a
sqrt(num_neighbors) normalisation; [E3J] 3.1.2 and E.2.2 (stream edges, CSR
receiver aggregation). Here the radial factor arrives as per-edge weights
w[e] (one per path and channel), so for a destination node n:

  out[n] = scale * sum_{e : dst(e) = n} TP(x[src(e)], Y[e], w[e])

summed in CSR order. Edge-indexed inputs (Y, w) are in CSR order; ``row_ptr``
and ``src`` are the CSR arrays of ``graph.csr_from_coo``.
"""

import numpy as np

from . import sh as _sh
from . import tp
from .graph import dst_of_csr


def padding_mask(row_ptr, pad_node):
    """Edges whose destination is the padding node ([E3J] 3.1.2 and 3.2: a
    fixed-shape caller pads the edge list with edges into one shared padding
    node); they contribute nothing. None: no padding."""
    E = int(row_ptr[-1])
    m = np.zeros(E, bool)
    if pad_node is not None:
        m[row_ptr[pad_node]:row_ptr[pad_node + 1]] = True
    return m


def forward_loops(L, row_ptr, src, x, Y, w, scale):
    """Explicit per-node, per-edge loops (for tiny graphs)."""
    N = len(row_ptr) - 1
    out = np.zeros((N, L.dim_out))
    for n in range(N):
        acc = np.zeros(L.dim_out)
        for e in range(row_ptr[n], row_ptr[n + 1]):
            acc += tp.forward(L, x[src[e]][None], Y[e][None], w[e][None])[0]
        out[n] = scale * acc
    return out


def forward(L, row_ptr, src, x, Y, w, scale, pad_node=None):
    """Materialised-message route: TP on gathered rows, then a scatter-add.
    Padding edges (into pad_node) carry no message."""
    x = np.asarray(x, np.float64)
    N = len(row_ptr) - 1
    dst = dst_of_csr(row_ptr)
    msg = tp.forward(L, x[np.asarray(src)], Y, w)
    msg[padding_mask(row_ptr, pad_node)] = 0.0
    out = np.zeros((N, L.dim_out))
    np.add.at(out, dst, msg)
    return scale * out


def backward(L, row_ptr, src, x, Y, w, scale, g, pad_node=None):
    """Cotangents (dx [N, dim_x], dY [E, dim_y], dw [E, W]) for out cotangent g [N, dim_out].
    Padding edges (into pad_node) get zero gradients and add nothing to dx."""
    x = np.asarray(x, np.float64)
    dst = dst_of_csr(row_ptr)
    src = np.asarray(src)
    ge = scale * np.asarray(g, np.float64)[dst]
    ge[padding_mask(row_ptr, pad_node)] = 0.0
    dxe, dY, dw = tp.backward(L, x[src], Y, w, ge)
    dx = np.zeros_like(x)
    np.add.at(dx, src, dxe)
    return dx, dY, dw


def double_backward(L, row_ptr, src, x, Y, w, scale, g, gx=None, gY=None, gw=None, pad_node=None):
    """Reverse mode of ``backward`` (twice-differentiable convolution, e.g. for
    training on forces): cotangents of (x, Y, w, g) for cotangents (gx, gY, gw)
    of (dx, dY, dw); a missing one counts as zero.

    The backward is the tensor-product backward on the gathered rows
    (x[src], Y, w, scale * g[dst]) followed by a scatter-add of dx over src, so
    its reverse mode gathers gx over src, runs the tensor-product double
    backward per edge, and scatters: ddx over src, ddg (times scale) over dst.
    """
    x = np.asarray(x, np.float64)
    dst = dst_of_csr(row_ptr)
    src = np.asarray(src)
    ge = scale * np.asarray(g, np.float64)[dst]
    pm = padding_mask(row_ptr, pad_node)
    ge[pm] = 0.0
    gxe = None if gx is None else np.asarray(gx, np.float64)[src]
    ddxe, ddY, ddw, ddge = tp.double_backward(L, x[src], Y, w, ge, gxe, gY, gw)
    ddge[pm] = 0.0
    ddx = np.zeros_like(x)
    np.add.at(ddx, src, ddxe)
    ddg = np.zeros((len(row_ptr) - 1, L.dim_out))
    np.add.at(ddg, dst, scale * ddge)
    return ddx, ddY, ddw, ddg


def avg_neighbors_scale(N, E):
    """1 / sqrt(E / N): the sqrt(num_neighbors) normalisation of [V2106] with the
    average degree of the built graph."""
    return 1.0 / np.sqrt(E / N) if E > 0 else 1.0


def edge_vector_grad(lmax, vec, grad_sh, grad_r):
    """Gradient with respect to the edge vectors (the force chain).

    [V2106] "Fixed-topology compilation": position gradients pass through the
    edge vectors, their lengths, the radial basis and the harmonics, with the
    edge set held fixed. The harmonics see only the direction of vec and the
    radial network only its length r = |vec|, so for cotangents grad_sh of
    Y = real_sh(vec) and grad_r of r:

      d/dvec = real_sh_grad(vec, grad_sh) + grad_r * vec / |vec|

    grad_r is the radial network's vector-Jacobian product of the weight
    cotangent (computed by the caller's radial network).
    """
    vec = np.asarray(vec, np.float64)
    r = np.linalg.norm(vec, axis=1)
    rs = np.where(r == 0.0, 1.0, r)
    return _sh.real_sh_grad(lmax, vec, grad_sh) + (np.asarray(grad_r, np.float64) / rs)[:, None] * vec
