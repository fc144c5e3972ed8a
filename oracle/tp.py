"""uvu Clebsch-Gordan tensor product, forward and backward (oracle; test infrastructure).

[COURSE] lesson 03b: the learnable layer x (x)_w y built from instructions in a
connection mode (uvw, uvu, ...), reproducible "with a bare einsum"; [E3J] 3.1.1
(full CG tensor product) and E.1 (reverse-mode rules obtained by transposing the
linear maps, using bilinearity and index permutations).

For every path p = (i1, i2, l3) with x block i1 of multiplicity u:

  out[z, p, m3, u] = w[(z,) p, u] * sum_{m1, m2} C_p[m1, m2, m3] x[z, i1, m1, u] y[z, i2, m2]

``w`` is either shared, shape [W], or one row per z, shape [B, W], where
W = sum_p mul_p. Two forward routes are given: explicit loops over the nonzero
CG entries (``forward``) and one dense einsum per path (``forward_dense``).
With a collapsed layout several paths share an output block and their
outputs are added there; in the backward each of them reads that block's
cotangent.
"""

import numpy as np

from .cg import cg_real
from .irreps import Layout


def _w_of(L, w, p, B):
    wb = L.w_block(w, p)
    if wb.ndim == 1:
        wb = np.broadcast_to(wb, (B, wb.shape[0]))
    return wb


def forward(L, x, y, w):
    """Sparse route: loop over paths and the nonzero entries of each CG block."""
    x = np.asarray(x, np.float64)
    y = np.asarray(y, np.float64)
    w = np.asarray(w, np.float64)
    B = x.shape[0]
    out = np.zeros((B, L.dim_out))
    for p in L.paths:
        C = cg_real(p["l1"], p["l2"], p["l3"])
        xb = L.x_block(x, p["i1"])            # [B, 2l1+1, u]
        yb = L.y_block(y, p["i2"])            # [B, 2l2+1]
        ob = np.zeros((B, 2 * p["l3"] + 1, p["mul"]))
        for m1, m2, m3 in zip(*np.nonzero(C)):
            ob[:, m3, :] += C[m1, m2, m3] * xb[:, m1, :] * yb[:, m2][:, None]
        ob *= _w_of(L, w, p, B)[:, None, :]
        L.out_block(out, p)[...] += ob
    return out


def forward_dense(L, x, y, w):
    """Dense route: one einsum per path over the full CG block ([COURSE] 03b)."""
    x = np.asarray(x, np.float64)
    y = np.asarray(y, np.float64)
    w = np.asarray(w, np.float64)
    B = x.shape[0]
    out = np.zeros((B, L.dim_out))
    for p in L.paths:
        C = cg_real(p["l1"], p["l2"], p["l3"])
        ob = np.einsum("abc,zau,zb,zu->zcu", C, L.x_block(x, p["i1"]),
                       L.y_block(y, p["i2"]), _w_of(L, w, p, B))
        L.out_block(out, p)[...] += ob
    return out


def backward(L, x, y, w, g):
    """Cotangents of x, y, w given the output cotangent g (transposition rules).

      dx[z,i1,m1,u] = sum_p w * sum_{m2,m3} C y[m2] g[m3,u]
      dy[z,i2,m2]   = sum_p sum_u w * sum_{m1,m3} C x[m1,u] g[m3,u]
      dw[(z,)p,u]   = sum_{(z),m1,m2,m3} C x[m1,u] y[m2] g[m3,u]
    A shared w gets its cotangent summed over rows.
    """
    x = np.asarray(x, np.float64)
    y = np.asarray(y, np.float64)
    w = np.asarray(w, np.float64)
    g = np.asarray(g, np.float64)
    B = x.shape[0]
    dx = np.zeros_like(x)
    dy = np.zeros_like(y)
    dw_rows = np.zeros((B, L.w_numel))
    for p in L.paths:
        C = cg_real(p["l1"], p["l2"], p["l3"])
        xb = L.x_block(x, p["i1"])
        yb = L.y_block(y, p["i2"])
        gb = L.out_block(g, p)
        wb = _w_of(L, w, p, B)
        L.x_block(dx, p["i1"])[...] += np.einsum("abc,zb,zcu,zu->zau", C, yb, gb, wb)
        L.y_block(dy, p["i2"])[...] += np.einsum("abc,zau,zcu,zu->zb", C, xb, gb, wb)
        dw_rows[:, p["w_off"]:p["w_off"] + p["mul"]] = np.einsum("abc,zau,zb,zcu->zu", C, xb, yb, gb)
    dw = dw_rows if w.ndim == 2 else dw_rows.sum(axis=0)
    return dx, dy, dw


def double_backward(L, x, y, w, g, gx=None, gy=None, gw=None):
    """Reverse mode of ``backward``: cotangents of (x, y, w, g) for cotangents
    (gx, gy, gw) of its outputs (dx, dy, dw); a missing one counts as zero.

    The backward's outputs are the transposed maps of [E3J] E.1, each linear in
    the other three tensors; differentiating
      S = <gx, dx> + <gy, dy> + <gw, dw>
    entry by entry gives, per path (C the CG block, u the channel):
      ddx[m1, u] = sum C (gy[m2] g[m3, u] w[u] + y[m2] g[m3, u] gw[u])
      ddy[m2]    = sum C (gx[m1, u] g[m3, u] w[u] + x[m1, u] g[m3, u] gw[u])
      ddw[u]     = sum C (gx[m1, u] y[m2] + x[m1, u] gy[m2]) g[m3, u]
      ddg[m3, u] = sum C (gx[m1, u] y[m2] w[u] + x[m1, u] gy[m2] w[u] + x[m1, u] y[m2] gw[u])
    (sums over the indices not on the left; a shared w gets ddw summed over rows).
    """
    x, y, w, g = (np.asarray(t, np.float64) for t in (x, y, w, g))
    B = x.shape[0]
    z = lambda t, like: np.zeros_like(like) if t is None else np.asarray(t, np.float64)
    gx, gy, gw = z(gx, x), z(gy, y), z(gw, w)
    ddx, ddy, ddg = np.zeros_like(x), np.zeros_like(y), np.zeros((B, L.dim_out))
    ddw_rows = np.zeros((B, L.w_numel))
    for p in L.paths:
        C = cg_real(p["l1"], p["l2"], p["l3"])
        xb, ax = L.x_block(x, p["i1"]), L.x_block(gx, p["i1"])
        yb, by = L.y_block(y, p["i2"]), L.y_block(gy, p["i2"])
        gb = L.out_block(g, p)
        wb, cw = _w_of(L, w, p, B), _w_of(L, gw, p, B)
        L.x_block(ddx, p["i1"])[...] += (np.einsum("abc,zb,zcu,zu->zau", C, by, gb, wb)
                                         + np.einsum("abc,zb,zcu,zu->zau", C, yb, gb, cw))
        L.y_block(ddy, p["i2"])[...] += (np.einsum("abc,zau,zcu,zu->zb", C, ax, gb, wb)
                                         + np.einsum("abc,zau,zcu,zu->zb", C, xb, gb, cw))
        ddw_rows[:, p["w_off"]:p["w_off"] + p["mul"]] = (np.einsum("abc,zau,zb,zcu->zu", C, ax, yb, gb)
                                                         + np.einsum("abc,zau,zb,zcu->zu", C, xb, by, gb))
        L.out_block(ddg, p)[...] += (np.einsum("abc,zau,zb,zu->zcu", C, ax, yb, wb)
                                     + np.einsum("abc,zau,zb,zu->zcu", C, xb, by, wb)
                                     + np.einsum("abc,zau,zb,zu->zcu", C, xb, yb, cw))
    ddw = ddw_rows if w.ndim == 2 else ddw_rows.sum(axis=0)
    return ddx, ddy, ddw, ddg


def make_layout(irreps_x, irreps_y, irreps_out, select="all", collapse=False):
    return Layout(irreps_x, irreps_y, irreps_out, select, collapse)
