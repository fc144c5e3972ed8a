"""Connection modes of the weighted tensor product (oracle; test infrastructure).

[COURSE] lesson 03b turns the Clebsch-Gordan decomposition into a learnable layer
x (x)_w y built from instructions in a connection mode (uvw, uvu, ...), shows that a
bare einsum reproduces it, and counts its weights; o3.FullyConnectedTensorProduct is
the uvw layer over every allowed path. The pages name the modes without formulas;
the reading taken is e3nn's. For a path p = (i1, i2, l3) with x block i1 of
multiplicity u and y block i2 of multiplicity v:

  uvu:  out[z, p, m3, a] = sum_b     w_p[a, b]    sum_{m1,m2} C_p[m1,m2,m3] x[z,i1,m1,a] y[z,i2,m2,b]
  uvw:  out[z, p, m3, k] = sum_{a,b} W_p[a, b, k] sum_{m1,m2} C_p[m1,m2,m3] x[z,i1,m1,a] y[z,i2,m2,b]

uvu keeps x's multiplicity u on the output (channel-wise); uvw takes the output
multiplicity w from irreps_out (its first entry of type (l3, p3)) and mixes every
(x channel, y channel) pair into every output channel. Weights per path are
[u][v] (uvu) or [u][v][w] (uvw), row-major, concatenated in path order, either
shared ([W]) or one row per z ([B, W]). No normalisation factor (a caller folds
any into the weights). With v = 1, uvu is the channel-wise product of ``tp``.
Paths are those of ``irreps.paths_uvu`` (triangle rule, p3 = p1 p2, (l3, p3) in
irreps_out, order i1, i2, l3; optional parity selection). Collapsed outputs add
the paths of one (l3, p3) into one block ([E3J] B.1 and B.3); uvw over every path
with collapsed outputs is the fully connected product.

Rows are ir_mul blocks [2l+1][mul] everywhere (y blocks too, [2l2+1][v]).
"""

import numpy as np

from .cg import cg_real
from .irreps import SELECTIONS, block_offsets, dim, parse_irreps

MODES = ("uvu", "uvw")


class ModeLayout:
    """Paths, row layouts and weight offsets of a tensor product in a connection mode."""

    def __init__(self, irreps_x, irreps_y, irreps_out, mode="uvu", select="all", collapse=False):
        if mode not in MODES:
            raise ValueError("mode must be one of %s" % (MODES,))
        if select not in SELECTIONS:
            raise ValueError("select must be one of %s" % (SELECTIONS,))
        self.mode, self.select, self.collapse = mode, select, collapse
        self.X, self.Y = parse_irreps(irreps_x), parse_irreps(irreps_y)
        O = parse_irreps(irreps_out)
        out_mul = {}
        for mul, l, par in O:
            out_mul.setdefault((l, par), mul)
        self.x_off, self.y_off = block_offsets(self.X), block_offsets(self.Y)
        self.dim_x, self.dim_y = dim(self.X), dim(self.Y)
        self.paths = []
        w = 0
        for i1, (u, l1, p1) in enumerate(self.X):
            for i2, (v, l2, p2) in enumerate(self.Y):
                for l3 in range(abs(l1 - l2), l1 + l2 + 1):
                    p3 = p1 * p2
                    if (l3, p3) not in out_mul:
                        continue
                    if select != "all" and ((l1 + l2 + l3) % 2 == 0) != (select == "symmetric"):
                        continue
                    wo = u if mode == "uvu" else out_mul[(l3, p3)]
                    nw = u * v if mode == "uvu" else u * v * wo
                    self.paths.append(dict(i1=i1, i2=i2, l1=l1, l2=l2, l3=l3, p3=p3, u=u, v=v, mul=wo,
                                           w_off=w, w_len=nw))
                    w += nw
        self.w_numel = w
        self.groups = []
        o = 0
        if not collapse:
            for p in self.paths:
                p["out_off"] = o
                self.groups.append(dict(l3=p["l3"], p3=p["p3"], mul=p["mul"], out_off=o))
                o += p["mul"] * (2 * p["l3"] + 1)
        else:
            order = []
            for _, l, par in O:
                if (l, par) not in order:
                    order.append((l, par))
            for l3, p3 in order:
                feeding = [p for p in self.paths if (p["l3"], p["p3"]) == (l3, p3)]
                if not feeding:
                    continue
                muls = {p["mul"] for p in feeding}
                if len(muls) != 1:
                    raise ValueError("collapsed output %d%s fed by different multiplicities %s"
                                     % (l3, "e" if p3 > 0 else "o", sorted(muls)))
                mul = muls.pop()
                for p in feeding:
                    p["out_off"] = o
                self.groups.append(dict(l3=l3, p3=p3, mul=mul, out_off=o))
                o += mul * (2 * l3 + 1)
        self.dim_out = o

    def x_block(self, x, i):
        u, l, _ = self.X[i]
        o = self.x_off[i]
        return x[..., o:o + u * (2 * l + 1)].reshape(x.shape[:-1] + (2 * l + 1, u))

    def y_block(self, y, i):
        v, l, _ = self.Y[i]
        o = self.y_off[i]
        return y[..., o:o + v * (2 * l + 1)].reshape(y.shape[:-1] + (2 * l + 1, v))

    def out_block(self, out, p):
        o, n = p["out_off"], 2 * p["l3"] + 1
        return out[..., o:o + n * p["mul"]].reshape(out.shape[:-1] + (n, p["mul"]))

    def w_block(self, w, p, B):
        """Weights of path p as [B, u, v] (uvu) or [B, u, v, w] (uvw)."""
        shape = (p["u"], p["v"]) if self.mode == "uvu" else (p["u"], p["v"], p["mul"])
        wb = w[..., p["w_off"]:p["w_off"] + p["w_len"]]
        if wb.ndim == 1:
            return np.broadcast_to(wb.reshape(shape), (B,) + shape)
        return wb.reshape((B,) + shape)


def forward(ML, x, y, w):
    """One einsum per path over the dense CG block ([COURSE] 03b)."""
    x, y, w = (np.asarray(t, np.float64) for t in (x, y, w))
    B = x.shape[0]
    out = np.zeros((B, ML.dim_out))
    for p in ML.paths:
        C = cg_real(p["l1"], p["l2"], p["l3"])
        xb, yb, wb = ML.x_block(x, p["i1"]), ML.y_block(y, p["i2"]), ML.w_block(w, p, B)
        if ML.mode == "uvu":
            ob = np.einsum("ijk,zia,zjb,zab->zka", C, xb, yb, wb)
        else:
            ob = np.einsum("ijk,zia,zjb,zabc->zkc", C, xb, yb, wb)
        ML.out_block(out, p)[...] += ob
    return out


def backward(ML, x, y, w, g):
    """Cotangents (dx, dy, dw) for the output cotangent g: each input's slot of the
    trilinear form <g, out(x, y, w)> with that input removed ([E3J] E.1, the
    reverse mode of a multilinear map by transposition). A shared w gets its
    cotangent summed over rows."""
    x, y, w, g = (np.asarray(t, np.float64) for t in (x, y, w, g))
    B = x.shape[0]
    dx, dy = np.zeros_like(x), np.zeros_like(y)
    dw_rows = np.zeros((B, ML.w_numel))
    for p in ML.paths:
        C = cg_real(p["l1"], p["l2"], p["l3"])
        xb, yb, wb, gb = ML.x_block(x, p["i1"]), ML.y_block(y, p["i2"]), ML.w_block(w, p, B), ML.out_block(g, p)
        if ML.mode == "uvu":
            ML.x_block(dx, p["i1"])[...] += np.einsum("ijk,zjb,zka,zab->zia", C, yb, gb, wb)
            ML.y_block(dy, p["i2"])[...] += np.einsum("ijk,zia,zka,zab->zjb", C, xb, gb, wb)
            dwp = np.einsum("ijk,zia,zjb,zka->zab", C, xb, yb, gb)
        else:
            ML.x_block(dx, p["i1"])[...] += np.einsum("ijk,zjb,zkc,zabc->zia", C, yb, gb, wb)
            ML.y_block(dy, p["i2"])[...] += np.einsum("ijk,zia,zkc,zabc->zjb", C, xb, gb, wb)
            dwp = np.einsum("ijk,zia,zjb,zkc->zabc", C, xb, yb, gb)
        dw_rows[:, p["w_off"]:p["w_off"] + p["w_len"]] = dwp.reshape(B, -1)
    dw = dw_rows if w.ndim == 2 else dw_rows.sum(axis=0)
    return dx, dy, dw
