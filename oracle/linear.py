"""Equivariant linear map (channel mixing) between irreps features (oracle; test infrastructure).

[E3J] A.3 lists linear mixing among the library's core operations, next to the
harmonic embedding, the tensor products and message passing; [COURSE] 03b
counts the weights of such layers and shows why mixing raw components would
break equivariance. Mixing channels only *within* one irrep type (same l and
parity) commutes with every rotation, since the Wigner-D matrix acts on the m
index and the weights on the channel index. Reading taken (the pages give no
formula; this is e3nn's o3.Linear): every pair (input block i, output block o)
with the same (l, parity) is a path with its own weight matrix W_p [u_i][v_o],
paths ordered input-major, and

  out[z, o, m, v] = sum over paths p = (i, o) of  sum_u x[z, i, m, u] W_p[u, v]

with no normalisation factor (a caller folds any scale into W). Output blocks
that no input reaches are zero. Rows are ir_mul blocks [2l+1][mul] as
everywhere else.

A fully connected ("uvw") tensor product with y of multiplicity 1 is this map
applied to the path outputs of the uvu product with unit weights.
"""

import numpy as np

from .irreps import block_offsets, dim, parse_irreps


class LinearLayout:
    """Blocks, paths and weight offsets of a linear map irreps_in -> irreps_out."""

    def __init__(self, irreps_in, irreps_out):
        self.I = parse_irreps(irreps_in) if isinstance(irreps_in, str) else list(irreps_in)
        self.O = parse_irreps(irreps_out) if isinstance(irreps_out, str) else list(irreps_out)
        self.in_off = block_offsets(self.I)
        self.out_off = block_offsets(self.O)
        self.dim_in, self.dim_out = dim(self.I), dim(self.O)
        self.paths = []
        w = 0
        for i, (mu, li, pi) in enumerate(self.I):
            for o, (mv, lo, po) in enumerate(self.O):
                if li == lo and pi == po:
                    self.paths.append(dict(i=i, o=o, l=li, mu=mu, mv=mv, w_off=w))
                    w += mu * mv
        self.w_numel = w

    def x_block(self, x, i):
        mu, l, _ = self.I[i]
        return x[:, self.in_off[i]:self.in_off[i] + mu * (2 * l + 1)].reshape(-1, 2 * l + 1, mu)

    def out_block(self, out, o):
        mv, l, _ = self.O[o]
        return out[:, self.out_off[o]:self.out_off[o] + mv * (2 * l + 1)].reshape(-1, 2 * l + 1, mv)

    def w_block(self, W, p):
        return W[p["w_off"]:p["w_off"] + p["mu"] * p["mv"]].reshape(p["mu"], p["mv"])


def forward(LL, x, W):
    """out [B, dim_out] from x [B, dim_in] and the flat weights W [w_numel]."""
    x = np.asarray(x, np.float64)
    W = np.asarray(W, np.float64)
    out = np.zeros((x.shape[0], LL.dim_out))
    for p in LL.paths:
        LL.out_block(out, p["o"])[...] += np.einsum("zmu,uv->zmv", LL.x_block(x, p["i"]), LL.w_block(W, p))
    return out


def backward(LL, x, W, g):
    """Cotangents (dx [B, dim_in], dW [w_numel]) for the output cotangent g."""
    x = np.asarray(x, np.float64)
    W = np.asarray(W, np.float64)
    g = np.asarray(g, np.float64)
    dx = np.zeros_like(x)
    dW = np.zeros(LL.w_numel)
    for p in LL.paths:
        gb = LL.out_block(g, p["o"])
        LL.x_block(dx, p["i"])[...] += np.einsum("zmv,uv->zmu", gb, LL.w_block(W, p))
        dW[p["w_off"]:p["w_off"] + p["mu"] * p["mv"]] = np.einsum("zmu,zmv->uv", LL.x_block(x, p["i"]), gb).ravel()
    return dx, dW
