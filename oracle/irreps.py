"""Irreps strings, tensor-product paths and row layouts (oracle; test infrastructure).

Follows [COURSE] lesson 02a ("Irreps as a type system": an irreps string such as
"16x0e + 8x1o" lists multiplicity x degree with parity e/o) and lesson 03a (the
parity rule p3 = p1 * p2 and the Clebsch-Gordan decomposition of l1 x l2 into
|l1-l2| ... l1+l2). The uvu connection mode of lesson 03b is read as e3nn's
channel-wise mode: output channel u = the x channel, one weight per (path, u),
and the second operand carries multiplicity 1.
"""

import re

IRREP_RE = re.compile(r"(?:(\d+)x)?(\d+)([eo])")


def parse_irreps(s):
    """Parse "MxLp + ..." into a list of (mul, l, parity) tuples, order kept.

    Whitespace is ignored, a missing "Mx" means multiplicity 1, parity e -> +1,
    o -> -1 ([COURSE] 02a). An empty string is the empty list.
    """
    s = "".join(s.split())
    if s == "":
        return []
    out = []
    for term in s.split("+"):
        m = IRREP_RE.fullmatch(term)
        if m is None:
            raise ValueError("bad irreps term %r in %r" % (term, s))
        mul = int(m.group(1)) if m.group(1) is not None else 1
        if mul < 1:
            raise ValueError("multiplicity must be >= 1 in %r" % term)
        out.append((mul, int(m.group(2)), 1 if m.group(3) == "e" else -1))
    return out


def block_dims(irreps):
    """Element count of each block: mul * (2l+1)."""
    return [mul * (2 * l + 1) for mul, l, _ in irreps]


def block_offsets(irreps):
    """Start offset of each block inside a row (blocks are concatenated)."""
    offs, o = [], 0
    for d in block_dims(irreps):
        offs.append(o)
        o += d
    return offs


def dim(irreps):
    return sum(block_dims(irreps))


SELECTIONS = ("all", "symmetric", "skew")


def paths_uvu(irreps_x, irreps_y, irreps_out, select="all"):
    """Enumerate the uvu paths of the full tensor product.

    For every x block i1, every y block i2 and every l3 in |l1-l2| ... l1+l2
    (the Clebsch-Gordan decomposition, [COURSE] 03a) the output parity is
    p3 = p1 * p2 ([COURSE] 03a); the path is kept when (l3, p3) occurs in
    irreps_out, whose multiplicities are ignored (it is a filter).
    Order: i1, then i2, then l3 ascending. One output block per path, not
    collapsed (collapsing by degree is a separate comparison mode in [E3J] B.1).

    ``select`` keeps a parity class of paths ([E3J] B.1: the Gaunt product
    covers the symmetric paths, the vector signal product the skew-symmetric
    ones, and e3j picks the matching paths by parity): "symmetric" keeps
    l1 + l2 + l3 even, "skew" keeps it odd, "all" keeps every path.

    Returns a list of dicts with keys i1, i2, l1, l2, l3, p3, mul.
    """
    if select not in SELECTIONS:
        raise ValueError("select must be one of %s" % (SELECTIONS,))
    X, Y, O = parse_irreps(irreps_x), parse_irreps(irreps_y), parse_irreps(irreps_out)
    allowed = {(l, p) for _, l, p in O}
    for mul, _, _ in Y:
        if mul != 1:
            raise ValueError("uvu needs multiplicity 1 on the second operand")
    paths = []
    for i1, (u, l1, p1) in enumerate(X):
        for i2, (_, l2, p2) in enumerate(Y):
            for l3 in range(abs(l1 - l2), l1 + l2 + 1):
                p3 = p1 * p2
                if select != "all" and ((l1 + l2 + l3) % 2 == 0) != (select == "symmetric"):
                    continue
                if (l3, p3) in allowed:
                    paths.append(dict(i1=i1, i2=i2, l1=l1, l2=l2, l3=l3, p3=p3, mul=u))
    return paths


class Layout:
    """Row layouts of x, y, out and w for a uvu plan.

    Within a block the layout is [2l+1][mul] (the ir_mul order of [COURSE] 12a:
    the channel index is the fast one). Output blocks follow path order; the
    weights of a row are [path][mul] concatenated.

    With ``collapse`` the paths of one output type are summed into one block
    ([E3J] B.1 and B.3: outputs collapsed by degree, summing the isomorphic
    copies of each irreducible output space). Reading taken: one block per
    (l3, p3) that some path reaches, blocks in the order of irreps_out (first
    occurrence), multiplicity = that of the x blocks feeding it, which must
    agree. ``groups`` lists the output blocks as dicts (l3, p3, mul, out_off).
    """

    def __init__(self, irreps_x, irreps_y, irreps_out, select="all", collapse=False):
        self.X = parse_irreps(irreps_x)
        self.Y = parse_irreps(irreps_y)
        self.paths = paths_uvu(irreps_x, irreps_y, irreps_out, select)
        self.select, self.collapse = select, collapse
        self.x_off = block_offsets(self.X)
        self.y_off = block_offsets(self.Y)
        self.dim_x = dim(self.X)
        self.dim_y = dim(self.Y)
        w = 0
        for p in self.paths:
            p["w_off"] = w
            w += p["mul"]
        self.w_numel = w
        self.groups = []
        if not collapse:
            o = 0
            for p in self.paths:
                p["out_off"] = o
                self.groups.append(dict(l3=p["l3"], p3=p["p3"], mul=p["mul"], out_off=o))
                o += p["mul"] * (2 * p["l3"] + 1)
            self.dim_out = o
            return
        order = []
        for _, l, par in parse_irreps(irreps_out):
            if (l, par) not in order:
                order.append((l, par))
        o = 0
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
        """View of block i of x rows as [..., 2l+1, mul]."""
        mul, l, _ = self.X[i]
        o = self.x_off[i]
        return x[..., o:o + mul * (2 * l + 1)].reshape(x.shape[:-1] + (2 * l + 1, mul))

    def y_block(self, y, i):
        _, l, _ = self.Y[i]
        o = self.y_off[i]
        return y[..., o:o + 2 * l + 1]

    def out_block(self, out, p):
        o = p["out_off"]
        n = 2 * p["l3"] + 1
        return out[..., o:o + n * p["mul"]].reshape(out.shape[:-1] + (n, p["mul"]))

    def w_block(self, w, p):
        return w[..., p["w_off"]:p["w_off"] + p["mul"]]
