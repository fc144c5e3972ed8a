"""Seeded synthetic workloads shared by the oracle tests, the GPU tests and the bench.

This module holds no tensor-product, harmonic or aggregation arithmetic: only
random draws, the geometry of synthetic boxes, the neighbour search that turns
positions into an edge list, and the radial network that turns distances into
per-edge weights (the caller's model, outside the library).

Workloads stand in for the water-box MACE runs of [E3J] 1 and 3.2 (periodic
water boxes, uniform point clouds); no dataset is read.

Seeds: every tensor draws from its own child of ``SeedSequence(seed)`` spawned
with a fixed stream index, so adding a tensor never changes another one.
"""

import math

import numpy as np

# stream indices of SeedSequence(seed).spawn(...)
S_X, S_Y, S_W, S_VEC, S_G, S_POS, S_ORIENT, S_MLP1, S_MLP2 = range(9)


def rng(seed, stream):
    return np.random.default_rng(np.random.SeedSequence(seed).spawn(stream + 1)[stream])


def gaussian(shape, seed, stream):
    return rng(seed, stream).standard_normal(shape)


def unit_vectors(n, seed, stream=S_VEC):
    """Uniform random directions: normalised standard-normal triples."""
    v = rng(seed, stream).standard_normal((n, 3))
    return v / np.linalg.norm(v, axis=1, keepdims=True)


def to_bf16_values(a):
    """Round fp64/fp32 values to the nearest bfloat16 (ties to even), returned as float32."""
    a32 = np.ascontiguousarray(a, dtype=np.float32)
    u = a32.view(np.uint32).astype(np.uint64)
    lsb = (u >> 16) & 1
    u = (u + 0x7FFF + lsb) & 0xFFFF0000
    return u.astype(np.uint32).view(np.float32)


# ----------------------------------------------------------------- geometry

def _random_rotations(n, r):
    """Haar-random rotation matrices from uniform unit quaternions (Shoemake)."""
    u1, u2, u3 = r.random(n), r.random(n), r.random(n)
    q = np.stack([np.sqrt(1 - u1) * np.sin(2 * np.pi * u2),
                  np.sqrt(1 - u1) * np.cos(2 * np.pi * u2),
                  np.sqrt(u1) * np.sin(2 * np.pi * u3),
                  np.sqrt(u1) * np.cos(2 * np.pi * u3)], axis=1)
    x, y, z, w = q.T
    R = np.empty((n, 3, 3))
    R[:, 0, 0] = 1 - 2 * (y * y + z * z)
    R[:, 0, 1] = 2 * (x * y - z * w)
    R[:, 0, 2] = 2 * (x * z + y * w)
    R[:, 1, 0] = 2 * (x * y + z * w)
    R[:, 1, 1] = 1 - 2 * (x * x + z * z)
    R[:, 1, 2] = 2 * (y * z - x * w)
    R[:, 2, 0] = 2 * (x * z - y * w)
    R[:, 2, 1] = 2 * (y * z + x * w)
    R[:, 2, 2] = 1 - 2 * (x * x + y * y)
    return R


def water_box(n_mol, box, seed, r_oh=0.96, angle_deg=104.5, min_oo=2.5):
    """Periodic cubic box of rigid water molecules.

    Oxygens are placed by random sequential insertion, rejecting any trial
    closer than ``min_oo`` (minimum image) to an accepted oxygen; each molecule
    gets a Haar-random orientation. Atom order is (O, H, H) per molecule and
    positions are wrapped into [0, box). Returns positions [3*n_mol, 3].
    """
    r = rng(seed, S_POS)
    ncell = max(1, int(box // min_oo))
    cs = box / ncell
    cells = {}
    oxy = np.empty((n_mol, 3))
    k = 0
    trials = 0
    while k < n_mol:
        trials += 1
        if trials > 200 * n_mol + 10000:
            raise RuntimeError("water_box: could not place %d molecules" % n_mol)
        p = r.random(3) * box
        c = np.floor(p / cs).astype(int) % ncell
        ok = True
        for dx in (-1, 0, 1):
            for dy in (-1, 0, 1):
                for dz in (-1, 0, 1):
                    key = ((c[0] + dx) % ncell, (c[1] + dy) % ncell, (c[2] + dz) % ncell)
                    for j in cells.get(key, ()):
                        d = oxy[j] - p
                        d -= box * np.round(d / box)
                        if d @ d < min_oo * min_oo:
                            ok = False
                            break
                    if not ok:
                        break
                if not ok:
                    break
            if not ok:
                break
        if ok:
            oxy[k] = p
            cells.setdefault((c[0], c[1], c[2]), []).append(k)
            k += 1
    half = math.radians(angle_deg) / 2.0
    ref = np.array([[0.0, 0.0, 0.0],
                    [r_oh * math.sin(half), 0.0, r_oh * math.cos(half)],
                    [-r_oh * math.sin(half), 0.0, r_oh * math.cos(half)]])
    R = _random_rotations(n_mol, rng(seed, S_ORIENT))
    atoms = oxy[:, None, :] + np.einsum("mij,aj->mai", R, ref)
    return np.mod(atoms.reshape(-1, 3), box)


def uniform_box(n, box, seed):
    """n points uniform in [0, box)^3."""
    return rng(seed, S_POS).random((n, 3)) * box


def radius_graph(pos, box, r_cut):
    """Directed, loop-free periodic radius graph (src=j -> dst=i for |r_j - r_i| < r_cut).

    Uses a periodic k-d tree for the candidate pairs, then keeps the strict
    inequality. Requires r_cut < box/2 (one image per pair). Returns
    (src, dst, vec) sorted by (dst, src), vec = min_image(pos[src] - pos[dst]).
    """
    from scipy.spatial import cKDTree

    if not r_cut < box / 2:
        raise ValueError("radius_graph needs r_cut < box/2")
    pos = np.mod(np.asarray(pos, np.float64), box)
    tree = cKDTree(pos, boxsize=box)
    pairs = tree.query_pairs(r_cut, output_type="ndarray")
    i, j = pairs[:, 0], pairs[:, 1]
    d = pos[j] - pos[i]
    d -= box * np.round(d / box)
    keep = np.einsum("ij,ij->i", d, d) < r_cut * r_cut
    i, j, d = i[keep], j[keep], d[keep]
    src = np.concatenate([j, i])
    dst = np.concatenate([i, j])
    vec = np.concatenate([d, -d])
    order = np.lexsort((src, dst))
    return src[order], dst[order], vec[order]


# ------------------------------------------------------------ radial network

def bessel_envelope(r, r_cut, n_basis=8, p=6):
    """Bessel radial basis times a polynomial envelope ([COURSE] 05b).

    B_n(r) = sqrt(2/r_cut) sin(n pi r / r_cut) / r, n = 1..n_basis, times the
    DimeNet envelope u(d) = 1 - (p+1)(p+2)/2 d^p + p(p+2) d^{p+1} - p(p+1)/2 d^{p+2}
    (d = r/r_cut, zero beyond the cut-off). Returns [E, n_basis] fp64.
    """
    r = np.asarray(r, np.float64)
    d = r / r_cut
    n = np.arange(1, n_basis + 1)
    b = math.sqrt(2.0 / r_cut) * np.sin(n[None, :] * np.pi * d[:, None]) / r[:, None]
    u = (1 - (p + 1) * (p + 2) / 2 * d ** p + p * (p + 2) * d ** (p + 1) - p * (p + 1) / 2 * d ** (p + 2))
    u = np.where(d < 1.0, u, 0.0)
    return b * u[:, None]


def mlp_params(n_in, hidden, n_out, seed):
    """Random-init two-layer MLP (no biases): N(0,1)/sqrt(fan_in)."""
    W1 = rng(seed, S_MLP1).standard_normal((n_in, hidden)) / math.sqrt(n_in)
    W2 = rng(seed, S_MLP2).standard_normal((hidden, n_out)) / math.sqrt(hidden)
    return W1, W2


def _silu(a):
    return a / (1.0 + np.exp(-a))


def radial_weights_np(r, r_cut, W1, W2):
    """Per-edge weights: Linear(8->64) -> SiLU -> Linear(64->W), fp64 on the host."""
    return _silu(bessel_envelope(r, r_cut) @ W1) @ W2


def radial_weights_backward_np(r, r_cut, W1, W2, dw, eps=None):
    """d/dr of sum(dw * radial_weights_np(r)), analytic, fp64. Returns [E]."""
    r = np.asarray(r, np.float64)
    p = 6
    d = r / r_cut
    n = np.arange(1, 9)
    s = np.sin(n[None, :] * np.pi * d[:, None])
    c = np.cos(n[None, :] * np.pi * d[:, None])
    k = math.sqrt(2.0 / r_cut)
    b = k * s / r[:, None]
    db = k * (c * (n[None, :] * np.pi / r_cut) / r[:, None] - s / (r[:, None] ** 2))
    u = (1 - (p + 1) * (p + 2) / 2 * d ** p + p * (p + 2) * d ** (p + 1) - p * (p + 1) / 2 * d ** (p + 2))
    du = (-(p + 1) * (p + 2) / 2 * p * d ** (p - 1) + p * (p + 2) * (p + 1) * d ** p
          - p * (p + 1) / 2 * (p + 2) * d ** (p + 1)) / r_cut
    inside = d < 1.0
    u = np.where(inside, u, 0.0)
    du = np.where(inside, du, 0.0)
    f = b * u[:, None]
    df = db * u[:, None] + b * du[:, None]
    a = f @ W1
    sig = 1.0 / (1.0 + np.exp(-a))
    h = a * sig
    dh = dw @ W2.T
    da = dh * (sig + a * sig * (1 - sig))
    dfe = da @ W1.T
    return np.einsum("ek,ek->e", dfe, df)


def radial_weights_torch(r, r_cut, W1, W2):
    """Same network on a torch device (r: 1-D tensor; W1, W2 tensors); differentiable in r."""
    import torch

    p = 6
    d = r / r_cut
    n = torch.arange(1, 9, device=r.device, dtype=r.dtype)
    b = math.sqrt(2.0 / r_cut) * torch.sin(n[None, :] * math.pi * d[:, None]) / r[:, None]
    u = (1 - (p + 1) * (p + 2) / 2 * d ** p + p * (p + 2) * d ** (p + 1) - p * (p + 1) / 2 * d ** (p + 2))
    u = torch.where(d < 1.0, u, torch.zeros_like(u))
    a = (b * u[:, None]) @ W1
    return torch.nn.functional.silu(a) @ W2


# ------------------------------------------------------------ configurations

# The five workloads of the benchmark description, with the irreps readings:
# "all parity-allowed paths to lout <= L" keeps both parities for every l <= L.
def _sh_irreps(L):
    return "+".join("1x%d%s" % (l, "e" if l % 2 == 0 else "o") for l in range(L + 1))


def _out_irreps(L):
    return "+".join("%d%s" % (l, par) for l in range(L + 1) for par in ("e", "o"))


CONFIGS = {
    "tp_small": dict(kind="tp", irreps_x="32x0e+32x1o+32x2e", L=2, B=4096, wkind="shared"),
    "tp_large": dict(kind="tp", irreps_x="128x0e+128x1o+128x2e+128x3o", L=3, B=1048576,
                     wkind="per_row"),
    "conv_water1k": dict(kind="conv", irreps_x="128x0e+128x1o", L=3, system="water",
                         n_mol=1000, box=31.0, r_cut=5.0),
    "conv_water8k": dict(kind="conv", irreps_x="128x0e+128x1o+128x2e", L=3, system="water",
                         n_mol=8000, box=62.1, r_cut=6.0),
    "conv_uniform100k": dict(kind="conv", irreps_x="64x0e+64x1o+64x2e+64x3o+64x4e", L=4,
                             system="uniform", n=100000, box=100.0, r_cut=5.0),
    # The collapsed-output comparison setting of [E3J] B.3: 2048 nodes, 45 edges per
    # node, 128 channels per degree; uniform points in a periodic cube with the
    # cutoff giving 45 neighbours on average (4/3 pi r^3 * 2047 / 20^3 = 45).
    "conv_collapsed_l3": dict(kind="conv", irreps_x="128x0e+128x1o+128x2e+128x3o", L=3, system="uniform",
                              n=2048, box=20.0, r_cut=3.475, collapse=True),
    "conv_collapsed_l4": dict(kind="conv", irreps_x="128x0e+128x1o+128x2e+128x3o+128x4e", L=4,
                              system="uniform", n=2048, box=20.0, r_cut=3.475, collapse=True),
}
for _c in CONFIGS.values():
    _c["irreps_y"] = _sh_irreps(_c["L"])
    _c["irreps_out"] = _out_irreps(_c["L"])


def positions_for(cfg, seed=0):
    if cfg["system"] == "water":
        return water_box(cfg["n_mol"], cfg["box"], seed)
    return uniform_box(cfg["n"], cfg["box"], seed)
