"""Graph layouts for the convolution (oracle; test infrastructure).

[V2106] "Fixed-topology compilation": a directed, loop-free radius graph; edges
given as edge_src / edge_dst. [COURSE] 05a: edge vector r_ij = r_j - r_i with
messages aggregated at the receiver i; periodic cells need the shifted image.
[E3J] E.2.2 / E.3: receiver (destination) ordered CSR aggregation without
atomics.

Reading taken: the CSR key is (dst, src) ascending, ties kept in input order
(a stable sort), so the order inside a destination segment is fixed and the
result does not depend on the input edge order. The transpose orders edges by
(src, CSR position).
"""

import numpy as np


def csr_from_coo(N, src, dst):
    """Return (row_ptr[N+1], src_sorted[E], perm[E]) for CSR by destination.

    perm[k] is the input index of the k-th CSR edge; np.lexsort is stable.
    """
    src = np.asarray(src, np.int64)
    dst = np.asarray(dst, np.int64)
    perm = np.lexsort((src, dst))
    counts = np.bincount(dst, minlength=N)
    row_ptr = np.zeros(N + 1, np.int64)
    row_ptr[1:] = np.cumsum(counts)
    return row_ptr, src[perm], perm


def csr_transpose(N, row_ptr, src_sorted):
    """Return (col_ptr[N+1], eid[E]): edges grouped by source, in CSR-position order."""
    src_sorted = np.asarray(src_sorted, np.int64)
    E = src_sorted.shape[0]
    pos = np.arange(E)
    eid = np.lexsort((pos, src_sorted))
    counts = np.bincount(src_sorted, minlength=N)
    col_ptr = np.zeros(N + 1, np.int64)
    col_ptr[1:] = np.cumsum(counts)
    return col_ptr, eid


def dst_of_csr(row_ptr):
    """Destination node of each CSR edge."""
    row_ptr = np.asarray(row_ptr, np.int64)
    N = row_ptr.shape[0] - 1
    return np.repeat(np.arange(N), np.diff(row_ptr))


def min_image(d, box):
    """Minimum-image displacement in a cubic periodic cell of side ``box``."""
    return d - box * np.round(d / box)


def radius_graph_bruteforce(pos, box, r_cut):
    """All ordered pairs (src=j -> dst=i), i != j, with |min_image(pos_j - pos_i)| < r_cut.

    O(N^2) over every pair; returns (src, dst, vec) sorted by (dst, src) with
    vec = min_image(pos[src] - pos[dst]) (the r_ij = r_j - r_i convention).
    """
    pos = np.asarray(pos, np.float64)
    N = pos.shape[0]
    srcs, dsts, vecs = [], [], []
    for i in range(N):
        d = min_image(pos - pos[i], box)          # row j: pos_j - pos_i
        r = np.linalg.norm(d, axis=1)
        js = np.nonzero((r < r_cut) & (np.arange(N) != i))[0]
        srcs.append(js)
        dsts.append(np.full(js.shape[0], i))
        vecs.append(d[js])
    return np.concatenate(srcs), np.concatenate(dsts), np.concatenate(vecs)
