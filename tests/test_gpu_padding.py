"""GPU parity of padding-edge skipping against the oracle.

A fixed-shape caller pads the edge list with edges into one shared padding
node; a graph created with that node skips them: out[pad] = 0, zero grad_sh
and grad_w rows for them, no grad_x from them, and they are left out of the
transpose. Checked for the fused and general kernels, collapsed outputs, the
double backward, fp32 / bf16 / fp64, with 25 % padding edges (plus a few real
edges out of the padding node).
"""

import numpy as np
import pytest

from oracle import conv as oconv
from oracle import graph as ograph
from oracle import sh as osh
from oracle.irreps import Layout
from clebsch_gordan_tensor_amd import synth
from tests.gpu_util import assert_close, dev, host, out_blocks, w_blocks, x_blocks, y_blocks

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
if not torch.cuda.is_available():
    pytest.skip("no GPU", allow_module_level=True)
cgtp = pytest.importorskip("clebsch_gordan_tensor_amd.cgtp")


def padded_graph(seed=0):
    """60 points in a periodic box plus padding node 60: 25 % of the edges are
    padding edges 60 -> 60, and 5 real edges leave the padding node."""
    pos = synth.uniform_box(60, 6.0, seed)
    src, dst, vec = synth.radius_graph(pos, 6.0, 2.5)
    npad = len(src) // 3
    rng = np.random.default_rng(seed)
    out_of_pad = rng.integers(0, 60, 5)
    src = np.concatenate([src, np.full(npad, 60), np.full(5, 60)])
    dst = np.concatenate([dst, np.full(npad, 60), out_of_pad])
    vec = np.concatenate([vec, rng.standard_normal((npad + 5, 3))])
    row_ptr, s, perm = ograph.csr_from_coo(61, src, dst)
    return 61, row_ptr, s, vec[perm], npad


PLANS = [
    ("16x0e+16x1o+16x2e", "0e+1o+2e", "0e+0o+1e+1o+2e+2o", 2),
    ("3x1o+3x0e", "1o+1e", "0e+1o+1e+2e", -1),                # general kernels
]


@pytest.mark.parametrize("collapse", [False, True])
@pytest.mark.parametrize("ix,iy,io,lmax", PLANS)
@pytest.mark.parametrize("dtype", ["f32", "bf16", "f64"])
def test_padding_edges_skipped(ix, iy, io, lmax, collapse, dtype):
    L = Layout(ix, iy, io, "all", collapse)
    N, row_ptr, src, vec, npad = padded_graph(5)
    E = len(src)
    plan = cgtp.Plan(ix, iy, io, dtype=dtype, collapse=collapse)
    graph = cgtp.Graph(N, torch.from_numpy(row_ptr.astype(np.int32)).cuda(),
                       torch.from_numpy(src.astype(np.int32)).cuda(), pad_node=60)
    col_ptr, eid = graph.transpose()
    assert int(col_ptr[-1]) == E - npad and eid.shape[0] == E - npad
    Y = osh.real_sh(lmax, vec) if lmax >= 0 else synth.gaussian((E, L.dim_y), 6, synth.S_Y)
    h = [synth.gaussian((N, L.dim_x), 6, synth.S_X), Y, synth.gaussian((E, L.w_numel), 6, synth.S_W),
         synth.gaussian((N, L.dim_out), 6, synth.S_G)]
    d = [dev(a, dtype) for a in h]
    hd = [host(t) for t in d]
    gY, gw = dev(synth.gaussian((E, L.dim_y), 7, synth.S_Y), dtype), dev(synth.gaussian((E, L.w_numel), 7, synth.S_W), dtype)
    sc = 0.5
    tag = "%s collapse=%s %s" % (ix, collapse, dtype)
    out = plan.conv_forward(graph, d[0], d[1], d[2], sc)
    dx, dY, dw = plan.conv_backward(graph, d[0], d[1], d[2], sc, d[3])
    dd = plan.conv_double_backward(graph, d[0], d[1], d[2], sc, d[3], gg=(None, gY, gw))
    torch.cuda.synchronize()
    assert_close(host(out), oconv.forward(L, row_ptr, src, *hd[:3], sc, pad_node=60), out_blocks(L), dtype,
                 "padded forward " + tag)
    rdx, rdY, rdw = oconv.backward(L, row_ptr, src, *hd[:3], sc, hd[3], pad_node=60)
    assert_close(host(dx), rdx, x_blocks(L), dtype, "padded grad_x " + tag)
    assert_close(host(dY), rdY, y_blocks(L), dtype, "padded grad_sh " + tag)
    assert_close(host(dw), rdw, w_blocks(L), dtype, "padded grad_w " + tag)
    pe0, pe1 = row_ptr[60], row_ptr[61]
    assert float(dw[pe0:pe1].abs().max()) == 0.0 and float(dY[pe0:pe1].abs().max()) == 0.0
    rdd = oconv.double_backward(L, row_ptr, src, *hd[:3], sc, hd[3], None, host(gY), host(gw), pad_node=60)
    blocks = [x_blocks(L), y_blocks(L), w_blocks(L), out_blocks(L)]
    for k in range(4):
        assert_close(host(dd[k]), rdd[k], blocks[k], dtype, "padded double backward %d %s" % (k, tag))


def test_padding_node_out_of_range():
    rp = torch.zeros(4, dtype=torch.int32, device="cuda")
    s = torch.zeros(0, dtype=torch.int32, device="cuda")
    with pytest.raises(cgtp.CgtpError):
        cgtp.Graph(3, rp, s, pad_node=3)
