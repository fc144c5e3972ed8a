"""The compute calls under HIP graph capture.

After a plan's first call on a device (which uploads its tables), every
compute call of the library is kernel launches on the caller's stream only, so
a caller can capture a whole step (double backward included) in a HIP graph
(torch.cuda.CUDAGraph) and replay it. Each test captures a step once, then replays it several times with
new values copied into the captured input tensors and the program's own eager
work (the same calls outside the graph) between replays; every replay must
equal the eager result bit for bit (the kernels are deterministic).
"""

import gc

import numpy as np
import pytest

from oracle import graph as ograph
from clebsch_gordan_tensor_amd import synth

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
if not torch.cuda.is_available():
    pytest.skip("no GPU", allow_module_level=True)
cgtp = pytest.importorskip("clebsch_gordan_tensor_amd.cgtp")

REPLAYS = 3


def capture(step):
    """Capture step() in a CUDA/HIP graph on a side stream (torch's recipe).

    Plans and graphs of earlier tests that sit in reference cycles (a
    pytest.raises traceback holds its test's frame) are freed by Python's
    cyclic collector whenever it runs; their destructors free device memory,
    and a hipFree during a global-mode capture invalidates it. So the collector
    runs before the capture and is off during it."""
    gc.collect()
    gc.disable()
    try:
        s = torch.cuda.Stream()
        s.wait_stream(torch.cuda.current_stream())
        g = torch.cuda.CUDAGraph()
        with torch.cuda.stream(s):
            with torch.cuda.graph(g, stream=s):
                step()
        torch.cuda.current_stream().wait_stream(s)
        torch.cuda.synchronize()
    finally:
        gc.enable()
    return g


def refill(tensors, seed):
    gen = torch.Generator(device="cuda")
    gen.manual_seed(seed)
    for t in tensors:
        t.copy_(torch.randn(t.shape, generator=gen, device="cuda", dtype=t.dtype))


def check_replays(graph, inputs, outputs, eager, tag):
    """Replay with new inputs; eager() recomputes into fresh tensors."""
    for k in range(REPLAYS):
        refill(inputs, 100 + k)
        expect = eager()                      # the program's own work between replays
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        for i, (got, exp) in enumerate(zip(outputs, expect)):
            assert torch.equal(got, exp), "%s: output %d differs on replay %d" % (tag, i, k)


@pytest.mark.parametrize("wkind", ["shared", "per_row"])
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_tensor_product_step(wkind, dtype):
    c = synth.CONFIGS["tp_small"]
    plan = cgtp.Plan(c["irreps_x"], c["irreps_y"], c["irreps_out"], dtype=dtype, wkind=wkind)
    td = plan.torch_dtype
    B = 1000
    vec = torch.randn(B, 3, device="cuda", dtype=torch.float32).to(td)
    x = torch.randn(B, plan.dim_x, device="cuda").to(td)
    w = torch.randn(*((plan.w_numel,) if wkind == "shared" else (B, plan.w_numel)), device="cuda").to(td)
    g = torch.randn(B, plan.dim_out, device="cuda").to(td)
    y = torch.empty(B, plan.dim_y, device="cuda", dtype=td)
    out = torch.empty(B, plan.dim_out, device="cuda", dtype=td)
    dx, dy, dw = torch.empty_like(x), torch.empty_like(y), torch.empty_like(w)
    ws = torch.empty(max(plan.workspace_size(cgtp.OP_TP_BACKWARD, B), 1), dtype=torch.uint8, device="cuda")
    gx, gy, gw = torch.randn_like(x), torch.randn_like(y), torch.randn_like(w)
    dd = [torch.empty_like(t) for t in (x, y, w, g)]
    ws2 = torch.empty(plan.workspace_size(cgtp.OP_TP_DOUBLE_BACKWARD, B), dtype=torch.uint8, device="cuda")

    def step():
        cgtp.sh_forward(c["L"], vec, out=y)
        plan.tp_forward(x, y, w, out=out)
        plan.tp_backward(x, y, w, g, out=(dx, dy, dw), ws=ws)
        plan.tp_double_backward(x, y, w, g, gg=(gx, gy, gw), out=tuple(dd), ws=ws2)

    step()                                    # first call uploads the plan's tables
    torch.cuda.synchronize()
    graph = capture(step)

    def eager():
        ye = cgtp.sh_forward(c["L"], vec)
        oe = plan.tp_forward(x, ye, w)
        return ((ye, oe) + tuple(plan.tp_backward(x, ye, w, g))
                + tuple(plan.tp_double_backward(x, ye, w, g, gg=(gx, gy, gw))))

    check_replays(graph, [vec, x, w, g, gx, gw], [y, out, dx, dy, dw] + dd, eager, "tp %s %s" % (dtype, wkind))


@pytest.mark.parametrize("collapse", [False, True])
def test_convolution_step(collapse):
    """Harmonics, convolution forward and backward, harmonics backward and the
    double backward (the force-training step of the library) on a small radius
    graph; the collapsed plan also captures its output fill kernel."""
    ix, iy, io, L = "16x0e+16x1o+16x2e", "0e+1o+2e", "0e+0o+1e+1o+2e+2o", 2
    plan = cgtp.Plan(ix, iy, io, collapse=collapse)
    pos = synth.uniform_box(80, 6.0, 3)
    src, dst, vec_np = synth.radius_graph(pos, 6.0, 2.5)
    N = 80
    row_ptr, s, perm = ograph.csr_from_coo(N, src, dst)
    E = len(s)
    graph = cgtp.Graph(N, torch.from_numpy(row_ptr.astype(np.int32)).cuda(), torch.from_numpy(s.astype(np.int32)).cuda())
    vec = torch.from_numpy(vec_np[perm]).float().cuda()
    x = torch.randn(N, plan.dim_x, device="cuda")
    w = torch.randn(E, plan.w_numel, device="cuda")
    g = torch.randn(N, plan.dim_out, device="cuda")
    Y = torch.empty(E, plan.dim_y, device="cuda")
    out = torch.empty(N, plan.dim_out, device="cuda")
    dx, dY, dw = torch.empty_like(x), torch.empty_like(Y), torch.empty_like(w)
    gvec = torch.empty_like(vec)
    ws = torch.empty(plan.workspace_size(cgtp.OP_CONV_BACKWARD, graph=graph), dtype=torch.uint8, device="cuda")
    sc = 0.37

    gY, gw = torch.randn_like(Y), torch.randn_like(w)
    dd = [torch.empty_like(t) for t in (x, Y, w, g)]
    ws2 = torch.empty(plan.workspace_size(cgtp.OP_CONV_DOUBLE_BACKWARD, graph=graph), dtype=torch.uint8,
                      device="cuda")

    def step():
        cgtp.sh_forward(L, vec, out=Y)
        plan.conv_forward(graph, x, Y, w, sc, out=out)
        plan.conv_backward(graph, x, Y, w, sc, g, out=(dx, dY, dw), ws=ws)
        cgtp.sh_backward(L, vec, dY, out=gvec)
        plan.conv_double_backward(graph, x, Y, w, sc, g, gg=(None, gY, gw), out=tuple(dd), ws=ws2)

    step()
    torch.cuda.synchronize()
    hg = capture(step)

    def eager():
        Ye = cgtp.sh_forward(L, vec)
        oe = plan.conv_forward(graph, x, Ye, w, sc)
        dxe, dYe, dwe = plan.conv_backward(graph, x, Ye, w, sc, g)
        return ((Ye, oe, dxe, dYe, dwe, cgtp.sh_backward(L, vec, dYe))
                + tuple(plan.conv_double_backward(graph, x, Ye, w, sc, g, gg=(None, gY, gw))))

    check_replays(hg, [vec, x, w, g, gY, gw], [Y, out, dx, dY, dw, gvec] + dd, eager,
                  "conv collapse=%s" % collapse)


def test_linear_step():
    irreps = "32x0e+32x1o+32x2e"
    lin = cgtp.Linear(irreps, irreps)
    B = 700
    x = torch.randn(B, lin.dim_in, device="cuda")
    w = torch.randn(lin.w_numel, device="cuda")
    g = torch.randn(B, lin.dim_out, device="cuda")
    out, dx, dw = torch.empty(B, lin.dim_out, device="cuda"), torch.empty_like(x), torch.empty_like(w)
    ws = torch.empty(max(lin.workspace_size(B), 1), dtype=torch.uint8, device="cuda")

    def step():
        lin.forward(x, w, out=out)
        lin.backward(x, w, g, out=(dx, dw), ws=ws)

    step()
    torch.cuda.synchronize()
    hg = capture(step)

    def eager():
        return (lin.forward(x, w),) + tuple(lin.backward(x, w, g))

    check_replays(hg, [x, w, g], [out, dx, dw], eager, "linear")


def test_forked_launches_under_capture():
    """Calls that move enough memory run their x-block launches on the
    library's own streams beside the caller's (fork and join by events). Under
    capture those waits become graph dependencies: the tensor-product forward
    and the convolution forward and backward of sizes that fork are captured
    and replayed, each replay bitwise equal to eager calls."""
    c = synth.CONFIGS["tp_small"]
    plan = cgtp.Plan(c["irreps_x"], c["irreps_y"], c["irreps_out"], wkind="per_row")
    B = 40000
    assert B * (plan.dim_out + plan.dim_x) * 4 >= 256 << 20      # the forward forks
    x = torch.randn(B, plan.dim_x, device="cuda")
    y = torch.randn(B, plan.dim_y, device="cuda")
    w = torch.randn(B, plan.w_numel, device="cuda")
    out = torch.empty(B, plan.dim_out, device="cuda")

    ix, iy, io = "64x0e+64x1o+64x2e", "0e+1o+2e", "0e+0o+1e+1o+2e+2o"
    cp = cgtp.Plan(ix, iy, io)
    pos = synth.uniform_box(4000, 20.0, 7)
    src, dst, _ = synth.radius_graph(pos, 20.0, 3.0)
    N = pos.shape[0]
    row_ptr, s, _ = ograph.csr_from_coo(N, src, dst)
    E = len(s)
    assert E * (cp.w_numel + cp.dim_y) * 4 >= 256 << 20          # the convolution calls fork
    graph = cgtp.Graph(N, torch.from_numpy(row_ptr.astype(np.int32)).cuda(),
                       torch.from_numpy(s.astype(np.int32)).cuda())
    cx = torch.randn(N, cp.dim_x, device="cuda")
    Y = torch.randn(E, cp.dim_y, device="cuda")
    cw = torch.randn(E, cp.w_numel, device="cuda")
    g = torch.randn(N, cp.dim_out, device="cuda")
    cout = torch.empty(N, cp.dim_out, device="cuda")
    dx, dY, dw = torch.empty_like(cx), torch.empty_like(Y), torch.empty_like(cw)
    ws = torch.empty(cp.workspace_size(cgtp.OP_CONV_BACKWARD, graph=graph), dtype=torch.uint8, device="cuda")
    sc = 0.21

    def step():
        plan.tp_forward(x, y, w, out=out)
        cp.conv_forward(graph, cx, Y, cw, sc, out=cout)
        cp.conv_backward(graph, cx, Y, cw, sc, g, out=(dx, dY, dw), ws=ws)

    step()
    torch.cuda.synchronize()
    hg = capture(step)

    def eager():
        return ((plan.tp_forward(x, y, w), cp.conv_forward(graph, cx, Y, cw, sc))
                + tuple(cp.conv_backward(graph, cx, Y, cw, sc, g)))

    check_replays(hg, [x, y, w, cx, Y, cw, g], [out, cout, dx, dY, dw], eager, "forked launches")
