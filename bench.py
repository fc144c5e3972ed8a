"""Benchmark of the hot path on one MI355X; prints one JSON line.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload tp_large]
                    [--no-conv] [--no-extra] [--no-cpu-baseline]
    python bench.py --profile WORKLOAD      (a few calls of every operation, for rocprofv3)
    python bench.py --calibrate-copy        (a plain copy of known size, for the byte counters)

Workload (default tp_large): 1,048,576 rows of x = 128x(0e+1o+2e+3o), y = the
real spherical harmonics (L = 3) of random unit vectors, per-row weights for
all 34 paths to lout <= 3, fp32. One step = harmonics of the row directions
(cgtp_sh_forward) -> tensor product forward -> tensor product backward (grads
of x, y and w), with every input already resident in HBM. `value` is rows
("pairs") per second of whole steps.

Besides the headline line's `roofline` (dominant kernel, algorithmic bytes per
call over its mean HIP-event duration against 8 TB/s) and `cpu_baseline` (the
fp64 oracle on a bounded sample, on the host cores), `extra` carries the
per-kernel figures, the same workload in bf16 storage and with outputs
collapsed by (l3, p3) (all, symmetric and skew path sets), the equivariant
linear map on the same rows (matrix cores) and, unless --no-conv,
the fused convolution (forward and backward, fp32) on the 1000- and
8000-molecule water boxes (the latter with the harmonics forward/backward of
the force chain), the 100,000-point uniform cloud, and 2048 points with 45
neighbours and 128 channels per degree with outputs collapsed by (l3, p3)
(L = 3 and 4), the water8k double backward in the force-training shape, and
water1k with 25 % padding edges with and without padding-edge skipping.
"""

import argparse
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0
METRIC = "TP pairs/s + conv edges/s (fwd, fwd+bwd) as HBM GB/s and % of MI355X peak"
PROFILES = os.path.join(ROOT, "profiles")
WORKLOADS = ["tp_large", "tp_large_bf16", "conv_water1k", "conv_water8k", "conv_uniform100k", "linear_large",
             "linear_large_bf16", "tp_large_collapsed", "conv_collapsed_l3", "conv_collapsed_l4",
             "conv_uniform100k_f64", "conv_water8k_radial", "conv_uniform100k_radial", "uvw_tp_large",
             "uvw_tp_large_bf16"]
MFMA_FP32_PEAK_TFS = 157.3
MFMA_BF16_PEAK_TFS = 2500.0


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=10)
    ap.add_argument("--warmup", type=int, default=2)
    ap.add_argument("--workload", default="tp_large", choices=["tp_large"])
    ap.add_argument("--no-conv", action="store_true")
    ap.add_argument("--no-extra", action="store_true",
                    help="only the headline step (for a kernel trace of exactly its launches)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=12.0, help="target oracle time")
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="only run a plain 4 GiB device copy (reference for HBM byte counters) and exit")
    ap.add_argument("--profile", choices=WORKLOADS, default=None,
                    help="only run a few calls of every operation of one workload (for rocprofv3) and exit")
    return ap.parse_args()


def calibrate_copy(torch):
    """A plain elementwise copy of known size: 4 GiB read + 4 GiB written per launch."""
    n = 1 << 30
    a = torch.ones(n, device="cuda")
    b = torch.empty_like(a)
    for _ in range(3):
        torch.mul(a, 1.0, out=b)
    torch.cuda.synchronize()
    print(json.dumps({"calibration": "elementwise copy", "bytes_read_per_launch": 4 * n,
                      "bytes_written_per_launch": 4 * n, "launches": 3}), flush=True)


def traffic_for(kernel, workload, units):
    """HBM bytes of one call from the committed counter summary, or None when the
    kernel's sources changed since the counters were taken."""
    from clebsch_gordan_tensor_amd.profsum import source_hash
    path = os.path.join(PROFILES, "hbm_traffic.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        rec = json.load(f).get("%s@%s" % (kernel, workload))
    if not rec or rec.get("source_hash") != source_hash(rec["sources"]):
        return None
    return rec["bytes_per_unit"] * units


class KernelTimer:
    """Mean device duration of one call site, from HIP events on the launch stream."""

    def __init__(self, torch):
        self.torch = torch
        self.pairs = []

    def __call__(self, fn):
        s = self.torch.cuda.Event(enable_timing=True)
        e = self.torch.cuda.Event(enable_timing=True)
        s.record()
        r = fn()
        e.record()
        self.pairs.append((s, e))
        return r

    def mean_ms(self):
        return sum(s.elapsed_time(e) for s, e in self.pairs) / len(self.pairs)


# ------------------------------------------------------------------ workloads

class TPWorkload:
    """tp_large: 2^20 rows, per-row weights; fp32 (with the harmonics of the row
    directions computed in the step) or bf16 storage (harmonics drawn directly)."""

    def __init__(self, torch, cgtp, synth, dtype, select="all", collapse=False):
        c = synth.CONFIGS["tp_large"]
        self.torch, self.cgtp, self.dtype = torch, cgtp, dtype
        self.plan = cgtp.Plan(c["irreps_x"], c["irreps_y"], c["irreps_out"], dtype=dtype, wkind="per_row",
                              select=select, collapse=collapse)
        self.irreps_x = c["irreps_x"]
        self.B = B = c["B"]
        p = self.plan
        gen = torch.Generator(device="cuda")
        gen.manual_seed(0)
        td = torch.float32 if dtype == "f32" else torch.bfloat16
        self.x = torch.randn((B, p.dim_x), generator=gen, device="cuda").to(td)
        self.w = torch.randn((B, p.w_numel), generator=gen, device="cuda").to(td)
        self.g = torch.randn((B, p.dim_out), generator=gen, device="cuda").to(td)
        if dtype == "f32":
            v = torch.randn((B, 3), generator=gen, device="cuda")
            self.v = v / v.norm(dim=1, keepdim=True)
            self.y = torch.empty((B, p.dim_y), device="cuda")
            cgtp.sh_forward(3, self.v, out=self.y)
        else:
            self.v = None
            self.y = torch.randn((B, p.dim_y), generator=gen, device="cuda").to(td)
        self.out = torch.empty((B, p.dim_out), device="cuda", dtype=td)
        self.dx, self.dy, self.dw = torch.empty_like(self.x), torch.empty_like(self.y), torch.empty_like(self.w)
        self.es = 4 if dtype == "f32" else 2

    def sh(self):
        if self.v is not None:
            self.cgtp.sh_forward(3, self.v, out=self.y)

    def fwd(self):
        self.plan.tp_forward(self.x, self.y, self.w, out=self.out)

    def bwd(self):
        self.plan.tp_backward(self.x, self.y, self.w, self.g, out=(self.dx, self.dy, self.dw))

    def bytes_fwd(self):  # per row: x, y, w read, out written
        p = self.plan
        return self.es * (p.dim_x + p.dim_y + p.w_numel + p.dim_out)

    def bytes_bwd(self):  # per row: x, y, w, grad_out read, grad x, y, w written
        p = self.plan
        return self.es * (2 * p.dim_x + 2 * p.dim_y + 2 * p.w_numel + p.dim_out)


class ConvWorkload:
    """One convolution workload at full size: graph, harmonics and radial
    weights built as the benchmark description states (weights by the caller's
    radial network, not timed), then forward / backward calls. fp32 by default;
    ``dtype="f64"`` builds the inputs in fp64 for the forward alone (the grads
    of the 100k-point workload would not fit beside fp64 weights)."""

    def __init__(self, torch, cgtp, synth, name, dtype="f32"):
        import numpy as np
        c = synth.CONFIGS[name]
        self.torch, self.cgtp, self.c = torch, cgtp, c
        self.es = 8 if dtype == "f64" else 4
        td = torch.float64 if dtype == "f64" else torch.float32
        dev = torch.device("cuda:0")
        self.plan = p = cgtp.Plan(c["irreps_x"], c["irreps_y"], c["irreps_out"], dtype=dtype, wkind="per_row",
                                  collapse=c.get("collapse", False))
        pos = synth.positions_for(c, 0)
        src, dst, vec = synth.radius_graph(pos, c["box"], c["r_cut"])
        self.N, self.E = N, E = pos.shape[0], src.shape[0]
        row_ptr, src_s, perm = cgtp.csr_from_coo(N, torch.from_numpy(src.astype(np.int32)).to(dev),
                                                 torch.from_numpy(dst.astype(np.int32)).to(dev))
        self.row_ptr, self.src_s = row_ptr, src_s
        self.graph = cgtp.Graph(N, row_ptr, src_s)
        self.vec = torch.from_numpy(vec).to(dev)[perm.long()].to(td).contiguous()
        self.Y = cgtp.sh_forward(c["L"], self.vec)
        W1, W2 = synth.mlp_params(8, 64, p.w_numel, 0)
        W1, W2 = torch.from_numpy(W1).to(td).to(dev), torch.from_numpy(W2).to(td).to(dev)
        r = self.vec.norm(dim=1)
        self.w = torch.empty((E, p.w_numel), device=dev, dtype=td)
        for a in range(0, E, 1 << 20):
            self.w[a:a + (1 << 20)] = synth.radial_weights_torch(r[a:a + (1 << 20)], c["r_cut"], W1, W2)
        gen = torch.Generator(device=dev)
        gen.manual_seed(0)
        self.x = torch.randn((N, p.dim_x), generator=gen, device=dev, dtype=td)
        self.scale = 1.0 / math.sqrt(E / N)
        self.out = torch.empty((N, p.dim_out), device=dev, dtype=td)
        if dtype == "f64":
            return
        self.gout = torch.randn((N, p.dim_out), generator=gen, device=dev)
        self.dx, self.dY, self.dw = torch.empty_like(self.x), torch.empty_like(self.Y), torch.empty_like(self.w)
        self.ws = torch.empty(p.workspace_size(cgtp.OP_CONV_BACKWARD, graph=self.graph), dtype=torch.uint8,
                              device=dev)
        self.gvec = torch.empty_like(self.vec)

    def sh_fwd(self):
        self.cgtp.sh_forward(self.c["L"], self.vec, out=self.Y)

    def fwd(self):
        self.plan.conv_forward(self.graph, self.x, self.Y, self.w, self.scale, out=self.out)

    def bwd(self):
        self.plan.conv_backward(self.graph, self.x, self.Y, self.w, self.scale, self.gout,
                                out=(self.dx, self.dY, self.dw), ws=self.ws)

    def sh_bwd(self):
        self.cgtp.sh_backward(self.c["L"], self.vec, self.dY, out=self.gvec)

    def bytes_fwd(self):  # w, sh read per edge; x read and out written per node; src, row_ptr
        p = self.plan
        return (self.es * (p.w_numel + p.dim_y) + 4) * self.E + (self.es * (p.dim_out + p.dim_x) + 4) * self.N

    def bytes_bwd(self):  # + grad w, grad sh written per edge; grad_out read, grad x written per node
        p = self.plan
        return 4 * (2 * p.w_numel + 2 * p.dim_y + 1) * self.E + 4 * (p.dim_out + 2 * p.dim_x + 1) * self.N


class LinearWorkload:
    """Equivariant linear map on the tensor-product rows: 2^20 rows of
    128x(0e+1o+2e+3o) -> the same irreps (4 paths of 128 x 128 weights)."""

    def __init__(self, torch, cgtp, synth, dtype):
        irreps = synth.CONFIGS["tp_large"]["irreps_x"]
        self.B = B = synth.CONFIGS["tp_large"]["B"]
        self.lin = lin = cgtp.Linear(irreps, irreps, dtype=dtype)
        td = torch.float32 if dtype == "f32" else torch.bfloat16
        gen = torch.Generator(device="cuda")
        gen.manual_seed(0)
        self.x = torch.randn((B, lin.dim_in), generator=gen, device="cuda").to(td)
        self.w = (torch.randn(lin.w_numel, generator=gen, device="cuda") / math.sqrt(128.0)).to(td)
        self.g = torch.randn((B, lin.dim_out), generator=gen, device="cuda").to(td)
        self.out = torch.empty((B, lin.dim_out), device="cuda", dtype=td)
        self.dx, self.dw = torch.empty_like(self.x), torch.empty_like(self.w)
        self.ws = torch.empty(lin.workspace_size(B), dtype=torch.uint8, device="cuda")
        self.es = 4 if dtype == "f32" else 2
        # 2 u v flops per (row, component) and path
        self.flops = 2 * B * sum((2 * int(l) + 1) * int(mu) * int(mv) for _, _, l, mu, mv in lin.paths())

    def fwd(self):
        self.lin.forward(self.x, self.w, out=self.out)

    def bwd_x(self):
        self.lin.backward(self.x, self.w, self.g, need=(True, False), out=(self.dx, None))

    def bwd_w(self):
        self.lin.backward(self.x, self.w, self.g, need=(False, True), out=(None, self.dw), ws=self.ws)


class RadialWorkload(ConvWorkload):
    """A convolution workload with the radial network's last layer joined: h
    [E][64] are the network's hidden activations, W2 [64][W] its last layer."""

    def __init__(self, torch, cgtp, synth, name):
        super().__init__(torch, cgtp, synth, name)
        c, p, dev = self.c, self.plan, self.x.device
        W1, W2 = synth.mlp_params(8, 64, p.w_numel, 0)
        W1 = torch.from_numpy(W1).float().to(dev)
        self.W2 = torch.from_numpy(W2).float().to(dev)
        eye = torch.eye(64, device=dev)
        r = self.vec.norm(dim=1)
        del self.w, self.dw, self.ws
        torch.cuda.empty_cache()
        self.h = torch.empty((self.E, 64), device=dev)
        for a in range(0, self.E, 1 << 20):
            self.h[a:a + (1 << 20)] = synth.radial_weights_torch(r[a:a + (1 << 20)], c["r_cut"], W1, eye)
        self.dh, self.dW2 = torch.empty_like(self.h), torch.empty_like(self.W2)
        self.ws = torch.empty(p.radial_workspace_size(self.graph, 64), dtype=torch.uint8, device=dev)

    def fwd(self):
        self.plan.conv_forward_radial(self.graph, self.x, self.Y, self.h, self.W2, self.scale, out=self.out)

    def bwd(self):
        self.plan.conv_backward_radial(self.graph, self.x, self.Y, self.h, self.W2, self.scale, self.gout,
                                       out=(self.dx, self.dY, self.dh, self.dW2), ws=self.ws)


class UvwWorkload:
    """The fully connected (uvw) product on the tp_large rows with collapsed
    outputs: 2^20 rows of 128x(0e+1o+2e+3o), harmonics L = 3, every output
    type (l <= 3, both parities) at 128 channels, shared 128 x 128 weights."""

    def __init__(self, torch, cgtp, synth, dtype):
        c = synth.CONFIGS["tp_large"]
        io = "+".join("128x%d%s" % (l, p) for l in range(4) for p in "eo")
        self.B = B = c["B"]
        td = torch.float32 if dtype == "f32" else torch.bfloat16
        gen = torch.Generator(device="cuda")
        gen.manual_seed(0)
        self.plan = p = cgtp.Plan(c["irreps_x"], c["irreps_y"], io, mode="uvw", dtype=dtype, wkind="shared",
                                  collapse=True)
        self.x = torch.randn((B, p.dim_x), generator=gen, device="cuda").to(td)
        v = torch.randn((B, 3), generator=gen, device="cuda")
        self.y = cgtp.sh_forward(3, v / v.norm(dim=1, keepdim=True)).to(td)
        self.w = (torch.randn((p.w_numel,), generator=gen, device="cuda") / 16.0).to(td)
        self.g = torch.randn((B, p.dim_out), generator=gen, device="cuda").to(td)
        self.out = torch.empty((B, p.dim_out), device="cuda", dtype=td)
        self.dx, self.dy, self.dw = torch.empty_like(self.x), torch.empty_like(self.y), torch.empty_like(self.w)
        self.ws = torch.empty(p.workspace_size(cgtp.OP_TP_BACKWARD, B), dtype=torch.uint8, device="cuda")

    def fwd(self):
        self.plan.tp_forward(self.x, self.y, self.w, out=self.out)

    def bwd(self):
        self.plan.tp_backward(self.x, self.y, self.w, self.g, out=(self.dx, self.dy, self.dw), ws=self.ws)


def make_workload(torch, cgtp, synth, name):
    if name.startswith("uvw"):
        return UvwWorkload(torch, cgtp, synth, "bf16" if name.endswith("bf16") else "f32")
    if name.endswith("_radial"):
        return RadialWorkload(torch, cgtp, synth, name[:-len("_radial")])
    if name.startswith("linear"):
        return LinearWorkload(torch, cgtp, synth, "bf16" if name.endswith("bf16") else "f32")
    if name == "tp_large":
        return TPWorkload(torch, cgtp, synth, "f32")
    if name == "tp_large_bf16":
        return TPWorkload(torch, cgtp, synth, "bf16")
    if name == "tp_large_collapsed":
        return TPWorkload(torch, cgtp, synth, "f32", collapse=True)
    if name.endswith("_f64"):
        return ConvWorkload(torch, cgtp, synth, name[:-4], "f64")
    return ConvWorkload(torch, cgtp, synth, name)


def profile(torch, cgtp, synth, name):
    """Three calls of every operation of one workload (the first one warms up)."""
    wl = make_workload(torch, cgtp, synth, name)
    if name.startswith("linear"):
        ops = [wl.fwd, wl.bwd_x, wl.bwd_w]
    elif name.endswith("_f64"):
        ops = [wl.fwd]
    elif name.startswith("uvw") or name.endswith("_radial"):
        ops = [wl.fwd, wl.bwd]
    else:
        ops = [wl.sh, wl.fwd, wl.bwd] if name.startswith("tp") else [wl.sh_fwd, wl.fwd, wl.bwd, wl.sh_bwd]
    for _ in range(3):
        for op in ops:
            op()
    torch.cuda.synchronize()
    rowwise = name.startswith("tp") or name.startswith("linear") or name.startswith("uvw")
    units = wl.B if rowwise else wl.E
    print(json.dumps({"profiled": name, "calls": 3, "units": units,
                      "unit": "row" if rowwise else "edge"}), flush=True)


# ------------------------------------------------------------------ benches

def tp_large_bench(args, torch, cgtp, synth, extra):
    wl = TPWorkload(torch, cgtp, synth, "f32")
    B = wl.B
    t_sh, t_fwd, t_bwd = KernelTimer(torch), KernelTimer(torch), KernelTimer(torch)

    def step(timed):
        if timed:
            t_sh(wl.sh)
            t_fwd(wl.fwd)
            t_bwd(wl.bwd)
        else:
            wl.sh()
            wl.fwd()
            wl.bwd()

    for _ in range(args.warmup):
        step(False)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        step(True)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms_step = 1000.0 * wall / args.steps

    kern = {}
    for name, t, bpr in (("tp_fwd_kernel", t_fwd, wl.bytes_fwd()),   # 105,536 B/row
                         ("tp_bwd_kernel", t_bwd, wl.bytes_bwd()),   # 131,200 B/row
                         ("sh_fwd_kernel", t_sh, 4 * (3 + wl.plan.dim_y))):
        ms = t.mean_ms()
        gbs = bpr * B / (ms * 1e-3) / 1e9
        kern[name] = dict(ms=round(ms, 4), bytes_per_row=bpr, algorithmic_GBs=round(gbs, 1),
                          frac_of_hbm_peak=round(gbs / HBM_PEAK_GBS, 4), rows_per_s=B / (ms * 1e-3),
                          traffic=traffic_for(name, "tp_large", B))
    dom = max(("tp_fwd_kernel", "tp_bwd_kernel"), key=lambda k: kern[k]["ms"])
    d = kern[dom]
    nblk = len([t for t in wl.irreps_x.split("+") if t])
    how = ("1 launch of tp_bwd_kernel over all %d x blocks" % nblk if dom == "tp_bwd_kernel"
           else "%d launches of tp_fwd_kernel (one per x block, degree-specialised), timed as one" % nblk)
    roofline = {"bound": "hbm", "kernel": dom, "achieved": d["algorithmic_GBs"], "peak": HBM_PEAK_GBS,
                "unit": "GB/s", "frac": d["frac_of_hbm_peak"], "traffic": d["traffic"],
                "algorithmic_bytes_per_launch": d["bytes_per_row"] * B, "mean_launch_ms": d["ms"],
                "launch": "one call = " + how}
    extra["tp_large_kernels"] = kern
    extra["tp_large_fwd_pairs_per_s"] = kern["tp_fwd_kernel"]["rows_per_s"]
    extra["tp_large_fwd_bwd_pairs_per_s"] = B / ((kern["tp_fwd_kernel"]["ms"] + kern["tp_bwd_kernel"]["ms"]) * 1e-3)
    plan = wl.plan
    del wl
    torch.cuda.empty_cache()
    return B * args.steps / wall, ms_step, roofline, plan


def tp_large_bf16(args, torch, cgtp, synth):
    """tp_large in bf16 storage (fp32 arithmetic): forward and backward call times."""
    wl = TPWorkload(torch, cgtp, synth, "bf16")
    B = wl.B
    tf, tb = KernelTimer(torch), KernelTimer(torch)
    wl.fwd()
    wl.bwd()
    for _ in range(3):
        tf(wl.fwd)
        tb(wl.bwd)
    torch.cuda.synchronize()
    by_f, by_b = wl.bytes_fwd(), wl.bytes_bwd()
    f, b = tf.mean_ms(), tb.mean_ms()
    del wl
    torch.cuda.empty_cache()
    return dict(fwd_ms=round(f, 3), fwd_pairs_per_s=B / (f * 1e-3), fwd_algorithmic_GBs=round(by_f * B / f / 1e6, 1),
                bwd_ms=round(b, 3), fwd_bwd_pairs_per_s=B / ((f + b) * 1e-3),
                bwd_algorithmic_GBs=round(by_b * B / b / 1e6, 1), bytes_per_row_fwd=by_f, bytes_per_row_bwd=by_b,
                fwd_traffic_bytes=traffic_for("tp_fwd_kernel", "tp_large_bf16", B),
                bwd_traffic_bytes=traffic_for("tp_bwd_kernel", "tp_large_bf16", B))


def conv_bench(args, torch, cgtp, synth, name, steps, forces=False):
    """Fused convolution forward + backward on one synthetic workload (extra figures).

    With ``forces`` the edge harmonics are recomputed from the edge vectors in the
    forward and the harmonics backward (grad_sh -> grad wrt edge vectors) follows
    the convolution backward; both are timed and reported on their own. The
    radial network's part of the force chain belongs to the caller and is not
    timed."""
    wl = ConvWorkload(torch, cgtp, synth, name)
    E, N = wl.E, wl.N
    tf, tb, tsf, tsb = KernelTimer(torch), KernelTimer(torch), KernelTimer(torch), KernelTimer(torch)
    wl.fwd()
    wl.bwd()
    for _ in range(steps):
        if forces:
            tsf(wl.sh_fwd)
        tf(wl.fwd)
        tb(wl.bwd)
        if forces:
            tsb(wl.sh_bwd)
    torch.cuda.synchronize()
    bf, bb = wl.bytes_fwd(), wl.bytes_bwd()
    msf, msb = tf.mean_ms(), tb.mean_ms()
    # backward call: the x blocks' fused launches, the grad_sh sum over their
    # copies and the grad-x gather
    bparts = [traffic_for(k, name, E) for k in ("conv_bwd_fused_kernel", "dsh_sum_kernel", "dx_gather_kernel")]
    res = dict(N=N, E=E, paths=wl.plan.num_paths,
               fwd_traffic_bytes=traffic_for("conv_fwd_fused_kernel", name, E),
               bwd_traffic_bytes=sum(bparts) if None not in bparts else None,
               fwd_ms=round(msf, 3), fwd_edges_per_s=E / (msf * 1e-3),
               fwd_algorithmic_GBs=round(bf / (msf * 1e-3) / 1e9, 1),
               fwd_frac_of_hbm_peak=round(bf / (msf * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
               bwd_ms=round(msb, 3), fwd_bwd_edges_per_s=E / ((msf + msb) * 1e-3),
               bwd_algorithmic_GBs=round(bb / (msb * 1e-3) / 1e9, 1),
               fwd_bytes_per_edge=bf / E, bwd_bytes_per_edge=bb / E)
    if forces:
        res.update(sh_fwd_ms=round(tsf.mean_ms(), 4), sh_bwd_ms=round(tsb.mean_ms(), 4),
                   fwd_bwd_forces_edges_per_s=E / ((msf + msb + tsf.mean_ms() + tsb.mean_ms()) * 1e-3))
    del wl
    torch.cuda.empty_cache()
    return res


def conv_f64_forward_bench(args, torch, cgtp, synth, name="conv_uniform100k"):
    """The convolution forward with fp64 storage and arithmetic on one full-size
    workload (the 100k-point stress case asks for it), three timed calls."""
    wl = ConvWorkload(torch, cgtp, synth, name, "f64")
    E = wl.E
    tf = KernelTimer(torch)
    wl.fwd()
    for _ in range(3):
        tf(wl.fwd)
    torch.cuda.synchronize()
    bf, ms = wl.bytes_fwd(), tf.mean_ms()
    res = dict(N=wl.N, E=E, paths=wl.plan.num_paths, fwd_ms=round(ms, 3), fwd_edges_per_s=E / (ms * 1e-3),
               fwd_algorithmic_GBs=round(bf / (ms * 1e-3) / 1e9, 1),
               fwd_frac_of_hbm_peak=round(bf / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
               fwd_bytes_per_edge=bf / E,
               fwd_traffic_bytes=traffic_for("conv_fwd_fused_kernel", name + "_f64", E))
    del wl
    torch.cuda.empty_cache()
    return res


def padding_bench(args, torch, cgtp, synth, name="conv_water1k"):
    """Padding edges ([E3J] 3.1.2, 3.2): the workload's graph plus one padding
    node and padding edges into it making up 25 % of all edges (what a
    fixed-shape caller produces), convolution forward + backward with the
    padding edges skipped (graph created with the padding node) and without."""
    import numpy as np
    c = synth.CONFIGS[name]
    p = cgtp.Plan(c["irreps_x"], c["irreps_y"], c["irreps_out"])
    pos = synth.positions_for(c, 0)
    src, dst, vec = synth.radius_graph(pos, c["box"], c["r_cut"])
    N0, E0 = pos.shape[0], src.shape[0]
    npad = E0 // 3
    pad = N0
    rng = np.random.default_rng(0)
    src = np.concatenate([src, np.full(npad, pad)]).astype(np.int32)
    dst = np.concatenate([dst, np.full(npad, pad)]).astype(np.int32)
    vec = np.concatenate([vec, rng.standard_normal((npad, 3)) + 1.0])
    N, E = N0 + 1, src.shape[0]
    d_src, d_dst = torch.from_numpy(src).cuda(), torch.from_numpy(dst).cuda()
    cgtp.csr_from_coo(N, d_src, d_dst)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    row_ptr, s, perm = cgtp.csr_from_coo(N, d_src, d_dst)
    torch.cuda.synchronize()
    t_csr = time.perf_counter() - t0
    v = torch.from_numpy(vec).cuda()[perm.long()].float().contiguous()
    Y = cgtp.sh_forward(c["L"], v)
    gen = torch.Generator(device="cuda")
    gen.manual_seed(1)
    w = torch.randn((E, p.w_numel), generator=gen, device="cuda")
    x = torch.randn((N, p.dim_x), generator=gen, device="cuda")
    g = torch.randn((N, p.dim_out), generator=gen, device="cuda")
    sc = 1.0 / math.sqrt(E0 / N0)
    res = dict(workload=name, E=E, padding_edges=npad, padding_fraction=round(npad / E, 3),
               csr_from_coo_s=round(t_csr, 4))
    for key, pn in (("skipped", pad), ("not_skipped", None)):
        t0 = time.perf_counter()
        graph = cgtp.Graph(N, row_ptr, s, pad_node=pn)
        torch.cuda.synchronize()
        t_graph = time.perf_counter() - t0
        ws = torch.empty(p.workspace_size(cgtp.OP_CONV_BACKWARD, graph=graph), dtype=torch.uint8, device="cuda")
        out = torch.empty((N, p.dim_out), device="cuda")
        dx, dY, dw = torch.empty_like(x), torch.empty_like(Y), torch.empty_like(w)
        fwd = lambda: p.conv_forward(graph, x, Y, w, sc, out=out)
        bwd = lambda: p.conv_backward(graph, x, Y, w, sc, g, out=(dx, dY, dw), ws=ws)
        tf, tb = KernelTimer(torch), KernelTimer(torch)
        fwd()
        bwd()
        for _ in range(3):
            tf(fwd)
            tb(bwd)
        torch.cuda.synchronize()
        res[key] = dict(fwd_ms=round(tf.mean_ms(), 3), bwd_ms=round(tb.mean_ms(), 3),
                        graph_create_s=round(t_graph, 3))
        del graph, ws, out, dx, dY, dw
    torch.cuda.empty_cache()
    return res


def double_backward_bench(args, torch, cgtp, synth, name="conv_water8k"):
    """Convolution double backward in the force-training shape (cotangents on
    grad_sh and grad_w, all four outputs) on one full-size workload, next to its
    forward and backward."""
    wl = ConvWorkload(torch, cgtp, synth, name)
    p, E = wl.plan, wl.E
    gen = torch.Generator(device="cuda")
    gen.manual_seed(5)
    gY = torch.randn(wl.Y.shape, generator=gen, device="cuda")
    gw = torch.randn(wl.w.shape, generator=gen, device="cuda")
    outs = (torch.empty_like(wl.x), torch.empty_like(wl.Y), torch.empty_like(wl.w), torch.empty_like(wl.gout))
    ws = torch.empty(p.workspace_size(cgtp.OP_CONV_DOUBLE_BACKWARD, graph=wl.graph), dtype=torch.uint8,
                     device="cuda")

    def dd():
        p.conv_double_backward(wl.graph, wl.x, wl.Y, wl.w, wl.scale, wl.gout, gg=(None, gY, gw), out=outs, ws=ws)

    tf, tb, td = KernelTimer(torch), KernelTimer(torch), KernelTimer(torch)
    wl.fwd()
    wl.bwd()
    dd()
    for _ in range(3):
        tf(wl.fwd)
        tb(wl.bwd)
        td(dd)
    torch.cuda.synchronize()
    res = dict(workload=name, E=E, cotangents="grad_sh, grad_w", fwd_ms=round(tf.mean_ms(), 3),
               bwd_ms=round(tb.mean_ms(), 3), double_bwd_ms=round(td.mean_ms(), 3),
               calls="2 forwards + 2 backwards + 3 adds", workspace_GB=round(ws.numel() / 1e9, 2))
    del wl, outs, ws, gY, gw
    torch.cuda.empty_cache()
    return res


def tp_variants_bench(args, torch, cgtp, synth):
    """tp_large fp32 with outputs collapsed by (l3, p3), all / symmetric / skew
    paths: forward and backward call times and algorithmic GB/s."""
    res = {}
    for sel in ("all", "symmetric", "skew"):
        wl = TPWorkload(torch, cgtp, synth, "f32", select=sel, collapse=True)
        B = wl.B
        tf, tb = KernelTimer(torch), KernelTimer(torch)
        wl.fwd()
        wl.bwd()
        for _ in range(3):
            tf(wl.fwd)
            tb(wl.bwd)
        torch.cuda.synchronize()
        f, b = tf.mean_ms(), tb.mean_ms()
        res[sel] = dict(paths=wl.plan.num_paths, dim_out=wl.plan.dim_out, fwd_ms=round(f, 3),
                        fwd_algorithmic_GBs=round(wl.bytes_fwd() * B / (f * 1e-3) / 1e9, 1),
                        bwd_ms=round(b, 3), bwd_algorithmic_GBs=round(wl.bytes_bwd() * B / (b * 1e-3) / 1e9, 1),
                        fwd_bwd_pairs_per_s=B / ((f + b) * 1e-3))
        if sel == "all":
            # the collapsed forward is one dispatch per output parity (the counter
            # summary holds one dispatch); the backward one per x block
            npar = len({int(r[1]) for r in wl.plan.outputs()})
            t = traffic_for("tp_fwd_collapsed_kernel", "tp_large_collapsed", B)
            res[sel]["fwd_traffic"] = t * npar if t is not None else None
            res[sel]["bwd_traffic"] = traffic_for("tp_bwd_kernel", "tp_large_collapsed", B)
        del wl
        torch.cuda.empty_cache()
    return res


def linear_bench(args, torch, cgtp, synth, dtype):
    """Equivariant linear map on the tensor-product rows (fp32 matrix cores for fp32
    storage, bf16 matrix cores for bf16 storage): call times, TFLOP/s against the
    matching matrix-core peak, and algorithmic GB/s."""
    wl = LinearWorkload(torch, cgtp, synth, dtype)
    B = wl.B
    tf, tx, tw = KernelTimer(torch), KernelTimer(torch), KernelTimer(torch)
    wl.fwd()
    wl.bwd_x()
    wl.bwd_w()
    for _ in range(3):
        tf(wl.fwd)
        tx(wl.bwd_x)
        tw(wl.bwd_w)
    torch.cuda.synchronize()
    res = {"rows": B, "irreps": "128x0e+128x1o+128x2e+128x3o -> same", "flops_per_call": wl.flops}
    dim = wl.lin.dim_in
    wname = "linear_large" if dtype == "f32" else "linear_large_bf16"
    for key, t, nbytes, kern in (("fwd", tf, wl.es * B * 2 * dim, "lin_rows_kernel"),
                                 ("bwd_x", tx, wl.es * B * 2 * dim, "lin_rows_kernel"),
                                 ("bwd_w", tw, wl.es * B * 2 * dim, "lin_dw_kernel")):
        ms = t.mean_ms()
        tfs = wl.flops / (ms * 1e-3) / 1e12
        gbs = nbytes / (ms * 1e-3) / 1e9
        # fp32 storage: fp32 matrix cores; bf16 storage (this shape): bf16 matrix cores
        peak = MFMA_FP32_PEAK_TFS if dtype == "f32" else MFMA_BF16_PEAK_TFS
        res[key] = dict(kernel=kern if dtype == "f32" else kern.replace("_kernel", "_bf16_kernel"), ms=round(ms, 3),
                        TFLOPs=round(tfs, 1), mfma_peak_TFLOPs=peak, frac_of_mfma_peak=round(tfs / peak, 3),
                        algorithmic_GBs=round(gbs, 1), frac_of_hbm_peak=round(gbs / HBM_PEAK_GBS, 3),
                        traffic=traffic_for(kern if dtype == "f32" else kern.replace("_kernel", "_bf16_kernel"),
                                            wname, B))
    del wl
    torch.cuda.empty_cache()
    return res


def radial_bench(args, torch, cgtp, synth, name):
    """The convolution with the radial network's last layer joined to it, on one
    full-size workload: h = the hidden activations (64 wide) of the radial
    network, W2 its last layer. Fused forward (w = h W2 formed on the matrix
    cores inside the kernel) against the same result as two library calls (the
    linear map writing w to memory, then the convolution reading it), and the
    backward (composed: grad_x, grad_sh, grad_h, grad_W2)."""
    import numpy as np
    c = synth.CONFIGS[name]
    dev = torch.device("cuda:0")
    p = cgtp.Plan(c["irreps_x"], c["irreps_y"], c["irreps_out"], wkind="per_row")
    pos = synth.positions_for(c, 0)
    src, dst, vec = synth.radius_graph(pos, c["box"], c["r_cut"])
    N, E = pos.shape[0], src.shape[0]
    row_ptr, src_s, perm = cgtp.csr_from_coo(N, torch.from_numpy(src.astype(np.int32)).to(dev),
                                             torch.from_numpy(dst.astype(np.int32)).to(dev))
    graph = cgtp.Graph(N, row_ptr, src_s)
    v = torch.from_numpy(vec).to(dev)[perm.long()].float().contiguous()
    Y = cgtp.sh_forward(c["L"], v)
    H = 64
    W1, W2 = synth.mlp_params(8, H, p.w_numel, 0)
    W1, W2 = torch.from_numpy(W1).float().to(dev), torch.from_numpy(W2).float().to(dev)
    eye = torch.eye(H, device=dev)
    r = v.norm(dim=1)
    h = torch.empty((E, H), device=dev)
    for a in range(0, E, 1 << 20):
        h[a:a + (1 << 20)] = synth.radial_weights_torch(r[a:a + (1 << 20)], c["r_cut"], W1, eye)
    gen = torch.Generator(device=dev)
    gen.manual_seed(0)
    x = torch.randn((N, p.dim_x), generator=gen, device=dev)
    g = torch.randn((N, p.dim_out), generator=gen, device=dev)
    sc = 1.0 / math.sqrt(E / N)
    out = torch.empty((N, p.dim_out), device=dev)
    fused = lambda: p.conv_forward_radial(graph, x, Y, h, W2, sc, out=out)
    tf = KernelTimer(torch)
    fused()
    for _ in range(3):
        tf(fused)
    torch.cuda.synchronize()
    lin = cgtp.Linear("%dx0e" % H, "%dx0e" % p.w_numel)
    w = torch.empty((E, p.w_numel), device=dev)
    out2 = torch.empty_like(out)
    tl, tc = KernelTimer(torch), KernelTimer(torch)
    W2f = W2.reshape(-1)  # the linear map's flat weights, W_p = W2 [H][W]
    lin.forward(h, W2f, out=w)
    p.conv_forward(graph, x, Y, w, sc, out=out2)
    for _ in range(3):
        tl(lambda: lin.forward(h, W2f, out=w))
        tc(lambda: p.conv_forward(graph, x, Y, w, sc, out=out2))
    torch.cuda.synchronize()
    rel = float((out - out2).abs().max() / out2.abs().max())
    del w, out2
    torch.cuda.empty_cache()
    ws = torch.empty(p.radial_workspace_size(graph, H), dtype=torch.uint8, device=dev)
    grads = (torch.empty_like(x), torch.empty_like(Y), torch.empty_like(h), torch.empty_like(W2))
    bwd = lambda: p.conv_backward_radial(graph, x, Y, h, W2, sc, g, out=grads, ws=ws)
    tb = KernelTimer(torch)
    bwd()
    for _ in range(2):
        tb(bwd)
    torch.cuda.synchronize()
    flops = 2 * E * H * p.w_numel
    res = dict(workload=name, E=E, hidden=H, W=p.w_numel, last_layer_flops=flops,
               fused_fwd_ms=round(tf.mean_ms(), 3), fused_fwd_edges_per_s=E / (tf.mean_ms() * 1e-3),
               unfused_linear_ms=round(tl.mean_ms(), 3), unfused_conv_fwd_ms=round(tc.mean_ms(), 3),
               unfused_fwd_ms=round(tl.mean_ms() + tc.mean_ms(), 3), fused_vs_unfused_max_rel_diff=rel,
               bwd_ms=round(tb.mean_ms(), 3),
               bwd="w = h W2 (linear map) + convolution backward + linear map backward (grad_h, grad_W2)",
               bytes_not_moved_GB=round(2 * 4 * E * p.w_numel / 1e9, 1))
    del ws, grads, h, x, g, out, Y, graph
    torch.cuda.empty_cache()
    return res


def uvw_bench(args, torch, cgtp, synth, dtype):
    """Fully connected (uvw) product on the tp_large rows: 2^20 rows of
    128x(0e+1o+2e+3o), harmonics L = 3, every output type (l <= 3, both
    parities) at 128 channels, shared 128 x 128 weights per path. Collapsed
    outputs (the fully connected product, 4,096 outputs per row): the fused
    forward against the same product as two library calls (unit-weight uvu
    forward writing the 19,968 path outputs per row, then the linear map from
    them to the outputs), and the backward. Uncollapsed outputs (one 128-channel
    block per path, 19,968 per row): forward. MFMA work: 2 sum_p (2 l3 + 1) u w
    flops per row."""
    c = synth.CONFIGS["tp_large"]
    ix, iy = c["irreps_x"], c["irreps_y"]
    io = "+".join("128x%d%s" % (l, p) for l in range(4) for p in "eo")
    B = c["B"]
    td = torch.float32 if dtype == "f32" else torch.bfloat16
    es = 4 if dtype == "f32" else 2
    gen = torch.Generator(device="cuda")
    gen.manual_seed(0)
    peak = MFMA_FP32_PEAK_TFS if dtype == "f32" else MFMA_BF16_PEAK_TFS
    res = {"rows": B, "irreps_x": ix, "irreps_out": io, "dtype": dtype,
           "mfma": ("v_mfma_f32_16x16x4_f32" if dtype == "f32" else
                    "v_mfma_f32_16x16x32_bf16 (bf16 operands, fp32 sums; path outputs rounded to bf16 in LDS)"),
           "mfma_peak_TFLOPs": peak}
    x = torch.randn((B, 2048), generator=gen, device="cuda").to(td)
    v = torch.randn((B, 3), generator=gen, device="cuda")
    y = cgtp.sh_forward(3, v / v.norm(dim=1, keepdim=True)).to(td)
    del v
    for collapse in (True, False):
        p = cgtp.Plan(ix, iy, io, mode="uvw", dtype=dtype, wkind="shared", collapse=collapse)
        flops = 2 * B * sum((2 * int(r[4]) + 1) * 128 * 128 for r in p.paths())
        w = (torch.randn((p.w_numel,), generator=gen, device="cuda") / 16.0).to(td)
        out = torch.empty((B, p.dim_out), device="cuda", dtype=td)
        fwd = lambda: p.tp_forward(x, y, w, out=out)
        tf = KernelTimer(torch)
        fwd()
        for _ in range(3):
            tf(fwd)
        torch.cuda.synchronize()
        ms = tf.mean_ms()
        nbytes = es * B * (p.dim_x + p.dim_y + p.dim_out) + es * p.w_numel
        key = "collapsed" if collapse else "uncollapsed"
        res[key] = dict(paths=p.num_paths, dim_out=p.dim_out, fwd_ms=round(ms, 3), fwd_pairs_per_s=B / (ms * 1e-3),
                        fwd_TFLOPs=round(flops / (ms * 1e-3) / 1e12, 1),
                        fwd_frac_of_mfma_peak=round(flops / (ms * 1e-3) / 1e12 / peak, 3),
                        fwd_algorithmic_GBs=round(nbytes / (ms * 1e-3) / 1e9, 1), flops=flops)
        if collapse:
            # the same product as two calls: unit-weight uvu forward, then the linear map
            unit = cgtp.Plan(ix, iy, io, dtype=dtype, wkind="shared")
            ones = torch.ones((unit.w_numel,), device="cuda", dtype=td)
            t_irreps = "+".join("128x%d%s" % (int(r[4]), "e" if int(r[5]) > 0 else "o") for r in unit.paths())
            o_irreps = "+".join("%dx%d%s" % (int(r[2]), int(r[0]), "e" if int(r[1]) > 0 else "o") for r in p.outputs())
            lin = cgtp.Linear(t_irreps, o_irreps, dtype=dtype)
            T = torch.empty((B, unit.dim_out), device="cuda", dtype=td)
            out2 = torch.empty_like(out)
            comp = lambda: (unit.tp_forward(x, y, ones, out=T), lin.forward(T, w, out=out2))
            tc = KernelTimer(torch)
            comp()
            for _ in range(3):
                tc(comp)
            torch.cuda.synchronize()
            res[key]["composition_fwd_ms"] = round(tc.mean_ms(), 3)
            res[key]["composition_matches"] = bool(torch.allclose(out.float(), out2.float(), rtol=1e-2, atol=1e-2))
            del T, out2, ones
            torch.cuda.empty_cache()
            g = torch.randn((B, p.dim_out), generator=gen, device="cuda").to(td)
            dx, dy, dw = torch.empty_like(x), torch.empty_like(y), torch.empty_like(w)
            ws = torch.empty(p.workspace_size(cgtp.OP_TP_BACKWARD, B), dtype=torch.uint8, device="cuda")
            bwd = lambda: p.tp_backward(x, y, w, g, out=(dx, dy, dw), ws=ws)
            tb = KernelTimer(torch)
            bwd()
            for _ in range(2):
                tb(bwd)
            torch.cuda.synchronize()
            res[key]["bwd_ms"] = round(tb.mean_ms(), 3)
            res[key]["bwd"] = "unit-weight uvu forward + linear backward + unit-weight uvu backward (workspace)"
            del g, dx, dy, dw, ws
        del out, w, p
        torch.cuda.empty_cache()
    del x, y
    torch.cuda.empty_cache()
    return res


def uvu_ymul_bench(args, torch, cgtp, synth):
    """uvu with y of multiplicity 4 (generic kernels): 2^18 rows of
    32x(0e+1o+2e) with y = 4x(0e+1o+2e), per-row weights [u][v] per path."""
    ix, iy, io = "32x0e+32x1o+32x2e", "4x0e+4x1o+4x2e", "0e+0o+1e+1o+2e+2o"
    p = cgtp.Plan(ix, iy, io, wkind="per_row")
    B = 1 << 18
    gen = torch.Generator(device="cuda")
    gen.manual_seed(0)
    x = torch.randn((B, p.dim_x), generator=gen, device="cuda")
    y = torch.randn((B, p.dim_y), generator=gen, device="cuda")
    w = torch.randn((B, p.w_numel), generator=gen, device="cuda")
    g = torch.randn((B, p.dim_out), generator=gen, device="cuda")
    out = torch.empty((B, p.dim_out), device="cuda")
    dx, dy, dw = torch.empty_like(x), torch.empty_like(y), torch.empty_like(w)
    ws = torch.empty(p.workspace_size(cgtp.OP_TP_BACKWARD, B), dtype=torch.uint8, device="cuda")
    tf, tb = KernelTimer(torch), KernelTimer(torch)
    fwd = lambda: p.tp_forward(x, y, w, out=out)
    bwd = lambda: p.tp_backward(x, y, w, g, out=(dx, dy, dw), ws=ws)
    fwd()
    bwd()
    for _ in range(3):
        tf(fwd)
        tb(bwd)
    torch.cuda.synchronize()
    f, b = tf.mean_ms(), tb.mean_ms()
    bytes_f = 4 * B * (p.dim_x + p.dim_y + p.w_numel + p.dim_out)
    res = dict(rows=B, irreps_x=ix, irreps_y=iy, paths=p.num_paths, w_per_row=p.w_numel, fwd_ms=round(f, 3),
               bwd_ms=round(b, 3), fwd_algorithmic_GBs=round(bytes_f / (f * 1e-3) / 1e9, 1),
               fwd_bwd_pairs_per_s=B / ((f + b) * 1e-3))
    del x, y, w, g, out, dx, dy, dw, ws
    torch.cuda.empty_cache()
    return res


def tp_small_bench(args, torch, cgtp, synth):
    """tp_small (4096 rows of 32x(0e+1o+2e), SH L = 2, 15 paths, shared weights,
    fp32): forward and backward call times. Its 31.6 MB working set fits the
    256 MB Infinity Cache, so it is timed twice: back to back (cache-resident)
    and with a 1 GiB buffer written between calls (caches flushed, every input
    from HBM)."""
    c = synth.CONFIGS["tp_small"]
    p = cgtp.Plan(c["irreps_x"], c["irreps_y"], c["irreps_out"], wkind="shared")
    B = c["B"]
    gen = torch.Generator(device="cuda")
    gen.manual_seed(0)
    x = torch.randn((B, p.dim_x), generator=gen, device="cuda")
    v = torch.randn((B, 3), generator=gen, device="cuda")
    y = cgtp.sh_forward(2, v / v.norm(dim=1, keepdim=True))
    w = torch.randn((p.w_numel,), generator=gen, device="cuda")
    g = torch.randn((B, p.dim_out), generator=gen, device="cuda")
    out = torch.empty((B, p.dim_out), device="cuda")
    dx, dy, dw = torch.empty_like(x), torch.empty_like(y), torch.empty_like(w)
    ws = torch.empty(p.workspace_size(cgtp.OP_TP_BACKWARD, B), dtype=torch.uint8, device="cuda")
    flush = torch.empty(1 << 28, device="cuda")  # 1 GiB
    fwd = lambda: p.tp_forward(x, y, w, out=out)
    bwd = lambda: p.tp_backward(x, y, w, g, out=(dx, dy, dw), ws=ws)
    res = {"rows": B, "paths": p.num_paths, "weights": "shared"}
    es = 4
    bytes_fwd = es * (B * (p.dim_x + p.dim_y + p.dim_out) + p.w_numel)
    bytes_bwd = es * (B * (2 * p.dim_x + 2 * p.dim_y + p.dim_out) + 2 * p.w_numel)
    for key, flushed in (("resident", False), ("flushed", True)):
        tf, tb = KernelTimer(torch), KernelTimer(torch)
        fwd()
        bwd()
        for _ in range(20):
            if flushed:
                flush.fill_(1.0)
            tf(fwd)
            if flushed:
                flush.fill_(2.0)
            tb(bwd)
        torch.cuda.synchronize()
        f, b = tf.mean_ms(), tb.mean_ms()
        res[key] = dict(fwd_ms=round(f, 4), bwd_ms=round(b, 4), fwd_pairs_per_s=B / (f * 1e-3),
                        fwd_bwd_pairs_per_s=B / ((f + b) * 1e-3),
                        fwd_algorithmic_GBs=round(bytes_fwd / (f * 1e-3) / 1e9, 1),
                        bwd_algorithmic_GBs=round(bytes_bwd / (b * 1e-3) / 1e9, 1))
    res["bytes_fwd"], res["bytes_bwd"] = bytes_fwd, bytes_bwd
    del flush, x, y, w, g, out, dx, dy, dw, ws
    torch.cuda.empty_cache()
    return res


def hbm_ceiling(torch):
    """Plain streaming rates of this device, HIP events around torch's own
    kernels: a 4 GiB elementwise copy (4 GiB read + 4 GiB written), a 4 GiB
    fill (write only) and row sums of a [2^20, 1024] view (4 GiB read, 4 MiB
    written); and the tensor product's two row mixes with torch's kernels on
    2^15 rows: a row repeated 3 times (26.6 KB read, 79.9 KB written per row,
    the forward's mix) and the sum of a row's 3 thirds (79.9 KB read, 26.6 KB
    written, the backward's); best of 5."""
    n = 1 << 30
    a = torch.ones(n, device="cuda")
    b = torch.empty_like(a)
    R, k = 1 << 15, 6656  # 3 k = 19968 floats per row: the tp_large output row
    xr = a[:R * k].view(R, k)
    xo = b[:3 * R * k].view(R, 3 * k)
    res = {}
    for key, fn, nbytes in (("copy", lambda: torch.mul(a, 1.0, out=b), 8 * n),
                            ("write", lambda: b.fill_(3.0), 4 * n),
                            ("read", lambda: a.view(1 << 20, 1024).sum(dim=1), 4 * n + 4 * (1 << 20)),
                            ("mix_read1_write3", lambda: xo.view(R, 3, k).copy_(xr.view(R, 1, k).expand(R, 3, k)),
                             4 * R * k * 4),
                            ("mix_read3_write1", lambda: torch.sum(xo.view(R, 3, k), dim=1, out=xr),
                             4 * R * k * 4)):
        fn()
        best = None
        for _ in range(5):
            t = KernelTimer(torch)
            t(fn)
            torch.cuda.synchronize()
            ms = t.mean_ms()
            best = ms if best is None else min(best, ms)
        res[key] = dict(ms=round(best, 3), GBs=round(nbytes / (best * 1e-3) / 1e9, 1),
                        frac_of_8TBs=round(nbytes / (best * 1e-3) / 1e9 / HBM_PEAK_GBS, 3))
    del a, b
    torch.cuda.empty_cache()
    return res


def _host_cores():
    """Worker count for the host-side oracle (the GPU machine's CPU share is 16
    cores whatever the OS reports) and the CPU model."""
    n = min(16, os.cpu_count() or 1)
    model = "unknown"
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    return n, model


def _oracle_tp_chunk(job):
    """Worker: the oracle's tensor-product forward + backward on one chunk of
    rows of the tp_large shapes, its inputs drawn from the chunk's own seed."""
    seed, rows = job
    from clebsch_gordan_tensor_amd import synth
    from oracle import sh as osh
    from oracle import tp as otp
    from oracle.irreps import Layout
    c = synth.CONFIGS["tp_large"]
    L = Layout(c["irreps_x"], c["irreps_y"], c["irreps_out"])
    x = synth.gaussian((rows, L.dim_x), seed, synth.S_X)
    y = osh.real_sh(3, synth.unit_vectors(rows, seed))
    w = synth.gaussian((rows, L.w_numel), seed, synth.S_W)
    g = synth.gaussian((rows, L.dim_out), seed, synth.S_G)
    t0 = time.perf_counter()
    otp.forward(L, x, y, w)
    otp.backward(L, x, y, w, g)
    return time.perf_counter() - t0


def _oracle_conv_chunk(job):
    """Worker: the oracle's convolution forward + backward on the CSR segments of
    receivers [n0, n1) of the water1k graph (their edges and cotangents)."""
    n0, n1 = job
    import numpy as np
    from clebsch_gordan_tensor_amd import synth
    from oracle import conv as oconv
    from oracle import graph as ograph
    from oracle import sh as osh
    from oracle.irreps import Layout
    c = synth.CONFIGS["conv_water1k"]
    L = Layout(c["irreps_x"], c["irreps_y"], c["irreps_out"])
    pos = synth.positions_for(c, 0)
    src, dst, vec = synth.radius_graph(pos, c["box"], c["r_cut"])
    N = pos.shape[0]
    row, s, perm = ograph.csr_from_coo(N, src, dst)
    e0, e1 = row[n0], row[n1]
    sub_row = row[n0:n1 + 1] - e0
    x = synth.gaussian((N, L.dim_x), 0, synth.S_X)
    v = vec[perm][e0:e1]
    Y = osh.real_sh(c["L"], v)
    W1, W2 = synth.mlp_params(8, 64, L.w_numel, 0)
    w = synth.radial_weights_np(np.linalg.norm(v, axis=1), c["r_cut"], W1, W2)
    g = synth.gaussian((N, L.dim_out), 0, synth.S_G)[n0:n1]
    scale = oconv.avg_neighbors_scale(N, len(src))
    t0 = time.perf_counter()
    oconv.forward(L, sub_row, s[e0:e1], x, Y, w, scale)
    oconv.backward(L, sub_row, s[e0:e1], x, Y, w, scale, g)
    return time.perf_counter() - t0, int(e1 - e0)


def cpu_baseline(args, synth):
    """The oracle as it stands (fp64 NumPy, not tuned), on the host cores: a
    process pool over row chunks of a bounded tp_large sample, forward +
    backward; rate = rows / wall time of the pool."""
    import concurrent.futures as cf
    cores, model = _host_cores()
    probe = 64
    dt = _oracle_tp_chunk((1, probe))
    per = int(min(16384, max(probe, probe * args.cpu_seconds / max(dt, 1e-3))))
    with cf.ProcessPoolExecutor(max_workers=cores) as ex:
        list(ex.map(_oracle_tp_chunk, [(1, 8)] * cores))  # import and warm every worker
        t0 = time.perf_counter()
        times = list(ex.map(_oracle_tp_chunk, [(1 + k, per) for k in range(cores)]))
        wall = time.perf_counter() - t0
    rows = per * cores
    return {"value": rows / wall, "unit": "pairs/s", "cores": cores, "kind": "oracle",
            "sample": "tp_large fwd+bwd (harmonics excluded) on %d rows, fp64 NumPy, %d worker processes of "
                      "%d rows each, %.1f s wall (of which the slowest worker's oracle arithmetic %.1f s, its input "
                      "draws the rest); CPU %s" % (rows, cores, per, wall, max(times), model)}


def cpu_baseline_conv(args, synth):
    """The oracle's convolution forward + backward on the water1k graph, on
    the host cores (a process pool over receiver ranges), in edges/s."""
    import concurrent.futures as cf
    cores, model = _host_cores()
    nodes = 480  # receivers in the sample (about 25,000 edges)
    per = (nodes + cores - 1) // cores
    jobs = [(n, min(n + per, nodes)) for n in range(0, nodes, per)]
    with cf.ProcessPoolExecutor(max_workers=cores) as ex:
        list(ex.map(_oracle_conv_chunk, [(0, 1)] * cores))
        t0 = time.perf_counter()
        res = list(ex.map(_oracle_conv_chunk, jobs))
        wall = time.perf_counter() - t0
    edges = sum(e for _, e in res)
    return {"value": edges / wall, "unit": "edges/s", "cores": cores, "kind": "oracle",
            "sample": "conv_water1k fwd+bwd on the %d edges into receivers 0-%d, fp64 NumPy, %d worker "
                      "processes over receiver ranges, %.1f s wall; CPU %s" % (edges, nodes - 1, cores, wall, model)}


def main():
    args = parse()
    if args.gpus != 1:
        print("bench.py measures one GPU only: the library has no multi-GPU path (--gpus %d refused)"
              % args.gpus, file=sys.stderr)
        sys.exit(2)
    import torch
    from clebsch_gordan_tensor_amd import cgtp, synth
    assert torch.cuda.is_available(), "bench.py needs a GPU"
    torch.cuda.set_device(0)
    if args.calibrate_copy:
        calibrate_copy(torch)
        return
    if args.profile:
        profile(torch, cgtp, synth, args.profile)
        return
    extra = {"device": torch.cuda.get_device_name(0)}
    value, ms_step, roofline, plan = tp_large_bench(args, torch, cgtp, synth, extra)
    if not args.no_extra:
        extra["hbm_ceiling"] = hbm_ceiling(torch)
        extra["tp_small"] = tp_small_bench(args, torch, cgtp, synth)
        extra["tp_large_bf16"] = tp_large_bf16(args, torch, cgtp, synth)
        extra["tp_large_collapsed"] = tp_variants_bench(args, torch, cgtp, synth)
        extra["linear_large"] = linear_bench(args, torch, cgtp, synth, "f32")
        extra["linear_large_bf16"] = linear_bench(args, torch, cgtp, synth, "bf16")
        extra["uvw_tp_large"] = uvw_bench(args, torch, cgtp, synth, "f32")
        extra["uvw_tp_large_bf16"] = uvw_bench(args, torch, cgtp, synth, "bf16")
        extra["uvu_ymul4"] = uvu_ymul_bench(args, torch, cgtp, synth)
    if not args.no_conv and not args.no_extra:
        for name in ("conv_water1k", "conv_water8k", "conv_uniform100k", "conv_collapsed_l3", "conv_collapsed_l4"):
            extra[name] = conv_bench(args, torch, cgtp, synth, name, max(2, min(args.steps, 5)),
                                     forces=name == "conv_water8k")
        extra["conv_uniform100k_f64"] = conv_f64_forward_bench(args, torch, cgtp, synth)
        extra["conv_water8k_double_backward"] = double_backward_bench(args, torch, cgtp, synth)
        extra["conv_water1k_padded"] = padding_bench(args, torch, cgtp, synth)
        extra["conv_water8k_radial"] = radial_bench(args, torch, cgtp, synth, "conv_water8k")
        extra["conv_uniform100k_radial"] = radial_bench(args, torch, cgtp, synth, "conv_uniform100k")
    cpu = None if args.no_cpu_baseline else cpu_baseline(args, synth)
    if not args.no_cpu_baseline and not args.no_extra:
        extra["cpu_baseline_conv"] = cpu_baseline_conv(args, synth)
    line = {
        "metric": METRIC, "value": value, "unit": "pairs/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": ms_step, "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "f32", "data": "synthetic",
        "config": {"workload": "tp_large", "rows": 1048576, "irreps_x": "128x0e+128x1o+128x2e+128x3o",
                   "irreps_y": "SH lmax=3", "paths": plan.num_paths, "weights": "per-row",
                   "step": "sh_forward + tp_forward + tp_backward"},
        "roofline": roofline, "cpu_baseline": cpu, "extra": extra,
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
