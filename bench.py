"""Benchmark of the hot path on one MI355X; prints one JSON line.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload tp_large]
                    [--no-conv] [--no-cpu-baseline]

Workload (default tp_large): 1,048,576 rows of x = 128x(0e+1o+2e+3o), y = the
real spherical harmonics (L = 3) of random unit vectors, per-row weights for
all 34 paths to lout <= 3, fp32. One step = harmonics of the row directions
(cgtp_sh_forward) -> tensor product forward -> tensor product backward (grads
of x, y and w), with every input already resident in HBM. `value` is rows
("pairs") per second of whole steps.

Besides the headline line's `roofline` (dominant kernel, algorithmic bytes per
launch over its mean HIP-event duration against 8 TB/s) and `cpu_baseline`
(the fp64 oracle on a bounded sample, on the host cores), `extra` carries the
per-kernel figures and, unless --no-conv, the fused convolution (forward and
backward, fp32) on the 1000- and 8000-molecule water boxes (the latter with the
harmonics forward/backward of the force chain) and the 100,000-point uniform
cloud.
"""

import argparse
import hashlib
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


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=10)
    ap.add_argument("--warmup", type=int, default=2)
    ap.add_argument("--workload", default="tp_large", choices=["tp_large"])
    ap.add_argument("--no-conv", action="store_true")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=12.0, help="target oracle time")
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="only run a plain 4 GiB device copy (reference for HBM byte counters) and exit")
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


def kernel_source_hash(names):
    h = hashlib.sha256()
    for n in names:
        with open(os.path.join(ROOT, "clebsch_gordan_tensor_amd", "csrc", n), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def traffic_for(kernel, src_files, per_launch_units):
    """HBM bytes per launch from the committed counter summary, or None when the
    kernel sources changed since the counters were taken."""
    path = os.path.join(PROFILES, "hbm_traffic.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        rec = json.load(f).get(kernel)
    if not rec or rec.get("source_hash") != kernel_source_hash(src_files):
        return None
    return rec["bytes_per_unit"] * per_launch_units


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


def plan_blocks(plan):
    """x blocks of a plan (one kernel launch each)."""
    return [t for t in plan.irreps_x.replace(" ", "").split("+") if t]


def tp_large_bench(args, torch, cgtp, synth, extra):
    c = synth.CONFIGS["tp_large"]
    plan = cgtp.Plan(c["irreps_x"], c["irreps_y"], c["irreps_out"], dtype="f32", wkind="per_row")
    B = c["B"]
    dev = torch.device("cuda:0")
    gen = torch.Generator(device=dev)
    gen.manual_seed(0)
    x = torch.randn((B, plan.dim_x), generator=gen, device=dev)
    w = torch.randn((B, plan.w_numel), generator=gen, device=dev)
    g = torch.randn((B, plan.dim_out), generator=gen, device=dev)
    v = torch.randn((B, 3), generator=gen, device=dev)
    v = v / v.norm(dim=1, keepdim=True)
    y = torch.empty((B, plan.dim_y), device=dev)
    out = torch.empty((B, plan.dim_out), device=dev)
    dx, dy, dw = torch.empty_like(x), torch.empty_like(y), torch.empty_like(w)
    t_sh, t_fwd, t_bwd = KernelTimer(torch), KernelTimer(torch), KernelTimer(torch)

    def step(timed):
        if timed:
            t_sh(lambda: cgtp.sh_forward(3, v, out=y))
            t_fwd(lambda: plan.tp_forward(x, y, w, out=out))
            t_bwd(lambda: plan.tp_backward(x, y, w, g, out=(dx, dy, dw)))
        else:
            cgtp.sh_forward(3, v, out=y)
            plan.tp_forward(x, y, w, out=out)
            plan.tp_backward(x, y, w, g, out=(dx, dy, dw))

    for _ in range(args.warmup):
        step(False)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        step(True)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms_step = 1000.0 * wall / args.steps

    by_fwd = 4 * (plan.dim_x + plan.dim_y + plan.w_numel + plan.dim_out)          # 105,536 B/row
    by_bwd = 4 * (2 * plan.dim_x + 2 * plan.dim_y + 2 * plan.w_numel + plan.dim_out)  # 131,200 B/row
    by_sh = 4 * (3 + plan.dim_y)
    kern = {}
    for name, t, bpr, srcs in (
            ("tp_fwd_kernel", t_fwd, by_fwd, ["tp_impl.hpp", "tp_core.hpp", "cg_pattern.h", "device_util.hpp"]),
            ("tp_bwd_kernel", t_bwd, by_bwd, ["tp_impl.hpp", "tp_core.hpp", "cg_pattern.h", "device_util.hpp"]),
            ("sh_fwd_kernel", t_sh, by_sh, ["sh_kernels.hip", "device_util.hpp"])):
        ms = t.mean_ms()
        gbs = bpr * B / (ms * 1e-3) / 1e9
        kern[name] = dict(ms=round(ms, 4), bytes_per_row=bpr, algorithmic_GBs=round(gbs, 1),
                          frac_of_hbm_peak=round(gbs / HBM_PEAK_GBS, 4), rows_per_s=B / (ms * 1e-3),
                          traffic=traffic_for(name, srcs, B))
        kern[name]["_srcs"] = srcs
    dom = max(("tp_fwd_kernel", "tp_bwd_kernel"), key=lambda k: kern[k]["ms"])
    d = kern[dom]
    roofline = {"bound": "hbm", "kernel": dom, "achieved": d["algorithmic_GBs"], "peak": HBM_PEAK_GBS,
                "unit": "GB/s", "frac": d["frac_of_hbm_peak"], "traffic": d["traffic"],
                "algorithmic_bytes_per_launch": d["bytes_per_row"] * B, "mean_launch_ms": d["ms"],
                "launch": "one call = %d launches of %s (one per x block, degree-specialised)"
                          % (len(plan_blocks(plan)), dom)}
    for k in kern.values():
        k.pop("_srcs")
    extra["tp_large_kernels"] = kern
    extra["tp_large_fwd_pairs_per_s"] = kern["tp_fwd_kernel"]["rows_per_s"]
    extra["tp_large_fwd_bwd_pairs_per_s"] = B / ((kern["tp_fwd_kernel"]["ms"] + kern["tp_bwd_kernel"]["ms"]) * 1e-3)
    del x, w, g, v, y, out, dx, dy, dw
    torch.cuda.empty_cache()
    return B * args.steps / wall, ms_step, roofline, plan


def tp_large_bf16(args, torch, cgtp, synth):
    """tp_large in bf16 storage (fp32 arithmetic): forward and backward call times."""
    c = synth.CONFIGS["tp_large"]
    plan = cgtp.Plan(c["irreps_x"], c["irreps_y"], c["irreps_out"], dtype="bf16", wkind="per_row")
    B = c["B"]
    gen = torch.Generator(device="cuda")
    gen.manual_seed(0)
    bf = torch.bfloat16
    x = torch.randn((B, plan.dim_x), generator=gen, device="cuda").to(bf)
    w = torch.randn((B, plan.w_numel), generator=gen, device="cuda").to(bf)
    g = torch.randn((B, plan.dim_out), generator=gen, device="cuda").to(bf)
    y = torch.randn((B, plan.dim_y), generator=gen, device="cuda").to(bf)
    out = torch.empty((B, plan.dim_out), device="cuda", dtype=bf)
    dx, dy, dw = torch.empty_like(x), torch.empty_like(y), torch.empty_like(w)
    tf, tb = KernelTimer(torch), KernelTimer(torch)
    for k in range(4):
        if k == 0:
            plan.tp_forward(x, y, w, out=out)
            plan.tp_backward(x, y, w, g, out=(dx, dy, dw))
        else:
            tf(lambda: plan.tp_forward(x, y, w, out=out))
            tb(lambda: plan.tp_backward(x, y, w, g, out=(dx, dy, dw)))
    torch.cuda.synchronize()
    by_f = 2 * (plan.dim_x + plan.dim_y + plan.w_numel + plan.dim_out)
    by_b = 2 * (2 * plan.dim_x + 2 * plan.dim_y + 2 * plan.w_numel + plan.dim_out)
    f, b = tf.mean_ms(), tb.mean_ms()
    del x, w, g, y, out, dx, dy, dw
    torch.cuda.empty_cache()
    return dict(fwd_ms=round(f, 3), fwd_pairs_per_s=B / (f * 1e-3), fwd_algorithmic_GBs=round(by_f * B / f / 1e6, 1),
                bwd_ms=round(b, 3), fwd_bwd_pairs_per_s=B / ((f + b) * 1e-3),
                bwd_algorithmic_GBs=round(by_b * B / b / 1e6, 1), bytes_per_row_fwd=by_f, bytes_per_row_bwd=by_b)


def conv_bench(args, torch, cgtp, synth, name, steps, forces=False):
    """Fused convolution forward + backward on one synthetic workload (extra figures).

    With ``forces`` the edge harmonics are recomputed from the edge vectors in the
    forward and the harmonics backward (grad_sh -> grad wrt edge vectors) follows
    the convolution backward; both are timed and reported on their own. The
    radial network's part of the force chain belongs to the caller and is not
    timed."""
    import numpy as np
    c = synth.CONFIGS[name]
    dev = torch.device("cuda:0")
    plan = cgtp.Plan(c["irreps_x"], c["irreps_y"], c["irreps_out"], dtype="f32", wkind="per_row")
    pos = synth.positions_for(c, 0)
    src, dst, vec = synth.radius_graph(pos, c["box"], c["r_cut"])
    N, E = pos.shape[0], src.shape[0]
    row_ptr, src_s, perm = cgtp.csr_from_coo(N, torch.from_numpy(src.astype(np.int32)).to(dev),
                                             torch.from_numpy(dst.astype(np.int32)).to(dev))
    graph = cgtp.Graph(N, row_ptr, src_s)
    vec_d = torch.from_numpy(vec).to(dev)[perm.long()].float().contiguous()
    Y = cgtp.sh_forward(c["L"], vec_d)
    W1, W2 = synth.mlp_params(8, 64, plan.w_numel, 0)
    W1, W2 = torch.from_numpy(W1).float().to(dev), torch.from_numpy(W2).float().to(dev)
    r = vec_d.norm(dim=1)
    w = torch.empty((E, plan.w_numel), device=dev)
    for a in range(0, E, 1 << 20):
        w[a:a + (1 << 20)] = synth.radial_weights_torch(r[a:a + (1 << 20)], c["r_cut"], W1, W2)
    gen = torch.Generator(device=dev)
    gen.manual_seed(0)
    x = torch.randn((N, plan.dim_x), generator=gen, device=dev)
    gout = torch.randn((N, plan.dim_out), generator=gen, device=dev)
    scale = 1.0 / math.sqrt(E / N)
    out = torch.empty((N, plan.dim_out), device=dev)
    dx, dY, dw = torch.empty_like(x), torch.empty_like(Y), torch.empty_like(w)
    ws = torch.empty(plan.workspace_size(cgtp.OP_CONV_BACKWARD, graph=graph), dtype=torch.uint8, device=dev)
    gvec = torch.empty_like(vec_d)
    tf, tb, tsf, tsb = KernelTimer(torch), KernelTimer(torch), KernelTimer(torch), KernelTimer(torch)
    for k in range(steps + 1):
        if k == 0:
            plan.conv_forward(graph, x, Y, w, scale, out=out)
            plan.conv_backward(graph, x, Y, w, scale, gout, out=(dx, dY, dw), ws=ws)
        else:
            if forces:
                tsf(lambda: cgtp.sh_forward(c["L"], vec_d, out=Y))
            tf(lambda: plan.conv_forward(graph, x, Y, w, scale, out=out))
            tb(lambda: plan.conv_backward(graph, x, Y, w, scale, gout, out=(dx, dY, dw), ws=ws))
            if forces:
                tsb(lambda: cgtp.sh_backward(c["L"], vec_d, dY, out=gvec))
    torch.cuda.synchronize()
    bf = 4 * (plan.w_numel + plan.dim_y + 1) * E + 4 * (plan.dim_out + plan.dim_x + 1) * N
    bb = 4 * (2 * plan.w_numel + 2 * plan.dim_y + 1) * E + 4 * (plan.dim_out + 2 * plan.dim_x + 1) * N
    msf, msb = tf.mean_ms(), tb.mean_ms()
    cv = ["conv_impl.hpp", "conv_kernels.hip", "tp_core.hpp", "cg_pattern.h", "device_util.hpp"]
    tr_f = traffic_for("conv_fwd_fused_kernel", cv, E) if name == "conv_uniform100k" else None
    tr_b = None
    if name == "conv_uniform100k":
        b1, b2 = traffic_for("conv_bwd_fused_kernel", cv, E), traffic_for("dx_gather_kernel", cv, E)
        tr_b = b1 + b2 if b1 is not None and b2 is not None else None
    res = dict(N=N, E=E, paths=plan.num_paths, fwd_traffic_bytes=tr_f, bwd_traffic_bytes=tr_b,
               fwd_ms=round(msf, 3), fwd_edges_per_s=E / (msf * 1e-3),
               fwd_algorithmic_GBs=round(bf / (msf * 1e-3) / 1e9, 1),
               fwd_frac_of_hbm_peak=round(bf / (msf * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
               bwd_ms=round(msb, 3), fwd_bwd_edges_per_s=E / ((msf + msb) * 1e-3),
               bwd_algorithmic_GBs=round(bb / (msb * 1e-3) / 1e9, 1),
               fwd_bytes_per_edge=bf / E, bwd_bytes_per_edge=bb / E)
    if forces:
        res.update(sh_fwd_ms=round(tsf.mean_ms(), 4), sh_bwd_ms=round(tsb.mean_ms(), 4),
                   fwd_bwd_forces_edges_per_s=E / ((msf + msb + tsf.mean_ms() + tsb.mean_ms()) * 1e-3))
    del w, dw, ws, x, gout, out, dx, dY, Y, graph, gvec
    torch.cuda.empty_cache()
    return res


def cpu_baseline(args, synth):
    """The oracle as it stands, tp_large fwd+bwd on a bounded row sample."""
    import numpy as np
    from oracle import sh as osh
    from oracle import tp as otp
    from oracle.irreps import Layout
    c = synth.CONFIGS["tp_large"]
    L = Layout(c["irreps_x"], c["irreps_y"], c["irreps_out"])

    def run(rows):
        x = synth.gaussian((rows, L.dim_x), 1, synth.S_X)
        y = osh.real_sh(3, synth.unit_vectors(rows, 1))
        w = synth.gaussian((rows, L.w_numel), 1, synth.S_W)
        g = synth.gaussian((rows, L.dim_out), 1, synth.S_G)
        t0 = time.perf_counter()
        otp.forward(L, x, y, w)
        otp.backward(L, x, y, w, g)
        return time.perf_counter() - t0

    probe = 64
    dt = run(probe)
    rows = int(min(65536, max(probe, probe * args.cpu_seconds / max(dt, 1e-3))))
    dt = run(rows)
    return {"value": rows / dt, "unit": "pairs/s", "cores": 1, "kind": "oracle",
            "sample": "tp_large fwd+bwd (harmonics excluded) on %d rows, fp64 NumPy, single thread, %.1f s"
                      % (rows, dt)}


def main():
    args = parse()
    if args.gpus != 1:
        print("bench.py measures one GPU only: this build has no multi-GPU path (--gpus %d refused)"
              % args.gpus, file=sys.stderr)
        sys.exit(2)
    import torch
    from clebsch_gordan_tensor_amd import cgtp, synth
    assert torch.cuda.is_available(), "bench.py needs a GPU"
    torch.cuda.set_device(0)
    if args.calibrate_copy:
        calibrate_copy(torch)
        return
    extra = {"device": torch.cuda.get_device_name(0)}
    value, ms_step, roofline, plan = tp_large_bench(args, torch, cgtp, synth, extra)
    extra["tp_large_bf16"] = tp_large_bf16(args, torch, cgtp, synth)
    if not args.no_conv:
        for name in ("conv_water1k", "conv_water8k", "conv_uniform100k"):
            extra[name] = conv_bench(args, torch, cgtp, synth, name, max(2, min(args.steps, 5)),
                                     forces=name == "conv_water8k")
    cpu = None if args.no_cpu_baseline else cpu_baseline(args, synth)
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
