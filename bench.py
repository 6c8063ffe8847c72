"""Benchmark of the MoE layer hot path (forward + backward) on one MI355X.

One step = one pass of the whole path over one synthetic batch, through the
C ABI: moe_route, moe_permute, moe_grouped_gemm_fwd, moe_unpermute_combine,
moe_unpermute_combine_bwd, moe_route_bwd, moe_grouped_gemm_bwd,
moe_permute_bwd (every microbatch of the workload, weight gradients
accumulating in fp32). Inputs are resident in HBM before timing starts.

Prints one JSON line. ``value`` is the layer's algorithmic TFLOP/s
(18*R*d*F per step, R = T*k routed rows, plus 6*T*d*E when the router GEMM
runs) over the stream time of K timed steps. A second run of K steps brackets
every kernel with HIP events on its launch stream: the per-kernel table and
``roofline`` (the dominant kernel) come from it. ``cpu_baseline`` is the
fp64 oracle timed on a bounded sample of the same workload on this host's
cores.

``--mode recompute`` runs the same step with MOE_FLAG_RECOMPUTE (no h/a kept
between forward and backward; the backward recomputes them): ``value`` stays
the algorithmic rate (the recompute product is extra work the method does not
need) and ``executed_tflops`` counts it. ``--mode nograd`` times the forward
alone under MOE_FLAG_RECOMPUTE (no activations kept), value = 6*R*d*F per
step over its time. The default (``train``) is the headline measurement.
``--optimizer`` appends the fused AdamW update of both expert weight tensors
(fp32 masters and moments, bf16 working copies written in place, gradients
zeroed in the same pass) to every training step; its kernel is reported as
``adamw`` with 34 bytes per weight element.

With the default workload (ep_share_32k) the line also carries
``other_32k_workloads``: the empty-microbatch accumulation run, the d=4096
uniform and Zipf shares, each timed the same way over ``--other-steps``
steps (ms/step, layer TFLOP/s, grouped-GEMM % of peak, permute/combine GB/s,
per-kernel times), and two expert-parallel ranks simulated on one GPU with
uneven token counts (``ep2_loopback_32k``: 64 experts, 32 per rank, the
exchanges as device copies; the exchange and regroup kernels in GB/s). ``attainable`` holds the rates the library's probes reach
on this GPU (a bf16 MFMA loop from registers and a 1 GiB device copy); every
GEMM and memory kernel is also reported as a percentage of those
(``pct_attainable``). Routing kernels report GB/s on their algorithmic bytes
(fp32 logits and int32 tables), and as a percentage of the same copy probe
run at 4 MiB (``pct_copy_4MiB``), the size at which such kernels live.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "MoE layer fwd+bwd TFLOP/s & % bf16 MFMA peak; permute/combine GB/s"
METRIC_NOGRAD = "MoE layer forward (no-grad) TFLOP/s & % bf16 MFMA peak; permute/combine GB/s"
PEAK_BF16_TFLOPS = 2500.0   # MI355X dense bf16 MFMA
PEAK_F32_TFLOPS = 157.3     # MI355X fp32 vector
PEAK_HBM_GBPS = 8000.0      # MI355X HBM3E

GEMM_KERNELS = {
    # name: FLOPs per launch in units of R*d*F
    "gg_gateup_fwd": 4, "gg_down_fwd": 2, "gg_down_dgrad": 2, "gg_down_wgrad": 2, "gg_gateup_dgrad": 4,
    "gg_gateup_wgrad": 4, "gg_gateup_recompute": 4,
}
MEM_KERNELS = ("permute", "combine", "combine_bwd", "permute_bwd")
ROUTE_TOKENS = 64  # tokens per workgroup of the route pass (its histograms are [T/64, E] int32)
# size of the copy the routing kernels are set against: 4 MiB copied (8 MiB of HBM traffic), the order of the
# 7-13 MB a routing kernel moves on the 32k-token workloads
ROUTE_COPY_BYTES = 4 << 20

# HBM-side bytes per launch measured with rocprofv3 FETCH_SIZE and WRITE_SIZE
# passes (each scaled by what the counter reads for a plain 1 GiB device copy:
# x2.0 and x1.0), on the ep_share_32k workload. Valid only for the GEMM
# sources and build options they were taken on: any change to those files
# reports null.
TRAFFIC_SOURCES = ("token_dispatch_grouped_amd/csrc/gemm_bf16.hip", "token_dispatch_grouped_amd/csrc/gemm_bf16_ilp.hip",
                   "token_dispatch_grouped_amd/csrc/gemm_bf16_kernel.h", "token_dispatch_grouped_amd/csrc/gemm_common.h",
                   "token_dispatch_grouped_amd/csrc/common.h", "token_dispatch_grouped_amd/build.py")
TRAFFIC = {
    "sources_sha256": "5cb16b5d5c047803b0bcdf39d692ce7317c4aa2be384891d536bff0bd5b661b7",
    "workload": "ep_share_32k",
    "bytes_per_launch": {
        # read GiB + write GiB, x 2^30
        "gg_gateup_fwd": (6.646 + 2.062) * 2 ** 30,
        "gg_down_fwd": (2.419 + 1.000) * 2 ** 30,
        "gg_down_dgrad": (4.589 + 1.375) * 2 ** 30,
        "gg_down_wgrad": (6.364 + 0.322) * 2 ** 30,
        "gg_gateup_dgrad": (5.061 + 1.000) * 2 ** 30,
        "gg_gateup_wgrad": (10.677 + 0.645) * 2 ** 30,
    },
}


def measured_traffic(kernel, workload):
    """Bytes per launch from the counter passes, or None when the GEMM
    sources or the workload differ from those the counters were taken on."""
    import hashlib
    h = hashlib.sha256()
    try:
        for f in TRAFFIC_SOURCES:
            h.update(open(os.path.join(ROOT, f), "rb").read())
    except OSError:
        return None
    if h.hexdigest() != TRAFFIC["sources_sha256"] or workload != TRAFFIC["workload"]:
        return None
    return TRAFFIC["bytes_per_launch"].get(kernel)


def mem_bytes(name, T, d, k, s, router=False):
    """Algorithmic HBM bytes of one launch of a data-movement kernel."""
    if name == "permute":
        return T * ((1 + k) * d * s + 4 * k)
    if name == "combine":
        return T * ((k + 1) * d * s + 8 * k)
    if name == "combine_bwd":
        return T * ((1 + 2 * k) * d * s + 12 * k)
    if name == "permute_bwd":
        return T * ((k + 1) * d * s + 4 * k + (4 * d if router else 0))
    raise KeyError(name)


def parse():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="ep_share_32k")
    ap.add_argument("--cpu-seconds", type=float, default=15.0,
                    help="target wall time of the oracle's timed sample (0 disables the CPU baseline)")
    ap.add_argument("--renorm", action="store_true")
    ap.add_argument("--mode", choices=("train", "recompute", "nograd"), default="train",
                    help="train: forward+backward keeping h and a (default); recompute: forward+backward with "
                         "MOE_FLAG_RECOMPUTE; nograd: forward alone with MOE_FLAG_RECOMPUTE")
    ap.add_argument("--aux", action="store_true",
                    help="add the auxiliary losses (load balancing 0.01, router z-loss 0.001) and routing metrics "
                         "to the forward and their gradient to the backward")
    ap.add_argument("--optimizer", action="store_true",
                    help="append the fused AdamW update of the expert weights to every step (train/recompute)")
    ap.add_argument("--other-steps", type=int, default=10,
                    help="timed steps of each other 32k-token workload (microbatches_32k, large_share_uniform, "
                         "large_share_zipf) measured after the default ep_share_32k one; 0 skips them")
    ap.add_argument("--no-attainable", dest="attainable", action="store_false",
                    help="skip the MFMA-loop and copy probes of the attainable peaks")
    ap.add_argument("--calibrate-copy", type=int, default=0, metavar="BYTES",
                    help="also run one plain device copy of BYTES bytes before timing (a known-size reference "
                         "for the FETCH_SIZE / WRITE_SIZE counters)")
    return ap.parse_args()


def host_cpu_model():
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return None


def cpu_baseline(w, inp, target_s, fwd_only=False):
    """Time the fp64 oracle (as it is) on the first T_s tokens of the first
    microbatch: one forward+backward (forward alone if fwd_only), T_s sized
    to take about target_s."""
    import numpy as np
    import oracle
    from workloads import to_f64
    try:
        from threadpoolctl import threadpool_info
        threads = max([i.get("num_threads", 1) for i in threadpool_info()] + [1])
    except Exception:
        threads = os.cpu_count() or 1
    W = inp["weights"]
    wgu, wdn = to_f64(W["w_gu"], w.dtype), to_f64(W["w_down"], w.dtype)
    router = w.routing == "router"
    wr = to_f64(W["w_router"], w.dtype) if router else None
    bias = W["bias"].astype(np.float64) if router else None
    mb = next(m for m in inp["micro"] if m["x"].shape[0] > 0)
    T_full = mb["x"].shape[0]

    def run(Ts):
        x = to_f64(mb["x"][:Ts], w.dtype)
        dout = to_f64(mb["dout"][:Ts], w.dtype)
        t0 = time.perf_counter()
        if router:
            _, sv = oracle.layer_fwd(x, wgu, wdn, w.k, w_router=wr, bias=bias)
        else:
            _, sv = oracle.layer_fwd(x, wgu, wdn, w.k, logits=mb["logits"][:Ts].astype(np.float64))
        if not fwd_only:
            oracle.layer_bwd(dout, sv, wgu, wdn, x=x, w_router=wr)
        return time.perf_counter() - t0

    # size the sample from a 1024-token probe (small probes overstate the
    # per-token cost: per-expert overheads dominate them)
    Ts = min(T_full, 1024)
    dt = run(Ts)
    if dt < target_s and Ts < T_full:
        Ts = int(min(T_full, max(Ts, Ts * target_s / max(dt, 1e-3))))
        dt = run(Ts)
    flops = w.flops_fwd(Ts) if fwd_only else w.flops_fwd_bwd(Ts)
    what = "forward" if fwd_only else "forward+backward"
    return {"value": flops / dt / 1e12, "unit": "TFLOP/s", "cores": threads, "kind": "oracle",
            "sample": f"fp64 NumPy oracle, one {what} of the first {Ts} of {T_full} tokens "
                      f"of the same inputs ({dt:.1f} s)"}


def route_bytes(name, T, E, k, nblk, renorm=False):
    """Algorithmic HBM bytes of one launch of a routing kernel (fp32 logits,
    int32 tables), or None for a kernel without a model."""
    if name == "route_topk":      # logits in; ids, weights, in-workgroup ranks out; histograms out
        return T * (4 * E + 12 * k) + 4 * nblk * E
    if name == "route_scan":      # histograms scanned in place; counts out
        return 8 * nblk * E + 4 * E
    if name == "route_rows":      # ids and ranks in (+ the histogram table once); rows and inverse out
        return 16 * T * k + 4 * nblk * E + 8 * E
    if name == "route_bwd":       # dtopk_w, ids, weights in; logits in (no renorm); dlogits out
        return T * ((4 if renorm else 8) * E + 12 * k)
    return None


def attainable_peaks(dev):
    """Rates measured on this GPU by the library's probes: the bf16 MFMA loop
    (best of three ~5 ms launches) and a 2 x 1 GiB device copy (median of
    ten), each timed with HIP events on the launch stream."""
    import torch
    import token_dispatch_grouped_amd as moe
    stream = torch.cuda.current_stream()
    out = torch.empty(moe.moe_peak_mfma_size(), dtype=torch.float32, device=dev)
    best = 0.0
    for i in range(4):
        ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        ev0.record(stream)
        fl = moe.moe_peak_mfma(out, 40000)
        ev1.record(stream)
        torch.cuda.synchronize()
        if i:  # the first launch warms up
            best = max(best, fl / (ev0.elapsed_time(ev1) * 1e-3) / 1e12)
    nbytes = 1 << 30
    src = torch.empty(nbytes, dtype=torch.uint8, device=dev).fill_(1)
    dst = torch.empty(nbytes, dtype=torch.uint8, device=dev)
    rates = []
    for i in range(13):
        ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        ev0.record(stream)
        moe.moe_peak_copy(src, dst, nbytes)
        ev1.record(stream)
        torch.cuda.synchronize()
        if i >= 3:
            rates.append(2 * nbytes / (ev0.elapsed_time(ev1) * 1e-3) / 1e9)
    # the same copy at the routing kernels' size (a few MB per launch), where
    # launch and first-access latency, not bandwidth, set the time
    small = ROUTE_COPY_BYTES
    small_rates = []
    for i in range(23):
        ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        ev0.record(stream)
        moe.moe_peak_copy(src, dst, small)
        ev1.record(stream)
        torch.cuda.synchronize()
        if i >= 3:
            small_rates.append(2 * small / (ev0.elapsed_time(ev1) * 1e-3) / 1e9)
    del src, dst, out
    torch.cuda.empty_cache()
    rates.sort()
    small_rates.sort()
    return {"mfma_bf16_tflops": round(best, 1), "copy_GBps": round(rates[len(rates) // 2], 1),
            "copy_4MiB_GBps": round(small_rates[len(small_rates) // 2], 1),
            "mfma_probe": "v_mfma_f32_32x32x16_bf16 from registers, 2 wavefronts per SIMD x 4 accumulator chains",
            "copy_probe": f"16-byte non-temporal device copy of {nbytes >> 20} MiB (2x that in HBM traffic)",
            "copy_4MiB_probe": f"the same copy of {small >> 20} MiB (median of 20 launches)"}


def measure(w, args, steps, warmup, attain=None, keep_inputs=False):
    """Warm up, then time K steps of the workload without instrumentation and
    K more with per-kernel events. Returns the line's fields."""
    import numpy as np
    import torch

    import token_dispatch_grouped_amd as moe
    from token_dispatch_grouped_amd.layer import MoeLayer
    from workloads import BF16, F32, make_inputs

    dev = torch.device("cuda:0")
    t_gen = time.perf_counter()
    inp = make_inputs(w)
    t_gen = time.perf_counter() - t_gen

    def dev_t(a):
        if a.dtype == np.uint16:
            return torch.from_numpy(a.view(np.int16)).view(torch.bfloat16).to(dev)
        return torch.from_numpy(a).to(dev)

    dt = moe.MOE_DTYPE_BF16 if w.dtype == BF16 else moe.MOE_DTYPE_F32
    router = w.routing == "router"
    Tmax = max(max(w.microbatches), 1)
    torch.cuda.reset_peak_memory_stats(dev)
    layer = MoeLayer(Tmax, w.d, w.E, w.k, w.F, dt, renorm=args.renorm, router=router,
                     recompute=args.mode != "train", aux=(0.01, 1e-3) if args.aux else None)
    W = inp["weights"]
    wgu, wdn = dev_t(W["w_gu"]), dev_t(W["w_down"])
    wr = dev_t(W["w_router"]) if router else None
    bias = dev_t(W["bias"]) if router else None
    mbs = []
    for mb in inp["micro"]:
        T = mb["x"].shape[0]
        mbs.append(dict(T=T, x=dev_t(mb["x"]), dout=dev_t(mb["dout"]),
                        logits=None if router else dev_t(np.ascontiguousarray(mb["logits"]))))
    dw_gu = torch.zeros(w.E, 2 * w.F, w.d, dtype=torch.float32, device=dev)
    dw_dn = torch.zeros(w.E, w.d, w.F, dtype=torch.float32, device=dev)
    dw_r = torch.zeros(w.E, w.d, dtype=torch.float32, device=dev) if router else None
    torch.cuda.synchronize()

    nograd = args.mode == "nograd"
    opt = None
    if args.optimizer and not nograd:
        from token_dispatch_grouped_amd.optim import ExpertAdamW
        opt = ExpertAdamW([wgu, wdn], lr=1e-5, betas=(0.9, 0.95), eps=1e-8, weight_decay=0.1)

    def step():
        for mb in mbs:
            T = mb["T"]
            layer.forward(T, mb["x"], wgu, wdn, logits=mb["logits"], w_router=wr, bias=bias)
            if not nograd:
                layer.backward(T, mb["dout"], wgu, wdn, dw_gu, dw_dn, x=mb["x"], w_router=wr, dw_router=dw_r)
        if opt is not None:
            opt.step([dw_gu, dw_dn], grad_scale=1.0 / len(mbs), zero_grad=True)

    if args.calibrate_copy > 0:
        src = torch.empty(args.calibrate_copy, dtype=torch.uint8, device=dev).fill_(1)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst

    for _ in range(warmup):
        step()
    torch.cuda.synchronize()

    stream = torch.cuda.current_stream()

    def timed(profile):
        """K steps between a synchronize and HIP events on the launch stream;
        with profile, every kernel is also bracketed by events of its own."""
        ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        moe.moe_profiler_reset()
        moe.moe_profiler_enable(profile)
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        ev0.record(stream)
        for _ in range(steps):
            step()
        ev1.record(stream)
        torch.cuda.synchronize()
        wall_s = time.perf_counter() - t0
        moe.moe_profiler_enable(False)
        return ev0.elapsed_time(ev1), wall_s

    # the step rate without instrumentation, then the same K steps with the
    # per-kernel events (whose recording adds a little time of its own)
    stream_ms, wall = timed(False)
    prof_ms, _ = timed(True)
    kern = moe.moe_profiler_read_all()
    ms_per_step = stream_ms / steps

    flops_step = w.flops_fwd() if nograd else w.flops_fwd_bwd()
    value = flops_step / (ms_per_step * 1e-3) / 1e12
    s = 2 if w.dtype == BF16 else 4
    peak = PEAK_BF16_TFLOPS if w.dtype == BF16 else PEAK_F32_TFLOPS
    att_tf = attain["mfma_bf16_tflops"] if attain and w.dtype == BF16 else None
    att_bw = attain["copy_GBps"] if attain else None
    att_bw_small = attain.get("copy_4MiB_GBps") if attain else None

    kernels = {}
    for name, (n, ms) in kern.items():
        avg = ms / max(n, 1)
        entry = {"launches": n, "avg_ms": round(avg, 5), "total_ms_per_step": round(ms / steps, 4)}
        base = name.replace("_f32", "")
        by = None
        if base in GEMM_KERNELS:
            fl_step = sum(GEMM_KERNELS[base] * mb["T"] * w.k * w.d * w.F for mb in mbs)
            launches_step = max(1, n // steps)
            tf = fl_step / (ms / steps * 1e-3) / 1e12
            entry.update(tflops=round(tf, 2), pct_peak=round(100 * tf / peak, 2),
                         flops_per_launch=fl_step / launches_step)
            if att_tf:
                entry["pct_attainable"] = round(100 * tf / att_tf, 2)
        elif name in MEM_KERNELS:
            by = sum(mem_bytes(name, mb["T"], w.d, w.k, s, router) for mb in mbs)
        elif name == "adamw":
            # theta, grad, m, v read; theta, m, v, bf16 copy, zeroed grad written
            by = 3 * w.E * w.F * w.d * (28 + (2 if w.dtype == BF16 else 0) + 4)
        elif route_bytes(name, 1, w.E, w.k, 1) is not None:
            by = sum(route_bytes(name, mb["T"], w.E, w.k, -(-mb["T"] // ROUTE_TOKENS), args.renorm) for mb in mbs if mb["T"])
        if by is not None:
            gbps = by / (ms / steps * 1e-3) / 1e9
            entry.update(GBps=round(gbps, 1), pct_peak=round(100 * gbps / PEAK_HBM_GBPS, 2))
            if att_bw:
                entry["pct_attainable"] = round(100 * gbps / att_bw, 2)
            if att_bw_small and name.startswith("route_"):
                entry["pct_copy_4MiB"] = round(100 * gbps / att_bw_small, 2)
        kernels[name] = entry

    gemm_names = [n for n in kernels if n.replace("_f32", "") in GEMM_KERNELS]
    gemm_ms = sum(kernels[n]["total_ms_per_step"] for n in gemm_names)
    gemm_fl = sum(GEMM_KERNELS[n.replace("_f32", "")] * mb["T"] * w.k * w.d * w.F for n in gemm_names for mb in mbs)
    mem_names = [n for n in kernels if n in MEM_KERNELS]
    mem_ms = sum(kernels[n]["total_ms_per_step"] for n in mem_names)
    mem_by = sum(mem_bytes(n, mb["T"], w.d, w.k, s, router) for n in mem_names for mb in mbs)
    route_names = [n for n in kernels if route_bytes(n, 1, w.E, w.k, 1) is not None]
    route_ms = sum(kernels[n]["total_ms_per_step"] for n in route_names)
    route_by = sum(route_bytes(n, mb["T"], w.E, w.k, -(-mb["T"] // ROUTE_TOKENS), args.renorm)
                   for n in route_names for mb in mbs if mb["T"])
    # executed GEMM FLOPs (the recompute product included) over GEMM time
    gemm_tf = gemm_fl / (gemm_ms * 1e-3) / 1e12 if gemm_ms else 0.0
    pc_gbps = mem_by / (mem_ms * 1e-3) / 1e9 if mem_ms else 0.0
    route_gbps = route_by / (route_ms * 1e-3) / 1e9 if route_ms else 0.0

    # dominant kernel: largest share of the step
    # among the kernels with a roofline model (grouped GEMMs, dispatch/combine)
    modeled = [n for n in kernels if n.replace("_f32", "") in GEMM_KERNELS or n in MEM_KERNELS]
    dom = max(modeled, key=lambda n: kernels[n]["total_ms_per_step"])
    dbase = dom.replace("_f32", "")
    if dbase in GEMM_KERNELS:
        per_launch = kernels[dom]["flops_per_launch"]
        ach = per_launch / (kernels[dom]["avg_ms"] * 1e-3) / 1e12
        tr = measured_traffic(dom, w.name)
        roof = {"kernel": dom, "bound": "mfma", "achieved": round(ach, 2), "peak": peak, "unit": "TFLOP/s",
                "frac": round(ach / peak, 4), "traffic": None if tr is None else round(tr),
                "work_per_launch": f"{GEMM_KERNELS[dbase]}*R*d*F = {per_launch:.4g} FLOP"}
        if att_tf:
            roof["frac_of_attainable"] = round(ach / att_tf, 4)
    else:
        per_launch = sum(mem_bytes(dom, mb["T"], w.d, w.k, s, router) for mb in mbs) / max(1, kernels[dom][
            "launches"] // steps)
        ach = per_launch / (kernels[dom]["avg_ms"] * 1e-3) / 1e9
        roof = {"kernel": dom, "bound": "hbm", "achieved": round(ach, 1), "peak": PEAK_HBM_GBPS, "unit": "GB/s",
                "frac": round(ach / PEAK_HBM_GBPS, 4), "traffic": None}
        if att_bw:
            roof["frac_of_attainable"] = round(ach / att_bw, 4)

    # the recompute product is work done beyond the method's own FLOPs
    executed_fl = flops_step + (GEMM_KERNELS["gg_gateup_recompute"] * sum(mb["T"] for mb in mbs) * w.k * w.d * w.F
                                if args.mode == "recompute" else 0.0)
    res = {
        "value": round(value, 2), "ms_per_step": round(ms_per_step, 4), "steps": steps, "warmup": warmup,
        "pct_bf16_peak": round(100 * value / PEAK_BF16_TFLOPS, 2),
        "grouped_gemm_tflops": round(gemm_tf, 2),
        "grouped_gemm_pct_peak": round(100 * gemm_tf / peak, 2),
        "permute_combine_GBps": round(pc_gbps, 1),
        "permute_combine_pct_hbm": round(100 * pc_gbps / PEAK_HBM_GBPS, 2),
        "route_GBps": round(route_gbps, 1),
        "route_pct_hbm": round(100 * route_gbps / PEAK_HBM_GBPS, 2),
        "route_pct_copy_4MiB": round(100 * route_gbps / att_bw_small, 2) if att_bw_small else None,
        "executed_tflops": round(executed_fl / (ms_per_step * 1e-3) / 1e12, 2),
        "wall_s_timed": round(wall, 3),
        "ms_per_step_with_kernel_events": round(prof_ms / steps, 4),
        "device_memory_GB": round(torch.cuda.max_memory_allocated(dev) / 1e9, 2),
        "input_gen_s": round(t_gen, 2),
        "kernels": kernels,
        "roofline": roof,
    }
    if att_tf:
        res["grouped_gemm_pct_attainable"] = round(100 * gemm_tf / att_tf, 2)
    if att_bw:
        res["permute_combine_pct_attainable"] = round(100 * pc_gbps / att_bw, 2)
    del layer, mbs, wgu, wdn, wr, bias, dw_gu, dw_dn, dw_r, opt
    torch.cuda.synchronize()
    torch.cuda.empty_cache()
    return res, (inp if keep_inputs else None)


# the other 32k-token workloads, timed after the headline one in the default run
OTHER_32K = ("microbatches_32k", "large_share_uniform", "large_share_zipf")

# Expert-parallel ranks simulated on one GPU: two ranks of 32 local experts
# (64 in all), the second rank holding half the tokens of the first (uneven
# data-parallel inputs), Zipf(1.2) popularity over the 64 experts with 4 empty
EP_LOOPBACK = dict(name="ep2_loopback_32k", ep=2, Ts=(32768, 16384), d=2048, e_local=32, k=8, F=1408, seed=7,
                   zipf_s=1.2, n_empty=4)
EP_ROW_KERNELS = ("ep_exchange_rows", "ep_return_rows", "ep_regroup", "ep_ungroup")  # the last two: unfused only


def measure_ep(cfg, steps, warmup, attain=None):
    """The EP loopback step (forward + backward of every simulated rank,
    exchanges included), timed like measure(); GEMM and memory kernels summed
    over the ranks."""
    import numpy as np
    import torch

    import token_dispatch_grouped_amd as moe
    from token_dispatch_grouped_amd.ep import EpLoopback
    from workloads import make_ep_inputs

    dev = torch.device("cuda:0")
    ep, Ts, d, el, k, F = cfg["ep"], cfg["Ts"], cfg["d"], cfg["e_local"], cfg["k"], cfg["F"]
    t_gen = time.perf_counter()
    inp = make_ep_inputs(ep, Ts, d, el, k, F, "bf16", seed=cfg["seed"], routing="zipf", zipf_s=cfg["zipf_s"],
                         n_empty=cfg["n_empty"])
    t_gen = time.perf_counter() - t_gen

    def dev_t(a):
        if a.dtype == np.uint16:
            return torch.from_numpy(a.view(np.int16)).view(torch.bfloat16).to(dev)
        return torch.from_numpy(np.ascontiguousarray(a)).to(dev)

    torch.cuda.reset_peak_memory_stats(dev)
    lay = EpLoopback(ep, max(Ts), d, el, k, F, moe.MOE_DTYPE_BF16)
    wgu, wdn = dev_t(inp["weights"]["w_gu"]), dev_t(inp["weights"]["w_down"])
    xs = [dev_t(mb["x"]) for mb in inp["micro"]]
    lgs = [dev_t(mb["logits"]) for mb in inp["micro"]]
    douts = [dev_t(mb["dout"]) for mb in inp["micro"]]
    dw_gu = torch.zeros(ep * el, 2 * F, d, dtype=torch.float32, device=dev)
    dw_dn = torch.zeros(ep * el, d, F, dtype=torch.float32, device=dev)

    def step():
        lay.forward(Ts, xs, lgs, wgu, wdn)
        lay.backward(douts, wgu, wdn, dw_gu, dw_dn)

    for _ in range(warmup):
        step()
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream()

    def timed(profile):
        ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        moe.moe_profiler_reset()
        moe.moe_profiler_enable(profile)
        torch.cuda.synchronize()
        ev0.record(stream)
        for _ in range(steps):
            step()
        ev1.record(stream)
        torch.cuda.synchronize()
        moe.moe_profiler_enable(False)
        return ev0.elapsed_time(ev1)

    ms = timed(False) / steps
    timed(True)
    kern = moe.moe_profiler_read_all()
    R = sum(T * k for T in Ts)
    flops = 18.0 * R * d * F
    kernels = {}
    for name, (n, tot) in kern.items():
        e = {"launches_per_step": n // steps, "total_ms_per_step": round(tot / steps, 4)}
        if name in GEMM_KERNELS:
            # summed over the destination ranks: each product's FLOPs over all rows
            tf = GEMM_KERNELS[name] * R * d * F / (tot / steps * 1e-3) / 1e12
            e.update(tflops=round(tf, 2), pct_peak=round(100 * tf / PEAK_BF16_TFLOPS, 2))
        by = None
        if name in MEM_KERNELS:
            by = sum(mem_bytes(name, T, d, k, 2) for T in Ts)
        elif name in EP_ROW_KERNELS:
            # two calls per step (x and dy out, y and dx back); every row read and written once,
            # the regroup also reads its row map
            by = 2 * R * (2 * d * 2 + (4 if name in ("ep_regroup", "ep_ungroup") else 0))
        if by is not None:
            gbps = by / (tot / steps * 1e-3) / 1e9
            e.update(GBps=round(gbps, 1), pct_peak=round(100 * gbps / PEAK_HBM_GBPS, 2))
            if attain:
                e["pct_attainable"] = round(100 * gbps / attain["copy_GBps"], 2)
        kernels[name] = e
    gemm_ms = sum(kernels[n]["total_ms_per_step"] for n in kernels if n in GEMM_KERNELS)
    xch = [n for n in kernels if n in EP_ROW_KERNELS]
    xch_ms = sum(kernels[n]["total_ms_per_step"] for n in xch)
    xch_by = sum(2 * R * (2 * d * 2 + (4 if n in ("ep_regroup", "ep_ungroup") else 0)) for n in xch)
    res = {"value": round(flops / (ms * 1e-3) / 1e12, 2), "ms_per_step": round(ms, 4), "steps": steps,
           "ep": ep, "T_per_rank": list(Ts), "d": d, "E_local": el, "E_total": ep * el, "k": k, "F": F,
           "grouped_gemm_tflops": round(flops / (gemm_ms * 1e-3) / 1e12, 2) if gemm_ms else None,
           "exchange_regroup_GBps": round(xch_by / (xch_ms * 1e-3) / 1e9, 1) if xch_ms else None,
           "exchange_regroup_ms_per_step": round(xch_ms, 4),
           "device_memory_GB": round(torch.cuda.max_memory_allocated(dev) / 1e9, 2), "input_gen_s": round(t_gen, 2),
           "kernels": kernels,
           "note": "all ranks simulated on one GPU; the row and counts exchanges are device copies standing in for "
                   "the all-to-all(v) between GPUs"}
    if res["grouped_gemm_tflops"]:
        res["grouped_gemm_pct_peak"] = round(100 * res["grouped_gemm_tflops"] / PEAK_BF16_TFLOPS, 2)
    del lay, wgu, wdn, xs, lgs, douts, dw_gu, dw_dn
    torch.cuda.synchronize()
    torch.cuda.empty_cache()
    return res


def main():
    args = parse()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print("bench.py measures one GPU only: this library models one expert-parallel rank's local share "
              "on a single MI355X and has no multi-GPU path; run with --gpus 1.", file=sys.stderr)
        sys.exit(2)

    import torch

    import token_dispatch_grouped_amd as moe
    from workloads import BF16, WORKLOADS

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    moe.load()

    attain = attainable_peaks(dev) if args.attainable else None
    if args.workload == EP_LOOPBACK["name"]:
        # the expert-parallel loopback alone: layer TFLOP/s over all simulated ranks
        r = measure_ep(EP_LOOPBACK, args.steps, args.warmup, attain)
        line = {"metric": METRIC + " (EP ranks simulated on one GPU)", "value": r.pop("value"), "unit": "TFLOP/s",
                "n_gpus": 1, "steps": r.pop("steps"), "warmup": args.warmup, "ms_per_step": r.pop("ms_per_step"),
                "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
                "data": "synthetic", "config": {"workload": EP_LOOPBACK["name"], "seed": EP_LOOPBACK["seed"]},
                "attainable": attain, "cpu_baseline": None}
        line.update(r)
        print(json.dumps(line), flush=True)
        return
    w = WORKLOADS[args.workload]
    res, inp = measure(w, args, args.steps, args.warmup, attain, keep_inputs=args.cpu_seconds > 0)

    nograd = args.mode == "nograd"
    cfg = {"workload": w.name, "seed": w.seed, "T": list(w.microbatches) if w.micro_T else w.T, "d": w.d,
           "E_local": w.E, "k": w.k, "F": w.F, "routing": w.routing, "renorm": bool(args.renorm), "mode": args.mode,
           "optimizer": "adamw" if args.optimizer and not nograd else None, "aux_losses": bool(args.aux),
           "description": w.description}
    line = {
        "metric": METRIC_NOGRAD if nograd else METRIC, "value": res.pop("value"), "unit": "TFLOP/s", "n_gpus": 1,
        "steps": res.pop("steps"), "warmup": res.pop("warmup"), "ms_per_step": res.pop("ms_per_step"),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "bf16" if w.dtype == BF16 else "f32", "data": "synthetic", "config": cfg,
    }
    line.update(res)
    line["host_cpu"] = host_cpu_model()
    line["attainable"] = attain

    # the other 32k-token workloads (empty-microbatch accumulation, d = 4096
    # uniform and Zipf) under the same clock, fewer steps each
    if args.other_steps > 0 and w.name == "ep_share_32k":
        others = {}
        for name in OTHER_32K:
            ow = WORKLOADS[name]
            print(f"[bench] {name}", file=sys.stderr, flush=True)
            r, _ = measure(ow, args, args.other_steps, min(args.warmup, 3), attain)
            keep = ("value", "ms_per_step", "steps", "grouped_gemm_tflops", "grouped_gemm_pct_peak",
                    "grouped_gemm_pct_attainable", "permute_combine_GBps", "permute_combine_pct_hbm",
                    "permute_combine_pct_attainable", "route_GBps", "route_pct_hbm", "route_pct_copy_4MiB",
                    "device_memory_GB")
            o = {k: r[k] for k in keep if k in r}
            o["T"] = list(ow.microbatches) if ow.micro_T else ow.T
            o["d"], o["E_local"], o["F"] = ow.d, ow.E, ow.F
            o["kernels"] = {n: {k: v for k, v in e.items() if k in ("avg_ms", "total_ms_per_step", "tflops", "GBps",
                                                                     "pct_peak")}
                            for n, e in r["kernels"].items()}
            others[name] = o
        print(f"[bench] {EP_LOOPBACK['name']}", file=sys.stderr, flush=True)
        others[EP_LOOPBACK["name"]] = measure_ep(EP_LOOPBACK, args.other_steps, min(args.warmup, 3), attain)
        line["other_32k_workloads"] = others

    if args.cpu_seconds > 0:
        line["cpu_baseline"] = cpu_baseline(w, inp, args.cpu_seconds, fwd_only=nograd)
    else:
        line["cpu_baseline"] = None
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
