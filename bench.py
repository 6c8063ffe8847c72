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

# HBM-side bytes per launch measured with rocprofv3 FETCH_SIZE and WRITE_SIZE
# passes (each scaled by what the counter reads for a plain 1 GiB device copy:
# x2.0 and x1.0), on the ep_share_32k workload. Valid only for the GEMM
# sources they were taken on: any change to those files reports null.
TRAFFIC_SOURCES = ("token_dispatch_grouped_amd/csrc/gemm_bf16.hip", "token_dispatch_grouped_amd/csrc/gemm_common.h",
                   "token_dispatch_grouped_amd/csrc/common.h")
TRAFFIC = {
    "sources_sha256": "26df0d780eb7acba45fa54e98f68a4257e29deceb907aa68d1bc026f2041b7af",
    "workload": "ep_share_32k",
    "bytes_per_launch": {
        # read GiB + write GiB, x 2^30
        "gg_gateup_fwd": (7.186 + 2.064) * 2 ** 30,
        "gg_down_fwd": (2.454 + 1.000) * 2 ** 30,
        "gg_down_dgrad": (4.888 + 1.375) * 2 ** 30,
        "gg_down_wgrad": (5.709 + 0.322) * 2 ** 30,
        "gg_gateup_dgrad": (5.048 + 1.000) * 2 ** 30,
        "gg_gateup_wgrad": (10.663 + 0.645) * 2 ** 30,
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


def main():
    args = parse()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print("bench.py measures one GPU only: this library models one expert-parallel rank's local share "
              "on a single MI355X and has no multi-GPU path; run with --gpus 1.", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    import token_dispatch_grouped_amd as moe
    from token_dispatch_grouped_amd.layer import MoeLayer
    from workloads import BF16, F32, WORKLOADS, make_inputs

    w = WORKLOADS[args.workload]
    assert torch.cuda.is_available(), "bench.py needs a GPU"
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    moe.load()

    t_gen = time.perf_counter()
    inp = make_inputs(w)
    t_gen = time.perf_counter() - t_gen

    def dev_t(a, dtype):
        if a.dtype == np.uint16:
            return torch.from_numpy(a.view(np.int16)).view(torch.bfloat16).to(dev)
        return torch.from_numpy(a).to(dev)

    dt = moe.MOE_DTYPE_BF16 if w.dtype == BF16 else moe.MOE_DTYPE_F32
    router = w.routing == "router"
    Tmax = max(max(w.microbatches), 1)
    layer = MoeLayer(Tmax, w.d, w.E, w.k, w.F, dt, renorm=args.renorm, router=router,
                     recompute=args.mode != "train", aux=(0.01, 1e-3) if args.aux else None)
    W = inp["weights"]
    wgu, wdn = dev_t(W["w_gu"], w.dtype), dev_t(W["w_down"], w.dtype)
    wr = dev_t(W["w_router"], w.dtype) if router else None
    bias = dev_t(W["bias"], F32) if router else None
    mbs = []
    for mb in inp["micro"]:
        T = mb["x"].shape[0]
        mbs.append(dict(T=T, x=dev_t(mb["x"], w.dtype), dout=dev_t(mb["dout"], w.dtype),
                        logits=None if router else dev_t(np.ascontiguousarray(mb["logits"]), F32)))
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

    for _ in range(args.warmup):
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
        for _ in range(args.steps):
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
    ms_per_step = stream_ms / args.steps

    flops_step = w.flops_fwd() if nograd else w.flops_fwd_bwd()
    value = flops_step / (ms_per_step * 1e-3) / 1e12
    s = 2 if w.dtype == BF16 else 4
    peak = PEAK_BF16_TFLOPS if w.dtype == BF16 else PEAK_F32_TFLOPS

    kernels = {}
    for name, (n, ms) in kern.items():
        avg = ms / max(n, 1)
        entry = {"launches": n, "avg_ms": round(avg, 5), "total_ms_per_step": round(ms / args.steps, 4)}
        base = name.replace("_f32", "")
        if base in GEMM_KERNELS:
            fl_step = sum(GEMM_KERNELS[base] * mb["T"] * w.k * w.d * w.F for mb in mbs)
            launches_step = max(1, n // args.steps)
            tf = fl_step / (ms / args.steps * 1e-3) / 1e12
            entry.update(tflops=round(tf, 2), pct_peak=round(100 * tf / peak, 2),
                         flops_per_launch=fl_step / launches_step)
        elif name in MEM_KERNELS:
            by = sum(mem_bytes(name, mb["T"], w.d, w.k, s, router) for mb in mbs)
            gbps = by / (ms / args.steps * 1e-3) / 1e9
            entry.update(GBps=round(gbps, 1), pct_peak=round(100 * gbps / PEAK_HBM_GBPS, 2))
        elif name == "adamw":
            # theta, grad, m, v read; theta, m, v, bf16 copy, zeroed grad written
            by = 3 * w.E * w.F * w.d * (28 + (2 if w.dtype == BF16 else 0) + 4)
            gbps = by / (ms / args.steps * 1e-3) / 1e9
            entry.update(GBps=round(gbps, 1), pct_peak=round(100 * gbps / PEAK_HBM_GBPS, 2))
        kernels[name] = entry

    gemm_names = [n for n in kernels if n.replace("_f32", "") in GEMM_KERNELS]
    gemm_ms = sum(kernels[n]["total_ms_per_step"] for n in gemm_names)
    gemm_fl = sum(GEMM_KERNELS[n.replace("_f32", "")] * mb["T"] * w.k * w.d * w.F for n in gemm_names for mb in mbs)
    mem_names = [n for n in kernels if n in MEM_KERNELS]
    mem_ms = sum(kernels[n]["total_ms_per_step"] for n in mem_names)
    mem_by = sum(mem_bytes(n, mb["T"], w.d, w.k, s, router) for n in mem_names for mb in mbs)
    # executed GEMM FLOPs (the recompute product included) over GEMM time
    gemm_tf = gemm_fl / (gemm_ms * 1e-3) / 1e12 if gemm_ms else 0.0
    pc_gbps = mem_by / (mem_ms * 1e-3) / 1e9 if mem_ms else 0.0

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
    else:
        per_launch = sum(mem_bytes(dom, mb["T"], w.d, w.k, s, router) for mb in mbs) / max(1, kernels[dom][
            "launches"] // args.steps)
        ach = per_launch / (kernels[dom]["avg_ms"] * 1e-3) / 1e9
        roof = {"kernel": dom, "bound": "hbm", "achieved": round(ach, 1), "peak": PEAK_HBM_GBPS, "unit": "GB/s",
                "frac": round(ach / PEAK_HBM_GBPS, 4), "traffic": None}

    # the recompute product is work done beyond the method's own FLOPs
    executed_fl = flops_step + (GEMM_KERNELS["gg_gateup_recompute"] * sum(mb["T"] for mb in mbs) * w.k * w.d * w.F
                                if args.mode == "recompute" else 0.0)
    cfg = {"workload": w.name, "seed": w.seed, "T": list(w.microbatches) if w.micro_T else w.T, "d": w.d, "E_local": w.E,
           "k": w.k, "F": w.F, "routing": w.routing, "renorm": bool(args.renorm), "mode": args.mode,
           "optimizer": "adamw" if opt is not None else None, "aux_losses": bool(args.aux),
           "description": w.description}
    line = {
        "metric": METRIC_NOGRAD if nograd else METRIC, "value": round(value, 2), "unit": "TFLOP/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(ms_per_step, 4), "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "bf16" if w.dtype == BF16 else "f32", "data": "synthetic",
        "config": cfg,
        "pct_bf16_peak": round(100 * value / PEAK_BF16_TFLOPS, 2),
        "grouped_gemm_tflops": round(gemm_tf, 2),
        "grouped_gemm_pct_peak": round(100 * gemm_tf / peak, 2),
        "permute_combine_GBps": round(pc_gbps, 1),
        "permute_combine_pct_hbm": round(100 * pc_gbps / PEAK_HBM_GBPS, 2),
        "executed_tflops": round(executed_fl / (ms_per_step * 1e-3) / 1e12, 2),
        "wall_s_timed": round(wall, 3),
        "ms_per_step_with_kernel_events": round(prof_ms / args.steps, 4),
        "device_memory_GB": round(torch.cuda.max_memory_allocated(dev) / 1e9, 2),
        "host_cpu": host_cpu_model(),
        "input_gen_s": round(t_gen, 2),
        "kernels": kernels,
        "roofline": roof,
    }
    if args.cpu_seconds > 0:
        line["cpu_baseline"] = cpu_baseline(w, inp, args.cpu_seconds, fwd_only=nograd)
    else:
        line["cpu_baseline"] = None
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
