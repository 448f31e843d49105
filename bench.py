"""Benchmark of the routed MoE layer forward on one MI355X.

python bench.py [--steps K] [--warmup W] [--config NAME] [--n N] [--accum slot|atomic]

A step is one moe_forward call (router, top-k, experts, weighted sum and
shared-expert blend) on one batch of N synthetic tokens with the inputs
already in HBM. Token batches rotate through a pool and the weights through
enough copies that a call does not find its experts in the 256 MB Infinity
Cache left by earlier calls. Prints one JSON line: us per call (the metric),
expert-weight GB/s, per-kernel times from HIP events that bracket each kernel
(hipExtLaunchKernel start/stop events, the interval a kernel trace reports),
the roofline of the dominant kernel, and the FP64 oracle timed on the host
cores as a reference point.

Default workload: the Qwen3-30B-A3B-shaped MXFP4 layer at N = 1 token (decode
path, one fused kernel). --config grouped_fp8_h4096 / prefill_bf16_h4096 run
the grouped path (five launches: router, top-k with the grouping, gate+up,
down, combine).
"""

import argparse
import ctypes
import glob
import hashlib
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

H = None                       # libamdhip64 (ctypes), loaded by main()
HBM_PEAK_GBS = 8000.0          # MI355X HBM3E
MFMA_BF16_PEAK_TFLOPS = 2500.0  # MI355X dense BF16 MFMA
MALL_BYTES = 256 << 20
KERNELS = {1: ["k_moe_decode"],
           5: ["k_g_router", "k_g_topk", "k_g_gate_up", "k_g_down", "k_g_combine"]}
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "hbm_traffic.json")
MFMA_FILE = os.path.join(ROOT, "profiles", "mfma_counters.json")


def hip():
    L = ctypes.CDLL("libamdhip64.so")
    L.hipEventCreate.argtypes = [ctypes.POINTER(ctypes.c_void_p)]
    L.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.c_void_p,
                                      ctypes.c_void_p]
    L.hipEventSynchronize.argtypes = [ctypes.c_void_p]
    L.hipEventDestroy.argtypes = [ctypes.c_void_p]
    return L


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=400)
    p.add_argument("--warmup", type=int, default=50)
    p.add_argument("--config", default=None,
                   help="workload (default: qwen3_30b_a3b_mxfp4 at N=1, plus the points "
                        "N=3 of the same layer and deepseek_v3_nvfp4 at N=4)")
    p.add_argument("--no-points", action="store_true",
                   help="default run: time only the N=1 headline workload")
    p.add_argument("--n", type=int, default=None, help="tokens per call")
    p.add_argument("--accum", default=None, choices=[None, "slot", "atomic"])
    p.add_argument("--path", default="auto", choices=["auto", "decode", "grouped"])
    p.add_argument("--pool", type=int, default=64, help="distinct token batches")
    p.add_argument("--copies", type=int, default=None,
                   help="weight copies to rotate through (default: enough that a copy's "
                        "bytes have left the 256 MB Infinity Cache before it is used again)")
    p.add_argument("--cpu-seconds", type=float, default=12.0,
                   help="budget of the oracle baseline (0 = skip)")
    p.add_argument("--no-trace", action="store_true", help="time without per-kernel events")
    p.add_argument("--graph", action="store_true",
                   help="time the K calls as one captured HIP graph (replayed once) instead "
                        "of K eager launches")
    p.add_argument("--copy-calibration", action="store_true",
                   help="only run a plain 256 MiB device copy three times (for scaling "
                        "FETCH_SIZE / WRITE_SIZE counter readings) and exit")
    p.add_argument("--read-calibration", action="store_true",
                   help="only run a 256 MiB read-only reduction three times (a second "
                        "FETCH_SIZE scale) and exit")
    return p.parse_args()


def copy_calibration():
    """A plain copy kernel of known size: 256 MiB read and 256 MiB written
    per dispatch, so counter readings of it give the counters' scale."""
    import torch
    nbytes = 256 << 20
    a = torch.empty(nbytes, dtype=torch.uint8, device="cuda:0").random_(0, 255)
    b = torch.empty_like(a)
    torch.cuda.synchronize()
    for _ in range(3):
        b.copy_(a)
    torch.cuda.synchronize()
    print(json.dumps({"copy_bytes_per_dispatch": nbytes, "dispatches": 3}), flush=True)


def read_calibration():
    """A reduction that reads 256 MiB and writes a few bytes per dispatch: a
    FETCH_SIZE reading of it gives the counter's scale for a pure read
    stream."""
    import torch
    nbytes = 256 << 20
    a = torch.ones(nbytes // 4, dtype=torch.float32, device="cuda:0")
    torch.cuda.synchronize()
    for _ in range(3):
        s = a.sum()
    torch.cuda.synchronize()
    print(json.dumps({"read_bytes_per_dispatch": nbytes, "dispatches": 3,
                      "sum": float(s.item())}), flush=True)


def kernel_sources_sha256() -> str:
    """Hash of the kernel sources: counter readings taken on other sources are
    not reported."""
    h = hashlib.sha256()
    for f in sorted(glob.glob(os.path.join(ROOT, "mixture_experts_layer_35_amd", "csrc", "*"))):
        with open(f, "rb") as fh:
            h.update(os.path.basename(f).encode())
            h.update(fh.read())
    return h.hexdigest()


def _counter_file(path: str, key: str):
    """(file record, entry) of a committed counter summary, or None when there
    is none for this kernel and workload or the sources changed since."""
    try:
        with open(path) as fh:
            rec = json.load(fh)
    except (OSError, ValueError):
        return None
    if rec.get("sources_sha256") != kernel_sources_sha256():
        return None
    ent = rec.get("entries", {}).get(key)
    return (rec, ent) if ent else None


def traffic_for(key: str):
    """(HBM bytes per launch, algorithmic bytes per launch) of the counter
    run: FETCH_SIZE and WRITE_SIZE scaled by a copy kernel's readings, taken
    on the profiling driver's layer of the same workload, whose routing (and
    so its algorithmic bytes) differs a little from this run's."""
    got = _counter_file(TRAFFIC_FILE, key)
    if got is None:
        return None
    rec, ent = got
    hbm = (ent["fetch_kib"] * rec["fetch_scale"] + ent["write_kib"] * rec["write_scale"]) * 1024.0
    return hbm, ent.get("alg_bytes_per_launch")


def mfma_counters_for(key: str):
    """MFMA busy fraction and executed BF16 MFMA FLOP per launch from the
    committed counter summary (SQ_VALU_MFMA_BUSY_CYCLES over GRBM_GUI_ACTIVE
    of one XCD times the 1024 SIMDs; SQ_INSTS_VALU_MFMA_MOPS_BF16 x 512)."""
    got = _counter_file(MFMA_FILE, key)
    if got is None:
        return None
    _, ent = got
    return {"busy_frac": ent["busy_frac"], "mfma_flop_per_launch": ent["mfma_flop_per_launch"]}


def measure(args, config, n, accum=None, layer=None, cpu_seconds=0.0):
    """Time K calls of one workload (config, n tokens) after W warm-up calls;
    returns the record of that workload (value, per-kernel times, roofline)
    and the layer it built."""
    import numpy as np
    import torch

    import synth
    from mixture_experts_layer_35_amd import Layer, num_launches

    dev = "cuda:0"
    cfg = dict(synth.CONFIGS[config])
    accum = accum or cfg["accum"]
    if layer is None:
        layer = synth.make_layer(config, device=dev)
    by = synth.layer_bytes(layer)

    # rotate weight copies so that the traffic between two uses of a copy is
    # more than twice the Infinity Cache
    per_call_guess = min(cfg["E"], n * cfg["k"]) * by["expert"] + by["shared"]
    copies = max(1, min(32, math.ceil(2 * MALL_BYTES / max(1, per_call_guess)) + 1))
    if args.copies:
        copies = args.copies
    layers = [layer] + [synth.clone_weights(layer) for _ in range(copies - 1)]
    bound = [Layer(l, n, accum=accum, path=args.path) for l in layers]
    xs = [synth.make_tokens(layer, n, 1000 + i) for i in range(args.pool)]
    out = torch.empty_like(xs[0])
    k = cfg["k"]
    idx_all = torch.zeros((args.steps, n, k), dtype=torch.int32, device=dev)

    nl = num_launches(bound[0].cfg, n)
    names = KERNELS[nl]
    stream = torch.cuda.current_stream().cuda_stream

    def mk_events(count):
        evs = []
        for _ in range(count):
            e = ctypes.c_void_p()
            assert H.hipEventCreate(ctypes.byref(e)) == 0
            evs.append(e.value)
        return evs

    ev = None if args.no_trace else [mk_events(2 * nl) for _ in range(args.steps)]

    # the timed calls are plain launches; the same K calls are then replayed
    # with per-kernel events (a launch that records events costs the host more
    # than the decode kernel takes, so the events would throttle the timed loop)
    calls = [bound[(args.warmup + i) % copies].prepare(
        xs[i % args.pool], out, idx=idx_all[i], stream=stream) for i in range(args.steps)]
    traced = None if ev is None else [bound[(args.warmup + i) % copies].prepare(
        xs[i % args.pool], out, stream=stream, events=ev[i]) for i in range(args.steps)]
    warm = [bound[i % copies].prepare(xs[i % args.pool], out, stream=stream)
            for i in range(args.warmup)]
    for c in warm:
        c()
    torch.cuda.synchronize()

    if args.graph:
        # the same K calls captured once and replayed once (a warm-up replay
        # first); the library enqueues only kernel launches
        side = torch.cuda.Stream()
        gcalls = [bound[(args.warmup + i) % copies].prepare(
            xs[i % args.pool], out, idx=idx_all[i], stream=side.cuda_stream)
            for i in range(args.steps)]
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph, stream=side):
            for c in gcalls:
                c()
        graph.replay()
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        graph.replay()
        torch.cuda.synchronize()
        wall = time.perf_counter() - t0
    else:
        t0 = time.perf_counter()
        for c in calls:
            c()
        torch.cuda.synchronize()
        wall = time.perf_counter() - t0
    us_per_call = wall / args.steps * 1e6
    traced_us = None
    if traced is not None:
        t0 = time.perf_counter()
        for c in traced:
            c()
        torch.cuda.synchronize()
        traced_us = (time.perf_counter() - t0) / args.steps * 1e6
    for b in bound:
        err = int(b.workspace[128:132].view(torch.int32).item())
        if err:
            raise RuntimeError(f"device error word {err}: a workgroup wait expired")

    # distinct experts per call -> algorithmic bytes
    idx_np = idx_all.cpu().numpy()
    U = np.array([len(np.unique(idx_np[i])) for i in range(args.steps)])
    sgu = sdn = 0
    if layer["shared"] is not None:
        sh = layer["shared"]
        sgu = synth.projection_bytes(sh["gate"]) + synth.projection_bytes(sh["up"])
        sdn = synth.projection_bytes(sh["down"])
    bytes_gu = U * by["expert_gate_up"] + sgu
    bytes_dn = U * by["expert_down"] + sdn
    expert_bytes = bytes_gu + bytes_dn
    total_bytes = expert_bytes + by["router"]
    Hd, I, Is = cfg["H"], cfg["I"], cfg["I_s"]
    flops_gu = 2.0 * n * k * 2 * Hd * I + 2.0 * n * 2 * Hd * Is
    flops_dn = 2.0 * n * k * Hd * I + 2.0 * n * Hd * Is

    per_kernel = {}
    roof = None
    kernels_us = None
    if ev is not None:
        durs = np.zeros((args.steps, nl), np.float64)
        f = ctypes.c_float()
        for i in range(args.steps):
            for j in range(nl):
                H.hipEventElapsedTime(ctypes.byref(f), ctypes.c_void_p(ev[i][2 * j]),
                                      ctypes.c_void_p(ev[i][2 * j + 1]))
                durs[i, j] = f.value * 1e3  # us
        per_kernel = {names[j]: round(float(durs[:, j].mean()), 3) for j in range(nl)}
        kernels_us = float(durs.sum(axis=1).mean())
        if nl == 1:
            # one fused launch: its algorithmic bytes are the whole call's
            dom, dom_bytes, dom_us = "k_moe_decode", total_bytes, durs[:, 0]
        else:
            dom, dom_bytes, dom_us = "k_g_gate_up", bytes_gu, durs[:, 2]
        achieved = float(dom_bytes.sum() / (dom_us.sum() * 1e-6) / 1e9)
        key = f"{dom}:{config}:N={n}:{accum}"
        traffic = traffic_for(key)
        roof = {"bound": "hbm", "kernel": dom, "achieved": round(achieved, 1),
                "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4),
                "traffic": None if traffic is None else round(traffic[0]),
                "bytes_per_launch": float(dom_bytes.mean()), "avg_launch_us": float(dom_us.mean())}
        if traffic is not None and traffic[1]:
            # the counter run's own algorithmic bytes per launch (its layer
            # routes a little differently), and the ratio of the two
            roof["traffic_alg_bytes"] = traffic[1]
            roof["traffic_over_alg"] = round(traffic[0] / traffic[1], 4)
        if nl > 1:
            gu_tf = flops_gu / (durs[:, 2].mean() * 1e-6) / 1e12
            dn_tf = flops_dn / (durs[:, 3].mean() * 1e-6) / 1e12
            dn_gbs = float(bytes_dn.sum() / (durs[:, 3].sum() * 1e-6) / 1e9)
            roof["mfma"] = {"gate_up_tflops": round(gu_tf, 1), "down_tflops": round(dn_tf, 1),
                            "peak_bf16_tflops": MFMA_BF16_PEAK_TFLOPS,
                            "gate_up_util": round(gu_tf / MFMA_BF16_PEAK_TFLOPS, 4),
                            "down_util": round(dn_tf / MFMA_BF16_PEAK_TFLOPS, 4),
                            "flops_per_call": flops_gu + flops_dn}
            for kn in ("k_g_gate_up", "k_g_down"):
                mc = mfma_counters_for(f"{kn}:{config}:N={n}:{accum}")
                if mc is not None:  # rocprofv3 counter readings (padding rows included)
                    roof["mfma"][f"{kn}_counter_busy_frac"] = mc["busy_frac"]
                    roof["mfma"][f"{kn}_counter_mfma_flop"] = mc["mfma_flop_per_launch"]
            roof["down_gbps"] = round(dn_gbs, 1)
        experts_gbs = float(expert_bytes.sum() / (durs.sum() * 1e-6) / 1e9)
        for row in ev:
            for e in row:
                H.hipEventDestroy(ctypes.c_void_p(e))
    else:
        experts_gbs = None

    cpu = None
    if cpu_seconds > 0:
        cpu = cpu_baseline(layer, xs, n, cpu_seconds)

    path = "decode" if nl == 1 else "grouped"
    rec = {
        "value": round(us_per_call, 3),
        "unit": "us/call",
        "config": {"workload": f"{config} H={cfg['H']} I={cfg['I']} E={cfg['E']} "
                               f"k={k} I_s={cfg['I_s']} {cfg['routed_fmt']} N={n}",
                   "n_tokens": n, "routed_format": cfg["routed_fmt"], "path": path,
                   "accum": accum, "weight_copies": copies, "token_batches": args.pool,
                   "launch": (f"one HIP graph of {args.steps} calls" if args.graph else
                              "eager stream") + f", {nl} launch(es) per call"},
        "expert_weight_gbps_call": round(float(expert_bytes.mean() / (us_per_call * 1e-6) / 1e9), 1),
        "expert_weight_gbps_kernels": None if experts_gbs is None else round(experts_gbs, 1),
        "pct_hbm_peak_kernels": None if experts_gbs is None else round(100 * experts_gbs / HBM_PEAK_GBS, 2),
        "kernels_us_per_call": None if kernels_us is None else round(kernels_us, 3),
        "traced_us_per_call": None if traced_us is None else round(traced_us, 3),
        "distinct_experts_mean": float(U.mean()),
        "bytes_per_call_mean": float(total_bytes.mean()),
        "per_kernel_us": per_kernel,
        "roofline": roof,
        "cpu_baseline": cpu,
    }
    del bound, layers, calls, traced, warm, xs, out, idx_all
    torch.cuda.synchronize()
    return rec, layer


# the other points of the headline metric, measured in the default run
# beside the N = 1 line: (config, tokens)
DEFAULT_POINTS = (("qwen3_30b_a3b_mxfp4", 3), ("deepseek_v3_nvfp4", 4))


def main():
    args = parse()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: the library has no multi-GPU path "
              "(expert parallelism would shard experts across GPUs; moe_forward_ep_partial "
              "computes one GPU's share).",
              file=sys.stderr)
        sys.exit(2)
    if args.copy_calibration:
        copy_calibration()
        return
    if args.read_calibration:
        read_calibration()
        return

    import torch

    global H
    H = hip()
    torch.cuda.set_device(0)
    config = args.config or "qwen3_30b_a3b_mxfp4"
    n = args.n or __import__("synth").CONFIGS[config]["n_list"][0]
    rec, layer = measure(args, config, n, args.accum, cpu_seconds=args.cpu_seconds)
    points = []
    if args.config is None and args.n is None and not args.no_points:
        # the headline metric's other token counts, each timed the same way
        # (K calls after W warm-up calls) with its own roofline
        for pc, pn in DEFAULT_POINTS:
            print(f"[bench] point {pc} N={pn}", file=sys.stderr, flush=True)
            prec, _ = measure(args, pc, pn, None, layer=layer if pc == config else None)
            points.append(prec)
            torch.cuda.empty_cache()
    line = {
        "metric": "MoE layer us/call + expert-weight HBM GB/s (% peak) at N=1,3,4 tokens",
        "value": rec["value"],
        "unit": "us/call",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(rec["value"] / 1e3, 6),
        "higher_is_better": False,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
    }
    line.update({k: v for k, v in rec.items() if k not in ("value", "unit")})
    if points:
        line["points"] = points
    print(json.dumps(line), flush=True)


def host_cores() -> int:
    """CPU threads this process may use: the OpenMP thread budget when one is
    set (a scheduler that gives the process a CPU share sets it), else the affinity
    mask."""
    env = os.environ.get("OMP_NUM_THREADS", "")
    if env.isdigit() and int(env) > 0:
        return int(env)
    return len(os.sched_getaffinity(0))


def cpu_model() -> str:
    try:
        with open("/proc/cpuinfo") as fh:
            for line in fh:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def cpu_baseline(layer, xs, n, budget_s):
    """The FP64 oracle on the host: as many calls of the same workload as fit
    in the budget (at least one), reported per call, with NumPy's BLAS given
    every host thread."""
    import numpy as np
    import torch
    import synth
    from oracle import moe_forward
    from threadpoolctl import threadpool_limits
    npl = synth.as_numpy(layer)
    cores = host_cores()
    times = []
    start = time.perf_counter()
    i = 0
    with threadpool_limits(cores):
        while True:
            xb = xs[i % len(xs)].cpu().view(torch.int16).numpy().view(np.uint16)
            t = time.perf_counter()
            moe_forward(npl["cfg"], npl, xb)
            times.append(time.perf_counter() - t)
            i += 1
            if time.perf_counter() - start > budget_s:
                break
    us = float(np.median(times) * 1e6)
    return {"value": round(us, 1), "unit": "us/call", "cores": cores, "kind": "oracle",
            "cpu_model": cpu_model(),
            "sample": f"{len(times)} full calls of the same workload (N={n}), median; "
                      f"NumPy FP64, BLAS on {cores} threads (the element-wise dequantisation "
                      f"runs on one)"}


if __name__ == "__main__":
    main()
