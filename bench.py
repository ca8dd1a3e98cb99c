"""Benchmark of one GPU's share of the MoE layer, forward + backward.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--config C4]

A step is one forward + backward of the whole layer (router, permute,
grouped FFN, combine and their backward) over one batch of seeded synthetic
input already resident in HBM.  The default workload is the largest one
(c4_large: T=32768, d=4096, E=128, top-8, f=1536).  Prints ONE JSON line
with tokens/s -- the primary value with cold caches (a 512 MiB fill before
each timed step, outside its timing), the back-to-back warm rate beside it
-- the roofline position of the dominant kernel (its launches timed with
HIP events on the stream they run on, inside the timed region) and the CPU
oracle timed on a bounded sample of the same workload.

This build runs on one GPU: --gpus above 1 exits with a message.
"""
from __future__ import annotations

import argparse
import dataclasses
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "MoE layer fwd+bwd tokens/sec on 1 MI355X; % bf16 MFMA peak, % HBM BW"
PEAK_BF16_TFLOPS = 2516.6   # MI355X dense bf16 MFMA
PEAK_FP32_TFLOPS = 157.3    # MI355X fp32 vector
PEAK_HBM_GBS = 8000.0       # MI355X HBM3E
COLD_FLUSH_BYTES = 512 << 20  # twice the MI355X memory-side cache (256 MB)

# CPU-oracle sample sizes (tokens).  Most take 10-30 s on 8-16 cores; the
# c4_large oracle is bound by its 128 experts' weights (about 1 min on 8
# cores whatever the token count), so it gets a small token sample.
CPU_SAMPLE_T = {"tiny_f32": 64, "c1_bf16": 4096, "c2_zipf": 2048, "c3_epshare": 1024,
                "c4_large": 256}


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def parse():
    ap = argparse.ArgumentParser(description="MoE layer fwd+bwd benchmark (1 GPU)")
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--config", default="C4",
                    help="workload: C0..C4 or its name (default C4, the largest)")
    ap.add_argument("--seed", type=int, default=0)
    ap.add_argument("--kernel", default=None,
                    help="kernel timed for the roofline (default: GEMM_DH, dA = (dYp W2^T) "
                         "* gelu'(A), the longest single launch on c4_large)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-cold", action="store_true",
                    help="time warm back-to-back steps only (the primary value is then the "
                         "warm rate)")
    ap.add_argument("--aux-coeff", type=float, default=0.0,
                    help="coefficient of the load-balancing loss (default 0: the bare "
                         "layer); > 0 also computes the loss and drop rate every step")
    ap.add_argument("--renorm", action="store_true",
                    help="gates renormalised over the selected experts")
    ap.add_argument("--priority", choices=("token", "slot"), default="token",
                    help="capacity priority: token-major (default) or slot-major")
    ap.add_argument("--fallback", choices=("none", "identity"), default="none",
                    help="dropped assignments: dropped (default) or the identity fallback")
    ap.add_argument("--graph", action="store_true",
                    help="capture one step into a HIP graph and time K replays of it")
    ap.add_argument("--recompute", action="store_true",
                    help="selective recomputation: A and H are not saved and the "
                         "backward recomputes them (one extra grouped GEMM)")
    ap.add_argument("--copy-probe", type=int, default=0, metavar="BYTES",
                    help="before the warmup, run one plain device-to-device copy of BYTES "
                         "(calibration of the HBM byte counters)")
    ap.add_argument("--summarize-counters", nargs=2, metavar=("FETCH_DIR", "WRITE_DIR"),
                    help="instead of running: read the rocprofv3 --pmc FETCH_SIZE and "
                         "WRITE_SIZE outputs of a run with --copy-probe and print the "
                         "per-launch HBM traffic of --kernel as a JSON line")
    return ap.parse_args()


# name fragments of each timed kernel in a rocprofv3 trace (template
# arguments: mode, K-contiguous B, epilogue): the eight-wave kernel that runs
# the 256 x 256 row tiles, or the four-wave one for the other tile sizes
KERNEL_NAMES = {"GEMM_UP": ("gemm_pp_kernel<0, false, 1>", "gemm_bf16_kernel<0, false, 1,"),
                "GEMM_DOWN": ("gemm_pp_kernel<0, false, 0>", "gemm_bf16_kernel<0, false, 0,"),
                "GEMM_DH": ("gemm_pp_kernel<0, true, 2>", "gemm_bf16_kernel<0, true, 2,"),
                "GEMM_DX": ("gemm_pp_kernel<0, true, 0>", "gemm_bf16_kernel<0, true, 0,")}
GEMM_SOURCES = ("expert_router_gemm_softmax_amd/csrc/gemm.hip",
                "expert_router_gemm_softmax_amd/csrc/gemm.h",
                "expert_router_gemm_softmax_amd/csrc/common.h")
COUNTERS_GLOB = "profiles/*_hbm_counters.md"


def gemm_source_hash():
    import hashlib
    h = hashlib.sha256()
    for f in GEMM_SOURCES:
        with open(os.path.join(ROOT, f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def summarize_counters(a, w):
    """Per-launch HBM bytes of --kernel from FETCH_SIZE / WRITE_SIZE (KiB per
    dispatch), each scaled by bytes-copied / counter of the --copy-probe copy
    (the largest device copy dispatch in the same run)."""
    import csv
    import glob

    def per_dispatch(d, counter):
        vals = {}
        for f in glob.glob(os.path.join(d, "**", "*counter_collection.csv"), recursive=True):
            for r in csv.DictReader(open(f)):
                if r["Counter_Name"] != counter:
                    continue
                key = (r["Dispatch_Id"], r["Kernel_Name"])
                vals[key] = vals.get(key, 0.0) + float(r["Counter_Value"])
        return vals

    frags = KERNEL_NAMES[a.kernel or "GEMM_DH"]
    out = {"kernel": a.kernel or "GEMM_DH", "workload": w.name,
           "gemm_source_sha256_16": gemm_source_hash(), "copy_probe_bytes": a.copy_probe}
    total = 0.0
    for d, counter in zip(a.summarize_counters, ("FETCH_SIZE", "WRITE_SIZE")):
        vals = per_dispatch(d, counter)
        copies = [v for (i, n), v in vals.items() if "copyBuffer" in n]
        ks = [v for (i, n), v in vals.items() if any(f in n for f in frags)]
        if not copies or not ks:
            raise SystemExit(f"{counter}: copy probe or kernel not found in {d}")
        factor = a.copy_probe / (max(copies) * 1024.0)
        kib = sum(ks) / len(ks)
        key = counter.lower()
        out[f"{key}_kib_per_launch"] = round(kib, 1)
        out[f"{key}_copy_kib"] = round(max(copies), 1)
        out[f"{key}_factor"] = round(factor, 4)
        out[f"{key}_launches"] = len(ks)
        total += kib * 1024.0 * factor
    out["traffic_bytes_per_launch"] = round(total)
    print(json.dumps(out))
    return 0


def recorded_traffic(kernel, workload):
    """HBM bytes per launch recorded under profiles/ for this kernel and
    workload, or None when there is none or the GEMM source has changed."""
    import glob
    want = gemm_source_hash()
    for f in sorted(glob.glob(os.path.join(ROOT, COUNTERS_GLOB))):
        for line in open(f):
            line = line.strip()
            if not line.startswith("{"):
                continue
            try:
                rec = json.loads(line)
            except ValueError:
                continue
            if (rec.get("kernel") == kernel and rec.get("workload") == workload
                    and rec.get("gemm_source_sha256_16") == want):
                return rec.get("traffic_bytes_per_launch")
    return None


def dev(a):
    import numpy as np
    import torch
    if a.dtype == np.uint16:
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).cuda().view(
            torch.bfloat16)
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


def cpu_baseline(w, seed, inp_full=None):
    """The oracle, as it stands, on the first T' tokens of the workload: the
    same weights and the first T' rows of x and dOut of the inputs the GPU
    ran (an expert-share workload draws its ragged batch for T' rows)."""
    import oracle as O
    import workloads as W
    Ts = min(w.T, CPU_SAMPLE_T.get(w.name, 1024))
    ws = w.replace(T=Ts)
    if w.kind == "layer" and inp_full is not None:
        inp = dict(inp_full)
        inp["x"] = inp_full["x"][:Ts]
        inp["dOut"] = inp_full["dOut"][:Ts]
    else:
        inp = W.make_inputs(ws, seed=seed)
    threads = None
    try:
        import threadpoolctl
        info = threadpoolctl.threadpool_info()
        threads = max((i.get("num_threads") or 0) for i in info) if info else None
    except Exception:
        pass
    t0 = time.perf_counter()
    fw = O.layer_fwd(inp, ws)
    O.layer_bwd(inp, ws, fw)
    dt = time.perf_counter() - t0
    unit = "rows/s" if w.kind == "ep_share" else "tokens/s"
    cap = "" if ws.cf is None else f", capacity C'={O.capacity(Ts, w.k, w.E, w.cf)} from cf={w.cf}"
    return {"value": Ts / dt, "unit": unit, "cores": threads or os.cpu_count(),
            "kind": "oracle",
            "sample": f"oracle fwd+bwd of the same layer (same weights) on the first {Ts} of "
                      f"{w.T} tokens (seed {seed}{cap}), one run, {dt:.1f} s; host has "
                      f"{os.cpu_count()} logical CPUs"}


def main():
    a = parse()
    if a.gpus != 1:
        print(f"bench.py: the library runs one GPU's share of the MoE layer; --gpus {a.gpus} "
              "is not supported (multi-GPU sharding is a design note only).",
              file=sys.stderr)
        return 2
    import numpy as np
    import torch

    import workloads as W
    w = W.get(a.config)
    if a.aux_coeff or a.renorm or a.priority != "token" or a.fallback != "none":
        w = dataclasses.replace(w, aux_coeff=a.aux_coeff, renorm=a.renorm, priority=a.priority,
                                fallback=a.fallback)
    if a.summarize_counters:
        return summarize_counters(a, w)
    import expert_router_gemm_softmax_amd as M

    torch.cuda.set_device(0)
    log(f"[bench] workload {w.name}: T={w.T} d={w.d} E={w.E} k={w.k} f={w.f} {w.dtype} "
        f"cf={w.cf}")
    inp = W.make_inputs(w, seed=a.seed)
    d = {k: dev(v) for k, v in inp.items()}
    if w.cf is None:
        cap = None
    else:
        cap = M.moe_capacity(w.T, w.k, w.E, w.cf)
    cfg = M.make_cfg(w.T, w.d, w.E, w.k, w.f, w.dtype, capacity=cap,
                     aux_coeff=a.aux_coeff, recompute=a.recompute, renorm=a.renorm,
                     priority=a.priority, fallback=a.fallback)
    sdt = torch.bfloat16 if w.dtype == "bf16" else torch.float32

    if w.kind == "layer":
        layer = M.MoeLayer(cfg, d["Wr"], d["b"], d["W1"], d["W2"])
        out = torch.empty(w.T, w.d, dtype=sdt, device="cuda")
        dX = torch.empty_like(out)
        grads = layer.alloc_grads()

        def step():
            layer.forward(d["x"], out)
            layer.backward(d["x"], d["dOut"], dX, grads)

        offsets = layer.saved["offsets"]
    else:
        # one EP rank's share: the batch arrives already permuted
        Rmax = M.moe_rows_max(cfg)
        ws = torch.empty(M.moe_workspace_bytes(cfg), dtype=torch.uint8, device="cuda")
        e = lambda *s, dt=sdt: torch.empty(*s, dtype=dt, device="cuda")
        A, H, Y = e(Rmax, w.f), e(Rmax, w.f), e(Rmax, w.d)
        if a.recompute:
            A = H = None
        out, dYp, dXp = e(w.T, w.d), e(Rmax, w.d), e(Rmax, w.d)
        dg = e(w.T, 1, dt=torch.float32)
        dW1, dW2 = torch.empty_like(d["W1"]), torch.empty_like(d["W2"])
        offsets = d["offsets"]

        def step():
            M.moe_grouped_ffn(cfg, d["x_perm"], offsets, d["W1"], d["W2"], A, H, Y, ws)
            M.moe_combine(cfg, Y, d["row_of"], d["gate"], out)
            M.moe_combine_bwd(cfg, d["dOut"], Y, d["row_of"], d["gate"], dYp, dg)
            M.moe_grouped_ffn_bwd(cfg, d["x_perm"], offsets, d["W1"], d["W2"], A, H, dYp,
                                  dXp, dW1, dW2, ws)

    if a.copy_probe:
        src = torch.empty(a.copy_probe, dtype=torch.uint8, device="cuda")
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst
    for i in range(a.warmup):
        step()
    torch.cuda.synchronize()
    R = int(offsets[-1].item())
    log(f"[bench] warmup done, R={R} kept rows of {w.T * w.k}")

    run = step
    if a.graph:
        # one capture on a side stream (a warm-up there first), then replays
        side = torch.cuda.Stream()
        side.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(side):
            step()
        torch.cuda.current_stream().wait_stream(side)
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph, stream=side):
            step()
        torch.cuda.synchronize()
        run = graph.replay

    # warm: K steps back to back
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(a.steps):
        run()
    torch.cuda.synchronize()
    warm_wall = time.perf_counter() - t0
    log(f"[bench] warm: {a.steps} steps back to back, {warm_wall * 1e3 / a.steps:.4f} ms/step")

    # The timed region of the primary value: K steps, each with cold caches
    # (a 512 MiB fill, twice the 256 MB memory-side cache, evicts the step's
    # data first) and bracketed by its own synchronisations; the fill is
    # outside the timing.  The probe records the roofline kernel's launches
    # inside these steps, on the stream they run on.  (Graph replays record
    # no probe events: the kernel is then timed on as many eager steps.)
    kernel = a.kernel or "GEMM_DH"
    probe = M.KernelProbe(kernel, a.steps)
    if not a.graph:
        probe.attach(cfg)
    flush = None if a.no_cold else torch.empty(COLD_FLUSH_BYTES, dtype=torch.uint8,
                                               device="cuda")
    step_s = []
    for i in range(a.steps):
        if flush is not None:
            flush.fill_(i & 0xFF)
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        run()
        torch.cuda.synchronize()
        step_s.append(time.perf_counter() - t0)
    wall = sum(step_s)
    if a.graph:
        probe.attach(cfg)
        for i in range(a.steps):
            step()
        torch.cuda.synchronize()
    probe.detach(cfg)
    k_ms, k_n, k_each = probe.read()
    probe.close()
    del flush
    ms_per_step = wall * 1e3 / a.steps
    log(f"[bench] {'cold' if not a.no_cold else 'warm'}: {a.steps} steps, "
        f"{ms_per_step:.4f} ms/step; {kernel}: {k_n} launches, "
        f"{k_ms / max(k_n, 1):.4f} ms avg")

    # algorithmic work of the timed kernel per launch: 2 R d f flop per expert
    # GEMM; bytes the method must move for the gathers
    flops = {"GEMM_UP": 2.0 * R * w.d * w.f, "GEMM_DOWN": 2.0 * R * w.d * w.f,
             "GEMM_DH": 2.0 * R * w.d * w.f, "GEMM_DX": 2.0 * R * w.d * w.f,
             "GEMM_DW1": 2.0 * R * w.d * w.f, "GEMM_DW2": 2.0 * R * w.d * w.f,
             "GEMM_RECOMPUTE": 2.0 * R * w.d * w.f}
    s_b = 2 if w.dtype == "bf16" else 4
    Tk = w.T * w.k
    hbm_bytes = {"COMBINE": R * w.d * s_b + w.T * w.d * s_b + 8 * Tk,
                 "COMBINE_BWD": w.T * w.d * s_b + 2 * R * w.d * s_b + 12 * Tk,
                 # every token's row read once, each kept copy written
                 "PERMUTE_COPY": (w.T + R) * w.d * s_b + 4 * Tk,
                 "ROUTE_AUX": 4 * w.T * w.E + 8 * w.E + 4}
    avg_s = (k_ms / 1e3) / max(k_n, 1)
    if kernel in hbm_bytes and avg_s > 0:
        achieved = hbm_bytes[kernel] / avg_s / 1e9
        roof = {"bound": "hbm", "achieved": round(achieved, 1), "peak": PEAK_HBM_GBS,
                "unit": "GB/s", "frac": round(achieved / PEAK_HBM_GBS, 4), "traffic": None,
                "kernel": kernel, "avg_ms": round(avg_s * 1e3, 5),
                "algorithmic_bytes": hbm_bytes[kernel]}
    elif kernel in flops:
        peak = PEAK_BF16_TFLOPS if w.dtype == "bf16" else PEAK_FP32_TFLOPS
        achieved = flops[kernel] / avg_s / 1e12 if avg_s > 0 else 0.0
        roof = {"bound": "mfma", "achieved": round(achieved, 2), "peak": peak,
                "unit": "TFLOP/s", "frac": round(achieved / peak, 4),
                "traffic": recorded_traffic(kernel, w.name),
                "kernel": kernel, "avg_ms": round(avg_s * 1e3, 5),
                "algorithmic_flop": flops[kernel]}
    else:
        roof = {"bound": "hbm", "achieved": None, "peak": PEAK_HBM_GBS, "unit": "GB/s",
                "frac": None, "traffic": None, "kernel": kernel,
                "avg_ms": round(avg_s * 1e3, 5)}

    unit = "rows/s" if w.kind == "ep_share" else "tokens/s"
    value = w.T * a.steps / wall
    line = {
        "metric": METRIC,
        "value": round(value, 1), "unit": unit, "n_gpus": 1, "steps": a.steps,
        "warmup": a.warmup, "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": w.dtype, "data": "synthetic (seeded; random-init weights)",
        "config": {"workload": f"{w.name}: T={w.T} d={w.d} E={w.E} k={w.k} f={w.f} "
                               f"cf={w.cf} bias={w.bias}",
                   "tokens": w.T, "d": w.d, "experts": w.E, "top_k": w.k, "ffn": w.f,
                   "capacity": cap, "kept_rows": R, "parallelism": "single GPU",
                   "caches": "warm" if a.no_cold else
                             "cold (512 MiB fill before each timed step, outside its timing)",
                   "aux_coeff": a.aux_coeff, "recompute": a.recompute,
                   "renorm": a.renorm, "priority": a.priority, "fallback": a.fallback,
                   "graph_replay": a.graph},
        "roofline": roof,
        "warm": {"value": round(w.T * a.steps / warm_wall, 1),
                 "ms_per_step": round(warm_wall * 1e3 / a.steps, 4),
                 "note": "the same K steps back to back, one synchronisation each side"},
    }
    if not a.no_cpu_baseline:
        log("[bench] timing the CPU oracle on a bounded sample ...")
        line["cpu_baseline"] = cpu_baseline(w, a.seed, inp)
    print(json.dumps(line), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
