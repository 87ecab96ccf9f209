#!/usr/bin/env python3
"""Benchmark of the RankMixerBlock forward+backward on one MI355X.

One step = rm_block_fwd + rm_block_bwd over one batch of synthetic input
(every step of the block, both directions, all 15 gradient tensors).
Default workload: B=1024, T=64, D=1280, k=2 (H=2560), bf16 storage, fp32
accumulation, inputs resident in HBM before timing starts.

Printed as the last stdout line: one JSON object with
  value        tokens/s (B*T per step / seconds per step) over K timed steps
  roofline     the kernel with the largest share of step time, its algorithmic
               flops (or bytes) per launch / its mean launch time from HIP
               events recorded on the library's stream during a timed pass
  cpu_baseline the float64 oracle on a bounded sample, on the host's cores
Also reported: the pages' timing protocol (flush, sync, event span per
iteration, first sample dropped, mean/min/max in us), per-kernel times, % of
MFMA peak for the whole step, peak device memory.

Workload and protocol follow "Subgraph-fusion-based Mega-kernel Generation"
(page 1): "Workload and interfaces", "Run the benchmark" (WARMUP=5,
NUM_TESTS=20) and "Exact timing behavior".
"""
from __future__ import annotations

import argparse
import json
import os
import subprocess
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

from rankmixer_inputs import PRODUCTION, WORKLOADS, make_case  # noqa: E402

# MI355X published peaks
PEAK_TFLOPS = {"bf16": 2516.6, "f16": 2516.6, "f32": 157.3}   # dense MFMA: 256 CU x 2.4 GHz x (4096 | 256) flop/clk
PEAK_HBM_GBS = 8000.0
PEAK_VALU_F32 = 157.3   # TFLOP/s, fp32 vector FMA: the small-batch kernels' contractions run on the VALU


def log(msg):
    print(msg, file=sys.stderr, flush=True)


def gemm_flops(d):
    """Algorithmic flops of each GEMM launch (one launch covers all T tokens)."""
    B, T, D, H = d.B, d.T, d.D, d.k * d.D
    return {"gemm_up": 2.0 * B * T * D * 2 * H, "gemm_down": 2.0 * B * T * H * D,
            "gemm_dhid": 2.0 * B * T * D * H, "gemm_dwout": 2.0 * T * H * D * B,
            "gemm_dw1": 2.0 * T * D * 2 * H * B, "gemm_dh1": 2.0 * B * T * 2 * H * D}


def small_flops(d):
    """Algorithmic flops of the small-batch kernels (B <= 8), whose per-token contractions are fp32
    VALU FMA loops: the forward's two products, the backward's four; the last kernel has none."""
    B, T, D, H = d.B, d.T, d.D, d.k * d.D
    f = 2.0 * B * T * D * 2 * H + 2.0 * B * T * H * D
    return {"small_fwd": f, "small_bwd": 2.0 * f}


def rows_per_group(B, T):
    """Samples per group of the backward's parameter-gradient partials (the library's row groups):
    128, halved down to 16 while T * ceil(B / rows) < 512 workgroups."""
    r = 128
    while r > 16 and T * -(-B // r) < 512:
        r //= 2
    return r


def tail_per_sample(d, sz):
    """The backward tail runs one sample per workgroup in LDS (16-bit samples of at most 160 KB with
    16-byte rows and 4-element token-mix chunks) and writes per-sample partials."""
    return sz == 2 and d.D % 8 == 0 and (d.D // d.T) % 4 == 0 and d.T * d.D * 2 <= 64 * 1280 * 2


def row_bytes(d, sz):
    """Algorithmic HBM bytes of each row-kernel launch: its inputs read once, outputs written once."""
    B, T, D, H = d.B, d.T, d.D, d.k * d.D
    N = B * T
    nb = -(-B // rows_per_group(B, T))
    p_ln2, p_gate = 3 * nb * T * D * 4, (4 * nb * T * H + nb * T * 2 * H) * 4
    p_tail = 4 * (B if tail_per_sample(d, sz) else nb * T) * D * 4
    return {
        "prologue": N * D * sz * 2 + N * 16,                              # x -> out1, 4 stats
        "gate_fwd": N * 2 * H * sz + N * H * sz + N * 16,                 # Z -> hidden, 4 stats
        "ln2_fwd": 2 * N * D * sz + N * 8,                                # r2 -> y
        "ln2_bwd": 3 * N * D * sz + p_ln2,                                # r2, dy -> d(out2), partials
        "gate_bwd": N * 2 * H * sz + N * H * sz + N * 2 * H * sz + p_gate,  # Z, dhid -> dZ, partials
        "ln1_bwd": 3 * N * D * sz + p_tail // 2,                          # x, d(out1) -> dr1, partials
        "ln0_bwd": 3 * N * D * sz + p_tail // 2,                          # x, dr1 -> dx, partials
        "tail_bwd": 3 * N * D * sz + 4 * B * D * 4,                       # x, d(out1) -> dx, per-sample partials
        "finalize": p_ln2 + p_gate + p_tail,                              # partials -> 14 small gradients
    }


def unfused_elementwise_bytes(d, sz):
    """HBM bytes of the block's norm / elementwise work done one eager operator at a time: every
    operator reads its inputs once and writes its output once (GEMM operand and result traffic
    excluded).  U_D, U_H = one [B,T,D] / [B,T,H] tensor in the storage dtype.
      forward:  norm0 2 U_D, token-mix copy 2, residual add 3, norm1 2, +bout 2, residual add 3,
                norm2 2 (16 U_D); +b1 on Z 4 U_H, LN_x 2, LN_gate 2, silu 2, gating product 3 (13 U_H)
      backward: norm2 bwd with its affine sums 5 U_D, dbout 1, residual add of dh1 3, norm1 bwd 5,
                inverse token mix 2, norm0 bwd 5, dx = dr1 + dx0 3 (24 U_D); gating product bwd
                5 U_H, silu bwd 3, LN_x bwd 5, LN_gate bwd 5, concatenating dZ 4, db1 2 (24 U_H)"""
    N = d.B * d.T
    u_d, u_h = N * d.D * sz, N * d.k * d.D * sz
    return 40 * u_d + 37 * u_h


def fused_elementwise_bytes(d, sz, row_kernels):
    """The same work in this library: the row kernels' algorithmic bytes (row_bytes) plus what the
    GEMM epilogues read for it (the two residuals and the two biases)."""
    rb = row_bytes(d, sz)
    N = d.B * d.T
    epi = 2 * N * d.D * sz + d.T * (2 * d.k * d.D + d.D) * sz
    return sum(rb[k] for k in row_kernels) + epi


def step_flops(d):
    return 18.0 * d.B * d.T * d.D * d.k * d.D


def host_cpu():
    """CPU model and physical core count of the host, as /proc/cpuinfo states them."""
    model, cores = "unknown", set()
    phys = core = None
    try:
        for line in open("/proc/cpuinfo"):
            k, _, v = line.partition(":")
            k, v = k.strip(), v.strip()
            if k == "model name" and model == "unknown":
                model = v
            elif k == "physical id":
                phys = v
            elif k == "core id":
                core = v
            elif not k and phys is not None and core is not None:
                cores.add((phys, core))
                phys = core = None
        if phys is not None and core is not None:
            cores.add((phys, core))
    except OSError:
        pass
    return model, len(cores) or None


def cpu_baseline(name, batch, min_seconds):
    """The float64 oracle (unchanged) on the first `batch` samples of the workload."""
    import oracle
    from rankmixer_inputs import as_f64
    try:
        from threadpoolctl import threadpool_info
        cores = max([int(i.get("num_threads", 1)) for i in threadpool_info()] or [1])
    except Exception:
        cores = os.cpu_count() or 1
    case = make_case(name, batch=batch)
    x, p, dy = as_f64(case)
    d = case["dims"]
    oracle.forward_backward(x, p, dy)   # untimed warm run
    reps, t0 = 0, time.perf_counter()
    while True:
        oracle.forward_backward(x, p, dy)
        reps += 1
        el = time.perf_counter() - t0
        if el >= min_seconds:
            break
    tokens = reps * d.B * d.T
    model, physical = host_cpu()
    return {"value": tokens / el, "unit": "tokens/s", "cores": cores, "kind": "oracle",
            "cpu_model": model, "physical_cores": physical, "threads_available": len(os.sched_getaffinity(0)),
            "sample": f"first {batch} of {WORKLOADS[name].dims.B} samples of {name} "
                      f"(all parameters), float64 fwd+bwd x{reps} in {el:.1f} s"}


def library_gemms(d, dtype, reps=10):
    """The block's six per-token GEMM shapes through torch.bmm (hipBLASLt on this stack), for
    comparison with the library's kernels: every operand a dense contiguous [T, rows, cols]
    tensor (no transposed views), so the strides differ from the library's [B, T, .] operands."""
    import torch
    B, T, D, H = d.B, d.T, d.D, d.k * d.D
    tdt = {"bf16": torch.bfloat16, "f16": torch.float16, "f32": torch.float32}[dtype]
    shapes = {"gemm_up": (B, D, 2 * H), "gemm_down": (B, H, D), "gemm_dhid": (B, D, H),
              "gemm_dwout": (H, B, D), "gemm_dw1": (D, B, 2 * H), "gemm_dh1": (B, 2 * H, D)}
    out = {}
    for name, (m, k, n) in shapes.items():
        a = torch.randn(T, m, k, device="cuda").to(tdt).contiguous()
        b = torch.randn(T, k, n, device="cuda").to(tdt).contiguous()
        c = torch.empty(T, m, n, device="cuda", dtype=tdt)
        for _ in range(3):
            torch.bmm(a, b, out=c)
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(reps):
            torch.bmm(a, b, out=c)
        e1.record()
        torch.cuda.synchronize()
        ms = e0.elapsed_time(e1) / reps
        out[name] = {"avg_ms": round(ms, 5), "tflops": round(2.0 * T * m * k * n / (ms / 1e3) / 1e12, 2)}
        log(f"  torch.bmm {name} [{T} x {m}x{k} @ {k}x{n}]: {ms:.4f} ms, {out[name]['tflops']} TFLOP/s")
        del a, b, c
    torch.cuda.empty_cache()
    return out


def power_sampler(path, max_seconds=900.0):
    """Child process: socket power (W) and gfx clock (MHz) of GPU 0 every 20 ms into a csv, until
    terminated (or max_seconds).  Reads the SMI counters only; never touches HIP."""
    import amdsmi
    amdsmi.amdsmi_init()
    h = amdsmi.amdsmi_get_processor_handles()[0]
    t_end = time.time() + max_seconds
    with open(path, "w") as f:
        cap = amdsmi.amdsmi_get_power_cap_info(h).get("power_cap")
        f.write(f"# power_cap_uw {cap}\n")
        while time.time() < t_end:
            p = amdsmi.amdsmi_get_power_info(h).get("current_socket_power")
            c = amdsmi.amdsmi_get_clock_info(h, amdsmi.AmdSmiClkType.GFX).get("clk")
            f.write(f"{time.time():.3f},{p},{c}\n")
            f.flush()
            time.sleep(0.02)


def power_summary(path, t0, t1):
    """Mean / max socket power and mean gfx clock over the samples taken in [t0, t1]."""
    cap, pw, ck = None, [], []
    for line in open(path):
        if line.startswith("# power_cap_uw"):
            v = line.split()[-1]
            cap = float(v) / 1e6 if v.replace(".", "").isdigit() else None
            continue
        t, p, c = line.strip().split(",")
        if t0 <= float(t) <= t1:
            if p.replace(".", "").isdigit():
                pw.append(float(p))
            if c.replace(".", "").isdigit():
                ck.append(float(c))
    if not pw:
        return {"error": "no power samples in the timed region"}
    return {"avg_w": round(sum(pw) / len(pw), 1), "max_w": max(pw), "cap_w": cap,
            "gfx_mhz_avg": round(sum(ck) / len(ck), 1) if ck else None, "samples": len(pw),
            "window": "timed region"}


def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default=PRODUCTION, choices=sorted(WORKLOADS))
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-batch", type=int, default=8)
    ap.add_argument("--cpu-seconds", type=float, default=10.0)
    ap.add_argument("--no-protocol", action="store_true", help="skip the per-iteration flush protocol pass")
    ap.add_argument("--no-kernel-times", action="store_true", help="skip the event-instrumented pass")
    ap.add_argument("--graph", action="store_true",
                    help="also time the step replayed from one captured HIP graph (launch-bound small shapes)")
    ap.add_argument("--kernels", choices=["auto", "main"], default="auto",
                    help="auto: B<=8, D<=128, H<=256 shapes take the small-batch kernels (3 launches per step); "
                         "main: every shape takes the main kernel set")
    ap.add_argument("--library-gemms", action="store_true",
                    help="also time the six GEMM shapes through torch.bmm (hipBLASLt) for comparison")
    ap.add_argument("--power-log", default=None, metavar="CSV",
                    help="sample socket power and gfx clock (child process, SMI counters) into CSV and report "
                         "their means over the timed region")
    ap.add_argument("--zero-operands", action="store_true",
                    help="zero x, dy, w1, b1, wout and bout before timing: the same kernels and schedule on "
                         "operands that barely toggle (a power-dependence measurement, not a throughput claim)")
    ap.add_argument("--copy-calibration-mib", type=int, default=0,
                    help="run one plain device-to-device copy of this many MiB first (reference for HBM counters)")
    args = ap.parse_args()

    if args.gpus != 1:
        print(f"bench.py: this build runs on one GPU only (asked for --gpus {args.gpus}); "
              "multi-GPU sharding is not built", file=sys.stderr)
        sys.exit(2)

    sampler = None
    if args.power_log:
        sampler = subprocess.Popen([sys.executable, os.path.abspath(__file__), "--power-sampler", args.power_log])

    import torch
    import transformer_block_norm0_amd as rb
    if not torch.cuda.is_available():
        print("bench.py: no GPU visible", file=sys.stderr)
        sys.exit(1)
    rb.library()

    w = WORKLOADS[args.workload]
    d = w.dims
    log(f"generating {w.name} (seed {w.seed})")
    case = make_case(w)
    sys.path.insert(0, os.path.join(ROOT, "tests"))
    from rm_gpu import DeviceCase  # noqa: E402  (moves the case to the device, calls the C ABI)
    dc = DeviceCase(case, kernels=args.kernels)
    del case
    if args.zero_operands:
        for t in (dc.x, dc.dy, dc.params["w1"], dc.params["b1"], dc.params["wout"], dc.params["bout"]):
            t.zero_()
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream()
    if args.copy_calibration_mib:
        n = args.copy_calibration_mib * 1024 * 1024 // 4
        src = torch.ones(n, dtype=torch.float32, device="cuda")
        dst = torch.empty_like(src)
        evict = torch.empty(1024 * 1024 * 1024 // 4, dtype=torch.float32, device="cuda")
        evict.fill_(0.0)   # 1 GiB written after src: src is no longer cache-resident when copied
        torch.cuda.synchronize()
        del evict
        dst.copy_(src)
        torch.cuda.synchronize()
        log(f"calibration copy: {args.copy_calibration_mib} MiB read + {args.copy_calibration_mib} MiB written")
        del src, dst

    def step():
        dc.fwd(stream)
        dc.bwd(stream)

    # warmup (untimed), then exactly K timed steps bracketed by synchronisation
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    torch.cuda.reset_peak_memory_stats()
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    h0 = time.perf_counter()
    wall0 = time.time()
    ev0.record(stream)
    for _ in range(args.steps):
        step()
    ev1.record(stream)
    torch.cuda.synchronize()
    host_s = time.perf_counter() - h0
    wall1 = time.time()
    ms_total = ev0.elapsed_time(ev1)
    ms_step = ms_total / args.steps
    peak_mem = torch.cuda.max_memory_allocated()
    tokens = d.B * d.T
    value = tokens / (ms_step / 1e3)
    tflops = step_flops(d) / (ms_step / 1e3) / 1e12
    pct_peak = 100.0 * tflops / PEAK_TFLOPS[w.dtype]
    log(f"B={d.B} T={d.T} D={d.D} k={d.k} H={d.H} T_local={d.T} a2a_bytes=0 mode=fwd+bwd")
    log(f"{args.steps} steps: {ms_step:.3f} ms/step (host {1e3 * host_s / args.steps:.3f}), "
        f"{value:.4g} tokens/s, {tflops:.1f} TFLOP/s = {pct_peak:.1f}% of {w.dtype} MFMA peak")

    # the same step captured once into a HIP graph and replayed (no per-launch host work)
    graph = None
    if args.graph:
        side = torch.cuda.Stream()
        side.wait_stream(stream)
        with torch.cuda.stream(side):
            step_on = lambda: (dc.fwd(side), dc.bwd(side))  # noqa: E731
            step_on()
        side.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g, stream=side):
            dc.fwd(side)
            dc.bwd(side)
        for _ in range(args.warmup):
            g.replay()
        torch.cuda.synchronize()
        gs = torch.cuda.current_stream()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(gs)
        for _ in range(args.steps):
            g.replay()
        e1.record(gs)
        torch.cuda.synchronize()
        g_ms = e0.elapsed_time(e1) / args.steps
        graph = {"ms_per_step": round(g_ms, 4), "tokens_per_s": round(tokens / (g_ms / 1e3), 1),
                 "eager_ms_per_step": round(ms_step, 4)}
        log(f"graph replay: {g_ms:.4f} ms/step ({tokens / (g_ms / 1e3):.4g} tokens/s) vs eager {ms_step:.4f}")
        del g

    # per-kernel HIP events (library instrumentation) over a second timed pass
    kernels = {}
    roofline = None
    if not args.no_kernel_times:
        rb.prof_enable(True)
        torch.cuda.synchronize()
        for _ in range(args.steps):
            step()
        torch.cuda.synchronize()
        rb.prof_enable(False)
        prof = rb.prof_collect()
        flops = gemm_flops(d)
        sflops = small_flops(d)
        sz = 4 if w.dtype == "f32" else 2
        rbytes = row_bytes(d, sz)
        step_ms_sum = 0.0
        for name, (ms, n) in prof.items():
            if n == 0:
                continue
            avg = ms / n
            step_ms_sum += ms / args.steps
            ent = {"avg_ms": round(avg, 5), "launches": n}
            if name in flops:
                ent["tflops"] = round(flops[name] / (avg / 1e3) / 1e12, 2)
                ent["frac_peak"] = round(ent["tflops"] / PEAK_TFLOPS[w.dtype], 4)
            elif name in sflops:
                ent["tflops"] = round(sflops[name] / (avg / 1e3) / 1e12, 4)
                ent["frac_peak"] = round(ent["tflops"] / PEAK_VALU_F32, 6)
            elif name in rbytes:
                ent["gbs"] = round(rbytes[name] / (avg / 1e3) / 1e9, 1)
                ent["frac_peak"] = round(ent["gbs"] / PEAK_HBM_GBS, 4)
            kernels[name] = ent
        for name, ent in sorted(kernels.items(), key=lambda kv: -kv[1]["avg_ms"]):
            log(f"  {name:12s} {ent['avg_ms'] * 1e3:9.1f} us  " +
                (f"{ent['tflops']:8.1f} TFLOP/s" if "tflops" in ent else f"{ent.get('gbs', 0):8.1f} GB/s"))
        log(f"  sum of kernel means {step_ms_sum:.3f} ms/step (instrumented)")
        dom = max(kernels.items(), key=lambda kv: kv[1]["avg_ms"])
        name, ent = dom
        if name in sflops:
            roofline = {"kernel": name, "bound": "alu", "achieved": ent["tflops"], "peak": PEAK_VALU_F32,
                        "unit": "TFLOP/s", "frac": ent["frac_peak"], "traffic": None, "avg_ms": ent["avg_ms"],
                        "per_launch": f"{sflops[name]:.4g} flop"}
        elif "tflops" in ent:
            roofline = {"kernel": name, "bound": "mfma", "achieved": ent["tflops"], "peak": PEAK_TFLOPS[w.dtype],
                        "unit": "TFLOP/s", "frac": round(ent["tflops"] / PEAK_TFLOPS[w.dtype], 4),
                        "traffic": None, "avg_ms": ent["avg_ms"],
                        "per_launch": f"{flops[name]:.4g} flop"}
        else:
            roofline = {"kernel": name, "bound": "hbm", "achieved": ent["gbs"], "peak": PEAK_HBM_GBS,
                        "unit": "GB/s", "frac": round(ent["gbs"] / PEAK_HBM_GBS, 4), "traffic": None,
                        "avg_ms": ent["avg_ms"], "per_launch": f"{rbytes[name]:.4g} B"}
        traffic = load_traffic(name, w.name)
        if traffic is not None:
            roofline["traffic"] = traffic

    # bytes of the norm / elementwise work: unfused count vs this library (algorithmic and measured);
    # not reported for the small-batch kernels, which hold a token's rows on chip
    sz = 4 if w.dtype == "f32" else 2
    small_run = any(k.startswith("small_") for k in kernels)
    rk = [k for k in kernels if k in row_bytes(d, sz)] or (
        ["prologue", "gate_fwd", "ln2_fwd", "ln2_bwd", "gate_bwd", "tail_bwd", "finalize"])
    unf = unfused_elementwise_bytes(d, sz)
    fus = fused_elementwise_bytes(d, sz, rk)
    meas = [load_traffic(k, w.name) for k in rk]
    elementwise = {"unfused_bytes_per_step": int(unf), "fused_bytes_per_step": int(fus),
                   "fused_row_kernels_measured_bytes": (int(sum(meas)) if meas and None not in meas else None),
                   "unfused_over_fused": round(unf / fus, 2), "row_kernels": rk}
    log(f"elementwise bytes per step: unfused {unf / 1e9:.2f} GB, fused {fus / 1e9:.2f} GB "
        f"({unf / fus:.2f}x less)")
    if small_run:
        elementwise = None

    # the pages' protocol: flush caches, sync, event span per iteration, drop the first sample
    protocol = None
    if not args.no_protocol:
        flush = torch.empty(512 * 1024 * 1024 // 4, dtype=torch.float32, device="cuda")
        samples = []
        n_iter = max(2, args.steps)
        for _ in range(n_iter):
            flush.zero_()
            torch.cuda.synchronize()
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record(stream)
            step()
            b.record(stream)
            torch.cuda.synchronize()
            samples.append(a.elapsed_time(b) * 1e3)
        kept = samples[1:]
        protocol = {"mean_us": round(float(np.mean(kept)), 1), "min_us": round(float(np.min(kept)), 1),
                    "max_us": round(float(np.max(kept)), 1), "iterations": len(kept),
                    "flush": "512 MiB fill before each iteration (untimed)"}
        log(f"pages' protocol: mean {protocol['mean_us']:.1f} us, min {protocol['min_us']:.1f}, "
            f"max {protocol['max_us']:.1f} over {len(kept)} iterations")
        del flush

    cpu = None
    if not args.no_cpu_baseline:
        log(f"cpu baseline: oracle on {args.cpu_batch} samples for >= {args.cpu_seconds} s")
        cpu = cpu_baseline(w.name, args.cpu_batch, args.cpu_seconds)
        log(f"  {cpu['value']:.4g} tokens/s on {cpu['cores']} threads")

    power = None
    if sampler is not None:
        sampler.terminate()
        sampler.wait(timeout=30)
        power = power_summary(args.power_log, wall0, wall1)
        log(f"power over the timed region: {power}")

    out = {
        "metric": ("fwd+bwd tokens/s and % MFMA peak, B1024 T64 D1280 k2 bf16, 1 GPU" if w.name == PRODUCTION
                   else f"fwd+bwd tokens/s and % MFMA peak, {w.name}, 1 GPU"),
        "value": round(value, 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": w.dtype,
        "data": ("synthetic, x dy w1 b1 wout bout all zero (power-dependence measurement)" if args.zero_operands
                 else "synthetic (seeded N(0,1) inputs and upstream grad, he-uniform weights)"),
        "config": {"workload": w.name, "B": d.B, "T": d.T, "D": d.D, "k": d.k, "H": d.H,
                   "tokens_per_step": tokens, "parallelism": "single GPU", "kernels": args.kernels},
        "tflops": round(tflops, 2),
        "pct_mfma_peak": round(pct_peak, 2),
        "peak_device_bytes": int(peak_mem),
        "elementwise_bytes": elementwise,
        "roofline": roofline,
        "cpu_baseline": cpu,
        "pages_protocol": protocol,
        "graph_replay": graph,
        "kernels": kernels,
        "power": power,
    }
    if args.library_gemms:
        log("library GEMMs (torch.bmm) on the same shapes:")
        out["library_gemms"] = library_gemms(d, w.dtype)
    print(json.dumps(out), flush=True)


def load_traffic(kernel, workload):
    """HBM bytes per launch of `kernel`, from the rocprofv3 counter summary in profiles/ (FETCH_SIZE and
    WRITE_SIZE scaled by a calibration copy), or None when there is none or it predates the current kernel
    sources (source digest mismatch)."""
    path = os.path.join(ROOT, "profiles", f"hbm_traffic_{workload}.md")
    if not os.path.exists(path):
        return None
    from transformer_block_norm0_amd.build import source_digest
    digest, total = None, None
    for line in open(path):
        if line.startswith("source_digest:"):
            digest = line.split(":", 1)[1].strip()
        cells = [c.strip() for c in line.strip().strip("|").split("|")]
        if len(cells) == 7 and cells[0] == kernel:
            try:
                total = int(float(cells[6]))
            except ValueError:
                total = None
    if digest != source_digest():
        return None
    return total


if __name__ == "__main__":
    if len(sys.argv) == 3 and sys.argv[1] == "--power-sampler":
        power_sampler(sys.argv[2])
    else:
        main()
