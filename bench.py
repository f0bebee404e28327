"""Benchmark: StreamKL fused attention-KL forward + recompute backward on one GPU.

One step = the whole hot path over one batch: the forward kernel (per-row
KL, LSE1, LSE2), then the two backward kernels (dK1/dK2 and dQ1/dQ2), on
synthetic inputs already resident in HBM.  Prints ONE JSON line on stdout.

Default workload: B=1, H=32, N_Q=N_K=32768, d=128, bf16, causal, teacher
Q1,K1 ~ N(0,1), student = teacher + 0.2 N(0,1).  Credited work per head:
forward 4 N_Q N_K d, forward+backward 16 N_Q N_K d, halved when causal.
"""
import argparse
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2500.0   # MI355X dense bf16 MFMA, published
PEAK_F32_TFLOPS = 157.3
PEAK_HBM_GBS = 8000.0       # MI355X HBM3E, published

CSRC = os.path.join(ROOT, "attention_distillation_kl_amd", "csrc")
# Sources of each kernel's translation unit: the traffic counters recorded in
# profiles/ are reported only while these hash to the recorded value.
KERNEL_SOURCES = {
    "fwd": ["streamkl_fwd.hip", "streamkl_device.h", "streamkl_launch.h"],
    "bwd_dk": ["streamkl_bwd.h", "streamkl_bwd_dk.hip", "streamkl_device.h", "streamkl_launch.h"],
    "bwd_dq": ["streamkl_bwd.h", "streamkl_bwd_dq.hip", "streamkl_device.h", "streamkl_launch.h"],
    "bwd_fused": ["streamkl_bwd_fused.hip", "streamkl_device.h", "streamkl_launch.h"],
}


def kernel_hash(kernel):
    """sha256 (first 16 hex) of the kernel's sources with comments and
    whitespace removed, so that only code changes invalidate recorded
    counters.  (The sources hold no string literal containing a comment
    marker.)"""
    import hashlib
    import re
    m = hashlib.sha256()
    for f in KERNEL_SOURCES[kernel]:
        with open(os.path.join(CSRC, f)) as fh:
            text = fh.read()
        text = re.sub(r"/\*.*?\*/", " ", text, flags=re.S)
        text = re.sub(r"//[^\n]*", " ", text)
        m.update(" ".join(text.split()).encode())
    return m.hexdigest()[:16]


def recorded_traffic(workload, kernel):
    """HBM bytes per launch from profiles/<workload>_traffic.md (rocprofv3
    FETCH_SIZE/WRITE_SIZE, copy-calibrated), or None when absent or stale."""
    path = os.path.join(ROOT, "profiles", f"{workload}_traffic.md")
    if not os.path.exists(path):
        return None
    want = kernel_hash(kernel)
    with open(path) as fh:
        for line in fh:
            parts = line.split()
            if len(parts) == 4 and parts[0] == "traffic" and parts[1] == kernel and parts[2] == want:
                return float(parts[3])
    return None


def log(msg):
    print(msg, file=sys.stderr, flush=True)


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", default="h32k")
    ap.add_argument("--no-cpu-baseline", action="store_true",
                    help="skip timing the CPU oracle (for profiler runs)")
    ap.add_argument("--cpu-seconds", type=float, default=15.0,
                    help="target duration of the CPU oracle sample")
    ap.add_argument("--copy-probe", type=int, default=0, metavar="BYTES",
                    help="only run a plain device copy of BYTES bytes (calibrates HBM byte counters)")
    ap.add_argument("--no-clock", action="store_true",
                    help="skip sampling the GPU clock under load after the timed steps (sampled only for steps of 20 ms and more)")
    ap.add_argument("--sweep", action="store_true",
                    help="context-length sweep instead of the headline: N = 4K..--sweep-max, "
                         "forward and each backward configuration, causal and not; one JSON line per N")
    ap.add_argument("--sweep-min", type=int, default=4096)
    ap.add_argument("--sweep-max", type=int, default=524288)
    ap.add_argument("--sweep-heads", type=int, default=32)
    return ap.parse_args()


def sample_clock():
    """Current graphics clock of GPU 0 (MHz, mean over its XCDs) from
    `amd-smi metric --clock --json`, else `rocm-smi --showclocks --json`;
    None when neither answers."""
    import re
    import subprocess

    def first_json(text):
        starts = [i for i in (text.find("["), text.find("{")) if i >= 0]
        return json.JSONDecoder().raw_decode(text[min(starts):])[0]

    try:
        r = subprocess.run(["amd-smi", "metric", "--clock", "--json", "-g", "0"], capture_output=True,
                           text=True, timeout=30)
        data = first_json(r.stdout)
        if isinstance(data, dict) and "gpu_data" in data:
            data = data["gpu_data"]
        gpu = data[0] if isinstance(data, list) else data
        clocks = gpu.get("clock", gpu)
        vals = [v["clk"]["value"] for k, v in clocks.items() if k.startswith("gfx") and isinstance(v, dict)]
        vals = [float(v) for v in vals if isinstance(v, (int, float))]
        if vals:
            return {"sclk_mhz": round(sum(vals) / len(vals), 1), "xcds": len(vals), "source": "amd-smi metric --clock"}
    except Exception:
        pass
    try:
        r = subprocess.run(["rocm-smi", "--showclocks", "--json"], capture_output=True, text=True, timeout=30)
        data = first_json(r.stdout)
        card = next(iter(data.values()))
        m = re.search(r"(\d+)\s*Mhz", card.get("sclk clock speed:", ""), re.I)
        if m:
            return {"sclk_mhz": float(m.group(1)), "xcds": None, "source": "rocm-smi --showclocks"}
    except Exception:
        pass
    return None


def copy_probe(nbytes):
    """A plain device-to-device copy of known size, for scaling FETCH_SIZE /
    WRITE_SIZE readings of the StreamKL kernels to bytes."""
    import torch
    src = torch.ones(nbytes, dtype=torch.uint8, device="cuda")
    dst = torch.empty_like(src)
    for _ in range(3):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"copy_probe_bytes": nbytes, "launches": 3}), flush=True)


def cpu_baseline(w, q1, k1, q2, k2, target_s):
    """Time the fp64 oracle (as it stands) on a sample of the workload.

    The sample is the last R query rows of head 0 (for causal workloads the
    longest rows), then -- once R covers the head -- whole heads 0..n-1; it
    grows until one run of it takes at least two thirds of ``target_s``
    seconds, and that run is the one reported.  The oracle computes what the
    workload's timed step computes (forward + backward, or the forward
    alone), credited with the GPU figure's count per admissible (query, key)
    pair: 16 d flops for forward + backward, 4 d for the forward."""
    import numpy as np
    import torch
    import oracle

    grads = w.passes == "fwd+bwd"
    per_pair = (16.0 if grads else 4.0) * w.d
    off = w.NK - w.NQ
    nheads = w.B * w.H
    cache = {}

    def head(hh):
        if hh not in cache:
            b, h = divmod(hh, w.H)
            cache[hh] = [t[b, h].to("cpu", torch.float64).numpy() for t in (q1, k1, q2, k2)]
        return cache[hh]

    def credited(rows):
        rb = w.NQ - rows
        keys = np.array([min(w.NK, i + off + 1) if w.causal else w.NK for i in range(rb, w.NQ)], dtype=np.float64)
        return per_pair * keys.sum()

    def run(rows, nh):
        hs = [head(hh) for hh in range(nh)]   # conversions are not timed
        t0 = time.perf_counter()
        for c in hs:
            oracle.head(*c, w.scale, w.causal, rows=(w.NQ - rows, w.NQ), grads=grads)
        return time.perf_counter() - t0

    rows, nh = min(w.NQ, 32), 1
    run(rows, nh)                      # threads and pages warm
    while True:                        # grow the sample until it takes two thirds of the target
        dt = run(rows, nh)
        if dt >= target_s * 2 / 3 or (rows >= w.NQ and nh >= nheads):
            break
        f = min(16.0, max(1.5, target_s / max(dt, 1e-3)))
        if rows < w.NQ:
            rows = min(w.NQ, int(rows * f))
        else:
            nh = min(nheads, int(math.ceil(nh * f)))
    fl = credited(rows) * nh
    what = "forward+backward" if grads else "forward"
    where = f"the last {rows} query rows of head 0" if nh == 1 else f"all {rows} query rows of heads 0..{nh - 1}"
    return {"value": fl / dt / 1e12, "unit": "TFLOP/s", "cores": oracle.num_threads(), "kind": "oracle",
            "sample": f"fp64 oracle, {what} of {where} ({fl / 1e12:.3f} TFLOP credited, {dt:.1f} s)"}


def sweep(args):
    """Latency and memory against context length, on the axes of the page's
    results ("Risultati Sperimentali": 4K to 512K tokens, doubling from
    --sweep-min; forward latency,
    causal and not; backward latency of Configuration 1 and Configuration 2;
    memory footprint).  B = 1, H = --sweep-heads, d = 128, bf16, student =
    teacher + 0.2 N(0,1).  For each N and mask the times are HIP events around
    one library call on the current stream (median of the timed calls), and
    `extra_hbm_bytes` is the peak device memory of the call minus its inputs
    and outputs: the workspace and anything else it needed."""
    import torch
    from attention_distillation_kl_amd import make_inputs, ops, _lib

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    H, d = args.sweep_heads, 128
    n = getattr(args, "sweep_min", 4096)
    while n <= args.sweep_max:
        q1, k1, q2, k2 = make_inputs(1, H, n, n, d, torch.bfloat16, "student", 0.2,
                                     seed=2000 + n.bit_length(), device=dev)
        reps = 3 if n <= 65536 else 1
        row = {"N": n, "B": 1, "H": H, "d": d, "dtype": "bf16",
               "input_bytes": 4 * q1.numel() * q1.element_size()}
        for causal in (True, False):
            tag = "causal" if causal else "noncausal"

            def timed(fn, out_bytes):
                fn()                          # warm-up (and the result the backward needs)
                torch.cuda.synchronize()
                torch.cuda.reset_peak_memory_stats(dev)
                base = torch.cuda.memory_allocated(dev)
                ms = []
                for _ in range(reps):
                    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                    e0.record()
                    r = fn()
                    e1.record()
                    torch.cuda.synchronize()
                    ms.append(e0.elapsed_time(e1))
                    del r
                extra = torch.cuda.max_memory_allocated(dev) - base - out_bytes
                return sorted(ms)[len(ms) // 2], max(0, extra)

            fwd_out = 3 * H * n * 4
            t, x = timed(lambda: ops.streamkl_fwd(q1, k1, q2, k2, None, causal), fwd_out)
            kl, lse1, lse2 = ops.streamkl_fwd(q1, k1, q2, k2, None, causal)
            fl = 4.0 * H * n * n * d * (0.5 if causal else 1.0)
            row[f"fwd_ms_{tag}"] = round(t, 4)
            row[f"fwd_tflops_{tag}"] = round(fl / (t * 1e-3) / 1e12, 1)
            row[f"fwd_extra_hbm_bytes_{tag}"] = x
            for cfg, mask in (("config1", _lib.GRAD_Q2K2), ("config2", _lib.GRAD_Q1K1)):
                grad_out = 2 * q1.numel() * q1.element_size()
                t, x = timed(lambda: ops.streamkl_bwd(q1, k1, q2, k2, kl, lse1, lse2, None, None, causal, mask),
                             grad_out)
                row[f"bwd_{cfg}_ms_{tag}"] = round(t, 4)
                row[f"bwd_{cfg}_extra_hbm_bytes_{tag}"] = x
            del kl, lse1, lse2
            log(f"bench: sweep N={n} {tag} done")
        print(json.dumps(row), flush=True)
        del q1, k1, q2, k2
        torch.cuda.empty_cache()
        n *= 2


def roofline_bound(w, kernel, peak_tflops):
    """(bound, algorithmic work per launch, peak, unit) of one timed kernel:
    HBM when its flops per algorithmic byte fall below the machine balance
    (peak flops / HBM bandwidth), MFMA otherwise.

    Algorithmic flops per admissible (query, key) pair of one head: the
    forward 4 d (S1, S2).  The backward is credited 12 d in all: the two
    recomputed score products (4 d) and the four gradient products (8 d).
    Each of its two kernels forms two of the gradients, so each is credited
    half of that, 6 d; the second recompute the two-kernel form executes is
    not algorithmic work (see executed_flops).  The fused backward (short
    query blocks) forms all four gradients in one kernel: 12 d."""
    fwd_fl = w.fwd_flops()
    flops = {"fwd": 1.0, "bwd_dk": 1.5, "bwd_dq": 1.5, "bwd_fused": 3.0}[kernel] * fwd_fl
    nbytes = w.fwd_bytes() if kernel == "fwd" else w.bwd_bytes(kernel)
    if flops / nbytes < peak_tflops * 1e12 / (PEAK_HBM_GBS * 1e9):
        return "hbm", nbytes, PEAK_HBM_GBS, "GB/s"
    return "mfma", flops, peak_tflops, "TFLOP/s"


def executed_flops(w, kernel):
    """MFMA flops one launch of the kernel executes: the forward's 4 d per
    pair; each two-kernel backward kernel recomputes both score blocks (4 d)
    and forms two gradients (4 d), 8 d per pair; the fused backward 12 d."""
    fwd_fl = w.fwd_flops()
    return {"fwd": 1.0, "bwd_dk": 2.0, "bwd_dq": 2.0, "bwd_fused": 3.0}[kernel] * fwd_fl


def main():
    args = parse()
    if args.copy_probe:
        copy_probe(args.copy_probe)
        return
    if args.sweep:
        if args.gpus != 1:
            print("bench.py measures one GPU only", file=sys.stderr)
            sys.exit(2)
        sweep(args)
        return
    if args.gpus != 1:
        print(f"bench.py measures one GPU only; --gpus {args.gpus} is not supported "
              "(the per-head work is independent and would shard over heads with no exchange)",
              file=sys.stderr)
        sys.exit(2)

    import torch
    from attention_distillation_kl_amd import WORKLOADS, workload_inputs
    from attention_distillation_kl_amd import _lib, ops

    w = WORKLOADS[args.workload]
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    log(f"bench: workload {w.name} {w.as_dict()}")
    q1, k1, q2, k2 = workload_inputs(w, dev)
    B, H, NQ, NK, d = w.B, w.H, w.NQ, w.NK, w.d
    kl = torch.empty(B, H, NQ, device=dev, dtype=torch.float32)
    lse1, lse2 = torch.empty_like(kl), torch.empty_like(kl)
    dq = (torch.empty_like(q1), torch.empty_like(q2))
    dk = (torch.empty_like(k1), torch.empty_like(k2))
    do_bwd = w.passes == "fwd+bwd"
    # The backward's workspace (short query blocks only), allocated once.
    # Where streamkl_bwd takes the fused form, the step runs it (one kernel
    # and its workspace fill and conversion); otherwise the two halves, the
    # query half with the workspace, i.e. the key-partitioned path where
    # streamkl_bwd takes it.
    ws = ops.streamkl_bwd_workspace(q1, k1, w.causal) if do_bwd else None
    dt = _lib.BF16 if w.dtype == "bf16" else _lib.F32
    fused = do_bwd and _lib.bwd_fused_selected(B, H, NQ, NK, d, int(w.causal), dt, _lib.GRAD_ALL) == 1

    def step(ev=None):
        if ev is not None:
            ev[0].record()
        kl_, l1_, l2_ = ops.streamkl_fwd(q1, k1, q2, k2, w.scale, w.causal)
        if ev is not None:
            ev[1].record()
        if do_bwd and fused:
            ops.streamkl_bwd_fused(q1, k1, q2, k2, kl_, l1_, l2_, None, w.scale, w.causal, workspace=ws,
                                   out=(dq[0], dk[0], dq[1], dk[1]))
            if ev is not None:
                ev[2].record()
        elif do_bwd:
            ops.streamkl_bwd_half("dk", q1, k1, q2, k2, kl_, l1_, l2_, None, w.scale, w.causal, out=dk,
                                  workspace=ws)
            if ev is not None:
                ev[2].record()
            ops.streamkl_bwd_half("dq", q1, k1, q2, k2, kl_, l1_, l2_, None, w.scale, w.causal, out=dq,
                                  workspace=ws)
            if ev is not None:
                ev[3].record()

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    log(f"bench: {args.warmup} warmup steps done")

    nev = (3 if fused else 4) if do_bwd else 2
    events = [[torch.cuda.Event(enable_timing=True) for _ in range(nev)] for _ in range(args.steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        step(events[i])
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    log(f"bench: {args.steps} timed steps done in {wall:.3f} s")

    def median(xs):
        xs = sorted(xs)
        return xs[len(xs) // 2]

    # Per-step and per-kernel figures are medians over the timed steps (means
    # are reported beside them).
    step_ev = sorted(e[0].elapsed_time(e[nev - 1]) for e in events)
    step_ms = median(step_ev)
    spans = {"fwd": (0, 1)}
    if fused:
        spans["bwd_fused"] = (1, 2)
    elif do_bwd:
        spans["bwd_dk"] = (1, 2)
        spans["bwd_dq"] = (2, 3)
    kern = {k: median(e[a].elapsed_time(e[b]) for e in events) for k, (a, b) in spans.items()}
    kern_mean = {k: sum(e[a].elapsed_time(e[b]) for e in events) / args.steps for k, (a, b) in spans.items()}
    fwd_ms = kern["fwd"]
    ms_per_step = wall * 1e3 / args.steps

    fwd_fl = w.fwd_flops()
    total_fl = w.fwdbwd_flops() if do_bwd else fwd_fl
    peak = PEAK_BF16_TFLOPS if w.dtype == "bf16" else PEAK_F32_TFLOPS
    value = total_fl / (step_ms * 1e-3) / 1e12
    fwd_tf = fwd_fl / (fwd_ms * 1e-3) / 1e12

    # Dominant kernel: the one with the largest median duration, priced in
    # algorithmic work per launch (roofline_bound).  Workloads below the
    # machine balance (decoding rows) are priced in algorithmic HBM bytes
    # against the HBM bandwidth instead.
    dom = max(kern, key=kern.get)
    bound, work, rpeak, runit = roofline_bound(w, dom, peak)
    scale_unit = 1e12 if runit == "TFLOP/s" else 1e9
    ach = work / (kern[dom] * 1e-3) / scale_unit
    roof = {"bound": bound, "kernel": dom, "achieved": round(ach, 2), "peak": rpeak, "unit": runit,
            "frac": round(ach / rpeak, 4), "traffic": recorded_traffic(w.name, dom),
            ("flops_per_launch" if bound == "mfma" else "bytes_per_launch"): work,
            "avg_launch_ms": round(kern[dom], 4)}
    if bound == "mfma":
        ex = executed_flops(w, dom)
        roof["executed_flops_per_launch"] = ex
        roof["executed_tflops"] = round(ex / (kern[dom] * 1e-3) / 1e12, 2)

    # The graphics clock, sampled while untimed steps keep the GPU busy (the
    # clock drops within milliseconds once the GPU idles, and takes a while to
    # come back).  Steps are queued about 20 ms at a time and run for about
    # 200 ms before the sample starts.  Only steps of 20 ms and more are
    # sampled: steps made of shorter kernels leave XCDs idle between them,
    # and the reading then swings between idle and load clocks.
    clock = None
    if not args.no_clock and step_ms >= 20.0:
        import threading
        got = {}
        per_sync = max(1, int(20.0 / max(step_ms, 1e-3)))
        for _ in range(10):
            for _ in range(per_sync):
                step()
            torch.cuda.synchronize()
        th = threading.Thread(target=lambda: got.update(c=sample_clock()))
        th.start()
        while th.is_alive():
            for _ in range(per_sync):
                step()
            torch.cuda.synchronize()
        th.join()
        clock = got.get("c")
        if clock is not None:
            clock["published_peak_mhz"] = 2400

    cpu = None
    if not args.no_cpu_baseline:
        log("bench: timing the CPU oracle sample")
        cpu = cpu_baseline(w, q1, k1, q2, k2, args.cpu_seconds)
        cpu["value"] = round(cpu["value"], 6)

    desc = (f"{w.name}: B={B},H={H},N_Q={NQ},N_K={NK},d={d},{w.dtype},"
            f"{'causal' if w.causal else 'non-causal'},{w.mode}" + (f" sigma={w.sigma}" if w.mode == "student" else ""))
    out = {
        "metric": "fused attention-KL TFLOP/s (fwd, fwd+bwd) at N=32K causal; % MFMA peak",
        "value": round(value, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": w.dtype,
        "data": "synthetic (seeded Gaussian teacher, student = teacher + noise)",
        "config": {"workload": desc, "passes": w.passes, "seed": w.seed, "scale": w.scale},
        "fwd_tflops": round(fwd_tf, 2),
        "pct_peak_fwd": round(100 * fwd_tf / peak, 2),
        "pct_peak_fwdbwd": round(100 * value / peak, 2),
        "event_ms_median": round(step_ms, 4),
        "event_ms_mean": round(sum(step_ev) / len(step_ev), 4),
        "event_ms_min": round(step_ev[0], 4),
        "observed_clock": clock,
        "kernel_ms": {k: round(v, 4) for k, v in kern.items()},
        "kernel_ms_mean": {k: round(v, 4) for k, v in kern_mean.items()},
        "roofline": roof,
        "cpu_baseline": cpu,
    }
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
