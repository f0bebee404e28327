"""Host-side checks of the benchmark's contract (no GPU needed)."""
import os
import subprocess
import sys

from attention_distillation_kl_amd import WORKLOADS

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_more_than_one_gpu_is_refused_with_a_message():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr


def test_headline_flop_credit():
    """Forward 4 N_Q N_K d per head and forward+backward 16 N_Q N_K d,
    halved for causal: 8.80 and 35.18 TFLOP at B=1, H=32, N=32768, d=128."""
    w = WORKLOADS["h32k"]
    assert (w.B, w.H, w.NQ, w.NK, w.d, w.causal) == (1, 32, 32768, 32768, 128, True)
    assert w.fwd_flops() == 4 * 32 * 32768 * 32768 * 128 // 2
    assert w.fwdbwd_flops() == 4 * w.fwd_flops()
    c4 = WORKLOADS["c4"]
    assert c4.fwd_flops() == 4 * 32 * 2048 * 65536 * 128


def test_profiling_options_exist():
    # --copy-probe (traffic-counter calibration) and --no-cpu-baseline (profiler
    # runs) need a GPU to run; here only their presence is checked.
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--help"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 0 and "--copy-probe" in r.stdout and "--no-cpu-baseline" in r.stdout
    assert "--sweep" in r.stdout


def test_recorded_traffic_lines_are_well_formed():
    sys.path.insert(0, ROOT)
    import bench
    for kernel in ("fwd", "bwd_dk", "bwd_dq"):
        t = bench.recorded_traffic("h32k", kernel)
        assert t is None or t > 1e9  # present only while the kernel's sources are unchanged


def test_clock_sampling_parses_amd_smi_then_rocm_smi(monkeypatch):
    """The graphics clock under load: amd-smi's per-XCD clocks (averaged),
    with text around the JSON; rocm-smi's single reading when amd-smi fails;
    None when neither answers."""
    import subprocess
    import types
    sys.path.insert(0, ROOT)
    import bench

    amd = ('WARNING: something\n{"gpu_data": [{"gpu": 0, "clock": {'
           '"gfx_0": {"clk": {"value": 2000, "unit": "MHz"}}, "gfx_1": {"clk": {"value": 1900, "unit": "MHz"}}, '
           '"mem_0": {"clk": {"value": 2000, "unit": "MHz"}}}}]}\n')
    rocm = '{"card0": {"sclk clock speed:": "(1960Mhz)", "sclk clock level:": "S"}}\nWARNING: x\n'
    answers = {}

    def fake_run(cmd, **kw):
        out = answers.get(cmd[0])
        if out is None:
            raise FileNotFoundError(cmd[0])
        return types.SimpleNamespace(stdout=out, returncode=0)

    monkeypatch.setattr(subprocess, "run", fake_run)
    answers.update({"amd-smi": amd, "rocm-smi": rocm})
    c = bench.sample_clock()
    assert c["sclk_mhz"] == 1950.0 and c["xcds"] == 2 and c["source"].startswith("amd-smi")
    answers.pop("amd-smi")
    c = bench.sample_clock()
    assert c["sclk_mhz"] == 1960.0 and c["source"].startswith("rocm-smi")
    answers.clear()
    assert bench.sample_clock() is None


def test_kernel_hash_ignores_comments_and_whitespace(tmp_path, monkeypatch):
    sys.path.insert(0, ROOT)
    import bench

    src = tmp_path / "k.hip"
    monkeypatch.setattr(bench, "CSRC", str(tmp_path))
    monkeypatch.setitem(bench.KERNEL_SOURCES, "probe", ["k.hip"])
    src.write_text("int f(int x) {\n  return x + 1;  // add one\n}\n")
    h0 = bench.kernel_hash("probe")
    src.write_text("/* a block\n comment */ int f(int x) {   return x + 1; }\n// trailing\n")
    assert bench.kernel_hash("probe") == h0
    src.write_text("int f(int x) {\n  return x + 2;\n}\n")
    assert bench.kernel_hash("probe") != h0


def test_cpu_baseline_times_what_the_step_computes(monkeypatch):
    """The oracle sample runs the workload's own passes (the forward alone
    for a forward-only workload), grows over whole heads once one head's rows
    are not enough, and is credited per admissible pair as the GPU figure is
    (16 d flops forward + backward, 4 d forward)."""
    import numpy as np
    import torch
    sys.path.insert(0, ROOT)
    import bench
    import oracle
    from attention_distillation_kl_amd.inputs import Workload

    calls = []
    real = oracle.head

    def spy(*a, **kw):
        calls.append((a[0].shape, kw["rows"], kw["grads"]))
        return real(*a, **kw)

    monkeypatch.setattr(oracle, "head", spy)
    monkeypatch.setattr(bench.time, "perf_counter", iter(np.arange(0.0, 1e6, 0.01)).__next__)
    g = torch.Generator().manual_seed(3)
    for passes, causal, per_pair in (("fwd", False, 4), ("fwd+bwd", True, 16)):
        w = Workload("t", 2, 3, 40, 56, 64, "f32", causal, "iid", 0.0, 1, passes)
        q = [torch.randn(2, 3, 40, 64, generator=g) for _ in range(2)]
        k = [torch.randn(2, 3, 56, 64, generator=g) for _ in range(2)]
        calls.clear()
        # Each timed run reads as 0.01 s: a 10 s target grows the sample to every head.
        r = bench.cpu_baseline(w, q[0], k[0], q[1], k[1], 10.0)
        assert all(c[2] == (passes == "fwd+bwd") for c in calls)
        assert calls[-1][1] == (0, 40) and len({c[0] for c in calls}) == 1
        nh = int(r["sample"].split("heads 0..")[1].split()[0]) + 1
        assert nh == 6 and ("forward+backward" in r["sample"]) == (passes == "fwd+bwd")
        keys = sum(min(56, i + 16 + 1) if causal else 56 for i in range(40))
        assert abs(r["value"] * 0.01 * 1e12 - per_pair * 64 * keys * nh) < 1e-3 * per_pair * 64 * keys * nh


def test_roofline_bound_follows_arithmetic_intensity():
    """Kernels whose flops per algorithmic byte fall below the machine balance
    (decoding rows) are priced against HBM bandwidth, the rest against MFMA;
    the byte counts are the inputs read once, the row vectors and the outputs."""
    sys.path.insert(0, ROOT)
    import bench
    h, dec = WORKLOADS["h32k"], WORKLOADS["decode"]
    for k in ("fwd", "bwd_dk", "bwd_dq"):
        assert bench.roofline_bound(h, k, 2500.0)[0] == "mfma"
    bound, nbytes, peak, unit = bench.roofline_bound(dec, "fwd", 2500.0)
    assert (bound, peak, unit) == ("hbm", 8000.0, "GB/s")
    assert nbytes == 32 * (2 * (1 + 65536) * 128 * 2 + 12 * 1)
    n = 32768
    assert h.bwd_bytes("bwd_dk") == 32 * (2 * 2 * n * 128 * 2 + 16 * n + 2 * n * 128 * 2)
    assert h.fwd_bytes() == 32 * (2 * 2 * n * 128 * 2 + 12 * n)


def test_roofline_credits_the_algorithmic_flops():
    """Per admissible (query, key) pair of a head the forward is credited
    4 d flops and each backward kernel 6 d (half of the backward's 12 d: two
    recomputed score products and four gradient products); the second
    recompute of the two-kernel form is reported as executed work only."""
    sys.path.insert(0, ROOT)
    import bench
    h = WORKLOADS["h32k"]
    pairs = 32 * 32768 * 32768 / 2
    assert bench.roofline_bound(h, "fwd", 2500.0)[1] == 4 * 128 * pairs
    for k in ("bwd_dk", "bwd_dq"):
        assert bench.roofline_bound(h, k, 2500.0)[1] == 6 * 128 * pairs
        assert bench.executed_flops(h, k) == 8 * 128 * pairs
    # the two backward kernels together carry the backward's 12 d, and with
    # the forward the 16 d of the headline figure
    assert 2 * bench.roofline_bound(h, "bwd_dk", 2500.0)[1] + bench.roofline_bound(h, "fwd", 2500.0)[1] \
        == h.fwdbwd_flops()
    assert abs(bench.roofline_bound(h, "bwd_dk", 2500.0)[1] - 1.319e13) < 1e10


def test_short_query_backward_is_priced_in_hbm_bytes():
    """64 queries over 64K keys: the fused backward forms all four gradients
    (12 d flops per pair) while it reads the four inputs and writes the four
    gradients once, about 96 flops per algorithmic byte, below the machine
    balance: it is priced in bytes against the HBM bandwidth."""
    sys.path.insert(0, ROOT)
    import bench
    w = WORKLOADS["shortq"]
    bound, nbytes, peak, unit = bench.roofline_bound(w, "bwd_fused", 2500.0)
    assert (bound, peak, unit) == ("hbm", 8000.0, "GB/s")
    per_head = 2 * (64 + 65536) * 128 * 2 + 16 * 64 + 2 * (64 + 65536) * 128 * 2
    assert nbytes == 32 * per_head
    assert bench.executed_flops(w, "bwd_fused") == 12 * 32 * 64 * 65536 * 128
