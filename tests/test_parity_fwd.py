"""GPU forward parity: per-row KL, LSE1, LSE2 from the HIP kernel (through
the C ABI) against the fp64 oracle on the very same inputs."""
import math

import numpy as np
import pytest
import torch

from attention_distillation_kl_amd import WORKLOADS, make_inputs, workload_inputs
from attention_distillation_kl_amd import ops
from parity_util import (check_rows, head64, log, magnitude_k, oracle_heads, oracle_row_blocks, row_blocks,
                         to64)

pytestmark = pytest.mark.gpu

DEV = "cuda"
DT = {"bf16": torch.bfloat16, "f32": torch.float32}


def run_and_compare(q1, k1, q2, k2, scale, causal, heads=None, tag="", by_magnitude=False, k=None,
                    tol_dtype=None):
    """Forward through the C ABI against the oracle, row by row.  With
    ``by_magnitude`` the bound adds k 2^-24 max(|LSE1_ref|, |LSE2_ref|), k
    from magnitude_k unless given; ``tol_dtype`` overrides the dtype whose
    stated tolerance applies."""
    kl, l1, l2 = ops.streamkl_fwd(q1, k1, q2, k2, scale, causal)
    torch.cuda.synchronize()
    B, H = q1.shape[:2]
    heads = range(B * H) if heads is None else heads
    ref = oracle_heads(q1, k1, q2, k2, scale, causal, heads)
    if by_magnitude and k is None:
        k = magnitude_k(q1.dtype, q1.shape[-1])
    tdt = q1.dtype if tol_dtype is None else tol_dtype
    worst = 0.0
    for hh in heads:
        b, h = divmod(hh, H)
        mag = np.maximum(np.abs(ref[hh]["lse1"]), np.abs(ref[hh]["lse2"])) if by_magnitude else None
        for name, got in (("kl", kl), ("lse1", l1), ("lse2", l2)):
            worst = max(worst, check_rows(to64(got[b, h]), ref[hh][name], tdt, f"{tag} head {hh} {name}", mag, k))
    return kl, l1, l2, worst


# Ragged shapes spanning several tiles, with tails in both N_Q and N_K.
SHAPES = [
    # B, H, NQ, NK, d, dtype, causal
    (1, 1, 1, 1, 64, "bf16", False),
    (1, 1, 1, 1, 128, "f32", True),
    (1, 2, 2, 3, 64, "bf16", True),
    (1, 1, 3, 2, 128, "bf16", False),
    (1, 3, 17, 63, 128, "bf16", True),
    (2, 1, 65, 65, 64, "f32", True),
    (1, 2, 129, 65, 64, "f32", False),
    (1, 2, 257, 257, 128, "bf16", True),
    (1, 2, 300, 333, 64, "bf16", True),
    (1, 2, 300, 333, 128, "f32", False),
    (2, 2, 513, 1000, 128, "bf16", True),
    (1, 1, 640, 129, 128, "bf16", False),
    (1, 1, 1000, 1000, 64, "f32", True),
]


@pytest.mark.parametrize("shape", SHAPES, ids=lambda s: "x".join(map(str, s)))
def test_fwd_ragged_shapes(shape):
    B, H, NQ, NK, d, dt, causal = shape
    log(f"fwd ragged {shape}")
    q1, k1, q2, k2 = make_inputs(B, H, NQ, NK, d, DT[dt], "student", 0.5, seed=NQ * 7 + NK, device=DEV)
    run_and_compare(q1, k1, q2, k2, 1.0 / math.sqrt(d), causal, tag=str(shape))


def test_fwd_c1_fp32_full():
    w = WORKLOADS["c1"]
    log("fwd c1")
    q1, k1, q2, k2 = workload_inputs(w, DEV)
    _, _, _, worst = run_and_compare(q1, k1, q2, k2, w.scale, w.causal, tag="c1")
    assert worst <= 1e-5


def test_fwd_c2_bf16_full():
    w = WORKLOADS["c2"]
    log("fwd c2")
    q1, k1, q2, k2 = workload_inputs(w, DEV)
    run_and_compare(q1, k1, q2, k2, w.scale, w.causal, tag="c2")


@pytest.mark.parametrize("name", ["c3", "c4", "c5", "h32k"])
def test_fwd_full_size_sampled_rows(name):
    """Full-size workloads in the benchmark's launch configuration; the oracle
    checks row blocks at the start, middle and end of the first and last head."""
    w = WORKLOADS[name]
    log(f"fwd {name} full size, sampled rows")
    q1, k1, q2, k2 = workload_inputs(w, DEV)
    kl, l1, l2 = ops.streamkl_fwd(q1, k1, q2, k2, w.scale, w.causal)
    torch.cuda.synchronize()
    assert torch.isfinite(kl).all() and torch.isfinite(l1).all() and torch.isfinite(l2).all()
    assert (kl > -1e-3).all()
    nh = w.B * w.H
    for hh in (0, nh - 1):
        b, h = divmod(hh, w.H)
        blocks = row_blocks(w.NQ)
        ref = oracle_row_blocks(head64(q1, k1, q2, k2, hh), w.scale, w.causal, blocks)
        idx = np.concatenate([np.arange(rb, re) for rb, re in blocks])
        for key, got in (("kl", kl), ("lse1", l1), ("lse2", l2)):
            check_rows(to64(got[b, h])[idx], ref[key][idx], q1.dtype, f"{name} head {hh} {key}")
    del q1, k1, q2, k2
    torch.cuda.empty_cache()


def test_fwd_c4_whole_heads():
    """C4 (2048 queries over 65536 keys, non-causal, forward only) in the
    benchmark's launch configuration -- the library's key partitions and the
    merge -- with every row of the first and last head compared with the
    oracle: all eight query blocks and every partition's keys."""
    w = WORKLOADS["c4"]
    log("fwd c4 full size, whole first and last heads")
    q1, k1, q2, k2 = workload_inputs(w, DEV)
    kl, l1, l2 = ops.streamkl_fwd(q1, k1, q2, k2, w.scale, w.causal)
    torch.cuda.synchronize()
    heads = [0, w.B * w.H - 1]
    ref = oracle_heads(q1, k1, q2, k2, w.scale, w.causal, heads)
    for hh in heads:
        b, h = divmod(hh, w.H)
        for key, got in (("kl", kl), ("lse1", l1), ("lse2", l2)):
            check_rows(to64(got[b, h]), ref[hh][key], q1.dtype, f"c4 head {hh} {key}")
    del q1, k1, q2, k2
    torch.cuda.empty_cache()


@pytest.mark.parametrize("dt", ["bf16", "f32"])
@pytest.mark.parametrize("causal", [False, True])
def test_fwd_identical_teacher_student_is_exactly_zero(dt, causal):
    q, k, _, _ = make_inputs(2, 2, 200, 260, 128, DT[dt], "iid", 0, seed=5, device=DEV)
    kl, l1, l2 = ops.streamkl_fwd(q, k, q, k, 0.1, causal)
    assert torch.equal(kl, torch.zeros_like(kl))
    assert torch.equal(l1, l2)


def test_fwd_uniform_student():
    """Q2 = 0: LSE2 = ln|J_i| (bottom-right causal count)."""
    q1, k1, _, k2 = make_inputs(1, 2, 100, 150, 64, torch.bfloat16, "iid", 0, seed=6, device=DEV)
    q2 = torch.zeros_like(q1)
    kl, l1, l2 = ops.streamkl_fwd(q1, k1, q2, k2, 0.125, True)
    J = torch.arange(100, device=DEV, dtype=torch.float64) + 51
    assert torch.allclose(l2.double(), J.log().expand_as(l2), atol=2e-6, rtol=0)
    run_and_compare(q1, k1, q2, k2, 0.125, True, tag="uniform student")


@pytest.mark.parametrize("dt", ["bf16", "f32"])
def test_fwd_peaked_and_large_inputs(dt):
    """scale = 1 on N(0, 1) d = 128 data gives logits with std ~11 (near one-hot
    rows); x8 inputs on top of that stress the max-shift.  Logits reach tens
    to hundreds here, so the bound adds the fp32 rounding of scores of that
    size (parity_util.magnitude_k: 45 u |LSE| for bf16, 269 u |LSE| for fp32
    at d = 128)."""
    q1, k1, q2, k2 = make_inputs(1, 2, 256, 256, 128, DT[dt], "student", 0.3, seed=8, device=DEV)
    kl, l1, l2, _ = run_and_compare(q1, k1, q2, k2, 1.0, True, tag="peaked", by_magnitude=True)
    assert torch.isfinite(kl).all()
    big = [t * 8 for t in (q1, k1, q2, k2)]
    kl, _, _, _ = run_and_compare(*big, 0.5, False, tag="large", by_magnitude=True)
    assert torch.isfinite(kl).all()


@pytest.mark.parametrize("dt", ["bf16", "f32"])
@pytest.mark.parametrize("direction", [1, -1])
@pytest.mark.parametrize("causal", [False, True])
def test_fwd_logits_that_rise_or_fall_along_the_keys(dt, direction, causal):
    """Keys along a common direction u with a linear ramp: the logits of
    every row grow (direction 1) by about 1.5 per key, i.e. by more than 64
    log2 units per 32-key block, so the running shift must be raised on
    every block; or they fall (direction -1), so the first block's maximum
    holds for the whole row.  The bound adds the fp32 rounding of scores of
    that size, as for the other inputs far outside unit scale."""
    g = torch.Generator(device=DEV).manual_seed(77)
    NQ, NK, d = 96, 700, 64
    u = torch.randn(d, device=DEV, generator=g)
    u = u / u.norm()
    ramp = torch.arange(NK, device=DEV, dtype=torch.float32)
    if direction < 0:
        ramp = ramp.flip(0)
    def keys():
        return (ramp[:, None] / 8.0) * u + 0.3 * torch.randn(NK, d, device=DEV, generator=g)
    def queries():
        return 12.0 * u + 0.3 * torch.randn(NQ, d, device=DEV, generator=g)
    q1, k1, q2, k2 = (x[None, None].to(DT[dt]).contiguous() for x in (queries(), keys(), queries(), keys()))
    kl, l1, l2, _ = run_and_compare(q1, k1, q2, k2, 1.0, causal, tag=f"ramp {direction}", by_magnitude=True)
    assert torch.isfinite(kl).all() and torch.isfinite(l1).all() and torch.isfinite(l2).all()


@pytest.mark.parametrize("dt", ["bf16", "f32"])
@pytest.mark.parametrize("direction", [1, -1])
@pytest.mark.parametrize("causal", [False, True])
def test_fwd_teacher_and_student_maxima_far_apart(dt, direction, causal):
    """The keys of the ramp test above, with the teacher's queries along u in
    every row but the student's only in even rows: in odd rows the student's
    logits stay near unit scale while the teacher's climb (or start) hundreds
    of log2 units above them, so the teacher's shift is raised on every block
    (rising logits) while the student's must stay near its own maximum, or
    its terms underflow to zero.  Every wave holds rows of both kinds.  Same
    bound as the ramp test."""
    g = torch.Generator(device=DEV).manual_seed(78)
    NQ, NK, d = 96, 700, 64
    u = torch.randn(d, device=DEV, generator=g)
    u = u / u.norm()
    ramp = torch.arange(NK, device=DEV, dtype=torch.float32)
    if direction < 0:
        ramp = ramp.flip(0)
    def keys():
        return (ramp[:, None] / 8.0) * u + 0.3 * torch.randn(NK, d, device=DEV, generator=g)
    q1 = 12.0 * u + 0.3 * torch.randn(NQ, d, device=DEV, generator=g)
    q2 = 0.3 * torch.randn(NQ, d, device=DEV, generator=g)
    q2[0::2] += 12.0 * u
    q1, k1, q2, k2 = (x[None, None].to(DT[dt]).contiguous() for x in (q1, keys(), q2, keys()))
    kl, l1, l2, _ = run_and_compare(q1, k1, q2, k2, 1.0, causal, tag=f"apart {direction}", by_magnitude=True)
    assert torch.isfinite(kl).all() and torch.isfinite(l1).all() and torch.isfinite(l2).all()
    gap = (l1 - l2)[0, 0].abs().cpu()
    assert (gap[1::2] > 64 * math.log(2)).all()   # odd rows: the maxima really are far apart


# KL / LSE rounding when every score is exact in fp32 (multiple of 2^-24
# |LSE_ref|).  Left: one rounding each in the exponent's shift -m c, in
# m * scale, in m * scale + log l and in the lane-half merge; the raises'
# rescale factors exp2((m - m') c), whose arguments sum to at most 2 |LSE|
# over a row: 6 per LSE.  KL adds both LSEs, the weights of acc / l1 (2)
# and the final sum and division (5): 12 + 2 + 5 = 19, taken as 20.
EXACT_SCORE_K = 20


@pytest.mark.parametrize("dt", ["bf16", "f32"])
@pytest.mark.parametrize("direction", [1, -1])
@pytest.mark.parametrize("causal", [False, True])
def test_fwd_raised_shifts_with_exact_scores(dt, direction, causal):
    """The shift-raising path with no score rounding in the way.  Every input
    is a multiple of 1/8 below 32 in magnitude (exact in bf16), so every
    product is a multiple of 1/64 and every dot product (|s| < 2^17) is exact
    in fp32, on both matrix-core paths.  Queries are 24 along axis 0 and keys
    climb (or fall) by 1/8 per key along it: the logits move by 3 per key,
    about 138 log2 units per 32-key block, so each block forces a raise of
    the running shift (or, falling, the first block's maximum holds).  The
    error left is the rounding of the shifts, rescales and finalisation,
    bounded by EXACT_SCORE_K 2^-24 |LSE| on top of the fp32 tolerance of
    1e-5 for both dtypes: about 1e-3 at |LSE| ~ 765, so a rescale of l or
    acc off by more than that fails (the earlier bounds for such logits were
    1e-2 in fp32 and 1.5 in bf16)."""
    g = torch.Generator(device="cpu").manual_seed(91)
    NQ, NK, d = 80, 256, 64
    ramp = torch.arange(NK, dtype=torch.float32) / 8.0
    if direction < 0:
        ramp = ramp.flip(0)

    def eighths(n, lim):
        return torch.randint(-lim, lim + 1, (n, d), generator=g).float() / 8.0

    def keys():
        k = eighths(NK, 8)
        k[:, 0] = ramp
        return k

    def queries():
        q = eighths(NQ, 8)
        q[:, 0] = 24.0
        return q

    q1, k1, q2, k2 = (x[None, None].to(DEV).to(DT[dt]).contiguous() for x in (queries(), keys(), queries(), keys()))
    for x in (q1, k1, q2, k2):   # the values survived the cast unchanged
        assert torch.equal(x.float().cpu() * 8, (x.float().cpu() * 8).round())
    kl, l1, l2, _ = run_and_compare(q1, k1, q2, k2, 1.0, causal, tag=f"exact ramp {direction}",
                                    by_magnitude=True, k=EXACT_SCORE_K, tol_dtype=torch.float32)
    assert l1.abs().max() > 500      # the logits really are far from unit scale


@pytest.mark.parametrize("shape", [(1, 16, 2048, 2048, 64), (2, 8, 1000, 1100, 128), (1, 24, 3000, 3000, 128),
                                   (1, 17, 500, 500, 64)],
                         ids=lambda s: "x".join(map(str, s)))
def test_fwd_longest_first_order_covers_every_row(shape):
    """The unsplit causal forward with fewer than 64 query blocks a head and
    whole heads per XCD takes its blocks longest first over each XCD's heads
    (2, 2, 3 and 2 heads per XCD here; the last grid, 34 workgroups, leaves
    its last two outside the eight XCD ranges, and those keep the head-major
    order).  Every row of every head against the oracle, so a workgroup that
    computed another head's block, or none, shows."""
    B, H, NQ, NK, d = shape
    q1, k1, q2, k2 = make_inputs(B, H, NQ, NK, d, torch.bfloat16, "student", 0.2, seed=NQ + H, device=DEV)
    kl, l1, l2 = ops.streamkl_fwd(q1, k1, q2, k2, d ** -0.5, True, splits=1)
    torch.cuda.synchronize()
    ref = oracle_heads(q1, k1, q2, k2, d ** -0.5, True, range(B * H))
    for hh in range(B * H):
        b, h = divmod(hh, H)
        for name, got in (("kl", kl), ("lse1", l1), ("lse2", l2)):
            check_rows(to64(got[b, h]), ref[hh][name], q1.dtype, f"longest-first head {hh} {name}")


def test_fwd_is_deterministic():
    q1, k1, q2, k2 = make_inputs(1, 4, 1024, 1024, 128, torch.bfloat16, "student", 0.2, seed=9, device=DEV)
    a = ops.streamkl_fwd(q1, k1, q2, k2, 0.09, True)
    b = ops.streamkl_fwd(q1, k1, q2, k2, 0.09, True)
    for x, y in zip(a, b):
        assert torch.equal(x, y)


def test_fwd_empty_rows_is_noop():
    q1, k1, q2, k2 = make_inputs(1, 2, 0, 16, 64, torch.bfloat16, "iid", 0, seed=1, device=DEV)
    kl, l1, l2 = ops.streamkl_fwd(q1, k1, q2, k2, 0.125, True)
    assert kl.numel() == 0
