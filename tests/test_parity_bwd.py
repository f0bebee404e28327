"""GPU backward parity: dQ1, dK1, dQ2, dK2 from the recompute kernels (through
the C ABI) against the fp64 oracle, plus properties that hold at any size."""
import math

import numpy as np
import pytest
import torch

from attention_distillation_kl_amd import WORKLOADS, make_inputs, workload_inputs
from attention_distillation_kl_amd import _lib, ops
from attention_distillation_kl_amd.inputs import upstream_grad
import oracle
from parity_util import (check_grad, check_rows, head64, log, oracle_heads, oracle_row_blocks, to64)

pytestmark = pytest.mark.gpu

DEV = "cuda"
DT = {"bf16": torch.bfloat16, "f32": torch.float32}
NAMES = ("dq1", "dk1", "dq2", "dk2")


def fwd_bwd(q1, k1, q2, k2, scale, causal, g=None, mask=3):
    kl, l1, l2 = ops.streamkl_fwd(q1, k1, q2, k2, scale, causal)
    grads = ops.streamkl_bwd(q1, k1, q2, k2, kl, l1, l2, g, scale, causal, mask)
    torch.cuda.synchronize()
    return (kl, l1, l2), dict(zip(NAMES, grads))


def compare_all_heads(q1, k1, q2, k2, scale, causal, g=None, tag=""):
    (kl, l1, l2), gr = fwd_bwd(q1, k1, q2, k2, scale, causal, g)
    B, H = q1.shape[:2]
    ref = oracle_heads(q1, k1, q2, k2, scale, causal, range(B * H), g=g, grads=True)
    worst = 0.0
    for hh in range(B * H):
        b, h = divmod(hh, H)
        check_rows(to64(kl[b, h]), ref[hh]["kl"], q1.dtype, f"{tag} head {hh} kl")
        for n in NAMES:
            worst = max(worst, check_grad(to64(gr[n][b, h]), ref[hh][n], q1.dtype, f"{tag} head {hh} {n}"))
    return gr, worst


SHAPES = [
    # B, H, NQ, NK, d, dtype, causal
    (1, 1, 1, 1, 64, "bf16", True),
    (1, 1, 2, 3, 128, "f32", False),
    (1, 2, 17, 63, 128, "bf16", True),
    (2, 1, 65, 65, 64, "f32", True),
    (1, 2, 129, 65, 64, "bf16", False),
    (1, 2, 257, 257, 128, "bf16", True),
    (1, 2, 300, 333, 64, "bf16", True),
    (1, 1, 300, 333, 128, "f32", True),
    (1, 2, 333, 300, 128, "bf16", False),
    (1, 1, 513, 1000, 128, "bf16", True),
    (1, 1, 640, 129, 64, "f32", False),
]


@pytest.mark.parametrize("shape", SHAPES, ids=lambda s: "x".join(map(str, s)))
def test_bwd_ragged_shapes(shape):
    B, H, NQ, NK, d, dt, causal = shape
    log(f"bwd ragged {shape}")
    q1, k1, q2, k2 = make_inputs(B, H, NQ, NK, d, DT[dt], "student", 0.5, seed=NQ * 3 + NK, device=DEV)
    compare_all_heads(q1, k1, q2, k2, 1.0 / math.sqrt(d), causal, tag=str(shape))


@pytest.mark.parametrize("dt", ["bf16", "f32"])
@pytest.mark.parametrize("causal", [False, True])
def test_bwd_upstream_gradient(dt, causal):
    """A random per-row upstream gradient with both signs and exact zeros."""
    log(f"bwd upstream g {dt} causal={causal}")
    q1, k1, q2, k2 = make_inputs(1, 2, 200, 230, 128, DT[dt], "student", 0.4, seed=11, device=DEV)
    g = upstream_grad(1, 2, 200, seed=11, device=DEV)
    compare_all_heads(q1, k1, q2, k2, 0.1, causal, g=g, tag="upstream")


def test_bwd_c2_full():
    w = WORKLOADS["c2"]
    log("bwd c2 full")
    q1, k1, q2, k2 = workload_inputs(w, DEV)
    compare_all_heads(q1, k1, q2, k2, w.scale, w.causal, tag="c2")


@pytest.mark.parametrize("d,causal", [(128, True), (64, True), (128, False)])
@pytest.mark.parametrize("mask", [1, 2])
def test_bwd_single_configuration_masks(mask, d, causal):
    """grad_mask = 1 (Configuration 2) / 2 (Configuration 1) produce exactly the
    corresponding tensors of the full backward and leave the others alone.
    (In bf16 the full backward's key gradients come from the paired kernel,
    the single ones from the unpaired kernel: both add the streamed blocks in
    the same order.)"""
    q1, k1, q2, k2 = make_inputs(1, 2, 300, 300, d, torch.bfloat16, "student", 0.3, seed=12, device=DEV)
    _, full = fwd_bwd(q1, k1, q2, k2, 0.09, causal)
    _, part = fwd_bwd(q1, k1, q2, k2, 0.09, causal, mask=mask)
    keep = ("dq1", "dk1") if mask == 1 else ("dq2", "dk2")
    for n in NAMES:
        if n in keep:
            assert torch.equal(part[n], full[n]), n
        else:
            assert part[n] is None


def test_bwd_single_configuration_masks_on_a_large_grid():
    """16 heads of 8192 causal tokens: the key-gradient role takes its
    unpaired layout (256-key workgroups, at least two rounds of them, long
    query streams).  Each single configuration must still give the full
    backward's tensors bit for bit, and one head is checked against the
    oracle."""
    B, H, N, d = 1, 16, 8192, 128
    q1, k1, q2, k2 = make_inputs(B, H, N, N, d, torch.bfloat16, "student", 0.2, seed=18, device=DEV)
    scale = d ** -0.5
    _, full = fwd_bwd(q1, k1, q2, k2, scale, True)
    for mask, keep in ((1, ("dq1", "dk1")), (2, ("dq2", "dk2"))):
        _, part = fwd_bwd(q1, k1, q2, k2, scale, True, mask=mask)
        for n in keep:
            assert torch.equal(part[n], full[n]), (mask, n)
    hh = H - 1
    ref = oracle_heads(q1, k1, q2, k2, scale, True, [hh], grads=True)[hh]
    for n in NAMES:
        check_grad(to64(full[n][0, hh]), ref[n], q1.dtype, f"16x8192 head {hh} {n}")


@pytest.mark.parametrize("shape", [(1, 16, 2048, 2048, 128, True), (1, 32, 4096, 4096, 64, False),
                                   (1, 36, 2048, 2048, 64, False)],
                         ids=lambda s: "x".join(map(str, s)))
def test_bwd_longest_first_order_covers_every_head(shape):
    """Causal grids whose backward kernels take their blocks longest first:
    over each XCD's heads for 16 heads x 2K tokens in the paired key-gradient
    kernel (32 blocks a head, 64 resident per XCD; its query gradients go by
    key partitions) and 32 heads x 4K tokens in the query-gradient kernel (16
    blocks a head, 32 resident, not partitioned); over the whole grid (rank
    major) for 36 heads x 2K tokens in both kernels (more than one round, and
    4.5 heads per XCD).  All four gradients of every head against the
    oracle."""
    B, H, NQ, NK, d, dq_partitioned = shape
    assert (_lib.bwd_workspace_size(B, H, NQ, NK, d, 1, _lib.BF16, 3) > 0) == dq_partitioned
    q1, k1, q2, k2 = make_inputs(B, H, NQ, NK, d, torch.bfloat16, "student", 0.2, seed=H + d, device=DEV)
    compare_all_heads(q1, k1, q2, k2, d ** -0.5, True, tag=f"longest-first {shape}")


@pytest.mark.parametrize("dt", ["bf16", "f32"])
def test_bwd_identical_teacher_student_gives_zero_gradients(dt):
    q, k, _, _ = make_inputs(1, 2, 150, 150, 64, DT[dt], "iid", 0, seed=13, device=DEV)
    _, gr = fwd_bwd(q, k, q, k, 0.125, True)
    for n in NAMES:
        assert torch.count_nonzero(gr[n]) == 0, n


def test_bwd_is_deterministic():
    q1, k1, q2, k2 = make_inputs(1, 4, 1000, 1000, 128, torch.bfloat16, "student", 0.2, seed=14, device=DEV)
    _, a = fwd_bwd(q1, k1, q2, k2, 0.09, True)
    _, b = fwd_bwd(q1, k1, q2, k2, 0.09, True)
    for n in NAMES:
        assert torch.equal(a[n], b[n]), n


def test_bwd_no_queries_gives_zero_key_gradients():
    q1, k1, q2, k2 = make_inputs(1, 2, 0, 70, 128, torch.bfloat16, "iid", 0, seed=15, device=DEV)
    kl, l1, l2 = ops.streamkl_fwd(q1, k1, q2, k2, 0.1, False)
    dq1, dk1, dq2, dk2 = ops.streamkl_bwd(q1, k1, q2, k2, kl, l1, l2, None, 0.1, False)
    torch.cuda.synchronize()
    assert torch.count_nonzero(dk1) == 0 and torch.count_nonzero(dk2) == 0


def identities(q1, k1, q2, k2, gr, tag):
    """sum_j dK_t[j] = 0 and sum_i <dQ_t, q_t> = sum_j <dK_t, k_t> per head,
    to the bf16 gradient tolerance."""
    for t, (q, k) in ((1, (q1, k1)), (2, (q2, k2))):
        dq, dk = gr[f"dq{t}"].double(), gr[f"dk{t}"].double()
        s = dk.sum(dim=2)                                       # [B, H, d]
        scale_ref = dk.pow(2).sum(dim=(2, 3)).sqrt()            # ||dK||_F per head
        assert (s.norm(dim=-1) <= 2e-2 * scale_ref + 1e-6).all(), f"{tag}: sum_j dK{t} not ~0"
        lhs = (dq * q.double()).sum(dim=(2, 3))
        rhs = (dk * k.double()).sum(dim=(2, 3))
        mag = (dq.abs() * q.double().abs()).sum(dim=(2, 3))
        assert ((lhs - rhs).abs() <= 2e-2 * mag + 1e-6).all(), f"{tag}: <dQ{t},Q{t}> != <dK{t},K{t}>"


@pytest.mark.parametrize("name", ["c3", "c5", "h32k"])
def test_bwd_full_size(name):
    """Full-size workloads in the benchmark's launch configuration.

    The last head is compared whole with the oracle: KL, LSE1, LSE2 per row
    and dQ1, dK1, dQ2, dK2 per (b, h) slice, and separately the key gradients
    of the first 2048 keys, which (causal) take the longest query streams:
    key block 0 accumulates over every query of the head.  The first head is
    checked on its first and last query rows (dQ) and, causally, the last
    keys (dK, reached only by the last rows); the rest of the batch is held to
    identities that hold at any size.  The whole head costs the oracle about
    10 s at 32K tokens and 40 s at 64K on 16 cores."""
    w = WORKLOADS[name]
    log(f"bwd {name} full size")
    q1, k1, q2, k2 = workload_inputs(w, DEV)
    (kl, l1, l2), gr = fwd_bwd(q1, k1, q2, k2, w.scale, w.causal)
    for n in NAMES:
        assert torch.isfinite(gr[n]).all(), n
    identities(q1, k1, q2, k2, gr, name)
    nh = w.B * w.H
    tail = 32
    hh = 0
    b, h = divmod(hh, w.H)
    h64 = head64(q1, k1, q2, k2, hh)
    # last rows: exact dQ for them and, causally, exact dK for the last keys
    ref = oracle_row_blocks(h64, w.scale, w.causal, [(w.NQ - tail, w.NQ)], grads=True)
    for t in (1, 2):
        check_grad(to64(gr[f"dq{t}"][b, h])[-tail:], ref[f"dq{t}"][-tail:], q1.dtype, f"{name} h{hh} dq{t} tail")
        check_grad(to64(gr[f"dk{t}"][b, h])[-tail:], ref[f"dk{t}"][-tail:], q1.dtype, f"{name} h{hh} dk{t} tail")
    ref = oracle_row_blocks(h64, w.scale, w.causal, [(0, tail)], grads=True)
    for t in (1, 2):
        check_grad(to64(gr[f"dq{t}"][b, h])[:tail], ref[f"dq{t}"][:tail], q1.dtype, f"{name} h{hh} dq{t} head")
    check_rows(to64(kl[b, h])[:tail], ref["kl"][:tail], q1.dtype, f"{name} h{hh} kl")
    # the last head, whole
    hh = nh - 1
    b, h = divmod(hh, w.H)
    log(f"bwd {name}: oracle on head {hh}, all {w.NQ} rows")
    ref = oracle.head(*head64(q1, k1, q2, k2, hh), w.scale, w.causal, grads=True)
    for key, got in (("kl", kl), ("lse1", l1), ("lse2", l2)):
        check_rows(to64(got[b, h]), ref[key], q1.dtype, f"{name} h{hh} {key} (whole head)")
    for n in NAMES:
        check_grad(to64(gr[n][b, h]), ref[n], q1.dtype, f"{name} h{hh} {n} (whole head)")
    for t in (1, 2):
        first = min(2048, w.NK)
        check_grad(to64(gr[f"dk{t}"][b, h])[:first], ref[f"dk{t}"][:first], q1.dtype,
                   f"{name} h{hh} dk{t} first {first} keys")
    del q1, k1, q2, k2, gr
    torch.cuda.empty_cache()


def test_autograd_function_matches_direct_calls():
    q1, k1, q2, k2 = make_inputs(1, 2, 128, 160, 64, torch.bfloat16, "student", 0.3, seed=16, device=DEV)
    xs = [t.clone().requires_grad_(True) for t in (q1, k1, q2, k2)]
    kl, l1, l2 = ops.kl(*xs, scale=0.125, causal=True)
    w = torch.linspace(-1, 1, kl.numel(), device=DEV).reshape(kl.shape)
    (kl * w).sum().backward()
    kl_d, l1_d, l2_d = ops.streamkl_fwd(q1, k1, q2, k2, 0.125, True)
    grads = ops.streamkl_bwd(q1, k1, q2, k2, kl_d, l1_d, l2_d, w, 0.125, True)
    assert torch.equal(kl.detach(), kl_d)
    for x, gd in zip(xs, grads):
        assert torch.equal(x.grad, gd)


def test_bwd_halves_match_full_backward():
    """streamkl_bwd == streamkl_bwd_dk then streamkl_bwd_dq, bit for bit, when
    it needs no workspace (no key partitions for the query gradients)."""
    q1, k1, q2, k2 = make_inputs(1, 2, 260, 300, 128, torch.bfloat16, "student", 0.3, seed=17, device=DEV)
    assert _lib.bwd_workspace_size(1, 2, 260, 300, 128, 1, _lib.BF16, 3) == 0
    g = upstream_grad(1, 2, 260, seed=17, device=DEV)
    kl, l1, l2 = ops.streamkl_fwd(q1, k1, q2, k2, 0.1, True)
    full = ops.streamkl_bwd(q1, k1, q2, k2, kl, l1, l2, g, 0.1, True)
    dk1, dk2 = ops.streamkl_bwd_half("dk", q1, k1, q2, k2, kl, l1, l2, g, 0.1, True)
    dq1, dq2 = ops.streamkl_bwd_half("dq", q1, k1, q2, k2, kl, l1, l2, g, 0.1, True)
    torch.cuda.synchronize()
    for a, b in zip(full, (dq1, dk1, dq2, dk2)):
        assert torch.equal(a, b)
