"""GPU parity of the backward's partitioned halves, through the C ABI, against
the fp64 oracle and against the unpartitioned kernels: the key-partitioned
query gradients of short query blocks (each (query block, key partition)
workgroup stores a partial dq_t and a second kernel adds the partitions) and
the query-partitioned key gradients of small key grids with long query
streams (the same for dk_t)."""
import numpy as np
import pytest
import torch

from attention_distillation_kl_amd import _lib, make_inputs, ops
from attention_distillation_kl_amd.inputs import upstream_grad
from parity_util import check_grad, check_rows, log, oracle_heads, to64

pytestmark = pytest.mark.gpu

DEV = "cuda"
DT = {"bf16": torch.bfloat16, "f32": torch.float32}
NAMES = ("dq1", "dk1", "dq2", "dk2")


def partitions_used(q1, k1, causal, mask):
    """Whether the query half takes key partitions: its workspace (which
    streamkl_bwd_workspace_size covers) exceeds what the fused form needs."""
    B, H, NQ, d = q1.shape
    dt = _lib.BF16 if q1.dtype == torch.bfloat16 else _lib.F32
    ws = _lib.bwd_workspace_size(B, H, NQ, k1.shape[2], d, int(causal), dt, mask)
    if _lib.bwd_fused_selected(B, H, NQ, k1.shape[2], d, int(causal), dt, mask):
        return ws > _lib.bwd_fused_workspace_size(B, H, NQ, k1.shape[2], d, int(causal), dt, mask)
    return ws > 0


def two_kernel_backward(q1, k1, q2, k2, kl, l1, l2, g, scale, causal, mask):
    """streamkl_bwd_dk_ws, then streamkl_bwd_dq_ws with the backward's
    workspace: the two-kernel form, whichever form streamkl_bwd picks."""
    ws = ops.streamkl_bwd_workspace(q1, k1, causal, mask)
    dk = ops.streamkl_bwd_half("dk", q1, k1, q2, k2, kl, l1, l2, g, scale, causal, mask, workspace=ws)
    dq = ops.streamkl_bwd_half("dq", q1, k1, q2, k2, kl, l1, l2, g, scale, causal, mask, workspace=ws)
    return dq[0], dk[0], dq[1], dk[1]


# B, H, NQ, NK, d, dtype, causal, mask
CASES = [
    (1, 2, 64, 4096, 128, "bf16", True, 3),
    (1, 2, 64, 4096, 128, "bf16", False, 3),
    (1, 3, 1, 8192, 128, "bf16", False, 3),       # decoding row
    (2, 1, 100, 2000, 64, "f32", True, 3),
    (1, 2, 70, 3000, 64, "bf16", True, 1),
    (1, 2, 70, 3000, 128, "bf16", False, 2),
    (1, 1, 300, 777, 128, "bf16", True, 3),       # partitions of 4 tiles, ragged tail
]


@pytest.mark.parametrize("case", CASES, ids=lambda c: "x".join(map(str, c)))
def test_partitioned_query_gradients_match_oracle(case):
    B, H, NQ, NK, d, dt, causal, mask = case
    log(f"bwd split case {case}")
    q1, k1, q2, k2 = make_inputs(B, H, NQ, NK, d, DT[dt], "student", 0.4, seed=NQ + NK, device=DEV)
    assert partitions_used(q1, k1, causal, mask)
    scale = d ** -0.5
    g = upstream_grad(B, H, NQ, seed=NQ, device=DEV)
    kl, l1, l2 = ops.streamkl_fwd(q1, k1, q2, k2, scale, causal)
    grads = dict(zip(NAMES, two_kernel_backward(q1, k1, q2, k2, kl, l1, l2, g, scale, causal, mask)))
    torch.cuda.synchronize()
    ref = oracle_heads(q1, k1, q2, k2, scale, causal, range(B * H), g=g, grads=True)
    want = [n for n in NAMES if (mask & 1 and n.endswith("1")) or (mask & 2 and n.endswith("2"))]
    for hh in range(B * H):
        b, h = divmod(hh, H)
        check_rows(to64(kl[b, h]), ref[hh]["kl"], q1.dtype, f"{case} head {hh} kl")
        for n in want:
            check_grad(to64(grads[n][b, h]), ref[hh][n], q1.dtype, f"{case} head {hh} {n}")
    for n in NAMES:
        assert (grads[n] is None) == (n not in want)


def test_partitioned_query_gradients_are_deterministic_and_agree_with_one_partition():
    q1, k1, q2, k2 = make_inputs(1, 4, 128, 8192, 128, torch.bfloat16, "student", 0.2, seed=51, device=DEV)
    assert partitions_used(q1, k1, True, 3)
    kl, l1, l2 = ops.streamkl_fwd(q1, k1, q2, k2, 0.0884, True)
    a = ops.streamkl_bwd(q1, k1, q2, k2, kl, l1, l2, None, 0.0884, True)
    b = ops.streamkl_bwd(q1, k1, q2, k2, kl, l1, l2, None, 0.0884, True)
    one = ops.streamkl_bwd_half("dq", q1, k1, q2, k2, kl, l1, l2, None, 0.0884, True)  # never partitioned
    torch.cuda.synchronize()
    for x, y in zip(a, b):
        assert torch.equal(x, y)
    for x, y in zip((a[0], a[2]), one):
        rel = ((x.double() - y.double()).norm() / y.double().norm()).item()
        assert rel < 4e-3, rel  # bf16 rounding of two fp32 summation orders


# B, H, NQ, NK, d, causal, mask, partitioned, fused (the form streamkl_bwd picks)
HALF_CASES = [
    (1, 4, 128, 8192, 128, True, 3, True, False),
    (1, 2, 70, 3000, 64, True, 1, True, False),
    (1, 3, 1, 8192, 64, False, 3, True, True),      # decoding row
    (1, 2, 70, 3000, 128, False, 2, True, False),
    (2, 2, 33, 5000, 64, True, 1, True, True),
    (2, 2, 70, 5000, 64, True, 1, True, False),
    (2, 2, 33, 5000, 128, True, 1, True, True),
    (1, 32, 2048, 2048, 128, True, 3, False, False),
    (1, 8, 2048, 2048, 64, True, 3, True, False),     # C2: both halves partitioned
    (1, 8, 8192, 1024, 64, False, 3, True, False),    # the key half alone partitioned
    (1, 4, 1500, 1600, 128, True, 1, True, False),    # one gradient, unpaired key half
]


@pytest.mark.parametrize("case", HALF_CASES, ids=lambda c: "x".join(map(str, c)))
def test_halves_with_the_workspace_reproduce_streamkl_bwd(case):
    """streamkl_bwd_dk_ws then streamkl_bwd_dq_ws is streamkl_bwd, bit for bit,
    whether or not the sizes call for key partitions -- where streamkl_bwd
    keeps the two-kernel form.  Where it takes the fused form, it is
    streamkl_bwd_fused: the same key gradients bit for bit, query gradients
    equal up to the order of the atomic fp32 additions; the halves agree
    with it to bf16 rounding."""
    B, H, NQ, NK, d, causal, mask, partitioned, fused = case
    log(f"bwd halves with workspace {case}")
    q1, k1, q2, k2 = make_inputs(B, H, NQ, NK, d, torch.bfloat16, "student", 0.3, seed=NQ + 7, device=DEV)
    scale = d ** -0.5
    g = upstream_grad(B, H, NQ, seed=11, device=DEV)
    assert _lib.bwd_fused_selected(B, H, NQ, NK, d, int(causal), _lib.BF16, mask) == int(fused)
    assert partitions_used(q1, k1, causal, mask) == partitioned
    kl, l1, l2 = ops.streamkl_fwd(q1, k1, q2, k2, scale, causal)
    full = ops.streamkl_bwd(q1, k1, q2, k2, kl, l1, l2, g, scale, causal, mask)
    ws = ops.streamkl_bwd_workspace(q1, k1, causal, mask)
    assert (ws is not None) == (partitioned or fused)
    if ws is None:  # the entry point with an empty workspace, which these sizes allow
        ws = torch.empty(0, device=DEV, dtype=torch.uint8)
    dk = ops.streamkl_bwd_half("dk", q1, k1, q2, k2, kl, l1, l2, g, scale, causal, mask, workspace=ws)
    dq = ops.streamkl_bwd_half("dq", q1, k1, q2, k2, kl, l1, l2, g, scale, causal, mask, workspace=ws)
    halves = (dq[0], dk[0], dq[1], dk[1])
    if fused:
        direct = ops.streamkl_bwd_fused(q1, k1, q2, k2, kl, l1, l2, g, scale, causal, mask)
    torch.cuda.synchronize()
    for i, (got, want) in enumerate(zip(halves, full)):
        assert (got is None) == (want is None)
        if want is None:
            continue
        if not fused:
            assert torch.equal(got, want)
            continue
        if i % 2 == 1:   # key gradients: no atomics
            assert torch.equal(direct[i], want)
        else:
            rel = ((direct[i].double() - want.double()).norm() / want.double().norm().clamp_min(1e-30)).item()
            assert rel < 4e-3, rel
        rel = ((got.double() - want.double()).norm() / want.double().norm().clamp_min(1e-30)).item()
        assert rel < 4e-3, rel
    if partitioned:  # a workspace one granule short is refused, before anything is enqueued, by the
        # half whose partitions need all of it (the halves share the workspace)
        short = ws[: ws.numel() - 16]
        refused = 0
        for which in ("dk", "dq"):
            try:
                ops.streamkl_bwd_half(which, q1, k1, q2, k2, kl, l1, l2, g, scale, causal, mask, workspace=short)
            except _lib.StreamKLError as e:
                assert "STREAMKL_ERR_WORKSPACE" in str(e)
                refused += 1
        torch.cuda.synchronize()
        assert refused >= 1


# B, H, NQ, NK, d, dtype, causal, mask: small key grids whose key blocks
# stream many query tiles, so that streamkl_bwd cuts each key block's query
# range into partitions; ragged query and key tails, one or both gradients,
# the paired and the unpaired key layout, fp32.
DK_CASES = [
    (1, 8, 2048, 2048, 64, "bf16", True, 3),      # C2
    (1, 3, 2100, 2200, 128, "bf16", True, 3),
    (2, 2, 2500, 3000, 64, "bf16", False, 3),
    (1, 4, 2200, 2300, 128, "bf16", True, 1),
    (1, 4, 2200, 2300, 128, "bf16", True, 2),
    (1, 2, 1100, 1150, 128, "f32", True, 3),
    (1, 8, 8192, 1024, 64, "bf16", False, 3),
    (1, 1, 8192, 8192, 128, "bf16", True, 3),
]


def dk_partitioned(q1, k1, q2, k2, kl, l1, l2, g, scale, causal, mask):
    """The key half with and without the backward's workspace."""
    ws = ops.streamkl_bwd_workspace(q1, k1, causal, mask)
    assert ws is not None
    a = ops.streamkl_bwd_half("dk", q1, k1, q2, k2, kl, l1, l2, g, scale, causal, mask, workspace=ws)
    b = ops.streamkl_bwd_half("dk", q1, k1, q2, k2, kl, l1, l2, g, scale, causal, mask)
    return a, b


@pytest.mark.parametrize("case", DK_CASES, ids=lambda c: "x".join(map(str, c)))
def test_partitioned_key_gradients_match_oracle(case):
    B, H, NQ, NK, d, dt, causal, mask = case
    log(f"bwd key-partition case {case}")
    q1, k1, q2, k2 = make_inputs(B, H, NQ, NK, d, DT[dt], "student", 0.3, seed=NQ + 3 * NK, device=DEV)
    scale = d ** -0.5
    g = upstream_grad(B, H, NQ, seed=NK, device=DEV)
    kl, l1, l2 = ops.streamkl_fwd(q1, k1, q2, k2, scale, causal)
    full = dict(zip(NAMES, ops.streamkl_bwd(q1, k1, q2, k2, kl, l1, l2, g, scale, causal, mask)))
    (pk1, pk2), (uk1, uk2) = dk_partitioned(q1, k1, q2, k2, kl, l1, l2, g, scale, causal, mask)
    torch.cuda.synchronize()
    ref = oracle_heads(q1, k1, q2, k2, scale, causal, range(B * H), g=g, grads=True)
    want = [n for n in NAMES if (mask & 1 and n.endswith("1")) or (mask & 2 and n.endswith("2"))]
    for hh in range(B * H):
        b, h = divmod(hh, H)
        for n in want:
            check_grad(to64(full[n][b, h]), ref[hh][n], q1.dtype, f"{case} head {hh} {n}")
    # streamkl_bwd's key gradients are the partitioned half's, bit for bit,
    # and differ from the unpartitioned half's only by summation order.
    for got, one, n in ((pk1, uk1, "dk1"), (pk2, uk2, "dk2")):
        if n not in want:
            assert got is None and one is None
            continue
        assert torch.equal(got, full[n])
        assert not torch.equal(got, one), f"{case}: {n} not partitioned"
        rel = ((got.double() - one.double()).norm() / one.double().norm().clamp_min(1e-30)).item()
        assert rel < (1e-5 if q1.dtype == torch.float32 else 4e-3), rel


def test_partitioned_key_gradients_are_deterministic():
    q1, k1, q2, k2 = make_inputs(1, 8, 2048, 2048, 64, torch.bfloat16, "student", 0.3, seed=61, device=DEV)
    kl, l1, l2 = ops.streamkl_fwd(q1, k1, q2, k2, 0.125, True)
    a = ops.streamkl_bwd(q1, k1, q2, k2, kl, l1, l2, None, 0.125, True)
    b = ops.streamkl_bwd(q1, k1, q2, k2, kl, l1, l2, None, 0.125, True)
    (pk1, pk2), (uk1, uk2) = dk_partitioned(q1, k1, q2, k2, kl, l1, l2, None, 0.125, True, 3)
    torch.cuda.synchronize()
    for x, y in zip(a, b):
        assert torch.equal(x, y)
    # the partitions are taken: a different summation order than one partition
    assert not (torch.equal(pk1, uk1) and torch.equal(pk2, uk2))
