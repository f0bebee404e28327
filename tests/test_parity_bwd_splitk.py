"""GPU parity of the backward's key-partitioned query gradients (short query
blocks: each (query block, key partition) workgroup stores a partial dq_t and
a second kernel adds the partitions), through the C ABI, against the fp64
oracle and against the unpartitioned query-gradient kernel."""
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
    B, H, NQ, d = q1.shape
    dt = _lib.BF16 if q1.dtype == torch.bfloat16 else _lib.F32
    return _lib.bwd_workspace_size(B, H, NQ, k1.shape[2], d, int(causal), dt, mask) > 0


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
    grads = dict(zip(NAMES, ops.streamkl_bwd(q1, k1, q2, k2, kl, l1, l2, g, scale, causal, mask)))
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


# B, H, NQ, NK, d, causal, mask, partitioned
HALF_CASES = [
    (1, 4, 128, 8192, 128, True, 3, True),
    (1, 2, 70, 3000, 64, True, 1, True),
    (1, 3, 1, 8192, 64, False, 3, True),      # decoding row
    (1, 2, 70, 3000, 128, False, 2, True),
    (2, 2, 33, 5000, 64, True, 1, True),
    (1, 32, 2048, 2048, 128, True, 3, False),
]


@pytest.mark.parametrize("case", HALF_CASES, ids=lambda c: "x".join(map(str, c)))
def test_halves_with_the_workspace_reproduce_streamkl_bwd(case):
    """streamkl_bwd_dk then streamkl_bwd_dq_ws is streamkl_bwd, bit for bit,
    whether or not the sizes call for key partitions."""
    B, H, NQ, NK, d, causal, mask, partitioned = case
    log(f"bwd halves with workspace {case}")
    q1, k1, q2, k2 = make_inputs(B, H, NQ, NK, d, torch.bfloat16, "student", 0.3, seed=NQ + 7, device=DEV)
    scale = d ** -0.5
    g = upstream_grad(B, H, NQ, seed=11, device=DEV)
    kl, l1, l2 = ops.streamkl_fwd(q1, k1, q2, k2, scale, causal)
    full = ops.streamkl_bwd(q1, k1, q2, k2, kl, l1, l2, g, scale, causal, mask)
    ws = ops.streamkl_bwd_workspace(q1, k1, causal, mask)
    assert (ws is not None) == partitioned
    if ws is None:  # the entry point with an empty workspace, which these sizes allow
        ws = torch.empty(0, device=DEV, dtype=torch.uint8)
    dk = ops.streamkl_bwd_half("dk", q1, k1, q2, k2, kl, l1, l2, g, scale, causal, mask)
    dq = ops.streamkl_bwd_half("dq", q1, k1, q2, k2, kl, l1, l2, g, scale, causal, mask, workspace=ws)
    torch.cuda.synchronize()
    for got, want in zip((dq[0], dk[0], dq[1], dk[1]), full):
        assert (got is None) == (want is None)
        if want is not None:
            assert torch.equal(got, want)
    if partitioned:  # a workspace one granule short is refused before anything is enqueued
        short = ws[: ws.numel() - 16]
        with pytest.raises(_lib.StreamKLError, match="STREAMKL_ERR_WORKSPACE"):
            ops.streamkl_bwd_half("dq", q1, k1, q2, k2, kl, l1, l2, g, scale, causal, mask, workspace=short)
