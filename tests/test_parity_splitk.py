"""GPU parity of the split-K forward (key dimension partitioned over
workgroups, partition states merged by a second kernel), through the C ABI,
against the fp64 oracle and against the unsplit kernel."""
import numpy as np
import pytest
import torch

from attention_distillation_kl_amd import WORKLOADS, _lib, make_inputs, ops
from parity_util import check_rows, log, oracle_heads, to64

pytestmark = pytest.mark.gpu

DEV = "cuda"
DT = {"bf16": torch.bfloat16, "f32": torch.float32}


def splitk_raw(q1, k1, q2, k2, scale, causal, splits):
    """streamkl_fwd_splitk with an explicit split count (workspace from torch)."""
    B, H, NQ, d = q1.shape
    NK = k1.shape[2]
    dt = _lib.BF16 if q1.dtype == torch.bfloat16 else _lib.F32
    kl = torch.empty(B, H, NQ, device=DEV, dtype=torch.float32)
    l1, l2 = torch.empty_like(kl), torch.empty_like(kl)
    wsb = _lib.fwd_workspace_size(B, H, NQ, NK, d, int(causal), dt, splits)
    ws = torch.empty(max(1, wsb // 4), device=DEV, dtype=torch.float32) if wsb else None
    st = _lib.fwd_splitk(q1.data_ptr(), k1.data_ptr(), q2.data_ptr(), k2.data_ptr(), B, H, NQ, NK, d,
                         scale, int(causal), dt, splits, kl.data_ptr(), l1.data_ptr(), l2.data_ptr(),
                         None if ws is None else ws.data_ptr(), wsb,
                         torch.cuda.current_stream().cuda_stream)
    assert st == _lib.OK, _lib.status_str(st)
    torch.cuda.synchronize()
    return kl, l1, l2


# B, H, NQ, NK, d, dtype, causal, splits: ragged tails, partitions that end
# inside a tile range, more partitions than key tiles (empty partitions), and
# causal rows whose frontier ends before some partitions start.
CASES = [
    (1, 2, 100, 1000, 128, "bf16", True, 3),
    (1, 2, 100, 1000, 128, "bf16", False, 5),
    (2, 1, 65, 333, 64, "f32", True, 2),
    (1, 1, 37, 130, 128, "f32", False, 7),
    (1, 2, 17, 63, 64, "bf16", True, 4),       # one key tile, four partitions
    (1, 3, 1, 4096, 128, "bf16", False, 16),   # decoding: one query row
    (1, 2, 64, 3000, 128, "bf16", True, 6),    # rows for two waves, ragged key tail
    (1, 1, 257, 2048, 64, "bf16", True, 9),
    (1, 1, 5, 20, 128, "bf16", False, 2),      # under 32 keys: one wave of each pair scores none
    (1, 2, 20, 20, 128, "bf16", True, 3),      # the same, causal, with empty partitions
    (1, 2, 40, 3000, 64, "bf16", True, 33),    # the merge's widest lane group, 31 lanes without a partition
    (1, 2, 3, 5000, 128, "bf16", False, 1024), # the most partitions: lanes take several, 945 are empty
]


@pytest.mark.parametrize("case", CASES, ids=lambda c: "x".join(map(str, c)))
def test_splitk_matches_oracle(case):
    B, H, NQ, NK, d, dt, causal, splits = case
    log(f"splitk case {case}")
    q1, k1, q2, k2 = make_inputs(B, H, NQ, NK, d, DT[dt], "student", 0.3, seed=40 + NQ, device=DEV)
    scale = d ** -0.5
    kl, l1, l2 = splitk_raw(q1, k1, q2, k2, scale, causal, splits)
    ref = oracle_heads(q1, k1, q2, k2, scale, causal, range(B * H))
    for hh in range(B * H):
        b, h = divmod(hh, H)
        for name, got in (("kl", kl), ("lse1", l1), ("lse2", l2)):
            check_rows(to64(got[b, h]), ref[hh][name], q1.dtype, f"{case} head {hh} {name}")


@pytest.mark.parametrize("causal", [False, True])
def test_one_partition_is_the_unsplit_kernel_bit_for_bit(causal):
    q1, k1, q2, k2 = make_inputs(1, 4, 700, 900, 128, torch.bfloat16, "student", 0.2, seed=41, device=DEV)
    a = ops.streamkl_fwd(q1, k1, q2, k2, 0.09, causal, splits=1)
    b = splitk_raw(q1, k1, q2, k2, 0.09, causal, 1)
    for x, y in zip(a, b):
        assert torch.equal(x, y)


def test_partition_count_changes_only_rounding():
    """Different partitionings are different summation orders of the same
    exact merge: they agree far inside the oracle tolerance."""
    q1, k1, q2, k2 = make_inputs(1, 2, 300, 5000, 128, torch.bfloat16, "student", 0.2, seed=42, device=DEV)
    base = splitk_raw(q1, k1, q2, k2, 0.0884, True, 1)
    for s in (2, 3, 8, 40, 100):
        got = splitk_raw(q1, k1, q2, k2, 0.0884, True, s)
        for x, y, name in zip(got, base, ("kl", "lse1", "lse2")):
            err = (x.double() - y.double()).abs().max().item()
            assert err < 2e-5, f"splits={s} {name}: max |diff| {err}"


@pytest.mark.parametrize("case", [(1, 8, 4096, 4096, 64, 8), (2, 3, 3000, 3100, 128, 16), (1, 5, 2500, 2500, 64, 40)],
                         ids=lambda c: "x".join(map(str, c)))
def test_causal_partitions_in_rank_major_order(case):
    """Causal grids with partitions of more than one round of workgroups take
    the rank-major order, each query block's own range cut into runs of equal
    length: every row of every head against the oracle (40 partitions leave
    the short blocks' last runs empty)."""
    B, H, NQ, NK, d, splits = case
    log(f"causal rank-major partitions {case}")
    assert ((NQ + 255) // 256) * B * H * splits > 2 * 256  # more than one round: the rank-major order
    q1, k1, q2, k2 = make_inputs(B, H, NQ, NK, d, torch.bfloat16, "student", 0.3, seed=NQ + splits, device=DEV)
    scale = d ** -0.5
    kl, l1, l2 = splitk_raw(q1, k1, q2, k2, scale, True, splits)
    one = splitk_raw(q1, k1, q2, k2, scale, True, 1)
    ref = oracle_heads(q1, k1, q2, k2, scale, True, range(B * H))
    for hh in range(B * H):
        b, h = divmod(hh, H)
        for name, got in (("kl", kl), ("lse1", l1), ("lse2", l2)):
            check_rows(to64(got[b, h]), ref[hh][name], q1.dtype, f"{case} head {hh} {name}")
    for x, y, name in zip((kl, l1, l2), one, ("kl", "lse1", "lse2")):
        err = (x.double() - y.double()).abs().max().item()
        assert err < 2e-5, f"{case} {name}: max |diff| against one partition {err}"


def test_default_partitioning():
    """Short query blocks over long keys are split; full grids are not."""
    c4, h = WORKLOADS["c4"], WORKLOADS["h32k"]
    assert _lib.fwd_splits(c4.B, c4.H, c4.NQ, c4.NK, c4.d, 0, _lib.BF16) > 1
    assert _lib.fwd_splits(h.B, h.H, h.NQ, h.NK, h.d, 1, _lib.BF16) == 1
    assert _lib.fwd_splits(1, 8, 1, 65536, 128, 0, _lib.BF16) > 1


def test_decoding_row_over_64k_keys():
    """N_Q = 1 (autoregressive decoding): one row per head, 64K keys."""
    q1, k1, q2, k2 = make_inputs(1, 4, 1, 65536, 128, torch.bfloat16, "student", 0.2, seed=43, device=DEV)
    kl, l1, l2 = ops.streamkl_fwd(q1, k1, q2, k2, 128 ** -0.5, True)
    torch.cuda.synchronize()
    ref = oracle_heads(q1, k1, q2, k2, 128 ** -0.5, True, range(4))
    for hh in range(4):
        for name, got in (("kl", kl), ("lse1", l1), ("lse2", l2)):
            check_rows(to64(got[0, hh]), ref[hh][name], q1.dtype, f"decode head {hh} {name}")
