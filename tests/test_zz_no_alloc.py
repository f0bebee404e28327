"""The forward entry point that allocates nothing (streamkl_fwd_splitk_noalloc)
against the split-K forward with a caller's workspace (streamkl_fwd_splitk),
through the C ABI.

Both run the same kernels with the same partition count, so the results must
agree bit for bit.  Each case makes two calls in a row on the one scratch
array of the GPU, the second on a smaller input, so a call that read states
left over from the one before would show.
"""
import math

import pytest
import torch

from attention_distillation_kl_amd import _lib, make_inputs
from parity_util import log

pytestmark = pytest.mark.gpu

DEV = "cuda"


def _outs(B, H, NQ):
    kl = torch.full((B, H, NQ), float("nan"), device=DEV, dtype=torch.float32)
    return kl, torch.full_like(kl, float("nan")), torch.full_like(kl, float("nan"))


def _stream():
    return torch.cuda.current_stream().cuda_stream


def _call_noalloc(q1, k1, q2, k2, scale, causal, splits):
    B, H, NQ, d = q1.shape
    NK = k1.shape[2]
    kl, l1, l2 = _outs(B, H, NQ)
    dt = _lib.BF16 if q1.dtype == torch.bfloat16 else _lib.F32
    before = torch.cuda.memory_allocated()
    st = _lib.fwd_splitk_noalloc(q1.data_ptr(), k1.data_ptr(), q2.data_ptr(), k2.data_ptr(), B, H, NQ, NK, d,
                                 scale, int(causal), dt, splits, kl.data_ptr(), l1.data_ptr(), l2.data_ptr(),
                                 _stream())
    assert st == _lib.OK, _lib.status_str(st)
    assert torch.cuda.memory_allocated() == before   # nothing taken from torch's allocator either
    return kl, l1, l2


def _call_workspace(q1, k1, q2, k2, scale, causal, splits):
    B, H, NQ, d = q1.shape
    NK = k1.shape[2]
    kl, l1, l2 = _outs(B, H, NQ)
    dt = _lib.BF16 if q1.dtype == torch.bfloat16 else _lib.F32
    nbytes = _lib.fwd_workspace_size(B, H, NQ, NK, d, int(causal), dt, splits)
    ws = torch.empty(max(1, nbytes // 4), device=DEV, dtype=torch.float32)
    st = _lib.fwd_splitk(q1.data_ptr(), k1.data_ptr(), q2.data_ptr(), k2.data_ptr(), B, H, NQ, NK, d, scale,
                         int(causal), dt, splits, kl.data_ptr(), l1.data_ptr(), l2.data_ptr(), ws.data_ptr(),
                         nbytes, _stream())
    assert st == _lib.OK, _lib.status_str(st)
    return kl, l1, l2


# (first call, second smaller call): B, H, N_Q, N_K, d, dtype, causal
CASES = [
    ((1, 32, 1, 65536, 128, torch.bfloat16, False), (1, 8, 1, 4000, 128, torch.bfloat16, False)),
    ((1, 4, 300, 5000, 128, torch.bfloat16, True), (1, 2, 70, 900, 128, torch.bfloat16, True)),
    ((2, 2, 64, 3000, 64, torch.bfloat16, False), (1, 1, 17, 700, 64, torch.bfloat16, True)),
    ((1, 2, 200, 2000, 128, torch.float32, False), (1, 1, 33, 400, 128, torch.float32, True)),
]


@pytest.mark.parametrize("first,second", CASES, ids=lambda c: "x".join(str(v) for v in c[:5]))
def test_noalloc_matches_the_workspace_entry_point(first, second):
    for i, (B, H, NQ, NK, d, dt, causal) in enumerate((first, second)):
        log(f"noalloc call {i}: {(B, H, NQ, NK, d, dt, causal)}")
        q1, k1, q2, k2 = make_inputs(B, H, NQ, NK, d, dt, "student", 0.3, seed=NQ + 7 * NK, device=DEV)
        scale = 1.0 / math.sqrt(d)
        splits = _lib.fwd_splits(B, H, NQ, NK, d, int(causal), _lib.BF16 if dt == torch.bfloat16 else _lib.F32)
        assert splits > 1, "the case must take the partitioned path"
        need = _lib.fwd_workspace_size(B, H, NQ, NK, d, int(causal), 1, splits)
        assert 0 < need <= _lib.NOALLOC_SCRATCH_BYTES
        got = _call_noalloc(q1, k1, q2, k2, scale, causal, splits)
        torch.cuda.synchronize()
        ref = _call_workspace(q1, k1, q2, k2, scale, causal, splits)
        torch.cuda.synchronize()
        for name, a, b in zip(("kl", "lse1", "lse2"), got, ref):
            assert torch.isfinite(a).all(), name
            assert torch.equal(a, b), name


def test_noalloc_with_one_partition_is_the_plain_forward():
    q1, k1, q2, k2 = make_inputs(1, 2, 130, 700, 128, torch.bfloat16, "student", 0.3, seed=3, device=DEV)
    got = _call_noalloc(q1, k1, q2, k2, 0.09, True, 1)
    ref = _call_workspace(q1, k1, q2, k2, 0.09, True, 1)
    torch.cuda.synchronize()
    for a, b in zip(got, ref):
        assert torch.equal(a, b)


def test_noalloc_rejects_states_beyond_its_scratch():
    """5 * splits * B * H * N_Q floats must fit the fixed array; larger
    problems are refused before anything is enqueued."""
    B, H, NQ, NK, d = 1, 32, 2048, 65536, 128
    splits = 64
    assert _lib.fwd_workspace_size(B, H, NQ, NK, d, 0, _lib.BF16, splits) > _lib.NOALLOC_SCRATCH_BYTES
    q = torch.empty(16, device=DEV, dtype=torch.bfloat16)
    kl = torch.empty(16, device=DEV, dtype=torch.float32)
    st = _lib.fwd_splitk_noalloc(q.data_ptr(), q.data_ptr(), q.data_ptr(), q.data_ptr(), B, H, NQ, NK, d, 0.1, 0,
                                 _lib.BF16, splits, kl.data_ptr(), kl.data_ptr(), kl.data_ptr(), _stream())
    assert st == _lib.ERR_WORKSPACE
