"""Heads whose key rows span more than 4 GiB (bf16, d = 128: more than 2^24
keys), where byte offsets within one head no longer fit in 32 bits.

The oracle cannot afford rows of 17M keys, so the check uses an identity that
holds at any size: tiling a key set R times along the keys divides every
probability by R.  Then KL and dQ are those of the untiled problem, each LSE
grows by ln R, and each copy of key j receives dK_j / R.  R is a power of two,
so multiplying a copy's bf16 gradient by R is exact.  The untiled problem is
itself checked against the oracle.
"""
import math

import pytest
import torch

from attention_distillation_kl_amd import make_inputs, ops
from attention_distillation_kl_amd.inputs import upstream_grad
from parity_util import check_grad, check_rows, log, oracle_heads, to64

pytestmark = pytest.mark.gpu

DEV = "cuda"
NAMES = ("dq1", "dk1", "dq2", "dk2")


def test_key_rows_beyond_4gib_by_the_tiling_identity():
    NQ, N0, d, R = 64, 4129, 128, 4096
    NK = N0 * R  # 16,912,384 keys: 4.33 GB per key tensor
    assert NK * d * 2 > 2 ** 32
    bf16 = torch.bfloat16
    log(f"large heads: N_Q={NQ}, N_K={N0}x{R}={NK}")
    q1, k1s, q2, k2s = make_inputs(1, 1, NQ, N0, d, bf16, "student", 0.4, seed=77, device=DEV)
    scale = d ** -0.5
    g = upstream_grad(1, 1, NQ, seed=5, device=DEV)

    # The untiled problem against the oracle.
    kl_s, l1_s, l2_s = ops.streamkl_fwd(q1, k1s, q2, k2s, scale, False)
    small = dict(zip(NAMES, ops.streamkl_bwd(q1, k1s, q2, k2s, kl_s, l1_s, l2_s, g, scale, False)))
    torch.cuda.synchronize()
    ref = oracle_heads(q1, k1s, q2, k2s, scale, False, [0], g=g, grads=True)[0]
    check_rows(to64(kl_s[0, 0]), ref["kl"], bf16, "untiled kl")
    for n in NAMES:
        check_grad(to64(small[n][0, 0]), ref[n], bf16, f"untiled {n}")

    # The tiled problem: every key row repeated R times.
    k1 = k1s.repeat(1, 1, R, 1)
    k2 = k2s.repeat(1, 1, R, 1)
    kl, l1, l2 = ops.streamkl_fwd(q1, k1, q2, k2, scale, False)
    big = dict(zip(NAMES, ops.streamkl_bwd(q1, k1, q2, k2, kl, l1, l2, g, scale, False)))
    torch.cuda.synchronize()

    lnR = math.log(R)
    check_rows(to64(kl[0, 0]), to64(kl_s[0, 0]), bf16, "tiled kl")
    check_rows(to64(l1[0, 0]), to64(l1_s[0, 0]) + lnR, bf16, "tiled lse1")
    check_rows(to64(l2[0, 0]), to64(l2_s[0, 0]) + lnR, bf16, "tiled lse2")
    for n in ("dq1", "dq2"):
        check_grad(to64(big[n][0, 0]), to64(small[n][0, 0]), bf16, f"tiled {n}")
    # Copies at the start, in the middle, at the first row past 4 GiB and at
    # the end of the key tensor.
    first_past = (2 ** 32 // (d * 2) + N0 - 1) // N0
    for n in ("dk1", "dk2"):
        copies = big[n][0, 0].view(R, N0, d)
        for r in (0, 1, R // 2, first_past - 1, first_past, R - 1):
            check_grad(to64(copies[r]) * R, to64(small[n][0, 0]), bf16, f"tiled {n} copy {r}")
