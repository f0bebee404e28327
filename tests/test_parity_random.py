"""GPU parity over seeded random shapes: every path at once.

Each case draws the shape, dtype, causal flag, gradient mask, upstream
gradient, split-K partition count and input recipe from a fixed seed, runs
the forward (library or explicit partitions), streamkl_bwd (whichever form
the library selects) and, for bf16, streamkl_bwd_fused, and compares KL,
LSE1, LSE2 and every requested gradient with the fp64 oracle at the stated
tolerances.  A fifth of the cases are wide grids (8-32 heads, 4K-20K keys),
where workgroups walk several key blocks, causal grids take the longest-first
order and the query gradients run by key partitions; those compare three
heads each."""
import random

import pytest
import torch

from attention_distillation_kl_amd import make_inputs, ops
from attention_distillation_kl_amd.inputs import upstream_grad
from parity_util import check_grad, check_rows, log, oracle_heads, to64

pytestmark = pytest.mark.gpu

DEV = "cuda"
NAMES = ("dq1", "dk1", "dq2", "dk2")


def draw(case):
    rng = random.Random(7919 * case + 13)
    c = dict(dt=torch.bfloat16 if rng.random() < 0.8 else torch.float32, d=rng.choice([64, 128]),
             B=rng.choice([1, 1, 2]), H=rng.randint(1, 4), causal=rng.random() < 0.6)
    short = rng.random() < 0.4
    c["NQ"] = rng.randint(1, 64) if short else rng.randint(1, 700)
    c["NK"] = rng.randint(c["NQ"] if c["causal"] else 1, 4000 if short else 1500)
    c["mask"] = rng.choice([1, 2, 3, 3])
    c["g"] = rng.random() < 0.4
    c["splits"] = rng.choice([None, None, 1, 2, 3, 5, 16, 33, 70])
    c["mode"] = rng.choice(["student", "iid"])
    c["big"] = rng.random() < 0.2
    if c["big"]:
        c.update(dt=torch.bfloat16, B=1, H=rng.choice([8, 16, 32]))
        c["NQ"] = rng.randint(1, 64) if rng.random() < 0.6 else rng.randint(65, 600)
        c["NK"] = rng.randint(max(c["NQ"], 4096), 20000)
    c["heads"] = sorted({0, c["B"] * c["H"] - 1, rng.randrange(c["B"] * c["H"])}) if c["big"] else list(range(c["B"] * c["H"]))
    return c


@pytest.mark.parametrize("case", range(40))
def test_random_shapes_every_path_matches_oracle(case):
    c = draw(case)
    tag = f"random case {case}: " + ", ".join(f"{k}={v}" for k, v in c.items() if k != "heads")
    log(tag)
    B, H, NQ, NK, d, dt = c["B"], c["H"], c["NQ"], c["NK"], c["d"], c["dt"]
    q1, k1, q2, k2 = make_inputs(B, H, NQ, NK, d, dt, c["mode"], 0.3, seed=5000 + case, device=DEV)
    scale = d ** -0.5
    g = upstream_grad(B, H, NQ, seed=case, device=DEV) if c["g"] else None
    kl, l1, l2 = ops.streamkl_fwd(q1, k1, q2, k2, scale, c["causal"], splits=c["splits"])
    grads = ops.streamkl_bwd(q1, k1, q2, k2, kl, l1, l2, g, scale, c["causal"], c["mask"])
    fused = ops.streamkl_bwd_fused(q1, k1, q2, k2, kl, l1, l2, g, scale, c["causal"], c["mask"]) \
        if dt == torch.bfloat16 else None
    torch.cuda.synchronize()
    ref = oracle_heads(q1, k1, q2, k2, scale, c["causal"], c["heads"], g=g, grads=True)
    for hh in c["heads"]:
        b, h = divmod(hh, H)
        for nm, t in (("kl", kl), ("lse1", l1), ("lse2", l2)):
            check_rows(to64(t[b, h]), ref[hh][nm], dt, f"{tag} head {hh} {nm}")
        for i, nm in enumerate(NAMES):
            if grads[i] is None:
                continue
            check_grad(to64(grads[i][b, h]), ref[hh][nm], dt, f"{tag} head {hh} {nm}")
            if fused is not None:
                check_grad(to64(fused[i][b, h]), ref[hh][nm], dt, f"{tag} head {hh} fused {nm}")
