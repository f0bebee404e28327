"""Shared helpers for the GPU parity tests: run the oracle on exact float64
copies of the very tensors the GPU saw, and apply the stated tolerances.

Tolerances (per query row for KL/LSE, per (b, h) slice for gradients):
  fp32 inputs:  |dKL| <= 1e-5, same for LSE1/LSE2; gradients rel-L2 <= 1e-4.
  bf16 inputs:  |dKL| <= 2e-3 + 1e-2 |KL_ref|, same for LSE; gradients
                ||g - g_ref||_2 <= 2e-2 ||g_ref||_2 + 1e-6 sqrt(n).
"""
import sys

import numpy as np
import torch

import oracle


def log(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def to64(t):
    return t.detach().to("cpu", torch.float64).numpy()


def row_tol(dtype):
    return (1e-5, 0.0) if dtype == torch.float32 else (2e-3, 1e-2)


U32 = 2.0 ** -24   # unit roundoff of fp32


def score_roundings(dtype, d):
    """fp32 roundings in one raw score s = <q, k> on the matrix cores: the
    bf16 products (v_mfma_f32_32x32x16_bf16) add 16 exact products per
    instruction into the fp32 accumulator, d / 16 instructions; the fp32
    ones (v_mfma_f32_32x32x2_f32) add 2, d / 2 instructions."""
    return d // 16 if dtype == torch.bfloat16 else d // 2


def magnitude_k(dtype, d):
    """Multiple of 2^-24 |LSE_ref| that bounds the kernels' fp32 rounding
    error in KL, LSE1 and LSE2 when the logits are far from unit scale.

    With n = score_roundings(dtype, d), each score carries at most n u M,
    M the magnitude of its partial sums (about |LSE| on the rows these inputs
    make).  LSE_t inherits one score error, plus one rounding each in the
    exponent's shift -m c, in m * scale and in m * scale + log l, and the
    same again through the lane-half merge: (n + 4) u |LSE|.  KL =
    scale acc / l1 + LSE2 - LSE1 adds both LSE errors, the error of
    acc / l1 (s1 - s2 carries two score errors, 2 n u |LSE|) and the two
    roundings of the final sum on terms of size |LSE|, 2 u |LSE| each,
    plus one for the division: 2 (n + 4) + 2 n + 5 = 4 n + 13."""
    return 4 * score_roundings(dtype, d) + 13


def check_rows(got, ref, dtype, what, mag=None, k=None):
    """got/ref: float64 arrays of per-row values; raise with the worst row.

    The bound is the stated per-row tolerance: fp32 inputs 1e-5, bf16 inputs
    2e-3 + 1e-2 |ref|.  ``mag`` (per-row max(|LSE1_ref|, |LSE2_ref|)) and
    ``k`` add the fp32 rounding of logits far outside unit scale, k 2^-24 mag
    with k from magnitude_k (or exact_score_k for inputs whose scores are
    exact in fp32); ``k`` is required with ``mag``."""
    atol, rtol = row_tol(dtype)
    err = np.abs(got - ref)
    bound = atol + rtol * np.abs(ref)
    if mag is not None:
        assert k is not None, "a magnitude term needs its derived multiple"
        bound = bound + k * U32 * np.abs(mag)
    bad = ~(err <= bound)
    if bad.any():
        i = int(np.argmax(np.where(bad, err - bound, -np.inf)))
        raise AssertionError(f"{what}: {int(bad.sum())} rows out of tolerance; worst index {i}: "
                             f"got {got.flat[i]!r} ref {ref.flat[i]!r} (|err| {err.flat[i]:.3g} > {bound.flat[i]:.3g})")
    return float(err.max()) if err.size else 0.0


def check_grad(got, ref, dtype, what):
    """Relative L2 over one (b, h) slice (or any array)."""
    got = np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    diff = np.linalg.norm(got - ref)
    nref = np.linalg.norm(ref)
    if dtype == torch.float32:
        bound = 1e-4 * nref + 1e-9 * np.sqrt(ref.size)
    else:
        bound = 2e-2 * nref + 1e-6 * np.sqrt(ref.size)
    if not diff <= bound:
        raise AssertionError(f"{what}: ||err|| {diff:.4g} > {bound:.4g} (||ref|| {nref:.4g})")
    return diff / max(nref, 1e-30)


def oracle_heads(q1, k1, q2, k2, scale, causal, heads, g=None, grads=False, rows=None):
    """Oracle results for the listed flat head indices (b*H + h)."""
    B, H, NQ, d = q1.shape
    out = {}
    for hh in heads:
        b, h = divmod(hh, H)
        gg = None if g is None else to64(g[b, h])
        out[hh] = oracle.head(to64(q1[b, h]), to64(k1[b, h]), to64(q2[b, h]), to64(k2[b, h]),
                              scale, causal, g=gg, rows=rows, grads=grads)
    return out


def sample_rows(n, k, seed):
    """First and last rows plus a seeded random sample, sorted, unique."""
    rng = np.random.default_rng(seed)
    edge = list(range(min(4, n))) + list(range(max(0, n - 4), n))
    rnd = rng.choice(n, size=min(k, n), replace=False).tolist() if n else []
    return sorted(set(edge + rnd))


def head64(q1, k1, q2, k2, hh):
    """Exact float64 numpy copies of one flat head."""
    H = q1.shape[1]
    b, h = divmod(hh, H)
    return to64(q1[b, h]), to64(k1[b, h]), to64(q2[b, h]), to64(k2[b, h])


def row_blocks(n, width=32):
    """Contiguous query-row blocks at the start, middle and end of [0, n)."""
    if n <= 3 * width:
        return [(0, n)]
    mid = (n // 2) - width // 2
    return [(0, width), (mid, mid + width), (n - width, n)]


def oracle_row_blocks(h64, scale, causal, blocks, g=None, grads=False):
    """Run the oracle on several row blocks of one head; returns a dict of
    per-row arrays (NaN outside the blocks) and, if grads, dq rows and the
    dk contribution of the union of blocks."""
    q1, k1, q2, k2 = h64
    res = None
    for (rb, re) in blocks:
        o = oracle.head(q1, k1, q2, k2, scale, causal, g=g, rows=(rb, re), grads=grads)
        if res is None:
            res = o
            continue
        for key in ("kl", "lse1", "lse2"):
            res[key][rb:re] = o[key][rb:re]
        if grads:
            res["dq1"][rb:re] = o["dq1"][rb:re]
            res["dq2"][rb:re] = o["dq2"][rb:re]
            res["dk1"] += o["dk1"]
            res["dk2"] += o["dk2"]
    return res
