"""Definitional brute force for tiny inputs (test infrastructure only).

Pure Python, exactly-rounded sums (``math.fsum``), no max shift, no shared
code with ``streamkl_oracle.c``: each probability is exp(S) / sum exp(S) and
KL(P1 || P2) = sum_j P1 log(P1 / P2), the textbook definition the StreamKL
summary page (Problem section) starts from.  Only for N, d <= ~16 and logits
of moderate size (no overflow handling on purpose).
"""
import math


def _scores(q, k, scale, keys):
    return [scale * math.fsum(a * b for a, b in zip(q, k[j])) for j in keys]


def kl_rows(q1, k1, q2, k2, scale, causal=False):
    """Per-row (KL, LSE1, LSE2) lists for one head given as nested lists."""
    n_q, n_k = len(q1), len(k1)
    kls, l1s, l2s = [], [], []
    for i in range(n_q):
        keys = [j for j in range(n_k) if (not causal) or j <= i + n_k - n_q]
        s1 = _scores(q1[i], k1, scale, keys)
        s2 = _scores(q2[i], k2, scale, keys)
        z1 = math.fsum(math.exp(x) for x in s1)
        z2 = math.fsum(math.exp(x) for x in s2)
        p1 = [math.exp(x) / z1 for x in s1]
        p2 = [math.exp(x) / z2 for x in s2]
        kls.append(math.fsum(a * math.log(a / b) for a, b in zip(p1, p2) if a > 0))
        l1s.append(math.log(z1))
        l2s.append(math.log(z2))
    return kls, l1s, l2s
