"""Pins for the fp64 CPU oracle, independent of the oracle's own code.

Each test checks the oracle against something fixed by the StreamKL summary
page or by mathematics: a definitional brute force, closed forms, textbook
special cases, invariants, finite differences and the page's one printed
figure.  Together they are chosen so that a dropped term, a wrong sign, a
wrong causal index or a swapped operand in the oracle fails at least one of
them (``test_oracle_mutants.py`` plants such mistakes and checks exactly that).
"""
import json
import math
import os

import numpy as np
import pytest
from scipy.special import logsumexp, softmax

import oracle
from oracle import brute

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def rnd(shape, seed, scale=1.0):
    return np.random.default_rng(seed).standard_normal(shape) * scale


def problem(nq, nk, d, seed, sigma=None):
    q1, k1 = rnd((nq, d), seed), rnd((nk, d), seed + 1)
    if sigma is None:
        q2, k2 = rnd((nq, d), seed + 2), rnd((nk, d), seed + 3)
    else:
        q2 = q1 + sigma * rnd((nq, d), seed + 2)
        k2 = k1 + sigma * rnd((nk, d), seed + 3)
    return q1, k1, q2, k2


def n_allowed(nq, nk, causal):
    return np.array([nk if not causal else min(nk, i + nk - nq + 1) for i in range(nq)])


# ---------------------------------------------------------------- brute force
@pytest.mark.parametrize("nq,nk,d,causal", [
    (1, 1, 1, False), (1, 1, 3, True), (3, 5, 4, False), (5, 5, 8, True),
    (4, 7, 3, True), (6, 2, 5, False), (8, 8, 2, True), (7, 8, 6, False)])
def test_forward_matches_definitional_brute_force(nq, nk, d, causal):
    q1, k1, q2, k2 = problem(nq, nk, d, seed=10 * nq + nk + d)
    scale = 1.0 / math.sqrt(d)
    o = oracle.head(q1, k1, q2, k2, scale, causal)
    kl, l1, l2 = brute.kl_rows(q1.tolist(), k1.tolist(), q2.tolist(), k2.tolist(), scale, causal)
    np.testing.assert_allclose(o["kl"], kl, rtol=1e-11, atol=1e-13)
    np.testing.assert_allclose(o["lse1"], l1, rtol=1e-12, atol=1e-13)
    np.testing.assert_allclose(o["lse2"], l2, rtol=1e-12, atol=1e-13)


# ---------------------------------------------------------------- closed forms
def softplus(x):
    return math.log1p(math.exp(-abs(x))) + max(x, 0.0)


def sigmoid(x):
    return 1.0 / (1.0 + math.exp(-x))


@pytest.mark.parametrize("seed", range(6))
def test_two_key_closed_form(seed):
    """N_K = 2: with a = S1_0 - S1_1, b = S2_0 - S2_1,
    KL = sigmoid(a) (a - b) - softplus(a) + softplus(b), LSE_t = S_t1 + softplus(.)."""
    rng = np.random.default_rng(seed)
    d = 3
    q1, q2 = rng.standard_normal((4, d)) * 2, rng.standard_normal((4, d)) * 2
    k1, k2 = rng.standard_normal((2, d)), rng.standard_normal((2, d))
    scale = 0.7
    o = oracle.head(q1, k1, q2, k2, scale, False)
    for i in range(4):
        s1 = [scale * float(q1[i] @ k1[j]) for j in range(2)]
        s2 = [scale * float(q2[i] @ k2[j]) for j in range(2)]
        a, b = s1[0] - s1[1], s2[0] - s2[1]
        kl = sigmoid(a) * (a - b) - softplus(a) + softplus(b)
        assert o["kl"][i] == pytest.approx(kl, rel=1e-12, abs=1e-15)
        assert o["lse1"][i] == pytest.approx(s1[1] + softplus(a), rel=1e-13)
        assert o["lse2"][i] == pytest.approx(s2[1] + softplus(b), rel=1e-13)


def test_hand_examples():
    """Small distributions whose KL is known by hand (d = 1, scale = 1)."""
    ln2, ln3 = math.log(2.0), math.log(3.0)
    # P1 = (3/4, 1/4), P2 = (1/2, 1/2): KL = 3/4 ln 3 - ln 2.
    o = oracle.head([[ln3]], [[1.0], [0.0]], [[0.0]], [[1.0], [0.0]], 1.0, False)
    assert o["kl"][0] == pytest.approx(0.75 * ln3 - ln2, rel=1e-14)
    assert o["lse1"][0] == pytest.approx(2 * ln2, rel=1e-15)
    assert o["lse2"][0] == pytest.approx(ln2, rel=1e-15)
    # P1 = (1/2, 1/4, 1/4), P2 = (1/4, 1/4, 1/2): KL = ln(2) / 4.
    o = oracle.head([[ln2]], [[1.0], [0.0], [0.0]], [[ln2]], [[0.0], [0.0], [1.0]], 1.0, False)
    assert o["kl"][0] == pytest.approx(0.25 * ln2, rel=1e-14)
    assert o["lse1"][0] == pytest.approx(2 * ln2, rel=1e-15)
    assert o["lse2"][0] == pytest.approx(2 * ln2, rel=1e-15)
    # Reversed direction of the first example: KL(P2 || P1) = ln 2 - 1/2 ln 3.
    o = oracle.head([[0.0]], [[1.0], [0.0]], [[ln3]], [[1.0], [0.0]], 1.0, False)
    assert o["kl"][0] == pytest.approx(ln2 - 0.5 * ln3, rel=1e-14)


def test_golden_materialisation_figure():
    """The page's only number for this path: two 64K x 64K x 32-head bf16
    probability tensors take about 512 GB (Problem section, item 1)."""
    with open(os.path.join(GOLDEN, "memory_figure.json")) as f:
        g = json.load(f)
    n, heads, nbytes, ntensors = g["context"], g["heads"], g["bytes_per_elem"], g["tensors"]
    total = ntensors * n * n * heads * nbytes
    assert total == g["expected_bytes"]
    assert total / 2**30 == pytest.approx(g["page_value_gb"], rel=0.0)


# ---------------------------------------------------------------- special cases
@pytest.mark.parametrize("causal", [False, True])
def test_identical_teacher_student_gives_zero(causal):
    q, k, _, _ = problem(9, 11, 5, seed=3)
    o = oracle.head(q, k, q, k, 0.4, causal, g=rnd(9, 4), grads=True)
    assert np.all(o["kl"] == 0.0)
    np.testing.assert_array_equal(o["lse1"], o["lse2"])
    for key in ("dq1", "dk1", "dq2", "dk2"):
        assert np.all(o[key] == 0.0), key


@pytest.mark.parametrize("causal", [False, True])
def test_uniform_student_entropy(causal):
    """Q2 = 0 makes P2 uniform over J_i: LSE2 = ln|J_i| and KL = ln|J_i| - H(P1)."""
    nq, nk, d = 7, 10, 4
    q1, k1, _, k2 = problem(nq, nk, d, seed=5)
    q2 = np.zeros_like(q1)
    scale = 0.9
    o = oracle.head(q1, k1, q2, k2, scale, causal)
    J = n_allowed(nq, nk, causal)
    S1 = scale * q1 @ k1.T
    for i in range(nq):
        p = softmax(S1[i, :J[i]])
        H = -np.sum(p * np.log(p))
        assert o["lse2"][i] == pytest.approx(math.log(J[i]), rel=1e-14)
        assert o["lse1"][i] == pytest.approx(logsumexp(S1[i, :J[i]]), rel=1e-13)
        assert o["kl"][i] == pytest.approx(math.log(J[i]) - H, rel=1e-11, abs=1e-14)


@pytest.mark.parametrize("nq,nk", [(6, 6), (4, 9)])
def test_zero_queries_count_allowed_keys(nq, nk):
    """Q1 = Q2 = 0: both distributions uniform over J_i, so KL = 0 and
    LSE_t = ln|J_i| -- this pins the causal frontier j <= i + N_K - N_Q."""
    _, k1, _, k2 = problem(nq, nk, 3, seed=6)
    z = np.zeros((nq, 3))
    for causal in (False, True):
        o = oracle.head(z, k1, z, k2, 1.0, causal)
        J = n_allowed(nq, nk, causal)
        np.testing.assert_allclose(o["lse1"], np.log(J), rtol=1e-15)
        np.testing.assert_allclose(o["lse2"], np.log(J), rtol=1e-15)
        np.testing.assert_array_equal(o["kl"], 0.0)


def test_single_allowed_key():
    """Causal square problem: row 0 sees only key 0, so KL = 0, LSE_t = S_t[0, 0]."""
    q1, k1, q2, k2 = problem(5, 5, 4, seed=7)
    o = oracle.head(q1, k1, q2, k2, 0.5, True)
    assert o["kl"][0] == 0.0
    assert o["lse1"][0] == pytest.approx(0.5 * q1[0] @ k1[0], rel=1e-15)
    assert o["lse2"][0] == pytest.approx(0.5 * q2[0] @ k2[0], rel=1e-15)


def test_peaked_distributions_stay_finite():
    """Huge logits (overflow for a naive exp): the teacher is one-hot on key j*,
    so KL = LSE2 - S2[j*] (the student's negative log-probability of j*)."""
    d, nk = 4, 6
    k1 = np.eye(nk, d) * 1.0
    k1[4:] = -1.0
    q1 = np.array([[800.0, 0, 0, 0], [0, 0, 900.0, 0]])
    q2, k2 = rnd((2, d), 8, 30.0), rnd((nk, d), 9)
    o = oracle.head(q1, k1, q2, k2, 1.0, False, grads=True)
    assert np.all(np.isfinite(o["kl"]))
    for key in ("dq1", "dk1", "dq2", "dk2"):
        assert np.all(np.isfinite(o[key])), key
    S2 = q2 @ k2.T
    for i, jstar in enumerate([0, 2]):
        assert o["kl"][i] == pytest.approx(logsumexp(S2[i]) - S2[i, jstar], rel=1e-12)


# ---------------------------------------------------------------- invariants
@pytest.mark.parametrize("causal", [False, True])
def test_gibbs_nonnegative(causal):
    for seed in range(5):
        q1, k1, q2, k2 = problem(12, 16, 6, seed=20 + seed)
        o = oracle.head(q1, k1, q2, k2, 0.8, causal)
        assert np.all(o["kl"] >= -1e-15)
        assert np.any(o["kl"] > 1e-3)


@pytest.mark.parametrize("causal", [False, True])
def test_key_shift_invariance(causal):
    """K_t -> K_t + 1 v^T adds scale <q_t[i], v> to row i of S_t: the
    distributions, KL and all gradients are unchanged, LSE_t moves by it."""
    q1, k1, q2, k2 = problem(8, 10, 5, seed=30)
    v1, v2 = rnd(5, 31), rnd(5, 32)
    s, g = 0.6, rnd(8, 33)
    a = oracle.head(q1, k1, q2, k2, s, causal, g=g, grads=True)
    b = oracle.head(q1, k1 + v1, q2, k2 + v2, s, causal, g=g, grads=True)
    np.testing.assert_allclose(b["kl"], a["kl"], rtol=1e-9, atol=1e-12)
    np.testing.assert_allclose(b["lse1"], a["lse1"] + s * q1 @ v1, rtol=1e-12)
    np.testing.assert_allclose(b["lse2"], a["lse2"] + s * q2 @ v2, rtol=1e-12)
    for key in ("dq1", "dq2", "dk1", "dk2"):
        np.testing.assert_allclose(b[key], a[key], rtol=1e-8, atol=1e-12, err_msg=key)


def test_joint_key_permutation():
    """Non-causal: permuting the keys of K1 and K2 together permutes dK rows
    and changes nothing else."""
    q1, k1, q2, k2 = problem(6, 9, 4, seed=40)
    perm = np.random.default_rng(41).permutation(9)
    g = rnd(6, 42)
    a = oracle.head(q1, k1, q2, k2, 0.5, False, g=g, grads=True)
    b = oracle.head(q1, k1[perm], q2, k2[perm], 0.5, False, g=g, grads=True)
    for key in ("kl", "lse1", "lse2", "dq1", "dq2"):
        np.testing.assert_allclose(b[key], a[key], rtol=1e-12, atol=1e-14, err_msg=key)
    np.testing.assert_allclose(b["dk1"], a["dk1"][perm], rtol=1e-12, atol=1e-14)
    np.testing.assert_allclose(b["dk2"], a["dk2"][perm], rtol=1e-12, atol=1e-14)


@pytest.mark.parametrize("causal", [False, True])
def test_gradient_identities(causal):
    """Each row of dS_t sums to zero, so sum_j dK_t[j] = 0; and
    sum_i <dQ_t[i], q_t[i]> = sum_j <dK_t[j], k_t[j]> (both are sum dS_t * S_t)."""
    q1, k1, q2, k2 = problem(10, 13, 6, seed=50, sigma=0.5)
    o = oracle.head(q1, k1, q2, k2, 0.45, causal, g=rnd(10, 51), grads=True)
    for t, (q, k) in ((1, (q1, k1)), (2, (q2, k2))):
        dq, dk = o[f"dq{t}"], o[f"dk{t}"]
        assert np.abs(dk.sum(0)).max() < 1e-13 * max(1.0, np.abs(dk).max())
        assert np.sum(dq * q) == pytest.approx(np.sum(dk * k), rel=1e-11, abs=1e-13)


def test_upstream_gradient_is_linear():
    q1, k1, q2, k2 = problem(7, 7, 3, seed=60)
    a = oracle.head(q1, k1, q2, k2, 0.5, True, grads=True)
    b = oracle.head(q1, k1, q2, k2, 0.5, True, g=np.full(7, -2.5), grads=True)
    for key in ("dq1", "dk1", "dq2", "dk2"):
        np.testing.assert_allclose(b[key], -2.5 * a[key], rtol=1e-13, atol=1e-15)


def test_row_ranges_compose():
    """Rows are independent for KL/LSE/dQ; dK is a sum over rows."""
    q1, k1, q2, k2 = problem(9, 12, 4, seed=70, sigma=0.3)
    full = oracle.head(q1, k1, q2, k2, 0.5, True, grads=True)
    a = oracle.head(q1, k1, q2, k2, 0.5, True, rows=(0, 4), grads=True)
    b = oracle.head(q1, k1, q2, k2, 0.5, True, rows=(4, 9), grads=True)
    for key in ("kl", "lse1", "lse2"):
        np.testing.assert_array_equal(np.concatenate([a[key][:4], b[key][4:]]), full[key])
    np.testing.assert_array_equal(np.concatenate([a["dq1"][:4], b["dq1"][4:]]), full["dq1"])
    np.testing.assert_allclose(a["dk1"] + b["dk1"], full["dk1"], rtol=1e-13, atol=1e-15)
    np.testing.assert_allclose(a["dk2"] + b["dk2"], full["dk2"], rtol=1e-13, atol=1e-15)


# ---------------------------------------------------------------- finite differences
@pytest.mark.parametrize("nq,nk,d,causal", [(5, 5, 3, True), (4, 6, 3, False), (3, 7, 2, True)])
def test_gradients_match_central_differences(nq, nk, d, causal):
    """Central differences of sum_i g_i KL_i in fp64 pin dS2 = g (P2 - P1) and
    dS1 = g P1 (logP1 - logP2 - KL), and the scale and transposes of dQ/dK."""
    q1, k1, q2, k2 = problem(nq, nk, d, seed=80 + nq, sigma=0.7)
    g = rnd(nq, 81)
    scale = 0.6
    o = oracle.head(q1, k1, q2, k2, scale, causal, g=g, grads=True)

    def loss(a, b, c, e):
        r = oracle.head(a, b, c, e, scale, causal)
        return float(np.dot(g, r["kl"]))

    h = 1e-5
    args = [q1, k1, q2, k2]
    names = ["dq1", "dk1", "dq2", "dk2"]
    for t in range(4):
        fd = np.zeros_like(args[t])
        for idx in np.ndindex(args[t].shape):
            plus = [x.copy() for x in args]
            minus = [x.copy() for x in args]
            plus[t][idx] += h
            minus[t][idx] -= h
            fd[idx] = (loss(*plus) - loss(*minus)) / (2 * h)
        err = np.abs(fd - o[names[t]]).max() / max(np.abs(fd).max(), 1e-12)
        assert err < 1e-7, (names[t], err)
