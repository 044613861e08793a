"""Pins for the oracle's parameter arithmetic (no GPU).

Printed values from the Prof-K paper (z, S*, the BatchTopK shape), library
routines (scipy's hypergeometric law), the cost model of Eq. 13 minimised
numerically (Theorem 5), and the decomposition of M through Eqs. 8 and 11
(Corollary 4).
"""
import json
import math
import os

import numpy as np
import pytest

import oracle.params as P

GOLD = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "paper_values.json")))


def test_z_printed_value():
    g = GOLD["z_eps_1e-3"]
    z = P.alg1(2 ** 28, 64, eps=GOLD["eps_default"]["value"])["z"]
    assert abs(z - g["value"]) <= g["abs_tol"]


def test_s_star_printed_value_is_the_proportionality():
    g = GOLD["s_star_N1e9_k100"]
    assert abs((g["N"] * g["k"]) ** (1 / 3) / g["value"] - 1) < g["rel_tol"]


def test_buffer_order_of_magnitude():
    g = GOLD["buffer_N2p29_k64"]            # loose figure: order of magnitude only
    M = P.alg1(g["N"], g["k"])["M"]
    assert g["value"] / 3 < M < g["value"] * 3


def test_batchtopk_shape_and_bounds():
    g = GOLD["batchtopk_shape"]
    assert g["B"] * g["d_dict"] == g["N"] and g["B"] * g["k"] == g["K"]
    assert P.S_MIN_DEFAULT == GOLD["s_bounds"]["s_min"]
    assert P.S_MAX_DEFAULT == GOLD["s_bounds"]["s_max"] == 2 ** 17


def test_s_star_minimises_cost_model():
    """Eq. 13 with tau_B/tau_A = 1, M from Eq. 12 with f = 1, log base 2:
    the closed form of Eq. 14 is its minimiser."""
    for N, k in [(10 ** 9, 100), (2 ** 28, 64), (2 ** 24, 4096)]:
        z = P.alg1(N, k)["z"]
        s_star = P.alg1(N, k, s_min=1, s_max=10 ** 12)["s_star"]

        def cost(S):
            return S + (k + z * math.sqrt(k * (N - k) / S)) * math.log2(k)
        grid = np.linspace(0.5 * s_star, 1.5 * s_star, 2001)
        best = grid[np.argmin([cost(s) for s in grid])]
        assert abs(best / s_star - 1) < 2e-3


def test_buffer_size_through_eqs_8_and_11():
    for N, k in [(2 ** 28, 131072), (2 ** 28, 2048), (2 ** 20, 64)]:
        a = P.alg1(N, k)
        z_a = z_b = a["z"] / 2
        alpha, S, f = a["alpha"], a["S"], a["f"]
        c0 = 1 + z_a / math.sqrt(S) * math.sqrt((1 - alpha) / alpha * f)
        c = c0 + z_b * math.sqrt((1 - alpha) * f / (alpha * S))
        assert a["M"] == math.ceil(c * k) or abs(a["M"] - c * k) < 1.0


def test_threshold_rank_gaussian_regime():
    """Where alpha*S is large (the BatchTopK shape) Eq. 6's t keeps the exact
    recall-failure probability near eps_A."""
    a = P.alg1(2 ** 28, 131072)
    assert a["t"] > 1
    p_rec, _ = P.failure_probs(2 ** 28, 131072, a["S"], a["t"], a["M"])
    assert 1e-4 < p_rec < 5e-3


@pytest.mark.parametrize("N,K,S,j", [(1000, 50, 100, 3), (10 ** 6, 63, 32768, 2),
                                     (2 ** 28, 81894, 32768, 1), (5000, 400, 300, 30),
                                     (2 ** 28, 262172, 131072, 92)])
def test_hypergeometric_tails_match_scipy(N, K, S, j):
    st = pytest.importorskip("scipy.stats")
    assert P.hyper_sf(N, K, S, j) == pytest.approx(st.hypergeom.sf(j - 1, N, K, S), rel=1e-6, abs=1e-300)
    assert P.hyper_cdf(N, K, S, j) == pytest.approx(st.hypergeom.cdf(j, N, K, S), rel=1e-6, abs=1e-300)


def test_rank_pmf_against_eq2():
    N, S, t = 600, 40, 3
    pm = np.array([P.rank_pmf(N, S, t, r) for r in range(1, N + 1)])
    r = np.arange(1, N + 1)
    mean, var = P.rank_mean_var(N, S, t)
    assert pm.sum() == pytest.approx(1.0, abs=1e-12)
    assert (pm * r).sum() == pytest.approx(mean, rel=1e-10)
    assert (pm * (r - mean) ** 2).sum() == pytest.approx(var, rel=1e-9)


@pytest.mark.parametrize("N,k", [(2 ** 28, 16), (2 ** 28, 64), (2 ** 28, 2048), (2 ** 20, 64),
                                 (2 ** 28, 131072), (10 ** 7, 1)])
def test_exact_tail_conditions_and_minimality(N, k):
    st = pytest.importorskip("scipy.stats")
    e = P.exact_tail(N, k)
    S, t, M, half = e["S"], e["t"], e["M"], 0.5e-3
    if k > 1:
        assert st.hypergeom.sf(t - 1, N, k - 1, S) <= half * (1 + 1e-6)
        if t > 1:
            assert st.hypergeom.sf(t - 2, N, k - 1, S) > half
    assert st.hypergeom.cdf(t - 1, N, M, S) <= half * (1 + 1e-6)
    if M > k:
        assert st.hypergeom.cdf(t - 1, N, M - 1, S) > half * (1 - 1e-6)


def test_five_workload_shapes():
    # the benchmark's five shapes: Algorithm 1 verbatim (regression values),
    # and the exact-tail (t, M), each checked here to be the least meeting its
    # bound by scipy's hypergeometric law (Lemma 1)
    cases = {(2 ** 28, 16): (32768, 1, 2399, 2, 81894),
             (2 ** 28, 64): (32768, 1, 4829, 2, 81894),
             (2 ** 28, 2048): (89638, 1, 18344, 6, 52130),
             (2 ** 20, 64): (32768, 1, 358, 9, 704),
             (2 ** 28, 131072): (131072, 91, 238844, 93, 262172)}
    st = pytest.importorskip("scipy.stats")
    half = 1e-3 / 2
    for (N, k), (S, t1, M1, te, Me) in cases.items():
        a, e = P.alg1(N, k), P.exact_tail(N, k)
        assert (a["S"], a["t"], a["M"]) == (S, t1, M1)
        assert (e["S"], e["t"], e["M"]) == (S, te, Me)
        # recall failure R < k is H(N, k - 1, S) >= t; overflow R > M is H(N, M, S) <= t - 1
        assert st.hypergeom.sf(te - 1, N, k - 1, S) <= half
        assert te == 1 or st.hypergeom.sf(te - 2, N, k - 1, S) > half
        assert st.hypergeom.cdf(te - 1, N, Me, S) <= half < st.hypergeom.cdf(te - 1, N, Me - 1, S)


# ------------------------------------------------------------ the tuned policy
def _scipy_tail(N, k, S, eps):
    """(t, M) of the exact-tail reading computed with scipy's hypergeometric
    law only: the least t with P(H(N, k-1, S) >= t) <= eps/2 and the least
    M >= k with P(H(N, M, S) <= t-1) <= eps/2, both by bisection (the first
    tail falls as t grows, the second as M grows)."""
    H = pytest.importorskip("scipy.stats").hypergeom
    half = eps / 2
    lo, hi = 1, S
    if k > 1:
        while lo < hi:
            mid = (lo + hi) // 2
            if H.sf(mid - 1, N, k - 1, S) <= half:
                hi = mid
            else:
                lo = mid + 1
    t = lo
    if H.cdf(t - 1, N, N, S) > half:
        return t, N
    lo, hi = k, N
    while lo < hi:
        mid = (lo + hi) // 2
        if H.cdf(t - 1, N, mid, S) <= half:
            hi = mid
        else:
            lo = mid + 1
    return t, lo


@pytest.mark.parametrize("N,k,eps,ratio", [(2 ** 28, 64, 1e-3, 0.13), (2 ** 28, 16, 1e-3, 0.13),
                                           (2 ** 28, 2048, 1e-3, 0.13),
                                           (2 ** 20, 64, 1e-3 / 128, 0.13),
                                           (2 ** 28, 131072, 1e-3, 0.01),
                                           (2 ** 22, 100, 1e-3, 0.13), (2 ** 24, 1, 1e-3, 0.13)])
def test_tuned_policy_brute_force(N, k, eps, ratio):
    """Eq. 13's overhead S + ratio * M(S) * log2(k) (section 4, "Optimal
    Sample Size") minimised by brute force over the quarter-octave grid
    1024 * 2^(j/4) <= min(2^17, N/8), with M(S) and t(S) from scipy's
    hypergeometric law (Lemma 1), independently of the oracle's own tail
    arithmetic; the first grid point wins a tie."""
    s_hi = min(131072, N // 8)
    best, j, prev = None, 0, None
    while True:
        S = int(round(1024 * 2 ** (j / 4)))
        j += 1
        if S > s_hi:
            break
        if S == prev:
            continue
        prev = S
        t, M = _scipy_tail(N, k, S, eps)
        cost = S + ratio * M * math.log2(k)
        if best is None or cost < best[0]:
            best = (cost, S, t, M)
    got = P.tuned(N, k, eps, s_lo=1024, s_hi=s_hi, ratio=ratio)
    assert (got["S"], got["t"], got["M"]) == best[1:]


def test_tuned_optimum_approaches_theorem5():
    """Theorem 5 (Eq. 14) gives the minimiser of Eq. 13 with Eq. 12's M.  In
    the Gaussian regime (alpha * S >> 1, the BatchTopK shape) the exact-tail
    M(S) follows Eq. 12 to first order, with a second-order excess that a
    normal expansion of Lemma 1's tails fixes: t ~ alpha S + (z/2) sqrt(alpha S)
    and the buffer's expected sample count mu = M S / N solves
    mu = t - 1 + (z/2) sqrt(mu), so
        (M - k) / (M_Eq12 - k) ~ 1 + (z / 4) / sqrt(alpha S).
    The exact tails must show that excess, shrinking as 1/sqrt(alpha S); and
    the minimiser of the exact-tail cost on a fine grid lies a little above
    S*, approaching it as the cost ratio (and with it alpha * S) grows."""
    N, k, eps = 2 ** 28, 131072, 1e-3
    z = P.alg1(N, k)["z"]
    prev = None
    for S in (32768, 131072, 524288):
        f = 1 - S / N
        m12 = k + z * math.sqrt(k * (N - k) / S * f)
        me = P.exact_tail(N, k, eps, s_min=S, s_max=S)["M"]
        c = ((me - k) / (m12 - k) - 1) * math.sqrt(k / N * S)
        assert abs(c - z / 4) < 0.15, (S, c, z / 4)
        assert prev is None or abs(c - z / 4) < prev
        prev = abs(c - z / 4)
    prev = None
    for ratio in (0.01, 0.05, 1.0):
        s_star = (z * ratio * math.log2(k) / 2) ** (2 / 3) * (k * (N - k)) ** (1 / 3)
        grid = np.unique(np.round(s_star * np.exp(np.linspace(-0.7, 0.7, 57))).astype(int))
        cost = [S + ratio * P.exact_tail(N, k, eps, s_min=int(S), s_max=int(S))["M"] * math.log2(k)
                for S in grid]
        q = grid[int(np.argmin(cost))] / s_star
        assert 1.0 < q < 1.5, (ratio, q)
        assert prev is None or q < prev
        prev = q
