"""Parameter selection for the sampled threshold (oracle side, test
infrastructure; the product library has its own C++ version).

``alg1``        Algorithm 1 of the Prof-K paper ("Adaptive parameter
                selection"), step by step in the paper's notation.
``exact_tail``  The reading used by default: S from Algorithm 1, then t and M
                from the two conditions of Theorem 3 (failure budget split
                eps_A = eps_B = eps/2) evaluated with the exact law of the
                threshold rank (Lemma 1) instead of its normal approximation
                (Lemma 2), which the paper itself calls unreliable when
                alpha*S is small.
``tuned``       t and M as in ``exact_tail``; S the point of the grid
                s_lo * 2^(j/4) (up to s_hi) with the least overhead of Eq. 13,
                tau_A*S + tau_B*M(S)*log2(k), written as S + ratio*M(S)*log2(k)
                with ratio = tau_B/tau_A (section 4, "Optimal Sample Size").

Lemma 1 (the t-th largest of S samples drawn without replacement from N
ranked items has rank R with a negative hypergeometric law) gives two
hypergeometric tails, with H(N, K, S) = number of sampled items among a fixed
set of K items:
  * recall failure  R < k   <=>  H(N, k-1, S) >= t
  * overflow        R > M   <=>  H(N, M, S)   <= t-1
"""
from __future__ import annotations

import math
from statistics import NormalDist

import numpy as np

S_MIN_DEFAULT = 32768
S_MAX_DEFAULT = 131072
EPS_DEFAULT = 1e-3
RATIO_DEFAULT = 1.0


def phi_inv(p: float) -> float:
    """Inverse standard normal CDF (Python standard library)."""
    return NormalDist().inv_cdf(p)


def alg1(N: int, k: int, eps: float = EPS_DEFAULT, s_min: int = S_MIN_DEFAULT,
         s_max: int = S_MAX_DEFAULT, ratio: float = RATIO_DEFAULT) -> dict:
    """Algorithm 1, verbatim (log base 2; round-to-nearest for S*)."""
    z = phi_inv(1 - eps / 2) + phi_inv(1 - eps / 2)
    alpha = k / N
    log2k = math.log2(k)
    s_star = (z * ratio * log2k / 2) ** (2.0 / 3.0) * (k * (N - k)) ** (1.0 / 3.0)
    S = min(s_max, max(s_min, int(math.floor(s_star + 0.5))))
    S = min(S, N)          # stage 1 draws S of the N items without replacement
    f = 1 - S / N
    t = max(1, math.ceil(S * alpha + (z / 2) * math.sqrt(S * alpha * (1 - alpha) * f)))
    M = math.ceil(k + z * math.sqrt(k * (N - k) / S * f))
    if alpha * S < -math.log(eps / 2):
        t = 1
    return {"z": z, "alpha": alpha, "s_star": s_star, "S": S, "f": f, "t": t, "M": M}


# ------------------------------------------------------------ hypergeometric
# H(N, K, S): number of the K marked items among S drawn without replacement
# from N.  P(H = 0) = prod_{i<m} (1 - a / (N - i)) with (m, a) the smaller and
# larger of (K, S); each later term follows from the ratio
# P(j+1) / P(j) = (K - j)(S - j) / ((j + 1)(N - K - S + j + 1)).
# Both are summed in log space (the lgamma form loses ~1e-6 relative at
# N = 2^28).
def _log_binom(a: int, b: int) -> float:
    return math.lgamma(a + 1) - math.lgamma(b + 1) - math.lgamma(a - b + 1)


def _log_pmf_walk(N: int, K: int, S: int, j_last: int):
    """log P(H = j) for j = j_min .. j_last (j_min = max(0, S - (N - K)))."""
    j_min = max(0, S - (N - K))
    if j_min == 0:
        m, a = (K, S) if K < S else (S, K)
        terms = np.log1p(-a / (N - np.arange(m, dtype=np.float64)))
        lp = math.fsum(terms.tolist())
    else:
        lp = _log_binom(K, j_min) + _log_binom(N - K, S - j_min) - _log_binom(N, S)
    out = []
    j = j_min
    while j <= j_last:
        out.append((j, lp))
        if j == min(K, S):
            break
        lp += math.log((K - j) * (S - j)) - math.log((j + 1) * (N - K - S + j + 1))
        j += 1
    return out


def hyper_pmf(N: int, K: int, S: int, j: int) -> float:
    """P(H = j)."""
    if j < max(0, S - (N - K)) or j > min(K, S):
        return 0.0
    return math.exp(_log_pmf_walk(N, K, S, j)[-1][1])


def hyper_cdf(N: int, K: int, S: int, t: int) -> float:
    """P(H <= t)."""
    if t < 0:
        return 0.0
    return math.fsum(math.exp(lp) for _, lp in _log_pmf_walk(N, K, S, t))


def hyper_sf(N: int, K: int, S: int, t: int) -> float:
    """P(H >= t), summed upward from t until the terms stop mattering."""
    hi = min(K, S)
    if t > hi:
        return 0.0
    if t <= max(0, S - (N - K)):
        return 1.0
    walk = _log_pmf_walk(N, K, S, t)
    j, lp = walk[-1]
    mode = (K + 1) * (S + 1) // (N + 2)
    terms = []
    running = 0.0
    while True:
        p = math.exp(lp)
        terms.append(p)
        running += p
        if j >= hi or (j > mode and p < running * 1e-18):
            break
        lp += math.log((K - j) * (S - j)) - math.log((j + 1) * (N - K - S + j + 1))
        j += 1
    return math.fsum(terms)


def _upper_tails(N: int, K: int, S: int):
    """(j0, sf) with sf[i] = P(H >= j0 + i), from one walk of the pmf."""
    hi = min(K, S)
    mode = (K + 1) * (S + 1) // (N + 2)
    walk = _log_pmf_walk(N, K, S, min(hi, mode))
    j, lp = walk[-1]
    pm = [math.exp(v) for _, v in walk]
    running = math.fsum(pm)
    while j < hi:
        lp += math.log((K - j) * (S - j)) - math.log((j + 1) * (N - K - S + j + 1))
        j += 1
        p = math.exp(lp)
        pm.append(p)
        running += p
        if j > mode and p < running * 1e-18:
            break
    sf = [0.0] * (len(pm) + 1)
    for i in range(len(pm) - 1, -1, -1):
        sf[i] = sf[i + 1] + pm[i]
    return walk[0][0], sf


def exact_tail(N: int, k: int, eps: float = EPS_DEFAULT, s_min: int = S_MIN_DEFAULT,
               s_max: int = S_MAX_DEFAULT, ratio: float = RATIO_DEFAULT) -> dict:
    """S from Algorithm 1; t = least t with P(R < k) <= eps/2; M = least M >= k
    with P(R > M) <= eps/2 (M capped at N)."""
    S = alg1(N, k, eps, s_min, s_max, ratio)["S"]
    half = eps / 2
    t = 1
    if k > 1:
        j0, sf = _upper_tails(N, k - 1, S)

        def tail(tt):
            if tt <= j0:
                return 1.0
            i = tt - j0
            return sf[i] if i < len(sf) else 0.0
        while t < S and tail(t) > half:
            t += 1
    lo, hi = k, N
    if hyper_cdf(N, hi, S, t - 1) > half:
        M = N
    else:
        while lo < hi:
            mid = (lo + hi) // 2
            if hyper_cdf(N, mid, S, t - 1) <= half:
                hi = mid
            else:
                lo = mid + 1
        M = lo
    return {"S": S, "t": t, "M": M,
            "p_recall": hyper_sf(N, k - 1, S, t),
            "p_overflow": hyper_cdf(N, M, S, t - 1)}


def tuned(N: int, k: int, eps: float = EPS_DEFAULT, s_lo: int = 1024,
          s_hi: int = S_MAX_DEFAULT, ratio: float = 0.13) -> dict:
    """Eq. 13 minimised over a quarter-octave grid of S, with the exact-tail
    buffer M(S) of each grid point; the smaller S wins a tie."""
    s_lo, s_hi = min(s_lo, N), min(s_hi, N)
    if s_hi < s_lo:
        return exact_tail(N, k, eps, s_min=s_lo, s_max=s_lo)
    best = None
    j = 0
    while True:
        S = int(round(s_lo * 2.0 ** (j / 4)))
        j += 1
        if S > s_hi:
            break
        r = exact_tail(N, k, eps, s_min=S, s_max=S)
        cost = S + ratio * r["M"] * math.log2(k)
        if best is None or cost < best[0]:
            best = (cost, r)
    return best[1]


def failure_probs(N: int, k: int, S: int, t: int, M: int) -> tuple[float, float]:
    """(P(R < k), P(R > M)) for distinct values, from Lemma 1."""
    return hyper_sf(N, k - 1, S, t), hyper_cdf(N, M, S, t - 1)


def rank_mean_var(N: int, S: int, t: int) -> tuple[float, float]:
    """Mean and variance of the threshold rank R (Lemma 1, Eq. 2)."""
    mean = (N + 1) / (S + 1) * t
    var = t * (S - t + 1) * (N + 1) * (N - S) / ((S + 1) ** 2 * (S + 2))
    return mean, var


def rank_pmf(N: int, S: int, t: int, r: int) -> float:
    """P(R = r) from Lemma 1, Eq. 1."""
    if r < t or r > N - S + t:
        return 0.0
    return math.exp(_log_binom(r - 1, t - 1) + _log_binom(N - r, S - t) - _log_binom(N, S))
