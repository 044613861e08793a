"""Pins for the oracle's sampler and sample threshold (no GPU).

Sampling S of N without replacement (Prof-K paper, section 3, stage 1) is read
as the first S images of a keyed permutation of [0, N).  The pins: the
network is a bijection on its domain, samples are distinct and in range, and
on ascending data the rank of the threshold follows the law of Lemma 1
(Eq. 1 and Eq. 2) over many seeds.
"""
import numpy as np
import pytest

import oracle
import oracle.params as P
import workloads


@pytest.mark.parametrize("n", [1, 2, 3, 4, 5, 17, 64, 1000, 4097, 65536])
def test_feistel_is_bijection_on_domain(n):
    b = max(2, int(np.ceil(np.log2(n))) if n > 1 else 0)
    h = (b + 1) // 2
    dom = 1 << (2 * h)
    img = oracle.feistel_raw(12345, 3, n, dom)
    assert np.array_equal(np.sort(img), np.arange(dom, dtype=np.uint64))


@pytest.mark.parametrize("n,S", [(1, 1), (5, 5), (100, 100), (1000, 37), (70001, 32768),
                                 (2 ** 20, 32768)])
def test_samples_distinct_in_range(n, S):
    s = oracle.sample_indices(77, 5, n, S)
    assert s.max() < n
    assert np.unique(s).size == S
    if S == n:
        assert np.array_equal(np.sort(s), np.arange(n, dtype=np.uint64))


def test_samples_depend_on_seed_and_row():
    a = oracle.sample_indices(1, 0, 10 ** 6, 1000)
    b = oracle.sample_indices(2, 0, 10 ** 6, 1000)
    c = oracle.sample_indices(1, 1, 10 ** 6, 1000)
    assert not np.array_equal(a, b) and not np.array_equal(a, c)


def test_inclusion_is_uniform():
    # every position is drawn with probability S/N; chi-square over seeds
    n, S, reps = 64, 8, 4000
    counts = np.zeros(n)
    for s in range(reps):
        counts[oracle.sample_indices(s, 0, n, S).astype(np.int64)] += 1
    expect = reps * S / n
    chi2 = float(((counts - expect) ** 2 / expect).sum())
    assert chi2 < 120          # 63 degrees of freedom; p ~ 1e-5 at 120


def test_tau_matches_definition():
    row = workloads.pareto_signed(1, 200000, 8)[0]
    S, t = 4096, 7
    tk, R, sk = oracle.tau(row, 99, 0, S, t, with_sample=True)
    idx = oracle.sample_indices(99, 0, row.size, S).astype(np.int64)
    keys = oracle.keys(row)
    assert np.array_equal(sk, keys[idx])
    assert tk == np.sort(keys[idx])[::-1][t - 1]
    assert R == int(np.count_nonzero(keys >= tk))


def test_threshold_rank_law_lemma1():
    """Ascending distinct data: R equals the rank of tau.  Compare the observed
    law over seeds with Eq. 1 (chi-square) and Eq. 2 (mean, variance)."""
    N, S, t, reps = 4096, 256, 5, 3000
    row = np.arange(N, dtype=np.int32)
    Rs = np.array([oracle.tau(row, s, 0, S, t)[1] for s in range(reps)])
    mean, var = P.rank_mean_var(N, S, t)
    assert abs(Rs.mean() - mean) < 4 * np.sqrt(var / reps)
    assert abs(Rs.var() / var - 1) < 0.15
    # chi-square on bins of equal Eq.-1 mass
    edges = [t]
    acc, target = 0.0, 1 / 12
    r = t
    cdf = []
    while r <= N - S + t:
        acc += P.rank_pmf(N, S, t, r)
        cdf.append(acc)
        r += 1
    cdf = np.array(cdf)
    qs = np.searchsorted(cdf, np.arange(1, 12) * target) + t
    obs = np.histogram(Rs, bins=np.concatenate([[t], qs, [N + 1]]))[0]
    exp_p = np.diff(np.concatenate([[0.0], cdf[qs - t - 1], [1.0]]))
    chi2 = float(((obs - reps * exp_p) ** 2 / (reps * exp_p)).sum())
    assert chi2 < 35          # 11 degrees of freedom
