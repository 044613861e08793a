"""Host side of the C ABI, without a GPU: the library loads, exports every
function include/topk.h declares, validates arguments, and its parameter
arithmetic (Prof-K Algorithm 1, the exact-tail reading of Theorem 3, and the
tuned sample size of Eq. 13) agrees with the oracle's."""
import ctypes
import math
import os
import re

import pytest

from oracle import params as P

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "topk.h")


@pytest.fixture(scope="module")
def lib():
    from top_selection_sample_amd import _lib
    return _lib


def _declared():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:int|const char\s*\*)\s*(topk(?:_\w+)?)\s*\(", text, flags=re.M)))


def test_every_declared_symbol_is_exported(lib):
    names = _declared()
    assert len(names) >= 10, names
    raw = ctypes.CDLL(lib.LIB_PATH)
    for name in names:
        assert hasattr(raw, name), name
    assert set(names) == set(lib.EXPORTS)


def test_params_layout(lib):
    assert ctypes.sizeof(lib.Params) == 136
    assert ctypes.sizeof(lib.RowStats) == 28
    p = lib.default_params()
    assert (p.use_force_tau, p.force_tau_key, p.test_flags) == (0, 0, 0)
    assert p.recall == 1.0
    assert (p.eps, p.s_min, p.s_max, p.cost_ratio) == (1e-3, 32768, 131072, 1.0)
    assert p.policy == lib.POLICY_TUNED and p.force_path == 0
    assert (p.tuned_ratio, p.tuned_s_min, p.tuned_ratio_large) == (0.13, 1024, 0.01)
    assert (p.tuned_ratio_batched, p.tuned_batch_rows) == (0.03, 32)
    assert (p.S, p.t, p.M, p.use_seed) == (0, 0, 0, 0)


def _plan(lib, n, rows, k, dt, **kw):
    info = lib.PlanInfo()
    rc = lib.lib.topk_plan(n, rows, k, dt, ctypes.byref(lib.default_params(**kw)), ctypes.byref(info))
    return rc, info


@pytest.mark.parametrize("n,k", [(2 ** 28, 16), (2 ** 28, 64), (2 ** 28, 2048), (2 ** 20, 64),
                                 (2 ** 28, 131072), (10 ** 6, 1000)])
def test_alg1_policy_matches_oracle(lib, n, k):
    rc, info = _plan(lib, n, 1, k, 1, policy=lib.POLICY_ALG1)
    assert rc == 0
    a = P.alg1(n, k)
    assert (info.S, info.t, info.M) == (a["S"], a["t"], a["M"])


@pytest.mark.parametrize("n,k", [(2 ** 28, 64), (2 ** 28, 2048), (2 ** 20, 64), (2 ** 24, 5000)])
def test_exact_tail_policy_matches_oracle(lib, n, k):
    rc, info = _plan(lib, n, 1, k, 1, policy=lib.POLICY_EXACT_TAIL)
    assert rc == 0
    e = P.exact_tail(n, k)
    assert (info.S, info.t, info.M) == (e["S"], e["t"], e["M"])
    assert info.p_recall <= 5e-4 * (1 + 1e-9) and info.p_overflow <= 5e-4 * (1 + 1e-9)


@pytest.mark.parametrize("n,k,s_max", [(2 ** 20, 64, 131072), (2 ** 22, 100, 16384),
                                       (2 ** 21, 1000, 32768), (2 ** 24, 1, 8192),
                                       (2 ** 22, 9000, 131072)])
def test_tuned_policy_matches_oracle(lib, n, k, s_max):
    rc, info = _plan(lib, n, 3, k, 1, s_max=s_max, s_min=min(32768, s_max))
    assert rc == 0
    p = lib.default_params()
    ratio = p.tuned_ratio if k <= 4096 else p.tuned_ratio_large   # the engine's two refines
    e = P.tuned(n, k, eps=1e-3 / 3, s_hi=min(s_max, n // 8), ratio=ratio)   # eps per call, 3 rows
    assert (info.S, info.t, info.M) == (e["S"], e["t"], e["M"])


@pytest.mark.parametrize("n,k,rows", [(2 ** 20, 64, 128), (2 ** 20, 64, 32), (2 ** 20, 64, 31),
                                      (2 ** 22, 1000, 64), (2 ** 20, 5000, 128)])
def test_tuned_policy_prices_batches(lib, n, k, rows):
    # calls of tuned_batch_rows rows or more price small k with the batched
    # ratio (their rows' samples are gathered together); large k keeps the
    # bucket sort's ratio whatever the row count
    rc, info = _plan(lib, n, rows, k, 1)
    assert rc == 0
    p = lib.default_params()
    if k > 4096:
        ratio = p.tuned_ratio_large
    else:
        ratio = p.tuned_ratio_batched if rows >= p.tuned_batch_rows else p.tuned_ratio
    e = P.tuned(n, k, eps=1e-3 / rows, s_hi=min(131072, n // 8), ratio=ratio)
    assert (info.S, info.t, info.M) == (e["S"], e["t"], e["M"])
    # the threshold is a parameter: a row count below it uses the one-row ratio
    rc, info2 = _plan(lib, n, rows, k, 1, tuned_batch_rows=rows + 1)
    e2 = P.tuned(n, k, eps=1e-3 / rows, s_hi=min(131072, n // 8),
                 ratio=p.tuned_ratio_large if k > 4096 else p.tuned_ratio)
    assert (info2.S, info2.t, info2.M) == (e2["S"], e2["t"], e2["M"])


def test_eps_is_spent_per_call(lib):
    # a batch of independent rows shares the budget: each row gets eps / rows
    n, k, rows = 2 ** 20, 64, 128
    rc, info = _plan(lib, n, rows, k, 1, policy=lib.POLICY_EXACT_TAIL)
    assert rc == 0
    e = P.exact_tail(n, k, eps=1e-3 / rows)
    assert (info.S, info.t, info.M) == (e["S"], e["t"], e["M"])
    assert info.p_recall + info.p_overflow <= 1e-3 / rows * (1 + 1e-9)
    # Algorithm 1 verbatim keeps its per-selection eps
    rc, info = _plan(lib, n, rows, k, 1, policy=lib.POLICY_ALG1)
    a = P.alg1(n, k)
    assert (info.S, info.t, info.M) == (a["S"], a["t"], a["M"])


def test_tuned_policy_limits(lib):
    # a vanishing refine cost picks the smallest grid point, a huge one the
    # largest (M(S) falls as S grows); k = 1 has log2 k = 0: the smallest S
    n, k = 2 ** 22, 64
    assert _plan(lib, n, 1, k, 1, tuned_ratio=1e-9)[1].S == 1024
    big = _plan(lib, n, 1, k, 1, tuned_ratio=1e9, s_max=65536)[1].S   # s_min <= s_max
    grid = [round(1024 * 2 ** (j / 4)) for j in range(40) if round(1024 * 2 ** (j / 4)) <= 65536]
    assert big == grid[-1]
    assert _plan(lib, n, 1, 1, 1)[1].S == 1024
    # the grid is capped at n/8
    assert _plan(lib, 2 ** 18, 1, 64, 1, tuned_ratio=1e9)[1].S <= 2 ** 15


def test_route_rules(lib):
    # short rows: one workgroup per row while that is estimated cheaper than
    # the sampled route (the pass costs about 22 us whatever the size); long
    # or few rows: the sampled filter
    assert _plan(lib, 4096, 1, 10, 0)[1].path == 2
    assert _plan(lib, 5000, 300, 17, 0)[1].path == 2          # n < 8 S
    assert _plan(lib, 16384, 256, 16, 1)[1].path == 2         # one round of rows
    assert _plan(lib, 65536, 1, 10, 0)[1].path == 0           # config 2: 64 us vs 21 us
    assert _plan(lib, 65536, 64, 64, 1)[1].path == 0
    assert _plan(lib, 2 ** 18 - 1, 1, 10, 1)[1].path == 0
    assert _plan(lib, 2 ** 18, 1, 10, 1)[1].path == 0
    assert _plan(lib, 2 ** 28, 1, 64, 1)[1].path == 0
    # a buffer of half the row or more: exact select over the row
    assert _plan(lib, 2 ** 20, 1, 2 ** 19, 1)[1].path == 1
    # forced routes
    assert _plan(lib, 2 ** 22, 1, 64, 1, force_path=2)[1].path == 1
    assert _plan(lib, 5000, 1, 64, 1, force_path=1)[1].path == 0


def test_index_bits_and_key_bits(lib):
    info = _plan(lib, 2 ** 28, 1, 64, 2)[1]
    assert (info.index_bits, info.key_bits) == (32, 16)
    info = _plan(lib, 65536, 1, 10, 0)[1]
    assert (info.index_bits, info.key_bits) == (24, 32)
    info = _plan(lib, 255, 1, 10, 1)[1]
    assert info.index_bits == 8


@pytest.mark.parametrize("args,status", [
    ((100, 1, 0, 1), -1), ((100, 1, 101, 1), -1), ((0, 1, 1, 1), -1), ((100, 0, 1, 1), -1),
    ((100, 1, 1, 3), -2), ((100, 1, 1, -1), -2), ((2 ** 32, 1, 1, 1), -1), ((10, 70000, 1, 1), -1)])
def test_shape_errors(lib, args, status):
    assert _plan(lib, *args)[0] == status


@pytest.mark.parametrize("kw", [dict(eps=0.0), dict(eps=1.0), dict(s_min=0), dict(s_max=10),
                                dict(cost_ratio=0.0), dict(policy=3), dict(policy=-1),
                                dict(force_path=3), dict(S=-1), dict(tuned_ratio=0.0),
                                dict(tuned_s_min=0), dict(recall=0.0), dict(recall=1.5),
                                dict(recall=-0.5), dict(recall=float("nan")),
                                dict(tuned_ratio_batched=0.0), dict(tuned_batch_rows=0)])
def test_param_errors(lib, kw):
    assert _plan(lib, 2 ** 20, 1, 64, 1, **kw)[0] == -1


def test_forced_threshold_plans_the_sampled_route(lib):
    # a caller-given threshold runs the filter route whatever the shape (the
    # sampler is skipped), and cannot be combined with the forced exact route
    for n, rows, k in [(4096, 1, 10), (2 ** 28, 1, 64), (5000, 300, 17)]:
        rc, info = _plan(lib, n, rows, k, 1, use_force_tau=1, force_tau_key=0x80000000)
        assert rc == 0 and info.path == 0 and k <= info.cap <= n
    assert _plan(lib, 2 ** 20, 1, 64, 1, use_force_tau=1, force_path=2)[0] == -1
    assert _plan(lib, 2 ** 20, 1, 64, 1, test_flags=lib.TEST_BARRIER_GIVEUP)[0] == 0
    assert _plan(lib, 2 ** 20, 1, 64, 1, test_flags=2)[0] == -1


@pytest.mark.parametrize("n,k,recall", [(2 ** 28, 64, 0.95), (2 ** 24, 1000, 0.9),
                                        (2 ** 24, 10_000, 0.5), (2 ** 22, 7, 0.01)])
def test_relaxed_recall_plans_for_k_eff(lib, n, k, recall):
    # the parameters are chosen for k_eff = ceil(recall * k), priced with the
    # refine that runs for k; the buffer still holds k winners
    rc, info = _plan(lib, n, 1, k, 1, recall=recall)
    assert rc == 0
    k_eff = max(1, math.ceil(recall * k - 1e-9))
    assert info.k_eff == k_eff
    p = lib.default_params()
    ratio = p.tuned_ratio if k <= 4096 else p.tuned_ratio_large
    e = P.tuned(n, k_eff, eps=1e-3, s_hi=min(131072, n // 8), ratio=ratio)
    assert (info.S, info.t, info.M) == (e["S"], e["t"], e["M"])
    assert info.cap >= k
    # recall 1 plans for k itself
    assert _plan(lib, n, 1, k, 1)[1].k_eff == k
    # the recall failure it bounds is R < k_eff
    assert info.p_recall <= 5e-4 * (1 + 1e-9) and info.p_overflow <= 5e-4 * (1 + 1e-9)


def test_null_pointers_rejected_before_any_launch(lib):
    L = lib.lib
    assert L.topk(None, 100, 1, 10, 1, None, None, None, 0, None) == -1
    assert L.topk_plan(100, 1, 10, 1, None, None) == -1
    assert L.topk_workspace_size(100, 1, 10, 1, None, None) == -1
    assert L.topk_default_params(None) == -1


def test_workspace_size_is_plan_size(lib):
    sz = ctypes.c_size_t()
    assert lib.lib.topk_workspace_size(2 ** 28, 1, 64, 1, None, ctypes.byref(sz)) == 0
    info = _plan(lib, 2 ** 28, 1, 64, 1)[1]
    assert sz.value == info.workspace_bytes
    # never O(N): the candidate buffer is bounded by the plan's capacity
    assert sz.value < 8 * info.cap + 4 * 2 ** 20


def test_status_strings(lib):
    seen = set()
    for st in (0, -1, -2, -3, -4, -5, -6):
        s = lib.lib.topk_status_string(st)
        assert s
        seen.add(s)
    assert len(seen) == 7
