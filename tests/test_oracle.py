"""Pins for the CPU oracle's exact top-k (no GPU).

Each test checks the oracle against something other than itself: the O(n^2)
rank-by-counting definition, closed forms, numpy's own sorts on the float
values, the counting bisection, or invariants that fix the answer.
"""
import json
import os

import numpy as np
import pytest

import oracle
import workloads

GOLD = os.path.join(os.path.dirname(__file__), "golden")


def _check_rank_order(x, k, dtype=None):
    """Oracle output must equal the elements of rank 0..k-1 in rank order."""
    x = np.asarray(x)
    ranks = oracle.rank_by_counting(x, dtype)
    assert sorted(ranks.tolist()) == list(range(x.size)), "ranks must be a permutation"
    expect_idx = np.argsort(ranks)[:k]
    ov, oi = oracle.topk(x, k, dtype)
    assert oi[0].tolist() == expect_idx.tolist()
    assert ov[0].view(np.uint8).tobytes() == x[expect_idx].view(np.uint8).tobytes()


# ------------------------------------------------------------------ keys
def test_key_order_special_floats():
    vals = np.array([np.nan, np.inf, 1.0, 1e-45, 0.0, -0.0, -1e-45, -1.0, -np.inf],
                    dtype=np.float32)
    k = oracle.keys(vals)
    assert k[0] == 0xFFFFFFFF                       # NaN above everything
    assert k[1] > k[2] > k[3] > k[4]
    assert k[4] == k[5] == 0x80000000               # -0.0 is +0.0
    assert k[5] > k[6] > k[7] > k[8]
    neg_nan = np.array([0xFFC00001], dtype=np.uint32).view(np.float32)
    assert oracle.keys(neg_nan)[0] == 0xFFFFFFFF


def test_keys_numpy_and_c_agree():
    g = workloads.rng(7)
    f = g.standard_normal(20000).astype(np.float32)
    f[:6] = [np.nan, -np.nan, np.inf, -np.inf, 0.0, -0.0]
    raw = g.integers(0, 2 ** 32, 5000, dtype=np.uint64).astype(np.uint32)
    for arr, dt in [(f, None), (raw.view(np.float32), None),
                    (g.integers(-2 ** 31, 2 ** 31, 20000, dtype=np.int64).astype(np.int32), None),
                    (raw.astype(np.uint16), "bf16")]:
        assert np.array_equal(oracle.keys(arr, dt), oracle.keys_c(arr, dt))


def test_key_order_matches_numpy_sort_f32_i32_bf16():
    g = workloads.rng(11)
    f = (g.standard_normal(5000) * 100).astype(np.float32)
    o = np.argsort(oracle.keys(f), kind="stable")
    assert np.all(np.diff(f[o].astype(np.float64)) >= 0)
    i = g.integers(-2 ** 31, 2 ** 31, 5000, dtype=np.int64).astype(np.int32)
    i[:2] = [-2 ** 31, 2 ** 31 - 1]
    o = np.argsort(oracle.keys(i), kind="stable")
    assert np.all(np.diff(i[o].astype(np.int64)) >= 0)
    b = workloads.f32_to_bf16_bits(f)
    as_f = (b.astype(np.uint32) << 16).view(np.float32)
    o = np.argsort(oracle.keys(b, "bf16"), kind="stable")
    assert np.all(np.diff(as_f[o].astype(np.float64)) >= 0)


# ------------------------------------------------------------------ rank definition
def test_rank_figure_fixture():
    fx = json.load(open(os.path.join(GOLD, "rank_figure.json")))
    x = np.array(fx["scores"], dtype=np.int32)
    r = oracle.rank_by_counting(x)
    assert r[fx["highlighted"]] == fx["rank"]
    assert r[np.argmax(x)] == 0
    assert sorted(r.tolist()) == list(range(len(x)))


def test_topk_equals_rank_order_config1_full():
    x, dt, ks, _ = workloads.config("c1")
    row = x[0]
    for k in ks + [1, 100, 4096]:
        _check_rank_order(row, k)


@pytest.mark.parametrize("seed", range(6))
def test_topk_equals_rank_order_random_ties(seed):
    g = workloads.rng(100 + seed)
    n = int(g.integers(1, 700))
    k = int(g.integers(1, n + 1))
    _check_rank_order(g.integers(-3, 4, n).astype(np.int32), k)
    f = g.integers(-4, 5, n).astype(np.float32) * np.float32(0.5)
    f[g.random(n) < 0.1] = -0.0
    f[g.random(n) < 0.05] = np.nan
    _check_rank_order(f, k)
    b = workloads.f32_to_bf16_bits(g.standard_normal(n).astype(np.float32) * 4)
    _check_rank_order(b, k, "bf16")


# ------------------------------------------------------------------ closed forms
def test_closed_forms():
    n = 1000
    eq = np.full(n, 7, dtype=np.int32)
    assert oracle.topk(eq, 37)[1][0].tolist() == list(range(37))
    asc = np.arange(n, dtype=np.float32) - 500
    assert oracle.topk(asc, 5)[1][0].tolist() == [n - 1, n - 2, n - 3, n - 4, n - 5]
    desc = asc[::-1].copy()
    assert oracle.topk(desc, 5)[1][0].tolist() == [0, 1, 2, 3, 4]
    g = workloads.rng(3)
    x = g.integers(0, 20, n).astype(np.float32)
    # k = n: a full stable sort, value descending, lower index first on ties
    full = np.lexsort((np.arange(n), -x.astype(np.float64)))
    assert oracle.topk(x, n)[1][0].tolist() == full.tolist()
    # k = 1: the lowest-index maximum
    assert oracle.topk(x, 1)[1][0, 0] == int(np.argmax(x))


def test_planted_rows_closed_form():
    x = workloads.planted(4, 5000, 64, 99)
    ov, oi = oracle.topk(x, 64)
    for r in range(4):
        assert np.all(ov[r] == 1.0)
        assert oi[r].tolist() == sorted(np.flatnonzero(x[r] == 1.0).tolist())


def test_nan_and_signed_zero_bits_are_returned():
    x = np.array([0.0, -0.0, np.nan, 1.0, -np.nan, -0.0], dtype=np.float32)
    x[4] = np.array([0xFFC00001], dtype=np.uint32).view(np.float32)[0]
    ov, oi = oracle.topk(x, 6)
    assert oi[0].tolist() == [2, 4, 3, 0, 1, 5]
    assert ov[0].view(np.uint32).tolist() == x[[2, 4, 3, 0, 1, 5]].view(np.uint32).tolist()


def test_int32_extremes():
    x = np.array([5, -2 ** 31, 2 ** 31 - 1, 0, -1, 2 ** 31 - 1], dtype=np.int32)
    ov, oi = oracle.topk(x, 6)
    assert oi[0].tolist() == [2, 5, 0, 3, 4, 1]


def test_rejects_bad_arguments():
    x = np.zeros(10, dtype=np.float32)
    with pytest.raises(ValueError):
        oracle.topk(x, 11)
    with pytest.raises(ValueError):
        oracle.topk(x, 0)


# ------------------------------------------------------------------ invariants
def _invariant(row, ov, oi, dtype=None):
    rk = oracle.keys(row, dtype)
    k = oi.size
    for r in range(k):
        assert oracle.outranking(rk, int(rk[oi[r]]), int(oi[r])) == r


def test_invariant_exactly_r_outrank_output_r():
    g = workloads.rng(5)
    row = workloads.pareto_signed(1, 50000, 5)[0]
    ov, oi = oracle.topk(row, 50)
    _invariant(row, ov[0], oi[0])
    ir = g.integers(0, 300, 20000).astype(np.int32)
    ov, oi = oracle.topk(ir, 64)
    _invariant(ir, ov[0], oi[0])


# ------------------------------------------------------------------ config 2 and the bisection
def test_config2_bisection_cutoff():
    x, dt, ks, meta = workloads.config("c2")
    row = x[0]
    k = ks[0]
    ov, oi = oracle.topk(row, k)
    cutoff, count, steps = oracle.bisection_cutoff(row, k)
    assert count == k                          # exactly k scores clear it
    assert cutoff == int(ov[0, k - 1]) - 1     # integer scores: one below the k-th
    assert 15 <= steps <= 30
    # with equal k-th and (k+1)-th scores no cutoff separates them
    tied = np.array([9, 9, 8, 5, 5, 5, 1], dtype=np.int32)
    c, cnt, _ = oracle.bisection_cutoff(tied, 4)
    assert cnt != 4


def test_bf16_rounding_matches_torch():
    torch = pytest.importorskip("torch")
    x = workloads.rng(2).standard_normal(100000).astype(np.float32) * 3
    ours = workloads.f32_to_bf16_bits(x)
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(ours, ref)


# ------------------------------------------------- BatchTopK consumer
@pytest.mark.parametrize("dtype,seed", [("f32", 5), ("bf16", 6), ("i32", 7)])
def test_sparse_activation_is_the_rank_mask(dtype, seed):
    # Prof-K section 5: the kept activations are the K largest of the
    # flattened matrix.  The expected sparse activation is built straight
    # from the rank definition (elements of rank < K keep their bits, the
    # rest are zero), with no top-k or scatter involved.
    g = np.random.default_rng(seed)
    B, d, K = 12, 40, 37
    if dtype == "f32":
        x = np.maximum(g.standard_normal((B, d)).astype(np.float32), 0)   # ReLU: many ties at 0
        dt = None
    elif dtype == "bf16":
        x = workloads.f32_to_bf16_bits(np.maximum(g.standard_normal((B, d)), 0).astype(np.float32))
        dt = "bf16"
    else:
        x = g.integers(-5, 6, size=(B, d)).astype(np.int32)
        dt = None
    flat = x.reshape(-1)
    ranks = oracle.rank_by_counting(flat, dt)
    expect = np.where(ranks < K, flat, np.zeros_like(flat)).reshape(B, d)
    vals, idx = oracle.topk(flat, K, dt)
    dense, mask = oracle.sparse_activation(vals, idx, B * d)
    assert np.array_equal(dense.reshape(B, d).view(np.uint8), expect.view(np.uint8))
    assert np.array_equal(mask.reshape(-1), (ranks < K).astype(np.uint8))
    assert int(mask.sum()) == K


def test_sparse_activation_brute_force_rows():
    # a second, loop-by-loop construction on tiny batched rows
    g = np.random.default_rng(11)
    vals = g.standard_normal((3, 4)).astype(np.float32)
    idx = np.stack([g.permutation(9)[:4] for _ in range(3)]).astype(np.int64)
    dense, mask = oracle.sparse_activation(vals, idx, 9)
    for r in range(3):
        for c in range(9):
            hit = [j for j in range(4) if idx[r, j] == c]
            if hit:
                assert dense[r, c] == vals[r, hit[0]] and mask[r, c] == 1
            else:
                assert dense[r, c] == 0 and mask[r, c] == 0


def test_relaxed_selection_worked_example():
    # values 1 5 3 4 2, tau at 3.0: three survivors (5, 4, 3).  With k = 4
    # and k_eff = 3 they are kept and the fourth slot is padding; with
    # k_eff = 4 the row falls back to the exact answer; beyond the capacity
    # too.
    row = np.array([1, 5, 3, 4, 2], dtype=np.float32)
    tau = int(oracle.keys(np.array([3.0], dtype=np.float32))[0])
    v, i, part = oracle.relaxed_selection(row, 4, 3, tau, 10)
    assert part and i.tolist() == [1, 3, 2, -1]
    assert v[:3].tolist() == [5.0, 4.0, 3.0] and np.isneginf(v[3])
    v, i, part = oracle.relaxed_selection(row, 4, 4, tau, 10)
    assert not part and i.tolist() == [1, 3, 2, 4]
    v, i, part = oracle.relaxed_selection(row, 4, 3, tau, 2)
    assert not part and i.tolist() == [1, 3, 2, 4]
    # enough survivors: exact whatever k_eff
    tau2 = int(oracle.keys(np.array([2.0], dtype=np.float32))[0])
    v, i, part = oracle.relaxed_selection(row, 4, 1, tau2, 10)
    assert not part and i.tolist() == [1, 3, 2, 4]


@pytest.mark.parametrize("dt", ["float32", "int32", "bf16"])
def test_relaxed_selection_brute_force(dt):
    # every threshold a tiny row can have, against the rank definition: a
    # partial row keeps exactly the elements of rank < R, element of rank r
    # in slot r, so at least k_eff of the true top-k are returned; the pad
    # is the dtype's lowest value
    g = np.random.default_rng({"float32": 21, "int32": 22, "bf16": 23}[dt])
    for trial in range(30):
        n = int(g.integers(1, 40))
        base = g.integers(-4, 5, n)
        if dt == "int32":
            row = base.astype(np.int32)
        elif dt == "float32":
            row = (base * 0.5).astype(np.float32)
        else:
            row = workloads.f32_to_bf16_bits((base * 0.5).astype(np.float32))
        ranks = oracle.rank_by_counting(row, dt)
        kr = oracle.keys(row, dt).astype(np.int64)
        for tau in sorted(set(kr.tolist())) + [int(kr.max()) + 1]:
            R = int((kr >= tau).sum())
            for k in range(1, n + 1):
                for k_eff in range(1, k + 1):
                    cap = int(g.integers(1, n + 2))
                    v, i, part = oracle.relaxed_selection(row, k, k_eff, tau, cap, dt)
                    assert part == (k_eff <= R < k and R <= cap)
                    if not part:
                        assert i.tolist() == np.argsort(ranks, kind="stable")[:k].tolist()
                        continue
                    assert [int(ranks[j]) for j in i[:R]] == list(range(R))
                    assert (i[R:] == -1).all() and R >= k_eff
                    assert v[:R].tobytes() == row[i[:R]].tobytes()
                    pad = {"float32": np.float32(-np.inf), "int32": np.int32(-2 ** 31),
                           "bf16": np.uint16(0xFF80)}[dt]
                    assert (v[R:].tobytes() == np.full(k - R, pad).tobytes())


@pytest.mark.parametrize("dt", ["float32", "int32", "bf16"])
def test_chunked_selection_equals_single_thread(dt):
    # the threaded variant used for the CPU timing returns the same bits and
    # indices as the plain partial sort: heavy ties across chunk borders,
    # more threads than elements, k larger than a chunk, k = n
    g = np.random.default_rng({"float32": 31, "int32": 32, "bf16": 33}[dt])
    for n, k, threads in [(1, 1, 4), (5, 3, 8), (1000, 10, 7), (1000, 300, 16), (4099, 4099, 3),
                          (20000, 64, 16)]:
        base = g.integers(-3, 4, size=(2, n))
        if dt == "int32":
            x = base.astype(np.int32)
        elif dt == "float32":
            x = (base * 0.25).astype(np.float32)
        else:
            x = workloads.f32_to_bf16_bits((base * 0.25).astype(np.float32))
        v1, i1 = oracle.topk(x, k, dt)
        v2, i2 = oracle.topk_chunked(x, k, threads, dt)
        assert np.array_equal(i1, i2) and v1.tobytes() == v2.tobytes(), (n, k, threads)
    # and against the rank definition on one tiny row
    row = x[0, :50]
    ranks = oracle.rank_by_counting(row, dt)
    _, ic = oracle.topk_chunked(row, 20, 6, dt)
    assert ic[0].tolist() == np.argsort(ranks, kind="stable")[:20].tolist()
