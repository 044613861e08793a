"""GPU parity: the HIP library against the CPU oracle, element by element
(indices and value bits, tolerance 0), through the C ABI.

Sizes here finish on the oracle in seconds and still span many workgroup
tiles and ragged tails; the full headline shapes are in test_gpu_full.py.
"""
import numpy as np
import pytest

import oracle
import workloads
from gpu_util import assert_same, run_gpu, say, to_dev

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def _tss():
    import top_selection_sample_amd as tss
    return tss


def _seeded(seed, **kw):
    return _tss().default_params(seed=seed, use_seed=1, **kw)


# ------------------------------------------------------------ small configs
def test_config1_heavy_ties():
    x, dt, ks, _ = workloads.config("c1")
    say("config 1: int32 [1, 4096] k=10")
    gv, gi = run_gpu(x, 10, dt)
    assert_same(gv, gi, x, 10, dt, "c1")
    ranks = oracle.rank_by_counting(x[0])
    assert gi[0].tolist() == np.argsort(ranks)[:10].tolist()


def test_config2_and_bisection():
    x, dt, ks, meta = workloads.config("c2")
    say(f"config 2: int32 [1, 65536] k=10 seed {meta['seed']}")
    gv, gi = run_gpu(x, 10, dt)
    assert_same(gv, gi, x, 10, dt, "c2")
    cutoff, count, _ = oracle.bisection_cutoff(x[0], 10)
    assert count == 10 and cutoff == int(gv[0, 9]) - 1


# ------------------------------------------------------------ edge cases
def _edge_rows(dt, n, kind, seed):
    g = workloads.rng(seed)
    if kind == "equal":
        base = np.full(n, 3.0)
    elif kind == "asc":
        base = np.arange(n, dtype=np.float64) - n / 2
    elif kind == "desc":
        base = -(np.arange(n, dtype=np.float64) - n / 2)
    elif kind == "ties":
        base = g.integers(-5, 6, n).astype(np.float64)
    else:
        base = g.standard_normal(n) * 100
    if dt == "int32":
        x = base.astype(np.int32)
        if kind == "special":
            x[: min(n, 4)] = np.array([2 ** 31 - 1, -2 ** 31, 0, -1], dtype=np.int32)[: min(n, 4)]
        return x[None, :]
    f = base.astype(np.float32)
    if kind == "special":
        sp = np.array([np.nan, np.inf, -np.inf, -0.0, 0.0, 1e-45, -1e-45], dtype=np.float32)
        f[g.choice(n, min(n, 40), replace=False)] = sp[g.integers(0, len(sp), min(n, 40))]
        if n > 3:
            f[1] = np.array([0xFFC00001], dtype=np.uint32).view(np.float32)[0]   # negative NaN
    if dt == "bf16":
        b = f.view(np.uint32)
        nan = (b & 0x7FFFFFFF) > 0x7F800000
        out = workloads.f32_to_bf16_bits(np.where(nan, 0, f).astype(np.float32))
        out[nan] = (b[nan] >> 16).astype(np.uint16) | 0x0040
        return out[None, :]
    return f[None, :]


@pytest.mark.parametrize("dt", ["float32", "int32", "bf16"])
@pytest.mark.parametrize("kind", ["equal", "asc", "desc", "ties", "special", "normal"])
@pytest.mark.parametrize("n,k", [(1, 1), (7, 3), (7, 7), (1000, 1), (1000, 1000), (4099, 64),
                                 (70001, 4096), (70001, 4097), (300007, 33)])
def test_edge_shapes(dt, kind, n, k):
    x = _edge_rows(dt, n, kind, n + k)
    say(f"edge {dt} {kind} n={n} k={k}")
    gv, gi = run_gpu(x, k, dt)
    assert_same(gv, gi, x, k, dt, f"{dt}/{kind}/{n}/{k}")


@pytest.mark.parametrize("offset", [1, 2, 3, 5])
def test_offset_pointer(offset):
    # a view that starts at an element offset: rows are not 16-byte aligned
    full = workloads.normal_f32(1, 400_000 + offset, 31)[0]
    x = full[offset:][None, :]
    say(f"offset pointer {offset}")
    xt = to_dev(full, "float32")[offset:]
    gv, gi = run_gpu(x, 100, "float32", xt=xt.reshape(1, -1))
    assert_same(gv, gi, x, 100, "float32", "offset")
    xb = workloads.relu_bf16(1, 400_000 + offset, 32)[0]
    xbt = to_dev(xb, "bf16")[offset:]
    gv, gi = run_gpu(xb[offset:][None, :], 100, "bf16", xt=xbt.reshape(1, -1))
    assert_same(gv, gi, xb[offset:][None, :], 100, "bf16", "offset bf16")


# ------------------------------------------------------------ sampled route
@pytest.mark.parametrize("k", [1, 16, 64, 2048, 4096])
def test_sampled_route_fp32(k):
    n = 3 * 2 ** 20 + 77
    x = workloads.normal_f32(1, n, 100 + k)
    say(f"sampled fp32 n={n} k={k}")
    gv, gi = run_gpu(x, k, "float32")
    assert_same(gv, gi, x, k, "float32", f"sampled k={k}")
    st = _tss().read_stats(1)
    assert st[0]["path"] in (0, 1)


@pytest.mark.parametrize("dt", ["float32", "int32", "bf16"])
def test_tau_and_R_match_sampler_spec(dt):
    """The device's threshold key and survivor count equal the oracle's
    sampler for the same seed (Prof-K stages 1-3)."""
    n = 2 ** 21 + 13
    if dt == "int32":
        x = workloads.scores_int(1, n, -10 ** 6, 10 ** 6, 41)
    elif dt == "bf16":
        x = workloads.relu_bf16(1, n, 42)
    else:
        x = workloads.pareto_signed(1, n, 43)
    k = 64
    tss = _tss()
    pl = tss.plan(n, 1, k, dt)
    for seed in (1, 2, 3):
        p = _seeded(seed)
        say(f"tau/R {dt} seed {seed}")
        gv, gi = run_gpu(x, k, dt, params=p)
        assert_same(gv, gi, x, k, dt, f"tau {dt}")
        st = tss.read_stats(1)[0]
        tk, R = oracle.tau(x[0], seed, 0, pl["S"], pl["t"], dt)
        assert st["tau_key"] == tk
        assert st["r_sampled"] == R
        path, G, E = _expected_route(x[0], dt, tk, k, pl["cap"])
        assert st["path"] == path and st["ties"] == E


def _expected_path(row, dt, tau_key, k, cap):
    return _expected_route(row, dt, tau_key, k, cap)[0]


def _expected_route(row, dt, tau_key, k, cap):
    """Route of a sampled row: the survivors split at tau into G above and E
    equal; the row is accepted when G alone holds k of them within the
    capacity, or when G < k <= G + E <= cap (the ties join the candidates)."""
    kk = oracle.keys(row, dt).astype(np.int64)
    G = int((kk > tau_key).sum())
    E = int((kk == tau_key).sum())
    if G > cap:
        return 1, G, E
    if G >= k:
        return 0, G, E
    return (0 if k <= G + E <= cap else 1), G, E


def test_forced_overflow_fallback():
    n = 2 ** 21 + 5
    x = workloads.normal_f32(1, n, 51)
    p = _seeded(7, M=100, force_path=1)
    say("forced overflow")
    gv, gi = run_gpu(x, 64, "float32", params=p)
    assert_same(gv, gi, x, 64, "float32", "overflow")
    st = _tss().read_stats(1)[0]
    assert st["path"] == 1 and st["r_sampled"] > 100 and st["flags"] == 0


def test_forced_recall_failure_fallback():
    n = 2 ** 21 + 5
    x = workloads.normal_f32(1, n, 52)
    p = _seeded(8, t=1, force_path=1)       # tau = sample maximum: R is small
    say("forced recall failure")
    gv, gi = run_gpu(x, 1000, "float32", params=p)
    assert_same(gv, gi, x, 1000, "float32", "recall")
    st = _tss().read_stats(1)[0]
    assert st["path"] == 1 and st["r_sampled"] < 1000 and st["flags"] == 0


@pytest.mark.parametrize("dt", ["float32", "bf16"])
def test_forced_exact_large_row(dt):
    n = 2 ** 22 + 3
    x = workloads.normal_f32(1, n, 53) if dt == "float32" else workloads.relu_bf16(1, n, 53)
    p = _tss().default_params(force_path=2)
    say(f"forced exact {dt}")
    for k in (10, 5000):
        gv, gi = run_gpu(x, k, dt, params=p)
        assert_same(gv, gi, x, k, dt, f"exact {dt} k={k}")
        assert _tss().read_stats(1)[0]["path"] == 2


def test_exact_route_all_equal_large_row():
    # ties far beyond the buffer capacity: the index digits decide
    n = 2 ** 21
    x = np.full((1, n), 2.5, dtype=np.float32)
    p = _tss().default_params(force_path=2)
    gv, gi = run_gpu(x, 300, "float32", params=p)
    assert_same(gv, gi, x, 300, "float32", "all-equal exact")
    gv, gi = run_gpu(x, 300, "float32")
    assert_same(gv, gi, x, 300, "float32", "all-equal auto")


def _plateau_row(n, n_top, n_tie, seed):
    # n_top distinct large values, n_tie copies of 5.0, the rest far below
    g = workloads.rng(seed)
    x = (g.standard_normal(n) - 1000.0).astype(np.float32)
    pos = g.choice(n, n_top + n_tie, replace=False)
    x[pos[:n_top]] = 10.0 + np.arange(n_top, dtype=np.float32)
    x[pos[n_top:]] = 5.0
    return x[None, :]


def test_ties_join_candidates():
    # 32 values above the plateau, k = 64: the threshold lands on the plateau
    # (w.h.p.), so the 32 lowest-index ties complete the answer from the tie region
    n, k = 2 ** 20, 64
    x = _plateau_row(n, 32, 50_000, 71)
    tss = _tss()
    p = _seeded(11, M=100_000, force_path=1)
    pl = tss.plan(n, 1, k, "float32", params=p)
    say("ties join the candidates")
    gv, gi = run_gpu(x, k, "float32", params=p)
    assert_same(gv, gi, x, k, "float32", "ties join")
    st = tss.read_stats(1)[0]
    tk, R = oracle.tau(x[0], 11, 0, pl["S"], pl["t"], "float32")
    assert st["tau_key"] == tk and st["r_sampled"] == R
    path, G, E = _expected_route(x[0], "float32", tk, k, pl["cap"])
    assert st["path"] == path and st["ties"] == E
    if tk == int(oracle.keys(np.array([5.0], dtype=np.float32))[0]):
        assert st["path"] == 0


def test_ties_beyond_capacity_fall_back():
    # the same, but the plateau does not fit the buffer: exact route
    n, k = 2 ** 20, 64
    x = _plateau_row(n, 32, 200_000, 72)
    tss = _tss()
    p = _seeded(12, M=100_000, force_path=1)
    pl = tss.plan(n, 1, k, "float32", params=p)
    say("ties beyond the capacity")
    gv, gi = run_gpu(x, k, "float32", params=p)
    assert_same(gv, gi, x, k, "float32", "ties overflow")
    st = tss.read_stats(1)[0]
    tk, R = oracle.tau(x[0], 12, 0, pl["S"], pl["t"], "float32")
    assert st["path"] == _expected_path(x[0], "float32", tk, k, pl["cap"])


def test_ties_ignored_when_enough_above():
    # all zeros but k ones: tau is 0 (w.h.p.) and the k ones alone are the
    # answer, so the row is accepted whatever the number of ties
    rows, n, k = 4, 2 ** 20, 64
    x = workloads.planted(rows, n, 64, 73)
    say("ties ignored")
    for dt in ("float32", "bf16"):
        xx = x if dt == "float32" else workloads.f32_to_bf16_bits(x)
        gv, gi = run_gpu(xx, k, dt)
        assert_same(gv, gi, xx, k, dt, f"planted {dt}")
        assert [r["path"] for r in _tss().read_stats(rows)] == [0] * rows


# ------------------------------------------------------------ batched rows
@pytest.mark.parametrize("variant", ["c4v1", "c4v2", "c4v3"])
def test_batched_rows_reduced(variant):
    rows, n, k = 12, 2 ** 20, 64
    if variant == "c4v3":
        x = workloads.planted(rows, n, 64, 61)
    else:
        x = workloads.pareto_signed(rows, n, 61)
        if variant == "c4v2":
            x = workloads.sorted_rows(x)
    say(f"batched {variant} rows={rows}")
    gv, gi = run_gpu(x, k, "float32")
    assert_same(gv, gi, x, k, "float32", variant)


def test_more_rows_than_workgroups_with_failures():
    # rows > compute units: a finishing workgroup owns several rows; every
    # 7th row is constant, so its sampled threshold admits the whole row
    # (overflow) and the row takes the exact route beside refined rows
    rows, n, k = 300, 2 ** 18, 16
    x = workloads.normal_f32(rows, n, 91)
    x[::7] = 1.5
    say(f"mixed failures rows={rows}")
    gv, gi = run_gpu(x, k, "float32")
    assert_same(gv, gi, x, k, "float32", "mixed rows")
    st = _tss().read_stats(rows)
    assert [r["path"] for r in st[::7]] == [1] * len(st[::7])
    assert sum(r["path"] == 0 for r in st) >= rows - len(st[::7]) - 3


def test_rows_listed_by_check_kernel():
    # more rows than one workgroup scans: a separate kernel lists the failures
    rows, n, k = 1030, 2 ** 18, 8
    x = workloads.scores_int(rows, n, -2 ** 31, 2 ** 31 - 1, 92)
    x[5::97] = 7
    say(f"listed failures rows={rows}")
    gv, gi = run_gpu(x, k, "int32")
    assert_same(gv, gi, x, k, "int32", "listed rows")
    st = _tss().read_stats(rows)
    assert all(r["path"] == 1 for r in st[5::97])


def test_batched_small_rows_exact():
    x = workloads.scores_int(300, 5000, 0, 50, 62)
    gv, gi = run_gpu(x, 17, "int32")
    assert_same(gv, gi, x, 17, "int32", "small rows")


# ------------------------------------------------------------ large k
def test_large_k_bf16_sampled():
    x = workloads.relu_bf16(1, 2 ** 23, 71)
    k = 8192
    say("large k bf16 sampled")
    gv, gi = run_gpu(x, k, "bf16")
    assert_same(gv, gi, x, k, "bf16", "large k")


@pytest.mark.parametrize("dt,S", [("bf16", 1024), ("bf16", 2048), ("float32", 1024)])
def test_large_k_sampled_short_row(dt, S):
    # a short row filtered by two workgroups: each wave stages hundreds of
    # candidates and flushes its stage several times on the way; the bucket
    # histogram's candidate count must include those flushes (the row is
    # accepted for these seeds: 6,000-7,300 candidates, buffer 7,884-9,278)
    n, k = 70_000, 5000
    x = workloads.relu_bf16(1, n, 9) if dt == "bf16" else workloads.normal_f32(1, n, 9)
    for seed in (0, 1):
        say(f"large k short row {dt} S={S} seed={seed}")
        gv, gi = run_gpu(x, k, dt, params=_seeded(seed, S=S, force_path=1))
        assert_same(gv, gi, x, k, dt, f"short row {dt} S={S} seed={seed}")
        assert _tss().read_stats(1)[0]["path"] == 0


def test_large_k_batched_fp32():
    x = workloads.normal_f32(3, 2 ** 20 + 3, 72)
    k = 20000
    gv, gi = run_gpu(x, k, "float32")
    assert_same(gv, gi, x, k, "float32", "large k rows")


def test_large_k_exact_small_rows():
    x = workloads.scores_int(2, 100_000, 0, 300, 73)
    gv, gi = run_gpu(x, 60_000, "int32")
    assert_same(gv, gi, x, 60_000, "int32", "large k exact")


def test_full_sort_k_equals_n():
    x = workloads.normal_f32(1, 50_000, 74)
    gv, gi = run_gpu(x, 50_000, "float32")
    assert_same(gv, gi, x, 50_000, "float32", "k = n")


def test_large_k_oversized_bucket():
    # zeros with a few huge values: the exact route keeps the huge values and
    # the lowest-index zeros; the zeros share one key far below the largest,
    # so they land in one bucket too big for one LDS sort and get split on
    # their index bits
    n, k = 2 ** 20, 20_000
    g = workloads.rng(75)
    x = np.zeros((1, n), dtype=np.float32)
    x[0, g.choice(n, 100, replace=False)] = (1e30 * (1 + g.random(100))).astype(np.float32)
    say("large k oversized bucket")
    gv, gi = run_gpu(x, k, "float32")
    assert_same(gv, gi, x, k, "float32", "oversized bucket")


def test_large_k_two_rows_ties_and_spread():
    # two rows: one with heavy bf16 ties, one all-equal (every candidate in
    # one key): both through the bucket sort
    n, k = 2 ** 20, 9000
    x = workloads.relu_bf16(2, n, 76)
    x[1] = x[1, 0] if x[1, 0] != 0 else np.uint16(0x3F80)
    say("large k ties and all-equal")
    gv, gi = run_gpu(x, k, "bf16")
    assert_same(gv, gi, x, k, "bf16", "large k ties")


def test_large_k_beyond_bucket_capacity():
    # a buffer larger than the bucket sort handles: tile sort and merges
    n, k = 2 ** 21 + 11, 2 ** 20 + 5
    x = workloads.normal_f32(1, n, 77)
    say("large k merge path")
    tss = _tss()
    assert tss.plan(n, 1, k, "float32")["cap"] > 2 ** 21
    gv, gi = run_gpu(x, k, "float32")
    assert_same(gv, gi, x, k, "float32", "merge path")


# ------------------------------------------------------------ determinism
def test_repeat_with_fresh_seeds_is_identical():
    x = workloads.relu_bf16(1, 2 ** 22, 81)
    xt = to_dev(x, "bf16")
    first = run_gpu(x, 4096, "bf16", xt=xt)
    for _ in range(20):
        again = run_gpu(x, 4096, "bf16", xt=xt)
        assert np.array_equal(first[0], again[0]) and np.array_equal(first[1], again[1])
    assert_same(first[0], first[1], x, 4096, "bf16", "repeat")


def test_argument_errors():
    tss = _tss()
    x = torch.zeros(1, 100, device="cuda")
    with pytest.raises(tss.TopkError):
        tss.topk(x, 101)
    with pytest.raises(tss.TopkError):
        tss.topk(x, 0)
    with pytest.raises(TypeError):
        tss.topk(x.double(), 5)


def test_out_tensors_checked_and_empty_batch():
    tss = _tss()
    x = torch.randn(3, 1000, device="cuda")
    good = (torch.empty(3, 7, device="cuda"), torch.empty(3, 7, dtype=torch.int64, device="cuda"))
    v, i = tss.topk(x, 7, out=good)
    assert v.data_ptr() == good[0].data_ptr() and i.data_ptr() == good[1].data_ptr()
    ov, oi = oracle.topk(x.cpu().numpy(), 7)
    assert np.array_equal(i.cpu().numpy(), oi)
    bad = [(torch.empty(3, 6, device="cuda"), good[1]),                        # too small
           (good[0], torch.empty(3, 7, dtype=torch.int32, device="cuda")),     # index dtype
           (torch.empty(3, 7, dtype=torch.bfloat16, device="cuda"), good[1]),  # value dtype
           (torch.empty(7, 3, device="cuda").t(), good[1]),                    # not contiguous
           (torch.empty(3, 7), good[1])]                                       # host memory
    for o in bad:
        with pytest.raises(ValueError):
            tss.topk(x, 7, out=o)
    # an empty batch gives empty outputs, and still checks k
    e = torch.empty(0, 1000, device="cuda")
    v, i = tss.topk(e, 5)
    assert v.shape == (0, 5) and i.shape == (0, 5) and i.dtype == torch.int64
    with pytest.raises(tss.TopkError):
        tss.topk(e, 1001)


def test_filter_trace_stamps_every_workgroup():
    # the workgroup trace (a measurement aid) stamps every filter workgroup's
    # start and end, leaves the answer exact, and stops when cleared
    tss = _tss()
    x = workloads.normal_f32(3, 2 ** 20 + 9, 431)
    xt = to_dev(x, "float32")
    trace = torch.zeros(2 * 4096, dtype=torch.int64, device="cuda")
    tss.filter_trace(trace)
    try:
        say("filter trace: 3 rows")
        v, i = tss.topk(xt, 64)
        torch.cuda.synchronize()
    finally:
        tss.filter_trace(None)
    assert np.array_equal(i.cpu().numpy(), oracle.topk(x, 64)[1])
    t = trace.cpu().numpy().reshape(-1, 2)
    used = np.nonzero(t[:, 0])[0]
    assert len(used) >= 3 and np.array_equal(used, np.arange(len(used)))   # rows x workgroups
    assert len(used) % 3 == 0
    assert (t[used, 1] > t[used, 0]).all()
    assert (t[used, 1] - t[used, 0]).max() < 100 * 100_000   # under 100 ms at 100 MHz
    assert not t[len(used):].any()
    trace.zero_()
    tss.topk(xt, 64)
    torch.cuda.synchronize()
    assert not trace.cpu().numpy().any()   # stopped
    with pytest.raises(ValueError):
        tss.filter_trace(torch.zeros(4, dtype=torch.int32, device="cuda"))


def test_stream_read_reads_and_writes_nothing():
    # the read-ceiling aid: valid sizes run, a ragged or misaligned buffer
    # is refused, and the data and the sink are left as they were
    tss = _tss()
    x = torch.arange(1 << 20, dtype=torch.int32, device="cuda")
    sink = torch.full((64,), -7, dtype=torch.int32, device="cuda")
    before = x.clone()
    tss.stream_read(x, sink)
    tss.stream_read(x[: (1 << 20) - 4 * 1000 - 4], sink)   # a ragged last step
    torch.cuda.synchronize()
    assert torch.equal(x, before)
    assert bool((sink == -7).all())
    with pytest.raises(tss.TopkError):
        tss.stream_read(x[1:5], sink)   # 4-byte aligned only
    with pytest.raises(tss.TopkError):
        tss.stream_read(x[:3], sink)    # 12 bytes


# ------------------------------------------------- BatchTopK consumer
def _dense_to_host(t, dt):
    import numpy as np
    if dt == "bf16":
        return t.view(torch.int16).cpu().numpy().view(np.uint16)
    return t.cpu().numpy()


@pytest.mark.parametrize("dt,rows,n,k", [("float32", 3, 5000, 37), ("bf16", 2, 70001, 900),
                                         ("int32", 1, 4096, 4096), ("float32", 4, 300000, 5000)])
def test_scatter_matches_oracle(dt, rows, n, k):
    from gpu_util import vals_to_host
    tss = _tss()
    g = np.random.default_rng(rows * 1000 + k)
    if dt == "float32":
        x = np.maximum(g.standard_normal((rows, n)), 0).astype(np.float32)
    elif dt == "bf16":
        x = workloads.f32_to_bf16_bits(np.maximum(g.standard_normal((rows, n)), 0).astype(np.float32))
    else:
        x = g.integers(-50, 50, size=(rows, n)).astype(np.int32)
    say(f"scatter {dt} rows={rows} n={n} k={k}")
    xt = to_dev(x, dt)
    v, i = tss.topk(xt, k)
    out, m = tss.scatter(v, i, n, mask=True)
    torch.cuda.synchronize()
    ov, oi = oracle.topk(x, k, dt)
    edense, emask = oracle.sparse_activation(ov, oi, n)
    assert _dense_to_host(out, dt).tobytes() == edense.tobytes()
    assert np.array_equal(m.cpu().numpy(), emask)


def test_batchtopk_flattened_matches_oracle():
    tss = _tss()
    g = np.random.default_rng(77)
    B, d, K = 64, 4096, 2048
    x = workloads.f32_to_bf16_bits(np.maximum(g.standard_normal((B, d)), 0).astype(np.float32))
    say(f"batchtopk bf16 [{B}, {d}] K={K}")
    acts = to_dev(x, "bf16")
    out, m = tss.batchtopk(acts, K, mask=True)
    torch.cuda.synchronize()
    ov, oi = oracle.topk(x.reshape(1, -1), K, "bf16")
    edense, emask = oracle.sparse_activation(ov, oi, B * d)
    assert out.shape == (B, d) and m.shape == (B, d)
    assert _dense_to_host(out, "bf16").reshape(-1).tobytes() == edense.reshape(-1).tobytes()
    assert np.array_equal(m.cpu().numpy().reshape(-1), emask.reshape(-1))


def test_scatter_unaligned_output_and_errors():
    # an output that starts 2 bytes past a 16-byte boundary: head and tail
    # bytes of the zero fill; stale data must not survive
    tss = _tss()
    n, k = 1000, 10
    x = torch.arange(n, dtype=torch.float32, device="cuda").reshape(1, n)
    v, i = tss.topk(x, k)
    big = torch.full((1 + n + 15,), float("nan"), dtype=torch.bfloat16, device="cuda")
    vb = v.to(torch.bfloat16)
    out = big[1:1 + n]
    tss.scatter(vb, i, n, out=out)
    torch.cuda.synchronize()
    got = out.float().cpu().numpy()
    expect = np.zeros(n, dtype=np.float32)
    expect[i.cpu().numpy().reshape(-1)] = vb.float().cpu().numpy().reshape(-1)   # bf16-rounded
    assert np.array_equal(got, expect)
    assert int(np.count_nonzero(got)) == k
    assert bool(torch.isnan(big[0].float())) and bool(torch.isnan(big[1 + n].float()))
    lib = tss._lib.lib
    with pytest.raises(tss.TopkError):
        tss._lib.check(lib.topk_scatter(v.data_ptr(), i.data_ptr(), 1, k, n, 1, None, None, None), "s")
    with pytest.raises(tss.TopkError):
        tss._lib.check(lib.topk_scatter(v.data_ptr(), i.data_ptr(), 1, n + 1, n, 1, out.data_ptr(),
                                        None, None), "s")


# ------------------------------------------------------------ relaxed recall
def _relaxed_case(x, dt, k, S, seed, recall=None, M=100_000):
    """Run one relaxed-recall call with the sampler forced to t = 1 (tau is
    the sample maximum, so few elements survive) and compare every row with
    the oracle's relaxed selection for the same threshold.  recall=None sets
    the target so that k_eff equals the first row's survivor count."""
    tss = _tss()
    rows, n = x.shape
    kw = dict(S=S, t=1, M=M, force_path=1)
    pl = tss.plan(n, rows, k, dt, params=_seeded(seed, **kw))
    taus = [oracle.tau(x[r], seed, r, pl["S"], pl["t"], dt) for r in range(rows)]
    if recall is None:
        recall = taus[0][1] / k
    p = _seeded(seed, recall=recall, **kw)
    pl = tss.plan(n, rows, k, dt, params=p)
    k_eff = pl["k_eff"]
    say(f"relaxed recall {dt} rows={rows} n={n} k={k} k_eff={k_eff} S={S} seed={seed}")
    gv, gi = run_gpu(x, k, dt, params=p)
    st = tss.read_stats(rows)
    gv, gi = gv.reshape(rows, k), gi.reshape(rows, k)
    kinds = []
    for r in range(rows):
        tk, R = taus[r]
        ov, oi, part = oracle.relaxed_selection(x[r], k, k_eff, tk, pl["cap"], dt)
        if not np.array_equal(gi[r], oi):
            c = int(np.argwhere(gi[r] != oi)[0][0])
            raise AssertionError(f"row {r} R={R}: index differs at slot {c}: gpu {gi[r, c]} "
                                 f"oracle {oi[c]}")
        assert gv[r].tobytes() == ov.tobytes(), f"row {r}: value bits differ"
        assert st[r]["tau_key"] == tk and st[r]["r_sampled"] == R
        assert st[r]["path"] == (3 if part else (0 if R >= k else 1)), (r, R, st[r])
        kinds.append("partial" if part else ("accepted" if R >= k else "fallback"))
    return kinds


@pytest.mark.parametrize("dt,gen_seed", [("float32", 301), ("int32", 301), ("bf16", 301)])
def test_relaxed_recall_keeps_partial_row(dt, gen_seed):
    # k = 4096, about n/S = 1000 survivors: the row keeps them (sorted in
    # the workgroup) and pads the remaining slots
    n = 2 ** 21 + 9
    if dt == "float32":
        x = workloads.normal_f32(1, n, gen_seed)
    elif dt == "int32":
        x = workloads.scores_int(1, n, -10 ** 6, 10 ** 6, gen_seed)
    else:
        x = workloads.relu_bf16(1, n, gen_seed)
    assert _relaxed_case(x, dt, 4096, 2048, 31) == ["partial"]


def test_relaxed_recall_few_survivors_ranked():
    # fewer than 256 survivors: the rank-by-counting writer
    x = workloads.normal_f32(1, 2 ** 21 + 9, 302)
    assert _relaxed_case(x, "float32", 512, 16384, 32) == ["partial"]


@pytest.mark.parametrize("dt,gen_seed,seed", [("float32", 303, 33), ("bf16", 304, 34)])
def test_relaxed_recall_large_k_bucket_sort(dt, gen_seed, seed):
    # k = 20000 with a few hundred survivors: the bucket sort writes them and
    # every later sort window is padding
    n = 2 ** 21 + 9
    x = workloads.normal_f32(1, n, gen_seed) if dt == "float32" else workloads.relu_bf16(1, n, gen_seed)
    assert _relaxed_case(x, dt, 20_000, 1024, seed) == ["partial"]


def test_relaxed_recall_merge_path():
    # k beyond the bucket sort's capacity: tile sort, merges, padded output
    x = workloads.normal_f32(1, 2 ** 22 + 3, 305)
    assert _tss().plan(2 ** 22 + 3, 1, 2 ** 21 + 1, "float32")["cap"] > 2 ** 21
    assert _relaxed_case(x, "float32", 2 ** 21 + 1, 1024, 35) == ["partial"]


def test_relaxed_recall_mixed_rows():
    # recall 0.5, k = n/S: rows with k or more survivors are exact, rows with
    # at least k/2 keep theirs, rows with fewer fall back to the exact route
    x = workloads.normal_f32(12, 2 ** 20, 306)
    kinds = _relaxed_case(x, "float32", 1024, 1024, 36, recall=0.5)
    assert {"partial", "accepted", "fallback"} <= set(kinds), kinds


def test_relaxed_recall_rows_listed_by_check_kernel():
    # more rows than one workgroup scans: the check kernel applies the same
    # three-way verdict
    x = workloads.scores_int(1030, 2 ** 16, -2 ** 31, 2 ** 31 - 1, 307)
    kinds = _relaxed_case(x, "int32", 512, 128, 37, recall=0.5)
    assert {"partial", "accepted", "fallback"} <= set(kinds)


def test_relaxed_selection_scatters_kept_slots_only():
    # a partial row's padded slots (index -1) write nothing in the consumer
    tss = _tss()
    n, k, S, seed = 2 ** 21 + 9, 4096, 2048, 31
    x = workloads.normal_f32(1, n, 301)
    kw = dict(S=S, t=1, M=100_000, force_path=1)
    pl = tss.plan(n, 1, k, "float32", params=_seeded(seed, **kw))
    tk, R = oracle.tau(x[0], seed, 0, pl["S"], pl["t"], "float32")
    p = _seeded(seed, recall=R / k, **kw)
    say(f"relaxed selection into the consumer, R={R}")
    xt = to_dev(x, "float32")
    v, i = tss.topk(xt, k, params=p)
    out, m = tss.scatter(v, i, n, mask=True)
    torch.cuda.synchronize()
    ov, oi, part = oracle.relaxed_selection(x[0], k, R, tk, tss.plan(n, 1, k, "float32", params=p)["cap"])
    assert part and (oi[R:] == -1).all()
    edense, emask = oracle.sparse_activation(ov[None, :R], oi[None, :R], n)
    assert _dense_to_host(out, "float32").tobytes() == edense.tobytes()
    assert np.array_equal(m.cpu().numpy(), emask)


@pytest.mark.parametrize("case", ["sampled", "large_k", "small_rows"])
def test_graph_capture_replays_match(case):
    # one topk call captured in a HIP graph (on its own workspace, allocated
    # before the capture), replayed several times with eager work and
    # synchronisations in between; every replay must equal the oracle
    tss = _tss()
    if case == "sampled":
        x, k = workloads.normal_f32(2, 2 ** 21 + 7, 401), 64
    elif case == "large_k":
        x, k = workloads.normal_f32(1, 2 ** 21 + 7, 402), 5000
    else:
        x, k = workloads.scores_int(5, 3000, 0, 40, 403), 17
    dt = "int32" if x.dtype == np.int32 else "float32"
    say(f"graph capture: {case} rows={x.shape[0]} n={x.shape[1]} k={k}")
    xt = to_dev(x, dt)
    ev, ei = oracle.topk(x, k, dt)
    ws = tss.Workspace()
    ov = torch.empty((x.shape[0], k), dtype=xt.dtype, device="cuda")
    oi = torch.empty((x.shape[0], k), dtype=torch.int64, device="cuda")
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        tss.topk(xt, k, workspace=ws, out=(ov, oi))   # sizes the workspace
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        tss.topk(xt, k, workspace=ws, out=(ov, oi))
    torch.cuda.synchronize()
    other = torch.randn(3, 50_000, device="cuda")
    for rep in range(4):
        ov.zero_()
        oi.fill_(-1)
        g.replay()
        torch.cuda.synchronize()
        assert np.array_equal(oi.cpu().numpy(), ei), f"replay {rep}: indices differ"
        assert ov.cpu().numpy().tobytes() == ev.tobytes(), f"replay {rep}: values differ"
        # eager work between replays, on the default workspace
        v2, i2 = tss.topk(other, 9)
        torch.cuda.synchronize()
        assert np.array_equal(i2.cpu().numpy(), oracle.topk(other.cpu().numpy(), 9)[1])
    del g


def test_two_streams_default_workspaces():
    # calls on two streams at once, each with its stream's default workspace:
    # both answers exact
    tss = _tss()
    xa = workloads.normal_f32(2, 2 ** 21 + 1, 501)
    xb = workloads.pareto_signed(3, 2 ** 20 + 3, 502)
    ta, tb = to_dev(xa, "float32"), to_dev(xb, "float32")
    sa, sb = torch.cuda.Stream(), torch.cuda.Stream()
    torch.cuda.synchronize()
    say("two streams, default workspaces")
    outs = []
    for rep in range(3):
        with torch.cuda.stream(sa):
            va, ia = tss.topk(ta, 64)
        with torch.cuda.stream(sb):
            vb, ib = tss.topk(tb, 300)
        torch.cuda.synchronize()
        outs.append((ia.cpu().numpy(), ib.cpu().numpy()))
    ea, eb = oracle.topk(xa, 64)[1], oracle.topk(xb, 300)[1]
    for ia, ib in outs:
        assert np.array_equal(ia, ea) and np.array_equal(ib, eb)


@pytest.mark.parametrize("dt", ["float32", "int32", "bf16"])
@pytest.mark.parametrize("kind", ["normal", "ties", "equal", "asc", "special"])
@pytest.mark.parametrize("n,k", [(8193, 1), (30001, 10), (65536, 256), (65535, 64)])
def test_short_rows_one_workgroup(dt, kind, n, k):
    # rows up to 65,536 through the one-workgroup route (forced): read in
    # 16-byte vectors with an unaligned head and tail (three rows of odd
    # length start at different alignments), binned on the key range, ranked;
    # heavy ties take the radix select instead
    x = np.concatenate([_edge_rows(dt, n, kind, 600 + r) for r in range(3)])
    p = _tss().default_params(force_path=2)
    say(f"short rows one workgroup {dt} {kind} n={n} k={k}")
    gv, gi = run_gpu(x, k, dt, params=p)
    assert_same(gv, gi, x, k, dt, f"short rows {dt} {kind} n={n} k={k}")


def test_max_rows():
    # the largest batch the library accepts (65,535 rows: one grid dimension)
    rows, n, k = 65_535, 100, 7
    x = workloads.scores_int(rows, n, -50, 50, 601)
    say(f"max rows {rows} x {n} k={k}")
    gv, gi = run_gpu(x, k, "int32")
    assert_same(gv, gi, x, k, "int32", "max rows")
    with pytest.raises(_tss().TopkError):
        _tss().topk(torch.zeros(rows + 1, 8, device="cuda"), 2)
