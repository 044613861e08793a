"""GPU stage-level parity: each step of the sampled route checked on its own
against the CPU oracle, through the C ABI.

* Threshold (Prof-K section 3, stage 2): for every way the device selects tau
  (top-t lists in the filter's prologue or in the threshold kernel; every
  sample key held in registers or streamed; a boundary bin larger than LDS or
  radix-selected in LDS), the device's tau key, survivor count R, tie count
  and route equal the oracle's sampler, threshold and detection rule for the
  same seed, in all three dtypes.  The route the device took is asserted too.
* A caller-given threshold drives detection from the host (section 4,
  "Failure Modes and Budget Allocation": the largest key forces R < k).
* Detection under relaxed recall with heavy ties at tau.
* The exact route when its grid-barrier waits give up (Appendix D,
  "Graceful Degradation via Fallback": the fallback stays exact).
* Workspaces holding arbitrary bytes.
* The fallback rate against Lemma 1 (Theorem 3; Eq. 1).
"""
import ctypes

import numpy as np
import pytest

import oracle
import oracle.params as P
import workloads
from gpu_util import assert_same, run_gpu, say, to_dev, vals_to_host

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


def _expected_route(row, dt, tau_key, k, cap):
    """Route of a sampled row under the detection rule: the survivors split at
    tau into G above and E equal; accepted when G alone holds k within the
    capacity, or when G < k <= G + E <= cap (the ties join the candidates)."""
    kk = oracle.keys(row, dt).astype(np.int64)
    G = int((kk > tau_key).sum())
    E = int((kk == tau_key).sum())
    if G > cap:
        return 1, G, E
    if G >= k:
        return 0, G, E
    return (0 if k <= G + E <= cap else 1), G, E


# ------------------------------------------------------------ row makers
def _row(dt, kind, n, seed):
    g = workloads.rng(seed)
    if kind == "spread":
        if dt == "float32":
            return workloads.normal_f32(1, n, seed)
        if dt == "int32":
            return workloads.scores_int(1, n, -10 ** 7, 10 ** 7, seed)
        return workloads.relu_bf16(1, n, seed)
    # "onebin": every value shares the top 11 key bits (one bin of the
    # threshold's first histogram): fp32 and bf16 in [1.0, 1.2), int32 in
    # [0, 2^21)
    if dt == "int32":
        return g.integers(0, 2 ** 21, size=(1, n), dtype=np.int32)
    f = g.uniform(1.0, 1.2, size=(1, n)).astype(np.float32)
    return f if dt == "float32" else workloads.f32_to_bf16_bits(f)


def _routes():
    """name: (data kind, S, t, expected source of tau, expected bin flags or
    None).  With spread data the boundary bin's size depends on the dtype's
    key range (the int32 scores' top-t keys share one bin, for instance), so
    only the source is asserted there; the one-bin rows force the flags.
    The sampler keeps per-workgroup lists (256 samples each) of its t
    largest keys for t <= 8 (by extraction) and of its 32 largest, sorted,
    for 8 < t <= 32; lists of at most 4096 keys
    in all are selected in the filter's prologue: by wave max extraction for
    t <= 8 and at most 2048 keys, by a radix select over [largest list tail,
    largest head] for t <= 8 and more keys, and by bitonic merges of the
    sorted lists for t > 8.  More list keys, or t beyond 32 (every sample
    key), go to the threshold kernel."""
    tss = _tss()
    return {
        "filter_lists": ("spread", 16384, 3, tss.TAU_FILTER_LISTS, 0),
        "filter_radix_t8": ("spread", 131072, 8, tss.TAU_FILTER_RADIX, 0),
        "filter_radix_onebin_t6": ("onebin", 100000, 6, tss.TAU_FILTER_RADIX, 0),
        "filter_merge_t12": ("spread", 16384, 12, tss.TAU_FILTER_MERGE, 0),
        "filter_merge_t16": ("spread", 32768, 16, tss.TAU_FILTER_MERGE, 0),
        "ktau_sorted_lists": ("spread", 131072, 16, tss.TAU_KTAU_LISTS, None),
        "filter_merge_t32": ("spread", 32768, 32, tss.TAU_FILTER_MERGE, 0),
        "filter_merge_t9_short": ("spread", 2048, 9, tss.TAU_FILTER_MERGE, 0),
        "filter_merge_onebin": ("onebin", 16384, 14, tss.TAU_FILTER_MERGE, 0),
        "filter_merge_onebin_t30": ("onebin", 4096, 30, tss.TAU_FILTER_MERGE, 0),
        "ktau_lists_many": ("spread", 200000, 8, tss.TAU_KTAU_LISTS, None),
        "ktau_lists_t32": ("spread", 262144, 32, tss.TAU_KTAU_LISTS, None),
        "ktau_regs": ("spread", 32768, 40, tss.TAU_KTAU_REGS, None),
        "ktau_stream": ("spread", 40000, 40, tss.TAU_KTAU_STREAM, None),
        "bin_streamed": ("onebin", 16384, 40, tss.TAU_KTAU_REGS, tss.TAU_BIN_STREAMED),
        "bin_radix": ("onebin", 4096, 40, tss.TAU_KTAU_REGS, tss.TAU_BIN_RADIX),
        "bin_streamed_keys_streamed": ("onebin", 40000, 40, tss.TAU_KTAU_STREAM,
                                       tss.TAU_BIN_STREAMED),
    }


ROUTE_NAMES = ["filter_lists", "filter_radix_t8", "filter_radix_onebin_t6", "filter_merge_t12",
               "filter_merge_t16", "ktau_sorted_lists", "filter_merge_t32",
               "filter_merge_t9_short",
               "filter_merge_onebin", "filter_merge_onebin_t30", "ktau_lists_many",
               "ktau_lists_t32", "ktau_regs", "ktau_stream", "bin_streamed", "bin_radix",
               "bin_streamed_keys_streamed"]


@pytest.mark.parametrize("dt", ["float32", "int32", "bf16"])
@pytest.mark.parametrize("name", ROUTE_NAMES)
def test_threshold_every_select_path(dt, name):
    kind, S, t, want_source, want_flags = _routes()[name]
    tss = _tss()
    n, k = 2 ** 22 + 5, 64
    x = _row(dt, kind, n, 700 + ROUTE_NAMES.index(name))
    xt = to_dev(x, dt)
    ws = tss.Workspace()   # fresh: the first call finds no usable sample histogram
    for seed in (1, 2, 3):
        p = _seeded(seed, S=S, t=t, M=n // 8, force_path=tss.PATH_FILTER)
        pl = tss.plan(n, 1, k, dt, params=p)
        assert (pl["S"], pl["t"]) == (S, t)
        say(f"tau path {name} {dt} S={S} t={t} seed={seed}")
        v, i = tss.topk(xt, k, params=p, workspace=ws)
        torch.cuda.synchronize()
        assert_same(vals_to_host(v, dt), i.cpu().numpy(), x, k, dt, f"{name} {dt}")
        st = tss.read_stats(1, workspace=ws)[0]
        tk, R = oracle.tau(x[0], seed, 0, S, t, dt)
        assert st["tau_route"] & 7 == want_source, (st, want_source)
        if want_flags is not None:
            assert st["tau_route"] & ~7 == want_flags, (st, want_flags)
        say(f"  route {st['tau_route']:#x} tau {st['tau_key']:#x} R={st['r_sampled']} "
            f"ties={st['ties']} path={st['path']}")
        assert st["tau_key"] == tk, (hex(st["tau_key"]), hex(tk))
        assert st["r_sampled"] == R
        path, G, E = _expected_route(x[0], dt, tk, k, pl["cap"])
        assert st["path"] == path and st["ties"] == E, (st, path, G, E)
        assert st["flags"] == 0


# ------------------------------------------------------------ caller-given threshold
def _key_of(value_bits_row, dt, j):
    return int(oracle.keys(value_bits_row[j:j + 1], dt)[0])


@pytest.mark.parametrize("dt", ["float32", "int32", "bf16"])
def test_forced_threshold_drives_detection(dt):
    tss = _tss()
    n, k = 2 ** 21 + 3, 100
    x = _row(dt, "spread", n, 811)
    if dt == "float32":
        x = workloads.pareto_signed(1, n, 811)
    xt = to_dev(x, dt)
    ov, oi = oracle.topk(x, 1000, dt)
    top = 0xFFFF if dt == "bf16" else 0xFFFFFFFF
    cases = {
        "top key: R < k": top,                                   # no element reaches it
        "rank 500: accepted": _key_of(ov[0], dt, 499),           # about 500 survivors
        "lowest key: overflow": 0,                                # the whole row survives
    }
    for label, key in cases.items():
        p = _seeded(5, use_force_tau=1, force_tau_key=key, M=4096)
        cap = tss.plan(n, 1, k, dt, params=p)["cap"]
        say(f"forced tau {dt}: {label} key={key:#x}")
        v, i = tss.topk(xt, k, params=p)
        torch.cuda.synchronize()
        assert_same(vals_to_host(v, dt), i.cpu().numpy(), x, k, dt, f"forced {dt} {label}")
        st = tss.read_stats(1)[0]
        assert st["tau_route"] == tss.TAU_FORCED and st["tau_key"] == key
        kk = oracle.keys(x[0], dt).astype(np.int64)
        assert st["r_sampled"] == int((kk >= key).sum()) or st["r_sampled"] > cap
        path, G, E = _expected_route(x[0], dt, key, k, cap)
        assert st["path"] == path, (label, st, path, G, E)
        if label.startswith("top"):
            assert st["path"] == 1 and st["r_sampled"] < k
        if label.startswith("rank"):
            assert st["path"] == 0 and k <= st["r_sampled"] <= cap
        if label.startswith("lowest"):
            assert st["path"] == 1


def _bf16_special_row(n, seed):
    """bf16 bits of every kind: spread normals of both signs, +-0, +-inf, NaN
    of both signs with several payloads, denormals of both signs, and the
    largest finite values; shuffled."""
    g = workloads.rng(seed)
    x = workloads.f32_to_bf16_bits(g.standard_normal(size=n).astype(np.float32) * 3.0)
    picks = np.array([0x0000, 0x8000, 0x7F80, 0xFF80, 0x7FC0, 0x7F81, 0x7FFF, 0xFFC0, 0xFF81,
                      0xFFFF, 0x0001, 0x8001, 0x007F, 0x807F, 0x7F7F, 0xFF7F, 0x3F80, 0xBF80],
                     dtype=np.uint16)
    m = n // 20
    x[:m] = g.choice(picks, size=m)
    g.shuffle(x)
    return x.reshape(1, n)


def test_bf16_screen_every_threshold_kind():
    """The bf16 filter screens each 16-byte vector on the magnitude bits of
    its eight elements and tests flagged vectors exactly.  Thresholds given
    from the host across every kind of bf16 value (negative, -0/+0, a
    denormal, +1, the largest finite, +inf, NaN): the survivor count R must
    equal the number of elements whose order-preserving key reaches tau (the
    definition, counted on the CPU), and the output the exact top-k."""
    tss = _tss()
    n, k = 2 ** 20 + 3, 100
    x = _bf16_special_row(n, 1201)
    xt = to_dev(x, "bf16")
    kk = oracle.keys(x[0], "bf16").astype(np.int64)
    for bits in (0xBF80, 0x8001, 0x8000, 0x0000, 0x0001, 0x3F80, 0x7F7F, 0x7F80):
        key = int(oracle.keys(np.array([bits], dtype=np.uint16), "bf16")[0])
        for tk in (key, 0xFFFF if bits == 0x7F80 else key):
            p = _seeded(7, use_force_tau=1, force_tau_key=tk, M=n)
            say(f"bf16 screen: tau bits {bits:#06x} key {tk:#06x}")
            v, i = tss.topk(xt, k, params=p)
            torch.cuda.synchronize()
            assert_same(vals_to_host(v, "bf16"), i.cpu().numpy(), x, k, "bf16", f"tau key {tk:#x}")
            st = tss.read_stats(1)[0]
            assert st["r_sampled"] == int((kk >= tk).sum()), (hex(tk), st)
            assert st["ties"] == int((kk == tk).sum()), (hex(tk), st)


# ------------------------------------------------------------ relaxed recall, ties at tau
@pytest.mark.parametrize("dt", ["float32", "bf16"])
def test_relaxed_recall_heavy_ties_every_workgroup_agrees(dt):
    """Rows kept partial with many ties at tau: G above, E equal, with
    k_eff <= G + E < k <= cap < G + 2E.  Every workgroup of the finish
    kernel must reach the same verdict for these rows while their owners
    rewrite the row records (the check reads only the filter's counts)."""
    tss = _tss()
    rows, n, k, n_top, n_tie = 8, 2 ** 20, 4000, 100, 2000
    xs = []
    for r in range(rows):
        g = workloads.rng(900 + r)
        f = (g.standard_normal(n) - 1000.0).astype(np.float32)
        pos = g.choice(n, n_top + n_tie, replace=False)
        f[pos[:n_top]] = 10.0 + np.arange(n_top, dtype=np.float32)
        f[pos[n_top:]] = 5.0
        xs.append(f)
    x = np.stack(xs)
    if dt == "bf16":
        x = workloads.f32_to_bf16_bits(x)
        tau = int(oracle.keys(workloads.f32_to_bf16_bits(np.array([5.0], np.float32)), "bf16")[0])
    else:
        tau = int(oracle.keys(np.array([5.0], np.float32))[0])
    p = _seeded(3, use_force_tau=1, force_tau_key=tau, M=3000, recall=0.5)
    pl = tss.plan(n, rows, k, dt, params=p)
    k_eff, cap = pl["k_eff"], pl["cap"]
    assert k_eff == 2000 and cap == k and n_top + 2 * n_tie > cap
    say(f"relaxed recall, ties at tau: {dt} rows={rows} k={k} k_eff={k_eff} cap={cap}")
    for rep in range(3):
        v, i = tss.topk(to_dev(x, dt), k, params=p)
        torch.cuda.synchronize()
        gv, gi = vals_to_host(v, dt), i.cpu().numpy()
        st = tss.read_stats(rows)
        for r in range(rows):
            ov, oi, part = oracle.relaxed_selection(x[r], k, k_eff, tau, cap, dt)
            assert part
            assert np.array_equal(gi[r], oi), f"rep {rep} row {r}: indices differ"
            assert gv[r].tobytes() == ov.tobytes()
            assert st[r]["path"] == tss.ROUTE_PARTIAL and st[r]["flags"] == 0
            assert (st[r]["r_sampled"], st[r]["ties"]) == (n_top + n_tie, n_tie)


# ------------------------------------------------------------ barrier give-ups
@pytest.mark.parametrize("case", ["exact_f32", "exact_i32", "exact_bf16", "exact_large_k",
                                  "sampled_failures", "sampled_failures_large_k"])
def test_barrier_giveup_still_exact_then_clean(case):
    """Every grid-barrier wait of the exact route gives up at once (the test
    flag): the workgroups leave the shared phases and the last one selects
    every listed row again on its own.  The answer is still exact and the
    call is flagged; the next call on the same workspace is exact and clean."""
    tss = _tss()
    n = 2 ** 19 + 3
    if case.startswith("exact"):
        dt = {"exact_f32": "float32", "exact_i32": "int32", "exact_bf16": "bf16"}.get(case, "float32")
        rows, k = 3, (20_000 if case == "exact_large_k" else 100)
        x = _row(dt, "spread", rows * n, 950).reshape(rows, n)
        base = dict(force_path=tss.PATH_EXACT)
    else:
        dt = "float32"
        rows, n = 12, 2 ** 20
        k = 5000 if case.endswith("large_k") else 64
        x = workloads.normal_f32(rows, n, 951)
        x[::4] = 1.5          # constant rows: their threshold admits the whole row
        base = dict(force_path=tss.PATH_FILTER)
    xt = to_dev(x, dt)
    ws = tss.Workspace()
    say(f"barrier give-up: {case} rows={rows} n={n} k={k}")
    for flags, want in ((tss.TEST_BARRIER_GIVEUP, 1), (0, 0), (tss.TEST_BARRIER_GIVEUP, 1), (0, 0)):
        p = tss.default_params(test_flags=flags, **base)
        v, i = tss.topk(xt, k, params=p, workspace=ws)
        torch.cuda.synchronize()
        assert_same(vals_to_host(v, dt), i.cpu().numpy(), x, k, dt, f"{case} flags={flags}")
        st = tss.read_stats(rows, workspace=ws)
        assert all((r["flags"] & 1) == want for r in st), (flags, st[0])
        if case.startswith("sampled"):
            assert [r["path"] for r in st[::4]] == [1] * len(st[::4])


# ------------------------------------------------------------ arbitrary workspaces
def _raw_call(x_t, k, dt, params, ws):
    tss = _tss()
    rows, n = x_t.shape
    vals = torch.empty((rows, k), dtype=x_t.dtype, device="cuda")
    idx = torch.empty((rows, k), dtype=torch.int64, device="cuda")
    stream = torch.cuda.current_stream().cuda_stream
    rc = tss._lib.lib.topk_ex(x_t.data_ptr(), n, rows, k, tss.dtype_code(dt), vals.data_ptr(),
                              idx.data_ptr(), ws.data_ptr(), ws.numel(), stream,
                              ctypes.byref(params))
    assert rc == 0
    torch.cuda.synchronize()
    return vals_to_host(vals, dt), idx.cpu().numpy()


def _raw_stats(ws, rows):
    tss = _tss()
    arr = (tss._lib.RowStats * rows)()
    rc = tss._lib.lib.topk_read_stats(ws.data_ptr(), rows, arr, torch.cuda.current_stream().cuda_stream)
    assert rc == 0
    return arr


@pytest.mark.parametrize("case", ["all_keys", "lists", "exact", "large_k", "batched"])
def test_workspace_with_arbitrary_bytes(case):
    """Through the raw C ABI, a workspace full of random bytes, reused at the
    same address with other random bytes in it: every call exact.  With all
    sample keys (the sample histogram carried between calls), tau also
    matches the oracle, whether or not the stamp happens to survive."""
    tss = _tss()
    dt = "float32"
    if case == "batched":
        x = workloads.pareto_signed(40, 2 ** 18, 961)
    else:
        x = workloads.normal_f32(1, 2 ** 22 + 1, 960)
    rows, n = x.shape
    k = {"large_k": 9000}.get(case, 64)
    kw = {"all_keys": dict(S=32768, t=40, M=n // 8, force_path=tss.PATH_FILTER),
          "lists": dict(),
          "exact": dict(force_path=tss.PATH_EXACT),
          "large_k": dict(),
          "batched": dict(S=8192, t=40, M=n // 8, force_path=tss.PATH_FILTER)}[case]
    xt = to_dev(x, dt)
    need = tss.workspace_size(n, rows, k, dt, tss.default_params(**kw))
    ws = torch.empty(need + 4096, dtype=torch.uint8, device="cuda")
    gen = torch.Generator(device="cuda")
    gen.manual_seed(962)
    for rep, keep_header in enumerate((False, False, True, True, False)):
        if keep_header:   # garbage everywhere but the 256-byte header (its stamp)
            ws[256:] = torch.randint(0, 256, (ws.numel() - 256,), dtype=torch.uint8,
                                     device="cuda", generator=gen)
        else:
            ws.copy_(torch.randint(0, 256, (ws.numel(),), dtype=torch.uint8, device="cuda",
                                   generator=gen))
        p = _seeded(10 + rep, **kw)
        say(f"arbitrary workspace {case} rep {rep} keep_header={keep_header}")
        gv, gi = _raw_call(xt, k, dt, p, ws)
        assert_same(gv, gi, x, k, dt, f"garbage workspace {case} rep {rep}")
        st = _raw_stats(ws, rows)
        assert all(s.flags == 0 for s in st)
        if case in ("all_keys", "batched") and not keep_header:
            pl = tss.plan(n, rows, k, dt, params=p)
            for r in range(rows):
                tk, R = oracle.tau(x[r], 10 + rep, r, pl["S"], pl["t"], dt)
                assert st[r].tau_key == tk and st[r].r_sampled == R


# ------------------------------------------------------------ fallback rate
@pytest.mark.parametrize("policy", ["alg1", "exact_tail", "tuned"])
def test_fallback_rate_matches_lemma1(policy):
    """Fallback rate over 400 calls with fresh seeds on a row of distinct
    values (a permutation), against the plan's probabilities from Lemma 1
    (Eq. 1): alg1 inside the 99.9% binomial interval of its predicted rate;
    the exact-tail and tuned policies consistent with at most eps."""
    st_ = pytest.importorskip("scipy.stats")
    tss = _tss()
    n, k, calls = 2 ** 22, 64, 400
    x = workloads.rng(970).permutation(n).astype(np.int32)[None, :]
    xt = to_dev(x, "int32")
    pol = {"alg1": tss.POLICY_ALG1, "exact_tail": tss.POLICY_EXACT_TAIL,
           "tuned": tss.POLICY_TUNED}[policy]
    p = tss.default_params(policy=pol)
    pl = tss.plan(n, 1, k, "int32", params=p)
    S, t, cap = pl["S"], pl["t"], pl["cap"]
    # With distinct values a row fails exactly when R < k or G = R - 1 > cap
    p_fail = P.hyper_sf(n, k - 1, S, t) + P.hyper_cdf(n, cap + 1, S, t - 1)
    say(f"fallback rate {policy}: S={S} t={t} cap={cap} predicted {p_fail:.4f}")
    fb = 0
    for c in range(calls):
        tss.topk(xt, k, params=p)
        fb += tss.read_stats(1)[0]["path"] == 1
    lo, hi = st_.binom.interval(0.999, calls, p_fail)
    say(f"  measured {fb}/{calls} = {fb / calls:.4f}; 99.9% interval [{lo}, {hi}]")
    assert lo <= fb <= hi
    if policy != "alg1":
        assert p_fail <= 1e-3 * (1 + 1e-9)
        assert fb <= st_.binom.ppf(0.999, calls, 1e-3)
