"""GPU parity at the full headline shapes, in the launch configuration the
benchmark times (default parameters, fresh sampler seed per call).  The CPU
oracle computes every one of these in seconds, so the comparison is complete:
every index and every value bit of every row."""
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


def test_config3_normal_2p28():
    x, dt, ks, _ = workloads.config("c3")
    xt = to_dev(x, dt)
    for k in ks:
        say(f"config 3: fp32 [1, 2^28] k={k}")
        gv, gi = run_gpu(x, k, dt, xt=xt)
        assert_same(gv, gi, x, k, dt, f"c3 k={k}")
    del xt


@pytest.mark.parametrize("variant", ["c4v1", "c4v2", "c4v3"])
def test_config4_batched(variant):
    x, dt, ks, _ = workloads.config(variant)
    say(f"config 4 {variant}: fp32 [128, 2^20] k=64")
    gv, gi = run_gpu(x, ks[0], dt)
    assert_same(gv, gi, x, ks[0], dt, variant)


def test_config5_batchtopk_bf16():
    x, dt, ks, _ = workloads.config("c5")
    flat = x.reshape(1, -1)
    say("config 5: bf16 [4096, 65536] flattened, k=131072")
    xt = to_dev(flat, dt)
    gv, gi = run_gpu(flat, ks[0], dt, xt=xt)
    assert_same(gv, gi, flat, ks[0], dt, "c5")


def test_config5_batchtopk_sparse_activation():
    # the BatchTopK consumer at full size: the [4096, 65536] bf16 activations
    # with their 131072 largest kept and zeros elsewhere, and the mask
    import torch
    import top_selection_sample_amd as tss
    x, dt, ks, _ = workloads.config("c5")
    K = ks[0]
    say("config 5 consumer: batchtopk [4096, 65536] bf16, K=131072")
    acts = to_dev(x, dt)
    out, m = tss.batchtopk(acts, K, mask=True)
    torch.cuda.synchronize()
    ov, oi = oracle.topk(x.reshape(1, -1), K, dt)
    flat = out.reshape(-1)
    assert int(m.sum()) == K
    assert int(torch.count_nonzero(flat)) == K   # every kept ReLU activation is positive
    idx = torch.from_numpy(oi.reshape(-1)).cuda()
    got = flat[idx].view(torch.int16).cpu().numpy().view(np.uint16)
    assert got.tobytes() == ov.reshape(-1).tobytes()
    assert int(m.reshape(-1)[idx].sum()) == K


def _route(row, dt, tau_key, k, cap):
    # the detection rule: G above tau, E equal; accepted when G holds k within
    # the capacity, or G < k <= G + E <= cap
    kk = oracle.keys(row, dt).astype(np.int64)
    G, E = int((kk > tau_key).sum()), int((kk == tau_key).sum())
    if G > cap:
        return 1, E
    if G >= k:
        return 0, E
    return (0 if k <= G + E <= cap else 1), E


@pytest.mark.parametrize("name", ["c3k16", "c3k64", "c3k2048", "c4v1", "c4v2", "c4v3", "c5"])
def test_full_size_threshold_and_route_seeded(name):
    """At full size, in the benchmark's launch configuration but with a fixed
    sampler seed: every row's tau key, survivor count R, tie count and route
    equal what the oracle's sampler and the detection rule predict, and the
    answer is exact."""
    import top_selection_sample_amd as tss
    cfg = {"c3k16": ("c3", 16), "c3k64": ("c3", 64), "c3k2048": ("c3", 2048), "c4v1": ("c4v1", 64),
           "c4v2": ("c4v2", 64), "c4v3": ("c4v3", 64), "c5": ("c5", 131072)}[name]
    x, dt, _, _ = workloads.config(cfg[0])
    k = cfg[1]
    if cfg[0] == "c5":
        x = x.reshape(1, -1)
    rows, n = x.shape
    seed = 4242
    p = tss.default_params(seed=seed, use_seed=1)
    pl = tss.plan(n, rows, k, dt, params=p)
    assert pl["path"] == 0
    say(f"full-size seeded route {name}: rows={rows} n={n} k={k} S={pl['S']} t={pl['t']} cap={pl['cap']}")
    gv, gi = run_gpu(x, k, dt, params=p)
    assert_same(gv, gi, x, k, dt, f"{name} seeded")
    st = tss.read_stats(rows)
    for r in range(rows):
        tk, R = oracle.tau(x[r], seed, r, pl["S"], pl["t"], dt)
        path, E = _route(x[r], dt, tk, k, pl["cap"])
        assert st[r]["tau_key"] == tk, (r, hex(st[r]["tau_key"]), hex(tk))
        assert st[r]["path"] == path, (r, st[r], path)
        if path == 0:
            assert st[r]["r_sampled"] == R and st[r]["ties"] == E, (r, st[r], R, E)
        assert st[r]["flags"] == 0
