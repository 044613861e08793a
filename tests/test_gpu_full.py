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
