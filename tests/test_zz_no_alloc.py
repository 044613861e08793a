"""The allocation-free entry point topk_noalloc (for callers that cannot
allocate device memory), through the C ABI: its output equals topk_ex's with
a caller workspace and the oracle's, bit for bit, over calls in a row on the
one built-in scratch array, each later call a smaller input than the one
before it, in other layouts and dtypes."""
import ctypes

import numpy as np
import pytest

import workloads
from gpu_util import assert_same, say, to_dev, vals_to_host

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def _tss():
    import top_selection_sample_amd as tss
    return tss


def _outs(xt, k):
    rows = xt.shape[0]
    return (torch.full((rows, k), 7, dtype=xt.dtype, device="cuda"),
            torch.full((rows, k), -7, dtype=torch.int64, device="cuda"))


def _noalloc(xt, k, dt, params=None):
    tss = _tss()
    rows, n = xt.shape
    v, i = _outs(xt, k)
    rc = tss._lib.lib.topk_noalloc(xt.data_ptr(), n, rows, k, tss.dtype_code(dt), v.data_ptr(),
                                   i.data_ptr(), torch.cuda.current_stream().cuda_stream,
                                   ctypes.byref(params) if params is not None else None)
    return rc, v, i


def _ex(xt, k, dt, params=None):
    tss = _tss()
    rows, n = xt.shape
    v, i = _outs(xt, k)
    ws = torch.empty(tss.workspace_size(n, rows, k, dt, params), dtype=torch.uint8, device="cuda")
    rc = tss._lib.lib.topk_ex(xt.data_ptr(), n, rows, k, tss.dtype_code(dt), v.data_ptr(),
                              i.data_ptr(), ws.data_ptr(), ws.numel(),
                              torch.cuda.current_stream().cuda_stream,
                              ctypes.byref(params) if params is not None else None)
    assert rc == 0
    return v, i


def _check(x, k, dt, label, params=None):
    tss = _tss()
    rows, n = x.shape
    need = tss.workspace_size(n, rows, k, dt, params)
    assert need <= tss._lib.NOALLOC_SCRATCH_BYTES, (label, need)
    say(f"noalloc {label}: {dt} [{rows}, {n}] k={k} ({need} workspace bytes)")
    xt = to_dev(x, dt)
    rc, v, i = _noalloc(xt, k, dt, params)
    assert rc == 0, tss._lib.lib.topk_status_string(rc)
    ev, ei = _ex(xt, k, dt, params)
    torch.cuda.synchronize()
    gv, gi = vals_to_host(v, dt), i.cpu().numpy()
    assert np.array_equal(gi, ei.cpu().numpy()), f"{label}: indices differ from topk_ex"
    assert gv.tobytes() == vals_to_host(ev, dt).tobytes(), f"{label}: values differ from topk_ex"
    assert_same(gv, gi, x, k, dt, label)
    return need


def test_noalloc_two_calls_second_smaller():
    # the headline's kind of call (sampled route), then a smaller batched
    # int32 call with another layout on the same scratch array
    a = _check(workloads.normal_f32(1, 2 ** 22 + 5, 1201), 64, "float32", "first call")
    b = _check(workloads.scores_int(3, 100_003, -50, 50, 1202), 10, "int32", "second, smaller")
    assert b < a


def test_noalloc_batched_then_large_k_then_tiny():
    # 128 short rows, then large k (the bucket sort's counters live in the
    # array), then one 4096-element row (one workgroup per row): each a
    # smaller workspace than the one before it
    sizes = [
        _check(workloads.pareto_signed(128, 2 ** 16, 1204), 64, "float32", "batched rows"),
        _check(workloads.relu_bf16(1, 2 ** 22, 1203), 8192, "bf16", "large k"),
        _check(workloads.scores_int(1, 4096, 0, 1000, 1001), 10, "int32", "config 1"),
    ]
    assert sizes[0] > sizes[1] > sizes[2]


def test_noalloc_all_keys_threshold_and_exact_route():
    # the sample histogram kept in the array between calls (all sample keys,
    # t > 32), twice in a row, then the exact route on a smaller row
    tss = _tss()
    x = workloads.normal_f32(1, 2 ** 22 + 3, 1205)
    p = tss.default_params(S=32768, t=40, M=2 ** 19, force_path=tss.PATH_FILTER)
    _check(x, 100, "float32", "all sample keys", p)
    _check(x, 100, "float32", "all sample keys again", p)
    _check(x[:, : 2 ** 20], 100, "float32", "exact route", tss.default_params(force_path=tss.PATH_EXACT))


def test_noalloc_refuses_calls_beyond_its_scratch():
    tss = _tss()
    n, k = 2 ** 24, 2 ** 22
    assert tss.workspace_size(n, 1, k, "float32") > tss._lib.NOALLOC_SCRATCH_BYTES
    xt = torch.zeros((1, n), dtype=torch.float32, device="cuda")
    rc, v, i = _noalloc(xt, k, "float32")
    torch.cuda.synchronize()
    assert rc == tss._lib.TOPK_ETOOBIG
    assert bool((i == -7).all())    # nothing was launched
