"""Helpers for the GPU parity tests: host<->device copies and bitwise
comparison of the library's output with the CPU oracle."""
from __future__ import annotations

import sys

import numpy as np

import oracle


def say(msg: str) -> None:
    print(msg, flush=True)
    sys.stdout.flush()


def to_dev(x: np.ndarray, dt: str):
    import torch
    if dt == "bf16":
        return torch.from_numpy(np.ascontiguousarray(x).view(np.int16)).cuda().view(torch.bfloat16)
    return torch.from_numpy(np.ascontiguousarray(x)).cuda()


def vals_to_host(v, dt: str) -> np.ndarray:
    import torch
    if dt == "bf16":
        return v.view(torch.int16).cpu().numpy().view(np.uint16)
    return v.cpu().numpy()


def run_gpu(x: np.ndarray, k: int, dt: str, params=None, xt=None):
    import torch
    import top_selection_sample_amd as tss
    if xt is None:
        xt = to_dev(x, dt)
    v, i = tss.topk(xt, k, params=params)
    torch.cuda.synchronize()
    return vals_to_host(v, dt), i.cpu().numpy()


def assert_same(gv, gi, x: np.ndarray, k: int, dt: str, label: str = ""):
    """Element-by-element equality with the oracle: indices and value bits."""
    ov, oi = oracle.topk(x, k, dt)
    gi2 = gi.reshape(oi.shape)
    gv2 = gv.reshape(ov.shape)
    if not np.array_equal(gi2, oi):
        bad = np.argwhere(gi2 != oi)
        r, c = bad[0]
        raise AssertionError(f"{label}: indices differ at row {r} slot {c}: gpu {gi2[r, c]} "
                             f"oracle {oi[r, c]} ({len(bad)} mismatches)")
    assert gv2.tobytes() == ov.tobytes(), f"{label}: value bits differ"
