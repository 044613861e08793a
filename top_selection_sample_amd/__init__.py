"""Exact top-k selection on one AMD MI355X (gfx950), Prof-K one-pass filtering.

    import torch, top_selection_sample_amd as tss
    values, indices = tss.topk(x, k)          # x: [rows, n] or [n] on the GPU

``x`` may be int32, float32 or bfloat16.  The result is the exact top-k of
each row in rank order (value descending, equal values by lower index), as
the input's own bits and int64 row-local indices.  PyTorch only supplies
device memory and the stream; the selection runs in libtopk_mi355x.so.
"""
from __future__ import annotations

import ctypes
from contextlib import nullcontext

import torch

from . import _lib
from ._lib import (PATH_AUTO, PATH_EXACT, PATH_FILTER, POLICY_ALG1, POLICY_EXACT_TAIL, POLICY_TUNED,
                   ROUTE_EXACT, ROUTE_FALLBACK, ROUTE_PARTIAL, ROUTE_SAMPLED, TAU_BIN_RADIX,
                   TAU_BIN_STREAMED, TAU_FILTER_LISTS, TAU_FILTER_MERGE, TAU_FILTER_RADIX,
                   TAU_FORCED,
                   TAU_KTAU_LISTS, TAU_KTAU_REGS,
                   TAU_KTAU_STREAM, TAU_NONE, TEST_BARRIER_GIVEUP, Params, TopkError,
                   default_params)

__all__ = ["topk", "plan", "profile_enable", "profile_read", "stream_read", "scatter", "batchtopk",
           "workspace_size", "read_stats",
           "Workspace", "Params",
           "default_params", "TopkError", "PATH_AUTO", "PATH_FILTER", "PATH_EXACT",
           "ROUTE_SAMPLED", "ROUTE_FALLBACK", "ROUTE_EXACT", "ROUTE_PARTIAL",
           "POLICY_EXACT_TAIL", "POLICY_ALG1", "POLICY_TUNED", "dtype_code",
           "TAU_NONE", "TAU_FILTER_LISTS", "TAU_KTAU_LISTS", "TAU_KTAU_REGS", "TAU_KTAU_STREAM",
           "TAU_FORCED", "TAU_FILTER_RADIX", "TAU_FILTER_MERGE", "TAU_BIN_STREAMED", "TAU_BIN_RADIX",
           "TEST_BARRIER_GIVEUP", "filter_trace"]

_TORCH_CODES = {torch.int32: 0, torch.float32: 1, torch.bfloat16: 2}
_NAME_CODES = _lib.DTYPE_CODES


def dtype_code(dtype) -> int:
    if isinstance(dtype, int):
        return dtype
    if isinstance(dtype, str):
        return _NAME_CODES[dtype]
    if dtype not in _TORCH_CODES:
        raise TypeError(f"unsupported dtype {dtype}; use int32, float32 or bfloat16")
    return _TORCH_CODES[dtype]


def _pp(params):
    return ctypes.byref(params) if params is not None else None


def plan(n: int, rows: int, k: int, dtype, params: Params | None = None) -> dict:
    """Host-side plan of a call shape (no GPU needed)."""
    info = _lib.PlanInfo()
    _lib.check(_lib.lib.topk_plan(n, rows, k, dtype_code(dtype), _pp(params), ctypes.byref(info)),
               "topk_plan")
    return {f: getattr(info, f) for f, _ in _lib.PlanInfo._fields_}


_ws_sizes: dict = {}


def workspace_size(n: int, rows: int, k: int, dtype, params: Params | None = None) -> int:
    code = dtype_code(dtype)
    key = (n, rows, k, code, bytes(params) if params is not None else None)
    size = _ws_sizes.get(key)
    if size is None:
        out = ctypes.c_size_t()
        _lib.check(_lib.lib.topk_workspace_size(n, rows, k, code, _pp(params), ctypes.byref(out)),
                   "topk_workspace_size")
        size = _ws_sizes[key] = out.value
    return size


class Workspace:
    """Device scratch for topk calls on one device; grows on demand.  A
    workspace serves one stream at a time.  It needs no initialisation (every
    call writes what it reads), so a new buffer is used as torch hands it
    out.  The library allocates nothing and records no memset, so a call can
    be captured in a HIP graph; the graph keeps the workspace's address, so
    give captured calls a workspace of their own, sized by an eager call of
    the same shape before the capture (a later, larger call would reallocate
    it under the graph)."""

    def __init__(self, device=None):
        self.device = _norm_device(device)
        self.buf = None

    def get(self, nbytes: int, stream) -> torch.Tensor:
        if self.buf is None or self.buf.numel() < nbytes:
            self.buf = torch.empty(max(nbytes, 256), dtype=torch.uint8, device=self.device)
        return self.buf


_default_ws: dict = {}


def _norm_device(device) -> torch.device:
    dev = torch.device(device if device is not None else "cuda")
    if dev.index is None:
        dev = torch.device("cuda", torch.cuda.current_device())
    return dev


def _workspace_for(device, stream: int) -> Workspace:
    """The default workspace of a (device, stream) pair: calls on different
    streams never share scratch memory."""
    device = _norm_device(device)
    key = (device.type, device.index, stream)
    if key not in _default_ws:
        _default_ws[key] = Workspace(device)
    return _default_ws[key]


def topk(x: torch.Tensor, k: int, params: Params | None = None, workspace: Workspace | None = None,
         out: tuple | None = None):
    """Exact top-k of each row of ``x`` ([rows, n] or [n], contiguous rows).

    Returns (values, indices) shaped [rows, k] (or [k] for 1-D input).  An
    empty batch (rows = 0) returns empty outputs.  ``out`` = (values,
    indices): contiguous tensors of rows * k elements on x's device, of x's
    dtype and int64; anything else raises ValueError before any launch."""
    if not x.is_cuda:
        raise ValueError("x must be a GPU tensor")
    squeeze = x.dim() == 1
    x2 = x.reshape(1, -1) if squeeze else x
    if x2.dim() != 2 or not x2.is_contiguous():
        raise ValueError("x must be a contiguous [rows, n] or [n] tensor")
    rows, n = x2.shape
    code = dtype_code(x2.dtype)
    dev = x2.device
    if out is not None:
        vals, idx = out
        for t, dt, name in ((vals, x2.dtype, "values"), (idx, torch.int64, "indices")):
            if (t.device != dev or t.dtype != dt or not t.is_contiguous()
                    or t.numel() != rows * k):
                raise ValueError(f"out {name}: need a contiguous {dt} tensor of {rows} x {k} "
                                 f"elements on {dev}")
    if rows == 0:   # an empty batch: nothing to select
        if not 1 <= k <= n:
            raise _lib.TopkError(_lib.TOPK_EINVAL, "topk")
        if out is None:
            vals = torch.empty((0, k), dtype=x2.dtype, device=dev)
            idx = torch.empty((0, k), dtype=torch.int64, device=dev)
        return vals, idx
    # the library launches on the current device: switch only when x lives
    # elsewhere (the switch costs more than the rest of a small call)
    ctx = torch.cuda.device(dev) if dev.index != torch.cuda.current_device() else nullcontext()
    with ctx:
        stream = torch.cuda.current_stream(dev).cuda_stream
        ws = workspace if workspace is not None else _workspace_for(dev, stream)
        if ws.device != dev:
            raise ValueError(f"workspace is on {ws.device}, x on {dev}")
        need = workspace_size(n, rows, k, code, params)
        buf = ws.get(need, stream)
        if out is None:
            vals = torch.empty((rows, k), dtype=x2.dtype, device=dev)
            idx = torch.empty((rows, k), dtype=torch.int64, device=dev)
        st = _lib.lib.topk_ex(x2.data_ptr(), n, rows, k, code, vals.data_ptr(), idx.data_ptr(),
                              buf.data_ptr(), buf.numel(), stream, _pp(params))
        _lib.check(st, "topk")
    if squeeze:
        return vals[0], idx[0]
    return vals, idx


def read_stats(rows: int, workspace: Workspace | None = None, device=None) -> list:
    """Per-row records of the last call on a workspace (synchronises).  With
    no workspace given: the default one of the current stream, the one that
    stream's last call used."""
    dev = _norm_device(device)
    with torch.cuda.device(dev):
        stream = torch.cuda.current_stream(dev).cuda_stream
        ws = workspace if workspace is not None else _workspace_for(dev, stream)
        if ws.buf is None:
            raise RuntimeError("no call has used this workspace yet")
        arr = (_lib.RowStats * rows)()
        _lib.check(_lib.lib.topk_read_stats(ws.buf.data_ptr(), rows, arr, stream), "topk_read_stats")
    return [{"tau_key": a.tau_key, "r_sampled": a.r_sampled, "path": a.path, "passes": a.passes,
             "flags": a.flags, "ties": a.ties, "tau_route": a.tau_route} for a in arr]


def filter_trace(buf) -> None:
    """Measurement aid: while set, every call's filter launch writes, per
    workgroup l (row * workgroups per row + index), the device's 100 MHz
    realtime counter at its start and at the end of its scan into buf[2l] and
    buf[2l + 1] (buf: an int64 CUDA tensor; None stops the trace)."""
    if buf is None:
        _lib.check(_lib.lib.topk_filter_trace(None, 0), "topk_filter_trace")
        return
    if not (buf.is_cuda and buf.dtype == torch.int64 and buf.is_contiguous()):
        raise ValueError("filter_trace: a contiguous int64 CUDA tensor")
    _lib.check(_lib.lib.topk_filter_trace(buf.data_ptr(), buf.numel()), "topk_filter_trace")


def profile_enable(on: bool = True) -> None:
    """Record HIP events around each pipeline stage of later calls."""
    _lib.check(_lib.lib.topk_profile_enable(1 if on else 0), "topk_profile_enable")


def profile_read() -> dict:
    """Summed milliseconds and bracket counts per stage since the last read
    (waits for the recorded events)."""
    t = _lib.StageTimes()
    _lib.check(_lib.lib.topk_profile_read(ctypes.byref(t)), "topk_profile_read")
    return {name: {"ms": t.ms[i], "count": t.count[i]} for i, name in enumerate(_lib.STAGES)}


def stream_read(x: torch.Tensor, sink: torch.Tensor) -> None:
    """One read of ``x`` with the filter's access pattern (a measurement aid:
    its time is the achievable read time of that pattern).  ``x``: contiguous
    GPU tensor, 16-byte aligned, a multiple of 16 bytes; ``sink``: int32 GPU
    tensor of at least 64 elements."""
    if not (x.is_cuda and x.is_contiguous() and sink.is_cuda and sink.dtype == torch.int32
            and sink.numel() >= 64):
        raise ValueError("x: contiguous GPU tensor; sink: int32 GPU tensor of >= 64 elements")
    with torch.cuda.device(x.device):
        stream = torch.cuda.current_stream(x.device).cuda_stream
        _lib.check(_lib.lib.topk_stream_read(x.data_ptr(), x.numel() * x.element_size(),
                                             sink.data_ptr(), stream), "topk_stream_read")


def scatter(values: torch.Tensor, indices: torch.Tensor, n: int, out: torch.Tensor | None = None,
            mask: torch.Tensor | bool | None = None):
    """Sparse activation from a selection: ``out[r, indices[r, j]] = values[r, j]``,
    every other element zero (BatchTopK, Prof-K section 5).  ``values`` and
    ``indices`` are [rows, k] (or [k]) as ``topk`` returns them; ``out`` is
    [rows, n] of the values' dtype (allocated when None).  ``mask=True`` also
    returns a uint8 [rows, n] mask of the kept places (or pass a tensor to fill).
    Returns ``out``, or ``(out, mask)`` when a mask is asked for."""
    squeeze = values.dim() == 1
    v2 = values.reshape(1, -1) if squeeze else values
    i2 = indices.reshape(1, -1) if squeeze else indices
    if not (v2.is_cuda and i2.is_cuda and v2.is_contiguous() and i2.is_contiguous()
            and i2.dtype == torch.int64 and v2.shape == i2.shape):
        raise ValueError("values, indices: contiguous GPU tensors of one shape, indices int64")
    rows, k = v2.shape
    dev = v2.device
    if out is None:
        out = torch.empty((rows, n), dtype=v2.dtype, device=dev)
    m = None
    if mask is True:
        m = torch.empty((rows, n), dtype=torch.uint8, device=dev)
    elif isinstance(mask, torch.Tensor):
        m = mask
    if not (out.device == dev and out.is_contiguous() and out.dtype == v2.dtype
            and out.numel() == rows * n):
        raise ValueError("out: contiguous tensor of rows * n elements, the values' dtype and device")
    if m is not None and not (m.device == dev and m.is_contiguous() and m.dtype == torch.uint8
                              and m.numel() == rows * n):
        raise ValueError("mask: contiguous uint8 tensor of rows * n elements on the values' device")
    with torch.cuda.device(dev):
        stream = torch.cuda.current_stream(dev).cuda_stream
        _lib.check(_lib.lib.topk_scatter(v2.data_ptr(), i2.data_ptr(), rows, k, n, dtype_code(v2.dtype),
                                         out.data_ptr(), m.data_ptr() if m is not None else None,
                                         stream), "topk_scatter")
    if squeeze:
        out = out.reshape(-1)
        m = m.reshape(-1) if m is not None else None
    return (out, m) if m is not None else out


def batchtopk(acts: torch.Tensor, k_total: int, params: Params | None = None, mask: bool = False):
    """BatchTopK (Prof-K section 5): keep the ``k_total`` largest entries of the
    whole [B, d] activation matrix (one flattened top-k) and zero the rest.
    Returns the sparse [B, d] activation, and its uint8 mask if asked."""
    if acts.dim() != 2 or not acts.is_contiguous():
        raise ValueError("acts must be a contiguous [B, d] tensor")
    flat = acts.reshape(1, -1)
    vals, idx = topk(flat, k_total, params=params)
    res = scatter(vals, idx, flat.shape[1], mask=mask)
    if mask:
        out, m = res
        return out.reshape(acts.shape), m.reshape(acts.shape)
    return res.reshape(acts.shape)
