"""CPU oracle for exact top-k selection (test infrastructure).

Only the test suite, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg
of ``bench.py`` may import this package.  The product library never does, and
the two share no code: this package has its own key functions, its own
sampler and its own parameter arithmetic.

Contents
--------
* ``topk``            exact top-k of each row: partial sort on (key desc,
                      index asc) (Prof-K paper, section 3; GPU.js Learn
                      "Rank by Counting" for the tie rule).  C++ core.
* ``topk_chunked``    the same selection on several threads (chunks of each
                      row, then one selection over the chunks' own top-k),
                      for the CPU timing.
* ``keys``            order-preserving unsigned keys, written with numpy.
* ``rank_by_counting``  O(n^2) rank of every element: how many elements
                      precede it (a bigger key, or the same key at a
                      smaller index; GPU.js Learn "Rank by Counting", Goal
                      and Hint 2).
* ``bisection_cutoff``  counting bisection on the value axis (GPU.js Learn
                      "Find the Cutoff Instead", Requirements and Hint 3).
* ``outranking``      number of elements that outrank a given (key, index).
* ``sample_indices`` / ``tau``  the sampler and the sample threshold
                      (Prof-K section 3, stages 1 and 2); C++ core.
* ``params``          Algorithm 1 and the exact-tail reading of Theorem 3
                      (submodule ``oracle.params``).
* ``sparse_activation``  the BatchTopK consumer (Prof-K section 5): the
                      selected activations kept in place, zero elsewhere,
                      and the mask of the kept places.
* ``relaxed_selection``  the relaxed-recall trade (Prof-K abstract and
                      section 1): a row whose survivors number at least
                      k_eff but fewer than k keeps them, in rank order, and
                      pads the other slots.

bf16 data is carried as its uint16 bit patterns with ``dtype="bf16"``.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "topk_oracle.cpp")
_LIB_PATH = os.path.join(_HERE, "liboracle.so")

DTYPES = {"int32": 0, "float32": 1, "bf16": 2}
_ELEM = {"int32": 4, "float32": 4, "bf16": 2}
_NP = {"int32": np.int32, "float32": np.float32, "bf16": np.uint16}


def build(force: bool = True) -> str:
    """Compile the C++ core with the host compiler (no GPU code)."""
    if force or not os.path.exists(_LIB_PATH):
        tmp = _LIB_PATH + ".tmp"
        subprocess.check_call(
            ["g++", "-O2", "-std=c++17", "-shared", "-fPIC", "-pthread", "-o", tmp, _SRC])
        os.replace(tmp, _LIB_PATH)
    return _LIB_PATH


_lib = None


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB_PATH):
            build(force=False)
        L = ctypes.CDLL(_LIB_PATH)
        vp, i64, u64, i32 = ctypes.c_void_p, ctypes.c_int64, ctypes.c_uint64, ctypes.c_int
        L.oracle_topk.argtypes = [vp, i64, i64, i64, i32, vp, vp]
        L.oracle_topk_chunked.argtypes = [vp, i64, i64, i64, i32, i32, vp, vp]
        L.oracle_keys.argtypes = [vp, i64, i32, vp]
        L.oracle_sample_indices.argtypes = [u64, u64, u64, u64, vp]
        L.oracle_feistel_raw.argtypes = [u64, u64, u64, u64, vp]
        L.oracle_tau.argtypes = [vp, u64, i32, u64, u64, u64, u64, vp, vp, vp]
        _lib = L
    return _lib


def _dtype_name(x: np.ndarray, dtype: str | None) -> str:
    if dtype is not None:
        return dtype
    if x.dtype == np.int32:
        return "int32"
    if x.dtype == np.float32:
        return "float32"
    raise TypeError("pass dtype='bf16' for uint16 bf16 bit patterns")


def _ptr(a: np.ndarray) -> int:
    return a.ctypes.data


# ---------------------------------------------------------------- keys (numpy)
def keys(x: np.ndarray, dtype: str | None = None) -> np.ndarray:
    """Order-preserving uint32 keys (numpy version, independent of the C++).

    int32: flip the sign bit.  float: negatives reverse all bits, positives set
    the sign bit; -0.0 takes +0.0's key; every NaN takes the largest key.
    """
    dt = _dtype_name(x, dtype)
    if dt == "int32":
        return x.view(np.uint32) ^ np.uint32(0x80000000)
    if dt == "float32":
        b = x.view(np.uint32).astype(np.uint32)
        sign, mag = np.uint32(0x80000000), np.uint32(0x7FFFFFFF)
        top = np.uint32(0xFFFFFFFF)
        k = np.where(b & sign, ~b, b | sign)
        k = np.where((b & mag) == 0, sign, k)
        k = np.where((b & mag) > np.uint32(0x7F800000), top, k)
        return k.astype(np.uint32)
    if dt == "bf16":
        b = x.view(np.uint16).astype(np.uint32)
        sign, mag = np.uint32(0x8000), np.uint32(0x7FFF)
        k = np.where(b & sign, (~b) & np.uint32(0xFFFF), b | sign)
        k = np.where((b & mag) == 0, sign, k)
        k = np.where((b & mag) > np.uint32(0x7F80), np.uint32(0xFFFF), k)
        return k.astype(np.uint32)
    raise ValueError(dt)


def keys_c(x: np.ndarray, dtype: str | None = None) -> np.ndarray:
    """Same keys through the C++ core (used to cross-check the two)."""
    dt = _dtype_name(x, dtype)
    x = np.ascontiguousarray(x)
    out = np.empty(x.size, dtype=np.uint32)
    rc = lib().oracle_keys(_ptr(x), x.size, DTYPES[dt], _ptr(out))
    assert rc == 0
    return out.reshape(x.shape)


# ---------------------------------------------------------------- exact top-k
def topk(x: np.ndarray, k: int, dtype: str | None = None):
    """Exact top-k of every row of a 1-D or 2-D array.

    Returns (values [rows, k] in the input's numpy dtype, indices [rows, k]
    int64), in rank order: key descending, ties by lower index.
    """
    dt = _dtype_name(x, dtype)
    x2 = np.ascontiguousarray(x.reshape(1, -1) if x.ndim == 1 else x)
    rows, n = x2.shape
    ov = np.empty((rows, k), dtype=_NP[dt])
    oi = np.empty((rows, k), dtype=np.int64)
    rc = lib().oracle_topk(_ptr(x2), n, rows, k, DTYPES[dt], _ptr(ov), _ptr(oi))
    if rc != 0:
        raise ValueError(f"oracle_topk rejected arguments (rc={rc})")
    return ov, oi


def topk_chunked(x: np.ndarray, k: int, threads: int, dtype: str | None = None):
    """``topk`` on `threads` CPU threads (contiguous chunks of each row, each
    keeps its own top-k, then one selection over the union); for timing the
    CPU side with every core."""
    dt = _dtype_name(x, dtype)
    x2 = np.ascontiguousarray(x.reshape(1, -1) if x.ndim == 1 else x)
    rows, n = x2.shape
    ov = np.empty((rows, k), dtype=_NP[dt])
    oi = np.empty((rows, k), dtype=np.int64)
    rc = lib().oracle_topk_chunked(_ptr(x2), n, rows, k, DTYPES[dt], threads, _ptr(ov), _ptr(oi))
    if rc != 0:
        raise ValueError(f"oracle_topk_chunked rejected arguments (rc={rc})")
    return ov, oi


# ---------------------------------------------------------------- definitions
def rank_by_counting(x: np.ndarray, dtype: str | None = None) -> np.ndarray:
    """Rank of every element of a 1-D row, as GPU.js Learn "Rank by Counting"
    (section Goal) defines the output position: count the elements that come
    before it, i.e. every element with a bigger key, plus every element with
    the same key and a smaller index.  O(n^2) memory and time: tiny rows
    only."""
    k = keys(x, dtype).astype(np.int64)
    n = k.size
    assert n <= 8192, "brute force is for tiny rows"
    idx = np.arange(n)
    larger = k[None, :] > k[:, None]
    equal_before = (k[None, :] == k[:, None]) & (idx[None, :] < idx[:, None])
    return (larger | equal_before).sum(axis=1)


def outranking(row_keys: np.ndarray, key: int, index: int) -> int:
    """#elements of a row that outrank the element (key, index)."""
    rk = row_keys
    gt = int(np.count_nonzero(rk > np.uint32(key)))
    eq_before = int(np.count_nonzero(rk[:index] == np.uint32(key)))
    return gt + eq_before


def bisection_cutoff(x: np.ndarray, k: int):
    """Counting bisection for integer scores: keep lo with count(> lo) >= k and
    hi with count(> hi) < k, halve until hi - lo <= 0.5, return floor(lo) and
    how many scores are strictly above it.

    Reading where the page is silent: the starting bracket is
    lo = min(x) - 1 (everything is above it) and hi = max(x) (nothing is).
    """
    v = x.astype(np.float64)
    lo, hi = float(v.min()) - 1.0, float(v.max())
    steps = 0
    while hi - lo > 0.5:
        mid = (lo + hi) / 2
        if np.count_nonzero(v > mid) >= k:
            lo = mid
        else:
            hi = mid
        steps += 1
    cutoff = int(np.floor(lo))
    return cutoff, int(np.count_nonzero(v > cutoff)), steps


# ---------------------------------------------------------------- sampler
def sample_indices(seed: int, row: int, n: int, S: int) -> np.ndarray:
    out = np.empty(S, dtype=np.uint64)
    rc = lib().oracle_sample_indices(seed, row, n, S, _ptr(out))
    assert rc == 0
    return out


def feistel_raw(seed: int, row: int, n: int, count: int) -> np.ndarray:
    out = np.empty(count, dtype=np.uint64)
    rc = lib().oracle_feistel_raw(seed, row, n, count, _ptr(out))
    assert rc == 0
    return out


def tau(row_values: np.ndarray, seed: int, row: int, S: int, t: int,
        dtype: str | None = None, with_sample: bool = False):
    """(tau_key, R[, sample_keys]) for one row."""
    dt = _dtype_name(row_values, dtype)
    rv = np.ascontiguousarray(row_values.reshape(-1))
    tk = ctypes.c_uint32()
    R = ctypes.c_uint64()
    sk = np.empty(S, dtype=np.uint32)
    rc = lib().oracle_tau(_ptr(rv), rv.size, DTYPES[dt], seed, row, S, t,
                          ctypes.addressof(tk), ctypes.addressof(R), _ptr(sk))
    if rc != 0:
        raise ValueError(f"oracle_tau rejected arguments (rc={rc})")
    if with_sample:
        return tk.value, R.value, sk
    return tk.value, R.value


def sparse_activation(values: np.ndarray, indices: np.ndarray, n: int):
    """BatchTopK consumer (Prof-K section 5, "Application: BatchTopK Sparse
    Autoencoders": the largest K of the flattened activations are selected;
    the sparse activation keeps them and is zero elsewhere).  values,
    indices: [rows, k] as ``topk`` returns them (bf16 as uint16 bits).
    Returns (dense [rows, n] of the values' dtype, mask [rows, n] uint8)."""
    values = np.asarray(values)
    indices = np.asarray(indices, dtype=np.int64)
    if values.ndim == 1:
        values, indices = values[None, :], indices[None, :]
    rows = values.shape[0]
    out = np.zeros((rows, n), dtype=values.dtype)
    mask = np.zeros((rows, n), dtype=np.uint8)
    for r in range(rows):
        out[r, indices[r]] = values[r]
        mask[r, indices[r]] = 1
    return out, mask


# lowest value of each dtype, the padding of a slot no winner fills (bf16 as
# its bit pattern)
PAD_VALUE = {"float32": np.float32(-np.inf), "int32": np.int32(-2 ** 31),
             "bf16": np.uint16(0xFF80)}


def relaxed_selection(row: np.ndarray, k: int, k_eff: int, tau_key: int, cap: int,
                      dtype: str | None = None):
    """One row under a relaxed recall target (Prof-K abstract and section 1:
    recall traded for speed, e.g. 95% of the true top-k).

    Reading: the survivors are the elements whose key is at least tau
    (stage 3), R of them.  When k_eff <= R < k and R <= cap the row keeps
    them: sorted by key descending, ties by lower index, they fill slots
    0..R-1, and slots R..k-1 get index -1 and the dtype's lowest value.
    Any other row ends with the exact top-k (accepted with R >= k, or taken
    by the exact fallback).  Returns (values [k], indices [k], partial).
    """
    dt = _dtype_name(row, dtype)
    rv = np.ascontiguousarray(np.asarray(row).reshape(-1))
    kk = keys(rv, dt).astype(np.int64)
    surv = np.flatnonzero(kk >= int(tau_key))
    R = int(surv.size)
    if not (k_eff <= R < k and R <= cap):
        v, i = topk(rv, k, dt)
        return v[0], i[0], False
    order = surv[np.lexsort((surv, -kk[surv]))]   # key descending, then index
    vals = np.full(k, PAD_VALUE[dt], dtype=_NP[dt])
    idx = np.full(k, -1, dtype=np.int64)
    vals[:R] = rv[order]
    idx[:R] = order
    return vals, idx, True
