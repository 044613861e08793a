"""ctypes binding of libtopk_mi355x.so (the C ABI declared in include/topk.h).

Argument marshalling only: every step of the selection runs in the HIP
library.  There is no CPU fallback; if the library is missing the import of
this module raises.
"""
from __future__ import annotations

import ctypes
import os

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libtopk_mi355x.so")

TOPK_OK, TOPK_EINVAL, TOPK_EDTYPE, TOPK_EWORKSPACE, TOPK_EHIP, TOPK_ENOTIMPL = 0, -1, -2, -3, -4, -5
TOPK_ETOOBIG = -6
NOALLOC_SCRATCH_BYTES = 32 << 20   # topk_noalloc's built-in scratch per GPU
DTYPE_CODES = {"int32": 0, "float32": 1, "bf16": 2}
POLICY_EXACT_TAIL, POLICY_ALG1, POLICY_TUNED = 0, 1, 2
PATH_AUTO, PATH_FILTER, PATH_EXACT = 0, 1, 2
# per-row route in read_stats: sampled accepted, sampled then exact fallback,
# exact only, sampled with fewer than k survivors kept (recall < 1)
ROUTE_SAMPLED, ROUTE_FALLBACK, ROUTE_EXACT, ROUTE_PARTIAL = 0, 1, 2, 3
# how the threshold was selected (read_stats "tau_route"): the source in the
# low 3 bits, plus flags for a boundary bin beyond LDS / radix-selected in LDS
(TAU_NONE, TAU_FILTER_LISTS, TAU_KTAU_LISTS, TAU_KTAU_REGS, TAU_KTAU_STREAM, TAU_FORCED,
 TAU_FILTER_RADIX, TAU_FILTER_MERGE) = range(8)
TAU_BIN_STREAMED, TAU_BIN_RADIX = 8, 16
# topk_params.test_flags: every exact-route grid-barrier wait gives up at once
TEST_BARRIER_GIVEUP = 1

# Names of every function include/topk.h declares.
EXPORTS = ("topk_default_params", "topk_plan", "topk_workspace_size", "topk_workspace_init",
           "topk", "topk_ex", "topk_read_stats", "topk_profile_enable", "topk_profile_read",
           "topk_scatter", "topk_stream_read", "topk_status_string", "topk_noalloc",
           "topk_filter_trace")
STAGES = ("sample", "tau", "filter", "refine", "exact", "sort")


class Params(ctypes.Structure):
    _fields_ = [("eps", ctypes.c_double), ("s_min", ctypes.c_int64), ("s_max", ctypes.c_int64),
                ("cost_ratio", ctypes.c_double), ("policy", ctypes.c_int32),
                ("force_path", ctypes.c_int32), ("seed", ctypes.c_uint64),
                ("use_seed", ctypes.c_int32), ("reserved", ctypes.c_int32),
                ("S", ctypes.c_int64), ("t", ctypes.c_int64), ("M", ctypes.c_int64),
                ("tuned_ratio", ctypes.c_double), ("tuned_s_min", ctypes.c_int64),
                ("tuned_ratio_large", ctypes.c_double), ("recall", ctypes.c_double),
                ("force_tau_key", ctypes.c_uint32), ("use_force_tau", ctypes.c_int32),
                ("test_flags", ctypes.c_uint32), ("tuned_batch_rows", ctypes.c_int32),
                ("tuned_ratio_batched", ctypes.c_double)]


class PlanInfo(ctypes.Structure):
    _fields_ = [("path", ctypes.c_int32), ("small_k", ctypes.c_int32), ("S", ctypes.c_int64),
                ("t", ctypes.c_int64), ("M", ctypes.c_int64), ("cap", ctypes.c_int64),
                ("index_bits", ctypes.c_int32), ("key_bits", ctypes.c_int32),
                ("p_recall", ctypes.c_double), ("p_overflow", ctypes.c_double),
                ("workspace_bytes", ctypes.c_size_t), ("k_eff", ctypes.c_int64)]


class StageTimes(ctypes.Structure):
    _fields_ = [("ms", ctypes.c_double * 8), ("count", ctypes.c_int64 * 8)]


class RowStats(ctypes.Structure):
    _fields_ = [("tau_key", ctypes.c_uint32), ("r_sampled", ctypes.c_uint32),
                ("path", ctypes.c_uint32), ("passes", ctypes.c_uint32),
                ("flags", ctypes.c_uint32), ("ties", ctypes.c_uint32),
                ("tau_route", ctypes.c_uint32)]


def _load():
    if not os.path.exists(LIB_PATH):
        raise ImportError(
            f"{LIB_PATH} is not built; run __graft_entry__.build() or "
            "python top_selection_sample_amd/build.py (hipcc, gfx950)")
    L = ctypes.CDLL(LIB_PATH)
    vp, i64, i32, sz = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int, ctypes.c_size_t
    P = ctypes.POINTER
    L.topk_default_params.argtypes = [P(Params)]
    L.topk_plan.argtypes = [i64, i64, i64, i32, P(Params), P(PlanInfo)]
    L.topk_workspace_size.argtypes = [i64, i64, i64, i32, P(Params), P(sz)]
    L.topk_workspace_init.argtypes = [vp, sz, vp]
    L.topk.argtypes = [vp, i64, i64, i64, i32, vp, vp, vp, sz, vp]
    L.topk_ex.argtypes = [vp, i64, i64, i64, i32, vp, vp, vp, sz, vp, P(Params)]
    L.topk_noalloc.argtypes = [vp, i64, i64, i64, i32, vp, vp, vp, P(Params)]
    L.topk_read_stats.argtypes = [vp, i64, P(RowStats), vp]
    L.topk_profile_enable.argtypes = [i32]
    L.topk_profile_read.argtypes = [P(StageTimes)]
    L.topk_filter_trace.argtypes = [ctypes.c_void_p, ctypes.c_size_t]
    L.topk_stream_read.argtypes = [vp, sz, vp, vp]
    L.topk_scatter.argtypes = [vp, vp, i64, i64, i64, i32, vp, vp, vp]
    L.topk_status_string.argtypes = [i32]
    L.topk_status_string.restype = ctypes.c_char_p
    for name in EXPORTS:
        if name != "topk_status_string":
            getattr(L, name).restype = i32
    return L


lib = _load()


class TopkError(RuntimeError):
    def __init__(self, status: int, where: str):
        super().__init__(f"{where}: {lib.topk_status_string(status).decode()} (status {status})")
        self.status = status


def check(status: int, where: str) -> None:
    if status != TOPK_OK:
        raise TopkError(status, where)


def default_params(**kw) -> Params:
    p = Params()
    check(lib.topk_default_params(ctypes.byref(p)), "topk_default_params")
    for k, v in kw.items():
        if not hasattr(p, k):
            raise KeyError(k)
        setattr(p, k, v)
    return p
