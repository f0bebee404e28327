"""fp64 CPU oracle for the attention-KL divergence (test infrastructure).

TEST INFRASTRUCTURE ONLY: the tests, the smoke check and the benchmark's
CPU-baseline leg may import this package; the product path never does.  It
shares no code with the HIP library (see ``streamkl_oracle.c`` for what it
computes and which passages of the StreamKL summary page each step follows).

``head`` takes the query and key rows of one attention head as numpy arrays
(or anything ``np.asarray`` accepts) shaped [N, d] and returns float64 arrays.
"""
import ctypes
import os

import numpy as np

from . import build_oracle

_lib = None
_dp = ctypes.POINTER(ctypes.c_double)


def load_library(path):
    """Open an oracle build at ``path`` (the default one, or a test's variant)."""
    lib = ctypes.CDLL(path)
    args = [_dp, _dp, _dp, _dp, _dp, ctypes.c_int, ctypes.c_int, ctypes.c_int,
            ctypes.c_double, ctypes.c_int, ctypes.c_int, ctypes.c_int,
            _dp, _dp, _dp, _dp, _dp, _dp, _dp]
    lib.oracle_head.argtypes = args
    lib.oracle_head.restype = ctypes.c_int
    lib.oracle_num_threads.argtypes = []
    lib.oracle_num_threads.restype = ctypes.c_int
    return lib


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(build_oracle.LIB):
            build_oracle.build()
        _lib = load_library(build_oracle.LIB)
    return _lib


def num_threads() -> int:
    return _load().oracle_num_threads()


def _f64(x):
    return np.ascontiguousarray(np.asarray(x, dtype=np.float64))


def _ptr(a):
    if a is None:
        return None
    return a.ctypes.data_as(_dp)


def head(q1, k1, q2, k2, scale, causal, g=None, rows=None, grads=False, lib=None):
    """One head.  q*: [N_Q, d], k*: [N_K, d] (converted to float64 exactly).

    rows: (begin, end) query-row range (default: all rows).  Returns a dict
    with 'kl', 'lse1', 'lse2' ([N_Q], only rows in range meaningful) and,
    if grads, 'dq1', 'dq2' ([N_Q, d], rows in range) and 'dk1', 'dk2'
    ([N_K, d], contribution of the rows in range).
    ``lib``: an alternative build from ``load_library`` (default: the oracle).
    """
    lib = lib or _load()
    q1, k1, q2, k2 = _f64(q1), _f64(k1), _f64(q2), _f64(k2)
    n_q, d = q1.shape
    n_k = k1.shape[0]
    assert q2.shape == (n_q, d) and k1.shape == (n_k, d) and k2.shape == (n_k, d)
    rb, re = (0, n_q) if rows is None else rows
    gv = None if g is None else _f64(g).reshape(n_q)
    out = {k: np.full(n_q, np.nan) for k in ("kl", "lse1", "lse2")}
    if grads:
        out["dq1"] = np.full((n_q, d), np.nan)
        out["dq2"] = np.full((n_q, d), np.nan)
        out["dk1"] = np.zeros((n_k, d))
        out["dk2"] = np.zeros((n_k, d))
    rc = lib.oracle_head(_ptr(q1), _ptr(k1), _ptr(q2), _ptr(k2), _ptr(gv),
                         n_q, n_k, d, float(scale), int(bool(causal)), rb, re,
                         _ptr(out["kl"]), _ptr(out["lse1"]), _ptr(out["lse2"]),
                         _ptr(out.get("dq1")), _ptr(out.get("dk1")),
                         _ptr(out.get("dq2")), _ptr(out.get("dk2")))
    if rc != 0:
        raise MemoryError("oracle scratch allocation failed")
    return out
