"""CPU fp64 oracle for the sparse mixture-of-experts feed-forward layer.

TEST INFRASTRUCTURE ONLY.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
benchmark's ``cpu_baseline`` leg may import this package.  The GPU library and
its Python binding never import, link or call it, and they share no code.

The arithmetic lives in ``moe_oracle.c`` (plain C, double precision, OpenMP over
tokens); this module only compiles it with gcc and marshals numpy arrays.
What it computes follows Mixtral of Experts (wikillm.com card, "Method"):
bias-free linear router, top-K with a softmax over the K kept logits only
(section 2.1 display 2), SwiGLU experts w2.(SiLU(x.w1) * (x.w3)) (SwiGLU
pseudocode), gate-weighted sum from zero (section 2.1 displays 1 and 3).

Parity pins (see ``tests/test_oracle_pins.py``): gate invariants and the
two-logit closed form, brute force over all experts with masked top-k, the
identical-experts reduction to a dense SwiGLU FFN, the K=1 / K=E / E=1 special
cases, the all-equal-logits tie case, permutation and scaling invariants,
uniform-routing statistics against the pages' table of routing repeats, and
the parameter counts of the pages' hyperparameter table.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
import threading

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "moe_oracle.c")
_BUILD_DIR = os.path.join(_HERE, "_build")
_LIB_PATH = os.path.join(_BUILD_DIR, "libmoe_oracle.so")

F32 = 0
BF16 = 1

_lib = None
_lock = threading.Lock()


def build(force: bool = True) -> str:
    """Compile moe_oracle.c into a shared library with gcc; returns its path."""
    if not force and os.path.exists(_LIB_PATH):
        return _LIB_PATH
    os.makedirs(_BUILD_DIR, exist_ok=True)
    tmp = _LIB_PATH + ".tmp%d" % os.getpid()
    cmd = ["gcc", "-O2", "-fopenmp", "-fPIC", "-shared", "-std=c11",
           "-Wall", "-Wextra", "-I", _HERE, _SRC, "-o", tmp, "-lm"]
    subprocess.run(cmd, check=True)
    os.replace(tmp, _LIB_PATH)
    return _LIB_PATH


def configure(lib):
    """Set the ctypes signatures of a loaded oracle library; returns it."""
    P = ctypes.c_void_p
    I64 = ctypes.c_int64
    lib.oracle_route.argtypes = [P, P, P, ctypes.c_int, I64, I64, I64, I64, P, P, P]
    lib.oracle_route.restype = ctypes.c_int
    lib.oracle_moe_tokens.argtypes = [P, P, P, P, P, P, ctypes.c_int,
                                      I64, I64, I64, I64, I64,
                                      P, I64, ctypes.c_int, P, P, P, P, P]
    lib.oracle_moe_tokens.restype = ctypes.c_int
    lib.oracle_rmsnorm.argtypes = [P, ctypes.c_int, I64, I64, ctypes.c_double, P]
    lib.oracle_rmsnorm.restype = ctypes.c_int
    lib.oracle_num_threads.argtypes = []
    lib.oracle_num_threads.restype = ctypes.c_int
    return lib


def _load():
    global _lib
    with _lock:
        if _lib is not None:
            return _lib
        if not os.path.exists(_LIB_PATH):
            build(force=True)
        _lib = configure(ctypes.CDLL(_LIB_PATH))
        return _lib


def _as_input(a: np.ndarray) -> tuple[np.ndarray, int]:
    """Accept float32 arrays or bfloat16 bit patterns stored as uint16."""
    a = np.ascontiguousarray(a)
    if a.dtype == np.float32:
        return a, F32
    if a.dtype == np.uint16:
        return a, BF16
    raise TypeError("oracle inputs must be float32 or uint16 (bfloat16 bits), got %s" % a.dtype)


def _ptr(a):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def num_threads() -> int:
    return int(_load().oracle_num_threads())


def route(x, w_router, k, bias=None):
    """Routing for all tokens.

    x [T,d], w_router [d,E] (float32, or uint16 holding bfloat16 bits).
    Returns (logits [T,E] f64, ids [T,k] i32, gates [T,k] f64).
    """
    lib = _load()
    x, dt = _as_input(x)
    w_router, dt2 = _as_input(w_router)
    if dt != dt2:
        raise TypeError("x and w_router must share a dtype")
    T, d = x.shape
    d2, E = w_router.shape
    if d2 != d:
        raise ValueError("w_router must be [d,E]")
    b = None if bias is None else np.ascontiguousarray(bias, dtype=np.float32)
    logits = np.zeros((T, E), np.float64)
    ids = np.zeros((T, k), np.int32)
    gates = np.zeros((T, k), np.float64)
    rc = lib.oracle_route(_ptr(x), _ptr(w_router), _ptr(b), dt, T, d, E, k,
                          _ptr(logits), _ptr(ids), _ptr(gates))
    if rc != 0:
        raise ValueError("oracle_route failed (%d)" % rc)
    return logits, ids, gates


def moe_tokens(x, w_router, w1, w3, w2, k, tokens=None, bias=None,
               forced_ids=None, forced_gates=None, want_y=False, want_h=False):
    """The layer for the listed tokens (all when ``tokens`` is None).

    Returns a dict with out [n,d], ids [n,k], gates [n,k] and, if asked,
    y [n,k,d] (expert outputs) and h [n,k,f] (SwiGLU activations); all f64.
    With forced_ids/forced_gates the router is skipped and the given
    selection is used.
    """
    lib = _load()
    x, dt = _as_input(x)
    ws = [_as_input(w) for w in (w1, w3, w2)]
    if any(w[1] != dt for w in ws):
        raise TypeError("x and expert weights must share a dtype")
    w1, w3, w2 = (w[0] for w in ws)
    T, d = x.shape
    E, d1, f = w1.shape
    if d1 != d or w3.shape != w1.shape or w2.shape != (E, f, d):
        raise ValueError("weights must be w1,w3 [E,d,f] and w2 [E,f,d]")
    forced = forced_ids is not None
    if forced:
        wr = None
    else:
        wr, dtr = _as_input(w_router)
        if dtr != dt or wr.shape != (d, E):
            raise ValueError("w_router must be [d,E] of the input dtype")
    if tokens is None:
        tok = None
        n = T
    else:
        tok = np.ascontiguousarray(tokens, dtype=np.int64)
        n = tok.shape[0]
    if forced:
        ids = np.ascontiguousarray(forced_ids, dtype=np.int32).reshape(n, k).copy()
        gates = np.ascontiguousarray(forced_gates, dtype=np.float64).reshape(n, k).copy()
    else:
        ids = np.zeros((n, k), np.int32)
        gates = np.zeros((n, k), np.float64)
    b = None if bias is None else np.ascontiguousarray(bias, dtype=np.float32)
    out = np.zeros((n, d), np.float64)
    y = np.zeros((n, k, d), np.float64) if want_y else None
    h = np.zeros((n, k, f), np.float64) if want_h else None
    rc = lib.oracle_moe_tokens(_ptr(x), _ptr(wr), _ptr(b), _ptr(w1), _ptr(w3), _ptr(w2), dt,
                               T, d, f, E, k, _ptr(tok), n, 1 if forced else 0,
                               _ptr(ids), _ptr(gates), _ptr(out), _ptr(y), _ptr(h))
    if rc != 0:
        raise ValueError("oracle_moe_tokens failed (%d)" % rc)
    res = {"out": out, "ids": ids, "gates": gates}
    if want_y:
        res["y"] = y
    if want_h:
        res["h"] = h
    return res


def rmsnorm(h, eps):
    """Unit-gain RMSNorm of each row of h [T,d]; returns f64 [T,d]."""
    lib = _load()
    h, dt = _as_input(h)
    T, d = h.shape
    out = np.zeros((T, d), np.float64)
    rc = lib.oracle_rmsnorm(_ptr(h), dt, T, d, float(eps), _ptr(out))
    if rc != 0:
        raise ValueError("oracle_rmsnorm failed (%d)" % rc)
    return out
