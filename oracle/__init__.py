"""Python access to the fp64 CPU oracle in ``oracle.c``.

TEST INFRASTRUCTURE ONLY: the tests, the smoke check and the benchmark's
CPU-baseline leg may call this; the product library never does.  The shared
object is compiled with gcc from ``oracle.c`` (``build()``); nothing here
shares code with the HIP library.

Logit arrays are numpy ``uint16`` (bf16 bit patterns) or ``float32``.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from typing import Optional

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(_HERE, "oracle.c")
LIB = os.path.join(_HERE, "liboracle.so")

F32, BF16 = 0, 1
TIE_EPS = 1e-6

_lib = None


def build(force: bool = True) -> str:
    """Compile oracle.c into liboracle.so with gcc (plain -O2, no fast-math)."""
    if force or not os.path.exists(LIB) or os.path.getmtime(LIB) < os.path.getmtime(SRC):
        tmp = LIB + f".tmp{os.getpid()}"
        subprocess.check_call(["gcc", "-O2", "-std=c11", "-fPIC", "-shared", "-Wall",
                               "-o", tmp, SRC, "-lm"])
        os.replace(tmp, LIB)
    return LIB


def load(path: Optional[str] = None):
    """Load the compiled oracle (building it first if it is missing or stale)."""
    global _lib
    if path is not None:
        lib = ctypes.CDLL(path)
        _declare(lib)
        return lib
    if _lib is None:
        build(force=False)
        _lib = ctypes.CDLL(LIB)
        _declare(_lib)
    return _lib


_p = ctypes.c_void_p
_i = ctypes.c_int
_d = ctypes.c_double


def _declare(lib):
    lib.oracle_verify_batch.restype = _i
    lib.oracle_verify_batch.argtypes = [_p, _i, _p, _i, _p, _p, _p, _p, _p, _i, _i, _i, _d,
                                        _p, _p, _p, _p, _p, _p, _p]
    lib.oracle_tv_accept_rate.restype = _i
    lib.oracle_tv_accept_rate.argtypes = [_p, _p, _i, _p, _i, _i, _p, _p]
    lib.oracle_markov_draft.restype = _i
    lib.oracle_markov_draft.argtypes = [_p, _i, _p, _p, _i, _p, _p, _p, _i, _i, _i, _i, _d,
                                        _p, _p, _p, _p]
    lib.oracle_inverse_cdf.restype = _i
    lib.oracle_inverse_cdf.argtypes = [_p, _i, _d, _p]


def _dt(x: np.ndarray) -> int:
    if x.dtype == np.uint16:
        return BF16
    if x.dtype == np.float32:
        return F32
    raise TypeError(f"logits must be uint16 (bf16 bits) or float32, got {x.dtype}")


def _c(x, dtype):
    return np.ascontiguousarray(x, dtype=dtype)


def _ptr(x: Optional[np.ndarray]):
    return None if x is None else x.ctypes.data_as(ctypes.c_void_p)


def verify_batch(target, draft, draft_tokens, verify_len, temperature, u_accept, u_sample,
                 tie_eps: float = TIE_EPS, lib=None) -> dict:
    """Batched verification of one call; returns a dict of numpy arrays:
    tokens [R, gamma+1], num_accepted [R], cstar / resid [R, gamma] (fp64),
    logq [R, gamma+1] (fp64), margin_min [R], first_tie [R], invalid (count)."""
    lib = lib or load()
    R, G1, V = target.shape
    gamma = G1 - 1
    assert draft.shape == (R, gamma, V), (draft.shape, target.shape)
    target = np.ascontiguousarray(target)
    draft = np.ascontiguousarray(draft)
    tok = _c(draft_tokens, np.int32)
    vl = _c(verify_len, np.int32)
    T = _c(temperature, np.float32)
    ua = _c(u_accept, np.float32)
    us = _c(u_sample, np.float32)
    out_tok = np.empty((R, G1), np.int32)
    out_n = np.empty((R,), np.int32)
    out_cs = np.empty((R, gamma), np.float64)
    out_rs = np.empty((R, gamma), np.float64)
    out_lq = np.empty((R, G1), np.float64)
    out_mg = np.empty((R,), np.float64)
    out_ft = np.empty((R,), np.int32)
    bad = lib.oracle_verify_batch(_ptr(target), _dt(target), _ptr(draft), _dt(draft), _ptr(tok),
                                  _ptr(vl), _ptr(T), _ptr(ua), _ptr(us), R, gamma, V,
                                  float(tie_eps), _ptr(out_tok), _ptr(out_n), _ptr(out_cs),
                                  _ptr(out_rs), _ptr(out_lq), _ptr(out_mg), _ptr(out_ft))
    if bad < 0:
        raise MemoryError("oracle_verify_batch")
    return dict(tokens=out_tok, num_accepted=out_n, cstar=out_cs, resid=out_rs, logq=out_lq,
                margin_min=out_mg, first_tie=out_ft, invalid=bad)


def verify_case(case, tie_eps: float = TIE_EPS, lib=None) -> dict:
    return verify_batch(case.target, case.draft, case.draft_tokens, case.verify_len,
                        case.temperature, case.u_accept, case.u_sample, tie_eps, lib)


def tv_accept_rate(draft, target, temperature, lib=None):
    """c* and Res for N row pairs [N, V]; returns (cstar, resid) fp64 arrays."""
    lib = lib or load()
    assert draft.shape == target.shape and draft.dtype == target.dtype
    N, V = target.shape
    draft = np.ascontiguousarray(draft)
    target = np.ascontiguousarray(target)
    T = _c(temperature, np.float32)
    cs = np.empty((N,), np.float64)
    rs = np.empty((N,), np.float64)
    bad = lib.oracle_tv_accept_rate(_ptr(draft), _ptr(target), _dt(target), _ptr(T), N, V,
                                    _ptr(cs), _ptr(rs))
    if bad < 0:
        raise MemoryError("oracle_tv_accept_rate")
    return cs, rs


def markov_draft(U, W1, W2, anchor, temperature, u_draft, tie_eps: float = TIE_EPS,
                 want_logits: bool = True, lib=None) -> dict:
    """Serial Markov-head draft; returns tokens [R, gamma], logits [R, gamma, V]
    fp32 (if want_logits), margin_min [R], first_tie [R], invalid (count)."""
    lib = lib or load()
    R, gamma, V = U.shape
    rank = W1.shape[1]
    assert W1.shape == (V, rank) and W2.shape == (rank, V) and W1.dtype == W2.dtype
    U = np.ascontiguousarray(U)
    W1 = np.ascontiguousarray(W1)
    W2 = np.ascontiguousarray(W2)
    a = _c(anchor, np.int32)
    T = _c(temperature, np.float32)
    ud = _c(u_draft, np.float32)
    tok = np.empty((R, gamma), np.int32)
    logits = np.empty((R, gamma, V), np.float32) if want_logits else None
    mg = np.empty((R,), np.float64)
    ft = np.empty((R,), np.int32)
    bad = lib.oracle_markov_draft(_ptr(U), _dt(U), _ptr(W1), _ptr(W2), _dt(W1), _ptr(a), _ptr(T),
                                  _ptr(ud), R, gamma, V, rank, float(tie_eps), _ptr(tok),
                                  _ptr(logits), _ptr(mg), _ptr(ft))
    if bad < 0:
        raise MemoryError("oracle_markov_draft")
    return dict(tokens=tok, logits=logits, margin_min=mg, first_tie=ft, invalid=bad)


def inverse_cdf(w, u: float, lib=None):
    """(token, margin) of the oracle's inverse-CDF draw on fp64 weights w."""
    lib = lib or load()
    w = _c(w, np.float64)
    m = ctypes.c_double(0.0)
    t = lib.oracle_inverse_cdf(_ptr(w), int(w.size), float(u), ctypes.byref(m))
    return t, m.value
