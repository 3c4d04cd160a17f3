"""CPU fp64 oracle for the activation-sparse FFN decode path (ctypes wrapper).

TEST INFRASTRUCTURE ONLY: the tests, the smoke check and the benchmark's
CPU-baseline leg are the only callers.  Nothing here imports the GPU package,
and the GPU package never imports this one.

The arithmetic lives in ``asf_oracle.c`` (plain C, double precision); this
module only builds it with gcc, marshals numpy arrays and returns numpy
results.  Each function cites the passage of the pages it follows in the C
source.

Parity status: every function is pinned by tests under ``tests/`` (closed
forms, brute force over tiny layers, numpy float64 cross-checks, exhaustive
binary16 decode, and the worked example of the single-layer figure).
"""
from __future__ import annotations

import ctypes
import os
import subprocess
import threading

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "asf_oracle.c")
_LIB = os.path.join(_HERE, "liboracle.so")
_lock = threading.Lock()
_lib = None

F32, F16 = 0, 1


def build(force: bool = False) -> str:
    """Compile asf_oracle.c into liboracle.so with gcc (OpenMP on)."""
    if force or not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
        tmp = _LIB + ".tmp%d" % os.getpid()
        cmd = ["gcc", "-O2", "-std=c99", "-ffp-contract=off", "-fno-fast-math",
               "-fPIC", "-shared", "-fopenmp", _SRC, "-o", tmp, "-lm"]
        subprocess.run(cmd, check=True)
        os.replace(tmp, _LIB)
    return _LIB


def _load():
    global _lib
    with _lock:
        if _lib is None:
            build()
            lib = ctypes.CDLL(_LIB)
            vp, ip, dp, fp = ctypes.c_void_p, ctypes.c_int, ctypes.c_double, ctypes.c_void_p
            lib.orc_half_to_double.argtypes = [ctypes.c_uint16]
            lib.orc_half_to_double.restype = ctypes.c_double
            lib.orc_predict.argtypes = [ip, ip, ip, ip, vp, fp, vp, fp, dp, fp, ip, vp, vp, vp]
            lib.orc_predict.restype = ip
            lib.orc_union.argtypes = [ip, ip, vp, vp]
            lib.orc_union.restype = None
            lib.orc_hot_first_table.argtypes = [ip, vp, vp]
            lib.orc_hot_first_table.restype = ip
            lib.orc_count_activations.argtypes = [ip, ip, vp, vp]
            lib.orc_count_activations.restype = None
            lib.orc_active_list.argtypes = [ip, vp, vp, vp]
            lib.orc_active_list.restype = ip
            lib.orc_ffn.argtypes = [ip, ip, ip, ip, vp, vp, fp, vp, fp, fp, fp, ip, vp, ip, vp, vp, vp]
            lib.orc_ffn.restype = ip
            lib.orc_dense_ffn.argtypes = [ip, ip, ip, ip, vp, vp, fp, vp, fp, fp, fp, ip, vp]
            lib.orc_dense_ffn.restype = ip
            lib.orc_true_mask.argtypes = [ip, ip, ip, ip, vp, vp, fp, fp, ip, vp, vp]
            lib.orc_true_mask.restype = ip
            lib.orc_num_threads.argtypes = []
            lib.orc_num_threads.restype = ip
            lib.orc_set_num_threads.argtypes = [ip]
            lib.orc_set_num_threads.restype = None
            _lib = lib
    return _lib


# ----------------------------------------------------------------- marshalling
def _ptr(a):
    return None if a is None else ctypes.c_void_p(a.ctypes.data)


def _weights(w):
    """Return (contiguous array, wtype) for a float32 or float16 weight."""
    a = np.ascontiguousarray(w)
    if a.dtype == np.float16:
        return a, F16
    if a.dtype == np.float32:
        return a, F32
    raise TypeError("weights must be float32 or float16, got %s" % a.dtype)


def _f32(v):
    return None if v is None else np.ascontiguousarray(v, dtype=np.float32)


def _x2d(x):
    x = np.ascontiguousarray(x, dtype=np.float32)
    if x.ndim == 1:
        x = x[None, :]
    return x


def num_threads() -> int:
    return _load().orc_num_threads()


def set_num_threads(n: int) -> None:
    _load().orc_set_num_threads(int(n))


def half_to_double(bits: int) -> float:
    return _load().orc_half_to_double(int(bits) & 0xFFFF)


def predict(P1, c1, P2, c2, x, theta: float = 0.0):
    """Predictor scores.  Returns (h [B][H], s [B][f], act [B][f] uint8)."""
    lib = _load()
    P1a, wt1 = _weights(P1)
    P2a, wt2 = _weights(P2)
    if wt1 != wt2:
        raise TypeError("P1 and P2 must share a dtype")
    H, d = P1a.shape
    f, H2 = P2a.shape
    assert H2 == H
    x = _x2d(x)
    B = x.shape[0]
    assert x.shape[1] == d
    c1a, c2a = _f32(c1), _f32(c2)
    h = np.zeros((B, H), np.float64)
    s = np.zeros((B, f), np.float64)
    act = np.zeros((B, f), np.uint8)
    rc = lib.orc_predict(d, f, H, wt1, _ptr(P1a), _ptr(c1a), _ptr(P2a), _ptr(c2a),
                         float(theta), _ptr(x), B, _ptr(h), _ptr(s), _ptr(act))
    if rc != 0:
        raise ValueError("orc_predict failed (%d)" % rc)
    return h, s, act


def predict_heads(Q1, c1, Q2, c2, x, theta: float = 0.0):
    """Attention-head predictor ("LLM模型之PowerInfer1.0", appendix "DejaVu",
    SP_A of Eq. -1): the two-layer MLP of ``predict`` with one output per
    head, head j selected when its logit s_j exceeds theta (the sigmoid-0.5
    decision at theta = 0).  Each token keeps its own set.  Returns
    (s [B][heads], selected [B][heads] uint8, per-token ascending lists)."""
    _, s, act = predict(Q1, c1, Q2, c2, x, theta)
    return s, act, [np.flatnonzero(act[b]).astype(np.int32) for b in range(act.shape[0])]


def union(act):
    lib = _load()
    act = np.ascontiguousarray(act, dtype=np.uint8)
    B, f = act.shape
    u = np.zeros(f, np.uint8)
    lib.orc_union(B, f, _ptr(act), _ptr(u))
    return u


def hot_first_table(counts):
    lib = _load()
    c = np.ascontiguousarray(counts, dtype=np.int64)
    perm = np.zeros(c.shape[0], np.int32)
    rc = lib.orc_hot_first_table(c.shape[0], _ptr(c), _ptr(perm))
    if rc != 0:
        raise ValueError("orc_hot_first_table failed (%d)" % rc)
    return perm


def count_activations(act, counts=None):
    lib = _load()
    act = np.ascontiguousarray(act, dtype=np.uint8)
    if act.ndim == 1:
        act = act[None, :]
    B, f = act.shape
    c = np.zeros(f, np.int64) if counts is None else np.ascontiguousarray(counts, dtype=np.int64).copy()
    lib.orc_count_activations(B, f, _ptr(act), _ptr(c))
    return c


def active_list(active_by_id, perm=None):
    """Original ids of the active neurons, in ascending stored-slot order."""
    lib = _load()
    m = np.ascontiguousarray(active_by_id, dtype=np.uint8)
    f = m.shape[0]
    p = None if perm is None else np.ascontiguousarray(perm, dtype=np.int32)
    out = np.zeros(f, np.int32)
    n = lib.orc_active_list(f, _ptr(p), _ptr(m), _ptr(out))
    return out[:n].copy()


def ffn(W_up, W_down, x, S, b1=None, b2=None, W_gate=None, resid=None,
        token_act=None, return_a: bool = False):
    """FFN over the neuron set S (original ids).  Returns y [B][d] float64
    (and a [B][len(S)] in ascending-id order when return_a)."""
    lib = _load()
    Wu, wt = _weights(W_up)
    Wd, wt2 = _weights(W_down)
    gated = W_gate is not None
    Wg = None
    if gated:
        Wg, wt3 = _weights(W_gate)
        assert wt3 == wt
    assert wt2 == wt
    f, d = Wu.shape
    assert Wd.shape == (d, f)
    x = _x2d(x)
    B = x.shape[0]
    S = np.ascontiguousarray(np.asarray(S, dtype=np.int32).reshape(-1))
    nS = S.shape[0]
    ta = None if token_act is None else np.ascontiguousarray(token_act, dtype=np.uint8)
    r = None if resid is None else _x2d(resid)
    y = np.zeros((B, d), np.float64)
    a = np.zeros((B, max(nS, 1)), np.float64) if return_a else None
    rc = lib.orc_ffn(d, f, wt, int(gated), _ptr(Wu), _ptr(Wg), _ptr(_f32(b1)), _ptr(Wd),
                     _ptr(_f32(b2)), _ptr(r), _ptr(x), B, _ptr(S), nS, _ptr(ta), _ptr(a), _ptr(y))
    if rc != 0:
        raise ValueError("orc_ffn failed (%d)" % rc)
    if return_a:
        return y, a[:, :nS]
    return y


def dense_ffn(W_up, W_down, x, b1=None, b2=None, W_gate=None, resid=None):
    lib = _load()
    Wu, wt = _weights(W_up)
    Wd, _ = _weights(W_down)
    gated = W_gate is not None
    Wg = _weights(W_gate)[0] if gated else None
    f, d = Wu.shape
    x = _x2d(x)
    B = x.shape[0]
    r = None if resid is None else _x2d(resid)
    y = np.zeros((B, d), np.float64)
    rc = lib.orc_dense_ffn(d, f, wt, int(gated), _ptr(Wu), _ptr(Wg), _ptr(_f32(b1)), _ptr(Wd),
                           _ptr(_f32(b2)), _ptr(r), _ptr(x), B, _ptr(y))
    if rc != 0:
        raise ValueError("orc_dense_ffn failed (%d)" % rc)
    return y


def true_mask(W_up, x, b1=None, W_gate=None):
    """(pre-activation [B][f], mask [B][f]) of FC1 (of the gate when gated)."""
    lib = _load()
    Wu, wt = _weights(W_up)
    gated = W_gate is not None
    Wg = _weights(W_gate)[0] if gated else None
    f, d = Wu.shape
    x = _x2d(x)
    B = x.shape[0]
    pre = np.zeros((B, f), np.float64)
    act = np.zeros((B, f), np.uint8)
    rc = lib.orc_true_mask(d, f, wt, int(gated), _ptr(Wu), _ptr(Wg), _ptr(_f32(b1)),
                           _ptr(x), B, _ptr(pre), _ptr(act))
    if rc != 0:
        raise ValueError("orc_true_mask failed (%d)" % rc)
    return pre, act
