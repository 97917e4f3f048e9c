"""Float64 CPU oracle for the attention forward pass (ctypes over oracle.c).

TEST INFRASTRUCTURE ONLY: the test suite, the smoke check and the bench's
CPU-baseline leg use it; the HIP product path never imports it.  It shares no
code with the HIP path.  ``brute`` holds a second, exact-arithmetic
implementation for tiny shapes.

Every function takes fp16 numpy arrays of shape [B, H, S, D] and returns
float64 results, unrounded.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "liboracle.so")
SRC_PATH = os.path.join(HERE, "oracle.c")

# -ffp-contract=off: no fused multiply-add, every operation rounds as written.
CFLAGS = ["-O2", "-fopenmp", "-ffp-contract=off", "-fno-fast-math", "-fPIC",
          "-shared", "-std=c99", "-Wall"]


def build(force: bool = True) -> str:
    """Compile oracle.c into liboracle.so with gcc."""
    if force or not os.path.exists(LIB_PATH):
        tmp = LIB_PATH + ".tmp"
        subprocess.check_call(["gcc", *CFLAGS, SRC_PATH, "-o", tmp, "-lm"])
        os.replace(tmp, LIB_PATH)
    return LIB_PATH


_lib = None


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            build()
        L = ctypes.CDLL(LIB_PATH)
        P = ctypes.c_void_p
        i = ctypes.c_int
        f = ctypes.c_float
        L.oracle_attn_fwd_f64.argtypes = [P, P, P, P, P, i, i, i, i, i, f, i]
        L.oracle_attn_fwd_f64_planted.argtypes = [P, P, P, P, P, i, i, i, i, i, f, i, i]
        L.oracle_attn_fwd_kv_f64.argtypes = [P, P, P, P, P, i, i, i, i, i, i, f, i, i]
        L.oracle_attn_bwd_f64.argtypes = [P, P, P, P, P, P, P, i, i, i, i, i, f, i, i]
        L.oracle_logits_f64.argtypes = [P, P, P, i, i, i, i, i, i, i, f, i]
        L.oracle_softmax_av_f64.argtypes = [P, P, P, P, i, i, i, i, i]
        L.oracle_half_to_double.argtypes = [ctypes.c_uint16]
        L.oracle_half_to_double.restype = ctypes.c_double
        for name in ("oracle_attn_fwd_f64", "oracle_attn_fwd_f64_planted", "oracle_attn_fwd_kv_f64",
                     "oracle_attn_bwd_f64",
                     "oracle_logits_f64", "oracle_softmax_av_f64",
                     "oracle_max_threads"):
            getattr(L, name).restype = ctypes.c_int
        _lib = L
    return _lib


def _f16(x: np.ndarray) -> np.ndarray:
    x = np.ascontiguousarray(x)
    if x.dtype != np.float16 or x.ndim != 4:
        raise TypeError("expected a 4-D float16 array [B, H, S, D]")
    return x


def _ptr(a: np.ndarray):
    return a.ctypes.data_as(ctypes.c_void_p)


def max_threads() -> int:
    return lib().oracle_max_threads()


def attn_fwd(q, k, v, causal: bool, scale: float, nthreads: int = 0,
             planted_mistake: int = 0):
    """(O float64 [B,H,S,D], LSE float64 [B,H,S]).  ``scale`` is rounded to
    float32, the value the GPU receives.  ``planted_mistake`` != 0 selects one
    deliberately wrong variant, for the oracle's own power tests."""
    q, k, v = _f16(q), _f16(k), _f16(v)
    if not (q.shape == k.shape == v.shape):
        raise ValueError("q, k, v shapes differ")
    B, H, S, D = q.shape
    o = np.empty((B, H, S, D), dtype=np.float64)
    lse = np.empty((B, H, S), dtype=np.float64)
    sc = float(np.float32(scale))
    if planted_mistake:
        rc = lib().oracle_attn_fwd_f64_planted(
            _ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse), B, H, S, D,
            int(bool(causal)), sc, int(nthreads), int(planted_mistake))
    else:
        rc = lib().oracle_attn_fwd_f64(
            _ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse), B, H, S, D,
            int(bool(causal)), sc, int(nthreads))
    if rc != 0:
        raise RuntimeError(f"oracle_attn_fwd_f64 failed: {rc}")
    return o, lse


def attn_fwd_kv(q, k, v, causal: bool, scale: float, nthreads: int = 0,
                planted_mistake: int = 0):
    """Decode form: q [B,H,Sq,D] against k, v [B,H,Sk,D] -> (O float64
    [B,H,Sq,D], LSE float64 [B,H,Sq]).  Causal uses bottom-right alignment:
    key j visible to query i iff j <= i + Sk - Sq."""
    q, k, v = _f16(q), _f16(k), _f16(v)
    if k.shape != v.shape or q.shape[:2] != k.shape[:2] or q.shape[3] != k.shape[3]:
        raise ValueError("q [B,H,Sq,D] and k, v [B,H,Sk,D] do not match")
    B, H, Sq, D = q.shape
    Sk = k.shape[2]
    o = np.empty((B, H, Sq, D), dtype=np.float64)
    lse = np.empty((B, H, Sq), dtype=np.float64)
    rc = lib().oracle_attn_fwd_kv_f64(
        _ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse), B, H, Sq, Sk, D,
        int(bool(causal)), float(np.float32(scale)), int(nthreads), int(planted_mistake))
    if rc != 0:
        raise RuntimeError(f"oracle_attn_fwd_kv_f64 failed: {rc}")
    return o, lse


def attn_bwd(q, k, v, do, causal: bool, scale: float, nthreads: int = 0,
             planted_mistake: int = 0):
    """Gradients (dQ, dK, dV), float64 [B,H,S,D], of sum(dO * O) for the
    forward softmax(scale Q K^T + mask) V; inputs fp16 [B,H,S,D]."""
    q, k, v, do = _f16(q), _f16(k), _f16(v), _f16(do)
    if not (q.shape == k.shape == v.shape == do.shape):
        raise ValueError("q, k, v, do shapes differ")
    B, H, S, D = q.shape
    dq, dk, dv = (np.empty((B, H, S, D), dtype=np.float64) for _ in range(3))
    rc = lib().oracle_attn_bwd_f64(
        _ptr(q), _ptr(k), _ptr(v), _ptr(do), _ptr(dq), _ptr(dk), _ptr(dv), B, H, S, D,
        int(bool(causal)), float(np.float32(scale)), int(nthreads), int(planted_mistake))
    if rc != 0:
        raise RuntimeError(f"oracle_attn_bwd_f64 failed: {rc}")
    return dq, dk, dv


def logits(q, k, causal: bool, scale: float, d0: int = 0, d1: int | None = None,
           nthreads: int = 0):
    """Scaled logits over head-dim range [d0, d1), float64 [B,H,S,S]; masked
    entries are -inf."""
    q, k = _f16(q), _f16(k)
    B, H, S, D = q.shape
    d1 = D if d1 is None else d1
    out = np.empty((B, H, S, S), dtype=np.float64)
    rc = lib().oracle_logits_f64(_ptr(q), _ptr(k), _ptr(out), B, H, S, D, d0,
                                 d1, int(bool(causal)), float(np.float32(scale)),
                                 int(nthreads))
    if rc != 0:
        raise RuntimeError(f"oracle_logits_f64 failed: {rc}")
    return out


def softmax_av(logit: np.ndarray, v, nthreads: int = 0):
    """Softmax of given float64 logits [B,H,S,S] (-inf = masked) applied to V:
    (O float64 [B,H,S,D], LSE float64 [B,H,S])."""
    v = _f16(v)
    B, H, S, D = v.shape
    logit = np.ascontiguousarray(logit, dtype=np.float64)
    if logit.shape != (B, H, S, S):
        raise ValueError("logits must be [B,H,S,S]")
    o = np.empty((B, H, S, D), dtype=np.float64)
    lse = np.empty((B, H, S), dtype=np.float64)
    rc = lib().oracle_softmax_av_f64(_ptr(logit), _ptr(v), _ptr(o), _ptr(lse),
                                     B, H, S, D, int(nthreads))
    if rc != 0:
        raise RuntimeError(f"oracle_softmax_av_f64 failed: {rc}")
    return o, lse


def half_to_double(bits: int) -> float:
    return lib().oracle_half_to_double(bits)
