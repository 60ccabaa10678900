"""fp64 CPU oracle for the Titans memory scan -- TEST INFRASTRUCTURE ONLY.

Only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may import this package.  The product path
(``sequence_models_amd``) never imports it; the two share no code.

The arithmetic lives in ``titans_oracle.c`` (plain C, double precision, one
token at a time; its header lists the passages of the Titans pages it
follows).  This module only builds it with gcc and marshals numpy arrays.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "titans_oracle.c")
# TITANS_ORACLE_LIB points the loader at another build of the same source (the tests'
# sanitizer build); build() always writes the default path.
_DEFAULT_LIB = os.path.join(_HERE, "libtitans_oracle.so")
_LIB = os.environ.get("TITANS_ORACLE_LIB") or _DEFAULT_LIB
_lib = None


def build(force: bool = True) -> str:
    """Compile the oracle with gcc (-O2, OpenMP over independent sequences)."""
    if force or not os.path.exists(_DEFAULT_LIB):
        tmp = _DEFAULT_LIB + ".tmp"
        subprocess.check_call(
            ["gcc", "-O2", "-std=c11", "-fPIC", "-shared", "-fopenmp", "-Wall",
             "-Wno-unused-variable", _SRC, "-o", tmp, "-lm"])
        os.replace(tmp, _DEFAULT_LIB)
    return _DEFAULT_LIB


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB):
            build()
        lib = ctypes.CDLL(_LIB)
        dp = ctypes.POINTER(ctypes.c_double)
        ip = ctypes.POINTER(ctypes.c_int)
        i64 = ctypes.c_int64
        lib.oracle_param_count.restype = i64
        lib.oracle_param_count.argtypes = [ctypes.c_int, ip]
        lib.oracle_mlp_forward.restype = None
        lib.oracle_mlp_forward.argtypes = [ctypes.c_int, ip, dp, dp, dp]
        lib.oracle_mlp_loss.restype = ctypes.c_double
        lib.oracle_mlp_loss.argtypes = [ctypes.c_int, ip, dp, dp, dp]
        lib.oracle_mlp_grad.restype = ctypes.c_double
        lib.oracle_mlp_grad.argtypes = [ctypes.c_int, ip, dp, dp, dp, dp]
        lib.oracle_scan.restype = ctypes.c_int
        lib.oracle_scan.argtypes = [i64, i64, i64, ctypes.c_int, ip, i64,
                                    dp, dp, dp, dp, dp, dp, dp, dp, i64,
                                    dp, dp, dp, ctypes.c_int]
        lib.oracle_mlp_loss_bias.restype = ctypes.c_double
        lib.oracle_mlp_loss_bias.argtypes = [ctypes.c_int, ip, dp, dp, dp, ctypes.c_int,
                                             ctypes.c_double]
        lib.oracle_mlp_grad_bias.restype = ctypes.c_double
        lib.oracle_mlp_grad_bias.argtypes = [ctypes.c_int, ip, dp, dp, dp, dp, ctypes.c_int,
                                             ctypes.c_double]
        lib.oracle_scan_bias.restype = ctypes.c_int
        lib.oracle_scan_bias.argtypes = [i64, i64, i64, ctypes.c_int, ip, i64,
                                         dp, dp, dp, dp, dp, dp, dp, dp, i64,
                                         dp, dp, dp, ctypes.c_int, ctypes.c_int, ctypes.c_double]
        lib.oracle_scan_full.restype = ctypes.c_int
        lib.oracle_scan_full.argtypes = [i64, i64, i64, ctypes.c_int, ip, i64,
                                         dp, dp, dp, dp, dp, dp, dp, dp, i64,
                                         dp, dp, dp, ctypes.c_int, ctypes.c_int, ctypes.c_double,
                                         ctypes.c_void_p]
        lib.oracle_retrieve.restype = ctypes.c_int
        lib.oracle_retrieve.argtypes = [i64, i64, i64, ctypes.c_int, ip, dp, dp, i64, dp,
                                        ctypes.c_int]
        _lib = lib
    return _lib


def _f64(a):
    return np.ascontiguousarray(a, dtype=np.float64)


def _ptr(a):
    return a.ctypes.data_as(ctypes.POINTER(ctypes.c_double))


def _widths(widths):
    w = (ctypes.c_int * len(widths))(*[int(x) for x in widths])
    return len(widths) - 1, w


def param_count(widths) -> int:
    return int(sum(widths[i] * widths[i - 1] for i in range(1, len(widths))))


def mlp_forward(widths, theta, x):
    lib = _load()
    L, w = _widths(widths)
    theta, x = _f64(theta), _f64(x)
    out = np.empty(widths[-1], dtype=np.float64)
    lib.oracle_mlp_forward(L, w, _ptr(theta), _ptr(x), _ptr(out))
    return out


# Attentional bias: None / ("l2",) = the squared loss; ("huber", delta); ("lp", p).
BIAS_KINDS = {"l2": 0, "huber": 1, "lp": 2}


def _bias(bias):
    if bias is None:
        return 0, 0.0
    kind = BIAS_KINDS[bias[0]]
    return kind, float(bias[1]) if len(bias) > 1 else 0.0


def mlp_loss(widths, theta, k, v, bias=None) -> float:
    """sum_i loss(M_theta(k)_i - v_i); the squared loss unless bias says otherwise."""
    lib = _load()
    L, w = _widths(widths)
    theta, k, v = _f64(theta), _f64(k), _f64(v)
    kind, prm = _bias(bias)
    return float(lib.oracle_mlp_loss_bias(L, w, _ptr(theta), _ptr(k), _ptr(v), kind, prm))


def mlp_grad(widths, theta, k, v, bias=None):
    """(loss, gradient) of sum_i loss(M_theta(k)_i - v_i), gradient in theta's layout."""
    lib = _load()
    L, w = _widths(widths)
    theta, k, v = _f64(theta), _f64(k), _f64(v)
    g = np.empty_like(theta)
    kind, prm = _bias(bias)
    loss = lib.oracle_mlp_grad_bias(L, w, _ptr(theta), _ptr(k), _ptr(v), _ptr(g), kind, prm)
    return float(loss), g


def scan(q, k, v, alpha, eta, beta, theta0, s0, chunk, widths, nthreads: int = 0, bias=None,
         surprise=False):
    """Sequential chunked scan in fp64 (bias: the attentional bias, see BIAS_KINDS; with
    surprise=True a fourth result [B, T, H] holds each token's gradient norm).

    q, k, v: [B, T, H, d]; alpha, eta, beta: [B, T, H];
    theta0, s0: [H, P] (shared over the batch) or [B, H, P].
    Returns (y [B,T,H,d], theta_T [B,H,P], s_T [B,H,P]) as float64.
    """
    lib = _load()
    L, w = _widths(widths)
    q, k, v = _f64(q), _f64(k), _f64(v)
    alpha, eta, beta = _f64(alpha), _f64(eta), _f64(beta)
    B, T, H, d = q.shape
    assert d == widths[0] == widths[-1]
    P = param_count(widths)
    theta0, s0 = _f64(theta0), _f64(s0)
    if theta0.ndim == 2:
        assert theta0.shape == (H, P) and s0.shape == (H, P)
        bstride = 0
    else:
        assert theta0.shape == (B, H, P) and s0.shape == (B, H, P)
        bstride = H * P
    for g in (alpha, eta, beta):
        assert g.shape == (B, T, H)
    y = np.zeros((B, T, H, d), dtype=np.float64)
    thT = np.zeros((B, H, P), dtype=np.float64)
    sT = np.zeros((B, H, P), dtype=np.float64)
    kind, prm = _bias(bias)
    sur = np.zeros((B, T, H), dtype=np.float64) if surprise else None
    rc = lib.oracle_scan_full(B, T, H, L, w, int(chunk), _ptr(q), _ptr(k), _ptr(v),
                              _ptr(alpha), _ptr(eta), _ptr(beta), _ptr(theta0), _ptr(s0),
                              bstride, _ptr(y), _ptr(thT), _ptr(sT), int(nthreads), kind, prm,
                              None if sur is None else sur.ctypes.data)
    if rc != 0:
        raise ValueError(f"oracle_scan rejected its arguments (rc={rc})")
    return (y, thT, sT, sur) if surprise else (y, thT, sT)


def retrieve(q, theta, widths, nthreads: int = 0):
    """y = M_theta(q) per (b, h) with fixed weights: q [B,T,H,d], theta [H,P] or [B,H,P]."""
    lib = _load()
    L, w = _widths(widths)
    q = _f64(q)
    B, T, H, d = q.shape
    P = param_count(widths)
    theta = _f64(theta)
    if theta.ndim == 2:
        assert theta.shape == (H, P)
        bstride = 0
    else:
        assert theta.shape == (B, H, P)
        bstride = H * P
    y = np.zeros_like(q)
    rc = lib.oracle_retrieve(B, T, H, L, w, _ptr(q), _ptr(theta), bstride, _ptr(y), int(nthreads))
    if rc != 0:
        raise ValueError(f"oracle_retrieve rejected its arguments (rc={rc})")
    return y
