"""ctypes wrapper around the CPU oracle (qb_oracle.cpp).

TEST INFRASTRUCTURE ONLY: imported by the test suite, the smoke check and the
benchmark's CPU-baseline leg.  The GPU library never imports or links it.

``build()`` compiles ``qb_oracle.cpp`` with g++ (single-threaded, no
fast-math, no FMA contraction) into ``oracle/_build/liboracle.so``.
"""
from __future__ import annotations

import ctypes as C
import os
import subprocess

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "qb_oracle.cpp")
LIB = os.path.join(HERE, "_build", "liboracle.so")

_lib = None

f32p = np.ctypeslib.ndpointer(np.float32, flags="C_CONTIGUOUS")
f64p = np.ctypeslib.ndpointer(np.float64, flags="C_CONTIGUOUS")
i32p = np.ctypeslib.ndpointer(np.int32, flags="C_CONTIGUOUS")
i64p = np.ctypeslib.ndpointer(np.int64, flags="C_CONTIGUOUS")
u16p = np.ctypeslib.ndpointer(np.uint16, flags="C_CONTIGUOUS")


def build(verbose: bool = False) -> str:
    os.makedirs(os.path.dirname(LIB), exist_ok=True)
    tmp = LIB + ".tmp"
    cmd = ["g++", "-O2", "-std=c++17", "-ffp-contract=off", "-fno-fast-math", "-fPIC",
           "-shared", "-o", tmp, SRC]
    if verbose:
        print(" ".join(cmd))
    subprocess.check_call(cmd)
    os.replace(tmp, LIB)
    return LIB


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(LIB):
            raise RuntimeError(f"oracle library {LIB} is not built; run oracle.oracle.build()")
        L = C.CDLL(LIB)
        L.oq_bf16_rne.restype = C.c_uint16
        L.oq_bf16_rne.argtypes = [C.c_float]
        L.oq_bf16_value.restype = C.c_float
        L.oq_bf16_value.argtypes = [C.c_uint16]
        L.oq_key.restype = C.c_uint16
        L.oq_key.argtypes = [C.c_uint16]
        L.oq_unkey.restype = C.c_uint16
        L.oq_unkey.argtypes = [C.c_uint16]
        L.oq_bf16_rne_array.restype = None
        L.oq_bf16_rne_array.argtypes = [f32p, u16p, C.c_int64]
        L.oq_alpha.restype = None
        L.oq_alpha.argtypes = [f32p, f32p, C.c_int64, C.c_int, C.c_int, f32p, C.c_void_p]
        L.oq_margin_keys.restype = None
        L.oq_margin_keys.argtypes = [f32p, f32p, C.c_int64, C.c_int, u16p]
        L.oq_eqb_layer.restype = C.c_int
        L.oq_eqb_layer.argtypes = [f32p, f32p, C.c_int64, C.c_int, C.c_int, f32p, C.c_void_p,
                                   i32p, i32p, i32p, i32p, u16p, f32p, f32p, f32p]
        L.oq_k3_bin.restype = C.c_int
        L.oq_k3_bin.argtypes = [C.c_float, C.c_float, C.c_float, C.c_int]
        L.oq_k3_layer.restype = C.c_int
        L.oq_k3_layer.argtypes = [f32p, f32p, C.c_int64, C.c_int, C.c_int, f32p, C.c_int, f32p,
                                  i32p, f32p, f32p, f32p]
        L.oq_bounds_of.restype = None
        L.oq_bounds_of.argtypes = [f32p, C.c_int, f32p]
        L.oq_lei.restype = None
        L.oq_lei.argtypes = [f32p, i32p, C.c_int64, C.c_int, C.c_int, C.c_float]
        L.oq_lei_bwd.restype = None
        L.oq_lei_bwd.argtypes = [f32p, C.c_void_p, i32p, C.c_int64, C.c_int, C.c_int, C.c_int64, C.c_float,
                                 C.c_int, C.c_void_p, C.c_void_p]
        L.oq_rank_average.restype = None
        L.oq_rank_average.argtypes = [f32p, C.c_int, C.c_int, f32p, f32p]
        L.oq_maxvio.restype = None
        L.oq_maxvio.argtypes = [i32p, C.c_int, C.c_int, C.c_int, C.c_int, C.c_int64, f32p,
                                C.c_void_p, C.c_void_p]
        L.oq_router_logits.restype = None
        L.oq_router_logits.argtypes = [u16p, u16p, C.c_int, C.c_int, i64p, C.c_int, f64p]
        _lib = L
    return _lib


def _f32(a):
    return np.ascontiguousarray(a, dtype=np.float32)


def bf16_rne(x) -> np.ndarray:
    x = _f32(np.asarray(x)).ravel()
    out = np.empty(x.shape, np.uint16)
    lib().oq_bf16_rne_array(x, out, x.size)
    return out


def bf16_value(u: int) -> float:
    return lib().oq_bf16_value(int(u))


def key(u: int) -> int:
    return lib().oq_key(int(u))


def unkey(k: int) -> int:
    return lib().oq_unkey(int(k))


def alpha(s, b, K: int, with_load: bool = True):
    s = _f32(s)
    b = _f32(b)
    N, E = s.shape
    a = np.empty(N, np.float32)
    load = np.zeros(E, np.int32)
    lib().oq_alpha(s, b, N, E, K, a, load.ctypes.data if with_load else None)
    return (a, load) if with_load else a


def margin_keys(s, alpha_):
    """Keys of the bf16 margins, expert-major [E, N]."""
    s = _f32(s)
    N, E = s.shape
    out = np.empty((E, N), np.uint16)
    lib().oq_margin_keys(s, _f32(alpha_), N, E, out)
    return out


def eqb_layer(s, b, K: int) -> dict:
    s = _f32(s)
    b = _f32(b)
    N, E = s.shape
    r = dict(alpha=np.empty(N, np.float32), load=np.zeros(E, np.int32),
             hist_hi=np.zeros((E, 256), np.int32), sel_hi=np.zeros(E, np.int32),
             rank_lo=np.zeros(E, np.int32), hist_lo=np.zeros((E, 256), np.int32),
             key=np.zeros(E, np.uint16), q=np.zeros(E, np.float32),
             b_next=np.zeros(E, np.float32), bounds=np.zeros(2, np.float32))
    rc = lib().oq_eqb_layer(s, b, N, E, K, r["alpha"], r["load"].ctypes.data, r["hist_hi"],
                            r["sel_hi"], r["rank_lo"], r["hist_lo"], r["key"], r["q"],
                            r["b_next"], r["bounds"])
    assert rc == 0
    return r


def bounds_of(b) -> np.ndarray:
    b = _f32(b)
    out = np.zeros(2, np.float32)
    lib().oq_bounds_of(b, b.size, out)
    return out


def k3_bin(r: float, lo: float, hi: float, n_bins: int) -> int:
    return lib().oq_k3_bin(float(r), float(lo), float(hi), int(n_bins))


def k3_layer(s, b, K: int, bounds, n_bins: int = 1000) -> dict:
    s = _f32(s)
    b = _f32(b)
    N, E = s.shape
    r = dict(alpha=np.empty(N, np.float32), hist_u=np.zeros((E, n_bins), np.int32),
             q=np.zeros(E, np.float32), b_next=np.zeros(E, np.float32),
             bounds=np.zeros(2, np.float32))
    rc = lib().oq_k3_layer(s, b, N, E, K, _f32(bounds), n_bins, r["alpha"], r["hist_u"], r["q"],
                           r["b_next"], r["bounds"])
    if rc != 0:
        raise ValueError("K3 histogram never reaches rank m")
    return r


def lei(g, load, K: int, eta) -> np.ndarray:
    g = np.array(g, dtype=np.float32, copy=True, order="C")
    N, E = g.shape
    lib().oq_lei(g, np.ascontiguousarray(load, dtype=np.int32), N, E, K, np.float32(eta))
    return g


def router_logits(hidden_bits, w_bits, rows) -> np.ndarray:
    """logits of the selected rows, float64; w_bits is [E, H]."""
    hidden_bits = np.ascontiguousarray(hidden_bits, dtype=np.uint16)
    w_bits = np.ascontiguousarray(w_bits, dtype=np.uint16)
    rows = np.ascontiguousarray(rows, dtype=np.int64)
    E, H = w_bits.shape
    out = np.zeros((rows.size, E), np.float64)
    lib().oq_router_logits(hidden_bits, w_bits, H, E, rows, rows.size, out)
    return out


def microbatch_loads(s, b, K: int, n_mb: int) -> np.ndarray:
    """Top-K loads of each consecutive n_mb-token microbatch, [C, E]: the
    oracle's top-K selection run on each chunk of rows."""
    s = _f32(s)
    N, E = s.shape
    assert N % n_mb == 0
    out = np.zeros((N // n_mb, E), np.int32)
    for c in range(N // n_mb):
        _, out[c] = alpha(s[c * n_mb:(c + 1) * n_mb], b, K)
    return out


def maxvio(load, K: int, n_tok: int):
    """load [L, C, E] -> (v [L, C], summary [L, 2], worst [2])."""
    load = np.ascontiguousarray(load, dtype=np.int32)
    L, C, E = load.shape
    v = np.zeros((L, C), np.float32)
    summary = np.zeros((L, 2), np.float32)
    worst = np.zeros(2, np.float32)
    lib().oq_maxvio(load, L, C, E, K, n_tok, v, summary.ctypes.data, worst.ctypes.data)
    return v, summary, worst


def rank_average(q) -> tuple:
    """q [R, E] rank-local quantiles -> (b [E], bounds [2]) of the
    rank-averaged update."""
    q = _f32(q)
    R, E = q.shape
    b = np.zeros(E, np.float32)
    bounds = np.zeros(2, np.float32)
    lib().oq_rank_average(q, R, E, b, bounds)
    return b, bounds


def rank_local_quantiles(s, b, K: int, R: int) -> np.ndarray:
    """The EQB quantile of each of R consecutive token shards, [R, E]: what
    each data-parallel rank would find from its own tokens alone."""
    s = _f32(s)
    N, E = s.shape
    assert N % R == 0
    n = N // R
    return np.stack([eqb_layer(s[r * n:(r + 1) * n], b, K)["q"] for r in range(R)])


def full_hist(s, b, K: int) -> np.ndarray:
    """Full 16-bit key histogram [E, 65536] of the bf16 margin keys (the
    one-pass alternative of the EQB paragraph): counts of the oracle's keys."""
    s = _f32(s)
    N, E = s.shape
    keys = margin_keys(s, alpha(s, b, K, with_load=False))
    return np.stack([np.bincount(keys[j], minlength=65536).astype(np.int32) for j in range(E)])


def lei_backward(g, load_mb, K: int, n_mb: int, eta, bounded: bool = False, s=None):
    """-> (g' [N, E], dlogits [N, E] or None)."""
    g = _f32(g)
    N, E = g.shape
    load_mb = np.ascontiguousarray(load_mb, dtype=np.int32)
    gout = np.zeros_like(g)
    d = np.zeros_like(g) if s is not None else None
    sp = _f32(s) if s is not None else None
    lib().oq_lei_bwd(g, sp.ctypes.data if sp is not None else None, load_mb, N, E, K, n_mb,
                     np.float32(eta), int(bool(bounded)), gout.ctypes.data,
                     d.ctypes.data if d is not None else None)
    return gout, d
