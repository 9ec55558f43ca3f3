"""Thin Python binding of libqb's C ABI (include/qb.h), same names.

Argument marshalling only: every function checks dtype / device / layout /
shape of torch tensors, passes raw device pointers and the current HIP
stream, and raises ``QBError`` on a non-zero status.  All arithmetic runs in
the HIP kernels of libqb.so; there is no CPU fallback -- a missing library
is an error.

Tensors may carry a leading layer dimension (s [L, N, E], b [L, E],
alpha [L, N], ...) or omit it for one layer.
"""
from __future__ import annotations

import ctypes as C
import os

import torch

PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(PKG, "libqb.so")

QB_OK, QB_EINVAL, QB_EUNSUPPORTED, QB_EHIP = 0, -1, -2, -3
QB_SELECT_HI, QB_SELECT_LO, QB_SELECT_UNIFORM, QB_SELECT_FULL = 0, 1, 2, 3
QB_ERR_ROW_TOTALS, QB_ERR_EMPTY, QB_ERR_RANK = 1, 2, 4
QB_NOALLOC_SCRATCH_BYTES = 64 << 20

SUPPORTED_E = (16, 32, 64, 128, 256)
MAX_K = 15

_lib = None


class QBError(RuntimeError):
    def __init__(self, status: int, msg: str):
        super().__init__(msg)
        self.status = status


def lib() -> C.CDLL:
    """Load libqb.so once.  torch is imported first so that libqb binds to
    the HIP runtime torch already mapped (one runtime per process)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is not built: run __graft_entry__.build() "
                               "(or python exact_quantile_selection_amd/build.py)")
        L = C.CDLL(LIB_PATH)
        vp, i32, i64, f32 = C.c_void_p, C.c_int, C.c_int64, C.c_float
        sig = {
            "qb_margins_topk": [vp, vp, i32, i64, i32, i32, vp, vp, vp, vp],
            "qb_radix_hist_hi": [vp, vp, i32, i64, i32, vp, vp],
            "qb_radix_hist_lo": [vp, vp, i32, i64, i32, vp, vp, vp],
            "qb_margin_keys": [vp, vp, i32, i64, i32, vp, vp],
            "qb_select_update": [i32, i32, i32, i32, vp, i32, vp, vp, vp, vp, vp, vp, vp, vp],
            "qb_uniform_hist": [vp, vp, i32, i64, i32, vp, i32, vp, vp],
            "qb_uniform_hist_ws": [vp, vp, i32, i64, i32, vp, i32, vp, i64, vp],
            "qb_select_uniform_ws": [i32, i64, i32, i32, i32, vp, i64, vp, vp, vp, vp, vp, vp],
            "qb_bias_bounds": [vp, i32, i32, vp, vp],
            "qb_fill_i32": [vp, i64, C.c_int32, vp],
            "qb_lei_grad": [vp, vp, i64, i32, i32, f32, vp],
            "qb_router_fused": [vp, vp, i64, i32, i32, i32, vp, vp, vp, vp, vp, vp, vp],
            "qb_router_scores": [vp, vp, i64, i32, i32, vp, vp, vp],
            "qb_microbatch_loads": [vp, vp, i32, i64, i32, i32, i64, vp, vp, vp],
            "qb_margins_topk_mb": [vp, vp, i32, i64, i32, i32, vp, vp, vp, i64, vp, vp],
            "qb_maxvio": [vp, i32, i32, i32, i32, i64, vp, vp, vp, vp],
            "qb_allreduce_sum_i32": [vp, i32, i64, vp],
            "qb_margins_full_hist": [vp, vp, i32, i64, i32, i32, vp, vp, vp],
            "qb_lei_backward": [vp, vp, vp, i64, i32, i32, i64, f32, i32, vp, vp, vp],
            "qb_radix_hist_lo_ws": [vp, vp, i32, i64, i32, vp, vp, i64, vp],
            "qb_radix_hist_lo_ws_loads": [vp, vp, i32, i64, i32, vp, vp, i64, vp, i32, vp, i64, vp, vp],
            "qb_select_lo_ws": [i32, i64, i32, vp, i64, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp],
            "qb_rank_average": [vp, i32, i32, vp, vp, vp],
            "qb_radix_lo_trip_rows": [i32],
            "qb_radix_lo_select_noalloc": [vp, vp, i32, i64, i32, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp],
        }
        for name, args in sig.items():
            fn = getattr(L, name)
            fn.argtypes = args
            fn.restype = C.c_int
        L.qb_hist_lo_workspace_bytes.argtypes = [i32, i64, i32]
        L.qb_hist_lo_workspace_bytes.restype = C.c_int64
        L.qb_uniform_hist_workspace_bytes.argtypes = [i32, i64, i32, i32]
        L.qb_uniform_hist_workspace_bytes.restype = C.c_int64
        L.qb_status_string.argtypes = [C.c_int]
        L.qb_status_string.restype = C.c_char_p
        L.qb_last_error.argtypes = []
        L.qb_last_error.restype = C.c_char_p
        _lib = L
    return _lib


def _check(rc: int):
    if rc != QB_OK:
        L = lib()
        raise QBError(rc, f"{L.qb_status_string(rc).decode()}: {L.qb_last_error().decode()}")


def _stream(stream) -> int:
    if stream is None:
        stream = torch.cuda.current_stream()
    return int(stream.cuda_stream)


def _ptr(t, dtype, name, shape=None, opt=False):
    if t is None:
        if opt:
            return None
        raise ValueError(f"{name} is required")
    if not isinstance(t, torch.Tensor) or t.device.type != "cuda":
        raise ValueError(f"{name} must be a GPU tensor")
    if t.dtype != dtype:
        raise ValueError(f"{name} must be {dtype}, got {t.dtype}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {tuple(shape)}")
    return t.data_ptr()


def _lne(s):
    if s.dim() == 2:
        return 1, s.shape[0], s.shape[1], ()
    if s.dim() == 3:
        return s.shape[0], s.shape[1], s.shape[2], (s.shape[0],)
    raise ValueError(f"s must be [N, E] or [L, N, E], got {tuple(s.shape)}")


def qb_margins_topk(s, b, K, alpha, load=None, hist_hi=None, stream=None):
    L, N, E, lead = _lne(s)
    rc = lib().qb_margins_topk(
        _ptr(s, torch.float32, "s"), _ptr(b, torch.float32, "b", lead + (E,)), L, N, E, K,
        _ptr(alpha, torch.float32, "alpha", lead + (N,)),
        _ptr(load, torch.int32, "load", lead + (E,), opt=True),
        _ptr(hist_hi, torch.int32, "hist_hi", lead + (E, 256), opt=True), _stream(stream))
    _check(rc)


def _ws(ws):
    if not isinstance(ws, torch.Tensor) or ws.dtype != torch.uint8 or not ws.is_contiguous() \
            or ws.device.type != "cuda":
        raise ValueError("ws must be a contiguous uint8 GPU tensor")
    return ws.data_ptr(), ws.numel()


def qb_radix_hist_hi(s, alpha, hist_hi, stream=None):
    L, N, E, lead = _lne(s)
    _check(lib().qb_radix_hist_hi(
        _ptr(s, torch.float32, "s"), _ptr(alpha, torch.float32, "alpha", lead + (N,)), L, N, E,
        _ptr(hist_hi, torch.int32, "hist_hi", lead + (E, 256)), _stream(stream)))


def qb_radix_hist_lo(s, alpha, sel_hi, hist_lo, stream=None):
    L, N, E, lead = _lne(s)
    _check(lib().qb_radix_hist_lo(
        _ptr(s, torch.float32, "s"), _ptr(alpha, torch.float32, "alpha", lead + (N,)), L, N, E,
        _ptr(sel_hi, torch.int32, "sel_hi", lead + (E,)),
        _ptr(hist_lo, torch.int32, "hist_lo", lead + (E, 256)), _stream(stream)))


def qb_margin_keys(s, alpha, keys, stream=None):
    L, N, E, lead = _lne(s)
    _check(lib().qb_margin_keys(
        _ptr(s, torch.float32, "s"), _ptr(alpha, torch.float32, "alpha", lead + (N,)), L, N, E,
        _ptr(keys, torch.uint16, "keys", lead + (N, E)), _stream(stream)))


def qb_select_update(phase, K, hist, sel_hi=None, rank_lo=None, key_out=None, q_out=None, b=None,
                     bounds=None, err=None, stream=None):
    if hist.dim() == 2:
        L, lead = 1, ()
    elif hist.dim() == 3:
        L, lead = hist.shape[0], (hist.shape[0],)
    else:
        raise ValueError("hist must be [E, bins] or [L, E, bins]")
    E, n_bins = hist.shape[-2], hist.shape[-1]
    _check(lib().qb_select_update(
        phase, L, E, K, _ptr(hist, torch.int32, "hist"), n_bins,
        _ptr(sel_hi, torch.int32, "sel_hi", lead + (E,), opt=True),
        _ptr(rank_lo, torch.int32, "rank_lo", lead + (E,), opt=True),
        _ptr(key_out, torch.uint16, "key_out", lead + (E,), opt=True),
        _ptr(q_out, torch.float32, "q_out", lead + (E,), opt=True),
        _ptr(b, torch.float32, "b", lead + (E,), opt=True),
        _ptr(bounds, torch.float32, "bounds", lead + (2,), opt=True),
        _ptr(err, torch.int32, "err", (1,), opt=True), _stream(stream)))


def qb_uniform_hist(s, alpha, bounds, hist_u, stream=None):
    L, N, E, lead = _lne(s)
    n_bins = hist_u.shape[-1]
    _check(lib().qb_uniform_hist(
        _ptr(s, torch.float32, "s"), _ptr(alpha, torch.float32, "alpha", lead + (N,)), L, N, E,
        _ptr(bounds, torch.float32, "bounds", lead + (2,)), n_bins,
        _ptr(hist_u, torch.int32, "hist_u", lead + (E, n_bins)), _stream(stream)))


def qb_uniform_hist_workspace_bytes(L, N, E, n_bins):
    n = lib().qb_uniform_hist_workspace_bytes(L, N, E, n_bins)
    if n < 0:
        _check(int(n))
    return int(n)


def qb_uniform_hist_ws(s, alpha, bounds, ws, n_bins, stream=None):
    """K3 binning into per-workgroup partial rows in ws (uint8 tensor of at
    least qb_uniform_hist_workspace_bytes bytes)."""
    L, N, E, lead = _lne(s)
    if ws.dtype != torch.uint8 or not ws.is_contiguous() or ws.device.type != "cuda":
        raise ValueError("ws must be a contiguous uint8 GPU tensor")
    _check(lib().qb_uniform_hist_ws(
        _ptr(s, torch.float32, "s"), _ptr(alpha, torch.float32, "alpha", lead + (N,)), L, N, E,
        _ptr(bounds, torch.float32, "bounds", lead + (2,)), n_bins, ws.data_ptr(), ws.numel(), _stream(stream)))


def qb_select_uniform_ws(N, K, n_bins, ws, q_out, b, bounds, hist_u=None, err=None, stream=None):
    """K3 select from the partial rows of qb_uniform_hist_ws, with the
    in-place bias / bounds update; hist_u (optional) receives the summed
    histogram."""
    if b.dim() == 1:
        L, E, lead = 1, b.shape[0], ()
    else:
        L, E = b.shape
        lead = (L,)
    p, n = _ws(ws)
    _check(lib().qb_select_uniform_ws(
        L, N, E, K, n_bins, p, n, _ptr(hist_u, torch.int32, "hist_u", lead + (E, n_bins), opt=True),
        _ptr(q_out, torch.float32, "q_out", lead + (E,)), _ptr(b, torch.float32, "b", lead + (E,)),
        _ptr(bounds, torch.float32, "bounds", lead + (2,)), _ptr(err, torch.int32, "err", (1,), opt=True),
        _stream(stream)))


def qb_bias_bounds(b, bounds, stream=None):
    L, E = (1, b.shape[0]) if b.dim() == 1 else (b.shape[0], b.shape[1])
    lead = () if b.dim() == 1 else (L,)
    _check(lib().qb_bias_bounds(_ptr(b, torch.float32, "b"), L, E,
                                _ptr(bounds, torch.float32, "bounds", lead + (2,)), _stream(stream)))


def qb_fill_i32(t, value=0, stream=None):
    _check(lib().qb_fill_i32(_ptr(t, torch.int32, "t"), t.numel(), int(value), _stream(stream)))


def qb_router_fused(hidden, w, b, K, s_out, alpha, logits_out=None, load=None, hist_hi=None,
                    stream=None):
    """hidden: bf16 [N, H]; w: bf16 [E, H] (nn.Linear layout).  Writes s_out
    = sigmoid(hidden @ w.T); the same kernel's epilogue computes alpha, the
    top-K loads and the high-byte histogram (pass 1) of those scores."""
    N, H = hidden.shape
    E = w.shape[0]
    _check(lib().qb_router_fused(
        _ptr(hidden, torch.bfloat16, "hidden"), _ptr(w, torch.bfloat16, "w", (E, H)), N, H, E, K,
        _ptr(b, torch.float32, "b", (E,)), _ptr(s_out, torch.float32, "s_out", (N, E)),
        _ptr(logits_out, torch.float32, "logits_out", (N, E), opt=True),
        _ptr(alpha, torch.float32, "alpha", (N,)),
        _ptr(load, torch.int32, "load", (E,), opt=True),
        _ptr(hist_hi, torch.int32, "hist_hi", (E, 256), opt=True), _stream(stream)))


def qb_router_scores(hidden, w, s_out, logits_out=None, stream=None):
    """The router GEMM + sigmoid alone: s_out = sigmoid(hidden @ w.T)."""
    N, H = hidden.shape
    E = w.shape[0]
    _check(lib().qb_router_scores(
        _ptr(hidden, torch.bfloat16, "hidden"), _ptr(w, torch.bfloat16, "w", (E, H)), N, H, E,
        _ptr(s_out, torch.float32, "s_out", (N, E)),
        _ptr(logits_out, torch.float32, "logits_out", (N, E), opt=True), _stream(stream)))


def qb_lei_grad(g, load, K, eta, stream=None):
    N, E = g.shape
    _check(lib().qb_lei_grad(_ptr(g, torch.float32, "g"), _ptr(load, torch.int32, "load", (E,)),
                             N, E, K, float(eta), _stream(stream)))


def qb_microbatch_loads(s, b, K, n_mb, alpha, load_mb, stream=None):
    """load_mb [C, E] (or [L, C, E]) += top-K loads of each n_mb-token microbatch."""
    L, N, E, lead = _lne(s)
    if n_mb < 1 or N % n_mb:
        raise ValueError(f"n_mb={n_mb} must divide N={N}")
    _check(lib().qb_microbatch_loads(
        _ptr(s, torch.float32, "s"), _ptr(b, torch.float32, "b", lead + (E,)), L, N, E, K, n_mb,
        _ptr(alpha, torch.float32, "alpha", lead + (N,)),
        _ptr(load_mb, torch.int32, "load_mb", lead + (N // n_mb, E)), _stream(stream)))


def qb_margins_topk_mb(s, b, K, alpha, load, n_mb, load_mb, hist_hi=None, stream=None):
    """Pass 1 with global loads, per-microbatch loads and (optionally) hist_hi."""
    L, N, E, lead = _lne(s)
    if n_mb < 1 or N % n_mb:
        raise ValueError(f"n_mb={n_mb} must divide N={N}")
    _check(lib().qb_margins_topk_mb(
        _ptr(s, torch.float32, "s"), _ptr(b, torch.float32, "b", lead + (E,)), L, N, E, K,
        _ptr(alpha, torch.float32, "alpha", lead + (N,)), _ptr(load, torch.int32, "load", lead + (E,)),
        _ptr(hist_hi, torch.int32, "hist_hi", lead + (E, 256), opt=True), n_mb,
        _ptr(load_mb, torch.int32, "load_mb", lead + (N // n_mb, E)), _stream(stream)))


def qb_maxvio(load, K, n_tok, maxvio, summary=None, worst=None, stream=None):
    """load int32 [L, C, E] -> maxvio [L, C]; optional summary [L, 2], worst [2]."""
    if load.dim() != 3:
        raise ValueError(f"load must be [L, C, E], got {tuple(load.shape)}")
    L, Cm, E = load.shape
    _check(lib().qb_maxvio(
        _ptr(load, torch.int32, "load"), L, Cm, E, K, n_tok, _ptr(maxvio, torch.float32, "maxvio", (L, Cm)),
        _ptr(summary, torch.float32, "summary", (L, 2), opt=True),
        _ptr(worst, torch.float32, "worst", (2,), opt=True), _stream(stream)))


def qb_margins_full_hist(s, b, K, alpha, hist_full, stream=None):
    """alpha, and hist_full [E, 65536] (or [L, E, 65536]) += full 16-bit key histogram."""
    L, N, E, lead = _lne(s)
    _check(lib().qb_margins_full_hist(
        _ptr(s, torch.float32, "s"), _ptr(b, torch.float32, "b", lead + (E,)), L, N, E, K,
        _ptr(alpha, torch.float32, "alpha", lead + (N,)),
        _ptr(hist_full, torch.int32, "hist_full", lead + (E, 65536)), _stream(stream)))


def qb_lei_backward(g, load_mb, K, n_mb, eta, bounded=False, s=None, g_out=None, dlogits=None,
                    stream=None):
    """Per-microbatch LEI on the score gradient g [N, E] (optionally bounded),
    written to g_out (may be g) and/or the logit gradient dlogits."""
    N, E = g.shape
    if n_mb < 1 or N % n_mb:
        raise ValueError(f"n_mb={n_mb} must divide N={N}")
    _check(lib().qb_lei_backward(
        _ptr(g, torch.float32, "g"), _ptr(s, torch.float32, "s", (N, E), opt=True),
        _ptr(load_mb, torch.int32, "load_mb", (N // n_mb, E)), N, E, K, n_mb, float(eta), int(bool(bounded)),
        _ptr(g_out, torch.float32, "g_out", (N, E), opt=True),
        _ptr(dlogits, torch.float32, "dlogits", (N, E), opt=True), _stream(stream)))


def qb_hist_lo_workspace_bytes(L, N, E):
    n = lib().qb_hist_lo_workspace_bytes(L, N, E)
    if n < 0:
        _check(int(n))
    return int(n)


def qb_radix_hist_lo_ws(s, alpha, sel_hi, ws, stream=None):
    """Pass 2 into per-workgroup partial histograms in ws (uint8 tensor of
    at least qb_hist_lo_workspace_bytes bytes)."""
    L, N, E, lead = _lne(s)
    if ws.dtype != torch.uint8 or not ws.is_contiguous() or ws.device.type != "cuda":
        raise ValueError("ws must be a contiguous uint8 GPU tensor")
    _check(lib().qb_radix_hist_lo_ws(
        _ptr(s, torch.float32, "s"), _ptr(alpha, torch.float32, "alpha", lead + (N,)), L, N, E,
        _ptr(sel_hi, torch.int32, "sel_hi", lead + (E,)), ws.data_ptr(), ws.numel(), _stream(stream)))


def qb_radix_hist_lo_ws_loads(s, alpha, sel_hi, ws, b, K, load, n_mb=None, load_mb=None, stream=None):
    """qb_radix_hist_lo_ws that also adds the top-K loads of s + b (alpha from
    pass 1 with the same b and K) into load [E] (or [L, E]) and, with
    load_mb [N // n_mb, E] (or [L, N // n_mb, E]), the per-microbatch loads;
    n_mb must divide N and be a multiple of the pass's row trip (2048 always
    is)."""
    L, N, E, lead = _lne(s)
    if ws.dtype != torch.uint8 or not ws.is_contiguous() or ws.device.type != "cuda":
        raise ValueError("ws must be a contiguous uint8 GPU tensor")
    if load_mb is not None and (n_mb is None or n_mb < 1 or N % n_mb):
        raise ValueError(f"n_mb={n_mb} must divide N={N}")
    C = N // n_mb if load_mb is not None else 0
    _check(lib().qb_radix_hist_lo_ws_loads(
        _ptr(s, torch.float32, "s"), _ptr(alpha, torch.float32, "alpha", lead + (N,)), L, N, E,
        _ptr(sel_hi, torch.int32, "sel_hi", lead + (E,)), ws.data_ptr(), ws.numel(),
        _ptr(b, torch.float32, "b", lead + (E,)), K, _ptr(load, torch.int32, "load", lead + (E,)),
        int(n_mb or 1), _ptr(load_mb, torch.int32, "load_mb", lead + (C, E), opt=True), _stream(stream)))


def qb_radix_lo_trip_rows(E):
    """Rows of one trip of the low-byte pass: per-microbatch loads counted
    there need microbatches that are a multiple of it."""
    n = lib().qb_radix_lo_trip_rows(E)
    if n < 0:
        _check(n)
    return n


def qb_select_lo_ws(N, ws, sel_hi, rank_lo, q_out, b, bounds, hist_lo=None, key_out=None, err=None,
                    hist_hi=None, stream=None):
    """Low-byte select from the workspace of qb_radix_hist_lo_ws, with the
    in-place bias / bounds update; hist_hi (optional) is zeroed in place."""
    if sel_hi.dim() == 1:
        L, E, lead = 1, sel_hi.shape[0], ()
    else:
        L, E = sel_hi.shape
        lead = (L,)
    p, n = _ws(ws)
    _check(lib().qb_select_lo_ws(
        L, N, E, p, n, _ptr(sel_hi, torch.int32, "sel_hi", lead + (E,)),
        _ptr(rank_lo, torch.int32, "rank_lo", lead + (E,)),
        _ptr(hist_lo, torch.int32, "hist_lo", lead + (E, 256), opt=True),
        _ptr(key_out, torch.uint16, "key_out", lead + (E,), opt=True),
        _ptr(q_out, torch.float32, "q_out", lead + (E,)), _ptr(b, torch.float32, "b", lead + (E,)),
        _ptr(bounds, torch.float32, "bounds", lead + (2,)),
        _ptr(hist_hi, torch.int32, "hist_hi", lead + (E, 256), opt=True),
        _ptr(err, torch.int32, "err", (1,), opt=True), _stream(stream)))


def qb_radix_lo_select_noalloc(s, alpha, sel_hi, rank_lo, q_out, b, bounds, hist_lo=None, key_out=None,
                               err=None, hist_hi=None, stream=None):
    """qb_radix_hist_lo_ws + qb_select_lo_ws on the library's own device
    scratch (QB_NOALLOC_SCRATCH_BYTES per GPU): nothing is allocated.  Calls
    that overlap on one GPU race."""
    L, N, E, lead = _lne(s)
    _check(lib().qb_radix_lo_select_noalloc(
        _ptr(s, torch.float32, "s"), _ptr(alpha, torch.float32, "alpha", lead + (N,)), L, N, E,
        _ptr(sel_hi, torch.int32, "sel_hi", lead + (E,)), _ptr(rank_lo, torch.int32, "rank_lo", lead + (E,)),
        _ptr(hist_lo, torch.int32, "hist_lo", lead + (E, 256), opt=True),
        _ptr(key_out, torch.uint16, "key_out", lead + (E,), opt=True),
        _ptr(q_out, torch.float32, "q_out", lead + (E,)), _ptr(b, torch.float32, "b", lead + (E,)),
        _ptr(bounds, torch.float32, "bounds", lead + (2,)),
        _ptr(hist_hi, torch.int32, "hist_hi", lead + (E, 256), opt=True),
        _ptr(err, torch.int32, "err", (1,), opt=True), _stream(stream)))


def qb_allreduce_sum_i32(buf, stream=None):
    """buf int32 [R, ...]: every rank's copy (leading index) becomes the sum
    of all copies, in place."""
    R = buf.shape[0]
    _check(lib().qb_allreduce_sum_i32(_ptr(buf, torch.int32, "buf"), R, buf.numel() // R, _stream(stream)))


def qb_rank_average(q, b, bounds=None, stream=None):
    """q float [R, E] rank-local quantiles -> b [E] (and bounds [2])."""
    R, E = q.shape
    _check(lib().qb_rank_average(_ptr(q, torch.float32, "q"), R, E, _ptr(b, torch.float32, "b", (E,)),
                                 _ptr(bounds, torch.float32, "bounds", (2,), opt=True), _stream(stream)))


# ---------------------------------------------------------------------------
# Composition of the calls above for one global batch (no arithmetic here).

class EqbBuffers:
    """Device buffers of one EQB update over L layers of E experts.

    The two histograms and the error word share one int32 block so that the
    in-place reset is a single fill launch."""

    def __init__(self, L: int, E: int, device="cuda", lead: bool = True):
        shp = (L,) if lead else ()
        kw = dict(device=device)
        nh = L * E * 256
        self.block = torch.zeros(2 * nh + 4, dtype=torch.int32, **kw)
        self.hist_hi = self.block[:nh].view(shp + (E, 256))
        self.hist_lo = self.block[nh:2 * nh].view(shp + (E, 256))
        self.err = self.block[2 * nh:2 * nh + 1]
        self.sel_hi = torch.zeros(shp + (E,), dtype=torch.int32, **kw)
        self.rank_lo = torch.zeros(shp + (E,), dtype=torch.int32, **kw)
        self.key = torch.zeros(shp + (E,), dtype=torch.uint16, **kw)
        self.q = torch.zeros(shp + (E,), dtype=torch.float32, **kw)
        self.bounds = torch.zeros(shp + (2,), dtype=torch.float32, **kw)

    def reset(self, stream=None):
        """In-place reset of both histograms and the error word (addresses
        unchanged), one fill kernel."""
        qb_fill_i32(self.block, 0, stream)


def eqb_update(s, b, K, alpha, buf: EqbBuffers, load=None, stream=None):
    """One exact quantile-balancing update: pass 1 (alpha + high-byte
    histogram), high-byte select, pass 2 (low-byte histogram), low-byte select
    and the in-place bias update.  Histograms must be zero on entry
    (buf.reset() clears them in place)."""
    qb_margins_topk(s, b, K, alpha, load=load, hist_hi=buf.hist_hi, stream=stream)
    qb_select_update(QB_SELECT_HI, K, buf.hist_hi, sel_hi=buf.sel_hi, rank_lo=buf.rank_lo,
                     err=buf.err, stream=stream)
    qb_radix_hist_lo(s, alpha, buf.sel_hi, buf.hist_lo, stream=stream)
    qb_select_update(QB_SELECT_LO, K, buf.hist_lo, sel_hi=buf.sel_hi, rank_lo=buf.rank_lo,
                     key_out=buf.key, q_out=buf.q, b=b, bounds=buf.bounds, err=buf.err,
                     stream=stream)


def eqb_update_ws(s, b, K, alpha, buf: EqbBuffers, ws, load=None, reset_hist_hi=False, stream=None):
    """eqb_update with pass 2 merged through the workspace `ws` (see
    qb_radix_hist_lo_ws): same results; buf.hist_lo receives the summed
    low-byte histogram.  buf.hist_hi must be zero on entry; with
    reset_hist_hi it is zero again on return (cleared by the select).  With
    `load`, the top-K loads are counted in pass 2 (qb_radix_hist_lo_ws_loads),
    where they cost less than in pass 1."""
    L, N, E, lead = _lne(s)
    qb_margins_topk(s, b, K, alpha, hist_hi=buf.hist_hi, stream=stream)
    qb_select_update(QB_SELECT_HI, K, buf.hist_hi, sel_hi=buf.sel_hi, rank_lo=buf.rank_lo,
                     err=buf.err, stream=stream)
    if load is not None:
        qb_radix_hist_lo_ws_loads(s, alpha, buf.sel_hi, ws, b, K, load, stream=stream)
    else:
        qb_radix_hist_lo_ws(s, alpha, buf.sel_hi, ws, stream=stream)
    qb_select_lo_ws(N, ws, buf.sel_hi, buf.rank_lo, buf.q, b, buf.bounds, hist_lo=buf.hist_lo,
                    key_out=buf.key, err=buf.err, hist_hi=buf.hist_hi if reset_hist_hi else None,
                    stream=stream)


def k3_update(s, b, K, alpha, bounds, hist_u, q_out, err=None, stream=None, b_in=None):
    """One K3 update: alpha pass, uniform-bin pass over the current bounds,
    select + in-place bias/bounds update.  hist_u must be zero on entry.
    b_in (optional): the bias the alpha pass reads when it is not b (the
    select writes b_next to b and never reads the old bias)."""
    qb_margins_topk(s, b if b_in is None else b_in, K, alpha, stream=stream)
    qb_uniform_hist(s, alpha, bounds, hist_u, stream=stream)
    qb_select_update(QB_SELECT_UNIFORM, K, hist_u, q_out=q_out, b=b, bounds=bounds, err=err,
                     stream=stream)


def k3_update_ws(s, b, K, alpha, bounds, ws, q_out, n_bins=1000, hist_u=None, err=None, stream=None,
                 b_in=None):
    """k3_update with the binning merged through the workspace ws
    (qb_uniform_hist_workspace_bytes): nothing to zero; same q, b and
    bounds.  b_in as in k3_update."""
    qb_margins_topk(s, b if b_in is None else b_in, K, alpha, stream=stream)
    qb_uniform_hist_ws(s, alpha, bounds, ws, n_bins, stream=stream)
    qb_select_uniform_ws(s.shape[-2], K, n_bins, ws, q_out, b, bounds, hist_u=hist_u, err=err, stream=stream)


def _mapped(tag):
    out = set()
    with open("/proc/self/maps") as f:
        for line in f:
            if tag in line:
                out.add(line.split()[-1])
    return sorted(out)


def runtime_libraries():
    """Paths of HIP runtime libraries mapped into this process."""
    return _mapped("libamdhip64")


def loaded_libqb():
    """Paths of the libqb shared objects mapped into this process."""
    return _mapped("libqb")
