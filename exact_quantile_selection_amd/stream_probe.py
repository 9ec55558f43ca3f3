"""Binding of libstreamprobe (include/stream_probe.h): the plain read kernel
whose rate is the measured HBM ceiling of the library's streaming passes.  Argument marshalling only; a missing library is an
error."""
from __future__ import annotations

import ctypes as C
import os

import torch

PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(PKG, "libstreamprobe.so")
UNROLLS = (1, 2, 4, 8, 16)

_lib = None


def lib() -> C.CDLL:
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is not built: run __graft_entry__.build()")
        L = C.CDLL(LIB_PATH)
        vp, i32, i64 = C.c_void_p, C.c_int, C.c_int64
        L.sp_read.argtypes = [vp, i64, i32, i32, vp, vp]
        L.sp_read.restype = i32
        L.sp_read_nt.argtypes = [vp, i64, i32, i32, vp, vp]
        L.sp_read_nt.restype = i32
        L.sp_copy.argtypes = [vp, vp, i64, i32, i32, vp]
        L.sp_copy.restype = i32
        _lib = L
    return _lib


def _check(t: torch.Tensor, name: str):
    if not t.is_cuda or not t.is_contiguous():
        raise ValueError(f"{name} must be a contiguous device tensor")


def _stream():
    return C.c_void_p(torch.cuda.current_stream().cuda_stream)


def read(t: torch.Tensor, sink: torch.Tensor, grid: int, unroll: int, nontemporal: bool = False) -> None:
    """Stream every byte of t once (sink: int32 [grid] on the same device),
    with non-temporal loads if asked."""
    _check(t, "t")
    _check(sink, "sink")
    if sink.dtype != torch.int32 or sink.numel() < grid:
        raise ValueError("sink must be int32 with at least `grid` elements")
    nbytes = t.numel() * t.element_size()
    fn = lib().sp_read_nt if nontemporal else lib().sp_read
    rc = fn(C.c_void_p(t.data_ptr()), nbytes, grid, unroll, C.c_void_p(sink.data_ptr()), _stream())
    if rc != 0:
        raise RuntimeError(f"sp_read{'_nt' if nontemporal else ''} failed ({rc}): bytes={nbytes} grid={grid} "
                           f"unroll={unroll}")


def copy(src: torch.Tensor, dst: torch.Tensor, grid: int, unroll: int) -> None:
    """Copy every byte of src into dst (same size, no overlap)."""
    _check(src, "src")
    _check(dst, "dst")
    nbytes = src.numel() * src.element_size()
    if dst.numel() * dst.element_size() != nbytes:
        raise ValueError("src and dst must have the same size in bytes")
    rc = lib().sp_copy(C.c_void_p(src.data_ptr()), C.c_void_p(dst.data_ptr()), nbytes, grid, unroll, _stream())
    if rc != 0:
        raise RuntimeError(f"sp_copy failed ({rc}): bytes={nbytes} grid={grid} unroll={unroll}")
