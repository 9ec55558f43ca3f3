"""Helpers for the GPU parity tests: device transfer, the EQB / K3 call
sequences through the C ABI, and bit-exact comparison with the oracle."""
import sys

import numpy as np
import torch

from exact_quantile_selection_amd import qb

DEV = torch.device("cuda:0")


def say(msg: str):
    """Name the case before a GPU step (visible even if the box dies)."""
    print(f"[gpu] {msg}", flush=True)
    sys.stdout.flush()


def dev(a):
    return torch.from_numpy(np.ascontiguousarray(a)).to(DEV)


def host(t):
    return t.detach().cpu().numpy()


def bits(a):
    a = np.ascontiguousarray(a)
    return a.view(np.uint8)


def assert_same(name, got, want):
    got = np.asarray(got)
    want = np.ascontiguousarray(want)
    assert got.shape == want.shape, f"{name}: shape {got.shape} vs {want.shape}"
    want = want.astype(got.dtype, copy=False)
    if not np.array_equal(bits(got), bits(want)):
        g = np.ascontiguousarray(got).ravel()
        w = np.ascontiguousarray(want).ravel()
        rows = np.any(g.view(np.uint8).reshape(g.size, -1) != w.view(np.uint8).reshape(w.size, -1), axis=1)
        idx = np.nonzero(rows)[0]
        raise AssertionError(f"{name}: {idx.size} of {g.size} differ; first at {idx[:5].tolist()}: "
                             f"got {g[idx[:5]].tolist()} want {w[idx[:5]].tolist()}")


def run_eqb(s_np, b_np, K, with_load=True):
    """Full EQB update of one layer on the GPU; returns host copies."""
    N, E = s_np.shape
    s = dev(s_np)
    b = dev(b_np)
    alpha = torch.empty(N, dtype=torch.float32, device=DEV)
    load = torch.zeros(E, dtype=torch.int32, device=DEV) if with_load else None
    buf = qb.EqbBuffers(1, E, device=DEV, lead=False)
    qb.eqb_update(s, b, K, alpha, buf, load=load)
    torch.cuda.synchronize()
    out = dict(alpha=host(alpha), hist_hi=host(buf.hist_hi), sel_hi=host(buf.sel_hi),
               rank_lo=host(buf.rank_lo), hist_lo=host(buf.hist_lo), key=host(buf.key),
               q=host(buf.q), b_next=host(b), bounds=host(buf.bounds), err=int(buf.err.item()))
    if with_load:
        out["load"] = host(load)
    return out


EQB_KEYS = ("alpha", "hist_hi", "sel_hi", "rank_lo", "hist_lo", "key", "q", "b_next", "bounds")


def compare_eqb(got, ref, with_load=True, tag=""):
    assert got["err"] == 0, f"{tag}: device error bits {got['err']}"
    for k in EQB_KEYS + (("load",) if with_load else ()):
        assert_same(f"{tag}{k}", got[k], ref[k])


def run_k3(s_np, b_np, K, bounds_np, n_bins):
    N, E = s_np.shape
    s = dev(s_np)
    b = dev(b_np)
    bounds = dev(bounds_np.astype(np.float32))
    alpha = torch.empty(N, dtype=torch.float32, device=DEV)
    hist_u = torch.zeros((E, n_bins), dtype=torch.int32, device=DEV)
    q = torch.zeros(E, dtype=torch.float32, device=DEV)
    err = torch.zeros(1, dtype=torch.int32, device=DEV)
    qb.k3_update(s, b, K, alpha, bounds, hist_u, q_out=q, err=err)
    torch.cuda.synchronize()
    return dict(alpha=host(alpha), hist_u=host(hist_u), q=host(q), b_next=host(b),
                bounds=host(bounds), err=int(err.item()))
