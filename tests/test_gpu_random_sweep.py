"""Seeded random sweep of the two update modes against the oracle.

Each seed draws a handful of cases: E in {16, ..., 256}, K from 1 to
min(15, E - 1), one or two layers, N log-uniform up to 40,000 (or a
multiple of pass 2's row trip, so that microbatch loads can be counted),
and one of five score recipes (Gaussian logits, logits quantised to 1/64,
Zipf-skewed quantised logits, four distinct logits, constant columns)
with a zero, uniform or quantised bias.  Every case runs

  * EQB with pass 2 merged by atomics and the loads counted in pass 1,
  * EQB with pass 2 merged through a garbage-filled workspace and the
    loads (and, where the trip allows, per-microbatch loads) counted in
    pass 2,
  * K3 through the workspace merge at a random bin count up to 2048,

and compares every output bit for bit with the oracle ("[Dev] Add
global-batch quantile balancing", sections "Quantile estimator" and
"Implementation"; "Exact Quantile Balancing and Load-Error Injection for
Mixture-of-Experts", EQB paragraph)."""
import json

import numpy as np
import pytest
import torch

from exact_quantile_selection_amd import qb

import gpu_util as G

pytestmark = pytest.mark.gpu
CASES_PER_SEED = 40


def _scores(rng, N, E, kind):
    if kind == "normal":
        x = rng.standard_normal((N, E))
    elif kind == "quant":
        x = np.round(rng.standard_normal((N, E)) * 64) / 64
    elif kind == "skew":
        off = rng.permutation(np.arange(1, E + 1)) ** -1.1
        off = 2 * (off - off.min()) / (off.max() - off.min())
        x = np.round((rng.standard_normal((N, E)) + off) * 64) / 64
    elif kind == "few":
        x = rng.choice(np.array([-1.0, 0.0, 0.5, 2.0]), size=(N, E))
    else:  # constant columns
        x = np.tile(rng.standard_normal(E), (N, 1))
    return (1.0 / (1.0 + np.exp(-x))).astype(np.float32)


def _bias(rng, E, kind):
    if kind == 0:
        return np.zeros(E, np.float32)
    if kind == 1:
        return rng.uniform(-0.2, 0.2, E).astype(np.float32)
    return (np.round(rng.uniform(-0.2, 0.2, E) * 64) / 64).astype(np.float32)


def _layer_out(buf, alpha, b, load, l):
    return dict(alpha=G.host(alpha[l]), hist_hi=G.host(buf.hist_hi[l]), sel_hi=G.host(buf.sel_hi[l]),
                rank_lo=G.host(buf.rank_lo[l]), hist_lo=G.host(buf.hist_lo[l]), key=G.host(buf.key[l]),
                q=G.host(buf.q[l]), b_next=G.host(b[l]), bounds=G.host(buf.bounds[l]), err=int(buf.err.item()),
                load=G.host(load[l]))


def _case(O, rng, idx):
    E = int(rng.choice([16, 32, 64, 128, 256]))
    K = int(rng.integers(1, min(15, E - 1) + 1))
    L = int(rng.choice([1, 2]))
    if rng.random() < 0.2:
        N = int(rng.choice([256, 2048, 4096])) * int(rng.integers(1, 5))
    else:
        N = int(np.exp(rng.uniform(0, np.log(40000))))
    kind = str(rng.choice(["normal", "quant", "skew", "few", "const"]))
    bk = int(rng.integers(0, 3))
    case = dict(i=idx, E=E, K=K, L=L, N=N, kind=kind, bias=bk)
    G.say(f"random sweep case {json.dumps(case)}")
    s_np = np.stack([_scores(rng, N, E, kind) for _ in range(L)])
    b_np = np.stack([_bias(rng, E, bk) for _ in range(L)])
    refs = [O.eqb_layer(s_np[l], b_np[l], K) for l in range(L)]
    s = G.dev(s_np)

    # EQB, atomic pass-2 merge, loads in pass 1
    b = G.dev(b_np)
    alpha = torch.empty((L, N), dtype=torch.float32, device=G.DEV)
    load = torch.zeros((L, E), dtype=torch.int32, device=G.DEV)
    buf = qb.EqbBuffers(L, E, device=G.DEV)
    qb.eqb_update(s, b, K, alpha, buf, load=load)
    torch.cuda.synchronize()
    for l in range(L):
        G.compare_eqb(_layer_out(buf, alpha, b, load, l), refs[l], tag=f"atomic {case} layer {l}: ")

    # EQB, workspace merge, loads in pass 2
    b = G.dev(b_np)
    load.zero_()
    buf = qb.EqbBuffers(L, E, device=G.DEV)
    ws = torch.full((qb.qb_hist_lo_workspace_bytes(L, N, E),), 0xA5, dtype=torch.uint8, device=G.DEV)
    qb.eqb_update_ws(s, b, K, alpha, buf, ws, load=load)
    torch.cuda.synchronize()
    for l in range(L):
        G.compare_eqb(_layer_out(buf, alpha, b, load, l), refs[l], tag=f"workspace {case} layer {l}: ")

    # per-microbatch loads in pass 2 when N is a whole number of its trips
    trip = max(256, 32768 // E)
    if N % trip == 0:
        n_mb = trip * int(rng.integers(1, N // trip + 1))
        while N % n_mb:
            n_mb -= trip
        G.say(f"random sweep case {idx}: microbatch loads, n_mb={n_mb}")
        b = G.dev(b_np)
        buf.hist_hi.zero_()
        qb.qb_margins_topk(s, b, K, alpha, hist_hi=buf.hist_hi)
        qb.qb_select_update(qb.QB_SELECT_HI, K, buf.hist_hi, sel_hi=buf.sel_hi, rank_lo=buf.rank_lo, err=buf.err)
        load.zero_()
        load_mb = torch.zeros((L, N // n_mb, E), dtype=torch.int32, device=G.DEV)
        qb.qb_radix_hist_lo_ws_loads(s, alpha, buf.sel_hi, ws, b, K, load, n_mb=n_mb, load_mb=load_mb)
        torch.cuda.synchronize()
        for l in range(L):
            G.assert_same(f"load {case}", G.host(load[l]), refs[l]["load"])
            G.assert_same(f"load_mb {case} n_mb={n_mb}", G.host(load_mb[l]),
                          O.microbatch_loads(s_np[l], b_np[l], K, n_mb))

    # K3 through the workspace merge
    n_bins = int(rng.choice([1, 7, 256, 1000, 1001, 2048])) if rng.random() < 0.5 else int(rng.integers(1, 2049))
    G.say(f"random sweep case {idx}: K3, n_bins={n_bins}")
    for l in range(L):
        bounds_np = O.bounds_of(b_np[l])
        try:
            kref = O.k3_layer(s_np[l], b_np[l], K, bounds_np, n_bins)
        except ValueError:  # the oracle's histogram never reaches rank m (cannot happen with these bounds)
            pytest.fail(f"oracle K3 failed on {case}")
        s1, b1, bounds = G.dev(s_np[l]), G.dev(b_np[l]), G.dev(bounds_np)
        a1 = torch.empty(N, dtype=torch.float32, device=G.DEV)
        q = torch.zeros(E, dtype=torch.float32, device=G.DEV)
        hist_u = torch.zeros((E, n_bins), dtype=torch.int32, device=G.DEV)
        err = torch.zeros(1, dtype=torch.int32, device=G.DEV)
        wsu = torch.full((qb.qb_uniform_hist_workspace_bytes(1, N, E, n_bins),), 0x5A, dtype=torch.uint8,
                         device=G.DEV)
        qb.k3_update_ws(s1, b1, K, a1, bounds, wsu, q, n_bins=n_bins, hist_u=hist_u, err=err)
        torch.cuda.synchronize()
        assert int(err.item()) == 0, f"K3 error bits on {case}"
        for k, v in (("alpha", a1), ("hist_u", hist_u), ("q", q), ("b_next", b1), ("bounds", bounds)):
            G.assert_same(f"k3 {k} {case} n_bins={n_bins}", G.host(v), kref[k])


@pytest.mark.parametrize("seed", range(20))
def test_random_cases_match_the_oracle(O, seed):
    rng = np.random.default_rng([20261203, seed])
    for i in range(CASES_PER_SEED):
        _case(O, rng, seed * CASES_PER_SEED + i)
