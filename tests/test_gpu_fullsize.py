"""GPU parity at the full workload sizes, in the launch configuration the
benchmark times: the 65,536-token single layer (EQB and K3), the 1,048,576-
token skewed layer with forced bf16 ties, and the 48-layer step (every layer
against the full oracle and the radix invariants)."""
from concurrent.futures import ThreadPoolExecutor

import numpy as np
import pytest
import torch

from exact_quantile_selection_amd import qb, synth

import gpu_util as G

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    qb.lib()


def test_single_layer_eqb_and_k3(O):
    s, b, K = synth.single()
    G.say(f"single EQB N={s.shape[0]}")
    G.compare_eqb(G.run_eqb(s, b, K), O.eqb_layer(s, b, K), tag="single ")
    bounds = O.bounds_of(b)
    ref = O.k3_layer(s, b, K, bounds, 1000)
    G.say("single K3")
    got = G.run_k3(s, b, K, bounds, 1000)
    assert got["err"] == 0
    for k in ("alpha", "hist_u", "q", "b_next", "bounds"):
        G.assert_same(f"k3 {k}", got[k], ref[k])


@pytest.mark.timeout(600)
def test_skew_full_size(O):
    s, b, K = synth.skew()
    G.say(f"skew N={s.shape[0]} E={s.shape[1]}")
    got = G.run_eqb(s, b, K)
    ref = O.eqb_layer(s, b, K)
    G.compare_eqb(got, ref, tag="skew ")


def _invariants(l, N, E, K, hist_hi, sel_hi, rank_lo, hist_lo, key, b_next):
    m = -(-K * N // E)
    assert (hist_hi.sum(axis=1) == N).all(), f"layer {l}: hist_hi row totals"
    C = np.cumsum(hist_hi, axis=1)
    for j in range(E):
        sel = sel_hi[j]
        below = C[j, sel - 1] if sel else 0
        assert below < m <= C[j, sel], f"layer {l} expert {j}: high-byte bin"
        assert rank_lo[j] == m - below
        assert hist_lo[j].sum() == hist_hi[j, sel]
        Cl = np.cumsum(hist_lo[j])
        lo = int(key[j]) & 0xFF
        assert int(key[j]) >> 8 == sel
        assert (Cl[lo - 1] if lo else 0) < rank_lo[j] <= Cl[lo], f"layer {l} expert {j}: low byte"
    half_ulp = 0.5 * np.spacing(np.abs(b_next).max())
    assert abs(b_next.astype(np.float64).sum()) <= E * half_ulp


@pytest.mark.timeout(900)
def test_step_48_layers(O):
    """All 48 layers of the step in one launch sequence, every layer
    compared with the oracle bit for bit (alpha, both histograms, the
    selections, key, q, b_next, bounds) as well as checked against the
    radix invariants.  The oracle runs layer by layer in a thread pool (its
    calls release the GIL), regenerating each layer's seeded inputs."""
    p = synth.WORKLOADS["step"]
    L, N, E, K = p["L"], p["N"], p["E"], p["K"]
    s = torch.empty((L, N, E), dtype=torch.float32, device=G.DEV)
    b = torch.empty((L, E), dtype=torch.float32, device=G.DEV)
    G.say(f"step: generating {L} layers")

    def gen(l):
        sl, bl, _ = synth.step_layer(l)
        return l, sl, bl

    with ThreadPoolExecutor(8) as ex:
        for l, sl, bl in ex.map(gen, range(L)):
            s[l].copy_(torch.from_numpy(sl))
            b[l].copy_(torch.from_numpy(bl))
    alpha = torch.empty((L, N), dtype=torch.float32, device=G.DEV)
    buf = qb.EqbBuffers(L, E, device=G.DEV)
    G.say("step: EQB over 48 layers")
    qb.eqb_update(s, b, K, alpha, buf)
    torch.cuda.synchronize()
    assert int(buf.err.item()) == 0
    del s
    hh, hl = G.host(buf.hist_hi), G.host(buf.hist_lo)
    sel, rk, key, bn = G.host(buf.sel_hi), G.host(buf.rank_lo), G.host(buf.key), G.host(b)
    al, q, bounds = G.host(alpha), G.host(buf.q), G.host(buf.bounds)
    for l in range(L):
        _invariants(l, N, E, K, hh[l], sel[l], rk[l], hl[l], key[l], bn[l])

    def check(l):
        sl, bl, _ = synth.step_layer(l)
        ref = O.eqb_layer(sl, bl, K)
        got = dict(alpha=al[l], hist_hi=hh[l], sel_hi=sel[l], rank_lo=rk[l], hist_lo=hl[l],
                   key=key[l], q=q[l], b_next=bn[l], bounds=bounds[l], err=0)
        G.compare_eqb(got, ref, with_load=False, tag=f"step layer {l} ")
        return l

    G.say("step: oracle on all 48 layers")
    done = 0
    with ThreadPoolExecutor(8) as ex:
        for l in ex.map(check, range(L)):
            done += 1
            if done % 8 == 0:
                G.say(f"step: {done} of {L} layers equal to the oracle")
    assert done == L


@pytest.mark.timeout(600)
@pytest.mark.parametrize("ws", [False, True])
def test_tiled_layer_beyond_int32_elements(O, ws):
    """A layer of 9,437,184 tokens x 256 experts (2.4e9 scores, 9.7 GB:
    element offsets past 2^31) built by repeating a 4096-row block T = 2304
    times.  Every expert column is the block's column repeated T times, so
    its order statistic of rank m = T * m_block (m_block = K * 4096 / E = 96)
    is the block's order statistic of rank m_block: the oracle run on the
    block gives the exact expected key, q, b_next and bounds, and the
    histograms and loads are T times the block's."""
    P, E, K, T = 4096, 256, 6, 2304
    N = P * T
    assert N * E > 2 ** 31 and (K * P) % E == 0
    blk, b_np, _ = synth.random_case(17, P, E, K, quant=64.0)
    ref = O.eqb_layer(blk, b_np, K)
    G.say(f"tiled layer N={N} E={E} ({'workspace' if ws else 'atomic'} pass 2)")
    s = G.dev(blk).repeat(T, 1)
    b = G.dev(b_np)
    alpha = torch.empty(N, dtype=torch.float32, device=G.DEV)
    load = torch.zeros(E, dtype=torch.int32, device=G.DEV)
    buf = qb.EqbBuffers(1, E, device=G.DEV, lead=False)
    if ws:
        wsb = torch.empty(qb.qb_hist_lo_workspace_bytes(1, N, E), dtype=torch.uint8, device=G.DEV)
        qb.eqb_update_ws(s, b, K, alpha, buf, wsb, load=load)
    else:
        qb.eqb_update(s, b, K, alpha, buf, load=load)
    torch.cuda.synchronize()
    assert int(buf.err.item()) == 0
    del s
    a = G.host(alpha).reshape(T, P)
    assert (a == ref["alpha"][None, :]).all(), "alpha differs from the block's in some repeat"
    G.assert_same("load", G.host(load), T * ref["load"])
    G.assert_same("hist_hi", G.host(buf.hist_hi), T * ref["hist_hi"])
    G.assert_same("sel_hi", G.host(buf.sel_hi), ref["sel_hi"])
    G.assert_same("rank_lo", G.host(buf.rank_lo), T * ref["rank_lo"])
    G.assert_same("hist_lo", G.host(buf.hist_lo), T * ref["hist_lo"])
    for k in ("key", "q", "b_next", "bounds"):
        G.assert_same(k, G.host({"key": buf.key, "q": buf.q, "b_next": b, "bounds": buf.bounds}[k]), ref[k])
    torch.cuda.empty_cache()


@pytest.mark.timeout(600)
@pytest.mark.parametrize("E,T,n_bins", [(64, 4096, 40), (256, 64, 2048), (256, 256, 1000)])
def test_k3_tiled_layer(O, E, T, n_bins):
    """K3 binning of a 4096-row block with heavy ties repeated T times, at
    sizes that take the wide expert slices of the binning pass: 16,777,216
    tokens x 64 experts (64-expert slices, about 65,000 rows per workgroup,
    so the packed 16-bit LDS counters run close to their limit), 262,144 x
    256 with 2048 bins (32-expert slices) and 1,048,576 x 256 with 1000
    bins (64-expert slices).  The histogram is T times the block's, and the
    interpolated quantile (rank m = T * m_block; every count scales by the
    same factor) and b_next are the block's exactly."""
    P, K = 4096, 6
    blk, b_np, _ = synth.random_case(23, P, E, K, quant=2.0)
    bounds = O.bounds_of(b_np)
    ref = O.k3_layer(blk, b_np, K, bounds, n_bins)
    N = P * T
    G.say(f"k3 tiled N={N} E={E} bins={n_bins}")
    s = G.dev(blk).repeat(T, 1)
    b = G.dev(b_np)
    bnd = G.dev(bounds.astype(np.float32))
    alpha = torch.empty(N, dtype=torch.float32, device=G.DEV)
    hist_u = torch.zeros((E, n_bins), dtype=torch.int32, device=G.DEV)
    q = torch.zeros(E, dtype=torch.float32, device=G.DEV)
    err = torch.zeros(1, dtype=torch.int32, device=G.DEV)
    qb.k3_update(s, b, K, alpha, bnd, hist_u, q_out=q, err=err)
    torch.cuda.synchronize()
    assert int(err.item()) == 0
    del s
    G.assert_same("hist_u", G.host(hist_u), T * ref["hist_u"])
    for k, t in (("q", q), ("b_next", b), ("bounds", bnd)):
        G.assert_same(k, G.host(t), ref[k])
    torch.cuda.empty_cache()


@pytest.mark.timeout(600)
def test_k3_more_bins_on_a_later_call(O):
    """Two K3 binning calls in a row that take the same 64-expert slice
    width, the second with more bins (a larger LDS table) than the first:
    600 then 1000 bins over 524,288 tokens x 256 experts (a 4096-row block
    repeated 128 times, so the expected results are the block's)."""
    P, E, K, T = 4096, 256, 6, 128
    blk, b_np, _ = synth.random_case(29, P, E, K, quant=8.0)
    bounds = O.bounds_of(b_np)
    N = P * T
    s = G.dev(blk).repeat(T, 1)
    for n_bins in (600, 1000):
        ref = O.k3_layer(blk, b_np, K, bounds, n_bins)
        G.say(f"k3 N={N} E={E} bins={n_bins} after a smaller table")
        b = G.dev(b_np)
        bnd = G.dev(bounds.astype(np.float32))
        alpha = torch.empty(N, dtype=torch.float32, device=G.DEV)
        hist_u = torch.zeros((E, n_bins), dtype=torch.int32, device=G.DEV)
        q = torch.zeros(E, dtype=torch.float32, device=G.DEV)
        err = torch.zeros(1, dtype=torch.int32, device=G.DEV)
        qb.k3_update(s, b, K, alpha, bnd, hist_u, q_out=q, err=err)
        torch.cuda.synchronize()
        assert int(err.item()) == 0
        G.assert_same(f"hist_u ({n_bins} bins)", G.host(hist_u), T * ref["hist_u"])
        for k, t in (("q", q), ("b_next", b), ("bounds", bnd)):
            G.assert_same(f"{k} ({n_bins} bins)", G.host(t), ref[k])
    del s
    torch.cuda.empty_cache()


@pytest.mark.timeout(600)
def test_streaming_passes_with_a_ragged_last_trip(O):
    """786,509 tokens x 256 experts: just above the size from which both
    passes read with non-temporal loads (768 MiB), pass 1 with 8 lanes per
    row, and 77 rows past a whole number of trips, so the last trip of the
    8-lane form clamps and masks its rows.  The update with and without the
    loads in pass 2, and the K3 update (whose binning pass streams too),
    equal the oracle's, bit for bit."""
    N, E, K = 786432 + 77, 256, 6
    assert N * E * 4 >= 768 << 20
    s_np, b_np, _ = synth.random_case(53, N, E, K, quant=64.0)
    G.say(f"streaming ragged layer N={N} E={E}")
    ref = O.eqb_layer(s_np, b_np, K)
    s = G.dev(s_np)
    ws = torch.empty(qb.qb_hist_lo_workspace_bytes(1, N, E), dtype=torch.uint8, device=G.DEV)
    for with_load in (False, True):
        b = G.dev(b_np)
        alpha = torch.empty(N, dtype=torch.float32, device=G.DEV)
        buf = qb.EqbBuffers(1, E, device=G.DEV, lead=False)
        load = torch.zeros(E, dtype=torch.int32, device=G.DEV)
        qb.eqb_update_ws(s, b, K, alpha, buf, ws, load=load if with_load else None)
        torch.cuda.synchronize()
        assert int(buf.err.item()) == 0
        got = dict(alpha=G.host(alpha), hist_hi=G.host(buf.hist_hi), sel_hi=G.host(buf.sel_hi),
                   hist_lo=G.host(buf.hist_lo), key=G.host(buf.key), q=G.host(buf.q), b_next=G.host(b),
                   bounds=G.host(buf.bounds))
        for k in ("alpha", "hist_hi", "sel_hi", "hist_lo", "key", "q", "b_next", "bounds"):
            G.assert_same(f"ragged {k}", got[k], ref[k])
        if with_load:
            G.assert_same("ragged load", G.host(load), ref["load"])
    # K3 on the same layer: its binning pass streams too (64-expert slices)
    bounds = O.bounds_of(b_np)
    k3 = O.k3_layer(s_np, b_np, K, bounds, 1000)
    b = G.dev(b_np)
    bnd = G.dev(bounds.astype(np.float32))
    alpha = torch.empty(N, dtype=torch.float32, device=G.DEV)
    hist_u = torch.zeros((E, 1000), dtype=torch.int32, device=G.DEV)
    q = torch.zeros(E, dtype=torch.float32, device=G.DEV)
    err = torch.zeros(1, dtype=torch.int32, device=G.DEV)
    qb.k3_update(s, b, K, alpha, bnd, hist_u, q_out=q, err=err)
    torch.cuda.synchronize()
    assert int(err.item()) == 0
    for k, t in (("alpha", alpha), ("hist_u", hist_u), ("q", q), ("b_next", b), ("bounds", bnd)):
        G.assert_same(f"ragged K3 {k}", G.host(t), k3[k])
    del s
    torch.cuda.empty_cache()


@pytest.mark.timeout(600)
@pytest.mark.parametrize("E", [32, 64, 128, 256])
def test_streaming_passes_on_a_tiled_gib_layer(O, E):
    """One GiB of scores per layer (a 4096-row block repeated 2^16 / E
    times): the size at which both passes read with non-temporal loads, pass
    1 with 8 lanes per row.  The workspace update without loads, with the
    loads in pass 2, and with per-microbatch loads in pass 2 all give the
    block's alpha (every repeat), key, q, b_next and bounds, and T times its
    histograms and loads.  The K3 update on the same layer (its alpha-only
    pass streams too, and so does its binning for 32 experts or more) gives
    the block's alpha, q, b_next and bounds and T times its 1000-bin
    histogram."""
    P, K = 4096, 6 if E >= 64 else 4
    T = (1 << 16) // E
    N = P * T
    assert N * E * 4 == 1 << 30
    blk, b_np, _ = synth.random_case(41 + E, P, E, K, quant=64.0)
    if E == 256:
        # Rows whose top K+1 all lie in one lane's columns of the 8-lane
        # split (experts 32 b + c, c < 4, sit in its first lane): alpha then
        # comes from one lane's list alone.
        cols = np.array([0, 1, 2, 3, 32, 33, 34, 35, 64])[:K + 1]
        blk[:64, cols] = (np.float32(3.0) - np.arange(K + 1, dtype=np.float32) / 64)[None, :]
    ref = O.eqb_layer(blk, b_np, K)
    n_mb = P * 8
    mb_ref = O.microbatch_loads(blk, b_np, K, P)  # one block per microbatch row of the oracle
    s = G.dev(blk).repeat(T, 1)
    ws = torch.empty(qb.qb_hist_lo_workspace_bytes(1, N, E), dtype=torch.uint8, device=G.DEV)
    for mode in ("plain", "loads", "microbatch loads"):
        G.say(f"streaming GiB layer E={E} {mode}")
        b = G.dev(b_np)
        alpha = torch.empty(N, dtype=torch.float32, device=G.DEV)
        buf = qb.EqbBuffers(1, E, device=G.DEV, lead=False)
        load = torch.zeros(E, dtype=torch.int32, device=G.DEV)
        if mode == "plain":
            qb.eqb_update_ws(s, b, K, alpha, buf, ws)
        elif mode == "loads":
            qb.eqb_update_ws(s, b, K, alpha, buf, ws, load=load)
        else:
            load_mb = torch.zeros((N // n_mb, E), dtype=torch.int32, device=G.DEV)
            qb.qb_margins_topk(s, b, K, alpha, hist_hi=buf.hist_hi)
            qb.qb_select_update(qb.QB_SELECT_HI, K, buf.hist_hi, sel_hi=buf.sel_hi, rank_lo=buf.rank_lo,
                                err=buf.err)
            qb.qb_radix_hist_lo_ws_loads(s, alpha, buf.sel_hi, ws, b, K, load, n_mb=n_mb, load_mb=load_mb)
            qb.qb_select_lo_ws(N, ws, buf.sel_hi, buf.rank_lo, buf.q, b, buf.bounds, hist_lo=buf.hist_lo,
                               key_out=buf.key, err=buf.err)
        torch.cuda.synchronize()
        assert int(buf.err.item()) == 0
        a = G.host(alpha).reshape(T, P)
        assert (a == ref["alpha"][None, :]).all(), f"{mode}: alpha differs from the block's in some repeat"
        G.assert_same(f"{mode} hist_hi", G.host(buf.hist_hi), T * ref["hist_hi"])
        G.assert_same(f"{mode} hist_lo", G.host(buf.hist_lo), T * ref["hist_lo"])
        for k, t in (("sel_hi", buf.sel_hi), ("key", buf.key), ("q", buf.q), ("b_next", b), ("bounds", buf.bounds)):
            G.assert_same(f"{mode} {k}", G.host(t), ref[k])
        if mode != "plain":
            G.assert_same(f"{mode} load", G.host(load), T * ref["load"])
        if mode == "microbatch loads":
            G.assert_same("load_mb", G.host(load_mb), np.tile(8 * mb_ref, (N // n_mb, 1)))
    G.say(f"streaming GiB layer E={E} K3")
    bounds = O.bounds_of(b_np)
    k3 = O.k3_layer(blk, b_np, K, bounds, 1000)
    b = G.dev(b_np)
    bnd = G.dev(bounds.astype(np.float32))
    alpha = torch.empty(N, dtype=torch.float32, device=G.DEV)
    hist_u = torch.zeros((E, 1000), dtype=torch.int32, device=G.DEV)
    q = torch.zeros(E, dtype=torch.float32, device=G.DEV)
    err = torch.zeros(1, dtype=torch.int32, device=G.DEV)
    qb.k3_update(s, b, K, alpha, bnd, hist_u, q_out=q, err=err)
    torch.cuda.synchronize()
    assert int(err.item()) == 0
    assert (G.host(alpha).reshape(T, P) == ref["alpha"][None, :]).all(), "K3: alpha differs in some repeat"
    G.assert_same("K3 hist_u", G.host(hist_u), T * k3["hist_u"])
    for k, t in (("q", q), ("b_next", b), ("bounds", bnd)):
        G.assert_same(f"K3 {k}", G.host(t), k3[k])
    del s
    torch.cuda.empty_cache()
