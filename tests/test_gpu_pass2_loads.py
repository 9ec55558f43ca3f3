"""GPU checks of the top-K loads counted in the low-byte pass
(qb_radix_hist_lo_ws_loads): the global loads and the per-microbatch loads
against the oracle and against pass 1's own counting, bit for bit, with the
pass's histogram output unchanged (the low-byte select after it matches the
oracle's EQB update)."""
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


def _run(s_np, b_np, K, n_mb=None, load_init=0):
    """Pass 1 (alpha, its own loads and microbatch loads, high-byte
    histogram), select HI, pass 2 with loads, select LO; host copies."""
    L, N, E = s_np.shape
    s, b = G.dev(s_np), G.dev(b_np)
    alpha = torch.empty((L, N), dtype=torch.float32, device=G.DEV)
    buf = qb.EqbBuffers(L, E, device=G.DEV, lead=True)
    load1 = torch.zeros((L, E), dtype=torch.int32, device=G.DEV)
    load2 = torch.full((L, E), load_init, dtype=torch.int32, device=G.DEV)
    mb1 = mb2 = None
    if n_mb:
        mb1 = torch.zeros((L, N // n_mb, E), dtype=torch.int32, device=G.DEV)
        mb2 = torch.full((L, N // n_mb, E), load_init, dtype=torch.int32, device=G.DEV)
        qb.qb_margins_topk_mb(s, b, K, alpha, load1, n_mb, mb1, hist_hi=buf.hist_hi)
    else:
        qb.qb_margins_topk(s, b, K, alpha, load=load1, hist_hi=buf.hist_hi)
    qb.qb_select_update(qb.QB_SELECT_HI, K, buf.hist_hi, sel_hi=buf.sel_hi, rank_lo=buf.rank_lo, err=buf.err)
    ws = torch.empty(qb.qb_hist_lo_workspace_bytes(L, N, E), dtype=torch.uint8, device=G.DEV)
    qb.qb_radix_hist_lo_ws_loads(s, alpha, buf.sel_hi, ws, b, K, load2, n_mb=n_mb, load_mb=mb2)
    qb.qb_select_lo_ws(N, ws, buf.sel_hi, buf.rank_lo, buf.q, b, buf.bounds, hist_lo=buf.hist_lo,
                       key_out=buf.key, err=buf.err)
    torch.cuda.synchronize()
    out = dict(alpha=G.host(alpha), load1=G.host(load1), load2=G.host(load2), hist_lo=G.host(buf.hist_lo),
               key=G.host(buf.key), q=G.host(buf.q), b_next=G.host(b), bounds=G.host(buf.bounds),
               err=int(buf.err.item()))
    if n_mb:
        out["mb1"], out["mb2"] = G.host(mb1), G.host(mb2)
    return out


def _layers(E, N, K, L, quant, bias_scale, seed=0):
    s = np.empty((L, N, E), np.float32)
    b = np.empty((L, E), np.float32)
    for l in range(L):
        s[l], b[l], _ = synth.random_case(seed + 31 * l, N, E, K, quant=quant, bias_scale=bias_scale)
    return s, b


def _check(O, s_np, b_np, K, got, n_mb=None, load_init=0):
    assert got["err"] == 0
    for l in range(s_np.shape[0]):
        ref = O.eqb_layer(s_np[l], b_np[l], K)
        G.assert_same(f"layer {l} alpha", got["alpha"][l], ref["alpha"])
        G.assert_same(f"layer {l} pass-1 load", got["load1"][l], ref["load"])
        G.assert_same(f"layer {l} pass-2 load", got["load2"][l] - load_init, ref["load"])
        for k in ("hist_lo", "key", "q", "b_next", "bounds"):
            G.assert_same(f"layer {l} {k}", got[k][l], ref[k])
        if n_mb:
            ref_mb = O.microbatch_loads(s_np[l], b_np[l], K, n_mb)
            G.assert_same(f"layer {l} pass-1 load_mb", got["mb1"][l], ref_mb)
            G.assert_same(f"layer {l} pass-2 load_mb", got["mb2"][l] - load_init, ref_mb)


@pytest.mark.parametrize("E", [16, 32, 64, 128, 256])
@pytest.mark.parametrize("N,K,quant,bias_scale", [
    (5000, 2, None, 0.1),     # ragged last trip
    (4097, 6, 64.0, 0.0),     # quantised scores, no bias: ties at alpha in most rows
    (300, 1, 8.0, 0.0),       # fewer rows than one trip; coarse ties
    (1, 3, None, 0.1),        # a single token
    (2500, 7, 16.0, 0.05),    # ties in s, broken or not by the bias
])
def test_loads_two_layers(O, E, N, K, quant, bias_scale):
    if K >= E:
        pytest.skip("K < E")
    s_np, b_np = _layers(E, N, K, 2, quant, bias_scale)
    G.say(f"pass-2 loads E={E} N={N} K={K} quant={quant} bias={bias_scale}")
    got = _run(s_np, b_np, K, load_init=5)
    _check(O, s_np, b_np, K, got, load_init=5)


@pytest.mark.parametrize("E,N,n_mb", [(16, 6144, 2048), (32, 4096, 1024), (64, 3584, 512),
                                      (128, 2304, 256), (256, 4352, 256), (256, 8192, 2048)])
@pytest.mark.parametrize("quant", [None, 32.0])
def test_microbatch_loads(O, E, N, n_mb, quant):
    """Microbatches of one trip (one flush per trip) up to several trips,
    including a ragged last workgroup share."""
    K = 4 if E > 16 else 2
    s_np, b_np = _layers(E, N, K, 2, quant, 0.0 if quant else 0.1, seed=5)
    G.say(f"pass-2 microbatch loads E={E} N={N} n_mb={n_mb} quant={quant}")
    got = _run(s_np, b_np, K, n_mb=n_mb, load_init=1)
    _check(O, s_np, b_np, K, got, n_mb=n_mb, load_init=1)


def test_rejects_microbatch_not_multiple_of_trip():
    E, N = 16, 4096
    s = torch.zeros((N, E), dtype=torch.float32, device=G.DEV)
    alpha = torch.zeros(N, dtype=torch.float32, device=G.DEV)
    sel = torch.zeros(E, dtype=torch.int32, device=G.DEV)
    ws = torch.empty(qb.qb_hist_lo_workspace_bytes(1, N, E), dtype=torch.uint8, device=G.DEV)
    b = torch.zeros(E, dtype=torch.float32, device=G.DEV)
    load = torch.zeros(E, dtype=torch.int32, device=G.DEV)
    mb = torch.zeros((4, E), dtype=torch.int32, device=G.DEV)
    with pytest.raises(qb.QBError, match="multiple of 2048"):
        qb.qb_radix_hist_lo_ws_loads(s, alpha, sel, ws, b, 2, load, n_mb=1024, load_mb=mb)


@pytest.mark.timeout(600)
def test_stream_workload_full_size(O):
    """262144 x 256, K = 6, microbatches of 4096 tokens (the controller
    stream's batch): pass-2 loads and microbatch loads equal pass 1's and the
    oracle's."""
    p = synth.WORKLOADS["stream"]
    N, E, K, n_mb = p["N"], p["E"], p["K"], p["n_mb"]
    s_np = synth.stream_batch(0, N, E)
    b_np = np.random.default_rng(3).uniform(-0.05, 0.05, (1, E)).astype(np.float32)
    G.say("pass-2 loads, stream workload full size")
    got = _run(s_np, b_np, K, n_mb=n_mb)
    G.say("pass-2 loads, stream workload: oracle")
    _check(O, s_np, b_np, K, got, n_mb=n_mb)


@pytest.mark.timeout(600)
def test_skew_full_size_loads(O):
    """1048576 x 256 (skewed offsets, scores quantised to 1/64), K = 6:
    global loads only."""
    s1, b1, K = synth.skew()
    s_np, b_np = s1[None], b1[None]
    G.say("pass-2 loads, skew full size")
    got = _run(s_np, b_np, K)
    G.assert_same("pass-2 vs pass-1 load", got["load2"], got["load1"])
    _, ref_load = O.alpha(s_np[0], b_np[0], K)
    G.assert_same("pass-2 load vs oracle", got["load2"][0], ref_load)
