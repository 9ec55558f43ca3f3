"""GPU checks of the fused router path (MFMA GEMM + sigmoid, with pass 1 in
the GEMM's epilogue), of the scores-only GEMM, and of the whole EQB + LEI
chain on the scores they produce.

Logits: within |d| <= 1e-2 * |ref| + 1e-4 * rms(ref) of a float64 host GEMM
of the same bf16 inputs (bf16 x bf16 products are exact in fp32; the only
error is the fp32 accumulation order over H terms).  Scores: the device's
sigmoid of its own logits is within 4 ulp of float32(1/(1+exp(-x))) taken
in float64 on the host (scores below the smallest normal float may flush
to zero).  Everything downstream (alpha, loads, histograms,
keys, b_next, bounds, LEI) is checked bit for bit against the oracle run on
the GPU-produced scores."""
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


def bf16_dev(bits):
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).to(G.DEV).view(torch.bfloat16)


def check_logits(O, hidden, w, got_rows, rows):
    """got_rows[i] holds the GPU logits of token rows[i]."""
    ref = O.router_logits(hidden, w, rows)
    got = got_rows.astype(np.float64)
    rms = np.sqrt(np.mean(ref * ref))
    bad = np.abs(got - ref) > 1e-2 * np.abs(ref) + 1e-4 * rms
    assert not bad.any(), f"{bad.sum()} logits out of tolerance; worst {np.abs(got - ref).max()}"


def check_scores(s, logits):
    """Within 4 ulp of the float64 sigmoid; scores below the smallest normal
    float (logits below about -87.3) may be flushed to zero."""
    with np.errstate(over="ignore"):
        host = (1.0 / (1.0 + np.exp(-logits.astype(np.float64)))).astype(np.float32)
    err = np.abs(s.astype(np.float64) - host)
    ok = err <= 4 * np.spacing(np.abs(host))
    tiny = host < np.finfo(np.float32).tiny
    ok |= tiny & (s >= 0) & (err <= np.finfo(np.float32).tiny)
    assert ok.all(), f"{(~ok).sum()} scores off; worst at logit {logits.ravel()[np.argmax(~ok.ravel())]}"


def run_router(hidden_np, w_np, b_np, K, with_logits=True):
    N, H = hidden_np.shape
    E = w_np.shape[0]
    hidden, w, b = bf16_dev(hidden_np), bf16_dev(w_np), G.dev(b_np)
    s = torch.empty((N, E), dtype=torch.float32, device=G.DEV)
    logits = torch.empty((N, E), dtype=torch.float32, device=G.DEV) if with_logits else None
    alpha = torch.empty(N, dtype=torch.float32, device=G.DEV)
    load = torch.zeros(E, dtype=torch.int32, device=G.DEV)
    buf = qb.EqbBuffers(1, E, device=G.DEV, lead=False)
    qb.qb_router_fused(hidden, w, b, K, s, alpha, logits_out=logits, load=load, hist_hi=buf.hist_hi)
    return s, logits, alpha, load, buf, b


@pytest.mark.parametrize("N,H,E,K", [(1000, 256, 256, 6), (333, 128, 64, 4), (129, 64, 32, 2),
                                     (4096, 512, 128, 7), (700, 128, 256, 8), (300, 64, 32, 15),
                                     (513, 128, 128, 15), (257, 64, 256, 1)])
def test_router_small(O, N, H, E, K):
    hidden_np, w_np, b_np, _, _, _ = synth.router(seed=3, N=N, H=H, E=E)
    G.say(f"router N={N} H={H} E={E} K={K}")
    s, logits, alpha, load, buf, b = run_router(hidden_np, w_np, b_np, K)
    torch.cuda.synchronize()
    s_np, lg = G.host(s), G.host(logits)
    check_logits(O, hidden_np, w_np, lg, np.arange(N))
    check_scores(s_np, lg)
    ref_a, ref_load = O.alpha(s_np, b_np, K)
    G.assert_same("alpha", G.host(alpha), ref_a)
    G.assert_same("load", G.host(load), ref_load)
    ref = O.eqb_layer(s_np, b_np, K)
    G.assert_same("hist_hi", G.host(buf.hist_hi), ref["hist_hi"])


def test_router_saturated_scores(O):
    """Router weights with std 1 instead of 0.02: logits spread over about
    +-150, so the scores cover exact 0 and 1, the flush-to-zero range and
    both tails of the sigmoid."""
    N, H, E, K = 512, 2048, 64, 4
    hidden_np, _, b_np, _, _, _ = synth.router(seed=5, N=N, H=H, E=E)
    w32 = np.random.default_rng(6).standard_normal((E, H), dtype=np.float32)
    w_np = torch.from_numpy(w32).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    s, logits, alpha, load, buf, b = run_router(hidden_np, w_np, b_np, K)
    torch.cuda.synchronize()
    s_np, lg = G.host(s), G.host(logits)
    assert lg.min() < -100 and lg.max() > 100
    check_logits(O, hidden_np, w_np, lg, np.arange(N))
    check_scores(s_np, lg)
    ref_a, ref_load = O.alpha(s_np, b_np, K)
    G.assert_same("alpha", G.host(alpha), ref_a)
    G.assert_same("load", G.host(load), ref_load)
    G.assert_same("hist_hi", G.host(buf.hist_hi), O.eqb_layer(s_np, b_np, K)["hist_hi"])


@pytest.mark.timeout(900)
def test_router_full_size_chain(O):
    """hidden [262144 x 2048] bf16, E=256, K=6: router, EQB update and LEI on
    the produced scores; logits checked on 4096 sampled rows."""
    p = synth.WORKLOADS["router"]
    G.say("router full size: generating")
    hidden_np, w_np, b_np, g_np, K, eta = synth.router()
    N, E = p["N"], p["E"]
    G.say("router full size: GPU")
    s, logits, alpha, load, buf, b = run_router(hidden_np, w_np, b_np, K)
    qb.qb_select_update(qb.QB_SELECT_HI, K, buf.hist_hi, sel_hi=buf.sel_hi, rank_lo=buf.rank_lo,
                        err=buf.err)
    qb.qb_radix_hist_lo(s, alpha, buf.sel_hi, buf.hist_lo)
    qb.qb_select_update(qb.QB_SELECT_LO, K, buf.hist_lo, sel_hi=buf.sel_hi, rank_lo=buf.rank_lo,
                        key_out=buf.key, q_out=buf.q, b=b, bounds=buf.bounds, err=buf.err)
    g = G.dev(g_np)
    qb.qb_lei_grad(g, load, K, eta)
    torch.cuda.synchronize()
    assert int(buf.err.item()) == 0
    rows = np.random.default_rng(1).choice(N, 4096, replace=False)
    s_np = G.host(s)
    lg_rows = G.host(logits[torch.from_numpy(rows).to(G.DEV)])
    G.say("router full size: oracle")
    check_logits(O, hidden_np, w_np, lg_rows, rows)
    check_scores(s_np[rows], lg_rows)
    ref = O.eqb_layer(s_np, b_np, K)
    got = dict(alpha=G.host(alpha), load=G.host(load), hist_hi=G.host(buf.hist_hi),
               sel_hi=G.host(buf.sel_hi), rank_lo=G.host(buf.rank_lo), hist_lo=G.host(buf.hist_lo),
               key=G.host(buf.key), q=G.host(buf.q), b_next=G.host(b), bounds=G.host(buf.bounds),
               err=0)
    G.compare_eqb(got, ref, tag="router ")
    G.assert_same("lei g", G.host(g), O.lei(g_np, ref["load"], K, eta))


def _fused_and_unfused(hidden_np, w_np, b_np, K):
    """qb_router_fused against qb_router_scores + qb_margins_topk on the same
    inputs: scores, logits, alpha, loads and histogram bit for bit."""
    N, H = hidden_np.shape
    E = w_np.shape[0]
    s, logits, alpha, load, buf, b = run_router(hidden_np, w_np, b_np, K)
    hidden, w = bf16_dev(hidden_np), bf16_dev(w_np)
    s2 = torch.empty((N, E), dtype=torch.float32, device=G.DEV)
    lg2 = torch.empty((N, E), dtype=torch.float32, device=G.DEV)
    qb.qb_router_scores(hidden, w, s2, logits_out=lg2)
    alpha2 = torch.empty(N, dtype=torch.float32, device=G.DEV)
    load2 = torch.zeros(E, dtype=torch.int32, device=G.DEV)
    hist2 = torch.zeros((E, 256), dtype=torch.int32, device=G.DEV)
    qb.qb_margins_topk(s2, b, K, alpha2, load=load2, hist_hi=hist2)
    torch.cuda.synchronize()
    for name, x, y in (("s", s, s2), ("logits", logits, lg2), ("alpha", alpha, alpha2), ("load", load, load2),
                       ("hist_hi", buf.hist_hi, hist2)):
        G.assert_same(f"fused vs unfused {name}", G.host(x), G.host(y))
    return G.host(s), G.host(alpha), G.host(load), G.host(buf.hist_hi)


@pytest.mark.parametrize("E,K", [(256, 6), (128, 7), (64, 8), (32, 3)])
def test_fused_epilogue_bias_and_ties(O, E, K):
    """A non-zero bias, a ragged last workgroup, and forced exact ties: expert
    rows of the weight repeated (equal logits, equal scores) with equal
    biases, and token rows repeated, so alpha is tied across experts in many
    rows and the loads depend on the lower-index rule."""
    N, H = 1000, 128
    hidden_np, w_np, _, _, _, _ = synth.router(seed=7, N=N, H=H, E=E)
    w_np = w_np.copy()
    w_np[1::2] = w_np[0::2]                  # experts 2i and 2i+1 share their weights
    hidden_np = hidden_np.copy()
    hidden_np[500:] = hidden_np[:500]        # repeated tokens
    b_np = np.random.default_rng(8).uniform(-0.1, 0.1, E).astype(np.float32)
    b_np[1::2] = b_np[0::2]
    G.say(f"fused epilogue E={E} K={K} with ties")
    s_np, a_np, load_np, hist_np = _fused_and_unfused(hidden_np, w_np, b_np, K)
    ref_a, ref_load = O.alpha(s_np, b_np, K)
    G.assert_same("alpha", a_np, ref_a)
    G.assert_same("load", load_np, ref_load)
    G.assert_same("hist_hi", hist_np, O.eqb_layer(s_np, b_np, K)["hist_hi"])


def test_fused_epilogue_saturated_equals_unfused(O):
    """Saturated scores (exact 0 and 1 in most rows: massive ties) through
    both paths at E = 256."""
    N, H, E, K = 777, 1024, 256, 6
    hidden_np, _, b_np, _, _, _ = synth.router(seed=9, N=N, H=H, E=E)
    w32 = np.random.default_rng(10).standard_normal((E, H), dtype=np.float32)
    w_np = torch.from_numpy(w32).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    G.say("fused epilogue saturated E=256")
    s_np, a_np, load_np, hist_np = _fused_and_unfused(hidden_np, w_np, b_np, K)
    ref_a, ref_load = O.alpha(s_np, b_np, K)
    G.assert_same("load", load_np, ref_load)
    G.assert_same("hist_hi", hist_np, O.eqb_layer(s_np, b_np, K)["hist_hi"])


def test_fused_epilogue_without_loads(O):
    """qb_router_fused with no load buffer (the loads then come from pass 2):
    alpha and the high-byte histogram as with it, and the loads that
    qb_radix_hist_lo_ws_loads counts afterwards equal the oracle's."""
    N, H, E, K = 1500, 256, 256, 6
    hidden_np, w_np, _, _, _, _ = synth.router(seed=12, N=N, H=H, E=E)
    b_np = np.random.default_rng(13).uniform(-0.05, 0.05, E).astype(np.float32)
    hidden, w, b = bf16_dev(hidden_np), bf16_dev(w_np), G.dev(b_np)
    s = torch.empty((N, E), dtype=torch.float32, device=G.DEV)
    alpha = torch.empty(N, dtype=torch.float32, device=G.DEV)
    buf = qb.EqbBuffers(1, E, device=G.DEV, lead=False)
    G.say("fused epilogue without loads")
    qb.qb_router_fused(hidden, w, b, K, s, alpha, hist_hi=buf.hist_hi)
    qb.qb_select_update(qb.QB_SELECT_HI, K, buf.hist_hi, sel_hi=buf.sel_hi, rank_lo=buf.rank_lo, err=buf.err)
    ws = torch.empty(qb.qb_hist_lo_workspace_bytes(1, N, E), dtype=torch.uint8, device=G.DEV)
    load = torch.zeros(E, dtype=torch.int32, device=G.DEV)
    qb.qb_radix_hist_lo_ws_loads(s, alpha, buf.sel_hi, ws, b, K, load)
    torch.cuda.synchronize()
    s_np = G.host(s)
    ref = O.eqb_layer(s_np, b_np, K)
    G.assert_same("alpha", G.host(alpha), ref["alpha"])
    G.assert_same("hist_hi", G.host(buf.hist_hi), ref["hist_hi"])
    G.assert_same("load (pass 2)", G.host(load), ref["load"])
