"""GPU checks of the closed-loop controller pieces: per-microbatch loads,
MaxVio, and the loop itself (route a batch with the current bias, measure,
replace the bias by that batch's EQB update), bit for bit against the oracle
run as the same loop on the CPU."""
import numpy as np
import pytest
import torch

from exact_quantile_selection_amd import qb, synth
from exact_quantile_selection_amd.controller import BiasController

import gpu_util as G

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    qb.lib()


@pytest.mark.parametrize("L,C,E,K,n", [(1, 1, 256, 6, 262144), (3, 64, 256, 6, 4096), (2, 7, 16, 2, 100),
                                       (1, 300, 37, 5, 64), (300, 40, 16, 2, 64), (1, 20000, 16, 3, 32),
                                       (2, 5000, 32, 4, 128)])
def test_maxvio_vs_oracle(O, L, C, E, K, n):
    G.say(f"maxvio L={L} C={C} E={E}")
    rng = np.random.default_rng([L, C, E])
    load = rng.integers(0, 3 * n * K // E + 2, size=(L, C, E)).astype(np.int32)
    v = torch.empty((L, C), dtype=torch.float32, device=G.DEV)
    summ = torch.empty((L, 2), dtype=torch.float32, device=G.DEV)
    worst = torch.empty(2, dtype=torch.float32, device=G.DEV)
    qb.qb_maxvio(G.dev(load), K, n, v, summ, worst)
    rv, rs, rw = O.maxvio(load, K, n)
    G.assert_same("maxvio", G.host(v), rv)
    G.assert_same("summary", G.host(summ), rs)
    G.assert_same("worst", G.host(worst), rw)


@pytest.mark.parametrize("N,E,K,n_mb,quant", [(4096, 256, 6, 512, None), (6000, 64, 4, 1000, 8.0),
                                             (2048, 16, 2, 64, None), (3072, 128, 7, 3072, 16.0),
                                             (1024, 32, 3, 1, None), (4096, 256, 8, 1024, 64.0)])
def test_microbatch_loads_vs_oracle(O, N, E, K, n_mb, quant):
    G.say(f"microbatch loads N={N} E={E} K={K} n_mb={n_mb}")
    s, b, _ = synth.random_case(21, N, E, K, quant=quant)
    alpha = torch.empty(N, dtype=torch.float32, device=G.DEV)
    load_mb = torch.zeros((N // n_mb, E), dtype=torch.int32, device=G.DEV)
    qb.qb_microbatch_loads(G.dev(s), G.dev(b), K, n_mb, alpha, load_mb)
    G.assert_same("load_mb", G.host(load_mb), O.microbatch_loads(s, b, K, n_mb))
    G.assert_same("alpha", G.host(alpha), O.alpha(s, b, K, with_load=False))


def test_microbatch_loads_multilayer(O):
    L, N, E, K, n_mb = 3, 2048, 64, 4, 256
    G.say("microbatch loads, 3 layers")
    s = synth.stream_batch(2, N, E, L=L)
    b = np.random.default_rng(5).uniform(-0.2, 0.2, (L, E)).astype(np.float32)
    alpha = torch.empty((L, N), dtype=torch.float32, device=G.DEV)
    load_mb = torch.zeros((L, N // n_mb, E), dtype=torch.int32, device=G.DEV)
    qb.qb_microbatch_loads(G.dev(s), G.dev(b), K, n_mb, alpha, load_mb)
    got = G.host(load_mb)
    for l in range(L):
        G.assert_same(f"load_mb layer {l}", got[l], O.microbatch_loads(s[l], b[l], K, n_mb))


def oracle_loop(O, batches, b0, K, n_mb):
    """The controller loop written with the oracle: per step the loads and
    MaxVio under the current bias, then b <- EQB update of the batch."""
    b = b0.copy()
    out = []
    for s in batches:
        L, N, E = s.shape
        rec = dict(load=np.zeros((L, E), np.int32), load_mb=np.zeros((L, N // n_mb, E), np.int32),
                   b_next=np.zeros((L, E), np.float32))
        for l in range(L):
            _, rec["load"][l] = O.alpha(s[l], b[l], K)
            rec["load_mb"][l] = O.microbatch_loads(s[l], b[l], K, n_mb)
            rec["b_next"][l] = O.eqb_layer(s[l], b[l], K)["b_next"]
        rec["global"] = O.maxvio(rec["load"][:, None, :], K, N)
        rec["local"] = O.maxvio(rec["load_mb"], K, n_mb)
        b = rec["b_next"]
        out.append(rec)
    return out


def run_controller(batches, K, n_mb, loads_in_pass2=None):
    L, N, E = batches[0].shape
    ctl = BiasController(L, N, E, K, n_mb, device=G.DEV, loads_in_pass2=loads_in_pass2)
    got = []
    for t, s in enumerate(batches):
        G.say(f"controller step {t}")
        ctl.step(G.dev(s))
        torch.cuda.synchronize()
        assert int(ctl.buf.err.item()) == 0
        got.append(dict(load=G.host(ctl.load), load_mb=G.host(ctl.load_mb), b_next=G.host(ctl.b),
                        mv_global=G.host(ctl.mv_global), sg=G.host(ctl.summary_global),
                        wg=G.host(ctl.worst_global), mv_local=G.host(ctl.mv_local),
                        sl=G.host(ctl.summary_local), wl=G.host(ctl.worst_local)))
    return got


def compare_loop(got, want):
    for t, (g, w) in enumerate(zip(got, want)):
        G.assert_same(f"step {t} load", g["load"], w["load"])
        G.assert_same(f"step {t} load_mb", g["load_mb"], w["load_mb"])
        G.assert_same(f"step {t} b_next", g["b_next"], w["b_next"])
        G.assert_same(f"step {t} global maxvio", g["mv_global"], w["global"][0])
        G.assert_same(f"step {t} global summary", g["sg"], w["global"][1])
        G.assert_same(f"step {t} global worst", g["wg"], w["global"][2])
        G.assert_same(f"step {t} local maxvio", g["mv_local"], w["local"][0])
        G.assert_same(f"step {t} local summary", g["sl"], w["local"][1])
        G.assert_same(f"step {t} local worst", g["wl"], w["local"][2])


@pytest.mark.parametrize("n_mb,in_pass2", [(1024, False), (2048, None), (512, None), (256, None)])
def test_closed_loop_two_layers(O, n_mb, in_pass2):
    """The loads counted in pass 1 (forced at n_mb = 1024; chosen for 256,
    which is not a whole 512-row trip of the low-byte pass at E = 64) and in
    the low-byte pass (2048 and 512, chosen by the controller)."""
    L, N, E, K, T = 2, 8192, 64, 4, 5
    ctl = BiasController(L, N, E, K, n_mb, device=G.DEV, loads_in_pass2=in_pass2)
    assert qb.qb_radix_lo_trip_rows(E) == 512
    assert ctl.loads_in_pass2 == (n_mb in (2048, 512))
    batches = [synth.stream_batch(t, N, E, L=L) for t in range(T)]
    got = run_controller(batches, K, n_mb, loads_in_pass2=in_pass2)
    want = oracle_loop(O, batches, np.zeros((L, E), np.float32), K, n_mb)
    compare_loop(got, want)
    # the first batch is routed with b = 0 under skewed offsets; once the
    # bias follows the quantiles, the busiest expert's excess shrinks
    assert got[-1]["wg"][0] < 0.5 * got[0]["wg"][0]


@pytest.mark.timeout(900)
def test_closed_loop_full_size(O):
    """262,144 tokens x 256 experts, K = 6, 4096-token microbatches, three
    steps; every step bit-exact against the oracle loop."""
    p = synth.WORKLOADS["stream"]
    N, E, K, n_mb, T = p["N"], p["E"], p["K"], p["n_mb"], 3
    G.say("controller full size: generating")
    batches = [synth.stream_batch(t, N, E) for t in range(T)]
    got = run_controller(batches, K, n_mb)
    G.say("controller full size: oracle")
    want = oracle_loop(O, batches, np.zeros((1, E), np.float32), K, n_mb)
    compare_loop(got, want)


@pytest.mark.parametrize("N,E,K,n_mb,quant", [(8192, 256, 6, 1024, None), (6000, 64, 4, 1000, 8.0),
                                             (2048, 16, 2, 2048, None), (4096, 128, 7, 128, 16.0),
                                             (3000, 16, 13, 1000, None)])
def test_fused_pass1_microbatch_loads(O, N, E, K, n_mb, quant):
    """qb_margins_topk_mb: alpha, global loads, per-microbatch loads and the
    high-byte histogram from one read of the scores."""
    G.say(f"fused pass 1 + microbatch loads N={N} E={E} n_mb={n_mb}")
    s, b, _ = synth.random_case(61, N, E, K, quant=quant)
    alpha = torch.empty(N, dtype=torch.float32, device=G.DEV)
    load = torch.zeros(E, dtype=torch.int32, device=G.DEV)
    load_mb = torch.zeros((N // n_mb, E), dtype=torch.int32, device=G.DEV)
    hist = torch.zeros((E, 256), dtype=torch.int32, device=G.DEV)
    qb.qb_margins_topk_mb(G.dev(s), G.dev(b), K, alpha, load, n_mb, load_mb, hist_hi=hist)
    ref = O.eqb_layer(s, b, K)
    G.assert_same("alpha", G.host(alpha), ref["alpha"])
    G.assert_same("load", G.host(load), ref["load"])
    G.assert_same("hist_hi", G.host(hist), ref["hist_hi"])
    G.assert_same("load_mb", G.host(load_mb), O.microbatch_loads(s, b, K, n_mb))


def test_controller_step_graph_replays():
    """One controller step (loads counted in pass 2) captured in a HIP graph
    and replayed four times, with eager steps and synchronizations between
    the replays: every replay gives the eager step's loads, microbatch
    loads, MaxVio and bias, bit for bit."""
    L, N, E, K, n_mb = 2, 8192, 64, 4, 2048
    s = G.dev(synth.stream_batch(0, N, E, L=L))
    ctl = BiasController(L, N, E, K, n_mb, device=G.DEV)
    assert ctl.loads_in_pass2
    b0 = ctl.b.clone()

    def snapshot():
        return [G.host(x) for x in (ctl.load, ctl.load_mb, ctl.mv_global, ctl.mv_local, ctl.b, ctl.buf.bounds)]

    G.say("controller step graph replays")
    ctl.step(s)  # eager reference from b0
    torch.cuda.synchronize()
    want = snapshot()
    stream = torch.cuda.Stream()
    ctl.b.copy_(b0)
    torch.cuda.synchronize()
    with torch.cuda.stream(stream):
        ctl.step(s)  # warm-up outside capture
    stream.synchronize()
    graph = torch.cuda.CUDAGraph()
    ctl.b.copy_(b0)
    torch.cuda.synchronize()
    with torch.cuda.graph(graph, stream=stream):
        ctl.step(s)
    for rep in range(4):
        ctl.step(s)  # eager work between the replays
        ctl.b.copy_(b0)
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        for name, g, w in zip(("load", "load_mb", "mv_global", "mv_local", "b", "bounds"), snapshot(), want):
            G.assert_same(f"replay {rep} {name}", g, w)
        assert int(ctl.buf.err.item()) == 0
