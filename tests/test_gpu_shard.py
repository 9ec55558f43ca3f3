"""GPU checks of the data-parallel emulation: the emulated all-reduce, the
rank-averaged update, EQB over R emulated ranks (bit-identical to the
unsharded update on every rank, whatever the sharding) and rank-averaged QB
(bit-exact against the oracle; differs from EQB and depends on the sharding)."""
import numpy as np
import pytest
import torch

from exact_quantile_selection_amd import qb, synth
from exact_quantile_selection_amd.shard import ShardedUpdate

import gpu_util as G

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    qb.lib()


@pytest.mark.parametrize("R,M", [(1, 7), (3, 1000), (8, 65536), (8, 1)])
def test_allreduce_sum(R, M):
    G.say(f"allreduce R={R} M={M}")
    a = np.random.default_rng([R, M]).integers(-1000, 100000, size=(R, M)).astype(np.int32)
    t = G.dev(a)
    qb.qb_allreduce_sum_i32(t)
    want = np.repeat(a.sum(axis=0, dtype=np.int64).astype(np.int32)[None, :], R, axis=0)
    G.assert_same("allreduce", G.host(t), want)


@pytest.mark.parametrize("R,E", [(1, 256), (8, 256), (5, 64), (2, 16)])
def test_rank_average_vs_oracle(O, R, E):
    q = np.random.default_rng([R, E]).normal(0, 0.3, (R, E)).astype(np.float32)
    b = torch.empty(E, dtype=torch.float32, device=G.DEV)
    bounds = torch.empty(2, dtype=torch.float32, device=G.DEV)
    qb.qb_rank_average(G.dev(q), b, bounds)
    rb, rbo = O.rank_average(q)
    G.assert_same("b", G.host(b), rb)
    G.assert_same("bounds", G.host(bounds), rbo)


CASES = [(8192, 64, 4, 16.0), (8192, 256, 6, None), (4096, 16, 2, 8.0)]


@pytest.mark.parametrize("N,E,K,quant", CASES)
@pytest.mark.parametrize("R", [1, 2, 8])
def test_eqb_sharded_equals_unsharded(O, N, E, K, quant, R):
    G.say(f"sharded EQB N={N} E={E} K={K} R={R}")
    s, b, _ = synth.random_case(31, N, E, K, quant=quant)
    sh = ShardedUpdate(R, N, E, K, device=G.DEV)
    sh.eqb(G.dev(s), G.dev(b))
    torch.cuda.synchronize()
    assert int(sh.buf.err.item()) == 0
    ref = O.eqb_layer(s, b, K)
    G.assert_same("b_next on every rank", G.host(sh.b), np.repeat(ref["b_next"][None, :], R, axis=0))
    G.assert_same("bounds on every rank", G.host(sh.buf.bounds), np.repeat(ref["bounds"][None, :], R, axis=0))
    G.assert_same("all-reduced hist_hi", G.host(sh.buf.hist_hi), np.repeat(ref["hist_hi"][None], R, axis=0))
    G.assert_same("all-reduced hist_lo", G.host(sh.buf.hist_lo), np.repeat(ref["hist_lo"][None], R, axis=0))


@pytest.mark.parametrize("N,E,K,quant", CASES)
@pytest.mark.parametrize("R", [1, 2, 8])
def test_rank_averaged_vs_oracle(O, N, E, K, quant, R):
    G.say(f"rank-averaged QB N={N} E={E} K={K} R={R}")
    s, b, _ = synth.random_case(31, N, E, K, quant=quant)
    sh = ShardedUpdate(R, N, E, K, device=G.DEV)
    sh.rank_averaged(G.dev(s), G.dev(b))
    torch.cuda.synchronize()
    assert int(sh.buf.err.item()) == 0
    q_local = O.rank_local_quantiles(s, b, K, R)
    G.assert_same("rank-local quantiles", G.host(sh.buf.q), q_local)
    rb, rbo = O.rank_average(q_local)
    G.assert_same("b (rank-averaged)", G.host(sh.b_avg), rb)
    G.assert_same("bounds (rank-averaged)", G.host(sh.bounds_avg), rbo)
    eqb = O.eqb_layer(s, b, K)["b_next"]
    if R == 1:
        G.assert_same("R = 1 is EQB", G.host(sh.b_avg), eqb)
    else:
        assert not np.array_equal(G.host(sh.b_avg), eqb)


def test_sharding_dependence(O):
    """Reordering the tokens of the batch (a different assignment of tokens
    to ranks) leaves EQB bit-identical and moves rank-averaged QB."""
    N, E, K, R = 8192, 64, 4, 8
    s, b, _ = synth.random_case(41, N, E, K, offset_std=0.8)
    perm = np.random.default_rng(7).permutation(N)
    outs = []
    for order in (np.arange(N), perm):
        G.say("sharding dependence")
        sh = ShardedUpdate(R, N, E, K, device=G.DEV)
        sd = G.dev(np.ascontiguousarray(s[order]))
        sh.eqb(sd, G.dev(b))
        e = G.host(sh.b)[0].copy()
        sh.rank_averaged(sd, G.dev(b))
        outs.append((e, G.host(sh.b_avg).copy()))
    torch.cuda.synchronize()
    G.assert_same("EQB under a token permutation", outs[1][0], outs[0][0])
    assert not np.array_equal(outs[1][1], outs[0][1])


@pytest.mark.timeout(900)
def test_full_size_eight_ranks(O):
    """The 1,048,576-token skewed layer over 8 ranks of 131,072 tokens."""
    s, b, K = synth.skew()
    N, E = s.shape
    R = 8
    G.say("8 ranks full size")
    sh = ShardedUpdate(R, N, E, K, device=G.DEV)
    sd = G.dev(s)
    sh.eqb(sd, G.dev(b))
    eqb_gpu = G.host(sh.b)
    sh.rank_averaged(sd, G.dev(b))
    q_gpu, bavg_gpu = G.host(sh.buf.q), G.host(sh.b_avg)
    torch.cuda.synchronize()
    G.say("8 ranks full size: oracle")
    ref = O.eqb_layer(s, b, K)
    G.assert_same("b_next on every rank", eqb_gpu, np.repeat(ref["b_next"][None, :], R, axis=0))
    q_local = O.rank_local_quantiles(s, b, K, R)
    G.assert_same("rank-local quantiles", q_gpu, q_local)
    G.assert_same("rank-averaged b", bavg_gpu, O.rank_average(q_local)[0])
