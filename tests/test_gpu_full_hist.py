"""GPU checks of the one-pass comparison path: alpha plus the full 16-bit
key histogram in one pass over the scores, then the quantile read from the
65,536 bins.  The histogram is bit-exact against the oracle's key counts,
and the update equals the two-pass EQB update bit for bit."""
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


def full_update(s_np, b_np, K):
    N, E = s_np.shape
    s, b = G.dev(s_np), G.dev(b_np)
    alpha = torch.empty(N, dtype=torch.float32, device=G.DEV)
    hist = torch.zeros((E, 65536), dtype=torch.int32, device=G.DEV)
    qb.qb_margins_full_hist(s, b, K, alpha, hist)
    key = torch.zeros(E, dtype=torch.uint16, device=G.DEV)
    q = torch.zeros(E, dtype=torch.float32, device=G.DEV)
    bounds = torch.zeros(2, dtype=torch.float32, device=G.DEV)
    err = torch.zeros(1, dtype=torch.int32, device=G.DEV)
    qb.qb_select_update(qb.QB_SELECT_FULL, K, hist, key_out=key, q_out=q, b=b, bounds=bounds, err=err)
    torch.cuda.synchronize()
    return dict(alpha=G.host(alpha), hist=G.host(hist), key=G.host(key), q=G.host(q), b_next=G.host(b),
                bounds=G.host(bounds), err=int(err.item()))


@pytest.mark.parametrize("N,E,K,quant", [(4096, 256, 6, None), (3000, 64, 4, 16.0), (777, 16, 2, None),
                                         (5000, 128, 7, 32.0), (1, 32, 3, None)])
def test_full_hist_and_select_vs_oracle(O, N, E, K, quant):
    G.say(f"full hist N={N} E={E} K={K}")
    s, b, _ = synth.random_case(51, N, E, K, quant=quant)
    got = full_update(s, b, K)
    assert got["err"] == 0
    G.assert_same("hist_full", got["hist"], O.full_hist(s, b, K))
    ref = O.eqb_layer(s, b, K)
    for k in ("alpha", "key", "q", "b_next", "bounds"):
        G.assert_same(k, got[k], ref[k])


def test_full_hist_two_layers(O):
    L, N, E, K = 2, 2048, 64, 4
    G.say("full hist, 2 layers")
    s = synth.stream_batch(3, N, E, L=L)
    b = np.random.default_rng(9).uniform(-0.2, 0.2, (L, E)).astype(np.float32)
    alpha = torch.empty((L, N), dtype=torch.float32, device=G.DEV)
    hist = torch.zeros((L, E, 65536), dtype=torch.int32, device=G.DEV)
    qb.qb_margins_full_hist(G.dev(s), G.dev(b), K, alpha, hist)
    got = G.host(hist)
    for l in range(L):
        G.assert_same(f"hist_full layer {l}", got[l], O.full_hist(s[l], b[l], K))


@pytest.mark.timeout(900)
def test_full_hist_skewed_full_size(O):
    """The 1,048,576-token skewed layer: the one-pass update equals EQB."""
    s, b, K = synth.skew()
    G.say("full hist full size")
    got = full_update(s, b, K)
    assert got["err"] == 0
    ref = O.eqb_layer(s, b, K)
    for k in ("key", "q", "b_next", "bounds"):
        G.assert_same(k, got[k], ref[k])
    assert (got["hist"].sum(axis=1) == s.shape[0]).all()
