"""GPU checks of per-microbatch LEI, its bounded variant and the gradient
through the sigmoid, against the oracle.  Unbounded results are bit-exact;
the bounded rescale evaluates tanh in float64 on each side (device math
library vs the host's), so its outputs are compared within 1 ulp of fp32."""
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


def case(seed, N, E, K, n_mb, skew):
    rng = np.random.default_rng([seed, N, E])
    g = rng.standard_normal((N, E), dtype=np.float32)
    x = rng.normal(0, 1.5, (N, E))
    s = (1.0 / (1.0 + np.exp(-x))).astype(np.float32)
    p = np.exp(skew * rng.standard_normal(E))
    load = np.stack([rng.multinomial(n_mb * K, p / p.sum()) for _ in range(N // n_mb)]).astype(np.int32)
    return g, s, load


def run(g, s, load, K, n_mb, eta, bounded, in_place=False):
    gd, sd = G.dev(g), G.dev(s)
    d = torch.empty_like(gd)
    gout = gd if in_place else torch.empty_like(gd)
    qb.qb_lei_backward(gd, G.dev(load), K, n_mb, eta, bounded=bounded, s=sd, g_out=gout, dlogits=d)
    torch.cuda.synchronize()
    return G.host(gout), G.host(d)


def within_ulp(name, got, want, ulps=1):
    err = np.abs(got.astype(np.float64) - want.astype(np.float64))
    ok = err <= ulps * np.spacing(np.abs(want)).astype(np.float64)
    assert ok.all(), f"{name}: {(~ok).sum()} values beyond {ulps} ulp"


@pytest.mark.parametrize("N,E,K,n_mb,skew", [(8192, 256, 6, 4096, 0.5), (6000, 64, 4, 1000, 2.0),
                                             (4096, 16, 2, 4096, 0.0), (2048, 128, 7, 64, 3.0)])
@pytest.mark.parametrize("bounded", [False, True])
def test_lei_backward_vs_oracle(O, N, E, K, n_mb, skew, bounded):
    G.say(f"lei backward N={N} E={E} n_mb={n_mb} bounded={bounded}")
    g, s, load = case(1, N, E, K, n_mb, skew)
    eta = np.float32(1e-5 if skew < 1 else 8e-5)
    got_g, got_d = run(g, s, load, K, n_mb, eta, bounded)
    ref_g, ref_d = O.lei_backward(g, load, K, n_mb, eta, bounded, s=s)
    if bounded:
        within_ulp("g'", got_g, ref_g)
        within_ulp("dlogits", got_d, ref_d, ulps=2)
    else:
        G.assert_same("g'", got_g, ref_g)
        G.assert_same("dlogits", got_d, ref_d)


def test_one_microbatch_unbounded_is_lei_grad(O):
    N, E, K = 4096, 256, 6
    g, s, load = case(2, N, E, K, N, 1.0)
    eta = np.float32(1e-5)
    got_g, _ = run(g, s, load, K, N, eta, False, in_place=True)
    gd = G.dev(g)
    qb.qb_lei_grad(gd, G.dev(load[0]), K, eta)
    G.assert_same("same as qb_lei_grad", got_g, G.host(gd))


@pytest.mark.timeout(600)
def test_lei_backward_router_size(O):
    """262,144 tokens x 256 experts, 4096-token microbatches, both variants."""
    N, E, K, n_mb = 262144, 256, 6, 4096
    g, s, load = case(3, N, E, K, n_mb, 1.0)
    for bounded in (False, True):
        G.say(f"lei backward router size bounded={bounded}")
        got_g, got_d = run(g, s, load, K, n_mb, np.float32(1e-5), bounded)
        ref_g, ref_d = O.lei_backward(g, load, K, n_mb, np.float32(1e-5), bounded, s=s)
        within_ulp("g'", got_g, ref_g, ulps=0 if not bounded else 1)
        within_ulp("dlogits", got_d, ref_d, ulps=0 if not bounded else 2)
