"""The hand-worked goldens run through the HIP path (C ABI), padded to an
expert count the library supports, so the GPU's K3 in-bin estimate and its
float64 mean are checked against values worked by hand, not only against
the oracle ("[Dev] Add global-batch quantile balancing", section "Quantile
estimator")."""
import json
import os

import numpy as np
import pytest
import torch

from exact_quantile_selection_amd import qb

pytestmark = pytest.mark.gpu

import gpu_util as G

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    qb.lib()


def test_mean_precision_golden(O):
    """The 8-expert golden twice over (E = 16): the same multiset of
    quantiles twice, so the mean and b_next are the golden's, repeated; the
    second copy of the top expert is pushed down (b = -1) so alpha stays 0."""
    g = json.load(open(os.path.join(GOLDEN, "mean_precision.json")))
    s = np.tile(np.array(g["s"], np.float32), (1, 2))
    b = np.tile(np.array(g["b"], np.float32), 2)
    b[8 + 4] = -1.0
    K = g["K"]
    G.say("golden mean precision E=16")
    got = G.run_eqb(s, b, K)
    G.compare_eqb(got, O.eqb_layer(s, b, K), tag="mean golden ")
    G.assert_same("b_next", got["b_next"], np.tile(np.array(g["b_next"], np.float32), 2))
    G.assert_same("bounds", got["bounds"], np.array(g["bounds"], np.float32))
    assert got["b_next"][3] == np.float32(2.0 ** -32)


def test_k3_interpolation_golden(O):
    """The 2-expert K3 golden (K/E = 1/2) inside E = 16, K = 8: seven
    experts always rank above both golden columns and seven below, so alpha,
    rank m = 4 and the two golden columns' margins are unchanged."""
    g = json.load(open(os.path.join(GOLDEN, "k3_interpolation.json")))
    s2 = np.array(g["s"], np.float32)
    N = s2.shape[0]
    E, K = 16, 8
    s = np.zeros((N, E), np.float32)
    b = np.zeros(E, np.float32)
    s[:, :2] = s2
    s[:, 2:9] = 0.0
    b[2:9] = 2.0       # v = 2: always in the top K
    s[:, 9:] = 1.0
    b[9:] = -2.0       # v = -1: always below both golden columns
    bounds = np.array(g["bounds_in"], np.float32)
    G.say("golden K3 interpolation E=16 K=8")
    got = G.run_k3(s, b, K, bounds, g["n_bins"])
    ref = O.k3_layer(s, b, K, bounds, g["n_bins"])
    assert got["err"] == 0
    for k in ("alpha", "hist_u", "q", "b_next", "bounds"):
        G.assert_same(k, got[k], ref[k])
    G.assert_same("alpha", got["alpha"], np.array(g["alpha"], np.float32))
    G.assert_same("hist_u[:2]", got["hist_u"][:2], np.array(g["hist_u"], np.int32))
    G.assert_same("q[:2]", got["q"][:2], np.array(g["q"], np.float32))
