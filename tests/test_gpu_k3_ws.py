"""GPU checks of the K3 mode merged through a workspace
(qb_uniform_hist_ws + qb_select_uniform_ws): the summed histogram, q, b and
bounds bit for bit against the atomic path (qb_uniform_hist into a zeroed
histogram + qb_select_update(QB_SELECT_UNIFORM)) and against the oracle,
over every slice width the binning pass picks, odd bin counts, rows stored
as bytes and as uint16, several layers, and the full-size skewed layer."""
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


def _both(s_np, b_np, K, n_bins):
    """Both K3 paths on the same inputs (bounds seeded from b); host copies."""
    L, N, E = s_np.shape
    s = G.dev(s_np)
    b0 = G.dev(b_np)
    bounds0 = torch.zeros((L, 2), dtype=torch.float32, device=G.DEV)
    qb.qb_bias_bounds(b0, bounds0)
    out = []
    for ws_path in (True, False):
        b, bounds = b0.clone(), bounds0.clone()
        alpha = torch.empty((L, N), dtype=torch.float32, device=G.DEV)
        q = torch.zeros((L, E), dtype=torch.float32, device=G.DEV)
        err = torch.zeros(1, dtype=torch.int32, device=G.DEV)
        if ws_path:
            hist_u = torch.full((L, E, n_bins), -7, dtype=torch.int32, device=G.DEV)  # overwritten
            ws = torch.full((qb.qb_uniform_hist_workspace_bytes(L, N, E, n_bins),), 0xA5, dtype=torch.uint8,
                            device=G.DEV)
            qb.k3_update_ws(s, b, K, alpha, bounds, ws, q, n_bins=n_bins, hist_u=hist_u, err=err)
        else:
            hist_u = torch.zeros((L, E, n_bins), dtype=torch.int32, device=G.DEV)
            qb.k3_update(s, b, K, alpha, bounds, hist_u, q, err=err)
        torch.cuda.synchronize()
        out.append(dict(hist_u=G.host(hist_u), q=G.host(q), b_next=G.host(b), bounds=G.host(bounds),
                        err=int(err.item()), bounds0=G.host(bounds0)))
    for k in ("hist_u", "q", "b_next", "bounds"):
        G.assert_same(f"workspace vs atomic {k}", out[0][k], out[1][k])
    assert out[0]["err"] == out[1]["err"]
    return out[0]


@pytest.mark.parametrize("E", [16, 32, 64, 128, 256])
@pytest.mark.parametrize("N,K,n_bins", [(3000, 2, 1000), (4097, 6, 7), (1, 1, 1), (2500, 3, 1025), (1500, 5, 2048)])
def test_k3_ws_matches_atomic_and_oracle(O, E, N, K, n_bins):
    if K >= E:
        pytest.skip("K < E")
    L = 2
    s_np = np.empty((L, N, E), np.float32)
    b_np = np.empty((L, E), np.float32)
    for l in range(L):
        s_np[l], b_np[l], _ = synth.random_case(40 + l, N, E, K, quant=64.0 if l else None)
    G.say(f"K3 workspace E={E} N={N} K={K} n_bins={n_bins}")
    got = _both(s_np, b_np, K, n_bins)
    assert got["err"] == 0
    for l in range(L):
        ref = O.k3_layer(s_np[l], b_np[l], K, got["bounds0"][l], n_bins)
        for k in ("hist_u", "q", "b_next", "bounds"):
            G.assert_same(f"layer {l} {k}", got[k][l], ref[k])


@pytest.mark.parametrize("N,E,n_bins", [(131072, 256, 1000), (262144, 64, 1000), (262144, 256, 2048)])
def test_k3_ws_wide_slices_and_uint16_rows(O, N, E, n_bins):
    """Shapes that take 64- or 32-expert slices; half the experts' scores
    are constant, so all their margins fall in one bin and a workgroup's
    count there exceeds 255 (uint16 rows beside byte rows)."""
    K = 6
    s1, b1, _ = synth.random_case(50, N, E, K)
    s1[:, ::2] = 0.25
    G.say(f"K3 workspace wide slices N={N} E={E} n_bins={n_bins}")
    got = _both(s1[None], b1[None], K, n_bins)
    assert got["err"] == 0
    ref = O.k3_layer(s1, b1, K, got["bounds0"][0], n_bins)
    for k in ("hist_u", "q", "b_next", "bounds"):
        G.assert_same(k, got[k][0], ref[k])


@pytest.mark.timeout(600)
def test_k3_ws_skew_full_size(O):
    """The 1,048,576-token skewed layer, 1000 bins: workspace path against
    the atomic path and the oracle."""
    s1, b1, K = synth.skew()
    G.say("K3 workspace skew full size")
    got = _both(s1[None], b1[None], K, 1000)
    assert got["err"] == 0
    ref = O.k3_layer(s1, b1, K, got["bounds0"][0], 1000)
    for k in ("hist_u", "q", "b_next", "bounds"):
        G.assert_same(k, got[k][0], ref[k])
