"""GPU checks of the workspace path of pass 2 (per-workgroup partial
histograms summed in the low-byte select instead of global atomics): the
whole EQB update is bit-exact against the oracle and equal to the atomic
path."""
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


def run_ws(s_np, b_np, K, reset=False, keep_ws=False):
    lead = s_np.shape[:-2]
    L = int(np.prod(lead)) if lead else 1
    N, E = s_np.shape[-2:]
    s, b = G.dev(s_np), G.dev(b_np)
    alpha = torch.empty(lead + (N,), dtype=torch.float32, device=G.DEV)
    load = torch.zeros(lead + (E,), dtype=torch.int32, device=G.DEV)
    buf = qb.EqbBuffers(L, E, device=G.DEV, lead=bool(lead))
    ws = torch.empty(qb.qb_hist_lo_workspace_bytes(L, N, E), dtype=torch.uint8, device=G.DEV)
    ws.fill_(0xAB)  # stale bytes: the path overwrites, never accumulates
    qb.eqb_update_ws(s, b, K, alpha, buf, ws, load=load, reset_hist_hi=reset)
    torch.cuda.synchronize()
    out = dict(alpha=G.host(alpha), hist_hi=G.host(buf.hist_hi), sel_hi=G.host(buf.sel_hi),
               rank_lo=G.host(buf.rank_lo), hist_lo=G.host(buf.hist_lo), key=G.host(buf.key),
               q=G.host(buf.q), b_next=G.host(b), bounds=G.host(buf.bounds), err=int(buf.err.item()),
               load=G.host(load))
    if keep_ws:
        out["ws"] = G.host(ws)
    return out


@pytest.mark.parametrize("N,E,K,quant", [(5000, 256, 6, None), (3333, 64, 4, 16.0), (1, 16, 2, None),
                                         (777, 32, 7, 8.0), (65536, 128, 3, 64.0), (100, 256, 1, None)])
def test_ws_update_vs_oracle(O, N, E, K, quant):
    G.say(f"ws update N={N} E={E} K={K}")
    s, b, _ = synth.random_case(71, N, E, K, quant=quant)
    G.compare_eqb(run_ws(s, b, K), O.eqb_layer(s, b, K), tag="ws ")


def test_ws_update_mixed_byte_and_wide_rows(O):
    """Partial rows with a count above 255 leave pass 2 as uint16, the
    others as bytes.  Experts 0-7 are constant and highest in every row, so
    alpha is the same for all rows; experts 8-127 are constant too, so each
    of them has one key and a workgroup's count in its selected bin is the
    workgroup's row count (256 rows: above 255); experts 128-255 are random
    below them (counts of a few per bin).  Both kinds of row meet in one
    select; N is ragged, so two workgroups also take a partial trip."""
    N, E, K = 65536 + 300, 256, 6
    G.say("ws update, byte and uint16 partial rows")
    rng = np.random.default_rng(12)
    s = np.empty((N, E), dtype=np.float32)
    s[:, :8] = (0.99 - 0.01 * np.arange(8)).astype(np.float32)
    s[:, 8:128] = rng.uniform(0.05, 0.6, 120).astype(np.float32)
    s[:, 128:] = rng.uniform(0.0, 0.7, (N, E - 128)).astype(np.float32)
    b = np.zeros(E, dtype=np.float32)
    got = run_ws(s, b, K, keep_ws=True)
    G.compare_eqb(got, O.eqb_layer(s, b, K), tag="ws mixed ")
    ws = got["ws"]
    rows = ws.size // 769  # L * E * G rows of (256 + 1 + 512) bytes, plus < 16 bytes of padding
    flags = ws[rows * 256: rows * 257]
    assert set(np.unique(flags).tolist()) == {0, 1}, "expected both byte and uint16 rows"


def test_ws_update_three_layers(O):
    L, N, E, K = 3, 4096, 64, 4
    G.say("ws update, 3 layers")
    s = synth.stream_batch(5, N, E, L=L)
    b = np.random.default_rng(4).uniform(-0.2, 0.2, (L, E)).astype(np.float32)
    got = run_ws(s, b, K)
    assert got["err"] == 0
    for l in range(L):
        ref = O.eqb_layer(s[l], b[l], K)
        for k in G.EQB_KEYS + ("load",):
            G.assert_same(f"layer {l} {k}", got[k][l], ref[k])


@pytest.mark.timeout(900)
def test_ws_update_skewed_full_size(O):
    """The 1,048,576-token skewed layer: the workspace path equals the
    atomic path and the oracle."""
    s, b, K = synth.skew()
    G.say("ws full size")
    got = run_ws(s, b, K)
    atomic = G.run_eqb(s, b, K)
    for k in G.EQB_KEYS + ("load",):
        G.assert_same(f"ws vs atomic {k}", got[k], atomic[k])
    G.compare_eqb(got, O.eqb_layer(s, b, K), tag="ws ")


def test_ws_select_resets_hist_hi_and_repeats(O):
    """With the reset, the select leaves the high-byte histogram zero (same
    buffer), so a second update from the same bias needs no clear and gives
    the same results; a repeated select over one workspace gives the same
    b_next again."""
    L, N, E, K = 2, 3000, 64, 5
    G.say("ws reset + repeat")
    s_np = synth.stream_batch(9, N, E, L=L)
    b_np = np.random.default_rng(2).uniform(-0.2, 0.2, (L, E)).astype(np.float32)
    s, b0 = G.dev(s_np), G.dev(b_np)
    alpha = torch.empty((L, N), dtype=torch.float32, device=G.DEV)
    buf = qb.EqbBuffers(L, E, device=G.DEV)
    ws = torch.empty(qb.qb_hist_lo_workspace_bytes(L, N, E), dtype=torch.uint8, device=G.DEV)
    ws.fill_(0xCD)
    ptr = buf.hist_hi.data_ptr()
    outs = []
    for _ in range(2):
        b = b0.clone()
        qb.eqb_update_ws(s, b, K, alpha, buf, ws, reset_hist_hi=True)
        torch.cuda.synchronize()
        assert buf.hist_hi.data_ptr() == ptr
        assert int(buf.hist_hi.abs().sum().item()) == 0, "hist_hi not cleared"
        assert int(buf.err.item()) == 0
        outs.append((G.host(b), G.host(buf.bounds), G.host(buf.q), G.host(buf.hist_lo)))
    for k, (x, y) in enumerate(zip(outs[0], outs[1])):
        G.assert_same(f"update 1 vs 2 [{k}]", x, y)
    for l in range(L):
        ref = O.eqb_layer(s_np[l], b_np[l], K)
        G.assert_same(f"layer {l} b_next", outs[0][0][l], ref["b_next"])
        G.assert_same(f"layer {l} bounds", outs[0][1][l], ref["bounds"])
        G.assert_same(f"layer {l} hist_lo", outs[0][3][l], ref["hist_lo"])
    # select again over the same workspace: same bias update from the same q
    b = b0.clone()
    qb.qb_select_lo_ws(N, ws, buf.sel_hi, buf.rank_lo, buf.q, b, buf.bounds, err=buf.err)
    torch.cuda.synchronize()
    G.assert_same("repeated select b_next", G.host(b), outs[0][0])
