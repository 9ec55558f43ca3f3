"""The entry point that allocates nothing (qb_radix_lo_select_noalloc,
pass 2 and the low-byte select on the library's own device scratch) against
the workspace pair it stands in for (qb_radix_hist_lo_ws +
qb_select_lo_ws), bit for bit, on two calls in a row, the second smaller;
the first spans several layer groups of the scratch."""
import numpy as np
import pytest
import torch

from exact_quantile_selection_amd import qb

import gpu_util as G

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    qb.lib()


def _inputs(L, N, E, seed, quant=None):
    g = torch.Generator(device=G.DEV)
    g.manual_seed(seed)
    off = torch.randn((L, 1, E), generator=g, device=G.DEV) * 0.5
    logits = torch.randn((L, N, E), generator=g, device=G.DEV) + off
    if quant:
        logits = torch.round(logits * quant) / quant
    s = torch.sigmoid(logits).contiguous()
    b = (torch.rand((L, E), generator=g, device=G.DEV) * 0.2 - 0.1).contiguous()
    return s, b


def _compare(L, N, E, K, seed, quant=None):
    G.say(f"no-alloc L={L} N={N} E={E} K={K} seed={seed}")
    s, b = _inputs(L, N, E, seed, quant)
    alpha = torch.empty((L, N), dtype=torch.float32, device=G.DEV)
    buf = qb.EqbBuffers(L, E, device=G.DEV)
    qb.qb_margins_topk(s, b, K, alpha, hist_hi=buf.hist_hi)
    qb.qb_select_update(qb.QB_SELECT_HI, K, buf.hist_hi, sel_hi=buf.sel_hi, rank_lo=buf.rank_lo, err=buf.err)
    torch.cuda.synchronize()
    assert int(buf.err.item()) == 0
    outs = []
    for variant in ("workspace", "noalloc"):
        o = dict(b=b.clone(), hist_hi=buf.hist_hi.clone(),
                 hist_lo=torch.full((L, E, 256), -7, dtype=torch.int32, device=G.DEV),
                 key=torch.zeros((L, E), dtype=torch.uint16, device=G.DEV),
                 q=torch.full((L, E), np.nan, dtype=torch.float32, device=G.DEV),
                 bounds=torch.zeros((L, 2), dtype=torch.float32, device=G.DEV),
                 err=torch.zeros(1, dtype=torch.int32, device=G.DEV))
        if variant == "workspace":
            ws = torch.empty(qb.qb_hist_lo_workspace_bytes(L, N, E), dtype=torch.uint8, device=G.DEV)
            qb.qb_radix_hist_lo_ws(s, alpha, buf.sel_hi, ws)
            qb.qb_select_lo_ws(N, ws, buf.sel_hi, buf.rank_lo, o["q"], o["b"], o["bounds"], hist_lo=o["hist_lo"],
                               key_out=o["key"], err=o["err"], hist_hi=o["hist_hi"])
        else:
            qb.qb_radix_lo_select_noalloc(s, alpha, buf.sel_hi, buf.rank_lo, o["q"], o["b"], o["bounds"],
                                          hist_lo=o["hist_lo"], key_out=o["key"], err=o["err"],
                                          hist_hi=o["hist_hi"])
        torch.cuda.synchronize()
        outs.append({k: G.host(v) for k, v in o.items()})
    ref, got = outs
    assert ref["err"][0] == 0 and not ref["hist_hi"].any()
    for k in ref:
        G.assert_same(f"L={L} N={N} {k}", got[k], ref[k])
    del s


def test_noalloc_equals_workspace_pair_twice():
    # 24 layers of 65,536 x 256: the partials need 151 MB at once, so the
    # scratch takes them in groups (16 layers, then 8)
    L, N, E = 24, 65536, 256
    assert qb.qb_hist_lo_workspace_bytes(L, N, E) > qb.QB_NOALLOC_SCRATCH_BYTES
    _compare(L, N, E, 6, seed=1)
    # then a smaller call on the same scratch: one ragged layer with ties
    _compare(1, 4097, 256, 6, seed=2, quant=64.0)
    _compare(1, 1000, 16, 2, seed=3)
