"""Closed-loop bias controller: each global batch is routed with the current
bias, its loads give the balance metrics, and the EQB update of that batch
becomes the bias of the next one.

The loop is the one the pages describe: the bias is updated in place once per
global batch from the K/E quantile of that batch's routing margins ("[Dev] Add
global-batch quantile balancing", sections "Quantile estimator" and
"Implementation"), and balance is reported as global MaxVio (all tokens of the
step) and local MaxVio (per microbatch) ("Exact Quantile Balancing and
Load-Error Injection for Mixture-of-Experts", summary page, background and
testbed paragraphs).

Every step below is a libqb call; this module only owns buffers and orders
the calls.
"""
from __future__ import annotations

import torch

from . import qb


class BiasController:
    """EQB bias state and metric buffers for L router layers of E experts."""

    def __init__(self, L: int, N: int, E: int, K: int, n_mb: int, b0=None, device="cuda",
                 loads_in_pass2=None):
        if N % n_mb:
            raise ValueError(f"n_mb={n_mb} must divide N={N}")
        self.L, self.N, self.E, self.K, self.n_mb = L, N, E, K, n_mb
        self.C = N // n_mb
        # The low-byte pass counts the loads when its microbatches are whole
        # row trips of that pass (qb_radix_lo_trip_rows: 256 rows at E = 256,
        # 2048 at E = 16); it then costs 2-3 us at 262144 x 256 against 13 us
        # for counting them in pass 1.  Other microbatch sizes count them in
        # pass 1; loads_in_pass2=False forces that path.
        fits = n_mb % qb.qb_radix_lo_trip_rows(E) == 0
        if loads_in_pass2 and not fits:
            raise ValueError(f"n_mb={n_mb} is not a multiple of the low-byte pass's "
                             f"{qb.qb_radix_lo_trip_rows(E)}-row trip at E={E}")
        self.loads_in_pass2 = fits if loads_in_pass2 is None else bool(loads_in_pass2)
        kw = dict(device=device)
        self.b = (torch.zeros((L, E), dtype=torch.float32, **kw) if b0 is None
                  else b0.to(device=device, dtype=torch.float32).reshape(L, E).clone())
        self.buf = qb.EqbBuffers(L, E, device=device)
        # pass 2 merges its counts through a workspace; the low-byte select
        # also clears the high-byte histogram for the next step
        self.ws = torch.empty(qb.qb_hist_lo_workspace_bytes(L, N, E), dtype=torch.uint8, **kw)
        self.alpha = torch.empty((L, N), dtype=torch.float32, **kw)
        # one int32 block: global loads [L][E] then microbatch loads [L][C][E],
        # cleared by one fill per step
        self.loads = torch.zeros(L * E * (1 + self.C), dtype=torch.int32, **kw)
        self.load = self.loads[:L * E].view(L, E)
        self.load_mb = self.loads[L * E:].view(L, self.C, E)
        self.mv_global = torch.empty((L, 1), dtype=torch.float32, **kw)
        self.mv_local = torch.empty((L, self.C), dtype=torch.float32, **kw)
        self.summary_global = torch.empty((L, 2), dtype=torch.float32, **kw)
        self.summary_local = torch.empty((L, 2), dtype=torch.float32, **kw)
        self.worst_global = torch.empty(2, dtype=torch.float32, **kw)
        self.worst_local = torch.empty(2, dtype=torch.float32, **kw)

    def step(self, s: torch.Tensor, stream=None):
        """Route batch s ([L, N, E] or [N, E] when L == 1) with the current
        bias, record its loads and MaxVio, then replace the bias by the EQB
        update of this batch.  Everything stays on the device; read
        `worst_global` / `worst_local` (and the per-layer arrays) afterwards."""
        L, N, E, K = self.L, self.N, self.E, self.K
        s3 = s.view(L, N, E)
        buf = self.buf
        qb.qb_fill_i32(self.loads, 0, stream)
        if self.loads_in_pass2:
            # pass 1 with the bias in force: alpha and the high-byte
            # histogram; pass 2 counts the loads and per-microbatch loads on
            # its own read of the scores (b is still the bias in force there)
            qb.qb_margins_topk(s3, self.b, K, self.alpha, hist_hi=buf.hist_hi, stream=stream)
            qb.qb_select_update(qb.QB_SELECT_HI, K, buf.hist_hi, sel_hi=buf.sel_hi, rank_lo=buf.rank_lo,
                                err=buf.err, stream=stream)
            qb.qb_radix_hist_lo_ws_loads(s3, self.alpha, buf.sel_hi, self.ws, self.b, K, self.load,
                                         n_mb=self.n_mb, load_mb=self.load_mb, stream=stream)
        else:
            # pass 1 with the bias in force: alpha, loads, per-microbatch
            # loads and the high-byte histogram in one read of the scores
            qb.qb_margins_topk_mb(s3, self.b, K, self.alpha, self.load, self.n_mb, self.load_mb,
                                  hist_hi=buf.hist_hi, stream=stream)
            qb.qb_select_update(qb.QB_SELECT_HI, K, buf.hist_hi, sel_hi=buf.sel_hi, rank_lo=buf.rank_lo,
                                err=buf.err, stream=stream)
            qb.qb_radix_hist_lo_ws(s3, self.alpha, buf.sel_hi, self.ws, stream=stream)
        qb.qb_maxvio(self.load.view(L, 1, E), K, N, self.mv_global, self.summary_global,
                     self.worst_global, stream=stream)
        qb.qb_maxvio(self.load_mb, K, self.n_mb, self.mv_local, self.summary_local, self.worst_local,
                     stream=stream)
        # EQB update of this batch, written over b
        qb.qb_select_lo_ws(N, self.ws, buf.sel_hi, buf.rank_lo, buf.q, self.b, buf.bounds,
                           hist_lo=buf.hist_lo, key_out=buf.key, err=buf.err, hist_hi=buf.hist_hi,
                           stream=stream)
