"""One-GPU emulation of the data-parallel bias update over R ranks.

Rank r owns tokens [r*N/R, (r+1)*N/R) of the global batch and its own copy of
every per-rank buffer (leading index r).  Two ways of combining the ranks are
compared on the summary page "Exact Quantile Balancing and Load-Error
Injection for Mixture-of-Experts" (background and EQB paragraphs):

* EQB: the byte histograms are all-reduced (summed) before each select, so
  every rank finds the global quantile; integer sums make the result
  bit-identical to the unsharded update whatever the sharding.
* rank-averaged QB (the MARIN implementation): every rank takes the quantile
  of its own tokens, and the quantiles are averaged across ranks; since an
  average of quantiles is not the quantile of the union, the bias changes
  when the same batch is split over the ranks differently.

Every step is a libqb call; this module only owns buffers and orders calls.
"""
from __future__ import annotations

import torch

from . import qb


class ShardedUpdate:
    """Buffers of R emulated ranks for one layer of E experts and N tokens."""

    def __init__(self, R: int, N: int, E: int, K: int, device="cuda"):
        if N % R:
            raise ValueError(f"R={R} must divide N={N}")
        self.R, self.N, self.E, self.K, self.n = R, N, E, K, N // R
        kw = dict(device=device)
        self.buf = qb.EqbBuffers(R, E, device=device)      # rank r: hist_hi[r], hist_lo[r], ...
        self.alpha = torch.empty((R, self.n), dtype=torch.float32, **kw)
        self.b = torch.zeros((R, E), dtype=torch.float32, **kw)   # each rank's bias copy
        self.b_avg = torch.zeros(E, dtype=torch.float32, **kw)
        self.bounds_avg = torch.zeros(2, dtype=torch.float32, **kw)

    def _passes(self, s, b, all_reduce: bool, stream):
        R, n, E, K = self.R, self.n, self.E, self.K
        sr = s.view(R, n, E)
        buf = self.buf
        buf.reset(stream)
        self.b.copy_(b.view(1, E).expand(R, E))  # the bias every rank holds
        qb.qb_margins_topk(sr, self.b, K, self.alpha, hist_hi=buf.hist_hi, stream=stream)
        if all_reduce:
            qb.qb_allreduce_sum_i32(buf.hist_hi, stream)
        qb.qb_select_update(qb.QB_SELECT_HI, K, buf.hist_hi, sel_hi=buf.sel_hi, rank_lo=buf.rank_lo,
                            err=buf.err, stream=stream)
        qb.qb_radix_hist_lo(sr, self.alpha, buf.sel_hi, buf.hist_lo, stream=stream)
        if all_reduce:
            qb.qb_allreduce_sum_i32(buf.hist_lo, stream)
        qb.qb_select_update(qb.QB_SELECT_LO, K, buf.hist_lo, sel_hi=buf.sel_hi, rank_lo=buf.rank_lo,
                            key_out=buf.key, q_out=buf.q, b=self.b, bounds=buf.bounds, err=buf.err,
                            stream=stream)

    def eqb(self, s, b, stream=None):
        """EQB over the R ranks: afterwards every row of `self.b` holds the
        global b_next (and `self.buf.bounds` every rank's bounds)."""
        self._passes(s, b, True, stream)

    def rank_averaged(self, s, b, stream=None):
        """Rank-averaged QB: `self.buf.q` holds each rank's local quantiles,
        `self.b_avg` / `self.bounds_avg` the averaged update."""
        self._passes(s, b, False, stream)
        qb.qb_rank_average(self.buf.q, self.b_avg, self.bounds_avg, stream)
