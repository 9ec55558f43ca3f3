"""Seeded synthetic inputs for the quantile-balancing bias update.

This module only draws random numbers and applies the upstream router
non-linearity (a sigmoid) that produces the score matrix the method consumes.
It holds none of the method's own arithmetic (no top-k, no margins, no
histograms, no quantiles), so both the HIP path and the CPU oracle may take
their inputs from here.

Workloads (every generator is seeded; seed 0 unless stated):

* ``tiny``   N=1024, E=16, K=2: logits ~ N(0,1) fp32, s = sigmoid(logits), b = 0.
* ``single`` N=65536, E=256, K=6: logits = N(0,1) + per-expert offset with
  offset ~ N(0, std 0.5); b ~ U(-0.1, 0.1).
* ``skew``   N=1,048,576 (256 x 4096), E=256, K=6: per-expert offsets from a
  seeded permutation of Zipf(1.1) ranks, min-max scaled to [0, 2] (rank 1 ->
  2.0); logits = round_half_even((N(0,1) + offset) * 64) / 64 so that many
  margins collide after rounding to bf16; b ~ U(-0.2, 0.2).
* ``step``   48 layers of N=262,144, E=256, K=6; layer l draws from
  ``default_rng([0, l])``: mu_l ~ U(-1,1), b_l ~ U(-0.1,0.1), logits ~ N(mu_l, 1).
* ``stream`` a sequence of batches for the closed-loop bias controller:
  batch t draws logits N(0,1) + fixed per-expert Zipf(1.1) offsets scaled to
  [0, 2] (layer l's offsets from ``default_rng([seed, 1000 + l])``, noise
  from ``default_rng([seed, t, l])``); the bias is the controller's own state.
* ``router`` hidden bf16 [262144 x 2048] ~ N(0,1), router weight bf16
  [2048 x 256] ~ N(0, std 0.02) (stored [256 x 2048]), b = 0, upstream score
  gradient g ~ N(0,1) fp32, eta = 1e-5.

The model these shapes come from (256 routed experts, top-6, 48 MoE layers) is
the 7.5B testbed of "Exact Quantile Balancing and Load-Error Injection for
Mixture-of-Experts" (summary page, testbed paragraph); its score distribution
is not published, so these recipes stand in for it.

Scores are computed as float32(1 / (1 + exp(-logit))) in float64; they are
the exact bytes handed to both implementations.
"""
from __future__ import annotations

import numpy as np

WORKLOADS = {
    "tiny": dict(N=1024, E=16, K=2, L=1),
    "single": dict(N=65536, E=256, K=6, L=1),
    "skew": dict(N=1048576, E=256, K=6, L=1),
    "step": dict(N=262144, E=256, K=6, L=48),
    "router": dict(N=262144, E=256, K=6, L=1, H=2048),
    "stream": dict(N=262144, E=256, K=6, L=1, n_mb=4096),
}

_CHUNK_ROWS = 65536


def sigmoid_f32(logits) -> np.ndarray:
    """float32(1/(1+exp(-x))) evaluated in float64."""
    x = np.asarray(logits, dtype=np.float64)
    return (1.0 / (1.0 + np.exp(-x))).astype(np.float32)


def _fill_scores(out: np.ndarray, rng: np.random.Generator, offset, quant: float | None):
    """Draw standard normals row-chunk by row-chunk (the draw sequence is the
    same as one big draw) and write sigmoid(z + offset) into ``out``."""
    N, E = out.shape
    for r0 in range(0, N, _CHUNK_ROWS):
        r1 = min(N, r0 + _CHUNK_ROWS)
        z = rng.standard_normal((r1 - r0, E), dtype=np.float32).astype(np.float64)
        z += offset
        if quant is not None:
            z = np.round(z * quant) / quant  # numpy rounds half to even
        out[r0:r1] = sigmoid_f32(z)


def tiny(seed: int = 0):
    p = WORKLOADS["tiny"]
    rng = np.random.default_rng(seed)
    logits = rng.standard_normal((p["N"], p["E"]), dtype=np.float32)
    s = sigmoid_f32(logits)
    b = np.zeros(p["E"], dtype=np.float32)
    return s, b, p["K"]


def single(seed: int = 0, N: int | None = None):
    p = WORKLOADS["single"]
    N = p["N"] if N is None else N
    E = p["E"]
    rng = np.random.default_rng(seed)
    off = rng.normal(0.0, 0.5, E)
    b = rng.uniform(-0.1, 0.1, E).astype(np.float32)
    s = np.empty((N, E), dtype=np.float32)
    _fill_scores(s, rng, off, None)
    return s, b, p["K"]


def zipf_offsets(rng: np.random.Generator, E: int, a: float = 1.1, span: float = 2.0):
    ranks = rng.permutation(E).astype(np.float64) + 1.0
    w = ranks ** (-a)
    return (w - w.min()) / (w.max() - w.min()) * span


def skew(seed: int = 0, N: int | None = None, out: np.ndarray | None = None):
    p = WORKLOADS["skew"]
    N = p["N"] if N is None else N
    E = p["E"]
    rng = np.random.default_rng(seed)
    off = zipf_offsets(rng, E)
    b = rng.uniform(-0.2, 0.2, E).astype(np.float32)
    s = np.empty((N, E), dtype=np.float32) if out is None else out
    _fill_scores(s, rng, off, 64.0)
    return s, b, p["K"]


def step_layer(layer: int, N: int | None = None, out: np.ndarray | None = None):
    p = WORKLOADS["step"]
    N = p["N"] if N is None else N
    E = p["E"]
    rng = np.random.default_rng([0, layer])
    mu = rng.uniform(-1.0, 1.0)
    b = rng.uniform(-0.1, 0.1, E).astype(np.float32)
    s = np.empty((N, E), dtype=np.float32) if out is None else out
    _fill_scores(s, rng, mu, None)
    return s, b, p["K"]


def stream_batch(step: int, N: int, E: int, L: int = 1, seed: int = 0):
    """Scores [L, N, E] of batch `step` of the controller stream; layer l
    uses its own fixed offsets (``default_rng([seed, 1000 + l])``)."""
    out = np.empty((L, N, E), dtype=np.float32)
    for l in range(L):
        off = zipf_offsets(np.random.default_rng([seed, 1000 + l]), E)
        _fill_scores(out[l], np.random.default_rng([seed, step, l]), off, None)
    return out


def router(seed: int = 0, N: int | None = None, H: int | None = None, E: int | None = None):
    """Returns (hidden_bf16_bits uint16 [N,H], w_bf16_bits uint16 [E,H], b, g, K, eta).

    The router weight is drawn as [H, E] and stored transposed, [E, H] (the
    nn.Linear weight layout; logits = hidden @ w.T).  bf16 values are float32
    draws rounded to nearest-even (torch's CPU cast)."""
    import torch

    p = WORKLOADS["router"]
    N = p["N"] if N is None else N
    H = p["H"] if H is None else H
    E = p["E"] if E is None else E
    rng = np.random.default_rng(seed)
    w = rng.normal(0.0, 0.02, (H, E)).astype(np.float32)
    hidden = np.empty((N, H), dtype=np.uint16)
    for r0 in range(0, N, _CHUNK_ROWS // 4):
        r1 = min(N, r0 + _CHUNK_ROWS // 4)
        x = rng.standard_normal((r1 - r0, H), dtype=np.float32)
        hidden[r0:r1] = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    wb = np.ascontiguousarray(
        torch.from_numpy(w).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16).T)
    g = np.empty((N, E), dtype=np.float32)
    for r0 in range(0, N, _CHUNK_ROWS):
        r1 = min(N, r0 + _CHUNK_ROWS)
        g[r0:r1] = rng.standard_normal((r1 - r0, E), dtype=np.float32)
    b = np.zeros(E, dtype=np.float32)
    return hidden, wb, b, g, p["K"], np.float32(1e-5)


def random_case(seed: int, N: int, E: int, K: int, quant: float | None = None,
                bias_scale: float = 0.1, offset_std: float = 0.5):
    """Small generic case for parity sweeps: logits N(0,1) + N(0, offset_std)
    per expert, optionally quantised to 1/quant; b ~ U(-bias_scale, bias_scale)."""
    rng = np.random.default_rng([seed, N, E, K])
    off = rng.normal(0.0, offset_std, E) if offset_std > 0 else np.zeros(E)
    b = rng.uniform(-bias_scale, bias_scale, E).astype(np.float32) if bias_scale > 0 \
        else np.zeros(E, dtype=np.float32)
    s = np.empty((N, E), dtype=np.float32)
    _fill_scores(s, rng, off, quant)
    return s, b, K
