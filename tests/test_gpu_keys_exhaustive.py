"""Every fp32 bit pattern through the GPU's margin -> bf16 -> key path,
against the oracle (which is itself pinned to torch's bf16 cast)."""
import numpy as np
import pytest
import torch

from exact_quantile_selection_amd import qb

import gpu_util as G

pytestmark = pytest.mark.gpu


@pytest.mark.timeout(900)
def test_all_fp32_patterns(O):
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    E = 16
    chunk = 1 << 26
    rows = chunk // E
    alpha = torch.zeros(rows, dtype=torch.float32, device=G.DEV)
    keys = torch.empty((rows, E), dtype=torch.uint16, device=G.DEV)
    a_host = np.zeros(chunk, np.float32)
    G.say("exhaustive fp32 -> key, 64 chunks")
    for c in range(1 << 32 >> 26):
        x = (np.arange(chunk, dtype=np.uint64) + np.uint64(c * chunk)).astype(np.uint32)
        nan = (((x >> 23) & 0xFF) == 0xFF) & ((x & 0x7FFFFF) != 0)
        x[nan] = 0  # NaN is outside the domain
        xf = x.view(np.float32)
        s_np = -xf  # margin r = 0 - s = x exactly for every non-zero x
        s = torch.from_numpy(s_np.reshape(rows, E)).to(G.DEV)
        qb.qb_margin_keys(s, alpha, keys)
        got = keys.cpu().numpy().ravel()
        want = O.margin_keys(s_np.reshape(chunk, 1), a_host)[0]
        if not np.array_equal(got, want):
            idx = np.nonzero(got != want)[0][:5]
            raise AssertionError(f"chunk {c}: patterns {x[idx].tolist()} got {got[idx]} want {want[idx]}")
        if c % 16 == 0:
            G.say(f"chunk {c} ok")
