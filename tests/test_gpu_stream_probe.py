"""The diagnostic streaming kernels (include/stream_probe.h) whose rates are
the measured ceilings the bench reports: the copy reproduces its source
byte for byte at every unroll, including a ragged tail shorter than one
trip, and the read runs to completion at every unroll."""
import pytest
import torch

from exact_quantile_selection_amd import stream_probe as sp

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("unroll", [1, 2, 4, 8])
@pytest.mark.parametrize("n16", [1, 1023, 1024 * 8 + 5, 1 << 20])
def test_copy_reproduces_the_source(unroll, n16):
    g = torch.Generator(device="cuda")
    g.manual_seed(n16 + unroll)
    src = torch.randint(-2**31, 2**31 - 1, (4 * n16,), generator=g, device="cuda", dtype=torch.int32)
    # dst sits between two 256-byte guard bands of the same allocation
    big = torch.full((4 * n16 + 128,), 7, dtype=torch.int32, device="cuda")
    dst = big[64:64 + 4 * n16]
    sp.copy(src, dst, 3, unroll)
    torch.cuda.synchronize()
    assert torch.equal(dst, src)
    assert int((big[:64] != 7).sum()) == 0 and int((big[-64:] != 7).sum()) == 0


@pytest.mark.parametrize("nt", [False, True])
@pytest.mark.parametrize("unroll", [1, 2, 4, 8, 16])
def test_read_completes(unroll, nt):
    t = torch.ones(1 << 22, dtype=torch.float32, device="cuda")
    sink = torch.zeros(512, dtype=torch.int32, device="cuda")
    sp.read(t, sink, 512, unroll, nontemporal=nt)
    torch.cuda.synchronize()
    assert int(sink.abs().sum()) == 0  # the fold of all-ones data never hits the sink's trigger value
