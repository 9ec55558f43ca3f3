"""Host-side checks of the C ABI that need no GPU: the library loads, exports
exactly what include/qb.h declares, and rejects bad arguments with the
documented status codes before touching the device."""
import ctypes as C
import os
import re
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "qb.h")
LIB = os.path.join(ROOT, "exact_quantile_selection_amd", "libqb.so")


@pytest.fixture(scope="module")
def libqb():
    if not os.path.exists(LIB):
        from exact_quantile_selection_amd import build

        build.build()
    import torch  # noqa: F401  (the binding always loads torch's HIP runtime first)

    from exact_quantile_selection_amd import qb

    return qb.lib()


def declared_functions():
    text = open(HEADER).read()
    return sorted(set(re.findall(r"QB_API\s+[\w\s\*]+?\b(qb_\w+)\s*\(", text)))


def test_header_declares_the_boundary():
    names = declared_functions()
    for n in ("qb_margins_topk", "qb_radix_hist_hi", "qb_radix_hist_lo", "qb_select_update",
              "qb_uniform_hist", "qb_status_string"):
        assert n in names


def test_library_exports_every_declared_symbol(libqb):
    for n in declared_functions():
        assert hasattr(libqb, n), n
    out = subprocess.run(["nm", "-D", "--defined-only", LIB], capture_output=True, text=True).stdout
    exported = sorted(set(re.findall(r" T (qb_\w+)", out)))
    assert exported == declared_functions()


def _last(libqb):
    return libqb.qb_last_error().decode()


def test_invalid_arguments_are_rejected_without_launch(libqb):
    from exact_quantile_selection_amd import qb

    fake = 0x1000  # never dereferenced: validation fails first
    rc = libqb.qb_margins_topk(None, fake, 1, 1024, 256, 6, fake, None, None, None)
    assert rc == qb.QB_EINVAL and "s is NULL" in _last(libqb)
    rc = libqb.qb_margins_topk(fake, fake, 1, 1024, 48, 6, fake, None, None, None)
    assert rc == qb.QB_EUNSUPPORTED and "E=48" in _last(libqb)
    rc = libqb.qb_margins_topk(fake, fake, 1, 1024, 256, 16, fake, None, None, None)
    assert rc == qb.QB_EUNSUPPORTED and "K=16" in _last(libqb) and "K <= 15" in _last(libqb)
    rc = libqb.qb_margins_topk(fake, fake, 1, 1024, 16, 16, fake, None, None, None)
    assert rc == qb.QB_EINVAL and "K=16" in _last(libqb)
    rc = libqb.qb_margins_topk(fake + 4, fake, 1, 1024, 256, 6, fake, None, None, None)
    assert rc == qb.QB_EINVAL and "16-byte aligned" in _last(libqb)
    rc = libqb.qb_margins_topk(fake, fake, 1, 0, 256, 6, fake, None, None, None)
    assert rc == qb.QB_EINVAL and "N=0" in _last(libqb)
    rc = libqb.qb_margins_topk(fake, fake, 0, 10, 256, 6, fake, None, None, None)
    assert rc == qb.QB_EINVAL and "L=0" in _last(libqb)
    rc = libqb.qb_radix_hist_lo(fake, fake, 1, 10, 256, None, fake, None)
    assert rc == qb.QB_EINVAL and "sel_hi" in _last(libqb)
    rc = libqb.qb_select_update(7, 1, 256, 6, fake, 256, fake, fake, None, None, fake, fake, None, None)
    assert rc == qb.QB_EINVAL and "phase=7" in _last(libqb)
    rc = libqb.qb_select_update(qb.QB_SELECT_LO, 1, 256, 6, fake, 256, fake, fake, None, None, None,
                                fake, None, None)
    assert rc == qb.QB_EINVAL and "[L=1][E=256]" in _last(libqb)
    rc = libqb.qb_select_update(qb.QB_SELECT_UNIFORM, 1, 256, 6, fake, 4096, None, None, None, fake,
                                fake, fake, None, None)
    assert rc == qb.QB_EINVAL and "n_bins=4096" in _last(libqb)
    rc = libqb.qb_select_update(qb.QB_SELECT_UNIFORM, 1, 256, 6, fake, 1000, None, None, None, None,
                                fake, fake, None, None)
    assert rc == qb.QB_EINVAL and "q_out" in _last(libqb)
    rc = libqb.qb_uniform_hist(fake, fake, 1, 10, 256, None, 1000, fake, None)
    assert rc == qb.QB_EINVAL
    rc = libqb.qb_lei_grad(fake, fake, 10, 100, 6, C.c_float(1e-5), None)
    assert rc == qb.QB_EUNSUPPORTED
    rc = libqb.qb_margin_keys(fake, fake, 1, 10, 256, fake + 2, None)
    assert rc == qb.QB_EINVAL and "8-byte aligned" in _last(libqb)
    rc = libqb.qb_microbatch_loads(fake, fake, 1, 1000, 256, 6, 300, fake, fake, None)
    assert rc == qb.QB_EINVAL and "divide N=1000" in _last(libqb)
    rc = libqb.qb_microbatch_loads(fake, fake, 1, 1024, 256, 6, 256, fake, None, None)
    assert rc == qb.QB_EINVAL and "[C=4][E=256]" in _last(libqb)
    rc = libqb.qb_margins_topk_mb(fake, fake, 1, 1024, 256, 6, fake, None, None, 256, fake, None)
    assert rc == qb.QB_EINVAL and "load (int32" in _last(libqb)
    rc = libqb.qb_maxvio(fake, 1, 4, 256, 300, 1024, fake, None, None, None)
    assert rc == qb.QB_EINVAL and "K=300" in _last(libqb)
    rc = libqb.qb_maxvio(fake, 1, 4, 256, 6, 1024, None, None, None, None)
    assert rc == qb.QB_EINVAL and "maxvio" in _last(libqb)
    libqb.qb_hist_lo_workspace_bytes.restype = C.c_int64
    assert libqb.qb_hist_lo_workspace_bytes(1, 1 << 20, 256) > 0
    assert libqb.qb_hist_lo_workspace_bytes(1, 1 << 20, 48) == qb.QB_EINVAL
    assert libqb.qb_hist_lo_workspace_bytes(0, 10, 256) == qb.QB_EINVAL
    rc = libqb.qb_radix_hist_lo_ws(fake, fake, 1, 1024, 256, fake, None, C.c_int64(0), None)
    assert rc == qb.QB_EINVAL and "ws are required" in _last(libqb)
    rc = libqb.qb_radix_hist_lo_ws(fake, fake, 1, 1024, 256, fake, fake, C.c_int64(16), None)
    assert rc == qb.QB_EINVAL and "ws_bytes=16" in _last(libqb)
    rc = libqb.qb_radix_hist_lo_ws(fake, fake, 1, 1024, 256, fake, fake + 4, C.c_int64(1 << 30), None)
    assert rc == qb.QB_EINVAL and "16-byte aligned" in _last(libqb)
    rc = libqb.qb_select_lo_ws(1, C.c_int64(1024), 48, fake, C.c_int64(1 << 30), fake, fake, None, None, fake,
                               None, None, None, None, None)
    assert rc == qb.QB_EUNSUPPORTED and "E=48" in _last(libqb)
    rc = libqb.qb_select_lo_ws(1, C.c_int64(1024), 256, fake, C.c_int64(16), fake, fake, None, None, fake,
                               fake, fake, None, None, None)
    assert rc == qb.QB_EINVAL and "ws_bytes=16" in _last(libqb)
    assert [libqb.qb_radix_lo_trip_rows(e) for e in (16, 32, 64, 128, 256)] == [2048, 1024, 512, 256, 256]
    assert libqb.qb_radix_lo_trip_rows(48) == qb.QB_EUNSUPPORTED
    assert libqb.qb_fill_i32(None, 0, 0, None) == qb.QB_OK  # empty fill is a no-op
    assert libqb.qb_fill_i32(None, 5, 0, None) == qb.QB_EINVAL
    for st in (0, -1, -2, -3):
        assert libqb.qb_status_string(st).startswith(b"QB_")


def test_misaligned_element_arrays_are_rejected(libqb):
    """float and int32 arrays must sit on 4-byte and the uint16 keys on
    2-byte boundaries; a pointer off by one element part is refused before
    any launch."""
    from exact_quantile_selection_amd import qb

    fake = 0x1000  # never dereferenced: validation fails first
    rc = libqb.qb_select_update(qb.QB_SELECT_LO, 1, 256, 6, fake, 256, fake + 2, fake, None, fake, fake, fake,
                                None, None)
    assert rc == qb.QB_EINVAL and "4-byte aligned" in _last(libqb)
    rc = libqb.qb_select_update(qb.QB_SELECT_LO, 1, 256, 6, fake, 256, fake, fake, fake + 1, fake, fake, fake,
                                None, None)
    assert rc == qb.QB_EINVAL and "key_out must be 2-byte aligned" in _last(libqb)
    rc = libqb.qb_select_lo_ws(1, C.c_int64(1024), 256, fake, C.c_int64(1 << 30), fake, fake, None, None, fake,
                               fake + 1, fake, None, None, None)
    assert rc == qb.QB_EINVAL and "4-byte aligned" in _last(libqb)
    rc = libqb.qb_radix_hist_lo(fake, fake + 2, 1, 10, 256, fake, fake, None)
    assert rc == qb.QB_EINVAL and "4-byte aligned" in _last(libqb)
    rc = libqb.qb_uniform_hist(fake, fake, 1, 10, 256, fake + 3, 1000, fake, None)
    assert rc == qb.QB_EINVAL and "4-byte aligned" in _last(libqb)
    rc = libqb.qb_bias_bounds(fake + 2, 1, 256, fake, None)
    assert rc == qb.QB_EINVAL and "4-byte aligned" in _last(libqb)
    rc = libqb.qb_lei_grad(fake, fake + 2, 10, 256, 6, C.c_float(1e-5), None)
    assert rc == qb.QB_EINVAL and "4-byte aligned" in _last(libqb)


def test_binding_fails_loudly_without_library(monkeypatch):
    from exact_quantile_selection_amd import qb

    monkeypatch.setattr(qb, "_lib", None)
    monkeypatch.setattr(qb, "LIB_PATH", "/nonexistent/libqb.so")
    with pytest.raises(RuntimeError, match="not built"):
        qb.lib()


def test_product_code_never_touches_the_oracle():
    """The package (library sources and binding) neither imports, links nor
    loads anything under oracle/."""
    pkg = os.path.join(ROOT, "exact_quantile_selection_amd")
    pat = re.compile(r"(from\s+oracle|import\s+oracle|liboracle|qb_oracle|oracle/)")
    for dirpath, _, files in os.walk(pkg):
        for f in files:
            if f.endswith((".py", ".hip", ".hpp", ".cpp", ".h")):
                text = open(os.path.join(dirpath, f)).read()
                assert not pat.search(text), f


PROBE_HEADER = os.path.join(ROOT, "include", "stream_probe.h")
PROBE_LIB = os.path.join(ROOT, "exact_quantile_selection_amd", "libstreamprobe.so")


def test_stream_probe_exports_its_header():
    """The diagnostic streaming library exports exactly what its header
    declares and rejects bad arguments without a launch."""
    if not os.path.exists(PROBE_LIB):
        from exact_quantile_selection_amd import build

        build.build_probe()
    declared = sorted(set(re.findall(r"SP_API\s+[\w\s\*]+?\b(sp_\w+)\s*\(", open(PROBE_HEADER).read())))
    assert declared == ["sp_copy", "sp_read", "sp_read_nt"]
    out = subprocess.run(["nm", "-D", "--defined-only", PROBE_LIB], capture_output=True, text=True).stdout
    assert sorted(set(re.findall(r" T (sp_\w+)", out))) == declared
    import torch  # noqa: F401

    from exact_quantile_selection_amd import stream_probe

    L = stream_probe.lib()
    fake = 0x1000  # never dereferenced: validation fails first
    assert L.sp_read(None, 1024, 1, 8, fake, None) == -1
    assert L.sp_read(fake, 1000, 1, 8, fake, None) == -1    # not a multiple of 16
    assert L.sp_read(fake + 4, 1024, 1, 8, fake, None) == -1  # misaligned
    assert L.sp_read(fake, 1024, 1, 5, fake, None) == -1    # unroll
    assert L.sp_read(fake, 1024, 0, 8, fake, None) == -1    # grid
    assert L.sp_read_nt(fake, 1000, 1, 8, fake, None) == -1  # not a multiple of 16
    assert L.sp_read_nt(fake, 1024, 1, 3, fake, None) == -1    # unroll
    assert L.sp_copy(fake, None, 1024, 1, 4, None) == -1
    assert L.sp_copy(fake, fake + 512, 1024, 1, 4, None) == -1  # overlapping
    assert L.sp_copy(fake, fake + 4096, 1024, 1, 16, None) == -1  # unroll
    assert L.sp_copy(fake, fake + 4100, 1024, 1, 4, None) == -1  # misaligned


def test_noalloc_rejects_a_layer_beyond_its_scratch(libqb):
    """qb_radix_lo_select_noalloc refuses a shape whose single layer needs
    more than its 64 MiB scratch, before any launch or device lookup."""
    from exact_quantile_selection_amd import qb

    N, E = 30_000_000, 256
    assert libqb.qb_hist_lo_workspace_bytes(1, N, E) > qb.QB_NOALLOC_SCRATCH_BYTES
    fake = 0x1000  # never dereferenced: validation fails first
    rc = libqb.qb_radix_lo_select_noalloc(fake, fake, 1, N, E, fake, fake, None, None, fake, fake, fake, None,
                                          None, None)
    assert rc == qb.QB_EINVAL and "scratch" in _last(libqb) and "qb_radix_hist_lo_ws" in _last(libqb)
    rc = libqb.qb_radix_lo_select_noalloc(fake, None, 1, 1024, E, fake, fake, None, None, fake, fake, fake,
                                          None, None, None)
    assert rc == qb.QB_EINVAL and "required" in _last(libqb)


def test_router_entry_points_reject_bad_shapes(libqb):
    """qb_router_fused and qb_router_scores refuse unsupported shapes before
    any launch."""
    from exact_quantile_selection_amd import qb

    fake = 0x1000  # never dereferenced: validation fails first
    rc = libqb.qb_router_scores(fake, fake, 1024, 100, 256, fake, None, None)
    assert rc == qb.QB_EINVAL and "H=100" in _last(libqb)
    rc = libqb.qb_router_scores(fake, fake, 1024, 128, 48, fake, None, None)
    assert rc == qb.QB_EUNSUPPORTED and "E=48" in _last(libqb)
    rc = libqb.qb_router_scores(fake + 2, fake, 1024, 128, 256, fake, None, None)
    assert rc == qb.QB_EINVAL and "aligned" in _last(libqb)
    rc = libqb.qb_router_fused(fake, fake, 1024, 128, 256, 16, fake, fake, None, fake, None, None, None)
    assert rc == qb.QB_EUNSUPPORTED and "K=16" in _last(libqb)
    rc = libqb.qb_router_fused(fake, fake, 1024, 128, 256, 6, fake, fake, None, fake, None, fake + 4, None)
    assert rc == qb.QB_EINVAL and "8-byte" in _last(libqb)


def test_pass2_loads_rejects_bad_arguments(libqb):
    """qb_radix_hist_lo_ws_loads refuses a missing load, K out of range and
    microbatches that are not whole trips, before any launch."""
    from exact_quantile_selection_amd import qb

    fake = 0x1000  # never dereferenced: validation fails first
    N, E = 8192, 16
    wsb = libqb.qb_hist_lo_workspace_bytes(1, N, E)
    rc = libqb.qb_radix_hist_lo_ws_loads(fake, fake, 1, N, E, fake, fake, wsb, fake, 2, None, 1, None, None)
    assert rc == qb.QB_EINVAL and "load" in _last(libqb)
    rc = libqb.qb_radix_hist_lo_ws_loads(fake, fake, 1, N, E, fake, fake, wsb, fake, 16, fake, 1, None, None)
    assert rc == qb.QB_EINVAL and "K=16" in _last(libqb)
    rc = libqb.qb_radix_hist_lo_ws_loads(fake, fake, 1, N, E, fake, fake, wsb, fake, 2, fake, 1024, fake, None)
    assert rc == qb.QB_EINVAL and "multiple of 2048" in _last(libqb)
    rc = libqb.qb_radix_hist_lo_ws_loads(fake, fake, 1, N, 256, fake, fake,
                                         libqb.qb_hist_lo_workspace_bytes(1, N, 256), fake, 6, fake, 3000, fake,
                                         None)
    assert rc == qb.QB_EINVAL and "n_mb=3000" in _last(libqb)
    rc = libqb.qb_radix_hist_lo_ws_loads(fake, fake, 1, N, E, fake, fake, wsb - 1, fake, 2, fake, 1, None, None)
    assert rc == qb.QB_EINVAL and "ws_bytes" in _last(libqb)


def test_k3_workspace_entry_points_reject_bad_arguments(libqb):
    """The K3 workspace pair refuses bad bin counts, a short or unaligned
    workspace and K out of range, before any launch."""
    from exact_quantile_selection_amd import qb

    fake = 0x1000  # never dereferenced: validation fails first
    N, E = 65536, 256
    assert libqb.qb_uniform_hist_workspace_bytes(1, N, E, 0) == qb.QB_EINVAL
    assert libqb.qb_uniform_hist_workspace_bytes(1, N, E, 2049) == qb.QB_EINVAL
    wsb = libqb.qb_uniform_hist_workspace_bytes(1, N, E, 1000)
    assert wsb > 0
    rc = libqb.qb_uniform_hist_ws(fake, fake, 1, N, E, fake, 1000, fake, wsb - 1, None)
    assert rc == qb.QB_EINVAL and "ws_bytes" in _last(libqb)
    rc = libqb.qb_uniform_hist_ws(fake, fake, 1, N, E, fake, 1000, fake + 4, wsb, None)
    assert rc == qb.QB_EINVAL and "16-byte" in _last(libqb)
    rc = libqb.qb_select_uniform_ws(1, N, E, 0, 1000, fake, wsb, None, fake, fake, fake, None, None)
    assert rc == qb.QB_EINVAL and "K=0" in _last(libqb)
    rc = libqb.qb_select_uniform_ws(1, N, 48, 6, 1000, fake, wsb, None, fake, fake, fake, None, None)
    assert rc == qb.QB_EUNSUPPORTED and "E=48" in _last(libqb)
    rc = libqb.qb_select_uniform_ws(1, N, E, 6, 1000, fake, wsb - 1, None, fake, fake, fake, None, None)
    assert rc == qb.QB_EINVAL and "ws_bytes" in _last(libqb)
