"""Benchmark of the exact quantile-balancing (EQB) bias update on one MI355X.

A step is one full EQB layer update of the skewed 1,048,576-token workload
(E=256, K=6): pass 1 (alpha + high-byte histogram), the high-byte select,
pass 2 (low-byte partial histograms) and the low-byte select with the
bias update and the in-place reset of the high-byte histogram.  Pass 1
reads the layer's bias and the select writes b_next into a second buffer
(the update reads q only, never the old bias), so every step is the same
update with no copy between steps.  Inputs are
resident in HBM before timing starts, and the untimed warm-up steps run for
at least 50 ms (after idle the clocks settle over tens of milliseconds of
load).  The timed steps run back to back from one HIP graph that holds all
of them.

Printed: one JSON line with the metric (tokens/s per layer), the roofline
of the dominant kernel (algorithmic bytes / average duration from HIP events
around each launch on its stream) and the CPU oracle timed on a bounded
sample of the same workload.  --suite adds the 65,536-token layer (EQB and
K3) and the 48-layer step.
"""
from __future__ import annotations

import argparse
import json
import os
import platform
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_HBM_GBS = 8000.0  # MI355X HBM3E, vendor figure


def log(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def cpu_model():
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return platform.processor()


class EqbStep:
    """Device state of one EQB layer update and its launch sequence."""

    def __init__(self, s, b0, K, qb, torch, L=None, ws=True):
        self.qb, self.torch = qb, torch
        self.s, self.b0, self.K = s, b0, K
        lead = s.dim() == 3
        N, E = s.shape[-2], s.shape[-1]
        Lx = s.shape[0] if lead else 1
        self.N = N
        # b0 is the bias pass 1 routes with; b receives b_next.  Kept apart,
        # every step computes the same update from the same input.
        self.b = b0.clone()
        self.alpha = torch.empty(((Lx,) if lead else ()) + (N,), dtype=torch.float32, device=s.device)
        self.buf = qb.EqbBuffers(Lx, E, device=s.device, lead=lead)
        # Pass 2 merges its histogram either through a workspace of per-
        # workgroup partials (default) or with global atomics.
        self.ws = (torch.empty(qb.qb_hist_lo_workspace_bytes(Lx, N, E), dtype=torch.uint8, device=s.device)
                   if ws else None)

    def launches(self):
        """(name, callable) of the step, in stream order.  The workspace
        step clears the high-byte histogram in its last select (the reset
        after the update), so it needs no separate clear; the atomic step
        clears both histograms with a fill kernel first."""
        qb, buf = self.qb, self.buf
        body = [
            ("pass1_topk_hist_hi", lambda: qb.qb_margins_topk(self.s, self.b0, self.K, self.alpha,
                                                              hist_hi=buf.hist_hi)),
            ("select_hi", lambda: qb.qb_select_update(qb.QB_SELECT_HI, self.K, buf.hist_hi,
                                                      sel_hi=buf.sel_hi, rank_lo=buf.rank_lo,
                                                      err=buf.err)),
        ]
        if self.ws is not None:
            return body + [
                ("pass2_hist_lo", lambda: qb.qb_radix_hist_lo_ws(self.s, self.alpha, buf.sel_hi, self.ws)),
                ("select_lo", lambda: qb.qb_select_lo_ws(self.N, self.ws, buf.sel_hi, buf.rank_lo, buf.q,
                                                         self.b, buf.bounds, hist_lo=buf.hist_lo,
                                                         key_out=buf.key, err=buf.err,
                                                         hist_hi=buf.hist_hi)),
            ]
        return [("reset_hist", lambda: buf.reset())] + body + [
            ("pass2_hist_lo", lambda: qb.qb_radix_hist_lo(self.s, self.alpha, buf.sel_hi, buf.hist_lo)),
            ("select_lo", lambda: qb.qb_select_update(qb.QB_SELECT_LO, self.K, buf.hist_lo,
                                                      sel_hi=buf.sel_hi, rank_lo=buf.rank_lo,
                                                      key_out=buf.key, q_out=buf.q, b=self.b,
                                                      bounds=buf.bounds, err=buf.err)),
        ]

    def run(self):
        for _, f in self.launches():
            f()


_CLOCK = {}


def sustain_clock(torch, ms=50.0):
    """Untimed streaming reads (libstreamprobe, non-temporal, unroll 16: a
    form the ceiling sweep never times) for at least `ms` before a timed
    region that has no step of its own to warm up with (the ceilings, the
    single-kernel timings).  After a second or two of idle (data
    generation, setup) the chip's clocks settle over tens of milliseconds;
    a training job runs the update on a chip kept busy, so timings are
    taken in that settled state."""
    import time as _t
    from exact_quantile_selection_amd import stream_probe as sp
    if "buf" not in _CLOCK:
        _CLOCK["buf"] = torch.empty(1 << 28, dtype=torch.float32, device="cuda")  # 1 GiB
        _CLOCK["sink"] = torch.zeros(4096, dtype=torch.int32, device="cuda")
    torch.cuda.synchronize()
    t0 = _t.perf_counter()
    while (_t.perf_counter() - t0) * 1e3 < ms:
        for _ in range(32):
            sp.read(_CLOCK["buf"], _CLOCK["sink"], 256, 16, nontemporal=True)
        torch.cuda.synchronize()


WARM_MS = 50.0


def time_graph(step, torch, steps, warmup, before_timed=None):
    """Run `warmup` steps eagerly (more if they take under 50 ms: after
    idle the clocks settle over tens of milliseconds of the step's own load;
    pass 1 over 1 GiB ran up to 226 us per launch in the first 50 launches
    against 175-181 us once settled), capture `steps` consecutive steps in one
    HIP graph (as a training step's graph holds its layers' updates back to
    back), replay it once untimed, then time one replay: exactly `steps`
    steps between two device synchronizations.  Returns seconds per step.
    The side stream first waits for the current one, where the step's
    inputs and buffers were written (generation, zero-filled histograms).
    before_timed (optional) runs after the untimed replay: it restores state
    that the steps accumulate, so the timed replay's result does not depend
    on how many warm-up steps ran."""
    stream = torch.cuda.Stream()
    stream.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(stream):
        # at least `warmup` steps, and at least 50 ms of them: the step's
        # own load is what the clocks settle to (a plain read draws less)
        t0, n = time.perf_counter(), 0
        while n < max(1, warmup) or (time.perf_counter() - t0) * 1e3 < WARM_MS:
            for _ in range(4):
                step.run()
            n += 4
            stream.synchronize()
    _CLOCK["warm_steps"] = n
    stream.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=stream):
        for _ in range(steps):
            step.run()
    g.replay()
    if before_timed is not None:
        before_timed()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    g.replay()
    torch.cuda.synchronize()
    return (time.perf_counter() - t0) / steps, g


def time_kernels(step, torch, reps):
    """Average duration of each launch of the step: `reps` steps launched
    eagerly in step order, a HIP event recorded on the kernels' stream
    right before and right after every launch, so each kernel runs in the
    same context as in the graph (after the same predecessor).  Returns
    seconds per launch by name."""
    stream = torch.cuda.current_stream()
    names = [n for n, _ in step.launches()]
    ev = []
    for _ in range(reps):
        for n, f in step.launches():
            e0 = torch.cuda.Event(enable_timing=True)
            e1 = torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            f()
            e1.record(stream)
            ev.append((n, e0, e1))
    torch.cuda.synchronize()
    out = {n: 0.0 for n in names}
    for n, e0, e1 in ev:
        out[n] += e0.elapsed_time(e1) * 1e-3 / reps
    return out


def ceilings(torch, s, reps=10):
    """The measured streaming ceiling over the same score tensor: the plain
    read kernel of libstreamprobe (include/stream_probe.h), with cached and
    with non-temporal loads, at every (grid, unroll) of a small sweep, each
    timed with HIP events around `reps` back-to-back launches; the fastest
    is the ceiling."""
    from exact_quantile_selection_amd import stream_probe as sp
    sustain_clock(torch)

    cus = torch.cuda.get_device_properties(s.device).multi_processor_count
    nbytes = s.numel() * 4
    sink = torch.zeros(16 * cus, dtype=torch.int32, device=s.device)
    stream = torch.cuda.current_stream()

    def timed(f):
        f()
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for _ in range(reps):
            f()
        e1.record(stream)
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) * 1e-3 / reps

    sweep = {}
    for nt in (False, True):
        for per_cu in (1, 2, 4, 8, 16):
            for u in (2, 4, 8):
                sec = timed(lambda: sp.read(s, sink, per_cu * cus, u, nontemporal=nt))
                sweep[f"{'nontemporal,' if nt else ''}grid={per_cu * cus},unroll={u}"] = round(nbytes / sec / 1e9, 1)
    best = max(sweep, key=sweep.get)
    out = {"read": dict(GBps=sweep[best], us=round(nbytes / sweep[best] / 1e3, 2), bytes=nbytes, best=best,
                        frac_of_peak=round(sweep[best] / PEAK_HBM_GBS, 4), sweep=sweep)}
    out["copy"] = copy_ceiling(torch, s.view(-1)[: s.numel() // 2], reps)
    return out


def copy_ceiling(torch, src, reps=10):
    """The measured ceiling of a stream that reads and writes equal amounts:
    libstreamprobe's plain copy of `src` into a buffer of the same size at a
    few (grid, unroll), HIP events around `reps` back-to-back launches;
    GB/s counts the bytes read plus the bytes written."""
    from exact_quantile_selection_amd import stream_probe as sp
    sustain_clock(torch)

    cus = torch.cuda.get_device_properties(src.device).multi_processor_count
    dst = torch.empty_like(src)
    moved = 2 * src.numel() * src.element_size()
    stream = torch.cuda.current_stream()
    sweep = {}
    for per_cu in (1, 2, 4, 8):
        for u in (2, 4):
            f = lambda: sp.copy(src, dst, per_cu * cus, u)
            f()
            e0 = torch.cuda.Event(enable_timing=True)
            e1 = torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            for _ in range(reps):
                f()
            e1.record(stream)
            torch.cuda.synchronize()
            sweep[f"grid={per_cu * cus},unroll={u}"] = round(moved / (e0.elapsed_time(e1) * 1e-3 / reps) / 1e9, 1)
    assert torch.equal(dst, src)
    del dst
    best = max(sweep, key=sweep.get)
    return dict(GBps=sweep[best], us=round(moved / sweep[best] / 1e3, 2), bytes_moved=moved, best=best,
                frac_of_peak=round(sweep[best] / PEAK_HBM_GBS, 4), sweep=sweep)


def cpu_baseline(s_np, b_np, K, rows):
    from oracle import oracle

    if not os.path.exists(oracle.LIB):
        oracle.build()
    sample = np.ascontiguousarray(s_np[:rows])
    t0 = time.perf_counter()
    oracle.eqb_layer(sample, b_np, K)
    dt = time.perf_counter() - t0
    return dict(value=rows / dt, unit="tokens/s", cores=1, kind="oracle",
                sample=f"first {rows} of {s_np.shape[0]} tokens of the skewed workload; full "
                       f"oracle EQB layer update (alpha, bf16 keys, per-expert sort-and-pick, "
                       f"histograms, b_next), single thread, {dt:.1f} s on {cpu_model()} "
                       f"(nproc={os.cpu_count()})")


KERNEL_SOURCES = ("qb_device.hpp", "qb_pass1.hip", "qb_radix.hip")


def kernel_source_hash():
    """Hash of the sources of the two streaming passes."""
    import hashlib

    h = hashlib.sha256()
    for f in KERNEL_SOURCES:
        with open(os.path.join(ROOT, "exact_quantile_selection_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def measured_traffic(kernel):
    """HBM bytes per launch of `kernel` from the committed rocprofv3 counter
    summary (FETCH_SIZE + WRITE_SIZE, each scaled by the same counter on a
    plain copy of known size), or None when that summary is missing or was
    taken on different kernel sources."""
    path = os.path.join(ROOT, "profiles", "traffic_skew_N1048576_E256.txt")
    if not os.path.exists(path):
        return None
    kv = {}
    for line in open(path):
        if "=" in line and not line.startswith("#"):
            k, v = line.split("=", 1)
            kv[k.strip()] = v.strip()
    if kv.get("kernel_source_hash") != kernel_source_hash():
        return None
    v = kv.get(f"{kernel}.hbm_bytes")
    return float(v) if v else None


def bytes_per_token(E):
    """Algorithmic HBM bytes per token of one EQB layer: two reads of the
    E fp32 scores (one per pass), alpha written once and read once."""
    return dict(pass1=4 * E + 4, pass2=4 * E + 4, step=8 * E + 8)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--suite", action="store_true", help="also time the other workloads")
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle baseline")
    ap.add_argument("--contrast", action="store_true",
                    help="also time the step with pass 2 merged by global atomics")
    ap.add_argument("--cpu-rows", type=int, default=1048576)
    ap.add_argument("--router", action="store_true",
                    help="time only the fused-router workload and print its JSON line")
    ap.add_argument("--only", default=None,
                    help="time only this workload of the suite and print its JSON line "
                         "(single, step_48_layers, router, controller, sharding, "
                         "one_pass_full_hist, k3_skew, lei_backward, calibration)")
    args = ap.parse_args()
    if args.only and args.only not in SUITES:
        print(f"unknown workload {args.only!r}; one of {', '.join(SUITES)}", file=sys.stderr)
        sys.exit(2)
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (got --gpus {args.gpus}); the update shards over "
              "tokens with one histogram all-reduce per pass, which this library does not implement.",
              file=sys.stderr)
        sys.exit(2)

    import torch

    from exact_quantile_selection_amd import qb, synth

    qb.lib()
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)

    only = "router" if args.router else args.only
    if only:
        log(f"{only} workload")
        print(json.dumps({"workload": only, only: SUITES[only](torch, qb, synth, dev, args)}), flush=True)
        return

    p = synth.WORKLOADS["skew"]
    N, E, K = p["N"], p["E"], p["K"]
    log(f"generating skew workload N={N} E={E} K={K}")
    s_np, b_np, _ = synth.skew()
    s = torch.from_numpy(s_np).to(dev)
    b0 = torch.from_numpy(b_np).to(dev)
    step = EqbStep(s, b0, K, qb, torch)

    log("timing")
    torch.cuda.synchronize()
    sec, _graph = time_graph(step, torch, args.steps, args.warmup)
    assert int(step.buf.err.item()) == 0
    b_ws = step.b.clone()
    del _graph
    per_k = time_kernels(step, torch, args.steps)
    contrast = None
    if args.contrast:
        # The same step with pass 2 merged by global atomics, for contrast.
        atomic = EqbStep(s, b0, K, qb, torch, ws=False)
        sec_atomic, _graph = time_graph(atomic, torch, args.steps, args.warmup)
        assert int(atomic.buf.err.item()) == 0 and torch.equal(atomic.b, b_ws)
        per_k_atomic = time_kernels(atomic, torch, args.steps)
        del _graph, atomic
        contrast = {"step_us": round(sec_atomic * 1e6, 2),
                    "pass2_us": round(per_k_atomic["pass2_hist_lo"] * 1e6, 2),
                    "select_lo_us": round(per_k_atomic["select_lo"] * 1e6, 2), "same_b_next": True}
    ceil = ceilings(torch, s)

    bpt = bytes_per_token(E)
    dominant = max(("pass1_topk_hist_hi", "pass2_hist_lo"), key=lambda n: per_k[n])
    dom_bytes = N * bpt["pass1" if dominant.startswith("pass1") else "pass2"]
    achieved = dom_bytes / per_k[dominant] / 1e9
    kernels = {n: dict(us=round(t * 1e6, 2)) for n, t in per_k.items()}
    for n, key in (("pass1_topk_hist_hi", "pass1"), ("pass2_hist_lo", "pass2")):
        kernels[n]["GBps"] = round(N * bpt[key] / per_k[n] / 1e9, 1)
    step_gbs = N * bpt["step"] / sec / 1e9

    out = {
        "metric": "EQB tokens/s per layer at E=256,K=6; achieved HBM GB/s vs peak",
        "value": N / sec,
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup, "warmup_steps_run": _CLOCK.get("warm_steps"),
        "ms_per_step": sec * 1e3,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "config": {"workload": "skew: N=1048576 tokens (256 x 4096), E=256, K=6, one layer, EQB",
                   "N": N, "E": E, "K": K, "L": 1, "launch": f"hip_graph ({args.steps} steps per graph)",
                   "step_algorithmic_bytes": N * bpt["step"],
                   "step_GBps": round(step_gbs, 1),
                   "step_frac_of_peak": round(step_gbs / PEAK_HBM_GBS, 4)},
        "roofline": {"bound": "hbm", "kernel": dominant, "achieved": round(achieved, 1),
                     "peak": PEAK_HBM_GBS, "unit": "GB/s", "frac": round(achieved / PEAK_HBM_GBS, 4),
                     "traffic": measured_traffic(dominant),
                     "traffic_source": "profiles/traffic_skew_N1048576_E256.txt (rocprofv3 FETCH_SIZE + "
                                       "WRITE_SIZE per dispatch, calibrated on a copy of known size; null "
                                       "when the pass sources changed since)",
                     "avg_launch_us": round(per_k[dominant] * 1e6, 2),
                     "timing": f"HIP events around each launch on its stream, {args.steps} eager steps in "
                               "step order after the timed graph replay (both after at least 50 ms of "
                               "untimed warm-up steps that settle the clocks)",
                     "frac_of_measured_read_ceiling": round(achieved / ceil["read"]["GBps"], 4),
                     "algorithmic_bytes_per_launch": dom_bytes},
        "kernels": kernels,
        "stream_ceilings": ceil,
    }

    if contrast:
        out["pass2_global_atomics_step"] = contrast
    if args.suite:
        out["suite"] = suite(torch, qb, synth, dev, args)

    if not args.no_cpu:
        log(f"cpu baseline on {args.cpu_rows} tokens")
        out["cpu_baseline"] = cpu_baseline(s_np, b_np, K, args.cpu_rows)
    print(json.dumps(out), flush=True)


def single_suite(torch, qb, synth, dev, args):
    """The 65,536-token layer (64 MiB of scores: they fit in the 256 MB
    Infinity Cache), EQB and K3, each step from one graph."""
    res = {}
    s_np, b_np, K = synth.single()
    N, E = s_np.shape
    s = torch.from_numpy(s_np).to(dev)
    b0 = torch.from_numpy(b_np).to(dev)
    st = EqbStep(s, b0, K, qb, torch)
    sec, _ = time_graph(st, torch, args.steps, args.warmup)
    res["single_eqb"] = dict(N=N, us_per_step=round(sec * 1e6, 2), tokens_per_s=N / sec,
                             effective_GBps=round(N * (8 * E + 8) / sec / 1e9, 1))
    bounds0 = torch.zeros(2, dtype=torch.float32, device=dev)
    qb.qb_bias_bounds(b0, bounds0)
    b = b0.clone()
    bounds = bounds0.clone()
    alpha = torch.empty(N, dtype=torch.float32, device=dev)
    hist_u = torch.zeros((E, 1000), dtype=torch.int32, device=dev)
    q_u = torch.zeros(E, dtype=torch.float32, device=dev)
    ws_u = torch.empty(qb.qb_uniform_hist_workspace_bytes(1, N, E, 1000), dtype=torch.uint8, device=dev)

    class K3Step:
        """K3 through the workspace merge (at this size the atomic flush of
        256 small tables is a larger tail than storing them); `atomic`
        selects the histogram merged with global atomics instead."""

        def __init__(self_, atomic=False):
            self_.atomic = atomic

        def run(self_):
            # the select reads the bounds it bins over, then writes the next
            # range: restored for every step; the bias is read from b0 and
            # b_next written to b
            bounds.copy_(bounds0)
            if self_.atomic:
                qb.qb_fill_i32(hist_u, 0)
                qb.k3_update(s, b, K, alpha, bounds, hist_u, q_u, b_in=b0)
            else:
                qb.k3_update_ws(s, b, K, alpha, bounds, ws_u, q_u, b_in=b0)

    sec, _ = time_graph(K3Step(), torch, args.steps, args.warmup)
    b_ws = b.clone()
    sec_atomic, _ = time_graph(K3Step(atomic=True), torch, args.steps, args.warmup)
    assert torch.equal(b, b_ws)
    res["single_k3"] = dict(N=N, n_bins=1000, us_per_step=round(sec * 1e6, 2), tokens_per_s=N / sec,
                            effective_GBps=round(N * (8 * E + 8) / sec / 1e9, 1),
                            merge="workspace", us_per_step_atomic_merge=round(sec_atomic * 1e6, 2),
                            same_b_next=True)
    del s, st
    torch.cuda.empty_cache()
    return res


def step48_suite(torch, qb, synth, dev, args):
    """The 48-layer step on device-generated scores of the same recipe
    (layer-batched launches, 12 GiB of scores)."""
    p = synth.WORKLOADS["step"]
    L, N, E, K = p["L"], p["N"], p["E"], p["K"]
    g = torch.Generator(device=dev)
    g.manual_seed(0)
    mu = torch.rand((L, 1, 1), generator=g, device=dev) * 2 - 1
    s = torch.empty((L, N, E), dtype=torch.float32, device=dev)
    for l in range(L):
        s[l].normal_(generator=g)
        s[l].add_(mu[l]).sigmoid_()
    b0 = (torch.rand((L, E), generator=g, device=dev) * 0.2 - 0.1).contiguous()
    st = EqbStep(s, b0, K, qb, torch)
    sec, _ = time_graph(st, torch, max(3, args.steps // 4), 1)
    out = dict(L=L, N=N, ms_per_step=round(sec * 1e3, 3), tokens_per_s_per_layer=L * N / sec,
               GBps=round(L * N * (8 * E + 8) / sec / 1e9, 1))
    del s, st
    torch.cuda.empty_cache()
    return out


def suite(torch, qb, synth, dev, args):
    res = single_suite(torch, qb, synth, dev, args)
    for name, f in SUITES.items():
        if name not in ("single", "calibration"):
            res[name] = f(torch, qb, synth, dev, args)
    return res


def lei_backward_suite(torch, qb, synth, dev, args):
    """Per-microbatch LEI (unbounded and bounded) with the gradient through
    the sigmoid at the router shape: 262,144 x 256 scores, 4096-token
    microbatches; reads g and s, writes g' and dlogits (16 B per score)."""
    N, E, K, n_mb = 262144, 256, 6, 4096
    g = torch.Generator(device=dev)
    g.manual_seed(0)
    grad = torch.randn((N, E), generator=g, device=dev)
    s = torch.sigmoid(torch.randn((N, E), generator=g, device=dev))
    load = torch.randint(0, 2 * n_mb * K // E, (N // n_mb, E), generator=g, device=dev, dtype=torch.int32)
    gout = torch.empty_like(grad)
    d = torch.empty_like(grad)
    out = dict(N=N, E=E, K=K, n_mb=n_mb, bytes_per_launch=16 * N * E)
    sustain_clock(torch)
    for bounded in (False, True):
        f = lambda: qb.qb_lei_backward(grad, load, K, n_mb, 1e-5, bounded=bounded, s=s, g_out=gout, dlogits=d)
        f()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(10):
            f()
        e1.record()
        torch.cuda.synchronize()
        us = e0.elapsed_time(e1) * 1e3 / 10
        out["bounded_us" if bounded else "unbounded_us"] = round(us, 2)
        out["bounded_GBps" if bounded else "unbounded_GBps"] = round(16 * N * E / us / 1e3, 1)
    del grad, s, gout, d
    torch.cuda.empty_cache()
    # the ceiling of a stream that reads 512 MiB and writes 512 MiB, as one
    # launch of this kernel does: the plain copy of the stream probe
    src = torch.ones(2 * N * E, dtype=torch.float32, device=dev)
    ceil = copy_ceiling(torch, src)
    del src
    torch.cuda.empty_cache()
    out["copy_ceiling"] = ceil
    for k in ("unbounded", "bounded"):
        out[f"{k}_frac_of_copy_ceiling"] = round(out[f"{k}_GBps"] / ceil["GBps"], 4)
    return out


def full_hist_suite(torch, qb, synth, dev, args):
    """The one-pass alternative on the skewed 1M-token layer: clear the
    65,536-bin histogram, alpha + full-key histogram in one pass over s, the
    quantile read from the 65,536 bins and the bias update; compared with
    the two-pass EQB step on the same layer (same result bit for bit)."""
    s_np, b_np, K = synth.skew()
    N, E = s_np.shape
    s = torch.from_numpy(s_np).to(dev)
    b0 = torch.from_numpy(b_np).to(dev)
    b = b0.clone()
    alpha = torch.empty(N, dtype=torch.float32, device=dev)
    hist = torch.zeros((E, 65536), dtype=torch.int32, device=dev)
    key = torch.zeros(E, dtype=torch.uint16, device=dev)
    q = torch.zeros(E, dtype=torch.float32, device=dev)
    bounds = torch.zeros(2, dtype=torch.float32, device=dev)
    err = torch.zeros(1, dtype=torch.int32, device=dev)

    class OnePass:
        def run(self_):
            qb.qb_fill_i32(hist, 0)
            qb.qb_margins_full_hist(s, b0, K, alpha, hist)
            qb.qb_select_update(qb.QB_SELECT_FULL, K, hist, key_out=key, q_out=q, b=b, bounds=bounds, err=err)

    sec, _ = time_graph(OnePass(), torch, max(5, args.steps // 2), 2)
    assert int(err.item()) == 0
    two = EqbStep(s, b0, K, qb, torch)
    sec2, _ = time_graph(two, torch, max(5, args.steps // 2), 2)
    same = bool(torch.equal(b, two.b))
    out = dict(N=N, E=E, K=K, one_pass_us=round(sec * 1e6, 2), two_pass_us=round(sec2 * 1e6, 2),
               one_pass_hist_MiB=E * 65536 * 4 / 2**20, two_pass_hist_MiB=2 * E * 256 * 4 / 2**20,
               same_b_next=same,
               note="one pass reads s once but makes one device atomic per score into a 64 MiB histogram")
    del s, hist
    torch.cuda.empty_cache()
    return out


def k3_skew_suite(torch, qb, synth, dev, args):
    """The K3 mode on the skewed 1M-token layer (1000 uniform bins over the
    bias range): the alpha pass, the binning pass over the same 1 GiB of
    scores, the interpolating select and the bias update, from one graph
    (merged through the workspace, and for comparison by global atomics);
    the atomic binning pass alone from HIP events around back-to-back
    launches."""
    s_np, b_np, K = synth.skew()
    N, E = s_np.shape
    s = torch.from_numpy(s_np).to(dev)
    b0 = torch.from_numpy(b_np).to(dev)
    bounds0 = torch.zeros(2, dtype=torch.float32, device=dev)
    qb.qb_bias_bounds(b0, bounds0)
    b, bounds = b0.clone(), bounds0.clone()
    alpha = torch.empty(N, dtype=torch.float32, device=dev)
    hist_u = torch.zeros((E, 1000), dtype=torch.int32, device=dev)
    q = torch.zeros(E, dtype=torch.float32, device=dev)
    err = torch.zeros(1, dtype=torch.int32, device=dev)

    ws_u = torch.empty(qb.qb_uniform_hist_workspace_bytes(1, N, E, 1000), dtype=torch.uint8, device=dev)

    class K3Step:
        """K3 with the histogram merged through the workspace (`ws`), or by
        global atomics into a zeroed histogram."""

        def __init__(self_, ws=True):
            self_.ws = ws

        def run(self_, i=0):
            # bounds restored (the select reads them, then writes the next
            # range); the bias is read from b0 and b_next written to b
            bounds.copy_(bounds0)
            if self_.ws:
                qb.k3_update_ws(s, b, K, alpha, bounds, ws_u, q, err=err, b_in=b0)
            else:
                qb.qb_fill_i32(hist_u, 0)
                qb.k3_update(s, b, K, alpha, bounds, hist_u, q, err=err, b_in=b0)

    sec, _ = time_graph(K3Step(), torch, max(5, args.steps // 2), 2)
    assert int(err.item()) == 0
    b_ws = b.clone()
    sec_atomic, _ = time_graph(K3Step(ws=False), torch, max(5, args.steps // 2), 2)
    assert int(err.item()) == 0 and torch.equal(b, b_ws)
    del ws_u
    f = lambda: qb.qb_uniform_hist(s, alpha, bounds, hist_u)
    f()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(10):
        f()
    e1.record()
    torch.cuda.synchronize()
    bin_us = e0.elapsed_time(e1) * 1e3 / 10
    out = dict(N=N, E=E, K=K, n_bins=1000, us_per_step=round(sec * 1e6, 2), tokens_per_s=N / sec,
               merge="workspace", us_per_step_atomic_merge=round(sec_atomic * 1e6, 2), same_b_next=True,
               step_GBps=round(N * (8 * E + 8) / sec / 1e9, 1), binning_pass_us=round(bin_us, 2),
               binning_pass_GBps=round(N * (4 * E + 4) / bin_us / 1e3, 1))
    del s, hist_u
    torch.cuda.empty_cache()
    return out


def sharding_suite(torch, qb, synth, dev, args, R=8):
    """EQB over R emulated ranks vs rank-averaged QB on the skewed 1M-token
    layer (R = 8 ranks of 131,072 tokens): stream times of both updates, the
    largest difference between their biases, and the global MaxVio of the
    same batch routed with each bias (and with the incoming bias)."""
    from exact_quantile_selection_amd.shard import ShardedUpdate

    s_np, b_np, K = synth.skew()
    N, E = s_np.shape
    s = torch.from_numpy(s_np).to(dev)
    b0 = torch.from_numpy(b_np).to(dev)
    sh = ShardedUpdate(R, N, E, K, device=dev)

    def timed(f, n=5):
        sustain_clock(torch)
        f()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(n):
            f()
        e1.record()
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) * 1e3 / n

    t_eqb = timed(lambda: sh.eqb(s, b0))
    b_eqb = sh.b[0].clone()
    t_avg = timed(lambda: sh.rank_averaged(s, b0))
    b_avg = sh.b_avg.clone()
    # heterogeneous ranks: the same tokens ordered by their preferred expert,
    # so each rank sees a different mix (as ranks fed different data do)
    s_het = s[torch.argsort(torch.argmax(s + b0, dim=1), stable=True)].contiguous()
    sh.eqb(s_het, b0)
    b_eqb_het = sh.b[0].clone()
    sh.rank_averaged(s_het, b0)
    b_avg_het = sh.b_avg.clone()
    torch.cuda.synchronize()
    alpha = torch.empty(N, dtype=torch.float32, device=dev)
    load = torch.zeros((1, 1, E), dtype=torch.int32, device=dev)
    mv = torch.empty((1, 1), dtype=torch.float32, device=dev)

    def maxvio(bias):
        load.zero_()
        qb.qb_margins_topk(s, bias, K, alpha, load=load.view(E))
        qb.qb_maxvio(load, K, N, mv)
        return round(float(mv.item()), 4)

    out = dict(N=N, E=E, K=K, ranks=R, tokens_per_rank=N // R,
               eqb_sharded_us=round(t_eqb, 2), rank_averaged_us=round(t_avg, 2),
               max_abs_bias_difference=float((b_avg - b_eqb).abs().max().item()),
               global_maxvio={"incoming_bias": maxvio(b0), "eqb": maxvio(b_eqb),
                              "rank_averaged": maxvio(b_avg)},
               heterogeneous_ranks={
                   "eqb_bias_unchanged": bool(torch.equal(b_eqb_het, b_eqb)),
                   "max_abs_bias_difference": float((b_avg_het - b_eqb).abs().max().item()),
                   "global_maxvio": {"eqb": maxvio(b_eqb_het), "rank_averaged": maxvio(b_avg_het)}},
               note="timings include the per-rank bias copies and histogram resets of the emulation")
    del s, s_het, sh
    torch.cuda.empty_cache()
    return out


def controller_suite(torch, qb, synth, dev, args, T=8):
    """Closed-loop bias controller on the batch stream (262,144 tokens x 256
    experts, K = 6, 4096-token microbatches): each step routes a fresh batch
    with the current bias, measures global / local MaxVio and replaces the
    bias by the batch's EQB update.  The batches follow synth.stream_batch's
    recipe, drawn on the device with torch's seeded generator."""
    import numpy as np
    from exact_quantile_selection_amd.controller import BiasController

    p = synth.WORKLOADS["stream"]
    N, E, K, n_mb = p["N"], p["E"], p["K"], p["n_mb"]
    off = torch.from_numpy(synth.zipf_offsets(np.random.default_rng([0, 1000]), E)).to(dev, torch.float32)
    g = torch.Generator(device=dev)
    g.manual_seed(0)
    batches = [torch.sigmoid(torch.randn((N, E), generator=g, device=dev) + off) for _ in range(T)]
    ctl = BiasController(1, N, E, K, n_mb, device=dev)
    traj = []
    for t in range(T):
        ctl.step(batches[t])
        traj.append((ctl.worst_global.clone(), ctl.worst_local.clone()))
    torch.cuda.synchronize()
    # timing: the T closed-loop steps from one graph (eager launching of the
    # dozen small calls per step would measure the host), from a zero bias
    stream = torch.cuda.Stream()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph, stream=stream):
        for t in range(T):
            ctl.step(batches[t])
    ctl.b.zero_()
    graph.replay()
    torch.cuda.synchronize()
    same = bool(torch.equal(ctl.worst_global, traj[-1][0]))
    # untimed replays of the same closed loop for at least 50 ms (the clocks
    # settle over tens of milliseconds of load after idle)
    tw = time.perf_counter()
    while (time.perf_counter() - tw) * 1e3 < WARM_MS:
        ctl.b.zero_()
        graph.replay()
        torch.cuda.synchronize()
    ctl.b.zero_()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    graph.replay()
    torch.cuda.synchronize()
    step_us = (time.perf_counter() - t0) * 1e6 / T
    del graph
    out = dict(N=N, E=E, K=K, n_mb=n_mb, steps=T,
               step_us=round(step_us, 2), graph_replay_matches_eager=same,
               global_maxvio=[round(float(a[0]), 4) for a, _ in traj],
               local_maxvio_mean=[round(float(b[1]), 4) for _, b in traj],
               local_maxvio_max=[round(float(b[0]), 4) for _, b in traj],
               step=("pass 1 (alpha, hist_hi), select HI, pass 2 (hist_lo partials, loads, microbatch "
                     "loads), 2 x MaxVio, select LO (b updated in place)" if ctl.loads_in_pass2 else
                     "pass 1 (alpha, loads, microbatch loads, hist_hi), select HI, pass 2, 2 x MaxVio, "
                     "select LO (b updated in place)"))
    del batches
    torch.cuda.empty_cache()
    return out


def router_suite(torch, qb, synth, dev, args):
    """Fused-router workload: hidden [262144 x 2048] bf16 x w [256 x 2048]
    bf16 on MFMA + sigmoid + pass 1 (qb_router_fused), then the rest of the
    EQB update on the produced scores and the LEI gradient offset."""
    p = synth.WORKLOADS["router"]
    N, H, E, K = p["N"], p["H"], p["E"], p["K"]
    g = torch.Generator(device=dev)
    g.manual_seed(0)
    hidden = torch.randn((N, H), generator=g, device=dev).to(torch.bfloat16)
    w = (torch.randn((E, H), generator=g, device=dev) * 0.02).to(torch.bfloat16)
    grad0 = torch.randn((N, E), generator=g, device=dev)
    grad = grad0.clone()
    b0 = torch.zeros(E, dtype=torch.float32, device=dev)
    b = b0.clone()
    s = torch.empty((N, E), dtype=torch.float32, device=dev)
    alpha = torch.empty(N, dtype=torch.float32, device=dev)
    load = torch.zeros(E, dtype=torch.int32, device=dev)
    buf = qb.EqbBuffers(1, E, device=dev, lead=False)

    def reps(f, n):
        f()
        torch.cuda.synchronize()
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(n):
            f()
        e1.record()
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) * 1e-3 / n

    n = max(3, args.steps // 2)
    hist = buf.hist_hi
    sustain_clock(torch)
    # pass 1 fused into the GEMM's epilogue, against the GEMM alone followed
    # by the standalone pass 1 over the scores it wrote (same results)
    t_fused = reps(lambda: qb.qb_router_fused(hidden, w, b, K, s, alpha, load=load, hist_hi=hist), n)
    t_gemm = reps(lambda: qb.qb_router_scores(hidden, w, s), n)
    t_pass1 = reps(lambda: qb.qb_margins_topk(s, b, K, alpha, load=load, hist_hi=hist), n)
    qb.qb_fill_i32(hist, 0)
    qb.qb_fill_i32(load, 0)
    # the vendor GEMM (torch.mm, hipBLASLt) for comparison: bf16 output
    # (half the score bytes) and fp32 output as the scores need, the latter
    # also with a separate sigmoid
    vendor = {}
    wt = w.t()
    vendor["bf16_out"] = reps(lambda: torch.mm(hidden, wt), n)
    try:
        s32 = torch.empty((N, E), dtype=torch.float32, device=dev)
        vendor["fp32_out"] = reps(lambda: torch.mm(hidden, wt, out_dtype=torch.float32), n)
        vendor["fp32_out_then_sigmoid"] = reps(
            lambda: torch.sigmoid(torch.mm(hidden, wt, out_dtype=torch.float32), out=s32), n)
        del s32
    except (RuntimeError, TypeError) as e:  # out_dtype not supported by this PyTorch
        vendor["fp32_out_error"] = str(e)[:120]
    torch.cuda.empty_cache()

    ws = torch.empty(qb.qb_hist_lo_workspace_bytes(1, N, E), dtype=torch.uint8, device=dev)

    class Chain:
        """Router forward, the EQB update and LEI; pass 1 either in the
        GEMM's epilogue (fused) or as its own pass over the scores, and the
        top-K loads counted in pass 1 or in the low-byte pass."""

        def __init__(self_, fused, loads_in_pass2=False):
            self_.fused = fused
            self_.p2 = loads_in_pass2

        def run(self_):
            # routed with b0; the select writes b_next to b
            qb.qb_fill_i32(load, 0)
            l1 = None if self_.p2 else load
            if self_.fused:
                qb.qb_router_fused(hidden, w, b0, K, s, alpha, load=l1, hist_hi=buf.hist_hi)
            else:
                qb.qb_router_scores(hidden, w, s)
                qb.qb_margins_topk(s, b0, K, alpha, load=l1, hist_hi=buf.hist_hi)
            qb.qb_select_update(qb.QB_SELECT_HI, K, buf.hist_hi, sel_hi=buf.sel_hi,
                                rank_lo=buf.rank_lo, err=buf.err)
            if self_.p2:
                qb.qb_radix_hist_lo_ws_loads(s, alpha, buf.sel_hi, ws, b0, K, load)
            else:
                qb.qb_radix_hist_lo_ws(s, alpha, buf.sel_hi, ws)
            qb.qb_select_lo_ws(N, ws, buf.sel_hi, buf.rank_lo, buf.q, b, buf.bounds, key_out=buf.key,
                               err=buf.err, hist_hi=buf.hist_hi)  # clears hist_hi for the next run
            qb.qb_lei_grad(grad, load, K, 1e-5)

    chains = {}
    b_ref = g_ref = None
    for name, fused, p2 in (("fused", True, False), ("unfused", False, False),
                            ("fused_loads_in_pass2", True, True), ("unfused_loads_in_pass2", False, True)):
        chains[name], _ = time_graph(Chain(fused, p2), torch, n, 1, before_timed=lambda: grad.copy_(grad0))
        if b_ref is None:
            b_ref, g_ref = b.clone(), grad.clone()
        assert torch.equal(b, b_ref), name
        assert torch.equal(grad, g_ref), name
    sec, sec_unfused = chains["fused"], chains["unfused"]
    flops = 2.0 * N * H * E
    gemm_bytes = N * H * 2 + N * E * 4 + E * H * 2
    out = dict(N=N, H=H, E=E, K=K,
               fused_gemm_pass1_us=round(t_fused * 1e6, 2),
               gemm_sigmoid_us=round(t_gemm * 1e6, 2),
               pass1_on_scores_us=round(t_pass1 * 1e6, 2),
               unfused_gemm_plus_pass1_us=round((t_gemm + t_pass1) * 1e6, 2),
               gemm_mfma_TFLOPs=round(flops / t_gemm / 1e12, 1),
               gemm_mfma_frac_of_2500=round(flops / t_gemm / 2.5e15, 4),
               gemm_hbm_GBps=round(gemm_bytes / t_gemm / 1e9, 1),
               fused_hbm_GBps=round(gemm_bytes / t_fused / 1e9, 1),
               chain_fused_us=round(sec * 1e6, 2), chain_fused_tokens_per_s=N / sec,
               chain_unfused_us=round(sec_unfused * 1e6, 2), chain_unfused_tokens_per_s=N / sec_unfused,
               chain_fused_loads_in_pass2_us=round(chains["fused_loads_in_pass2"] * 1e6, 2),
               chain_unfused_loads_in_pass2_us=round(chains["unfused_loads_in_pass2"] * 1e6, 2),
               chain_same_b_next_and_lei=True,
               vendor_gemm_us={k: (round(v * 1e6, 2) if isinstance(v, float) else v) for k, v in vendor.items()},
               chain="router GEMM + sigmoid, pass 1 (in the GEMM's epilogue, or after it), select HI, "
                     "pass 2, select LO, LEI; one graph of the steps",
               timing="HIP events around back-to-back launches of each call")
    del hidden, w, grad, grad0, s
    torch.cuda.empty_cache()
    return out


def calibration_suite(torch, qb, synth, dev, args):
    """Kernels of known traffic for calibrating the rocprofv3 FETCH_SIZE and
    WRITE_SIZE counters: a plain torch copy of 1 GiB (1 GiB read, 1 GiB
    written) and the stream probe's read of 1 GiB (1 GiB read)."""
    from exact_quantile_selection_amd import stream_probe as sp

    n = 1 << 28  # floats: 1 GiB
    src = torch.ones(n, dtype=torch.float32, device=dev)
    dst = torch.empty_like(src)
    sink = torch.zeros(4096, dtype=torch.int32, device=dev)
    cus = torch.cuda.get_device_properties(dev).multi_processor_count
    for _ in range(3):
        dst.copy_(src)
        sp.read(src, sink, 2 * cus, 4)
    torch.cuda.synchronize()
    del src, dst
    torch.cuda.empty_cache()
    return dict(copy_bytes_read=4 * n, copy_bytes_written=4 * n, read_bytes=4 * n, launches_each=3)


SUITES = {
    "single": single_suite,
    "step_48_layers": step48_suite,
    "router": router_suite,
    "controller": controller_suite,
    "sharding": sharding_suite,
    "one_pass_full_hist": full_hist_suite,
    "k3_skew": k3_skew_suite,
    "lei_backward": lei_backward_suite,
    "calibration": calibration_suite,
}


if __name__ == "__main__":
    main()
