#!/usr/bin/env python3
"""Throughput of the speculative-sampling verification step on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W]

A step is one spec_verify call (row statistics, decision, draw sums, locate)
over one batch of synthetic logits already resident in HBM. The default run
is a parent process that never touches the GPU: it starts one child process
per workload (c3, c4, c5, in that order), each of which times K steps after
W warm-up steps, and prints ONE JSON line. The headline is c5, the largest
configuration; every workload reports its per-call fraction of peak HBM
bandwidth (algorithmic bytes per step / ms per step / 8 TB/s), the row
kernel's own fraction (k_rowstats, timed with HIP events the library records
around it on the launch stream, on every --event-every'th timed step), and a
CPU baseline: the fp64 oracle timed on the host cores on the same batch,
whose outputs also give the flagged fraction of that batch's draws.

    python bench.py --workload cN [--extras]
runs one workload in this process (what each child runs; use it under a
profiler). --extras adds the other entry points on the same batch (early
exit always; top-p, top-k, tree and prompt lookup with --extras).

    python bench.py --copy-probe BYTES
runs a plain device copy of known size (the calibration for rocprofv3 HBM
counters) and exits.
"""
from __future__ import annotations

import argparse
import ctypes
import json
import os
import subprocess
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "verified draft positions/sec (B*(k+1)/s) + achieved HBM GB/s vs peak, 1 GPU"
PEAK_HBM_GBPS = 8000.0  # MI355X HBM3E, AMD specification
WORKLOADS = ("c3", "c4", "c5")  # the configurations with a bandwidth target
SMALL_STEPS = 100  # timed steps at least, for the workloads other than the headline
HEADLINE = "c5"
CHUNK_BYTES = 32 * 1024  # the library's row-statistics chunk (one k_draw workgroup)


EVENT_EVERY = 4  # set from --event-every


def counters_file(workload: str) -> str:
    return os.path.join(ROOT, "profiles", f"k_rowstats_{workload}_hbm_counters.txt")


def log(msg: str) -> None:
    print(msg, file=sys.stderr, flush=True)


def hip_runtime():
    import torch

    cands = [os.path.join(os.path.dirname(torch.__file__), "lib", "libamdhip64.so"),
             "libamdhip64.so.7", "libamdhip64.so"]
    for c in cands:
        try:
            lib = ctypes.CDLL(c)
            break
        except OSError:
            continue
    else:
        raise RuntimeError("HIP runtime not found")
    lib.hipEventCreate.argtypes = [ctypes.POINTER(ctypes.c_void_p)]
    lib.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.c_void_p,
                                        ctypes.c_void_p]
    lib.hipEventSynchronize.argtypes = [ctypes.c_void_p]
    lib.hipEventDestroy.argtypes = [ctypes.c_void_p]
    return lib


class HipEvents:
    """K pairs of raw hipEvent_t handles for the library to record into,
    owned in one place: ``close`` destroys them and drops the handles, so a
    handle can never reach the library after its event is gone (recording
    into a destroyed event is a use-after-free inside the HIP runtime)."""

    def __init__(self, hip, K: int):
        self.hip = hip
        self.pairs = [(ctypes.c_void_p(), ctypes.c_void_p()) for _ in range(K)]
        for a, b in self.pairs:
            assert hip.hipEventCreate(ctypes.byref(a)) == 0
            assert hip.hipEventCreate(ctypes.byref(b)) == 0

    def pair(self, i: int):
        if self.pairs is None:
            raise RuntimeError("HIP events used after close()")
        a, b = self.pairs[i]
        return a.value, b.value

    def elapsed_ms(self, K: int) -> list:
        return elapsed_ms(self.hip, [self.pair(i) for i in range(K)], K)

    def close(self):
        if self.pairs is not None:
            for a, b in self.pairs:
                self.hip.hipEventDestroy(a)
                self.hip.hipEventDestroy(b)
            self.pairs = None

    def __enter__(self):
        return self

    def __exit__(self, *exc):
        self.close()


def kernel_source_digest() -> str:
    from speculative_decoding_verification_11_amd.build import source_digest

    return source_digest()


def counter_summary(workload: str) -> dict:
    """The machine-readable lines of the workload's committed rocprofv3
    counter summary (empty if there is none)."""
    path = counters_file(workload)
    kv = {}
    if os.path.exists(path):
        for line in open(path):
            if ":" in line and not line.startswith("#") and not line.startswith(" "):
                key, _, val = line.partition(":")
                kv[key.strip()] = val.strip()
    return kv


def read_counter_traffic(workload: str):
    """HBM bytes per row-statistics launch from the committed rocprofv3
    counter summary of this workload, if it was taken on the current kernel
    source."""
    kv = counter_summary(workload)
    if kv.get("kernel_source_sha256_16") != kernel_source_digest() or kv.get("workload") != workload:
        return None
    try:
        return int(float(kv["hbm_bytes_per_launch"]))
    except (KeyError, ValueError):
        return None


def read_kernel_traffic(*kernels: str, workload: str = HEADLINE):
    """Scaled HBM bytes (read + written) per dispatch of the named kernels
    from the workload's committed counter summary, if it was taken on the
    current kernel source; else None."""
    if read_counter_traffic(workload) is None:
        return None
    out = {}
    for line in open(counters_file(workload)):
        cells = [c.strip() for c in line.strip().strip("|").split("|")]
        if len(cells) == 5 and cells[0] in kernels:
            try:
                out[cells[0]] = int(float(cells[3]) + float(cells[4]))
            except ValueError:
                pass
    return out or None


def copy_probe(nbytes: int, reps: int = 5) -> None:
    import torch

    n = nbytes // 4
    src = torch.ones(n, dtype=torch.float32, device="cuda")
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    for _ in range(reps):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"copy_probe_bytes": n * 4, "reps": reps}), flush=True)


def cpu_model() -> str:
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def cpu_baseline(batch, seed: int, nseq: int, gpu_out: dict) -> dict:
    """The oracle on the host cores: the batch (up to nseq sequences) on every
    core this process may use (at most 16 threads), and a 64-sequence slice
    on one thread; each the median of three runs.
    The oracle's outputs of the first run are compared with the GPU's outputs
    of the same batch and seed: the flagged fraction of the batch's draws
    (oracle margin below 1e-6, or below a final draw's wider fp32-resolution
    band), how many flagged draws the two sides decided differently, and
    whether any draw outside the band differs."""
    import oracle
    from oracle import parity
    from speculative_decoding_verification_11_amd import workloads as wl

    nthreads = parity.host_threads(cap=16)
    visible = len(os.sched_getaffinity(0))
    first = {}

    def median_time(host, nt, keep=False):
        times = []
        for _ in range(3):
            t0 = time.perf_counter()
            res = oracle.spec_verify_ref(host["target"], host["draft"], host["draft_tokens"],
                                         host["draft_len"], host["temperature"], seed,
                                         seq_base=0, nthreads=nt)
            times.append(time.perf_counter() - t0)
            if keep and not first:
                first.update(res)
        return sorted(times)[1]

    sample = batch.select(range(min(nseq, batch.B)))
    hs = wl.to_host_arrays(sample)
    dt = median_time(hs, nthreads, keep=True)
    positions = sample.B * (sample.k + 1)
    one = batch.select(range(min(64, batch.B)))
    dt1 = median_time(wl.to_host_arrays(one), 1)
    rows = list(range(sample.B))
    gpu = {key: v[:sample.B] for key, v in gpu_out.items()}
    rep = parity.compare(gpu, first, hs["draft_len"], hs["temperature"], sample.k, rows=rows)
    return {"value": positions / dt, "unit": "positions/s", "cores": nthreads, "kind": "oracle",
            "sample": f"first {sample.B} of {batch.B} sequences of the same batch "
                      f"({positions} positions), fp64 C oracle, {nthreads} threads "
                      f"({visible} CPUs visible to the process), "
                      f"median of 3: {dt:.2f} s wall",
            "value_1_thread": one.B * (one.k + 1) / dt1,
            "sample_1_thread": f"first {one.B} sequences, one thread, median of 3: "
                               f"{dt1:.2f} s wall",
            "cpu_model": cpu_model(),
            "parity": {"sequences": rep.sequences, "draws": rep.draws,
                       "flagged": rep.flagged, "flagged_fraction": rep.flagged_fraction,
                       "flagged_wide": rep.flagged_wide,
                       "flagged_disagree": rep.flagged_disagree,
                       "max_abs_dS": rep.max_abs_dS, "max_rel_dS_large": rep.max_rel_dS_large,
                       "mismatches": len(rep.mismatches),
                       "note": "GPU outputs of the timed batch and seed against this oracle "
                               "run; flagged = oracle margin below 1e-6, or below a final "
                               "draw's fp32-resolution band where that is wider "
                               "(flagged_wide)"}}


def roof(achieved_gbps: float, what: str) -> dict:
    """HBM roofline of an extra entry point: bytes read once over `what`."""
    return {"bound": "hbm", "achieved": achieved_gbps, "peak": PEAK_HBM_GBPS, "unit": "GB/s",
            "frac": achieved_gbps / PEAK_HBM_GBPS, "over": what}


def timed_oracle(fn, units: float, unit: str, sample: str) -> dict:
    from oracle import parity

    nthreads = parity.host_threads(cap=16)
    t0 = time.perf_counter()
    fn(nthreads)
    dt = time.perf_counter() - t0
    return {"value": units / dt, "unit": unit, "cores": nthreads, "kind": "oracle",
            "sample": f"{sample}, {nthreads} threads, {dt:.2f} s wall"}


def sampled(i: int) -> bool:
    """Timed steps that carry a kernel event pair."""
    return i % EVENT_EVERY == 0


def elapsed_ms(hip, ev, K: int) -> list:
    """Durations of the sampled steps' event pairs, sorted."""
    ms = []
    for i in range(K):
        if sampled(i):
            m = ctypes.c_float()
            assert hip.hipEventElapsedTime(ctypes.byref(m), ev[i][0], ev[i][1]) == 0
            ms.append(m.value)
    return sorted(ms)


def bench_tree(ev: HipEvents, K: int, W: int, cpu: bool) -> dict:
    """Greedy tree verification on workload t3: nodes per second, and the
    node-row kernel's bandwidth (each node row read once, HIP events)."""
    import torch
    import speculative_decoding_verification_11_amd as sv
    from speculative_decoding_verification_11_amd import workloads as wl

    tw = wl.TREE_WORKLOADS["t3"]
    log(f"[bench] tree: generating {tw.name}: {tw.description}")
    tb = wl.generate_tree(tw, "cuda:0")
    ws = torch.empty(sv.tree_workspace_size(tw.B, tw.N, tw.V, tw.dtype_code), dtype=torch.uint8,
                     device="cuda:0")
    out = (torch.empty((tw.B, tw.N), dtype=torch.int32, device="cuda:0"),
           torch.empty((tw.B, tw.N), dtype=torch.int32, device="cuda:0"),
           torch.empty((tw.B,), dtype=torch.int32, device="cuda:0"))

    def step(events=None):
        sv.spec_verify_tree(tb.target, tb.parents, tb.tokens, tb.n_nodes, workspace=ws, out=out,
                            events=events)

    for _ in range(W):
        step()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(K):
        step(events=ev.pair(i) if sampled(i) else None)
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    ms = ev.elapsed_ms(K)
    row_mean = sum(ms) / len(ms)
    nodes = int(tb.n_nodes.sum())
    nbytes = tb.bytes_read()
    ms_step = elapsed * 1e3 / K
    res = {"entry_point": "spec_verify_tree", "workload": f"{tw.name}: {tw.description}",
           "value": nodes / (ms_step * 1e-3), "unit": "nodes/s", "ms_per_step": ms_step,
           "bytes_read_once": nbytes, "row_kernel": "k_tree_rowstats",
           "row_kernel_us_mean": row_mean * 1e3,
           "row_kernel_GBps": nbytes / (row_mean * 1e-3) / 1e9,
           "mean_accepted_depth": float(out[2].float().mean()),
           "roofline": roof(nbytes / (row_mean * 1e-3) / 1e9, "k_tree_rowstats, HIP events"),
           "hbm_bytes_per_dispatch": read_kernel_traffic("k_tree_rowstats", "k_tree_decide")}
    if cpu:
        import oracle

        n_cpu = tw.B
        th = wl.tree_to_host_arrays(wl.TreeBatch(tw, tb.target[:n_cpu], tb.parents[:n_cpu],
                                                 tb.tokens[:n_cpu], tb.n_nodes[:n_cpu]))
        res["cpu_baseline"] = timed_oracle(
            lambda nt: oracle.spec_tree_ref(th["target"], th["parents"], th["tokens"],
                                            th["n_nodes"], nthreads=nt),
            n_cpu * tw.N, "nodes/s", f"all {tw.B} trees of the same batch, fp64 C oracle")
    log(f"[bench] tree {ms_step:.4f} ms/step; rows {row_mean * 1e3:.1f} us "
        f"({res['row_kernel_GBps']:.0f} GB/s)")
    return res


LOOKUP_BLOCK = 512 * 8  # candidate ends per block of the backward scan (lanes x loads)


def lookup_scanned_bytes(ctx, lens, lw) -> int:
    """Context bytes the lookup must read: each context is scanned from its
    end in blocks of LOOKUP_BLOCK candidate ends and stops after the block
    holding the latest match of size n_max (whole context if there is none)."""
    import torch
    import speculative_decoding_verification_11_amd as sv

    _, _, mn, ms = sv.spec_prompt_lookup(ctx, lens, lw.n_min, lw.n_max, lw.k, match=True)
    T = lens.to(torch.int64).cpu()
    n = mn.to(torch.int64).cpu()
    end = ms.to(torch.int64).cpu() + n - 1  # latest end of the winning match
    e_end = torch.clamp(T - 1, min=0)
    full = n == lw.n_max
    blocks = torch.div(e_end - 1 - end, LOOKUP_BLOCK, rounding_mode="floor") + 1
    ends = torch.where(full, torch.minimum(e_end, blocks * LOOKUP_BLOCK), e_end)
    return int(ends.sum()) * 4


def bench_lookup(K: int, W: int, cpu: bool) -> dict:
    """Prompt-lookup drafting on workload p3: contexts per second and the
    kernel's bandwidth over the context tokens (one kernel per call, timed
    with torch events on the stream it is launched on)."""
    import torch
    import speculative_decoding_verification_11_amd as sv
    from speculative_decoding_verification_11_amd import workloads as wl

    lw = wl.LOOKUP_WORKLOADS["p3"]
    log(f"[bench] prompt lookup: generating {lw.name}: {lw.description}")
    ctx_np, lens_np = wl.generate_contexts(lw)
    ctx = torch.from_numpy(ctx_np).to("cuda:0")
    lens = torch.from_numpy(lens_np).to("cuda:0")
    out = (torch.empty((lw.B, lw.k), dtype=torch.int32, device="cuda:0"),
           torch.empty((lw.B,), dtype=torch.int32, device="cuda:0"))
    for _ in range(W):
        sv.spec_prompt_lookup(ctx, lens, lw.n_min, lw.n_max, lw.k, out=out)
    torch.cuda.synchronize()
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
           for _ in range(K)]
    t0 = time.perf_counter()
    for i, (a, b) in enumerate(evs):
        if sampled(i):
            a.record()
        sv.spec_prompt_lookup(ctx, lens, lw.n_min, lw.n_max, lw.k, out=out)
        if sampled(i):
            b.record()
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    k_list = [a.elapsed_time(b) for i, (a, b) in enumerate(evs) if sampled(i)]
    k_ms = sum(k_list) / len(k_list)
    nbytes = int(lens.to(torch.int64).sum()) * 4
    scanned = lookup_scanned_bytes(ctx, lens, lw)
    ms_step = elapsed * 1e3 / K
    res = {"entry_point": "spec_prompt_lookup", "workload": f"{lw.name}: {lw.description}",
           "value": lw.B / (ms_step * 1e-3), "unit": "contexts/s", "ms_per_step": ms_step,
           "context_bytes": nbytes, "scanned_bytes": scanned, "kernel": "k_prompt_lookup",
           "kernel_us_mean": k_ms * 1e3, "kernel_GBps": scanned / (k_ms * 1e-3) / 1e9,
           "mean_draft_len": float(out[1].float().mean()),
           "roofline": roof(scanned / (k_ms * 1e-3) / 1e9,
                            "k_prompt_lookup over the context bytes it must scan (from the end "
                            "back to the block holding the latest full-size match), torch events"),
           "hbm_bytes_per_dispatch": read_kernel_traffic("k_prompt_lookup")}
    if cpu:
        import oracle

        res["cpu_baseline"] = timed_oracle(
            lambda nt: oracle.spec_prompt_lookup_ref(ctx_np, lens_np, lw.n_min, lw.n_max, lw.k),
            lw.B, "contexts/s", f"all {lw.B} contexts of the same batch, C oracle (one thread: "
                                "it searches from the end and stops at the first match)")
    log(f"[bench] prompt lookup {ms_step:.4f} ms/step; kernel {k_ms * 1e3:.1f} us "
        f"({res['kernel_GBps']:.0f} GB/s)")
    return res


def parse_args():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    # 100 calls of c5 take about 43 ms: the host's start and end of the timed
    # region (first launch, final synchronisation) then add well under 1 us
    # per call, where 20 calls carried about 1-2 us each.
    ap.add_argument("--steps", type=int, default=SMALL_STEPS)
    ap.add_argument("--event-every", type=int, default=4,
                    help="record the kernel's HIP event pair on every Nth timed step")
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--settle-ms", type=float, default=100.0,
                    help="untimed calls for at least this long before the warmup steps: "
                         "after an idle spell the GPU needs ~25 ms of load to reach its "
                         "steady clocks, and the first calls run up to 4x slower")
    ap.add_argument("--workload", default=None, choices=["c1", "c2", "c3", "c4", "c5"],
                    help="run this one workload in this process (default: a GPU-free parent "
                         "runs c3, c4 and c5, each in a child process)")
    ap.add_argument("--extras", action="store_true",
                    help="with --workload: also time top-p, top-k, tree and prompt lookup")
    ap.add_argument("--seed", type=lambda s: int(s, 0), default=None)
    ap.add_argument("--cpu-seqs", type=int, default=1024,
                    help="sequences of the batch the CPU oracle baseline runs on")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-early-exit", action="store_true",
                    help="skip timing the early-exit entry point on the same batch")
    ap.add_argument("--no-tree", action="store_true",
                    help="skip timing greedy tree verification (workload t3)")
    ap.add_argument("--no-lookup", action="store_true",
                    help="skip timing prompt-lookup drafting (workload p3)")
    ap.add_argument("--no-top-k", action="store_true",
                    help="skip timing spec_verify_top_k_top_p (top-k 50, top-p 0.95)")
    ap.add_argument("--no-top-p", action="store_true",
                    help="skip timing the top-p entry point on the same batch")
    ap.add_argument("--copy-probe", type=int, default=0)
    return ap.parse_args()


def per_call(alg_bytes: int, ms: float) -> dict:
    """The step's bandwidth over its algorithmic bytes (every needed row read
    once), as a fraction of peak, and the time 70% of peak would allow."""
    gbps = alg_bytes / (ms * 1e-3) / 1e9
    return {"step_GBps": gbps, "step_frac": gbps / PEAK_HBM_GBPS,
            "budget_ms_at_70pct": alg_bytes / (0.7 * PEAK_HBM_GBPS * 1e9) * 1e3}


def run_workload(args, name: str, extras: bool) -> dict:
    """Time spec_verify (and, on request, the other entry points) on one
    workload in this process; returns the JSON object of the run."""
    import torch

    import speculative_decoding_verification_11_amd as sv
    from speculative_decoding_verification_11_amd import workloads as wl

    w = wl.WORKLOADS[name]
    seed = args.seed if args.seed is not None else wl.philox_seeds(w.name, 1)[0]
    log(f"[bench] generating {w.name}: {w.description}")
    batch = wl.generate(w, "cuda:0")
    torch.cuda.synchronize()
    alg_bytes = batch.algorithmic_bytes()
    t_rows, d_rows = batch.rows_read()
    valid_positions = int((batch.draft_len.to(torch.int64) + 1).sum())
    positions = w.B * (w.k + 1)

    # Footprints below the 256 MiB last-level cache would measure cache, not
    # HBM: rotate through enough copies to exceed 1 GiB.
    copies = [batch]
    n_copies = max(1, -(-(1 << 30) // max(1, alg_bytes)))
    for _ in range(n_copies - 1):
        copies.append(wl.Batch(w, batch.target.clone(), batch.draft.clone(),
                               batch.draft_tokens.clone(), batch.draft_len.clone(),
                               batch.temperature.clone()))

    hip = hip_runtime()
    K, W = args.steps, args.warmup
    ev = HipEvents(hip, K)  # destroyed at the end of this workload, before the CPU leg
    ws = torch.empty(sv.workspace_size(w.B, w.k, w.V, w.dtype_code), dtype=torch.uint8,
                     device="cuda:0")
    outs = [(torch.empty((w.B, w.k + 1), dtype=torch.int32, device="cuda:0"),
             torch.empty((w.B,), dtype=torch.int32, device="cuda:0")) for _ in copies]

    def step(i: int, events=None, fn=sv.spec_verify):
        cb = copies[i % len(copies)]
        fn(cb.target, cb.draft, cb.draft_tokens, cb.draft_len, cb.temperature, seed,
           workspace=ws, out=outs[i % len(copies)], events=events)


    def timed(fn=sv.spec_verify):
        for i in range(W):
            step(i, fn=fn)
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for i in range(K):
            step(i, events=ev.pair(i) if sampled(i) else None, fn=fn)
        torch.cuda.synchronize()
        return (time.perf_counter() - t0) * 1e3 / K, ev.elapsed_ms(K)

    log(f"[bench] settle {args.settle_ms:.0f} ms, then warmup {W} steps, {len(copies)} "
        "rotating copies")
    n_settle = 0
    t_settle = time.perf_counter()
    while (time.perf_counter() - t_settle) * 1e3 < args.settle_ms:
        for _ in range(10):
            step(n_settle)
            n_settle += 1
        torch.cuda.synchronize()
    log(f"[bench] timing {K} steps")
    ms_per_step, k1_ms = timed()
    k1_mean = sum(k1_ms) / len(k1_ms)
    k1_median = k1_ms[len(k1_ms) // 2]
    achieved = alg_bytes / (k1_mean * 1e-3) / 1e9
    # outputs of the timed batch (copy 0) with diagnostics, for the CPU leg
    out0, n0, aux0 = sv.spec_verify(batch.target, batch.draft, batch.draft_tokens,
                                    batch.draft_len, batch.temperature, seed, aux=True)
    torch.cuda.synchronize()
    gpu_out = {key: v.cpu().numpy() for key, v in aux0.items()}
    gpu_out["out_tokens"] = out0.cpu().numpy()
    gpu_out["num_accepted"] = n0.cpu().numpy()
    n_acc = n0.to(torch.int64)
    tokens_per_round = float((n_acc + 1).float().mean())
    # The draw re-reads the decided row of every sampled sequence: target
    # and draft row at a rejection. A bonus token's chunk is located from the
    # row statistics, so the draw re-reads that one 32 KiB chunk of the
    # target row (on these unfiltered rows every bonus row has mass).
    n_cpu = n_acc.cpu()
    kind = aux0["draw_kind"].cpu()
    n_resid = int(((kind == sv.DRAW_RESIDUAL) | (kind == sv.DRAW_RESIDUAL_AS_P)).sum())
    n_bonus = int((kind == sv.DRAW_BONUS).sum())
    draw_rows = n_resid * 2 + n_bonus
    draw_bytes = n_resid * 2 * w.V * w.elem_bytes + n_bonus * min(w.V * w.elem_bytes, CHUNK_BYTES)
    pc = per_call(alg_bytes, ms_per_step)
    log(f"[bench] {w.name}: {ms_per_step:.4f} ms/step ({pc['step_frac']:.3f} of peak on "
        f"algorithmic bytes); k_rowstats mean {k1_mean * 1e3:.1f} us (median "
        f"{k1_median * 1e3:.1f}, min {k1_ms[0] * 1e3:.1f}, max {k1_ms[-1] * 1e3:.1f}); "
        f"{achieved:.0f} GB/s")

    early = None
    if not args.no_early_exit:
        # The same batch through the early-exit schedule (identical outputs;
        # only the rows up to each sequence's first rejection are read).
        log(f"[bench] early exit: warmup {W} steps, timing {K} steps")
        ee_ms, loop_ms = timed(sv.spec_verify_early_exit)
        loop_mean = sum(loop_ms) / len(loop_ms)
        n_ee = outs[0][1].to(torch.int64).cpu()
        L = copies[0].draft_len.to(torch.int64).cpu()
        samp = (copies[0].temperature.cpu() > 0)
        ee_t = int((n_ee + 1).sum())
        ee_d = int(torch.minimum(n_ee + 1, L)[samp].sum())
        ee_bytes = (ee_t + ee_d) * w.V * w.elem_bytes
        early = {
            "entry_point": "spec_verify_early_exit",
            "value": positions / (ee_ms * 1e-3),
            "unit": "positions/s",
            "ms_per_step": ee_ms,
            "faster_than_full_step": ee_ms < ms_per_step,
            "rows_read": {"target": ee_t, "draft": ee_d},
            "bytes_read_once": ee_bytes,
            "position_loop_us_mean": loop_mean * 1e3,
            "position_loop_GBps": ee_bytes / (loop_mean * 1e-3) / 1e9,
            "outputs_identical": bool(torch.equal(n_ee, n_cpu)),
            "roofline": roof(ee_bytes / (loop_mean * 1e-3) / 1e9,
                             "the position loop (rows up to each stop, read once), HIP events"),
            "cpu_baseline": "the oracle of this workload's cpu_baseline (identical outputs)",
            "hbm_bytes_per_dispatch": read_kernel_traffic("k_ee_rowstats0", "k_ee_rowstats",
                                                          "k_ee_tail", "k_draw", workload=name),
        }
        log(f"[bench] early exit {ee_ms:.4f} ms/step; position loop {loop_mean * 1e3:.1f} us "
            f"for {ee_bytes / 1e9:.3f} GB")
    topp = topk = tree = lookup = None
    if extras and not args.no_top_p:
        # The same batch with top-p 0.95 on every row (the drafted tokens were
        # sampled without it, so a few land outside the draft's nucleus and
        # end their sequence with status QZERO, as the contract says).
        log(f"[bench] top-p 0.95: warmup {W} steps, timing {K} steps")
        tp = torch.full((w.B,), 0.95, dtype=torch.float32, device="cuda:0")
        tp_ms, tp_pass = timed(lambda *a, **kw: sv.spec_verify_top_p(*a[:5], tp, *a[5:], **kw))
        tp_pass_mean = sum(tp_pass) / len(tp_pass)
        _, _, aux_tp = sv.spec_verify_top_p(copies[0].target, copies[0].draft,
                                            copies[0].draft_tokens, copies[0].draft_len,
                                            copies[0].temperature, tp, seed, aux=True)
        st = aux_tp["seq_status"].cpu()
        topp = {"entry_point": "spec_verify_top_p", "top_p": 0.95,
                "value": positions / (tp_ms * 1e-3), "unit": "positions/s", "ms_per_step": tp_ms,
                "rows_filtered": t_rows + d_rows,
                "sequences_ok": int((st == 0).sum()), "sequences_qzero": int((st == 4).sum()),
                "row_pass_us_mean": tp_pass_mean * 1e3,
                "roofline": roof(alg_bytes / (tp_pass_mean * 1e-3) / 1e9,
                                 "the row pass (k_filter reads each filtered row once; "
                                 "k_rowstats skips them), HIP events"),
                "hbm_bytes_per_dispatch": read_kernel_traffic("k_filter", "k_filter_fallback",
                                                              "k_draw", workload=name)}
        # half the sequences unfiltered (top_p = 1): their rows go through
        # the plain row-statistics pass
        tph = torch.tensor([(0.95, 1.0)[b % 2] for b in range(w.B)], dtype=torch.float32,
                           device="cuda:0")
        tph_ms, _ = timed(lambda *a, **kw: sv.spec_verify_top_p(*a[:5], tph, *a[5:], **kw))
        topp["mixed_half_unfiltered_ms_per_step"] = tph_ms
        if not args.no_cpu_baseline:
            from oracle import parity

            n_cpu_seq = 64
            hs = wl.to_host_arrays(batch.select(range(n_cpu_seq)))
            topp["cpu_baseline"] = timed_oracle(
                lambda nt: parity.oracle_on(hs, seed, nthreads=nt,
                                            top_p=np.full(n_cpu_seq, 0.95, np.float32)),
                n_cpu_seq * (w.k + 1), "positions/s",
                f"first {n_cpu_seq} of {w.B} sequences of the same batch, fp64 C oracle with "
                "top-p")
        log(f"[bench] top-p {tp_ms:.4f} ms/step; row pass {tp_pass_mean * 1e3:.1f} us; "
            f"half unfiltered {tph_ms:.4f} ms/step")
    if extras and not args.no_top_k:
        # The same batch with top-k 50 and then top-p 0.95 on every row.
        log(f"[bench] top-k 50 + top-p 0.95: warmup {W} steps, timing {K} steps")
        tk = torch.full((w.B,), 50, dtype=torch.int32, device="cuda:0")
        tp = torch.full((w.B,), 0.95, dtype=torch.float32, device="cuda:0")
        tk_ms, tk_pass = timed(
            lambda *a, **kw: sv.spec_verify_top_k_top_p(*a[:5], tk, tp, *a[5:], **kw))
        tk_pass_mean = sum(tk_pass) / len(tk_pass)
        _, _, aux_tk = sv.spec_verify_top_k_top_p(copies[0].target, copies[0].draft,
                                                  copies[0].draft_tokens, copies[0].draft_len,
                                                  copies[0].temperature, tk, tp, seed, aux=True)
        st = aux_tk["seq_status"].cpu()
        topk = {"entry_point": "spec_verify_top_k_top_p", "top_k": 50, "top_p": 0.95,
                "value": positions / (tk_ms * 1e-3), "unit": "positions/s", "ms_per_step": tk_ms,
                "rows_filtered": t_rows + d_rows,
                "sequences_ok": int((st == 0).sum()), "sequences_qzero": int((st == 4).sum()),
                "row_pass_us_mean": tk_pass_mean * 1e3,
                "roofline": roof(alg_bytes / (tk_pass_mean * 1e-3) / 1e9,
                                 "the row pass (k_filter reads each filtered row once; "
                                 "k_rowstats skips them), HIP events"),
                "hbm_bytes_per_dispatch": read_kernel_traffic("k_filter", "k_filter_fallback",
                                                              "k_draw", workload=name)}
        if not args.no_cpu_baseline:
            from oracle import parity

            n_cpu_seq = 64
            hs = wl.to_host_arrays(batch.select(range(n_cpu_seq)))
            topk["cpu_baseline"] = timed_oracle(
                lambda nt: parity.oracle_on(hs, seed, nthreads=nt,
                                            top_k=np.full(n_cpu_seq, 50, np.int32),
                                            top_p=np.full(n_cpu_seq, 0.95, np.float32)),
                n_cpu_seq * (w.k + 1), "positions/s",
                f"first {n_cpu_seq} of {w.B} sequences of the same batch, fp64 C oracle with "
                "top-k and top-p")
        log(f"[bench] top-k + top-p {tk_ms:.4f} ms/step; row pass {tk_pass_mean * 1e3:.1f} us")
    if extras and not args.no_tree:
        tree = bench_tree(ev, K, W, not args.no_cpu_baseline)
    if extras and not args.no_lookup:
        lookup = bench_lookup(K, W, not args.no_cpu_baseline)
    ev.close()

    result = {
        "metric": METRIC,
        "value": positions / (ms_per_step * 1e-3),
        "unit": "positions/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": W,
        "settle": {"ms": args.settle_ms, "calls": n_settle},
        "ms_per_step": ms_per_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "config": {
            "workload": f"{w.name}: {w.description}",
            "B": w.B, "k": w.k, "V": w.V, "logits": w.dtype,
            "valid_positions": valid_positions,
            "valid_positions_per_s": valid_positions / (ms_per_step * 1e-3),
            "rows_read": {"target": t_rows, "draft": d_rows},
            "algorithmic_bytes": alg_bytes,
            "per_call": pc,
            "draw_reread": {
                "rows": draw_rows,
                "bytes": draw_bytes,
                "note": "side figure, not the step's bandwidth: the draw re-reads the decided "
                        "rows of each sampled sequence (target and draft at a rejection; for a "
                        "bonus, the one 32 KiB chunk of the target row that holds it); the "
                        "algorithmic bytes exclude these re-reads",
            },
            "rotating_copies": len(copies),
            "mean_tokens_per_round": tokens_per_round,
            "parallelism": "single GPU",
        },
        "roofline": {
            "bound": "hbm",
            "kernel": counter_summary(w.name).get("kernel", "k_rowstats"),
            "achieved": achieved,
            "peak": PEAK_HBM_GBPS,
            "unit": "GB/s",
            "frac": achieved / PEAK_HBM_GBPS,
            "traffic": read_counter_traffic(w.name),
            "kernel_us_mean": k1_mean * 1e3,
            "kernel_us_median": k1_median * 1e3,
            "events": f"HIP event pair around the row-statistics launch on every "
                      f"{EVENT_EVERY}th of the {K} timed steps ({len(k1_ms)} samples)",
        },
    }
    for key, val in (("early_exit", early), ("top_p", topp), ("top_k_top_p", topk),
                     ("tree", tree), ("prompt_lookup", lookup)):
        if val is not None:
            result[key] = val
    if not args.no_cpu_baseline:
        log(f"[bench] CPU oracle baseline on {min(args.cpu_seqs, w.B)} sequences")
        result["cpu_baseline"] = cpu_baseline(batch, seed, args.cpu_seqs, gpu_out)
    return result


def summary(res: dict) -> dict:
    """Per-workload figures of a child's result for the parent's line."""
    c = res["config"]
    out = {"workload": c["workload"], "steps": res["steps"], "ms_per_step": res["ms_per_step"],
           "positions_per_s": res["value"], "valid_positions_per_s": c["valid_positions_per_s"],
           "algorithmic_bytes": c["algorithmic_bytes"], **c["per_call"],
           "k_rowstats_us_mean": res["roofline"]["kernel_us_mean"],
           "k_rowstats_frac": res["roofline"]["frac"],
           "k_rowstats_traffic": res["roofline"]["traffic"],
           "draw_reread_bytes": c["draw_reread"]["bytes"]}
    if "early_exit" in res:
        out["early_exit_ms_per_step"] = res["early_exit"]["ms_per_step"]
    if "cpu_baseline" in res:
        out["flagged"] = res["cpu_baseline"]["parity"]
    return out


def parent(args) -> int:
    """Run each workload in a child process of its own and print one line.
    This process never touches the GPU; it starts every child itself."""
    results = {}
    for name in WORKLOADS:
        # The headline times exactly the steps asked for. The smaller
        # workloads time at least SMALL_STEPS. Each takes the kernel's event
        # pairs on about five of its steps: an event pair stalls the stream
        # for a microsecond or two, a measurable share of a step of 50-100 us.
        steps, every = args.steps, args.event_every
        if name != HEADLINE:
            steps = max(steps, SMALL_STEPS)
        every = max(every, steps // 5)
        cmd = [sys.executable, os.path.abspath(__file__), "--workload", name,
               "--steps", str(steps), "--warmup", str(args.warmup),
               "--event-every", str(every), "--settle-ms", str(args.settle_ms),
               "--cpu-seqs", str(args.cpu_seqs)]
        if name == HEADLINE:
            cmd.append("--extras")
        for flag in ("no_cpu_baseline", "no_early_exit", "no_tree", "no_lookup", "no_top_k",
                     "no_top_p"):
            if getattr(args, flag):
                cmd.append("--" + flag.replace("_", "-"))
        if args.seed is not None:
            cmd += ["--seed", hex(args.seed)]
        log(f"[bench] child: {' '.join(cmd[1:])}")
        proc = subprocess.run(cmd, stdout=subprocess.PIPE, text=True, timeout=900)
        if proc.returncode != 0:
            log(f"[bench] child {name} failed with status {proc.returncode}")
            return proc.returncode or 1
        lines = [ln for ln in proc.stdout.splitlines() if ln.startswith("{")]
        results[name] = json.loads(lines[-1])
    result = results[HEADLINE]
    result["configs"] = {name: summary(res) for name, res in results.items()}
    result["configs_note"] = (
        "each workload timed in its own process (the headline on the steps asked for, the "
        f"others on at least {SMALL_STEPS}, each with about five kernel event pairs; the same "
        "warm-up); step_frac = "
        "algorithmic bytes (every needed row read once) / ms_per_step / 8 TB/s; the target is "
        "0.7 on c3, c4 and c5; the headline value and roofline are c5's")
    print(json.dumps(result), flush=True)
    return 0


def main() -> int:
    args = parse_args()
    global EVENT_EVERY
    EVENT_EVERY = max(1, args.event_every)

    if args.gpus != 1:
        log(f"bench.py: --gpus {args.gpus} is not supported: it measures one GPU only. "
            "Sequences shard across GPUs with no communication: each GPU would run the same "
            "kernels on its slice of the batch, with seq_base set to the slice's offset.")
        return 2
    if args.workload is None and not args.copy_probe:
        return parent(args)
    import torch

    if not torch.cuda.is_available():
        log("bench.py: no GPU visible")
        return 1
    if args.copy_probe:
        copy_probe(args.copy_probe)
        return 0
    print(json.dumps(run_workload(args, args.workload, args.extras)), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
