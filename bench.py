#!/usr/bin/env python3
"""Benchmark of the mHC fused post->pre pass on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload prefill]
    python bench.py --workload decode --graph [--graph-steps 16]  # the step replayed from a HIP graph
    python bench.py --workload decode --defer-sinkhorn  # the Sinkhorn on a side stream
    python bench.py --workload decode --cold-phi 64   # 64 prepacked projections in turn
    python bench.py --copy-probe           # copy kernel of known size (counter calibration)
    python bench.py --pmc-summary FILE...  # per-kernel means of rocprofv3 counter output

One step = one pass of the whole hot path over one batch of synthetic input
already resident in HBM: repack the next layer's projection (mhc_pack_phi)
and run the fused post -> coefficients -> pre pass
(mhc_post_pre_fused_prepacked).  Untimed steps run for --settle-ms of wall
time while the clocks ramp up, then W untimed warm-up steps, then K timed
steps between two device synchronisations; HIP events around every fused
launch give the dominant kernel's average duration for the roofline figure.
Two torch device copies of x and y (the bytes the fused pass streams) are
timed after it as a plain-copy reference.  Rank 0 prints one JSON line.
The default workload is prefill-shaped: T = 8192 tokens, C = 7168,
4 routes, 1% of the rows scaled by 100.
"""
from __future__ import annotations

import argparse
import csv
import hashlib
import json
import os
import re
import sqlite3
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0  # MI355X HBM3E peak, GB/s

METRIC = "mHC fused post+pre tokens/s and % peak HBM GB/s at C=7168, T=8192"

# Sources whose change invalidates the stored hardware counter figures.
KERNEL_SOURCES = ["mhc_kernels.hip", "mhc_device.h", "mhc_internal.h", "mhc_api.cpp"]
# counter figures of the fused kernel each schedule runs on the prefill workload
TRAFFIC_FILES = {"persistent": os.path.join(ROOT, "profiles", "k_persist_fused_prefill_traffic.txt"),
                 "staged": os.path.join(ROOT, "profiles", "k_split_fused_prefill_traffic.txt")}
KERNEL_NAMES = {"persistent": "k_persist (fused post->pre, persistent schedule)",
                "staged": "k_split (fused post->pre, staged schedule)"}
COPY_PROBE_BYTES = 1 << 30


def kernel_source_hash() -> str:
    h = hashlib.sha256()
    for name in KERNEL_SOURCES:
        with open(os.path.join(ROOT, "manifold_constrained_hyper_mhc_amd", "csrc", name), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def stored_traffic(workload: str, schedule: str):
    """HBM bytes per fused launch measured with rocprofv3 counters (FETCH_SIZE,
    WRITE_SIZE, each scaled by the copy-kernel calibration), or None when the
    kernel sources changed since the counters were taken."""
    path = TRAFFIC_FILES.get(schedule)
    if workload != "prefill" or path is None or not os.path.exists(path):
        return None
    kv = {}
    with open(path) as f:
        for line in f:
            m = re.match(r"^([a-z_0-9]+):\s*(.+)$", line.strip())
            if m:
                kv[m.group(1)] = m.group(2).strip()
    if kv.get("source_sha256") != kernel_source_hash():
        return None
    try:
        return int(kv["hbm_read_bytes"]) + int(kv["hbm_write_bytes"])
    except (KeyError, ValueError):
        return None


def pmc_summary(paths) -> int:
    """Mean value per dispatch of each counter of each kernel, from rocprofv3
    counter output (counter_collection.csv or a rocpd database)."""
    import collections
    agg = collections.defaultdict(list)
    for path in paths:
        if path.endswith(".db"):
            con = sqlite3.connect(path)
            rows = con.execute("select kernel_name, counter_name, value from counters_collection")
            for name, cname, val in rows:
                agg[(name, cname)].append(float(val))
        else:
            with open(path, newline="") as f:
                for r in csv.DictReader(f):
                    agg[(r["Kernel_Name"], r["Counter_Name"])].append(float(r["Counter_Value"]))
    for (name, cname), vals in sorted(agg.items(), key=lambda kv: -max(kv[1])):
        short = re.sub(r"\(.*", "", name)[-70:]
        print(f"{short:70s} {cname:11s} dispatches={len(vals):4d} mean={sum(vals) / len(vals):16.1f}")
    return 0


def copy_probe() -> int:
    """A plain device-to-device copy of COPY_PROBE_BYTES, three times: the
    counters it reads calibrate FETCH_SIZE and WRITE_SIZE against known bytes."""
    import torch
    dev = torch.device("cuda:0")
    src = torch.ones(COPY_PROBE_BYTES, dtype=torch.uint8, device=dev)
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(3):
        dst.copy_(src)
    torch.cuda.synchronize()
    dt = (time.perf_counter() - t0) / 3
    print(json.dumps({"copy_probe_bytes": COPY_PROBE_BYTES, "copies": 3,
                      "GB_per_s_read_plus_write": 2 * COPY_PROBE_BYTES / dt / 1e9}), flush=True)
    return 0


def algorithmic_bytes(T: int, C: int, mxfp8: bool, with_h: bool = True) -> int:
    """Bytes the fused pass must move: per token x (8C) + y (2C) + incoming
    post/res (80) + x' (8C) + outgoing coefficients (96) + h (2C bf16 and/or
    C + C/32 MXFP8); per call the projection (fp32, 384C), gamma (4C) and
    bias (96), each read once."""
    per_tok = 8 * C + 2 * C + 80 + 8 * C + 96
    if with_h:
        per_tok += 2 * C
    if mxfp8:
        per_tok += C + C // 32
    return T * per_tok + 384 * C + 4 * C + 96


def cpu_model() -> str:
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


_TP_LIMIT = None


def _oracle_worker_init():
    # one thread per worker process: the processes are the parallelism
    global _TP_LIMIT
    import threadpoolctl
    _TP_LIMIT = threadpoolctl.threadpool_limits(limits=1)


def _oracle_run(task):
    """Run the oracle's fused post->pre over chunks of the given rows for
    `budget` seconds; returns (tokens done, seconds)."""
    x, y, cf, phi, b, g, kw, budget, chunk = task
    import oracle as O

    n = x.shape[0]
    done, k = 0, 0
    t0 = time.perf_counter()
    while time.perf_counter() - t0 < budget:
        s = (k * chunk) % n
        rows = slice(s, min(s + chunk, n))
        O.post_pre_fused(x[rows], y[rows], cf[rows], phi, b, g, **kw)
        done += rows.stop - rows.start
        k += 1
    return done, time.perf_counter() - t0


def start_oracle_pool():
    """Worker processes for the all-cores oracle leg, forked before anything
    touches the GPU (a forked child of a process with a live GPU context is
    not safe).  At most 16 processes: the host cores one GPU is given."""
    import multiprocessing as mp

    n = max(1, min(16, len(os.sched_getaffinity(0))))
    return mp.get_context("fork").Pool(n, initializer=_oracle_worker_init), n


def cpu_baseline(pool, nproc: int, inp_host: dict, coeffs_host, params, budget_s: float = 10.0,
                 chunk: int = 64) -> dict:
    """The fp64 oracle, as it stands, on a bounded sample of the workload:
    `nproc` processes of one thread each, every one on its own slice of the
    sample, all for the same `budget_s` seconds (tokens/s summed), then one
    thread alone for a third of the budget."""
    import threadpoolctl

    f64 = lambda t: t.to("cpu").double().numpy()  # noqa: E731
    x, y = f64(inp_host["x"]), f64(inp_host["y"])
    cf = f64(coeffs_host)
    phi, b, g = f64(inp_host["phi_next"]), f64(inp_host["bias_next"]), f64(inp_host["gamma_next"])
    n = x.shape[0]
    kw = dict(hc_norm_eps=params.hc_norm_eps, rmsnorm_eps=params.rmsnorm_eps, hc_post_scale=params.hc_post_scale,
              sinkhorn_eps=params.sinkhorn_eps, sinkhorn_iters=params.sinkhorn_iters)
    per = max(chunk, n // nproc)
    tasks = []
    for i in range(nproc):
        s = (i * per) % n
        sl = slice(s, min(s + per, n))
        tasks.append((x[sl], y[sl], cf[sl], phi, b, g, kw, budget_s, chunk))
    res = pool.map(_oracle_run, tasks, chunksize=1)
    done = sum(d for d, _ in res)
    value = sum(d / t for d, t in res)
    with threadpoolctl.threadpool_limits(limits=1):
        done1, dt1 = _oracle_run((x, y, cf, phi, b, g, kw, budget_s / 3, chunk))
    return {"value": value, "unit": "tokens/s", "cores": nproc, "kind": "oracle",
            "value_1_thread": done1 / dt1, "cpu_model": cpu_model(),
            "sample": f"{nproc} processes x 1 thread, each on {per} of the first {n} tokens of the same workload "
                      f"in chunks of {chunk} for {budget_s:.0f} s ({done} tokens in all); one thread alone: "
                      f"{done1} tokens in {dt1:.1f} s; fp64 numpy oracle fused post->pre"}


def time_unfused(mhc, inp, coeffs_in, packed, params, outs, stream, args, fused_bytes, fused_ms):
    """The same step without fusion, on the same inputs: mhc_post writes x',
    mhc_coeffs_prepacked reads it back for the next layer's coefficients and
    mhc_pre reads it again for h.  HIP events around each launch; returns the
    per-kernel averages and the chain's algorithmic bytes (36C + 192 per
    token instead of the fused 20C + 176)."""
    import torch

    x, y = inp["x"], inp["y"]
    T, C = x.shape[0], x.shape[2]
    xp = torch.empty_like(x)
    cf = torch.empty_like(outs["coeffs_next"])
    h = torch.empty((T, C), dtype=torch.bfloat16, device=x.device)
    ws = mhc.workspace(T, C, x.device)

    def chain(ev=None):
        if ev is not None:
            ev[0].record(stream)
        mhc.post(x, y, coeffs_in, out=xp)
        if ev is not None:
            ev[1].record(stream)
        mhc.coeffs_prepacked(xp, packed, inp["bias_next"], params, ws=ws, out=cf)
        if ev is not None:
            ev[2].record(stream)
        mhc.pre(xp, cf, inp["gamma_next"], params, out=h)
        if ev is not None:
            ev[3].record(stream)

    for _ in range(args.warmup):
        chain()
    torch.cuda.synchronize()
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(4)] for _ in range(args.steps)]
    for k in range(args.steps):
        chain(evs[k])
    torch.cuda.synchronize()
    avg = lambda i, j: sum(e[i].elapsed_time(e[j]) for e in evs) / len(evs) * 1e3  # noqa: E731
    chain_us = avg(0, 3)
    chain_bytes = T * (36 * C + 192) + 388 * C + 96
    return {"chain_us": chain_us, "post_us": avg(0, 1), "coeffs_us": avg(1, 2), "pre_us": avg(2, 3),
            "chain_algorithmic_bytes": chain_bytes, "chain_gbs": chain_bytes / (chain_us * 1e-6) / 1e9,
            "fused_over_chain_time": fused_ms * 1e3 / chain_us,
            "note": "same inputs; x' written by post and read back by coeffs and pre"}


def copy_reference(inp, outs, stream, args, fused_gbs):
    """The plain-copy ceiling for the same tensors: torch device copies of x
    and y into buffers of their shape (reads and writes the bytes the fused
    pass streams, 20C per token).  HIP events around each pair of copies."""
    import torch

    from manifold_constrained_hyper_mhc_amd.binding import _placed_empty

    x, y = inp["x"], inp["y"]
    dx = outs["x_out"]
    dy = _placed_empty(tuple(y.shape), y.dtype, y.device, y)  # placed as the fused pass's h

    def run():
        dx.copy_(x)
        dy.copy_(y)

    for _ in range(3):
        run()
    torch.cuda.synchronize()
    n = max(5, min(args.steps, 20))
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(n)]
    for a, b in evs:
        a.record(stream)
        run()
        b.record(stream)
    torch.cuda.synchronize()
    us = sum(a.elapsed_time(b) for a, b in evs) / n * 1e3
    nbytes = 2 * (x.numel() * x.element_size() + y.numel() * y.element_size())
    gbs = nbytes / (us * 1e-6) / 1e9
    return {"what": "torch copies x -> [T,4,C] and y -> [T,C] buffers (reads + writes 20C bytes per token)",
            "us": us, "bytes": nbytes, "gbs": gbs, "frac_of_peak": gbs / HBM_PEAK_GBS,
            "fused_gbs_over_copy_gbs": fused_gbs / gbs}


def copy_ceiling(inp, stream, args, fused_gbs, lanes):
    """Hand-written copies and reads of x and y (libmhc_bench.so): the
    bandwidth a plain stream of the same tensors reaches, linear (16 bytes
    per lane, 4 loads in flight) and in the persistent fused kernel's access
    pattern (256-byte pieces of 128-row tiles, S splits x `lanes` workgroups).
    HIP events around each pair of launches (x, then y)."""
    import ctypes

    import torch

    lib_path = os.path.join(ROOT, "manifold_constrained_hyper_mhc_amd", "libmhc_bench.so")
    L = ctypes.CDLL(lib_path)
    L.bench_copy.argtypes = [ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int64, ctypes.c_int64,
                             ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p]
    L.bench_copy.restype = ctypes.c_int
    from manifold_constrained_hyper_mhc_amd.binding import _placed_empty

    x, y = inp["x"], inp["y"]
    T, _, C = x.shape
    # two placements of the destinations: aligned like x and y modulo 1 KiB,
    # and placed as the fused pass's x_out and h; each copy reports the
    # faster (a ceiling), and which it was
    dsts = {"aligned": (torch.empty_like(x), torch.empty_like(y)),
            "placed": (_placed_empty(tuple(x.shape), x.dtype, x.device, x),
                       _placed_empty(tuple(y.shape), y.dtype, y.device, y))}
    dx, dy = dsts["placed"]
    S = 2 * C // 256
    sink = torch.empty(max(1024, S * lanes) * 256 * 16, dtype=torch.uint8, device=x.device)
    st = ctypes.c_void_p(stream.cuda_stream)
    nbytes = x.numel() * 2 + y.numel() * 2

    def run(kind, ddx, ddy):
        for src, dst, rows in ((x, ddx, 4 * T), (y, ddy, T)):
            rc = L.bench_copy(kind, src.data_ptr(), dst.data_ptr(), rows, 2 * C, lanes, sink.data_ptr(), st)
            if rc != 0:
                raise RuntimeError(f"bench_copy kind {kind}: {rc}")

    out = {}
    names = {0: "linear_copy", 1: "linear_read", 2: "piece_copy", 3: "piece_read"}
    for kind, name in names.items():
        best = None
        for place, (ddx, ddy) in dsts.items():
            for _ in range(3):
                run(kind, ddx, ddy)
            torch.cuda.synchronize()
            n = max(5, min(args.steps, 20))
            evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(n)]
            for a, b in evs:
                a.record(stream)
                run(kind, ddx, ddy)
                b.record(stream)
            torch.cuda.synchronize()
            us = sum(a.elapsed_time(b) for a, b in evs) / n * 1e3
            moved = nbytes * (2 if kind in (0, 2) else 1)
            gbs = moved / (us * 1e-6) / 1e9
            if best is None or gbs > best["gbs"]:
                best = {"us": us, "bytes": moved, "gbs": gbs, "frac_of_peak": gbs / HBM_PEAK_GBS,
                        "destination": place}
        out[name] = best
    # the same copy with wider pieces (the fused kernel's projection slice in
    # LDS fixes its piece at 256 bytes): the stream workgroup count, and all CUs
    L.bench_copy_pieces.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int64, ctypes.c_int64, ctypes.c_int,
                                    ctypes.c_int, ctypes.c_void_p]
    L.bench_copy_pieces.restype = ctypes.c_int
    sweep = {}
    for wg in (S * lanes, torch.cuda.get_device_properties(x.device).multi_processor_count):
        for pb in (256, 512, 1024, 2048):
            def runw():
                for src, dst, rows in ((x, dx, 4 * T), (y, dy, T)):
                    rc = L.bench_copy_pieces(src.data_ptr(), dst.data_ptr(), rows, 2 * C, pb, wg, st)
                    if rc != 0:
                        raise RuntimeError(f"bench_copy_pieces {pb}: {rc}")
            for _ in range(2):
                runw()
            torch.cuda.synchronize()
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            n = 5
            a.record(stream)
            for _ in range(n):
                runw()
            b.record(stream)
            torch.cuda.synchronize()
            us = a.elapsed_time(b) / n * 1e3
            wgs = (2 * C // pb) * max(1, wg // (2 * C // pb))
            sweep[f"{pb}B_{wgs}wg"] = round(2 * nbytes / (us * 1e-6) / 1e9, 1)
    out["piece_width_sweep_gbs"] = sweep
    out["what"] = ("hand-written copies (read + write) and reads of x [T,4,C] and y [T,C]: linear, and in the fused "
                   f"kernel's pattern (256-byte pieces of 128-row tiles, {S} splits x {lanes} workgroups), each the "
                   "faster of two destination placements (aligned like the sources modulo 1 KiB, or placed as the "
                   "fused pass's outputs); piece_width_sweep_gbs: the piece copy with wider pieces (placed "
                   "destinations), at the stream workgroup count and at one workgroup per CU")
    out["fused_gbs_over_piece_copy_gbs"] = fused_gbs / out["piece_copy"]["gbs"]
    return out


def time_pre_broadcast(mhc, inp, packed, params, stream, args):
    """The first-layer pre (mhc_pre_broadcast_prepacked) on x0 = route 0 of x,
    [T, C]: coefficients and pre of x0 standing for all 4 routes.  HIP events
    around each call.  Algorithmic bytes 4C + 112 per token (x0 read once,
    h written, the coefficients written and their pre read back) + the
    projection, bias and gamma once.  Where the persistent schedule runs
    (prefill sizes) the library reads x0 once, in one pass; its two-pass
    path (coefficients, then the pre kernel) reads it twice, 6C + 112."""
    import torch

    x0 = inp["x"][:, 0, :].contiguous()
    T, C = x0.shape
    cf = torch.empty((T, 24), dtype=torch.float32, device=x0.device)
    h = torch.empty((T, C), dtype=torch.bfloat16, device=x0.device)
    ws = mhc.workspace(T, C, x0.device)

    def run():
        mhc.pre_broadcast(x0, None, inp["bias_next"], inp["gamma_next"], params, ws=ws, coeffs_out=cf, h_out=h,
                          phi_packed=packed)

    for _ in range(max(3, args.warmup)):
        run()
    torch.cuda.synchronize()
    n = max(5, args.steps)
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(n)]
    for a, b in evs:
        a.record(stream)
        run()
        b.record(stream)
    torch.cuda.synchronize()
    us = sum(a.elapsed_time(b) for a, b in evs) / n * 1e3
    nbytes = T * (4 * C + 112) + 388 * C + 96
    two_pass = T * (6 * C + 112) + 388 * C + 96
    return {"us": us, "algorithmic_bytes": nbytes, "gbs": nbytes / (us * 1e-6) / 1e9,
            "frac_of_peak": nbytes / (us * 1e-6) / 1e9 / HBM_PEAK_GBS,
            "two_pass_bytes": two_pass, "two_pass_frac_of_peak": two_pass / (us * 1e-6) / 1e9 / HBM_PEAK_GBS,
            "note": "mhc_pre_broadcast_prepacked on a [T, C] first-layer input (coefficients + pre); "
                    "algorithmic bytes read x0 once, as the one-pass schedule does (the two-pass path reads "
                    "it twice: two_pass_*)"}


def time_post_int8(mhc, inp, coeffs_in, stream, args):
    """Post of an int8 sublayer output with per-token scales (mhc_post_int8)
    on the workload's x and incoming coefficients.  HIP events around each
    call; algorithmic bytes 17C + 84 per token (x read, x' written, int8
    codes, the scale, post and res coefficients)."""
    import torch
    from manifold_constrained_hyper_mhc_amd.synthetic import make_int8_y

    T, _, C = inp["x"].shape
    yq = make_int8_y(T, C, seed=3, device=inp["x"].device)
    out = torch.empty_like(inp["x"])

    def run():
        mhc.post_int8(inp["x"], yq["y_q"], yq["y_scale"], coeffs_in, out=out)

    for _ in range(max(3, args.warmup)):
        run()
    torch.cuda.synchronize()
    n = max(5, args.steps)
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(n)]
    for a, b in evs:
        a.record(stream)
        run()
        b.record(stream)
    torch.cuda.synchronize()
    us = sum(a.elapsed_time(b) for a, b in evs) / n * 1e3
    nbytes = T * (17 * C + 84)
    res = {"us": us, "algorithmic_bytes": nbytes, "gbs": nbytes / (us * 1e-6) / 1e9,
           "frac_of_peak": nbytes / (us * 1e-6) / 1e9 / HBM_PEAK_GBS,
           "note": "mhc_post_int8: int8 sublayer output with per-token scales"}
    # the fused post -> next pre of the same int8 output (prepacked projection):
    # 19C + 180 bytes per token (x, codes, scale, coefficients in; x', h,
    # next coefficients out)
    packed = mhc.pack_phi(inp["phi_next"])
    ws = mhc.workspace(T, C, inp["x"].device)
    outs = {"x_out": out, "coeffs_next": torch.empty((T, 24), dtype=torch.float32, device=out.device),
            "h": torch.empty((T, C), dtype=torch.bfloat16, device=out.device)}

    def run_fused():
        mhc.post_int8_pre_fused(inp["x"], yq["y_q"], yq["y_scale"], coeffs_in, None, inp["bias_next"],
                                inp["gamma_next"], ws=ws, outs=outs, phi_packed=packed)

    for _ in range(max(3, args.warmup)):
        run_fused()
    torch.cuda.synchronize()
    for a, b in evs:
        a.record(stream)
        run_fused()
        b.record(stream)
    torch.cuda.synchronize()
    fus = sum(a.elapsed_time(b) for a, b in evs) / n * 1e3
    fbytes = T * (19 * C + 180)
    res["fused_us"] = fus
    res["fused_frac_of_peak"] = fbytes / (fus * 1e-6) / 1e9 / HBM_PEAK_GBS
    return res


def main() -> int:
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", default="prefill", choices=["prefill", "decode", "mxfp8", "long"])
    ap.add_argument("--settle-ms", type=float, default=50.0,
                    help="untimed steps for this long before the warm-up steps (clock ramp)")
    ap.add_argument("--cold-phi", type=int, default=0, metavar="N",
                    help="rotate N prepacked next-layer projections (no repack in the step), so that the "
                         "projection is read cold")
    ap.add_argument("--post-int8", action="store_true",
                    help="also time the post of an int8 sublayer output with per-token scales (mhc_post_int8)")
    ap.add_argument("--pre-broadcast", action="store_true",
                    help="also time the first-layer pre of a [T, C] input (mhc_pre_broadcast)")
    ap.add_argument("--graph", action="store_true",
                    help="capture the step (repack + fused call) in one HIP graph and time its replays")
    ap.add_argument("--graph-steps", type=int, default=1, metavar="N",
                    help="with --graph: capture N steps in the graph (one replay runs N steps)")
    ap.add_argument("--defer-sinkhorn", action="store_true",
                    help="fused call with the Sinkhorn deferred (MHC_FLAG_DEFER_SINKHORN) and mhc_sinkhorn on a "
                         "side stream after an event; the next step's repack overlaps it")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--unfused", action="store_true",
                    help="also time the unfused chain post -> coeffs -> pre on the same inputs "
                         "(default for the long workload)")
    ap.add_argument("--copy-probe", action="store_true", help="run the counter-calibration copy and exit")
    ap.add_argument("--pmc-summary", nargs="+", metavar="FILE", help="summarise rocprofv3 counter output and exit")
    args = ap.parse_args()
    if args.pmc_summary:
        return pmc_summary(args.pmc_summary)
    if args.copy_probe:
        return copy_probe()
    if args.graph and (args.cold_phi or args.defer_sinkhorn):
        print(json.dumps({"error": "--graph combines with neither --cold-phi nor --defer-sinkhorn"}))
        return 2
    if args.graph and args.steps % args.graph_steps != 0:
        print(json.dumps({"error": "--steps must be a multiple of --graph-steps"}))
        return 2
    if args.gpus != 1:
        print(json.dumps({"error": "this benchmark runs on exactly one GPU; the multi-GPU path is not built "
                                   "(every token is independent, so each GPU would run this same launch on its share of the tokens)",
                          "n_gpus": args.gpus}))
        return 2

    pool = nproc = None
    if not args.no_cpu_baseline:
        pool, nproc = start_oracle_pool()
    try:
        return run(args, pool, nproc)
    finally:
        if pool is not None:
            pool.terminate()
            pool.join()


def run(args, pool, nproc) -> int:
    import torch

    import manifold_constrained_hyper_mhc_amd as mhc
    from manifold_constrained_hyper_mhc_amd.params import Params
    from manifold_constrained_hyper_mhc_amd.synthetic import WORKLOADS, make_inputs

    if not torch.cuda.is_available():
        print(json.dumps({"error": "no GPU visible"}))
        return 1
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    w = WORKLOADS[args.workload]
    T, C = w.T, w.C
    mx = args.workload == "mxfp8"
    params = Params()
    sched = mhc.schedule(T, C)
    print(f"[bench] workload={w.name} T={T} C={C} mxfp8={mx} steps={args.steps} warmup={args.warmup} "
          f"schedule={sched} graph={args.graph}", file=sys.stderr, flush=True)
    inp = make_inputs(T, C, seed=0, rows=w.rows, device=dev)
    # incoming coefficients of this layer: computed by the library itself
    coeffs_in = mhc.coeffs(inp["x"], inp["phi"], inp["bias"], params)
    ws = mhc.workspace(T, C, dev)
    packed = torch.empty(int(mhc.lib().mhc_phi_packed_bytes(C)), dtype=torch.uint8, device=dev)
    # the outputs as the library allocates them (x_out and h placed off the
    # alignment of x and y modulo 1 KiB: binding.PLACE_OFFSET)
    with_h = not mx
    outs = mhc.fused_outputs(inp["x"], inp["y"], mxfp8=mx, want_h=with_h)
    stream = torch.cuda.current_stream(dev)

    # the two calls of a step, checked and marshalled once (mhc.Prepared)
    pack = mhc.prepare_pack_phi(inp["phi_next"], packed)
    fused = mhc.prepare_post_pre_fused_prepacked(inp["x"], inp["y"], coeffs_in, packed, inp["bias_next"],
                                                 inp["gamma_next"], params, mxfp8=mx, want_h=with_h, ws=ws, outs=outs,
                                                 defer_sinkhorn=args.defer_sinkhorn)
    pack()
    fused()
    torch.cuda.synchronize()
    sink = None
    if args.defer_sinkhorn:
        # the deferred Sinkhorn of each step on a side stream, after an event
        # recorded behind the fused call; the next step's fused call (which
        # rewrites the coefficients) waits for it, its repack does not
        side = torch.cuda.Stream(device=dev)
        sink = mhc.prepare_sinkhorn(outs["coeffs_next"], params, stream=side)
        sink_ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
                   for _ in range(args.steps)]
        fused_done, sink_done = torch.cuda.Event(), torch.cuda.Event()
        sink_done.record(side)
    steps_per_call = 1
    if args.graph:
        # graph_steps whole steps captured in one HIP graph (the library
        # allocates and synchronises nothing on its call path), then replayed:
        # one replay per graph_steps steps
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph):
            for _ in range(args.graph_steps):
                mhc.prepare_pack_phi(inp["phi_next"], packed)()
                mhc.post_pre_fused_prepacked(inp["x"], inp["y"], coeffs_in, packed, inp["bias_next"],
                                             inp["gamma_next"], params, mxfp8=mx, want_h=with_h, ws=ws, outs=outs)
        torch.cuda.synchronize()
        steps_per_call = args.graph_steps

        def pack():
            pass

        fused = graph.replay

    if args.cold_phi:
        # next-layer projections that do not stay in the caches: cold_phi
        # prepacked sets (4.6 MB each at C = 7168), one per step in turn, and
        # no repack in the step
        gen = torch.Generator(device=dev)
        gen.manual_seed(1)
        cold = []
        for _ in range(args.cold_phi):
            ph = torch.randn((4 * C, 24), generator=gen, device=dev) * 0.02
            pk = mhc.pack_phi(ph)
            cold.append(mhc.prepare_post_pre_fused_prepacked(inp["x"], inp["y"], coeffs_in, pk, inp["bias_next"],
                                                             inp["gamma_next"], params, mxfp8=mx, want_h=with_h,
                                                             ws=ws, outs=outs))
            del ph
        torch.cuda.synchronize()
        turn = [0]

        def pack():
            pass

        def fused():
            cold[turn[0] % len(cold)]()
            turn[0] += 1

    def step(ev=None, k=None):
        pack()
        if sink is not None:
            stream.wait_event(sink_done)
        if ev is not None:
            ev[0].record(stream)
        fused()
        if ev is not None:
            ev[1].record(stream)
        if sink is not None:
            fused_done.record(stream)
            side.wait_event(fused_done)
            if k is not None:
                sink_ev[k][0].record(side)
            sink()
            if k is not None:
                sink_ev[k][1].record(side)
            sink_done.record(side)

    # The GPU's clocks ramp for the first ~10-20 ms of sustained load after
    # an idle period (a fused pass measured 5% slower over its first ~30
    # launches in a fresh process): untimed steps until settle_ms of device
    # time have passed, then the W warm-up steps, then the K timed steps.
    settle_steps = 0
    settle0 = time.perf_counter()
    while (time.perf_counter() - settle0) * 1e3 < args.settle_ms:
        for _ in range(10):
            step()
        settle_steps += 10
        torch.cuda.synchronize()
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    n_calls = args.steps // steps_per_call
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(n_calls)]
    t_start, t_end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    wall0 = time.perf_counter()
    t_start.record(stream)
    for k in range(n_calls):
        step(evs[k], k)
    t_end.record(stream)
    if sink is not None:
        stream.wait_event(sink_done)
    torch.cuda.synchronize()
    wall = time.perf_counter() - wall0
    total_ms = t_start.elapsed_time(t_end)
    ms_per_step = total_ms / args.steps
    # (with a graph of several steps, one bracket covers steps_per_call steps)
    kern_ms = [a.elapsed_time(b) / steps_per_call for a, b in evs]
    kern_avg_ms = sum(kern_ms) / len(kern_ms)
    sink_us = None
    if sink is not None:
        sink_us = sum(a.elapsed_time(b) for a, b in sink_ev) / len(sink_ev) * 1e3
    kern_sorted = sorted(kern_ms)
    # a bounded wait that expired makes the outputs of that call invalid: the
    # run is then not a measurement of the pass
    err_word = int(ws[:4].view(torch.int32).item())
    if err_word != 0:
        print(f"[bench] ERROR: workspace error word {err_word}: a bounded wait expired, the outputs are invalid",
              file=sys.stderr, flush=True)

    nbytes = algorithmic_bytes(T, C, mx, with_h)
    achieved = nbytes / (kern_avg_ms * 1e-3) / 1e9
    print(f"[bench] step {ms_per_step * 1e3:.1f} us, fused kernel avg {kern_avg_ms * 1e3:.1f} us "
          f"(p10 {kern_sorted[len(kern_sorted) // 10] * 1e3:.1f}, p90 {kern_sorted[9 * len(kern_sorted) // 10] * 1e3:.1f}),"
          f" {achieved:.0f} GB/s algorithmic = {achieved / HBM_PEAK_GBS:.3f} of peak; wall {wall:.3f} s",
          file=sys.stderr, flush=True)

    unfused = None
    if args.unfused or args.workload == "long":
        unfused = time_unfused(mhc, inp, coeffs_in, packed, params, outs, stream, args, nbytes, kern_avg_ms)
        print(f"[bench] unfused chain post -> coeffs -> pre: {unfused['chain_us']:.1f} us "
              f"(post {unfused['post_us']:.1f}, coeffs {unfused['coeffs_us']:.1f}, pre {unfused['pre_us']:.1f}); "
              f"fused pass {kern_avg_ms * 1e3:.1f} us", file=sys.stderr, flush=True)

    first = None
    if args.pre_broadcast:
        first = time_pre_broadcast(mhc, inp, packed, params, stream, args)
        print(f"[bench] first-layer pre (broadcast [T, C] input): {first['us']:.1f} us, {first['gbs']:.0f} GB/s "
              f"algorithmic ({first['frac_of_peak']:.3f} of peak)", file=sys.stderr, flush=True)

    pq = None
    if args.post_int8:
        pq = time_post_int8(mhc, inp, coeffs_in, stream, args)
        print(f"[bench] post of int8 y: {pq['us']:.1f} us, {pq['gbs']:.0f} GB/s algorithmic "
              f"({pq['frac_of_peak']:.3f} of peak); fused post -> next pre of int8 y: {pq['fused_us']:.1f} us "
              f"({pq['fused_frac_of_peak']:.3f} of peak)", file=sys.stderr, flush=True)

    copy_ref = copy_reference(inp, outs, stream, args, achieved)
    print(f"[bench] plain copy of x and y: {copy_ref['us']:.1f} us, {copy_ref['gbs']:.0f} GB/s "
          f"({copy_ref['frac_of_peak']:.3f} of peak); the fused pass runs at "
          f"{copy_ref['fused_gbs_over_copy_gbs']:.3f} of it", file=sys.stderr, flush=True)
    cus = torch.cuda.get_device_properties(dev).multi_processor_count
    S = C // 128
    lanes = max(1, min((cus - 32) // S, 256 // S))
    ceiling = copy_ceiling(inp, stream, args, achieved, lanes)
    print("[bench] hand-written ceilings of x and y: " + ", ".join(
        f"{k} {v['gbs']:.0f} GB/s ({v['frac_of_peak']:.3f}, {v['destination']})" for k, v in ceiling.items()
        if isinstance(v, dict) and "gbs" in v), file=sys.stderr, flush=True)
    print("[bench] piece copy by piece width: " + ", ".join(
        f"{k} {v:.0f} GB/s" for k, v in ceiling["piece_width_sweep_gbs"].items()), file=sys.stderr, flush=True)

    cpu = None
    if not args.no_cpu_baseline:
        n_s = min(T, 1024)
        host = {k: inp[k][:n_s].cpu() for k in ("x", "y")}
        host.update({k: inp[k].cpu() for k in ("phi_next", "bias_next", "gamma_next")})
        cpu = cpu_baseline(pool, nproc, host, coeffs_in[:n_s].cpu(), params)
        print(f"[bench] cpu oracle {cpu['value']:.1f} tokens/s on {cpu['cores']} processes of one thread (one thread alone: {cpu['value_1_thread']:.1f})", file=sys.stderr, flush=True)

    rows = {"normal": "N(0,1)", "outliers": "N(0,1), 1% of rows x100", "decades": "N(0,1) x 10^U(-2,3) per row"}[w.rows]
    line = {
        "metric": METRIC,
        "value": T / (ms_per_step * 1e-3),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "settle": {"ms": args.settle_ms, "steps": settle_steps},
        "ms_per_step": ms_per_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": f"{w.name}: fused post->pre (" + (
                       f"fused pass per step, one of {args.cold_phi} prepacked projections in turn)" if args.cold_phi
                       else "projection repack + fused pass per step)"),
                   "tokens": T, "hidden": C, "routes": 4, "mxfp8": mx, "bf16_h": with_h, "rows": rows,
                   "schedule": sched, "hip_graph": bool(args.graph),
                   "graph_steps": steps_per_call if args.graph else None,
                   "defer_sinkhorn": bool(args.defer_sinkhorn),
                   "parallelism": "single GPU"},
        "roofline": {"bound": "hbm", "achieved": achieved, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": achieved / HBM_PEAK_GBS, "traffic": stored_traffic(args.workload, sched),
                     "kernel": KERNEL_NAMES[sched], "kernel_avg_us": kern_avg_ms * 1e3,
                     "algorithmic_bytes": nbytes},
        "cpu_baseline": cpu,
    }
    line["copy_reference"] = copy_ref
    line["copy_ceiling"] = ceiling
    if sink_us is not None:
        line["deferred_sinkhorn"] = {
            "fused_call_us": kern_avg_ms * 1e3, "sinkhorn_us": sink_us,
            "note": "the fused call (critical path: h complete at its end) on the main stream; mhc_sinkhorn on a "
                    "side stream after an event, overlapping the next step's repack"}
    if first is not None:
        line["pre_broadcast"] = first
    if pq is not None:
        line["post_int8"] = pq
    if unfused is not None:
        line["unfused_chain"] = unfused
    if err_word != 0:
        line["invalid"] = f"workspace error word {err_word}: a bounded wait expired during the timed steps"
        line["value"] = None
    print(json.dumps(line), flush=True)
    return 3 if err_word != 0 else 0


if __name__ == "__main__":
    sys.exit(main())
