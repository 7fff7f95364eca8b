#!/usr/bin/env python3
"""all_reduce bandwidth of R logical ranks on one MI355X.

One step is one pass of the measured workload: 8 logical ranks, 16,777,216
float32 elements (64 MiB) per rank, out of place, all_reduce Sum then
all_reduce Mean (two launches of the direct R-way kernel).  Inputs are seeded
synthetic N(0,1) buffers resident in HBM before the timed region.

Printed: one JSON line with the metric (algbw = N * 4 bytes / time per
all_reduce, in GB/s), the roofline of the dominant kernel (algorithmic HBM
bytes 2*R*N*4 per launch over its average duration, measured with HIP events
on the launch stream), the CPU oracle timed on the host cores (one core, and
all cores on independent blocks of the ring segments), and per-row context
for every other collective and workload.

    python bench.py [--steps K] [--warmup W] [--no-rows] [--no-cpu-baseline]

Profiling (rocprofv3 runs whose summaries are kept under profiles/):

    python bench.py --profile SET            # run only SET's calls (see PROFILE_SETS)
    python bench.py --summarize-profile DIR --profile SET
        # DIR holds rocprofv3 CSV output of that SET in DIR/trace, DIR/fetch
        # and DIR/write (kernel trace, FETCH_SIZE, WRITE_SIZE): writes
        # profiles/SET_kernel_stats.md and profiles/traffic_SET.txt
"""

import argparse
import csv
import ctypes
import glob
import hashlib
import json
import os
import re
import sys
import time
from pathlib import Path

ROOT = Path(__file__).resolve().parent
# the library reports each occupancy-tuner choice on stderr
os.environ.setdefault("RC_TUNE_LOG", "1")
if str(ROOT) not in sys.path:
    sys.path.insert(0, str(ROOT))

METRIC = "all_reduce algbw GB/s, fp32, R=8 ranks, 64 MiB/rank; % of HBM peak"
HBM_PEAK_GBPS = 8000.0  # MI355X HBM3E, published
CSRC = ROOT / "rank_reductions_amd" / "csrc"
# the sources that decide what the kernels compile to (a traffic summary
# applies to the kernels it was taken on only)
KERNEL_SOURCES = [CSRC / n for n in ("tiling.h", "kernels_impl.h", "kernels_fold.hip", "kernels_batch.hip",
                                     "kernels_copy.hip")]
PROFILES = ROOT / "profiles"
METRIC_KERNEL = "fold_table_kernel<8, OpSumF32, 1, true>"
# launches the occupancy tuner times on a shape's first calls: three
# occupancies, five launches each (rc_config.waves_per_cu in include/rc.h)
TUNER_LAUNCHES = 15


def log(msg):
    print(msg, file=sys.stderr, flush=True)


def parse():
    p = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=50)
    p.add_argument("--warmup", type=int, default=5)
    p.add_argument("--algo", default="auto", choices=["auto", "direct", "ring"])
    p.add_argument("--tile-elems", type=int, default=0)
    p.add_argument("--max-workgroups", type=int, default=0)
    p.add_argument("--cache-hint", default="auto", choices=["auto", "streaming", "normal"])
    p.add_argument("--no-rows", action="store_true",
                   help="skip the other collectives and the flushed per-call timing")
    p.add_argument("--layers", type=int, default=32,
                   help="layers of the transformer gradient list in the batched rows (32: all 289 tensors)")
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--cpu-seconds", type=float, default=10.0, help="seconds of oracle work per CPU leg")
    p.add_argument("--profile", default=None, help="run only this profile set's calls and exit")
    p.add_argument("--summarize-profile", default=None, metavar="DIR",
                   help="summarize rocprofv3 output of --profile SET found in DIR into profiles/")
    return p.parse_args()


# ---------------------------------------------------------------- timing

def ev(torch):
    return torch.cuda.Event(enable_timing=True)


def time_calls(torch, fn, iters, warmup=18):
    """Device time in ms per call of `iters` back-to-back calls (HIP events on
    torch's current stream, which every call below is launched on)."""
    for _ in range(warmup):
        fn()
    torch.cuda.synchronize()
    a, b = ev(torch), ev(torch)
    a.record()
    for _ in range(iters):
        fn()
    b.record()
    b.synchronize()
    return a.elapsed_time(b) / iters


def time_rotating(torch, fns, iters, warmup=None):
    """Device time in ms per call, back to back, cycling over calls on
    distinct buffer sets (fns[k] uses set k).  The sets are chosen so that the
    data each call touches was last touched over 1 GiB of traffic earlier:
    far more than the 256 MB Infinity Cache holds, so every call reads from
    HBM, as in a stream of collectives on fresh data, while launches still
    pipeline as they would there."""
    K = len(fns)
    # the occupancy tuner's fifteen calibrating launches fall in the warm-up
    for i in range(warmup if warmup is not None else max(2 * K, 18)):
        fns[i % K]()
    torch.cuda.synchronize()
    a, b = ev(torch), ev(torch)
    a.record()
    for i in range(iters):
        fns[i % K]()
    b.record()
    b.synchronize()
    return a.elapsed_time(b) / iters


def flush_cache(scratch, sink):
    """Evicts the Infinity Cache by reading a 512 MiB scratch buffer (a read
    leaves no dirty lines to be written back during the next call)."""
    sink.copy_(scratch.sum().view(1))


def cold_samples(torch, fn, iters, scratch, sink, warmup=8):
    """Device time in ms of each of `iters` calls timed one at a time, each
    after a cache flush (untimed); HIP events bracket the call alone, so each
    sample includes the launch latency that back-to-back calls hide.
    Returned sorted."""
    for _ in range(warmup):
        fn()
    torch.cuda.synchronize()
    evs = [(ev(torch), ev(torch)) for _ in range(iters)]
    for a, b in evs:
        flush_cache(scratch, sink)
        a.record()
        fn()
        b.record()
    torch.cuda.synchronize()
    return sorted(a.elapsed_time(b) for a, b in evs)


def rotation_sets(bytes_per_call):
    """Buffer sets for time_rotating: enough that >= 1 GiB of traffic passes
    between two calls on one set."""
    return max(3, min(16, -(-(1 << 30) // max(bytes_per_call, 1)) + 1))


def kernels_sha():
    h = hashlib.sha256()
    for p in KERNEL_SOURCES:
        h.update(p.name.encode() + b"\0" + p.read_bytes())
    return h.hexdigest()


def read_traffic_file(path, kernel):
    """HBM bytes per launch of `kernel` from a committed rocprofv3 counter
    summary, if it was taken on the current kernel sources; else None."""
    if not path.exists():
        return None
    vals = {}
    for line in path.read_text().splitlines():
        if "=" in line and not line.lstrip().startswith("#"):
            k, v = line.split("=", 1)
            vals[k.strip()] = v.strip()
    if vals.get("kernels_sha256") != kernels_sha():
        return None
    try:
        return int(float(vals[f"{kernel}.fetch_bytes_per_launch"]) + float(vals[f"{kernel}.write_bytes_per_launch"]))
    except (KeyError, ValueError):
        return None


def _roof(bytes_moved, us):
    gbps = bytes_moved / (us * 1e-6) / 1e9
    return {"us": round(us, 2), "hbm_GBps": round(gbps, 1), "frac": round(gbps / HBM_PEAK_GBPS, 4)}


def _roof_rot(bytes_moved, us_rot, flushed=None):
    """A row timed back to back over rotating buffer sets, with the median
    of one-at-a-time flushed calls beside it when given."""
    row = _roof(bytes_moved, us_rot)
    row["timing"] = "back to back over rotating buffer sets (cold data, >= 1 GiB of traffic between reuses)"
    if flushed is not None:
        row["flushed_median_us"] = round(flushed, 2)
        row["flushed_frac"] = round(bytes_moved / (flushed * 1e-6) / 1e9 / HBM_PEAK_GBPS, 4)
    return row


# ---------------------------------------------------------------- main

def main():
    args = parse()
    if args.summarize_profile:
        summarize_profile(Path(args.summarize_profile), args.profile or "all_reduce_r8_f32_64MiB")
        return
    if args.gpus != 1:
        print(f"bench.py measures one GPU only: the logical ranks all live in one GPU's HBM, and "
              f"the library has no multi-GPU path (asked for --gpus {args.gpus}).", file=sys.stderr)
        sys.exit(2)

    import torch

    import rank_reductions_amd as rr
    import synth_inputs as si

    torch.cuda.set_device(0)
    dev = "cuda:0"
    if args.profile:
        run_profile_set(args.profile, torch, rr, si, dev)
        return
    lib = rr.library()
    props = torch.cuda.get_device_properties(0)
    log(f"bench: device {props.name} {getattr(props, 'gcnArchName', '')} CUs={props.multi_processor_count}")

    w = si.WORKLOADS["ranks8_64MiB_f32"]
    R, N = w["R"], w["N"]
    log(f"bench: generating inputs R={R} N={N}")
    xs = si.torch_rank_inputs(R, N, "f32", w["dist"], w["seed"], device=dev)
    out_sum = [torch.empty_like(x) for x in xs]
    out_mean = [torch.empty_like(x) for x in xs]
    rr.register(R, device=0, algo=args.algo, tile_elems=args.tile_elems,
                max_workgroups=args.max_workgroups, cache_hint=args.cache_hint)
    stream = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    b_sum = rr.make_bufs([x.data_ptr() for x in xs], [o.data_ptr() for o in out_sum], (N,), rr.RC_F32, rr.RC_SUM)
    b_mean = rr.make_bufs([x.data_ptr() for x in xs], [o.data_ptr() for o in out_mean], (N,), rr.RC_F32, rr.RC_MEAN)
    p_sum = ctypes.cast(b_sum, ctypes.c_void_p)
    p_mean = ctypes.cast(b_mean, ctypes.c_void_p)
    all_reduce = lib.rc_all_reduce

    def call(p):
        rc = all_reduce(p, stream)
        if rc:
            raise rr.CollectiveError(rc, lib.rc_last_error().decode())

    def step():
        call(p_sum)
        call(p_mean)

    # The occupancy tuner times its candidates on a shape's first launches
    # (TUNER_LAUNCHES of them) and settles on the call that reads their
    # times.  Run those calls, then the warm-up, so that every timed launch
    # uses the settled occupancy.
    tuner_calls = 0
    for _ in range((TUNER_LAUNCHES + 1) // 2):
        step()
        tuner_calls += 2
    torch.cuda.synchronize()
    step()
    tuner_calls += 2
    torch.cuda.synchronize()
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    log(f"bench: {tuner_calls} calls for the occupancy tuner, {args.warmup} warm-up steps; timing {args.steps} steps")
    a, b = ev(torch), ev(torch)
    wall0 = time.perf_counter()
    a.record()
    for _ in range(args.steps):
        step()
    b.record()
    b.synchronize()
    ms = a.elapsed_time(b)
    wall = time.perf_counter() - wall0
    launches_per_call = 2 if args.algo == "ring" else 1
    ms_per_step = ms / args.steps
    calls_per_step = 2
    per_call_s = ms_per_step / calls_per_step / 1e3
    algbw = N * 4 / per_call_s / 1e9
    hbm_bytes = 2 * R * N * 4  # read R*N, write R*N elements per all_reduce
    launch_ms = ms / (args.steps * calls_per_step * launches_per_call)
    achieved = (hbm_bytes / launches_per_call) / (launch_ms / 1e3) / 1e9
    same = all(torch.equal(out_sum[0], o) for o in out_sum) and all(torch.equal(out_mean[0], o) for o in out_mean)
    log(f"bench: {ms_per_step:.4f} ms/step, algbw {algbw:.1f} GB/s, HBM {achieved:.1f} GB/s, "
        f"{100 * achieved / HBM_PEAK_GBPS:.1f}% of peak; ranks identical: {same}; wall {wall:.3f}s")

    # plain device copy of the same bytes: the practical ceiling, for context
    src = torch.empty(R * N, dtype=torch.float32, device=dev)
    dst = torch.empty_like(src)
    copy_ms = time_calls(torch, lambda: dst.copy_(src), 20)
    copy_gbps = 2 * src.numel() * 4 / (copy_ms / 1e3) / 1e9
    # the library's own 1 -> 1 copy of the same bytes (send/recv between two
    # ranks: the whole-tile copy kernel), on torch's current stream like the rest
    lib_copy_ms = time_calls(torch, lambda: rr.send_recv(src, 0, 1, out=dst), 20)
    lib_copy_gbps = 2 * src.numel() * 4 / (lib_copy_ms / 1e3) / 1e9
    del src, dst
    log(f"bench: device copy of {R * N * 4 >> 20} MiB: {copy_ms * 1e3:.1f} us, {copy_gbps:.1f} GB/s; "
        f"the library's send/recv: {lib_copy_ms * 1e3:.1f} us, {lib_copy_gbps:.1f} GB/s")

    # the same call timed one at a time after a cache flush: median and best
    # (skipped with --no-rows, so that a profiled run holds only the timed steps)
    cold = []
    if not args.no_rows:
        scratch = torch.empty(128 << 20, dtype=torch.float32, device=dev)
        sink = torch.empty(1, dtype=torch.float32, device=dev)
        cold = cold_samples(torch, lambda: call(p_sum), 50, scratch, sink)
        del scratch, sink
        cold_med, cold_best = cold[len(cold) // 2], cold[0]
        log(f"bench: one call at a time, cache flushed: median {cold_med * 1e3:.1f} us, "
            f"best {cold_best * 1e3:.1f} us")

    result = {
        "all_reduce_r8_f32_64MiB": METRIC,
        "value": round(algbw, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 6),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "config": {
            "workload": "ranks8_64MiB_f32: 8 logical ranks x 16,777,216 fp32 (64 MiB) per rank, "
                        "N(0,1) seed 1, out of place; step = all_reduce Sum + all_reduce Mean",
            "ranks": R,
            "elems_per_rank": N,
            "algo": args.algo,
            "tile_elems": args.tile_elems,
            "max_workgroups": args.max_workgroups,
            "cache_hint": args.cache_hint,
        },
        "roofline": {
            "bound": "hbm",
            "achieved": round(achieved, 1),
            "peak": HBM_PEAK_GBPS,
            "unit": "GB/s",
            "frac": round(achieved / HBM_PEAK_GBPS, 4),
            "traffic": read_traffic_file(PROFILES / "traffic_all_reduce_r8_f32_64MiB.txt", METRIC_KERNEL)
            if args.algo != "ring" else None,
            "kernel": METRIC_KERNEL if args.algo != "ring" else "ring phases",
            "algorithmic_bytes_per_launch": hbm_bytes // launches_per_call,
            "avg_launch_us": round(launch_ms * 1e3, 2),
        },
        "hbm_frac": round(achieved / HBM_PEAK_GBPS, 4),
        "tuner_calls_before_warmup": tuner_calls,
        "ranks_bit_identical": bool(same),
        "copy_ceiling": {"bytes": 2 * R * N * 4, "us": round(copy_ms * 1e3, 2), "GBps": round(copy_gbps, 1),
                         "what": "torch device-to-device copy of R*N fp32"},
        "copy_ceiling_library": {"bytes": 2 * R * N * 4, "us": round(lib_copy_ms * 1e3, 2),
                                 "GBps": round(lib_copy_gbps, 1),
                                 "what": "send_recv of the same R*N fp32 (copy_full_kernel<1>)",
                                 "metric_over_copy": round(achieved / lib_copy_gbps, 4)},
    }
    if cold:
        result["per_call_flushed"] = {
            "op": "all_reduce Sum", "calls": len(cold),
            "timing": "HIP events around each call, after an untimed 512 MiB scratch read that evicts the "
                      "Infinity Cache",
            "median_us": round(cold_med * 1e3, 2), "best_us": round(cold_best * 1e3, 2),
            "median_algbw_GBps": round(N * 4 / (cold_med / 1e3) / 1e9, 1),
            "best_algbw_GBps": round(N * 4 / (cold_best / 1e3) / 1e9, 1),
            "median_frac": round(hbm_bytes / (cold_med / 1e3) / 1e9 / HBM_PEAK_GBPS, 4),
        }

    if not args.no_cpu_baseline:
        result["cpu_baseline"] = cpu_baseline(torch, xs, out_sum, args.cpu_seconds)

    if not args.no_rows:
        rr.finish()
        del out_mean
        result["rows"] = rows(torch, rr, si, dev, xs, args)
        rr.register(R, device=0)

    rr.finish()
    print(json.dumps(result), flush=True)


# ---------------------------------------------------------------- rows

def prepared(torch, rr, name, sends, recvs, op="sum", root=0):
    """One collective's C call with its argument block built once, as the
    metric loop calls: no per-call marshalling in Python, whose host time
    would otherwise pace back-to-back calls of kernels that take tens of
    microseconds.  The first call checks the arguments like any other."""
    lib = rr.library()
    fn = getattr(lib, name)
    descr = [s if s is not None else r for s, r in zip(sends, recvs)]
    shapes = [tuple(t.shape) if t is not None else () for t in descr]
    dtypes = [rr.RC_I32 if t is not None and t.dtype == torch.int32 else rr.RC_F32 for t in descr]
    bufs = rr.make_bufs([t.data_ptr() if t is not None else None for t in sends],
                        [t.data_ptr() if t is not None else None for t in recvs], shapes, dtypes, rr.OPS[op], root)
    p = ctypes.cast(bufs, ctypes.c_void_p)
    stream = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)

    def call():
        rc = fn(p, stream)
        if rc:
            raise rr.CollectiveError(rc, lib.rc_last_error().decode())

    call.keep = bufs  # the argument block lives as long as the call
    return call


def prepared_send_recv(torch, rr, x, out, src, dst):
    lib = rr.library()
    bufs = rr.make_bufs([x.data_ptr(), None], [None, out.data_ptr()], [tuple(x.shape), tuple(out.shape)],
                        rr.RC_F32)
    p = ctypes.cast(bufs, ctypes.c_void_p)
    stream = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)

    def call():
        rc = lib.rc_send_recv(src, dst, p, stream)
        if rc:
            raise rr.CollectiveError(rc, lib.rc_last_error().decode())

    call.keep = bufs
    return call


def prepared_all_gather_list(torch, rr, shards, outs):
    lib = rr.library()
    R = len(shards)
    bufs = rr.make_bufs([x.data_ptr() for x in shards], [None] * R, [tuple(x.shape) for x in shards], rr.RC_F32)
    recvs = (ctypes.c_void_p * (R * R))(*[outs[r][k].data_ptr() for r in range(R) for k in range(R)])
    p = ctypes.cast(bufs, ctypes.c_void_p)
    stream = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)

    def call():
        rc = lib.rc_all_gather_list(p, recvs, stream)
        if rc:
            raise rr.CollectiveError(rc, lib.rc_last_error().decode())

    call.keep = (bufs, recvs)
    return call


def small_latency(torch, rr, si, dev, scratch, sink, calls=200):
    """The pages' own example size (4 ranks x 257 fp32): launch-bound, so
    microseconds per call: device time of back-to-back calls, host time to
    issue one call through the C ABI, the device time per call when `calls`
    calls are captured in one HIP graph and replayed, and the median of
    calls timed one at a time after a cache flush (HIP events around the
    call alone: the fixed cost that every one-at-a-time timing carries)."""
    w = si.WORKLOADS["ranks4_257_f32"]
    R, n = w["R"], w["N"]
    xs = si.torch_rank_inputs(R, n, "f32", w["dist"], w["seed"], device=dev)
    outs = [torch.empty_like(x) for x in xs]
    lib = rr.library()
    s_ptr = [x.data_ptr() for x in xs]
    o_ptr = [o.data_ptr() for o in outs]
    calls_of = {
        "all_reduce_sum": (lib.rc_all_reduce, rr.make_bufs(s_ptr, o_ptr, (n,), rr.RC_F32, rr.RC_SUM)),
        "all_reduce_mean": (lib.rc_all_reduce, rr.make_bufs(s_ptr, o_ptr, (n,), rr.RC_F32, rr.RC_MEAN)),
        "reduce_sum_to_0": (lib.rc_reduce, rr.make_bufs(s_ptr, [o_ptr[0], None, None, None], (n,), rr.RC_F32,
                                                       rr.RC_SUM, 0)),
        "broadcast_from_1": (lib.rc_broadcast, rr.make_bufs([None, s_ptr[1], None, None],
                                                            [o_ptr[0], None, o_ptr[2], o_ptr[3]], (n,),
                                                            rr.RC_F32, rr.RC_SUM, 1)),
    }
    rr.register(R, device=0)
    res = {}
    for name, (fn, bufs) in calls_of.items():
        p = ctypes.cast(bufs, ctypes.c_void_p)

        def call(handle, fn=fn, p=p):
            rc = fn(p, ctypes.c_void_p(handle))
            if rc:
                raise rr.CollectiveError(rc, lib.rc_last_error().decode())

        cur = torch.cuda.current_stream().cuda_stream
        dev_us = time_calls(torch, lambda: call(cur), calls, warmup=10) * 1e3
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for _ in range(calls):
            call(cur)
        host_us = (time.perf_counter() - t0) / calls * 1e6
        torch.cuda.synchronize()
        # the same calls captured into one graph (on torch's capture stream), replayed
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            cap = torch.cuda.current_stream().cuda_stream
            for _ in range(calls):
                call(cap)
        replay_ms = time_calls(torch, g.replay, 10, warmup=2)
        del g
        single = cold_samples(torch, lambda: call(cur), 30, scratch, sink)
        res[name] = {"us_per_call": round(dev_us, 2), "host_issue_us": round(host_us, 2),
                     "graph_replay_us_per_call": round(replay_ms * 1e3 / calls, 2),
                     "one_at_a_time_flushed_median_us": round(single[len(single) // 2] * 1e3, 2)}
    rr.finish()
    return res


def rows(torch, rr, si, dev, xs8, args):
    """Every other collective at its workload's size (context, not the metric)."""
    out = {}
    R, N = len(xs8), xs8[0].numel()
    b = N * 4
    scratch = torch.empty(128 << 20, dtype=torch.float32, device=dev)  # 512 MiB, twice the cache
    sink = torch.empty(1, dtype=torch.float32, device=dev)
    log("bench: rows: small-message latency (4 x 257), back to back, graph-replayed and one at a time")
    out["latency_r4_257_f32"] = small_latency(torch, rr, si, dev, scratch, sink)

    def flushed(fn, iters=15):
        s = cold_samples(torch, fn, iters, scratch, sink)
        return s[len(s) // 2] * 1e3

    # ring all-reduce on the metric workload
    rr.register(R, device=0, algo="ring")
    o = [torch.empty_like(x) for x in xs8]
    us = time_calls(torch, prepared(torch, rr, "rc_all_reduce", xs8, o), 10) * 1e3
    # the ring moves (R+1)*N*4 bytes in and R*N*4 out: its reduce-scatter
    # phase reads every input and writes the owner's segment, the all-gather
    # phase reads that segment back and writes the other R-1 copies
    out["all_reduce_ring_r8_64MiB_f32_sum"] = {
        **_roof((2 * R + 1) * b, us), "bytes": "read (R+1)*N*4, write R*N*4",
        "algbw_GBps": round(b / (us * 1e-6) / 1e9, 1)}
    rr.finish()
    # the same all-reduce through the per-rank front end: one host thread and
    # one stream per rank, calls matched by issue order
    log("bench: rows: per-rank front end")
    out["all_reduce_per_rank_threads_r8_64MiB_f32_sum_shared_stream"] = per_rank_row(torch, rr, xs8, o, 1)
    out["all_reduce_per_rank_threads_r8_64MiB_f32_sum_8_streams"] = per_rank_row(torch, rr, xs8, o, R)
    del o
    # a length whose ring segments start 4 bytes past a 256-byte boundary:
    # every job then begins with a short lead tile
    n_odd = N + R
    xo = si.torch_rank_inputs(R, n_odd, "f32", "normal", 1, device=dev)
    oo = [torch.empty_like(x) for x in xo]
    rr.register(R, device=0)
    us = time_calls(torch, prepared(torch, rr, "rc_all_reduce", xo, oo), 10) * 1e3
    out["all_reduce_r8_64MiB_plus_8_f32_sum"] = {**_roof(2 * R * n_odd * 4, us), "elems_per_rank": n_odd,
                                                 "segment_offset_mod_256_bytes": (-(-n_odd // R) * 4) % 256}
    del xo, oo
    # rank buffers that disagree modulo 16 bytes: views 0-3 elements into
    # larger buffers, inputs at r % 4 and outputs at (r + 1) % 4
    log("bench: rows: all_reduce over views off the 16-byte grid")
    base_in = si.torch_rank_inputs(R, N + 3, "f32", "normal", 1, device=dev)
    base_out = [torch.empty_like(x) for x in base_in]
    xm = [base_in[r][r % 4:r % 4 + N] for r in range(R)]
    om = [base_out[r][(r + 1) % 4:(r + 1) % 4 + N] for r in range(R)]
    us = time_calls(torch, prepared(torch, rr, "rc_all_reduce", xm, om), 10) * 1e3
    out["all_reduce_r8_64MiB_f32_sum_views_off_16B_grid"] = {
        **_roof(2 * R * N * 4, us), "input_offsets_elems": [r % 4 for r in range(R)],
        "output_offsets_elems": [(r + 1) % 4 for r in range(R)]}
    rr.finish()
    del base_in, base_out, xm, om
    rr.register(R, device=0)
    # the Communicator's copies on the metric workload's buffers
    log("bench: rows: all_to_all_single, all_gather list form, send/recv")
    o = [torch.empty_like(x) for x in xs8]
    us = time_calls(torch, prepared(torch, rr, "rc_all_to_all_single", xs8, o), 10) * 1e3
    out["all_to_all_single_r8_64MiB_f32"] = _roof(2 * R * b, us)
    del o
    M = N // R
    lst_bytes = (R + R * R) * M * 4
    K = rotation_sets(lst_bytes)
    srcs = [si.torch_rank_inputs(R, M, "f32", "normal", 40 + k, device=dev) for k in range(K)]
    dsts = [[[torch.empty(M, dtype=torch.float32, device=dev) for _ in range(R)] for _ in range(R)]
            for _ in range(K)]
    fns = [prepared_all_gather_list(torch, rr, srcs[k], dsts[k]) for k in range(K)]
    us = time_rotating(torch, fns, 8 * K) * 1e3
    row = _roof_rot(lst_bytes, us, flushed(fns[0]))
    row.update({"shard_MiB": M * 4 >> 20, "sets": K})
    out["all_gather_list_r8_8MiB_shards_f32"] = row
    del srcs, dsts, fns
    K = rotation_sets(2 * b)
    srcs = [si.torch_rank_inputs(1, N, "f32", "normal", 50 + k, device=dev)[0] for k in range(K)]
    dsts = [torch.empty_like(s) for s in srcs]
    fns = [prepared_send_recv(torch, rr, srcs[k], dsts[k], 0, 1) for k in range(K)]
    us = time_rotating(torch, fns, 8 * K) * 1e3
    out["send_recv_64MiB_f32"] = dict(_roof_rot(2 * b, us, flushed(fns[0])), sets=K)
    del srcs, dsts, fns
    rr.finish()
    # reduce_scatter and all_gather, 8 ranks x 256 MiB
    w = si.WORKLOADS["ranks8_256MiB_f32_rs_ag"]
    log("bench: rows: reduce_scatter / all_gather 8 x 256 MiB")
    rr.register(w["R"], device=0)
    big = si.torch_rank_inputs(w["R"], w["N"], "f32", w["dist"], w["seed"], device=dev)
    M = w["N"] // w["R"]
    shards = [torch.empty(M, dtype=torch.float32, device=dev) for _ in range(w["R"])]
    gathered = [torch.empty(w["N"], dtype=torch.float32, device=dev) for _ in range(w["R"])]
    us = time_calls(torch, prepared(torch, rr, "rc_reduce_scatter", big, shards), 10) * 1e3
    out["reduce_scatter_r8_256MiB_f32_sum"] = _roof((w["R"] + 1) * w["N"] * 4, us)
    us = time_calls(torch, prepared(torch, rr, "rc_all_gather", shards, gathered), 10) * 1e3
    out["all_gather_r8_32MiB_shards_f32"] = _roof((w["R"] + 1) * w["N"] * 4, us)
    rr.finish()
    del big, shards, gathered
    torch.cuda.empty_cache()
    # int32 workload, 4 ranks x 64 MiB, over rotating buffer sets
    w = si.WORKLOADS["ranks4_64MiB_i32"]
    log("bench: rows: int32 4 x 64 MiB")
    R4, N4 = w["R"], w["N"]
    K = rotation_sets(2 * R4 * N4 * 4)
    xi = [si.torch_rank_inputs(R4, N4, "i32", "int", w["seed"] + 100 * k, device=dev) for k in range(K)]
    oi = [[torch.empty_like(x) for x in xk] for xk in xi]
    rr.register(R4, device=0)
    c3 = {
        "all_reduce_r4_64MiB_i32_sum": (lambda k: prepared(torch, rr, "rc_all_reduce", xi[k], oi[k], "sum"),
                                        2 * R4 * N4 * 4),
        "all_reduce_r4_64MiB_i32_max": (lambda k: prepared(torch, rr, "rc_all_reduce", xi[k], oi[k], "max"),
                                        2 * R4 * N4 * 4),
        "reduce_r4_64MiB_i32_root2": (lambda k: prepared(torch, rr, "rc_reduce", xi[k],
                                                         [oi[k][r] if r == 2 else None for r in range(R4)], "sum",
                                                         2), (R4 + 1) * N4 * 4),
        "broadcast_r4_64MiB_i32_from3": (lambda k: prepared(torch, rr, "rc_broadcast",
                                                            [xi[k][3] if r == 3 else None for r in range(R4)],
                                                            [oi[k][r] if r != 3 else None for r in range(R4)],
                                                            "sum", 3), R4 * N4 * 4),
    }
    for name, (mk, nbytes) in c3.items():
        fns = [mk(k) for k in range(K)]
        us = time_rotating(torch, fns, 10 * K) * 1e3
        out[name] = dict(_roof_rot(nbytes, us, flushed(fns[0])), sets=K)
    rr.finish()
    del xi, oi, c3, fns, scratch, sink
    torch.cuda.empty_cache()
    out.update(batched_rows(torch, rr, si, dev, args.layers))
    return out


def batched_rows(torch, rr, si, dev, layers):
    """The transformer-shaped gradient list on 4 ranks (all 289 tensors of 32
    layers by default, 26.4 GB per rank): all_reduce_many, its
    allocation-free form, the parameter-keyed sync, and gradient
    accumulation fused into the sync against a separate add then the sync."""
    import random

    out = {}
    shapes = si.transformer_grad_shapes(layers=layers)
    log(f"bench: rows: batched Mean over {len(shapes)} tensors ({layers} layers)")
    w = si.WORKLOADS["ranks4_llama32_grads_f32"]
    R4 = w["R"]
    ts = [[si.torch_tensor_for(w["seed"], t, R4, r, shp, device=dev) for r in range(R4)]
          for t, shp in enumerate(shapes)]
    os_ = [[torch.empty_like(x) for x in per] for per in ts]
    elems = sum(x.numel() for x in (per[0] for per in ts))
    tag = f"r4_{layers}layer_grads_f32_mean"
    rr.register(R4, device=0)
    us = time_calls(torch, lambda: rr.all_reduce_many(ts, "mean", out=os_), 3, warmup=16) * 1e3
    row = _roof(2 * R4 * elems * 4, us)
    row.update({"tensors": len(shapes), "elems_per_rank": elems, "layers": layers})
    out[f"all_reduce_many_{tag}"] = row
    us = time_calls(torch, lambda: rr.all_reduce_many_static(ts, "mean", out=os_), 3, warmup=2) * 1e3
    row = _roof(2 * R4 * elems * 4, us)
    row.update({"tensors": len(shapes), "elems_per_rank": elems,
                "what": "rc_all_reduce_many_static: tables in the static device scratch, no allocation"})
    out[f"all_reduce_many_static_{tag}"] = row
    # the same list as per-rank maps keyed by parameter ID, each rank listing
    # its IDs in its own order
    grads = []
    for r in range(R4):
        ids = list(range(len(shapes)))
        random.Random(r).shuffle(ids)
        grads.append({t: ts[t][r] for t in ids})
    outs = [{t: os_[t][r] for t in range(len(shapes))} for r in range(R4)]
    us = time_calls(torch, lambda: rr.all_reduce_params(grads, "mean", out=outs), 3, warmup=4) * 1e3
    row = _roof(2 * R4 * elems * 4, us)
    row.update({"tensors": len(shapes), "elems_per_rank": elems})
    out[f"all_reduce_params_{tag}"] = row
    # gradient accumulation: the last microbatch added to the accumulators
    # inside the sync (one pass) against a separate elementwise add and then
    # the sync (two passes); both give the same bits.  Results go in place
    # into the accumulators' storage, so the list needs gradients plus
    # accumulators only.
    log("bench: rows: accumulated gradient sync, fused and separate")
    del outs, os_
    torch.cuda.empty_cache()
    accs = [{t: torch.empty_like(ts[t][r]).normal_(0.0, 1e-3) for t in range(len(shapes))} for r in range(R4)]
    us = time_calls(torch, lambda: rr.all_reduce_params(grads, "mean", out=accs, acc=accs), 3, warmup=16) * 1e3
    row = _roof(3 * R4 * elems * 4, us)
    row.update({"tensors": len(shapes), "elems_per_rank": elems,
                "bytes": "read acc and grad, write the output: 3*R*N*4"})
    out[f"all_reduce_params_acc_fused_{tag}"] = row

    def separate():
        for r in range(R4):
            for t in range(len(shapes)):
                accs[r][t].add_(grads[r][t])
        rr.all_reduce_params(accs, "mean", out=accs)

    us = time_calls(torch, separate, 3, warmup=2) * 1e3
    row = _roof(5 * R4 * elems * 4, us)
    row.update({"tensors": len(shapes), "elems_per_rank": elems,
                "bytes": "torch add (2 reads, 1 write) then the sync (1 read, 1 write): 5*R*N*4"})
    out[f"accumulate_then_sync_{tag}"] = row
    rr.finish()
    del ts, grads, accs
    torch.cuda.empty_cache()
    return out


def per_rank_row(torch, rr, xs, outs, n_streams, calls=100):
    """Wall time of `calls` all-reduce Sum collectives issued by R rank threads
    on n_streams streams (rank r on stream r mod n_streams), from a released
    barrier to the device's drain.  Each distinct stream beyond the launching
    rank's costs an event join per collective."""
    import threading

    R, N = len(xs), xs[0].numel()
    lib = rr.library()
    ref = outs[0].clone()  # the ring schedule's result of the same inputs
    for o in outs:
        o.fill_(float("nan"))
    torch.cuda.synchronize()
    pool = [torch.cuda.Stream() for _ in range(n_streams)]
    streams = [pool[r % n_streams] for r in range(R)]
    bufs = [rr.make_bufs([x.data_ptr()], [o.data_ptr()], (N,), rr.RC_F32, rr.RC_SUM) for x, o in zip(xs, outs)]
    warmed = threading.Barrier(R + 1)
    go = threading.Barrier(R + 1)
    bad = []

    def rank(r):
        p = ctypes.cast(bufs[r], ctypes.c_void_p)
        s = ctypes.c_void_p(streams[r].cuda_stream)
        for k in range(2 * calls):
            if k == calls:  # an untimed pass, then the timed one
                warmed.wait()
                go.wait()
            rc = lib.rc_rank_all_reduce(r, p, s)
            if rc:
                bad.append((rc, lib.rc_last_error().decode()))
                warmed.abort()
                go.abort()
                return

    for r in range(R):
        rr.rank_register(r, R, device=0)
    ts = [threading.Thread(target=rank, args=(r,)) for r in range(R)]
    for t in ts:
        t.start()
    try:
        warmed.wait()
        torch.cuda.synchronize()
        go.wait()
    except threading.BrokenBarrierError:
        pass
    t0 = time.perf_counter()
    for t in ts:
        t.join()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    for r in range(R):
        rr.rank_finish(r)
    if bad:
        raise rr.CollectiveError(*bad[0])
    row = _roof(2 * R * N * 4, wall / calls * 1e6)
    row.update({"calls": calls, "threads": R, "streams": n_streams,
                "matches_ring_bits": all(torch.equal(ref, o) for o in outs),
                "timing": "host wall clock from the released barrier to device drain"})
    return row


# ---------------------------------------------------------------- CPU baseline

def cpu_model():
    try:
        for line in Path("/proc/cpuinfo").read_text().splitlines():
            if line.lower().startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def cpu_baseline(torch, xs, out_sum, seconds):
    """The CPU oracle (ring simulation, NumPy) on this machine's host cores, on
    the metric workload's inputs (a host copy; the copy is not timed), Sum.

    One core: the oracle's all_reduce on the whole inputs, repeated for about
    `seconds`.  All cores: the same oracle on T independent sub-problems run
    in T threads, T = the cores this process may use.  Sub-problem b holds
    block b of every ring segment (segment c of rank r's input contributes
    [c*S + lo_b, c*S + hi_b)), so its own ring segments are exactly those
    blocks and every element is folded in the same rank order as in the whole
    call; gathering the blocks and placing the results are timed too.  NumPy
    releases the interpreter lock inside its array operations, so the threads
    run in parallel.  Both legs' bits are compared with the GPU's."""
    from concurrent.futures import ThreadPoolExecutor

    import numpy as np

    import oracle

    hx = [x.cpu().numpy() for x in xs]
    R, N = len(hx), hx[0].size
    gpu = out_sum[0].cpu().numpy().view(np.uint32)
    log("bench: timing the CPU oracle, one core")
    calls = 0
    t0 = time.perf_counter()
    while True:
        res = oracle.all_reduce(hx, "sum")
        calls += 1
        el = time.perf_counter() - t0
        if el >= seconds:
            break
    one_match = bool(np.array_equal(res[0].view(np.uint32), gpu))
    del res
    one = calls * N * 4 / el / 1e9

    T = len(os.sched_getaffinity(0))
    log(f"bench: timing the CPU oracle, {T} threads")
    S = N // R
    assert S * R == N
    edges = [S * i // T for i in range(T + 1)]
    full = np.empty(N, dtype=np.float32)

    def block(i, src=hx, dst=full):
        lo, hi = edges[i], edges[i + 1]
        if lo == hi:
            return
        sub = [np.concatenate([h[c * S + lo:c * S + hi] for c in range(R)]) for h in src]
        got = oracle.all_reduce(sub, "sum")[0]
        wdt = hi - lo
        for c in range(R):
            dst[c * S + lo:c * S + hi] = got[c * wdt:(c + 1) * wdt]

    pcalls = 0
    with ThreadPoolExecutor(T) as ex:
        t0 = time.perf_counter()
        while True:
            list(ex.map(block, range(T)))
            pcalls += 1
            pel = time.perf_counter() - t0
            if pel >= seconds:
                break
    all_match = bool(np.array_equal(full.view(np.uint32), gpu))
    allc = pcalls * N * 4 / pel / 1e9

    # Context only: an all-reduce staged through the host, as the pages' own
    # transfer path is (ruCCL README, section 5), with the all-cores oracle
    # as its compute: the R inputs copied to pinned host memory, folded, and
    # the result copied to every rank's output.
    log("bench: timing a host-staged all-reduce (context)")
    pin_in = [torch.empty(N, dtype=torch.float32, pin_memory=True) for _ in range(R)]
    pin_out = torch.empty(N, dtype=torch.float32, pin_memory=True)
    dev_out = [torch.empty_like(x) for x in xs]
    src, dst = [p.numpy() for p in pin_in], pin_out.numpy()
    phases = []
    with ThreadPoolExecutor(T) as ex:
        for _ in range(3):
            torch.cuda.synchronize()
            t0 = time.perf_counter()
            for p, x in zip(pin_in, xs):
                p.copy_(x)
            t1 = time.perf_counter()
            list(ex.map(lambda i: block(i, src, dst), range(T)))
            t2 = time.perf_counter()
            for o in dev_out:
                o.copy_(pin_out, non_blocking=True)
            torch.cuda.synchronize()
            phases.append((t1 - t0, t2 - t1, time.perf_counter() - t2))
    staged_match = bool(np.array_equal(dev_out[R - 1].cpu().numpy().view(np.uint32), gpu))
    best = min(phases, key=sum)
    del pin_in, pin_out, dev_out, src, dst
    host_staged = {
        "value": round(N * 4 / sum(best) / 1e9, 4), "unit": "GB/s",
        "what": "context, not a baseline of this path: device-to-host copies of the R inputs into pinned "
                "memory, the oracle on all cores, host-to-device copies of the result to every rank; "
                "best of 3 calls",
        "d2h_ms": round(best[0] * 1e3, 2), "oracle_ms": round(best[1] * 1e3, 2),
        "h2d_ms": round(best[2] * 1e3, 2), "matches_gpu_bits": staged_match}
    return {
        "value": round(allc, 4),
        "unit": "GB/s",
        "cores": T,
        "kind": "oracle",
        "sample": f"all_reduce Sum of the ring-simulation oracle on the same 8 x 16,777,216 fp32 inputs "
                  f"(host copy): {pcalls} calls in {pel:.1f} s on {T} threads, each running the oracle on "
                  f"one of {T} independent blocks of every ring segment; and {calls} whole calls in "
                  f"{el:.1f} s on one thread",
        "cpu_model": cpu_model(),
        "matches_gpu_bits": one_match and all_match,
        "one_core": {"value": round(one, 4), "unit": "GB/s", "cores": 1, "calls": calls,
                     "seconds": round(el, 2), "matches_gpu_bits": one_match},
        "all_cores": {"value": round(allc, 4), "unit": "GB/s", "cores": T, "calls": pcalls,
                      "seconds": round(pel, 2), "matches_gpu_bits": all_match},
        "host_staged_context": host_staged,
    }


# ---------------------------------------------------------------- profiling

# What each profile set runs, and the algorithmic HBM bytes of each kernel it
# launches: `per_wg` bytes per workgroup for whole-tile kernels (one round of
# 64 lanes x 16 B x unroll per stream: reads + writes), `per_call` for a
# kernel whose launches all move the same bytes.
PROFILE_SETS = {
    "all_reduce_r8_f32_64MiB": {
        "what": "all_reduce Sum and Mean, 8 ranks x 16,777,216 fp32 (64 MiB) per rank, out of place: the "
                "bench's own metric run without the other rows and the CPU legs (the 512 MiB torch copy of "
                "its copy ceiling calibrates the counters)",
        "kernels": {METRIC_KERNEL: {"per_wg": (8 + 8) * 1024}},
        # profiled as the metric is measured: the same timed loop, steps and warm-up
        "args": "--no-rows --no-cpu-baseline --steps 20 --warmup 5",
        "timed_launches": 40,  # the last launches of the metric kernel: 20 steps of Sum + Mean
        "steady": 40,
    },
    "int32_r4_64MiB": {
        "what": "int32, 4 ranks x 16,777,216 (64 MiB) per rank: all_reduce Sum and Max, reduce Sum to root 2, "
                "broadcast from rank 3; each back to back over rotating buffer sets (cold data), as the bench "
                "rows time them",
        "steady": 30,
        "kernels": {"fold_table_kernel<4, OpSumI32, 1, true>": {"per_wg": (4 + 4) * 1024},
                    "fold_table_kernel<4, OpMaxI32, 1, true>": {"per_wg": (4 + 4) * 1024},
                    "fold_table_kernel<4, OpSumI32, 2, true>": {"per_wg": (4 + 1) * 2048},
                    "copy_full_kernel<4, 2, true>": {"per_wg": (1 + 3) * 2048}},
    },
    "rs_ag_r8_f32_256MiB": {
        "what": "8 ranks x 67,108,864 fp32 (256 MiB) per rank: reduce_scatter Sum to shards of 8,388,608, "
                "then all_gather of the shards",
        "kernels": {METRIC_KERNEL: {"per_wg": (8 + 1) * 1024},
                    "copy_full_kernel<8, 2, true>": {"per_wg": (1 + 8) * 2048}},
    },
    "grads_r4_32layer_f32": {
        "what": "4 ranks, the 32-layer transformer gradient list (289 fp32 tensors, 26.4 GB per rank): "
                "all_reduce_many Mean, then the parameter-keyed sync fused with gradient accumulation",
        # steady: the launches of the last two calls (225 own launches per call of the list)
        "kernels": {"fold_table_kernel<4, OpSumF32, 1, true>": {"per_wg": (4 + 4) * 1024, "steady": 450},
                    "fold_table_acc_kernel<4, OpSumF32, 1, true>": {"per_wg": (8 + 4) * 1024, "steady": 450},
                    "batch_kernel<4, OpSumF32, 2, true, false>": {"per_call": 64 * 4096 * 4 * 8, "steady": 2},
                    "batch_kernel<4, OpSumF32, 1, true, true>": {"per_call": 64 * 4096 * 4 * 12, "steady": 2}},
    },
    "copies_r8_f32_64MiB": {
        "what": "send/recv of 64 MiB fp32 and the list all_gather of 8 shards of 8 MiB, each back to back over "
                "rotating buffer sets (cold data), all_to_all_single of 8 x 64 MiB, and an all_reduce of 8 x 64 MiB "
                "over views off the 16-byte grid (inputs at 0-3 elements, outputs at 1-3-0 elements into their "
                "buffers: the whole-tile fold with outputs shifted onto their 64-byte bursts)",
        "steady": 30,
        "kernels": {"copy_full_kernel<1, 2, true>": {"per_wg": (1 + 1) * 2048},
                    "copy_args_full_kernel<1, 2, true>": {"per_wg": (1 + 1) * 2048},
                    "copy_args_full_kernel<8, 2, true>": {"per_wg": (1 + 8) * 2048},
                    "fold_table_shift_kernel<8, OpSumF32, 1, true>": {"per_wg": (8 + 8) * 1024}},
    },
}


def profile_commands(name, dir_):
    """The three rocprofv3 runs of a profile set, as run from the repository
    root: rocprofv3 itself starts from /tmp ($OLDPWD is then the root), and
    writes under dir_ (relative to the root)."""
    base = "cd /tmp && export TMPDIR=/tmp && "
    run = f"-- python3 $OLDPWD/bench.py {PROFILE_SETS[name].get('args', '--profile ' + name)}"
    out = f"$OLDPWD/{dir_}"
    return [
        f"{base}rocprofv3 --kernel-trace --stats --output-format csv -d {out}/trace -o run {run}",
        f"{base}rocprofv3 --pmc FETCH_SIZE --output-format csv -d {out}/fetch -o run {run}",
        f"{base}rocprofv3 --pmc WRITE_SIZE --output-format csv -d {out}/write -o run {run}",
    ]


def run_profile_set(name, torch, rr, si, dev):
    """A few calls of the set's collectives (after a warm-up that lets the
    occupancy tuner settle), then a torch copy of 512 MiB: the plain copy of
    known size whose counters calibrate FETCH_SIZE and WRITE_SIZE."""
    if name not in PROFILE_SETS:
        raise SystemExit(f"unknown profile set {name!r}; sets: {', '.join(PROFILE_SETS)}")
    log(f"bench: profile set {name}: {PROFILE_SETS[name]['what']}")
    reps, warm = 4, 18
    steady = PROFILE_SETS[name].get("steady", reps)

    def rep(fn, n=reps):
        for _ in range(warm + n):
            fn()
        torch.cuda.synchronize()

    def rot(fns, n=steady):
        """Back to back over rotating buffer sets, as the bench rows time
        them: every call reads data that is not in the Infinity Cache."""
        for i in range(warm + n):
            fns[i % len(fns)]()
        torch.cuda.synchronize()

    if name == "all_reduce_r8_f32_64MiB":
        w = si.WORKLOADS["ranks8_64MiB_f32"]
        xs = si.torch_rank_inputs(w["R"], w["N"], "f32", w["dist"], w["seed"], device=dev)
        o = [torch.empty_like(x) for x in xs]
        rr.register(w["R"], device=0)
        rep(lambda: (rr.all_reduce(xs, "sum", out=o), rr.all_reduce(xs, "mean", out=o)))
    elif name == "int32_r4_64MiB":
        w = si.WORKLOADS["ranks4_64MiB_i32"]
        R, N = w["R"], w["N"]
        K = rotation_sets(2 * R * N * 4)
        xi = [si.torch_rank_inputs(R, N, "i32", "int", w["seed"] + 100 * k, device=dev) for k in range(K)]
        oi = [[torch.empty_like(x) for x in xk] for xk in xi]
        rr.register(R, device=0)
        rot([prepared(torch, rr, "rc_all_reduce", xi[k], oi[k], "sum") for k in range(K)])
        rot([prepared(torch, rr, "rc_all_reduce", xi[k], oi[k], "max") for k in range(K)])
        rot([prepared(torch, rr, "rc_reduce", xi[k], [oi[k][r] if r == 2 else None for r in range(R)], "sum", 2)
             for k in range(K)])
        rot([prepared(torch, rr, "rc_broadcast", [xi[k][3] if r == 3 else None for r in range(R)],
                      [oi[k][r] if r != 3 else None for r in range(R)], "sum", 3) for k in range(K)])
    elif name == "rs_ag_r8_f32_256MiB":
        w = si.WORKLOADS["ranks8_256MiB_f32_rs_ag"]
        R, N = w["R"], w["N"]
        xs = si.torch_rank_inputs(R, N, "f32", w["dist"], w["seed"], device=dev)
        sh = [torch.empty(N // R, dtype=torch.float32, device=dev) for _ in range(R)]
        ga = [torch.empty(N, dtype=torch.float32, device=dev) for _ in range(R)]
        rr.register(R, device=0)
        rep(lambda: rr.reduce_scatter(xs, "sum", out=sh))
        rep(lambda: rr.all_gather(sh, out=ga))
    elif name == "grads_r4_32layer_f32":
        w = si.WORKLOADS["ranks4_llama32_grads_f32"]
        R = w["R"]
        shapes = si.transformer_grad_shapes()
        ts = [[si.torch_tensor_for(w["seed"], t, R, r, shp, device=dev) for r in range(R)]
              for t, shp in enumerate(shapes)]
        os_ = [[torch.empty_like(x) for x in per] for per in ts]
        rr.register(R, device=0)
        for _ in range(18):  # fifteen of them the tuner's calibration launches
            rr.all_reduce_many(ts, "mean", out=os_)
        torch.cuda.synchronize()
        del os_
        torch.cuda.empty_cache()
        grads = [{t: ts[t][r] for t in range(len(shapes))} for r in range(R)]
        accs = [{t: torch.empty_like(ts[t][r]).normal_(0.0, 1e-3) for t in range(len(shapes))} for r in range(R)]
        for _ in range(18):
            rr.all_reduce_params(grads, "mean", out=accs, acc=accs)
        torch.cuda.synchronize()
        del ts, grads, accs
        torch.cuda.empty_cache()
    elif name == "copies_r8_f32_64MiB":
        w = si.WORKLOADS["ranks8_64MiB_f32"]
        R, N = w["R"], w["N"]
        xs = si.torch_rank_inputs(R, N, "f32", w["dist"], w["seed"], device=dev)
        o = [torch.empty_like(x) for x in xs]
        rr.register(R, device=0)
        K = rotation_sets(2 * N * 4)
        sx = [torch.empty(N, dtype=torch.float32, device=dev).normal_() for _ in range(K)]
        sy = [torch.empty_like(x) for x in sx]
        rot([prepared_send_recv(torch, rr, sx[k], sy[k], 0, 1) for k in range(K)], max(steady, 4 * K))
        del sx, sy
        rep(lambda: rr.all_to_all_single(xs, out=o), steady)
        M = N // R
        K = rotation_sets((R + R * R) * M * 4)
        shards = [[torch.empty(M, dtype=torch.float32, device=dev).normal_() for _ in range(R)] for _ in range(K)]
        lst = [[[torch.empty(M, dtype=torch.float32, device=dev) for _ in range(R)] for _ in range(R)]
               for _ in range(K)]
        rot([prepared_all_gather_list(torch, rr, shards[k], lst[k]) for k in range(K)])
        del shards, lst
        base_in = si.torch_rank_inputs(R, N + 3, "f32", "normal", 1, device=dev)
        base_out = [torch.empty_like(x) for x in base_in]
        xm = [base_in[r][r % 4:r % 4 + N] for r in range(R)]
        om = [base_out[r][(r + 1) % 4:(r + 1) % 4 + N] for r in range(R)]
        rep(lambda: rr.all_reduce(xm, "sum", out=om), steady)
    rr.finish()
    src = torch.empty(128 << 20, dtype=torch.float32, device=dev)
    dst = torch.empty_like(src)
    for _ in range(3):
        dst.copy_(src)
    torch.cuda.synchronize()
    log(f"bench: profile set {name} done")


def _short_name(name):
    s = name.replace("void ", "").replace("rc::(anonymous namespace)::", "").replace("rc::", "")
    s = re.sub(r"\((JobArgs|BatchArgs|CopyArgs|TableChunk|FoldTable)\)$", "", s.strip())
    return s.strip()


def _csv_rows(pattern):
    files = sorted(glob.glob(pattern, recursive=True))
    out = []
    for f in files:
        with open(f, newline="") as fh:
            out.extend(csv.DictReader(fh))
    return out


def summarize_profile(dir_, name):
    """Writes profiles/<name>_kernel_stats.md (per-kernel time from the trace
    run, achieved HBM rate on the algorithmic bytes, traffic over those bytes)
    and profiles/traffic_<name>.txt (FETCH_SIZE / WRITE_SIZE per dispatch,
    each scaled by what the same counter reads for the run's 512 MiB torch
    copy, the copy of known size)."""
    if name not in PROFILE_SETS:
        raise SystemExit(f"unknown profile set {name!r}; sets: {', '.join(PROFILE_SETS)}")
    spec = PROFILE_SETS[name]
    trace = _csv_rows(str(dir_ / "trace" / "**" / "*kernel_trace.csv"))
    if not trace:
        raise SystemExit(f"no kernel trace under {dir_}/trace")
    per = {}
    copy_us = []
    for row in trace:
        k = _short_name(row["Kernel_Name"])
        dur = (int(row["End_Timestamp"]) - int(row["Start_Timestamp"])) / 1e3
        items = int(row["Grid_Size_X"]) * int(row["Grid_Size_Y"]) * int(row["Grid_Size_Z"])
        wg = int(row["Workgroup_Size_X"]) * int(row["Workgroup_Size_Y"]) * int(row["Workgroup_Size_Z"])
        if k in spec["kernels"]:
            per.setdefault(k, []).append((dur, items // max(wg, 1)))
        elif "copyBuffer" in k:
            copy_us.append(dur)

    def alg_bytes(k, wgs):
        d = spec["kernels"][k]
        return d["per_wg"] * wgs if "per_wg" in d else d["per_call"]

    # counters, per kernel and dispatch; the largest torch copy calibrates
    counters, calib = {}, {}
    for ctr, sub in (("FETCH_SIZE", "fetch"), ("WRITE_SIZE", "write")):
        got = {}
        best_copy = 0.0
        for row in _csv_rows(str(dir_ / sub / "**" / "*counter_collection.csv")):
            if row.get("Counter_Name") != ctr:
                continue
            k = _short_name(row["Kernel_Name"])
            v = float(row["Counter_Value"])
            if k in spec["kernels"]:
                got.setdefault(k, []).append((v, int(row["Grid_Size"]) // 64))
            elif "copyBuffer" in k:
                best_copy = max(best_copy, v)
        counters[ctr] = got
        calib[ctr] = best_copy
    copy_kib = (512 << 20) / 1024
    scale = {c: (copy_kib / calib[c] if calib[c] else None) for c in calib}

    sha = kernels_sha()
    rel = os.path.relpath(dir_, ROOT) if dir_.is_absolute() else str(dir_)
    cmds = profile_commands(name, rel)
    md = [f"# Kernel time and HBM traffic: {name}", "",
          f"Workload: {spec['what']}.", "",
          "Commands (MI355X, ROCm 7.2; each run from the repository root), then `python3 bench.py "
          f"--summarize-profile {rel} --profile {name}` to write this file:", ""]
    md += [f"    {c}" for c in cmds]
    def steady_of(k):
        return spec["kernels"][k].get("steady", spec.get("steady", 4))

    md += ["", "| kernel | calls | avg us | min us | max us | last n | last n avg us | alg. bytes per call | "
               "achieved GB/s (last n) | % of 8 TB/s | counter bytes / alg. bytes |",
           "|---|---|---|---|---|---|---|---|---|---|---|"]
    tr = [f"# HBM traffic per launch of the {name} set's kernels, from rocprofv3 PMC counters.",
          "# FETCH_SIZE and WRITE_SIZE are KiB per dispatch; each is scaled by what it reads for a plain",
          f"# 512 MiB torch copy in the same run (FETCH_SIZE {calib['FETCH_SIZE']:.1f} KiB, WRITE_SIZE "
          f"{calib['WRITE_SIZE']:.1f} KiB, for 524288 KiB read and 524288 KiB written).",
          "# Commands:"] + [f"#   {c}" for c in cmds]
    tr.append(f"fetch_scale = {scale['FETCH_SIZE']:.6f}" if scale["FETCH_SIZE"] else "fetch_scale = none")
    tr.append(f"write_scale = {scale['WRITE_SIZE']:.6f}" if scale["WRITE_SIZE"] else "write_scale = none")
    for k in spec["kernels"]:
        if k not in per:
            md.append(f"| `{k}` | 0 | | | | | | | | | |")
            continue
        ds = [d for d, _ in per[k]]
        last = per[k][-steady_of(k):]
        last_avg = sum(d for d, _ in last) / len(last)
        alg = sum(alg_bytes(k, wg) for _, wg in last)
        gbps = alg / (sum(d for d, _ in last) * 1e-6) / 1e9
        ratio = ""
        fget, wget = counters["FETCH_SIZE"].get(k), counters["WRITE_SIZE"].get(k)
        if fget and wget and scale["FETCH_SIZE"] and scale["WRITE_SIZE"]:
            fb = sum(v for v, _ in fget) * 1024 * scale["FETCH_SIZE"] / len(fget)
            wb = sum(v for v, _ in wget) * 1024 * scale["WRITE_SIZE"] / len(wget)
            alg_f = sum(alg_bytes(k, wg) for _, wg in fget) / len(fget)
            ratio = f"{(fb + wb) / alg_f:.4f}"
            tr += [f"{k}.dispatches = {len(fget)}",
                   f"{k}.algorithmic_bytes_per_launch = {alg_f:.0f}",
                   f"{k}.fetch_bytes_per_launch = {fb:.0f}",
                   f"{k}.write_bytes_per_launch = {wb:.0f}",
                   f"{k}.traffic_over_algorithmic = {ratio}"]
        md.append(f"| `{k}` | {len(ds)} | {sum(ds) / len(ds):.1f} | {min(ds):.1f} | {max(ds):.1f} | "
                  f"{len(last)} | {last_avg:.1f} | {alg / len(last):.0f} | {gbps:.1f} | {100 * gbps / HBM_PEAK_GBPS:.1f}% | "
                  f"{ratio} |")
    timed = spec.get("timed_launches")
    if timed and per.get(METRIC_KERNEL):
        last = [d for d, _ in per[METRIC_KERNEL][-timed:]]
        avg = sum(last) / len(last)
        gbps = alg_bytes(METRIC_KERNEL, per[METRIC_KERNEL][-1][1]) / (avg * 1e-6) / 1e9
        md += ["", f"The bench's timed region (the last {len(last)} launches of `{METRIC_KERNEL}`): "
                   f"avg {avg:.1f} us, {gbps:.1f} GB/s, {100 * gbps / HBM_PEAK_GBPS:.1f}% of 8 TB/s "
                   f"(min {min(last):.1f}, max {max(last):.1f})."]
    if copy_us:
        md += ["", f"Torch copies in the traced run (host reads and the 512 MiB calibration copy): "
                   f"{len(copy_us)}, the longest {max(copy_us):.1f} us."]
    md += ["", "`avg`, `min` and `max` cover every call of the run, the occupancy tuner's calibrating launches "
               "among them; the achieved rate is over each kernel's last n launches, after the tuner settled.",
           "Algorithmic bytes: what the collective must read and write (each input element once, each output "
           "element once); the last column is the counters' scaled bytes over those.",
           f"Kernel sources sha256: {sha}"]
    tr.append(f"kernels_sha256 = {sha}")
    PROFILES.mkdir(exist_ok=True)
    (PROFILES / f"{name}_kernel_stats.md").write_text("\n".join(md) + "\n")
    (PROFILES / f"traffic_{name}.txt").write_text("\n".join(tr) + "\n")
    print("\n".join(md))


if __name__ == "__main__":
    main()
