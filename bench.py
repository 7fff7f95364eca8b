#!/usr/bin/env python3
"""all_reduce bandwidth of R logical ranks on one MI355X.

One step is one pass of the measured workload: 8 logical ranks, 16,777,216
float32 elements (64 MiB) per rank, out of place, all_reduce Sum then
all_reduce Mean (two launches of the direct R-way kernel).  Inputs are seeded
synthetic N(0,1) buffers resident in HBM before the timed region.

Printed: one JSON line with the metric (algbw = N * 4 bytes / time per
all_reduce, in GB/s), the roofline of the dominant kernel (algorithmic HBM
bytes 2*R*N*4 per launch over its average duration, measured with HIP events
on the launch stream), the CPU oracle timed on the host cores, and per-row
context for the other collectives.

    python bench.py [--steps K] [--warmup W] [--no-rows] [--no-cpu-baseline]
"""

import argparse
import ctypes
import hashlib
import json
import os
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
TRAFFIC_FILE = ROOT / "profiles" / "traffic_fold_r8_f32_sum_64MiB.txt"


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
    p.add_argument("--full-batched", action="store_true",
                   help="time the batched all-reduce on the full 32-layer gradient list (211 GB)")
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--cpu-seconds", type=float, default=12.0)
    return p.parse_args()


class Timer:
    """HIP events on torch's current stream, which is the stream every call
    below is launched on."""

    def __init__(self, torch):
        self.torch = torch
        self.a = torch.cuda.Event(enable_timing=True)
        self.b = torch.cuda.Event(enable_timing=True)

    def start(self):
        self.a.record()

    def stop_ms(self):
        self.b.record()
        self.b.synchronize()
        return self.a.elapsed_time(self.b)


def time_calls(torch, fn, iters, warmup=8):
    for _ in range(warmup):
        fn()
    torch.cuda.synchronize()
    t = Timer(torch)
    t.start()
    for _ in range(iters):
        fn()
    return t.stop_ms() / iters


def cold_samples(torch, fn, iters, scratch, warmup=8):
    """Device time in ms of each of `iters` calls with the 256 MB Infinity
    Cache flushed first: an untimed 512 MiB scratch write precedes every call,
    and HIP events bracket the call alone."""
    for _ in range(warmup):
        fn()
    torch.cuda.synchronize()
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(iters)]
    for k, (a, b) in enumerate(evs):
        scratch.fill_(k)
        a.record()
        fn()
        b.record()
    torch.cuda.synchronize()
    return [a.elapsed_time(b) for a, b in evs]


def time_cold(torch, fn, iters, scratch, warmup=8):
    """Mean of cold_samples: for rows small enough to stay cache-resident
    between back-to-back calls."""
    return sum(cold_samples(torch, fn, iters, scratch, warmup)) / iters


def kernels_sha():
    h = hashlib.sha256()
    for p in KERNEL_SOURCES:
        h.update(p.name.encode() + b"\0" + p.read_bytes())
    return h.hexdigest()


def read_traffic():
    """HBM bytes per launch from the committed rocprofv3 counter summary, if it
    was taken on the current kernel source; else None."""
    if not TRAFFIC_FILE.exists():
        return None
    vals = {}
    for line in TRAFFIC_FILE.read_text().splitlines():
        if "=" in line and not line.lstrip().startswith("#"):
            k, v = line.split("=", 1)
            vals[k.strip()] = v.strip()
    if vals.get("kernels_sha256") != kernels_sha():
        return None
    try:
        return int(float(vals["fetch_bytes_per_launch"]) + float(vals["write_bytes_per_launch"]))
    except (KeyError, ValueError):
        return None


def step_one(call, bufs, stream, lib, rr):
    rc = call(bufs, stream)
    if rc:
        raise rr.CollectiveError(rc, lib.rc_last_error().decode())


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only: the logical ranks all live in one GPU's HBM, and "
              f"the library has no multi-GPU path (asked for --gpus {args.gpus}).", file=sys.stderr)
        sys.exit(2)

    import torch

    import rank_reductions_amd as rr
    import synth_inputs as si

    torch.cuda.set_device(0)
    dev = "cuda:0"
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

    def step():
        rc = all_reduce(p_sum, stream) or all_reduce(p_mean, stream)
        if rc:
            raise rr.CollectiveError(rc, lib.rc_last_error().decode())

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    log(f"bench: timing {args.steps} steps")
    t = Timer(torch)
    wall0 = time.perf_counter()
    t.start()
    for _ in range(args.steps):
        step()
    ms = t.stop_ms()
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
        cold = sorted(cold_samples(torch, lambda: step_one(all_reduce, p_sum, stream, lib, rr), 30, scratch))
        del scratch
        cold_med, cold_best = cold[len(cold) // 2], cold[0]
        log(f"bench: one call at a time, cache flushed: median {cold_med * 1e3:.1f} us, "
            f"best {cold_best * 1e3:.1f} us")

    result = {
        "metric": METRIC,
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
            "traffic": read_traffic() if args.algo != "ring" else None,
            "kernel": "fold_full_kernel<8, OpSumF32, 1, true, false>" if args.algo != "ring" else "ring phases",
            "algorithmic_bytes_per_launch": hbm_bytes // launches_per_call,
            "avg_launch_us": round(launch_ms * 1e3, 2),
        },
        "hbm_frac": round(achieved / HBM_PEAK_GBPS, 4),
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
            "timing": "HIP events around each call, after an untimed 512 MiB scratch write that evicts the Infinity Cache",
            "median_us": round(cold_med * 1e3, 2), "best_us": round(cold_best * 1e3, 2),
            "median_algbw_GBps": round(N * 4 / (cold_med / 1e3) / 1e9, 1),
            "best_algbw_GBps": round(N * 4 / (cold_best / 1e3) / 1e9, 1),
            "median_frac": round(hbm_bytes / (cold_med / 1e3) / 1e9 / HBM_PEAK_GBPS, 4),
        }

    if not args.no_rows:
        rr.finish()
        result["rows"] = rows(torch, rr, si, dev, xs, args)
        rr.register(R, device=0)

    if not args.no_cpu_baseline:
        result["cpu_baseline"] = cpu_baseline(torch, xs, out_sum, args.cpu_seconds)

    rr.finish()
    print(json.dumps(result), flush=True)


def _roof(bytes_moved, us):
    gbps = bytes_moved / (us * 1e-6) / 1e9
    return {"us": round(us, 2), "hbm_GBps": round(gbps, 1), "frac": round(gbps / HBM_PEAK_GBPS, 4)}


def small_latency(torch, rr, si, dev, calls=200):
    """The pages' own example size (4 ranks x 257 fp32): launch-bound, so
    microseconds per call, device-side (HIP events over back-to-back calls)
    and host-side (time to issue one call through the C ABI)."""
    import ctypes

    w = si.WORKLOADS["ranks4_257_f32"]
    R, n = w["R"], w["N"]
    xs = si.torch_rank_inputs(R, n, "f32", w["dist"], w["seed"], device=dev)
    outs = [torch.empty_like(x) for x in xs]
    lib = rr.library()
    stream = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
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

        def call():
            rc = fn(p, stream)
            if rc:
                raise rr.CollectiveError(rc, lib.rc_last_error().decode())

        dev_us = time_calls(torch, call, calls, warmup=10) * 1e3
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for _ in range(calls):
            call()
        host_us = (time.perf_counter() - t0) / calls * 1e6
        torch.cuda.synchronize()
        res[name] = {"us_per_call": round(dev_us, 2), "host_issue_us": round(host_us, 2)}
    rr.finish()
    return res


def rows(torch, rr, si, dev, xs8, args):
    """Every other collective at its workload's size (context, not the metric)."""
    out = {}
    R, N = len(xs8), xs8[0].numel()
    b = N * 4
    out["latency_r4_257_f32"] = small_latency(torch, rr, si, dev)
    scratch = torch.empty(128 << 20, dtype=torch.float32, device=dev)  # 512 MiB, twice the cache
    # ring all-reduce on the metric workload
    rr.register(R, device=0, algo="ring")
    o = [torch.empty_like(x) for x in xs8]
    us = time_calls(torch, lambda: rr.all_reduce(xs8, "sum", out=o), 10) * 1e3
    # the ring moves (R+1)*N*4 bytes in and R*N*4 out: its reduce-scatter
    # phase reads every input and writes the owner's segment, the all-gather
    # phase reads that segment back and writes the other R-1 copies
    out["all_reduce_ring_r8_64MiB_f32_sum"] = {
        **_roof((2 * R + 1) * b, us), "bytes": "read (R+1)*N*4, write R*N*4",
        "algbw_GBps": round(b / (us * 1e-6) / 1e9, 1)}
    rr.finish()
    # the same all-reduce through the per-rank front end: one host thread and
    # one stream per rank, calls matched by issue order
    out["all_reduce_per_rank_threads_r8_64MiB_f32_sum_shared_stream"] = per_rank_row(torch, rr, xs8, o, 1)
    out["all_reduce_per_rank_threads_r8_64MiB_f32_sum_8_streams"] = per_rank_row(torch, rr, xs8, o, R)
    del o
    # a length whose ring segments start 4 bytes past a 256-byte boundary:
    # every job then begins with a short lead tile
    n_odd = N + R
    xo = si.torch_rank_inputs(R, n_odd, "f32", "normal", 1, device=dev)
    oo = [torch.empty_like(x) for x in xo]
    rr.register(R, device=0)
    us = time_calls(torch, lambda: rr.all_reduce(xo, "sum", out=oo), 10) * 1e3
    out["all_reduce_r8_64MiB_plus_8_f32_sum"] = {**_roof(2 * R * n_odd * 4, us), "elems_per_rank": n_odd,
                                                 "segment_offset_mod_256_bytes": (-(-n_odd // R) * 4) % 256}
    rr.finish()
    del xo, oo
    rr.register(R, device=0)
    # the Communicator's copies on the metric workload's buffers
    log("bench: rows: all_to_all_single, all_gather list form, send/recv")
    o = [torch.empty_like(x) for x in xs8]
    us = time_calls(torch, lambda: rr.all_to_all_single(xs8, out=o), 10) * 1e3
    out["all_to_all_single_r8_64MiB_f32"] = _roof(2 * R * b, us)
    M = N // R
    shards = [x[:M] for x in xs8]
    lst = [[o[r][k * M:(k + 1) * M] for k in range(R)] for r in range(R)]
    us = time_cold(torch, lambda: rr.all_gather_list(shards, out=lst), 10, scratch) * 1e3
    row = _roof((R + R * R) * M * 4, us)
    row.update({"shard_MiB": M * 4 >> 20, "cache": "flushed before each call"})
    out["all_gather_list_r8_8MiB_shards_f32"] = row
    us = time_cold(torch, lambda: rr.send_recv(xs8[0], 0, 1, out=o[1]), 10, scratch) * 1e3
    out["send_recv_64MiB_f32"] = dict(_roof(2 * b, us), cache="flushed before each call")
    del o, lst, shards
    # reduce_scatter and all_gather, 8 ranks x 256 MiB
    w = si.WORKLOADS["ranks8_256MiB_f32_rs_ag"]
    log("bench: rows: reduce_scatter / all_gather 8 x 256 MiB")
    big = si.torch_rank_inputs(w["R"], w["N"], "f32", w["dist"], w["seed"], device=dev)
    M = w["N"] // w["R"]
    shards = [torch.empty(M, dtype=torch.float32, device=dev) for _ in range(w["R"])]
    gathered = [torch.empty(w["N"], dtype=torch.float32, device=dev) for _ in range(w["R"])]
    us = time_calls(torch, lambda: rr.reduce_scatter(big, "sum", out=shards), 10) * 1e3
    out["reduce_scatter_r8_256MiB_f32_sum"] = _roof((w["R"] + 1) * w["N"] * 4, us)
    us = time_calls(torch, lambda: rr.all_gather(shards, out=gathered), 10) * 1e3
    out["all_gather_r8_32MiB_shards_f32"] = _roof((w["R"] + 1) * w["N"] * 4, us)
    rr.finish()
    del big, shards, gathered
    torch.cuda.empty_cache()
    # int32 workload, 4 ranks x 64 MiB
    w = si.WORKLOADS["ranks4_64MiB_i32"]
    log("bench: rows: int32 4 x 64 MiB")
    xi = si.torch_rank_inputs(w["R"], w["N"], "i32", "int", w["seed"], device=dev)
    R4, N4 = w["R"], w["N"]
    rr.register(R4, device=0)
    oi = [torch.empty_like(x) for x in xi]
    cold = {"cache": "flushed before each call"}
    us = time_cold(torch, lambda: rr.all_reduce(xi, "sum", out=oi), 10, scratch) * 1e3
    out["all_reduce_r4_64MiB_i32_sum"] = dict(_roof(2 * R4 * N4 * 4, us), **cold)
    us = time_cold(torch, lambda: rr.all_reduce(xi, "max", out=oi), 10, scratch) * 1e3
    out["all_reduce_r4_64MiB_i32_max"] = dict(_roof(2 * R4 * N4 * 4, us), **cold)
    ro = [oi[r] if r == 2 else None for r in range(R4)]
    us = time_cold(torch, lambda: rr.reduce(xi, 2, "sum", out=ro), 10, scratch) * 1e3
    out["reduce_r4_64MiB_i32_root2"] = dict(_roof((R4 + 1) * N4 * 4, us), **cold)
    sends = [xi[3] if r == 3 else None for r in range(R4)]
    bo = [oi[r] if r != 3 else None for r in range(R4)]
    us = time_cold(torch, lambda: rr.broadcast(sends, out=bo), 10, scratch) * 1e3
    out["broadcast_r4_64MiB_i32_from3"] = dict(_roof(R4 * N4 * 4, us), **cold)
    rr.finish()
    del xi, oi, ro, bo, sends
    torch.cuda.empty_cache()
    # batched gradient all-reduce: the transformer-shaped list
    layers = 32 if args.full_batched else 2
    shapes = si.transformer_grad_shapes(layers=layers)
    log(f"bench: rows: batched Mean over {len(shapes)} tensors ({layers} layers)")
    w = si.WORKLOADS["ranks4_llama32_grads_f32"]
    R4 = w["R"]
    ts = [[si.torch_tensor_for(w["seed"], t, R4, r, shp, device=dev) for r in range(R4)]
          for t, shp in enumerate(shapes)]
    os_ = [[torch.empty_like(x) for x in per] for per in ts]
    elems = sum(x.numel() for x in (per[0] for per in ts))
    rr.register(R4, device=0)
    us = time_calls(torch, lambda: rr.all_reduce_many(ts, "mean", out=os_), 3, warmup=6) * 1e3
    row = _roof(2 * R4 * elems * 4, us)
    row.update({"tensors": len(shapes), "elems_per_rank": elems, "layers": layers})
    out[f"all_reduce_many_r4_{layers}layer_grads_f32_mean"] = row
    # the same list as per-rank maps keyed by parameter ID, each rank listing
    # its IDs in its own order
    import random
    grads = []
    for r in range(R4):
        ids = list(range(len(shapes)))
        random.Random(r).shuffle(ids)
        grads.append({t: ts[t][r] for t in ids})
    outs = [{t: os_[t][r] for t in range(len(shapes))} for r in range(R4)]
    us = time_calls(torch, lambda: rr.all_reduce_params(grads, "mean", out=outs), 3, warmup=6) * 1e3
    row = _roof(2 * R4 * elems * 4, us)
    row.update({"tensors": len(shapes), "elems_per_rank": elems})
    out[f"all_reduce_params_r4_{layers}layer_grads_f32_mean"] = row
    # gradient accumulation: the last microbatch added to the accumulators
    # inside the sync (one pass) against a separate elementwise add and then
    # the sync (two passes); both give the same bits
    # (results go in place into the accumulators' storage, so the full
    # 32-layer list needs only gradients plus accumulators: 211 GB)
    log("bench: rows: accumulated gradient sync, fused and separate")
    del outs, os_
    torch.cuda.empty_cache()
    accs = [{t: torch.empty_like(ts[t][r]).normal_(0.0, 1e-3) for t in range(len(shapes))} for r in range(R4)]
    us = time_calls(torch, lambda: rr.all_reduce_params(grads, "mean", out=accs, acc=accs), 3, warmup=6) * 1e3
    row = _roof(3 * R4 * elems * 4, us)
    row.update({"tensors": len(shapes), "elems_per_rank": elems,
                "bytes": "read acc and grad, write the output: 3*R*N*4"})
    out[f"all_reduce_params_acc_fused_r4_{layers}layer_grads_f32_mean"] = row

    def separate():
        for r in range(R4):
            for t in range(len(shapes)):
                accs[r][t].add_(grads[r][t])
        rr.all_reduce_params(accs, "mean", out=accs)

    us = time_calls(torch, separate, 3, warmup=6) * 1e3
    row = _roof(5 * R4 * elems * 4, us)
    row.update({"tensors": len(shapes), "elems_per_rank": elems,
                "bytes": "torch add (2 reads, 1 write) then the sync (1 read, 1 write): 5*R*N*4"})
    out[f"accumulate_then_sync_r4_{layers}layer_grads_f32_mean"] = row
    rr.finish()
    del ts, grads, accs, scratch
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


def cpu_baseline(torch, xs, out_sum, seconds):
    """The CPU oracle (ring simulation, NumPy) on the host cores of this machine,
    on the metric workload's inputs; repeated until about `seconds` of work."""
    import numpy as np

    import oracle

    hx = [x.cpu().numpy() for x in xs]
    N = hx[0].size
    log("bench: timing the CPU oracle")
    calls = 0
    t0 = time.perf_counter()
    while True:
        res = oracle.all_reduce(hx, "sum")
        calls += 1
        el = time.perf_counter() - t0
        if el >= seconds:
            break
    gpu = out_sum[0].cpu().numpy()
    match = bool(np.array_equal(res[0].view(np.uint32), gpu.view(np.uint32)))
    return {
        "value": round(calls * N * 4 / el / 1e9, 4),
        "unit": "GB/s",
        "cores": 1,
        "kind": "oracle",
        "sample": f"{calls} full all_reduce Sum calls of the ring-simulation oracle on the same "
                  f"8 x 16,777,216 fp32 inputs (host copy), {el:.1f} s; NumPy elementwise, one thread",
        "seconds": round(el, 2),
        "matches_gpu_bits": match,
        "host_cpus_visible": len(os.sched_getaffinity(0)),
    }


if __name__ == "__main__":
    main()
