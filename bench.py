#!/usr/bin/env python3
"""Benchmark of the MLA / MLRA-4 latent-KV decode step on one MI355X.

A step is one whole decode call (absorbed-query prologue, split-K main loop, combine, W_UV
epilogue) over one batch of seeded synthetic input already resident in HBM.  Before every
step (warm-up and timed) a 512 MiB read (a sum over a scratch buffer) evicts L2 and the
256 MiB MALL with clean lines, so each step streams its latent cache from HBM; a write fill
would instead leave the MALL dirty and charge the step for the write-backs.  The per-step
time is taken with HIP events that the library records on its own stream around its
kernels (``mla_decode_timed``), so the flush is outside the measured interval.

Step time: a HIP event pair around [flush, decode] minus one around [flush] alone, both
averaged over the K timed steps.  The event overheads cancel and the decode's kernels run
back to back, as they would in a model.  A separate pass with ``mla_decode_timed``
gives per-stage times and the main-loop kernel time for the roofline; its interior events
add a few microseconds of idle gap per stage, which that pass does not report as step time.
The main-loop time is that pass's event interval around the main kernel minus the interval
of an empty event pair recorded the same way (the marker overhead both contain).

Prints ONE JSON line on stdout.  ``value`` is the latent-cache read rate in TB/s:
  sum_b L_b * (d_c + d_rope) * bytes_per_element / t_step.
"""

import argparse
import ctypes
import hashlib
import json
import os
import statistics
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "MLA decode attn: latent-KV read TB/s (% HBM peak), query tokens/s over B×L"
DEFAULT_WORKLOAD = "mla_bf16_b32_h128_l4096"
HBM_PEAK_GBPS = 8000.0  # MI355X published HBM3E bandwidth
PMC_SUMMARY = os.path.join(ROOT, "profiles", "main_loop_counters.json")
# sources of the main-loop kernels; the counter summary is valid only for these exact texts
MAIN_SRCS = [os.path.join(ROOT, "mlra_latent_kv_amd", "csrc", f) for f in
             ("main_bf16.hip", "main_bf16_wide.hip", "tile_bf16.h", "device_common.h")]


def log(*a):
    print(*a, file=sys.stderr, flush=True)


class HipEvents:
    """Raw hipEvent_t handles from libamdhip64 (the library records them on its stream)."""

    def __init__(self):
        # the runtime copy torch (and the library) already loaded, found by its soname
        self.hip = ctypes.CDLL("libamdhip64.so.7")
        self.hip.hipEventCreate.argtypes = [ctypes.POINTER(ctypes.c_void_p)]
        self.hip.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.c_void_p,
                                                 ctypes.c_void_p]
        self.hip.hipEventDestroy.argtypes = [ctypes.c_void_p]
        self.hip.hipEventRecord.argtypes = [ctypes.c_void_p, ctypes.c_void_p]

    def record(self, ev, stream):
        if self.hip.hipEventRecord(ev, stream) != 0:
            raise RuntimeError("hipEventRecord failed")

    def create(self, n):
        arr = (ctypes.c_void_p * n)()
        for i in range(n):
            h = ctypes.c_void_p()
            if self.hip.hipEventCreate(ctypes.byref(h)) != 0:
                raise RuntimeError("hipEventCreate failed")
            arr[i] = h
        return arr

    def ms(self, a, b):
        out = ctypes.c_float()
        if self.hip.hipEventElapsedTime(ctypes.byref(out), a, b) != 0:
            raise RuntimeError("hipEventElapsedTime failed")
        return out.value

    def destroy(self, arr):
        for h in arr:
            self.hip.hipEventDestroy(h)


def source_sha() -> str:
    h = hashlib.sha256()
    for f in MAIN_SRCS:
        h.update(open(f, "rb").read())
    return h.hexdigest()[:16]


def main_kernel(w) -> str:
    """Name of the kernel that runs the split-K main loop for workload w."""
    if w.dtype != "bf16":
        return "k_main_f32"
    return "k_main_bf16_wide" if (w.branches == 1 and w.heads % 128 == 0) else "k_main_bf16"


def counters_traffic(workload: str):
    """HBM bytes per main-kernel launch from the committed rocprofv3 counter summary, if it was
    taken on the current main-loop source; else None."""
    try:
        s = json.load(open(PMC_SUMMARY))
    except (OSError, ValueError):
        return None
    ent = s.get(workload)
    if not ent or ent.get("source_sha") != source_sha():
        return None
    return ent.get("hbm_bytes_per_launch")


def cpu_baseline(inp, seconds: float):
    """Time the fp64 oracle (as it stands) on a bounded sample of the same workload."""
    import numpy as np
    from threadpoolctl import threadpool_info
    from oracle import mla_oracle as O
    from mlra_latent_kv_amd import inputs as I
    w = inp["workload"]
    dt = inp["dtype"]
    lens = inp["seqlens"]
    kw = dict(d_rope=w.d_rope, scale=inp["softmax_scale"], out_scale=inp["out_scale"],
              theta=inp["rope_theta"], page_size=inp["page_size"],
              block_table=inp["block_table"], to_f64=lambda a: I.to_f64(a, dt))
    hchunk = 8
    done_bytes, pairs, t0 = 0.0, 0, time.perf_counter()
    b = 0
    while b < len(lens) and time.perf_counter() - t0 < seconds:
        for h0 in range(0, w.heads, hchunk):
            hs = list(range(h0, min(h0 + hchunk, w.heads)))
            O.mla_decode(inp["q_nope"], inp["q_rope"], inp["cache"], lens, inp["w_uk"],
                         inp["w_uv"], batches=[b], heads=hs, **kw)
            done_bytes += float(lens[b]) * w.row * w.elem_bytes * len(hs) / w.heads
            pairs += len(hs)
            if time.perf_counter() - t0 >= seconds:
                break
        b += 1
    el = time.perf_counter() - t0
    threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    return {"value": done_bytes / el / 1e12, "unit": "TB/s", "cores": threads, "kind": "oracle",
            "sample": f"{pairs} (sequence, head) outputs of {w.name} from sequence 0 on, "
                      f"fp64 un-absorbed oracle, {el:.1f} s wall; value = their share of the "
                      f"cache bytes / wall time",
            "seconds": round(el, 2), "cpu": _cpu_model()}


def _cpu_model():
    try:
        for ln in open("/proc/cpuinfo"):
            if ln.startswith("model name"):
                return ln.split(":", 1)[1].strip()
    except OSError:
        pass
    return None


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", default=DEFAULT_WORKLOAD)
    ap.add_argument("--num-splits", type=int, default=0)
    ap.add_argument("--cpu-seconds", type=float, default=12.0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--flush", choices=["read", "write", "none"], default="read",
                    help="cache eviction before each step (write/none are diagnostics)")
    ap.add_argument("--calibrate-copy-mib", type=int, default=0,
                    help="also run one plain copy kernel of this size (counter calibration)")
    args = ap.parse_args()
    if args.steps < 1 or args.warmup < 0:
        ap.error("--steps must be at least 1 and --warmup at least 0")

    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(f"bench.py measures one GPU only (got --gpus {args.gpus}, WORLD_SIZE {world}); the "
              f"decode path has no multi-GPU mode.", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch
    from mlra_latent_kv_amd import binding as B
    from mlra_latent_kv_amd import harness as Hn
    from mlra_latent_kv_amd import inputs as I

    if not os.path.exists(B.LIB_PATH):
        from mlra_latent_kv_amd import build
        build.build()
    B.load()
    w = I.WORKLOADS[args.workload]
    log(f"[bench] generating {w.name}")
    inp = I.make_inputs(w)
    case = Hn.to_device(inp, num_splits=args.num_splits)
    torch.cuda.synchronize()
    lens = np.asarray(inp["seqlens"], np.int64)
    cache_bytes = I.cache_bytes(w, lens)

    flush = torch.ones(128 << 20, dtype=torch.float32, device="cuda")  # 512 MiB
    ev = HipEvents()
    stream = torch.cuda.current_stream().cuda_stream
    K, W = args.steps, args.warmup

    def do_flush(i):
        if args.flush == "read":
            flush.sum()
        elif args.flush == "write":
            flush.fill_(float(i))

    for i in range(W):
        do_flush(i)
        case.run()
    torch.cuda.synchronize()
    log(f"[bench] warm-up done ({W} steps); timing {K} steps")

    # pass 1: the timed region -- K x [event, flush, decode, event], then K x [event, flush, event]
    pairs_fd = [ev.create(2) for _ in range(K)]
    pairs_f = [ev.create(2) for _ in range(K)]
    torch.cuda.synchronize()
    t_wall = time.perf_counter()
    for i in range(K):
        ev.record(pairs_fd[i][0], stream)
        do_flush(i)
        case.run()
        ev.record(pairs_fd[i][1], stream)
    torch.cuda.synchronize()
    t_wall = time.perf_counter() - t_wall
    plan = Hn.read_plan(case)  # the split plan the device made for these lengths
    for i in range(K):
        ev.record(pairs_f[i][0], stream)
        do_flush(i)
        ev.record(pairs_f[i][1], stream)
    torch.cuda.synchronize()
    t_fd = [ev.ms(e[0], e[1]) for e in pairs_fd]
    t_f = [ev.ms(e[0], e[1]) for e in pairs_f]
    total = [a - statistics.mean(t_f) for a in t_fd]

    # pass 2: per-stage times from the library's own stage events (diagnostic, main-loop time)
    staged = [ev.create(5) for _ in range(K)]
    for i in range(K):
        do_flush(i)
        case.run(events=staged[i])
    torch.cuda.synchronize()
    stage = {name: [ev.ms(e[j], e[j + 1]) for e in staged]
             for j, name in enumerate(["prologue", "main", "combine", "epilogue"])}
    # an event pair with nothing between it, recorded the same way (after the same flush):
    # its interval is the marker overhead that each stage interval above also contains
    empty = [ev.create(2) for _ in range(K)]
    for i in range(K):
        do_flush(i)
        ev.record(empty[i][0], stream)
        ev.record(empty[i][1], stream)
    torch.cuda.synchronize()
    pair_ms = statistics.mean(ev.ms(e[0], e[1]) for e in empty)
    for e in pairs_fd + pairs_f + staged + empty:
        ev.destroy(e)
    ms = statistics.mean(total)
    main_ms_raw = statistics.mean(stage["main"])
    main_ms = main_ms_raw - pair_ms

    if args.calibrate_copy_mib:
        n = args.calibrate_copy_mib << 20
        src = torch.ones(n // 4, dtype=torch.float32, device="cuda")
        dst = torch.empty_like(src)
        torch.mul(src, 1.0, out=dst)
        torch.cuda.synchronize()
        log(f"[bench] calibration copy kernel: {n} bytes read, {n} bytes written")

    value = cache_bytes / (ms * 1e-3) / 1e12
    achieved = cache_bytes / (main_ms * 1e-3) / 1e9
    line = {
        "metric": METRIC,
        "value": round(value, 4),
        "unit": "TB/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": W,
        "ms_per_step": round(ms, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16" if w.dtype == "bf16" else "f32",
        "data": "synthetic",
        "config": {"workload": w.name, "batch": int(len(lens)), "heads": w.heads,
                   "branches": w.branches, "seq_len": int(lens.max()),
                   "context_tokens": int(lens.sum()), "d_latent": w.d_c, "d_rope": w.d_rope,
                   "paged": bool(inp["paged"]), "work_items": plan["items"],
                   "pages_per_item": plan["pages"],
                   "cache_flush": args.flush},
        "pct_hbm_peak": round(100 * value * 1e3 / HBM_PEAK_GBPS, 2),
        "query_tokens_per_s": round(len(lens) / (ms * 1e-3), 1),
        "context_tokens_per_s": round(float(lens.sum()) / (ms * 1e-3), 1),
        "ms_p10_p50_p90": [round(float(np.percentile(total, q)), 5) for q in (10, 50, 90)],
        "stage_us": {k: round(1e3 * statistics.mean(v), 2) for k, v in stage.items()},
        "wall_s_timed_region": round(t_wall, 4),
        "flush_us": round(1e3 * statistics.mean(t_f), 2),
        "roofline": {
            "kernel": main_kernel(w),
            "bound": "hbm",
            "achieved": round(achieved, 1),
            "peak": HBM_PEAK_GBPS,
            "unit": "GB/s",
            "frac": round(achieved / HBM_PEAK_GBPS, 4),
            "algorithmic_bytes": int(cache_bytes),
            "traffic": counters_traffic(w.name),
            "main_us": round(main_ms * 1e3, 2),
            "main_us_event_pair": round(main_ms_raw * 1e3, 2),
            "event_pair_overhead_us": round(pair_ms * 1e3, 2),
        },
        "cpu_baseline": None,
    }
    if not args.no_cpu_baseline:
        log(f"[bench] timing the CPU oracle for ~{args.cpu_seconds:.0f} s")
        line["cpu_baseline"] = cpu_baseline(inp, args.cpu_seconds)
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
