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
gives per-stage times and the main-loop kernel time for the roofline: the HIP event pair
the library records on its stream around the main-loop launch (nothing subtracted, so the
figure includes the launch's own dispatch gap and is an upper bound on the kernel's run
time).  The rocprofv3 kernel-trace average of the same kernel, from the committed summary
taken on the current main-loop sources, is reported beside it with the fraction it gives
(``trace_avg_us``, ``frac_trace``; null when the summary is stale).

A read-stream probe (libmla_probe.so: 16-byte loads over 2 GiB, every byte once) gives the
practical HBM read ceiling of the device in the same run, reported next to the 8 TB/s peak.

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
# the largest single-GPU workload: 64 sequences of U[1024, 32768] tokens, 1.25 GB of cache
DEFAULT_WORKLOAD = "mla_bf16_paged_b64_h32_l1k-32k"
HBM_PEAK_GBPS = 8000.0  # MI355X published HBM3E bandwidth
PMC_SUMMARY = os.path.join(ROOT, "profiles", "main_loop_counters.json")
# sources of each main-loop kernel; a kernel's committed counters are valid only for these
# exact texts
KERNEL_SRCS = {
    "k_main_bf16": ("main_bf16.hip", "tile_bf16.h", "device_common.h"),
    "k_main_bf16_wide": ("main_bf16_wide.hip", "tile_bf16.h", "device_common.h"),
}


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


def read_probe(ev, stream, reps: int = 5, gib: int = 2):
    """Median HBM read rate (GB/s) of the read-stream probe over a ``gib`` GiB buffer."""
    import torch
    lib = ctypes.CDLL(os.path.join(ROOT, "mlra_latent_kv_amd", "libmla_probe.so"))
    lib.mla_probe_read.argtypes = [ctypes.c_void_p, ctypes.c_size_t, ctypes.c_void_p,
                                   ctypes.c_void_p]
    lib.mla_probe_out_words.restype = ctypes.c_size_t
    n = gib << 30
    buf = torch.ones(n // 4, dtype=torch.float32, device="cuda")
    out = torch.empty(lib.mla_probe_out_words(), dtype=torch.int32, device="cuda")
    e = ev.create(2)
    ms = []
    for i in range(reps + 1):
        ev.record(e[0], stream)
        if lib.mla_probe_read(buf.data_ptr(), n, out.data_ptr(), stream) != 0:
            raise RuntimeError("mla_probe_read failed")
        ev.record(e[1], stream)
        torch.cuda.synchronize()
        if i:  # the first run warms up
            ms.append(ev.ms(e[0], e[1]))
    ev.destroy(e)
    del buf
    torch.cuda.empty_cache()
    return n / (statistics.median(ms) * 1e-3) / 1e9


def read_pages_probe(ev, stream, inp, case, flush_fn, reps: int = 5):
    """Median rate (GB/s) of the page-gather probe over the workload's own paged pool: every
    page a sequence uses, sequence by sequence in block-table order (the order the decode's
    work items read them), caches flushed before each run.  Returns (GB/s, bytes read)."""
    import numpy as np
    import torch
    lib = ctypes.CDLL(os.path.join(ROOT, "mlra_latent_kv_amd", "libmla_probe.so"))
    lib.mla_probe_read_pages.argtypes = [ctypes.c_void_p, ctypes.c_size_t, ctypes.c_void_p,
                                         ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p]
    lib.mla_probe_out_words.restype = ctypes.c_size_t
    bt = np.asarray(inp["block_table"])
    lens = np.asarray(inp["seqlens"], np.int64)
    order = np.concatenate([bt[b, :(int(L) + 63) // 64] for b, L in enumerate(lens)])
    assert order.min() >= 0 and order.max() < case.cache.shape[0]  # inside the pool
    pages = torch.from_numpy(order.astype(np.int32)).to(case.cache.device)
    page_bytes = case.cache[0].numel() * case.cache.element_size()
    out = torch.empty(lib.mla_probe_out_words(), dtype=torch.int32, device=case.cache.device)
    e = ev.create(2)
    ms = []
    for i in range(reps + 1):
        flush_fn(i)
        ev.record(e[0], stream)
        if lib.mla_probe_read_pages(case.cache.data_ptr(), page_bytes, pages.data_ptr(),
                                    len(order), out.data_ptr(), stream) != 0:
            raise RuntimeError("mla_probe_read_pages failed")
        ev.record(e[1], stream)
        torch.cuda.synchronize()
        if i:
            ms.append(ev.ms(e[0], e[1]))
    ev.destroy(e)
    nbytes = len(order) * page_bytes
    return nbytes / (statistics.median(ms) * 1e-3) / 1e9, nbytes


def source_sha(kernel: str) -> str:
    """Hash of the sources the main-loop kernel is built from."""
    h = hashlib.sha256()
    for f in KERNEL_SRCS[kernel]:
        h.update(open(os.path.join(ROOT, "mlra_latent_kv_amd", "csrc", f), "rb").read())
    return h.hexdigest()[:16]


def main_kernel(w, num_queries: int = 1, fp8: bool = False) -> str:
    """Name of the kernel that runs the split-K main loop for workload w (its query rows are
    num_queries tokens x heads; an fp8 latent always runs on the 32-head kernel)."""
    if w.dtype != "bf16":
        return "k_main_f32"
    rows = num_queries * w.heads
    wide = w.branches == 1 and w.d_cb == 512 and rows % 128 == 0 and not fp8
    return "k_main_bf16_wide" if wide else "k_main_bf16"


def counters_key(workload: str, num_queries: int = 1, fp8: bool = False) -> str:
    """Key of a run in the committed counter summary: the workload name, then @qN for N query
    tokens per sequence and @fp8 for an fp8 latent cache."""
    return workload + (f"@q{num_queries}" if num_queries != 1 else "") + ("@fp8" if fp8 else "")


def counters_entry(workload: str, num_queries: int = 1, fp8: bool = False):
    """The committed rocprofv3 summary of the main kernel for this workload (HBM bytes per
    launch, kernel-trace average), if it was taken on that kernel's current sources; else
    None."""
    try:
        s = json.load(open(PMC_SUMMARY))
    except (OSError, ValueError):
        return None
    ent = s.get(counters_key(workload, num_queries, fp8))
    if not ent:
        return None
    kern = ent.get("kernel")
    if kern not in KERNEL_SRCS or ent.get("source_sha") != source_sha(kern):
        return None
    w = None
    try:
        from mlra_latent_kv_amd import inputs as I
        w = I.WORKLOADS[workload]
    except (ImportError, KeyError):
        return None
    if kern != main_kernel(w, num_queries, fp8):
        return None
    return ent


def counters_traffic(workload: str, num_queries: int = 1, fp8: bool = False):
    """HBM bytes per main-kernel launch from the committed counter summary, else None."""
    ent = counters_entry(workload, num_queries, fp8)
    return None if ent is None else ent.get("hbm_bytes_per_launch")


def cpu_baseline(inp, seconds: float):
    """Time the fp64 oracle (as it stands) on a bounded sample of the same workload."""
    import numpy as np
    from threadpoolctl import threadpool_limits
    from oracle import mla_oracle as O
    from mlra_latent_kv_amd import inputs as I
    w = inp["workload"]
    dt = inp["dtype"]
    lens = inp["seqlens"]
    kw = dict(d_rope=w.d_rope, scale=inp["softmax_scale"], out_scale=inp["out_scale"],
              theta=inp["rope_theta"], page_size=inp["page_size"],
              block_table=inp["block_table"], to_f64=lambda a: I.to_f64(a, dt))
    hchunk = 8
    cores = len(os.sched_getaffinity(0))
    done_bytes, pairs = 0.0, 0
    with threadpool_limits(limits=cores):  # BLAS threads = the cores this process may use
        t0 = time.perf_counter()
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
    return {"value": done_bytes / el / 1e12, "unit": "TB/s", "cores": cores, "kind": "oracle",
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


APPEND_METRIC = "MLA cache append: us per decode step (new token per sequence, paged)"


def bench_append(args, ev, stream):
    """One decode step's cache write for the paged variable-length batch (64 sequences, the
    lengths of mla_bf16_paged_b64_h32_l1k-32k), d_model 4096 (32 heads x 128).  Before every
    step the lengths and block table are restored and the caches flushed (outside the event
    pair), so every step writes the same rows from cold caches."""
    import numpy as np
    import torch
    from mlra_latent_kv_amd import binding as B
    from mlra_latent_kv_amd import inputs as I
    w = I.WORKLOADS["mla_bf16_paged_b64_h32_l1k-32k"]
    d_model, dc = 4096, w.d_c
    kids = np.random.SeedSequence(w.seed).spawn(8)
    lens = I.draw_seqlens(w, w.batch, np.random.default_rng(kids[6]))
    Bn = len(lens)
    inp = I.make_append_inputs(d_model, dc, Bn, seed=2001)
    pages = [-(-int(L) // 64) for L in lens]
    max_pages = -(-w.seqlen // 64) + 1
    pool = sum(pages) + Bn + 8
    perm = np.random.default_rng(7).permutation(pool).astype(np.int32)
    bt = np.full((Bn, max_pages), -1, np.int32)
    k = 0
    for b, n in enumerate(pages):
        bt[b, :n] = perm[k:k + n]
        k += n
    dev = lambda a: torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).cuda()
    cache = torch.zeros((pool, 64, dc + 64), dtype=torch.bfloat16, device="cuda")
    sl0 = torch.tensor(lens.astype(np.int32), device="cuda")
    bt0 = torch.tensor(bt, device="cuda")
    sl, btd = sl0.clone(), bt0.clone()
    free = torch.tensor(perm[k:], device="cuda")
    used = torch.zeros(1, dtype=torch.int32, device="cuda")
    p = B.MlaAppendParams()
    p.batch, p.d_model, p.d_latent, p.d_rope = Bn, d_model, dc, 64
    p.page_size, p.max_pages_per_seq, p.capacity, p.dtype = 64, max_pages, 0, B.MLA_BF16
    p.latent_stride_tok = p.rope_stride_tok = dc + 64
    p.latent_stride_seq = p.rope_stride_seq = 64 * (dc + 64)
    p.block_table_stride, p.rope_theta = max_pages, 10000.0
    ws = torch.empty(B.append_workspace_size(p), dtype=torch.uint8, device="cuda")
    h, wd, wk = dev(inp["hidden"]), dev(inp["w_dkv"]), dev(inp["w_kr"])
    flush = torch.ones(128 << 20, dtype=torch.float32, device="cuda")

    def step(events=None):
        sl.copy_(sl0)
        btd.copy_(bt0)
        flush.sum()
        if events is not None:
            ev.record(events[0], stream)
        B.mla_cache_append(p, h, wd, wk, cache.data_ptr(), cache.data_ptr() + dc * 2, sl, btd,
                           free, free.numel(), used, ws, stream=stream)
        if events is not None:
            ev.record(events[1], stream)

    for _ in range(args.warmup):
        step()
    pairs = [ev.create(2) for _ in range(args.steps)]
    torch.cuda.synchronize()
    for i in range(args.steps):
        step(pairs[i])
    torch.cuda.synchronize()
    t = [ev.ms(e[0], e[1]) for e in pairs]
    for e in pairs:
        ev.destroy(e)
    us = 1e3 * statistics.mean(t)
    need = int(sum(1 for L in lens if L % 64 == 0))
    assert int(used.item()) == need and bool((sl == sl0 + 1).all())
    nbytes = d_model * (dc + 64) * 2 + Bn * d_model * 2 + Bn * (dc + 64) * 2
    gbps = nbytes / (us * 1e-6) / 1e9
    return {
        "metric": APPEND_METRIC, "value": round(us, 3), "unit": "us", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(us / 1e3, 5),
        "higher_is_better": False, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": "append_paged_b64_dmodel4096", "batch": Bn, "d_model": d_model,
                   "d_latent": dc, "d_rope": 64, "pages_taken": need},
        "us_p10_p50_p90": [round(1e3 * float(np.percentile(t, q)), 3) for q in (10, 50, 90)],
        "roofline": {"kernel": "k_append_proj + k_append_write", "bound": "hbm",
                     "achieved": round(gbps, 1), "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                     "frac": round(gbps / HBM_PEAK_GBPS, 4), "algorithmic_bytes": nbytes,
                     "traffic": None},
        "cpu_baseline": None,
    }


PREFILL_METRIC = "MLA prefill (un-absorbed): TFLOP/s (% of the 2.5 PF bf16 MFMA peak)"
MFMA_PEAK_TFLOPS = 2500.0  # MI355X dense bf16 matrix peak


def prefill_flops(w, lens, sq):
    """Algorithmic work of one prefill call: the up-projection of every cached latent to its
    per-head key and value (2 * 512 * 256 per token and head, whether as one 512-wide branch
    or four 128-wide ones) and the causal attention, 2 * (192 + 128) per visible (query, key)
    pair, head and branch."""
    import numpy as np
    proj = 2.0 * float(np.sum(lens)) * w.d_c * (w.d_nope + w.d_v) * w.heads
    pairs = 0.0
    for L in lens:
        vis = np.clip(int(L) - sq + 1 + np.arange(sq), 0, int(L))
        pairs += float(vis.sum())
    attn = 2.0 * pairs * (w.d_nope + w.d_rope + w.d_v) * w.heads * w.branches
    return proj, attn


def cpu_baseline_prefill(inp, seconds: float):
    """The fp64 oracle's prefill (as it stands) on a bounded sample: whole heads of sequence 0,
    one at a time, until the time budget is spent; value = their share of the algorithmic
    work / wall time."""
    import numpy as np
    from threadpoolctl import threadpool_limits
    from oracle import mla_oracle as O
    from mlra_latent_kv_amd import inputs as I
    w, sq = inp["workload"], inp["num_queries"]
    lens = np.asarray(inp["seqlens"])
    proj, attn = prefill_flops(w, lens[:1], sq)
    per_head = (proj + attn) / w.heads
    cores = len(os.sched_getaffinity(0))
    done, heads = 0.0, 0
    with threadpool_limits(limits=cores):
        t0 = time.perf_counter()
        for h in range(w.heads):
            rows = [i * w.heads + h for i in range(sq)]
            O.mla_prefill(inp["q_nope"], inp["q_rope"], inp["cache"], inp["seqlens"], inp["w_uk"],
                          inp["w_uv"], num_queries=sq, d_rope=w.d_rope, scale=inp["softmax_scale"],
                          out_scale=inp["out_scale"], theta=inp["rope_theta"],
                          page_size=inp["page_size"], block_table=inp["block_table"],
                          to_f64=lambda a: I.to_f64(a, w.dtype), batches=[0], heads=rows)
            done += per_head
            heads += 1
            if time.perf_counter() - t0 >= seconds:
                break
        el = time.perf_counter() - t0
    return {"value": done / el / 1e12, "unit": "TFLOP/s", "cores": cores, "kind": "oracle",
            "sample": f"{heads} whole heads of sequence 0 of {w.name} ({sq} query tokens each), "
                      f"fp64 un-absorbed oracle, {el:.1f} s wall; value = their share of the "
                      f"algorithmic work / wall time",
            "seconds": round(el, 2), "cpu": _cpu_model()}


def bench_probe(args, ev, stream):
    """The issue probe (include/mla_probe.h): MFMA 32x32x16 bf16 chains and v_exp_f32 chains
    alone and side by side on each SIMD, both accumulator forms; median of 5 runs each."""
    import torch
    lib = ctypes.CDLL(os.path.join(ROOT, "mlra_latent_kv_amd", "libmla_probe.so"))
    lib.mla_probe_issue.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_void_p,
                                    ctypes.c_void_p]
    lib.mla_probe_issue_out_words.restype = ctypes.c_size_t
    out = torch.empty(lib.mla_probe_issue_out_words(), dtype=torch.float32, device="cuda")
    iters = 4096
    names = ["8 waves matrix", "waves 0-3 matrix + 4-7 vector", "waves 0-3 matrix",
             "waves 4-7 vector", "8 waves matrix+vector interleaved", "8 waves vector",
             "waves 0-3 matrix+vector interleaved (one wave per SIMD)"]
    e = ev.create(2)
    res = {}
    for agpr in (0, 1):
        for mode in range(7):
            ms = []
            for i in range(6):
                ev.record(e[0], stream)
                if lib.mla_probe_issue(mode, agpr, iters, out.data_ptr(), stream) != 0:
                    raise RuntimeError("mla_probe_issue failed")
                ev.record(e[1], stream)
                torch.cuda.synchronize()
                if i:
                    ms.append(ev.ms(e[0], e[1]))
            res[(agpr, mode)] = 1e3 * statistics.median(ms)
    ev.destroy(e)
    # a 32x32x16 bf16 MFMA holds the matrix core 32 cycles (8 passes of 4): the matrix-only
    # run with one wave per SIMD then gives the clock the SIMDs ran at
    mfma_cycles = iters * 4 * 32
    ghz = mfma_cycles / (res[(1, 2)] * 1e-6) / 1e9
    exp_cyc = res[(1, 3)] * 1e-6 * ghz * 1e9 / (iters * 16)
    taken = (res[(1, 1)] - res[(1, 3)]) * 1e-6 * ghz * 1e9 / (iters * 4)
    return {
        "metric": "issue_probe", "unit": "us", "iters": iters,
        "us": {f"{'agpr' if a else 'vgpr'} acc, mode {m}: {names[m]}": round(t, 1)
               for (a, m), t in sorted(res.items())},
        "clock_ghz_from_matrix_only": round(ghz, 3),
        "vector_cycles_per_mul_exp_pair": round(exp_cyc, 2),
        "vector_issue_cycles_lost_per_mfma_beside_it": round(taken, 1),
        "vgpr_over_agpr_accumulators_matrix_only": round(res[(0, 2)] / res[(1, 2)], 3),
        # one wave per SIMD issuing both streams: the share of the shorter stream's time that
        # is hidden behind the longer one (1: full overlap, 0: the two run one after the other)
        "one_wave_overlap_of_shorter_stream": round(
            (res[(1, 2)] + res[(1, 3)] - res[(1, 6)]) / min(res[(1, 2)], res[(1, 3)]), 3),
    }


def calibration_copy(args):
    """A plain copy kernel of known size (torch.mul into a fresh tensor) for scaling the HBM
    byte counters of a profiled run."""
    import torch
    if args.calibrate_copy_mib:
        n = args.calibrate_copy_mib << 20
        src = torch.ones(n // 4, dtype=torch.float32, device="cuda")
        dst = torch.empty_like(src)
        torch.mul(src, 1.0, out=dst)
        torch.cuda.synchronize()
        log(f"[bench] calibration copy kernel: {n} bytes read, {n} bytes written")


def bench_prefill(args, ev, stream):
    """One prefill call per step on a prefill workload (every token of the sequence new),
    caches flushed before every step, outside the event pair (as for the decode)."""
    import numpy as np
    import torch
    from mlra_latent_kv_amd import harness as Hn
    from mlra_latent_kv_amd import inputs as I
    name = args.workload if args.workload in I.PREFILL_WORKLOADS else "prefill_bf16_b1_h128_l4096"
    w = I.PREFILL_WORKLOADS[name]
    sq = args.num_queries if args.num_queries > 1 else w.seqlen
    log(f"[bench] generating {w.name} (s_q = {sq})")
    inp = I.make_inputs(w, num_queries=sq)
    case = Hn.to_device(inp, prefill=True)
    torch.cuda.synchronize()
    lens = np.asarray(inp["seqlens"], np.int64)
    proj, attn = prefill_flops(w, lens, sq)
    flush = torch.ones(128 << 20, dtype=torch.float32, device="cuda")
    K, W = args.steps, args.warmup
    for _ in range(W):
        flush.sum()
        Hn.run_prefill(case)
    torch.cuda.synchronize()
    log(f"[bench] warm-up done ({W} steps); timing {K} steps")
    pf = [ev.create(2) for _ in range(K)]
    pp = [ev.create(2) for _ in range(K)]
    st = [ev.create(3) for _ in range(K)]
    torch.cuda.synchronize()
    t_wall = time.perf_counter()
    for i in range(K):
        ev.record(pf[i][0], stream)
        flush.sum()
        Hn.run_prefill(case)
        ev.record(pf[i][1], stream)
    torch.cuda.synchronize()
    t_wall = time.perf_counter() - t_wall
    for i in range(K):
        ev.record(pp[i][0], stream)
        flush.sum()
        ev.record(pp[i][1], stream)
    for i in range(K):
        flush.sum()
        Hn.run_prefill(case, events=st[i])
    torch.cuda.synchronize()
    t_f = statistics.mean(ev.ms(a, b) for a, b in pp)
    total = [ev.ms(a, b) - t_f for a, b in pf]
    kv_ms = statistics.mean(ev.ms(e[0], e[1]) for e in st)
    at_ms = statistics.mean(ev.ms(e[1], e[2]) for e in st)
    for e in pf + pp + st:
        ev.destroy(e)
    calibration_copy(args)
    ms = statistics.mean(total)
    value = (proj + attn) / (ms * 1e-3) / 1e12
    at_tf = attn / (at_ms * 1e-3) / 1e12
    line = {
        "metric": PREFILL_METRIC, "value": round(value, 2), "unit": "TFLOP/s", "n_gpus": 1,
        "steps": K, "warmup": W, "ms_per_step": round(ms, 4), "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
        "config": {"workload": w.name, "batch": int(len(lens)), "heads": w.heads,
                   "seq_len": int(lens.max()), "query_tokens_per_seq": sq,
                   "d_latent": w.d_c, "d_rope": w.d_rope, "paged": bool(inp["paged"])},
        "pct_mfma_peak": round(100 * value / MFMA_PEAK_TFLOPS, 2),
        "query_tokens_per_s": round(sq * len(lens) / (ms * 1e-3), 1),
        "algorithmic_tflop": {"projection": round(proj / 1e12, 4), "attention": round(attn / 1e12, 4)},
        "stage_us": {"projection": round(1e3 * kv_ms, 2), "attention": round(1e3 * at_ms, 2)},
        "ms_p10_p50_p90": [round(float(np.percentile(total, q)), 4) for q in (10, 50, 90)],
        "wall_s_timed_region": round(t_wall, 4),
        "roofline": {"kernel": "k_prefill_attn", "bound": "mfma", "achieved": round(at_tf, 1),
                     "peak": MFMA_PEAK_TFLOPS, "unit": "TFLOP/s",
                     "frac": round(at_tf / MFMA_PEAK_TFLOPS, 4), "algorithmic_flops": attn,
                     "traffic": None, "main_us": round(1e3 * at_ms, 2)},
        "cpu_baseline": None,
    }
    if not args.no_cpu_baseline:
        log(f"[bench] timing the CPU oracle for ~{args.cpu_seconds:.0f} s")
        line["cpu_baseline"] = cpu_baseline_prefill(inp, args.cpu_seconds)
    return line


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", default=DEFAULT_WORKLOAD)
    ap.add_argument("--op", choices=["decode", "append", "prefill", "probe"], default="decode",
                    help="decode: the decode step (the metric); append: one step's cache write; "
                         "prefill: the un-absorbed many-query step on a prefill workload; "
                         "probe: the matrix-core / vector-ALU issue probe")
    ap.add_argument("--variant", default="none",
                    choices=["none", "gate", "query_latent", "output_latent",
                             "query_latent+output_latent"],
                    help="time a decode variant (gated output, folded query, latent output); "
                         "stage times and the main-loop roofline come from the plain call, "
                         "whose main loop is the same kernel")
    ap.add_argument("--num-queries", type=int, default=1,
                    help="query tokens per sequence decoded in one step (causal among them)")
    ap.add_argument("--latent", choices=["bf16", "fp8"], default="bf16",
                    help="latent cache format: bf16, or OCP FP8 E4M3 codes with a per-tensor "
                         "scale (the rotary key stays bf16; compute stays bf16/fp32)")
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
    if args.op == "append":
        print(json.dumps(bench_append(args, HipEvents(), torch.cuda.current_stream().cuda_stream)),
              flush=True)
        return
    if args.op == "probe":
        print(json.dumps(bench_probe(args, HipEvents(), torch.cuda.current_stream().cuda_stream)),
              flush=True)
        return
    if args.op == "prefill":
        print(json.dumps(bench_prefill(args, HipEvents(), torch.cuda.current_stream().cuda_stream)),
              flush=True)
        return
    w = I.WORKLOADS[args.workload]
    log(f"[bench] generating {w.name}")
    lf = "fp8" if args.latent == "fp8" else ""
    inp = I.make_inputs(w, num_queries=args.num_queries, latent_format=lf)
    case = Hn.to_device(inp, num_splits=args.num_splits)
    torch.cuda.synchronize()
    lens = np.asarray(inp["seqlens"], np.int64)
    cache_bytes = I.cache_bytes(w, lens, lf)

    step = case.run
    if args.variant != "none":
        var = I.make_variant_inputs(inp)
        v_gate = Hn._to_dev(var["gate"], w.dtype, "cuda") if "gate" in args.variant else None
        v_ql = (Hn._to_dev(var["q_latent"], w.dtype, "cuda") if "query_latent" in args.variant
                else None)
        v_lo = "output_latent" in args.variant

        def step():
            return Hn.run_variant(case, gate=v_gate, q_latent=v_ql, latent_out=v_lo)

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
        step()
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
        step()
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
    main_ms = statistics.mean(stage["main"])
    probe_gbps = read_probe(ev, stream)
    log(f"[bench] read-stream probe: {probe_gbps:.1f} GB/s")
    pages_gbps = pages_bytes = None
    if inp["paged"] and not lf:
        pages_gbps, pages_bytes = read_pages_probe(ev, stream, inp, case, do_flush)
        log(f"[bench] page-gather probe over the workload's pool: {pages_gbps:.1f} GB/s")

    calibration_copy(args)

    value = cache_bytes / (ms * 1e-3) / 1e12
    ent = None if args.variant != "none" else counters_entry(w.name, args.num_queries, bool(lf))
    trace_us = None if ent is None else ent.get("trace_avg_us")
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
                   "cache_flush": args.flush, "variant": args.variant,
                   "query_tokens_per_seq": args.num_queries,
                   "latent_cache": "fp8_e4m3" if lf else w.dtype},
        "pct_hbm_peak": round(100 * value * 1e3 / HBM_PEAK_GBPS, 2),
        "read_probe_GBps": round(probe_gbps, 1),
        "pct_read_probe": round(100 * value * 1e3 / probe_gbps, 2),
        "query_tokens_per_s": round(args.num_queries * len(lens) / (ms * 1e-3), 1),
        "context_tokens_per_s": round(float(lens.sum()) / (ms * 1e-3), 1),
        "ms_p10_p50_p90": [round(float(np.percentile(total, q)), 5) for q in (10, 50, 90)],
        "stage_us": {k: round(1e3 * statistics.mean(v), 2) for k, v in stage.items()},
        "wall_s_timed_region": round(t_wall, 4),
        "flush_us": round(1e3 * statistics.mean(t_f), 2),
        "roofline": {
            "kernel": main_kernel(w, args.num_queries, bool(lf)),
            "bound": "hbm",
            "achieved": round(achieved, 1),
            "peak": HBM_PEAK_GBPS,
            "unit": "GB/s",
            "frac": round(achieved / HBM_PEAK_GBPS, 4),
            "algorithmic_bytes": int(cache_bytes),
            "traffic": (None if args.variant != "none"
                        else counters_traffic(w.name, args.num_queries, bool(lf))),
            "main_us": round(main_ms * 1e3, 2),
            # the same kernel's rocprofv3 trace average from the committed summary (taken on
            # these main-loop sources), and the fraction it gives; null when stale
            "trace_avg_us": trace_us,
            "frac_trace": None if trace_us is None else round(
                cache_bytes / (trace_us * 1e-6) / 1e9 / HBM_PEAK_GBPS, 4),
            "frac_of_read_probe": round(achieved / probe_gbps, 4),
            # paged workloads: the same pages streamed in the same order by a plain kernel
            "page_probe_GBps": None if pages_gbps is None else round(pages_gbps, 1),
            "page_probe_bytes": pages_bytes,
            "frac_of_page_probe": None if pages_gbps is None else round(achieved / pages_gbps, 4),
            "empty_event_pair_us": round(pair_ms * 1e3, 2),
        },
        "cpu_baseline": None,
    }
    if not args.no_cpu_baseline and args.variant == "none" and args.num_queries == 1 and not lf:
        log(f"[bench] timing the CPU oracle for ~{args.cpu_seconds:.0f} s")
        line["cpu_baseline"] = cpu_baseline(inp, args.cpu_seconds)
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
