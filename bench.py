"""Benchmark: NVFP4 ScaleSearch quantize GB/s (in+out) on MI355X.

Workload (one step): the whole nvfp4_quantize call on the bf16 weight
8192 x 28672 ~ N(0, 0.02^2) (seeded, synthetic) with ScaleSearch offsets
[-2, 6] -- global amax pass, tensor scale, candidate search, packed codes and
scales. value = algorithmic bytes of the call (input read once, codes, scales
and the tensor scale written once) / time of the step, inputs resident in HBM.

Also printed (same JSON line): the dominant kernel's roofline (the search
kernel alone, timed with HIP events on its stream over its own launches), a
per-pass breakdown (amax pass, search pass given the tensor scale, max-scaling
control, dequantize, quantize then dequantize), and the CPU oracle timed on a
bounded sample, on all the host threads this process may use and on one.

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-cpu] [--profile]
       python bench.py --rocpd-summary DB [DB ...] [--sources quantize|attention]
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "NVFP4 ScaleSearch quantize GB/s (in+out) and % of MI355X HBM peak"
HBM_PEAK_GBS = 8000.0
# VALU issue ceiling in lane-instructions: 256 CUs x 4 SIMDs x 16 lanes x 2.4 GHz
# (one wave-instruction of 64 lanes per SIMD every four cycles).
VALU_PEAK_TLANE = 256 * 64 * 2.4e9 / 1e12
# FP32 operations of the exact search per element and candidate, as the scoring
# rule defines them: y = x * r, xhat = V * d, e = |x| - xhat, e * e, running sum.
# The certified kernel reaches the same argmin with fewer instructions, so this is
# a work count for comparison, not a roofline.
OPS_PER_ELEMENT_CANDIDATE = 5
SEARCH_KERNEL = "quantize_certified_kernel<-2, 6, true>"
CSRC = os.path.join(ROOT, "microscaling_fp4_block_amd", "csrc")
# the sources each committed profile's kernels are built from: a profile whose recorded
# hash differs from the current one was taken on other code
SOURCE_GROUPS = {
    "quantize": ("nvfp4_kernels.hip", "nvfp4_api.hip", "nvfp4_internal.h", "nvfp4_device.h"),
    "attention": ("nvfp4_attention.hip", "nvfp4_api.hip", "nvfp4_internal.h", "nvfp4_device.h"),
}
PROFILES = {
    "quantize_search_bf16_8192x28672.md": "quantize",
    "quantize_hadamard_bf16_q32x32768x128.md": "quantize",
    "attention_nvfp4_q32x32768_kv8.md": "attention",
    "attention_decode_split160_q32_kv8_32k.md": "attention",
}
PROFILE_SUMMARY = os.path.join(ROOT, "profiles", "quantize_search_bf16_8192x28672.md")


def kernel_source_hash(group: str = "quantize") -> str:
    import hashlib

    h = hashlib.sha256()
    for f in SOURCE_GROUPS[group]:
        h.update(open(os.path.join(CSRC, f), "rb").read())
    return h.hexdigest()[:16]


def recorded_hash(path: str):
    for line in open(path):
        if line.startswith("source_hash:"):
            return line.split(":", 1)[1].split()[0].strip()
    return None


def profile_status() -> dict:
    """Each committed profile summary: "current" when its recorded source hash is that of
    the sources its kernels come from, else "stale" (or "missing")."""
    out = {}
    for name, group in PROFILES.items():
        path = os.path.join(ROOT, "profiles", name)
        if not os.path.exists(path):
            out[name] = "missing"
        else:
            out[name] = "current" if recorded_hash(path) == kernel_source_hash(group) else "stale"
    return out


def committed_traffic(kernel: str):
    """HBM bytes per launch of `kernel` from the committed counter summary, if that
    summary was taken on the current kernel sources (else None)."""
    if not os.path.exists(PROFILE_SUMMARY):
        return None
    src_hash, traffic = None, None
    for line in open(PROFILE_SUMMARY):
        if line.startswith("source_hash:"):
            src_hash = line.split(":", 1)[1].split()[0].strip()
        if line.startswith("traffic_bytes_per_launch") and kernel in line:
            traffic = int(line.rsplit("|", 1)[1].strip())
    return traffic if src_hash == kernel_source_hash() else None


def committed_figure(key: str, kernel: str):
    """A `key | kernel | value` line of the committed counter summary, if that summary
    was taken on the current kernel sources (else None)."""
    if not os.path.exists(PROFILE_SUMMARY):
        return None
    src_hash, val = None, None
    for line in open(PROFILE_SUMMARY):
        if line.startswith("source_hash:"):
            src_hash = line.split(":", 1)[1].split()[0].strip()
        if line.startswith(key + " ") and kernel in line:
            val = float(line.rsplit("|", 1)[1].strip())
    return val if src_hash == kernel_source_hash() else None


def committed_valu_issue(kernel: str):
    """Fraction of the kernel's cycles in which its CUs issued VALU, from the committed
    counter summary (SQ_INSTS_VALU per CU over GRBM_GUI_ACTIVE per XCD)."""
    return committed_figure("valu_issue_frac", kernel)
ROWS, COLS = 8192, 28672
OFFSETS = (-2, 6)


def quantize_bytes(n_elem: int, in_bytes_per_elem: int) -> int:
    """Input once + codes (1/2 B) + scales (1/16 B) + the 4-byte tensor scale."""
    return n_elem * in_bytes_per_elem + n_elem // 2 + n_elem // 16 + 4


def dequantize_bytes(n_elem: int, out_bytes_per_elem: int) -> int:
    return n_elem // 2 + n_elem // 16 + 4 + n_elem * out_bytes_per_elem


def search_pass_bytes(n_elem: int, in_bytes_per_elem: int) -> int:
    """The search kernel alone (tensor scale given): input + codes + scales + S_g read."""
    return quantize_bytes(n_elem, in_bytes_per_elem)


def event_time_ms(torch, fn, iters: int, stream) -> float:
    start = torch.cuda.Event(enable_timing=True)
    end = torch.cuda.Event(enable_timing=True)
    start.record(stream)
    for _ in range(iters):
        fn()
    end.record(stream)
    end.synchronize()
    return start.elapsed_time(end) / iters


def launch_times_ms(torch, fn, iters: int, stream, between=None) -> np.ndarray:
    """GPU time of each of `iters` calls of fn, from an event pair around each call;
    `between` (if given) runs after each pair, outside the timed interval."""
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
          for _ in range(iters)]
    for a, b in ev:
        a.record(stream)
        fn()
        b.record(stream)
        if between is not None:
            between()
    torch.cuda.synchronize()
    return np.array([a.elapsed_time(b) for a, b in ev])


def percentiles(t: np.ndarray):
    p10, p50, p90 = np.percentile(t, [10, 50, 90])
    return float(p10), float(p50), float(p90)


def graph_time_ms(torch, fn, reps: int, stream, replays: int = 5) -> float:
    """Per-call GPU time with the host out of the loop: `reps` calls of fn captured in
    one HIP graph, replayed `replays` times."""
    side = torch.cuda.Stream()
    side.wait_stream(stream)
    with torch.cuda.stream(side):
        fn()
    stream.wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        for _ in range(reps):
            fn()
    graph.replay()
    torch.cuda.synchronize()
    t = event_time_ms(torch, graph.replay, replays, stream) / reps
    del graph
    return t


class CacheFlush:
    """Evicts the 256 MB Infinity Cache between timed launches: a 512 MiB device copy
    (1 GiB of traffic through the cache)."""

    def __init__(self, torch, dev):
        self.src = torch.empty(512 << 20, dtype=torch.uint8, device=dev)
        self.dst = torch.empty_like(self.src)

    def __call__(self):
        self.dst.copy_(self.src)


def copy_gbs(torch, dev, stream, nbytes: int = 1 << 30, iters: int = 10) -> float:
    """A plain device-to-device copy (torch's copy_, which the HIP runtime serves with its
    own blit kernel) in read + write GB/s: a streaming rate measured on the box, beside
    the published peak."""
    src = torch.empty(nbytes, dtype=torch.uint8, device=dev)
    dst = torch.empty_like(src)
    dst.copy_(src)
    torch.cuda.synchronize()
    ms = event_time_ms(torch, lambda: dst.copy_(src), iters, stream)
    del src, dst
    return 2 * nbytes / (ms * 1e-3) / 1e9


def host_cpus() -> dict:
    """The host this process runs on: CPU model, CPUs it may run on, CPUs the OS reports,
    and the threads the oracle uses (the CPUs it may run on, capped by OMP_NUM_THREADS
    where that is set: the share of the host given to one GPU's jobs)."""
    model = None
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                model = line.split(":", 1)[1].strip()
                break
    except OSError:
        pass
    allowed = len(os.sched_getaffinity(0))
    cap = os.environ.get("OMP_NUM_THREADS")
    threads = min(allowed, int(cap)) if cap and cap.isdigit() and int(cap) > 0 else allowed
    return {"model": model, "nproc": allowed, "cpu_count": os.cpu_count(), "threads": threads,
            "omp_num_threads": cap}


def cpu_baseline(x_host: np.ndarray, budget_s: float = 8.0) -> dict:
    """The oracle, as it stands, on a row sample of the same tensor: the whole quantize
    (amax, tensor scale, tables, search, pack), on every host thread this process may use
    and on one thread."""
    import oracle

    oracle.build(force=False)
    cpu = host_cpus()

    def run(rows, threads):
        xs = x_host[:rows]
        t0 = time.perf_counter()
        oracle.quantize(xs, *OFFSETS, nthreads=threads)
        return time.perf_counter() - t0

    def sample(threads):
        rows = 64
        t = run(rows, threads)
        rows = int(min(ROWS, max(64, rows * budget_s / max(t, 1e-3))))
        rows -= rows % 64
        t = run(rows, threads)
        n = rows * COLS
        return quantize_bytes(n, 2) / t / 1e9, rows, n, t

    gbs, rows, n, t = sample(cpu["threads"])
    gbs1, rows1, n1, t1 = sample(1)
    return {"value": round(gbs, 4), "unit": "GB/s", "cores": cpu["threads"], "kind": "oracle",
            "sample": f"rows 0..{rows - 1} of the 8192x28672 bf16 tensor ({n} elements): the whole "
                      f"quantize [-2,6], {t:.2f} s wall on {cpu['threads']} threads",
            "single_thread": {"value": round(gbs1, 4), "unit": "GB/s",
                              "sample": f"rows 0..{rows1 - 1} ({n1} elements), {t1:.2f} s wall "
                                        "on 1 thread"},
            "host": {"cpu_model": cpu["model"], "nproc": cpu["nproc"],
                     "os_cpu_count": cpu["cpu_count"], "omp_num_threads": cpu["omp_num_threads"]}}


COPY_BYTES = 1 << 30


def rocpd_summary(dbs):
    """Per-kernel durations and counters from rocprofv3 SQLite outputs of --profile."""
    import sqlite3
    from collections import defaultdict

    for path in dbs:
        db = sqlite3.connect(path)
        print(f"== {path}")
        rows = db.execute("select name, duration, grid_x, workgroup_x, vgpr_count, "
                          "accum_vgpr_count, sgpr_count, lds_size from kernels "
                          "order by start").fetchall()
        if rows:
            agg = defaultdict(list)
            info = {}
            for name, dur, gx, wx, vg, ag, sg, lds in rows:
                agg[name].append(dur / 1000.0)
                info[name] = (gx // max(wx, 1), wx, vg, ag, sg, lds)
            print("kernel | calls | avg us | min us | max us | workgroups x threads | "
                  "vgpr/agpr/sgpr | lds B")
            for name, ds in sorted(agg.items(), key=lambda kv: -sum(kv[1])):
                gx, wx, vg, ag, sg, lds = info[name]
                print(f"{name} | {len(ds)} | {sum(ds) / len(ds):.2f} | {min(ds):.2f} | "
                      f"{max(ds):.2f} | {gx} x {wx} | {vg}/{ag}/{sg} | {lds}")
        crow = db.execute("select kernel_name, counter_name, value from counters_collection "
                          "order by start").fetchall()
        if crow:
            agg = defaultdict(list)
            for name, cn, v in crow:
                agg[(name, cn)].append(v)
            print("kernel | counter | dispatches | avg KiB per dispatch")
            for (name, cn), vs in sorted(agg.items()):
                print(f"{name} | {cn} | {len(vs)} | {sum(vs) / len(vs):.1f}")
            factors = {}
            for (name, cn), vs in agg.items():
                # the calibration copies only: a run's own small copies (a few KiB) are no
                # measure of the counter's unit
                floor = COPY_BYTES / 1024.0 / 16.0
                if "copyBuffer" in name and cn in ("FETCH_SIZE", "WRITE_SIZE") and \
                        max(vs) >= floor:
                    big = [v for v in vs if v >= floor]
                    avg = sum(big) / len(big)
                    f = (COPY_BYTES / 1024.0) / avg
                    factors[cn] = f
                    print(f"calibration: {cn} over {len(big)} copies of {COPY_BYTES} B reads "
                          f"{avg:.1f} KiB per copy -> scale factor {f:.4f}")
            for (name, cn), vs in sorted(agg.items()):
                if cn in factors and "copyBuffer" not in name:
                    b = sum(vs) / len(vs) * 1024.0 * factors[cn]
                    print(f"scaled {cn} | {name} | {b:.0f} B per dispatch")


def workloads_table(torch, nv, workloads, iters: int = 50, warm_s: float = 0.1):
    """Markdown table of every workload, passes timed with HIP events: per-call GPU time
    of calls captured in a HIP graph (host out of the loop), the eager call rate (with
    the binding allocating the outputs and workspace per call, and with them passed), the
    search pass's per-launch p50 with p10 and p90, and its p50 with the Infinity Cache
    flushed before every launch; the oracle beside."""
    import oracle

    oracle.build(force=False)
    threads = host_cpus()["threads"]
    dev = torch.device("cuda:0")
    stream = torch.cuda.current_stream(dev)
    flush = CacheFlush(torch, dev)
    print("| # | workload | quantize call GB/s (eager; eager, outputs and workspace passed; graph) | search pass us, graph (GB/s) | "
          "search pass us per launch: p50 [p10, p90] warm; p50 cold | amax pass us | "
          "max-scaling control us | SS / control | dequantize us (GB/s) | oracle quantize s "
          f"({threads} threads) |")
    print("|---|---|---|---|---|---|---|---|---|---|")
    for idx in (1, 2, 3, 4, 5):
        w = workloads.WORKLOADS[idx]
        xh = workloads.workload(idx)
        if xh.dtype == np.uint16:
            x = torch.from_numpy(xh.view(np.int16)).view(torch.bfloat16).to(dev)
            esz = 2
        else:
            x = torch.from_numpy(xh).to(dev)
            esz = 4
        offs, had, sink = w["offsets"], w["hadamard"], w["sink"]
        n_all = x.numel()
        if sink:
            nf, nl = sink
            B, H, T, D = x.shape
            n = B * H * (T - nf - nl) * D
            ns = B * H * (nf + nl) * D
            call = lambda: nv.quantize_kv_sink(x, nf, nl, offs, hadamard=had)
            c, s, g, snk = call()
            call_pre = None  # the sink call allocates its outputs
            gfix = g.clone()
            search = lambda: nv.quantize_kv_sink(x, nf, nl, offs, hadamard=had, global_scale=gfix)
            control = lambda: nv.quantize_kv_sink(x, nf, nl, (0, 0), hadamard=had,
                                                   global_scale=gfix)
            mid = x[:, :, nf:T - nl].contiguous()
            amax = lambda: nv.global_scale(mid, hadamard=had)
            out_dt = x.dtype
            deq = lambda: nv.dequantize_kv_sink(c, s, g, snk, T, nf, nl, out_dt)
            qbytes = n * esz + n // 2 + n // 16 + 4 + 2 * ns * esz
            dbytes = n // 2 + n // 16 + 4 + ns * esz + n_all * esz
        else:
            n = n_all
            call = lambda: nv.quantize(x, offs, hadamard=had)
            c, s, g = call()
            gfix = g.clone()
            wsp = torch.empty(nv.workspace_bytes(n // x.shape[-1], x.shape[-1]),
                              dtype=torch.uint8, device=dev)
            outp = (torch.empty_like(c), torch.empty_like(s), torch.empty_like(g))
            call_pre = lambda: nv.quantize(x, offs, hadamard=had, workspace=wsp, out=outp)
            search = lambda: nv.quantize(x, offs, hadamard=had, global_scale=gfix)
            control = lambda: nv.quantize(x, (0, 0), hadamard=had, global_scale=gfix)
            amax = lambda: nv.global_scale(x, hadamard=had)
            out_dt = torch.float32 if esz == 4 or had else torch.bfloat16
            deq = lambda: nv.dequantize(c, s, g, out_dt)
            qbytes = quantize_bytes(n, esz)
            dbytes = n // 2 + n // 16 + 4 + n * (4 if out_dt == torch.float32 else 2)
        t0 = time.perf_counter()
        while time.perf_counter() - t0 < warm_s:
            call()
        torch.cuda.synchronize()
        reps = 20 if n >= (1 << 24) else 100
        ms = {k: graph_time_ms(torch, f, reps, stream)
              for k, f in (("call", call), ("search", search), ("amax", amax),
                           ("control", control), ("deq", deq))}
        ms["call_eager"] = event_time_ms(torch, call, iters, stream)
        if call_pre is not None:
            ms["call_eager_pre"] = event_time_ms(torch, call_pre, iters, stream)
        warm = percentiles(launch_times_ms(torch, search, iters, stream))
        cold = percentiles(launch_times_ms(torch, search, 30, stream, between=flush))
        t1 = time.perf_counter()
        if sink:
            oracle.quantize_kv_sink(xh, nf, nl, *offs, hadamard=had, nthreads=threads)
        else:
            oracle.quantize(xh, *offs, hadamard=had, nthreads=threads)
        t_or = time.perf_counter() - t1
        gbs = lambda b, m: b / (m * 1e-3) / 1e9
        pre = f"{gbs(qbytes, ms['call_eager_pre']):.0f}" if call_pre is not None else "-"
        print(f"| {idx} | {w['name']} | {gbs(qbytes, ms['call_eager']):.0f}; {pre}; "
              f"{gbs(qbytes, ms['call']):.0f} | "
              f"{ms['search'] * 1e3:.1f} ({gbs(qbytes, ms['search']):.0f}) | "
              f"{warm[1] * 1e3:.1f} [{warm[0] * 1e3:.1f}, {warm[2] * 1e3:.1f}]; "
              f"{cold[1] * 1e3:.1f} | "
              f"{ms['amax'] * 1e3:.1f} | {ms['control'] * 1e3:.1f} | "
              f"{ms['search'] / ms['control']:.2f} | {ms['deq'] * 1e3:.1f} "
              f"({gbs(dbytes, ms['deq']):.0f}) | {t_or:.2f} |", flush=True)


def kv_append_table(torch, nv, workloads, iters: int = 200):
    """Markdown table: KV append (K cache [1, 8, *, 128] bf16, sinks 128 + 128) per call."""
    dev = torch.device("cuda:0")
    stream = torch.cuda.current_stream(dev)
    B, H, D, nf, nl = 1, 8, 128, 128, 128
    print("| tokens appended per call | us per call | tokens/s (per head) | coded GB/s |")
    print("|---|---|---|---|")
    xh = workloads.workload(3, (B, H, 32768, D))
    x = torch.from_numpy(xh.view(np.int16)).view(torch.bfloat16).to(dev)
    g = nv.global_scale(x[:, :, nf:32768 - nl].contiguous())
    for t_new in (1, 16, 256, 4096):
        cap_tokens = 32768 + (iters + 4) * t_new + 8
        cache = nv.kv_cache_alloc(B, H, D, cap_tokens, nf, nl, torch.bfloat16, dev)
        nv.kv_append(cache, x, g)  # prefill 32768 tokens
        chunk = x[:, :, :t_new].contiguous()
        for _ in range(3):
            nv.kv_append(cache, chunk, g)
        torch.cuda.synchronize()
        ms = event_time_ms(torch, lambda: nv.kv_append(cache, chunk, g), iters, stream)
        coded = B * H * t_new * D  # elements leaving the window per call (steady state)
        nbytes = coded * 2 + coded // 2 + coded // 16 + B * H * t_new * D * 2
        print(f"| {t_new} | {ms * 1e3:.1f} | {t_new / (ms * 1e-3):.0f} | "
              f"{nbytes / (ms * 1e-3) / 1e9:.1f} |", flush=True)

    # A decode step at the device-resident length, captured once and replayed: append
    # one K and one V token to 32K-token caches, then attention of one query per head
    # (32 query heads over the 8 K/V heads) over the caches, unsplit or with the keys
    # split into pieces of S tokens (each piece on its own workgroups, then merged).
    steps, warm = 100, 5
    variants = [("append", 0), ("append2", 0)] + \
        [("append+attention", s) for s in (0, 128, 160, 256)] + \
        [("append2+attention", s) for s in (96, 128, 160)] + \
        [("attention", s) for s in (0, 64, 96, 128, 160, 192, 256, 512, 1024)]
    cap = 32768 + (steps + warm) * len(variants) + 8
    kc = nv.kv_cache_alloc(B, H, D, cap, nf, nl, torch.bfloat16, dev)
    vc = nv.kv_cache_alloc(B, H, D, cap, nf, nl, torch.bfloat16, dev)
    nv.kv_append_dev(kc, x, g)
    nv.kv_append_dev(vc, x, g)
    knew = x[:, :, :1].contiguous()
    vnew = x[:, :, 1:2].contiguous()
    q = nv.quantize(torch.from_numpy(workloads.workload(5, (1, 32, 1, 128)).view(np.int16))
                    .view(torch.bfloat16).to(dev))
    ws = torch.empty(max(nv.attention_split_workspace_bytes(1, 32, 1, cap, s)
                         for s in (64, 128)), dtype=torch.uint8, device=dev)
    torch.cuda.synchronize()
    graphs = []
    for parts, split in variants:
        gph = torch.cuda.CUDAGraph()
        side = torch.cuda.Stream()
        side.wait_stream(stream)
        with torch.cuda.graph(gph, stream=side):
            if parts.startswith("append2"):  # both appends in one call (one launch)
                nv.kv_append2_dev(kc, knew, g, vc, vnew, g)
            elif parts.startswith("append"):
                nv.kv_append_dev(kc, knew, g)
                nv.kv_append_dev(vc, vnew, g)
            if "attention" in parts:
                nv.attention_kv_cache(q, kc, g, vc, g, device_length=True, split=split,
                                      workspace=ws if split else None)
        graphs.append((parts, split, gph))
    torch.cuda.synchronize()
    print()
    print("| captured decode step (graph replay, device-resident length, ~32.9K tokens) "
          "| us per step |")
    print("|---|---|")
    for parts, split, gph in graphs:
        for _ in range(warm):
            gph.replay()
        ms = event_time_ms(torch, gph.replay, steps, stream)
        name = {"append": "append 1 K + 1 V token",
                "append2": "append 1 K + 1 V token in one call",
                "append+attention": "append 1 K + 1 V token, then attention of 32 query heads",
                "append2+attention": "append 1 K + 1 V token in one call, then attention of "
                                     "32 query heads",
                "attention": "attention of 32 query heads alone"}[parts]
        if "attention" in parts:
            name += f", keys split into pieces of {split}" if split else ", keys unsplit"
        print(f"| {name} | {ms * 1e3:.1f} |", flush=True)


def formats_table(torch, nv, workloads, iters: int = 50):
    """Markdown tables: relative quantization error (sum (x - x^)^2 / sum x^2) of NVFP4
    max scaling, NVFP4 ScaleSearch and MXFP4 (OCP rule and exponent search) on every
    workload (whole tensor, no sinks), the Hadamard variants on the 128-wide ones, and
    the MXFP4 kernels' times."""
    dev = torch.device("cuda:0")
    stream = torch.cuda.current_stream(dev)
    signs = np.random.default_rng(12345).integers(0, 2**32, 4, dtype=np.uint64).astype(np.uint32)

    def rel(yhat, ref, den):
        return float(((yhat.double() - ref.double()) ** 2).sum().item()) / den

    def chosen_offsets(x2d, scales, g):
        """Histogram of the chosen offset (scale pattern minus the max-scaling pattern
        E4M3(fl(fl(amax / 6) / S_g)), formed here with the same rounding rule) over the
        blocks with a finite amax and a normal default pattern."""
        am = x2d.float().abs().reshape(-1, 16).amax(1)
        t = (am / 6.0) / g.float()
        b = t.view(torch.int32)
        nrm = ((b + 0x7FFFF + ((b >> 20) & 1)) >> 20) - 960
        sub = torch.round(t * 512.0).to(torch.int32)
        p0 = torch.where(t < 2.0 ** -6, sub, nrm)
        p0 = torch.where(t >= 448.0, torch.full_like(p0, 126), p0)
        ok = torch.isfinite(am) & (p0 >= 8)
        f = scales.reshape(-1).to(torch.int32)[ok] - p0[ok]
        return torch.bincount(f + 8, minlength=17).cpu().numpy(), int(ok.sum().item())

    rows, times, hists = [], [], []
    for idx in (1, 2, 3, 4, 5):
        w = workloads.WORKLOADS[idx]
        xh = workloads.workload(idx)
        if xh.dtype == np.uint16:
            x = torch.from_numpy(xh.view(np.int16)).view(torch.bfloat16).to(dev)
            esz = 2
        else:
            x = torch.from_numpy(xh).to(dev)
            esz = 4
        x = x.reshape(-1, x.shape[-1])
        xf = x.float()
        den = float((xf.double() ** 2).sum().item())
        e = {}
        for offs in ((0, 0), (-2, 6), (-8, 8)):
            c, s, g = nv.quantize(x, offs)
            e[f"nv{offs}"] = rel(nv.dequantize(c, s, g), xf, den)
            if offs == (-2, 6):
                hists.append((idx,) + chosen_offsets(x, s, g))
        for offs in ((0, 0), (-1, 1)):
            c, s = nv.mxfp4_quantize(x, offs)
            e[f"mx{offs}"] = rel(nv.mxfp4_dequantize(c, s), xf, den)
        if esz == 2 and x.shape[-1] % 128 == 0:
            for name, kw in (("had", {}), ("rht", {"signs": signs})):
                yr = nv.hadamard128(x, **kw)
                dy = float((yr.double() ** 2).sum().item())
                c, s, g = nv.quantize(x, (-8, 8), hadamard=not kw, **kw)
                e[f"nv_{name}"] = rel(nv.dequantize(c, s, g), yr, dy)
                c, s = nv.mxfp4_quantize(yr, (0, 0))
                e[f"mx_{name}"] = rel(nv.mxfp4_dequantize(c, s), yr, dy)
        rows.append((idx, w["name"], e))
        n = x.numel()
        qb = n * esz + n // 2 + n // 32
        db = n // 2 + n // 32 + n * 4
        c, s = nv.mxfp4_quantize(x, (0, 0))
        t = {"q0": event_time_ms(torch, lambda: nv.mxfp4_quantize(x, (0, 0)), iters, stream),
             "q1": event_time_ms(torch, lambda: nv.mxfp4_quantize(x, (-1, 1)), iters, stream),
             "d": event_time_ms(torch, lambda: nv.mxfp4_dequantize(c, s), iters, stream)}
        times.append((idx, w["name"], t, qb, db))
        del xf

    scores = scores_table(torch, nv, workloads, signs)

    f = lambda v: f"{v:.3e}" if v is not None else "—"
    print("| # | workload | NVFP4 max scaling | NVFP4 ScaleSearch [-2,6] | NVFP4 SS [-8,8] | "
          "MXFP4 (OCP rule) | MXFP4 search [-1,1] | NVFP4 SS [-2,6] error below MXFP4 OCP |")
    print("|---|---|---|---|---|---|---|---|")
    for idx, name, e in rows:
        red = 1.0 - e["nv(-2, 6)"] / e["mx(0, 0)"]
        print(f"| {idx} | {name} | {f(e['nv(0, 0)'])} | {f(e['nv(-2, 6)'])} | "
              f"{f(e['nv(-8, 8)'])} | {f(e['mx(0, 0)'])} | {f(e['mx(-1, 1)'])} | "
              f"{100 * red:.1f}% |")
    print()
    print("| # | NVFP4 SS [-8,8] after Hadamard | after randomized Hadamard | "
          "MXFP4 after Hadamard | after randomized Hadamard |")
    print("|---|---|---|---|---|")
    for idx, name, e in rows:
        if "nv_had" in e:
            print(f"| {idx} | {f(e['nv_had'])} | {f(e['nv_rht'])} | {f(e['mx_had'])} | "
                  f"{f(e['mx_rht'])} |")
    print()
    print("| # | blocks | chosen offset of NVFP4 ScaleSearch [-2,6], share of blocks: "
          "-2 | -1 | 0 | 1 | 2 | 3 | 4 | 5 | 6 |")
    print("|---|---|---|---|---|---|---|---|---|---|---|")
    for idx, h, nb in hists:
        print(f"| {idx} | {nb} | " + " | ".join(f"{h[f + 8] / max(nb, 1):.3f}"
                                                 for f in range(-2, 7)) + " |")
    print()
    print("| Q (workload 5) against K (workload 3), 256 query rows per head x all 32768 keys | "
          "relative score error sum (S^ - S)^2 / sum S^2 | Q, K quantize ms |")
    print("|---|---|---|")
    for name, err, ms in scores:
        print(f"| {name} | {err:.4e} | {ms:.3f} |")
    print()
    gbs = lambda b, m: b / (m * 1e-3) / 1e9
    print("| # | MXFP4 quantize [0,0] us (GB/s) | MXFP4 quantize [-1,1] us (GB/s) | "
          "MXFP4 dequantize to FP32 us (GB/s) |")
    print("|---|---|---|---|")
    for idx, name, t, qb, db in times:
        print(f"| {idx} | {t['q0'] * 1e3:.1f} ({gbs(qb, t['q0']):.0f}) | "
              f"{t['q1'] * 1e3:.1f} ({gbs(qb, t['q1']):.0f}) | "
              f"{t['d'] * 1e3:.1f} ({gbs(db, t['d']):.0f}) |", flush=True)


def scores_table(torch, nv, workloads, signs, rows_per_head: int = 256):
    """Relative error of the attention scores QK^T computed from the coded operands, Q of
    workload 5 [1, 32, 32768, 128] (offsets [-8, 8]) against K of workload 3
    [1, 8, 32768, 128] (offsets [-2, 6]), grouped heads: plain ScaleSearch, the
    randomized Hadamard transform on both, the balancing pair (channel exponents from
    the calibration of Q against K) with and without the transform. Scores of
    `rows_per_head` sampled query rows per head against every key, in double."""
    dev = torch.device("cuda:0")
    stream = torch.cuda.current_stream(dev)
    bf = lambda a: torch.from_numpy(a.view(np.int16)).view(torch.bfloat16).to(dev)
    q, k = bf(workloads.workload(5)), bf(workloads.workload(3))
    rows = torch.from_numpy(np.sort(np.random.default_rng(7).choice(32768, rows_per_head,
                                                                    replace=False))).to(dev)
    e = nv.balance_exponents(q, k)
    qs, ks = q.double()[:, :, rows], k.double()
    ref = torch.matmul(qs.reshape(8, 4 * rows_per_head, 128), ks[0].transpose(1, 2).contiguous())
    den = float((ref ** 2).sum().item())
    variants = {
        "ScaleSearch": (dict(), dict()),
        "randomized Hadamard + ScaleSearch": (dict(signs=signs), dict(signs=signs)),
        "balancing pair + randomized Hadamard + ScaleSearch":
            (dict(signs=signs, balance=(e, "q")), dict(signs=signs, balance=(e, "k"))),
        "balancing pair + ScaleSearch": (dict(balance=(e, "q")), dict(balance=(e, "k"))),
    }
    out = []
    for name, (kq, kk) in variants.items():
        fn = lambda: (nv.quantize(q, (-8, 8), **kq), nv.quantize(k, (-2, 6), **kk))
        (qc, qsc, qg), (kc, ksc, kg) = fn()
        ms = event_time_ms(torch, fn, 5, stream)
        qd = nv.dequantize(qc, qsc, qg).double()[:, :, rows]
        kd = nv.dequantize(kc, ksc, kg).double()
        got = torch.matmul(qd.reshape(8, 4 * rows_per_head, 128), kd[0].transpose(1, 2).contiguous())
        out.append((name, float(((got - ref) ** 2).sum().item()) / den, ms))
        del qd, kd, got
    return out


def attention_operands(torch, nv, workloads):
    """Q [1, 32, 32768, 128] (workload 5 recipe), K [1, 8, 32768, 128] (workload 3 recipe),
    V [1, 8, 32768, 128] N(0, 1), all bf16, and random signs for the Hadamard transform."""
    dev = torch.device("cuda:0")
    rng = np.random.default_rng(17)
    qh = workloads.workload(5)
    kh = workloads.workload(3)
    vh = workloads.to_bf16_bits(rng.standard_normal(kh.shape).astype(np.float32))
    bf = lambda a: torch.from_numpy(a.view(np.int16)).view(torch.bfloat16).to(dev)
    signs = rng.integers(0, 2**32, 4, dtype=np.uint64).astype(np.uint32)
    return bf(qh), bf(kh), bf(vh), signs


def attention_profile(torch, nv, workloads, launches: int = 5):
    """Short run for rocprofv3: code Q, K, V once (ScaleSearch, randomized Hadamard on
    Q and K), then `launches` non-causal attention launches at 32K."""
    q, k, v, signs = attention_operands(torch, nv, workloads)
    ops = (nv.quantize(q, (-8, 8), signs=signs), nv.quantize(k, (-2, 6), signs=signs),
           nv.quantize(v, (-2, 6)))
    for _ in range(launches):
        nv.attention(*ops)
    torch.cuda.synchronize()


def hadamard_profile(torch, nv, workloads, launches: int = 5):
    """Short run for rocprofv3: workload 5 (bf16 Q [1, 32, 32768, 128]) quantized with the
    Hadamard transform and offsets [-8, 8] -- `launches` whole calls (amax pass with the
    transform, then the search pass with it), then the three 1 GiB device copies that
    calibrate the byte counters."""
    dev = torch.device("cuda:0")
    x = torch.from_numpy(workloads.workload(5).view(np.int16)).view(torch.bfloat16).to(dev)
    ws = torch.empty(nv.workspace_bytes(x.numel() // 128, 128), dtype=torch.uint8, device=dev)
    for _ in range(launches):
        nv.quantize(x, (-8, 8), hadamard=True, workspace=ws)
    src = torch.empty(1 << 30, dtype=torch.uint8, device=dev)
    dst = torch.empty_like(src)
    for _ in range(3):
        dst.copy_(src)
    torch.cuda.synchronize()
    print("[bench] hadamard profile run done", file=sys.stderr, flush=True)


def decode_profile(torch, nv, workloads, split: int = 160, launches: int = 5):
    """Short run for rocprofv3: K and V sink caches of 128 + 32768 + 128 tokens
    ([1, 8, *, 128], workload-3 recipe, ScaleSearch [-2, 6]), one query per head for 32
    query heads, then `launches` split-key cache attention calls (pieces of `split`,
    the token count read from device memory)."""
    dev = torch.device("cuda:0")
    B, H, D, nf, nl, T = 1, 8, 128, 128, 128, 32768 + 256
    x = torch.from_numpy(workloads.workload(3, (B, H, T, D)).view(np.int16)) \
        .view(torch.bfloat16).to(dev)
    g = nv.global_scale(x[:, :, nf:T - nl].contiguous())
    kc = nv.kv_cache_alloc(B, H, D, T, nf, nl, torch.bfloat16, dev)
    vc = nv.kv_cache_alloc(B, H, D, T, nf, nl, torch.bfloat16, dev)
    nv.kv_append_dev(kc, x, g)
    nv.kv_append_dev(vc, x, g)
    q = nv.quantize(torch.from_numpy(workloads.workload(5, (1, 32, 1, 128)).view(np.int16))
                    .view(torch.bfloat16).to(dev))
    # the token count read from device memory, as in a captured decode step
    ws = torch.empty(nv.attention_split_workspace_bytes(B, 32, 1, T - nf - nl, split),
                     dtype=torch.uint8, device=dev)
    for _ in range(launches):
        nv.attention_kv_cache(q, kc, g, vc, g, device_length=True, split=split, workspace=ws)
    torch.cuda.synchronize()


def attention_table(torch, nv, workloads, iters: int = 5):
    """Markdown table: attention on NVFP4 operands at 32K, Q [1, 32, 32768, 128] (workload 5
    recipe) against K [1, 8, 32768, 128] (workload 3 recipe) and V [1, 8, 32768, 128]
    N(0, 1), grouped heads; against PyTorch's bf16 scaled_dot_product_attention on the
    unquantized tensors."""
    import torch.nn.functional as F

    dev = torch.device("cuda:0")
    stream = torch.cuda.current_stream(dev)
    q, k, v, signs = attention_operands(torch, nv, workloads)
    B, Hq, N, D = q.shape
    flops = 4.0 * B * Hq * N * N * D
    quant = {
        "ScaleSearch, randomized Hadamard on Q and K": lambda: (
            nv.quantize(q, (-8, 8), signs=signs), nv.quantize(k, (-2, 6), signs=signs),
            nv.quantize(v, (-2, 6))),
        "max scaling, no transform": lambda: (
            nv.quantize(q, (0, 0)), nv.quantize(k, (0, 0)), nv.quantize(v, (0, 0))),
    }
    print("| operands | quantize Q, K, V ms | attention ms | attention TFLOP/s | "
          "fraction of bf16 MFMA peak | causal attention ms |")
    print("|---|---|---|---|---|---|")
    for name, fn in quant.items():
        ops = fn()
        torch.cuda.synchronize()
        tq = event_time_ms(torch, fn, iters, stream)
        attn = lambda: nv.attention(*ops)
        attn()
        torch.cuda.synchronize()
        ta = event_time_ms(torch, attn, iters, stream)
        tc = event_time_ms(torch, lambda: nv.attention(*ops, causal=True), iters, stream)
        print(f"| {name} | {tq:.3f} | {ta:.2f} | {flops / (ta * 1e-3) / 1e12:.0f} | "
              f"{flops / (ta * 1e-3) / 2.5e15:.3f} | {tc:.2f} |", flush=True)
    # the same operands through the sink cache (first and last 128 tokens in bf16)
    nf = nl = 128
    B, Hkv, T, D = k.shape
    qops = nv.quantize(q, (-8, 8), signs=signs)
    kg = nv.global_scale(k[:, :, nf:T - nl].contiguous(), signs=signs)
    vg = nv.global_scale(v[:, :, nf:T - nl].contiguous())
    kc = nv.kv_cache_alloc(B, Hkv, D, T, nf, nl, torch.bfloat16, dev)
    vc = nv.kv_cache_alloc(B, Hkv, D, T, nf, nl, torch.bfloat16, dev)
    nv.kv_append(kc, k, kg, (-2, 6), signs=signs)
    nv.kv_append(vc, v, vg, (-2, 6))
    cache_attn = lambda: nv.attention_kv_cache(qops, kc, kg, vc, vg)
    cache_attn()
    torch.cuda.synchronize()
    tk = event_time_ms(torch, cache_attn, iters, stream)
    print(f"| sink cache 128 + 128 bf16, middle ScaleSearch (K randomized Hadamard) | — | "
          f"{tk:.2f} | {flops / (tk * 1e-3) / 1e12:.0f} | {flops / (tk * 1e-3) / 2.5e15:.3f} | — |",
          flush=True)
    try:
        sdpa = lambda: F.scaled_dot_product_attention(q, k, v, enable_gqa=True)
        sdpa()
        torch.cuda.synchronize()
        ts = event_time_ms(torch, sdpa, iters, stream)
        print(f"| PyTorch bf16 scaled_dot_product_attention (unquantized) | — | {ts:.2f} | "
              f"{flops / (ts * 1e-3) / 1e12:.0f} | {flops / (ts * 1e-3) / 2.5e15:.3f} | — |")
    except Exception as e:  # noqa: BLE001 - report, do not fail the table
        print(f"| PyTorch bf16 scaled_dot_product_attention | failed: {type(e).__name__} | | | | |")


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    # ~0.1 s of warm-up: kernel durations settle after a power-management transient
    # of ~20 ms at the start of a run
    ap.add_argument("--steps", type=int, default=100)
    ap.add_argument("--warmup", type=int, default=200)
    ap.add_argument("--no-cpu", action="store_true")
    ap.add_argument("--profile", action="store_true",
                    help="short run for rocprofv3: a few launches of each kernel plus a "
                         "plain 1 GiB device copy for counter calibration; no JSON")
    ap.add_argument("--kv-append", action="store_true",
                    help="print a markdown table timing KV-cache appends (no JSON line)")
    ap.add_argument("--workloads", action="store_true",
                    help="print a markdown table timing all five workloads (no JSON line)")
    ap.add_argument("--formats", action="store_true",
                    help="print markdown tables of NVFP4 vs MXFP4 quantization error and the "
                         "MXFP4 kernel times (no JSON line)")
    ap.add_argument("--attention", action="store_true",
                    help="print a markdown table timing attention on NVFP4 operands at 32K "
                         "(no JSON line)")
    ap.add_argument("--decode-profile", action="store_true",
                    help="short run for rocprofv3: split-key cache attention, one query per "
                         "head over 32K-token caches")
    ap.add_argument("--decode-split", type=int, default=160,
                    help="piece size of --decode-profile (middle tokens per unit)")
    ap.add_argument("--hadamard-profile", action="store_true",
                    help="short run for rocprofv3: workload 5 quantized with the Hadamard "
                         "transform, offsets [-8, 8]")
    ap.add_argument("--attention-profile", action="store_true",
                    help="short run for rocprofv3: five non-causal attention launches at 32K")
    ap.add_argument("--sources", choices=sorted(SOURCE_GROUPS), default="quantize",
                    help="with --rocpd-summary: the source group whose hash the summary records")
    ap.add_argument("--rocpd-summary", nargs="+", metavar="DB",
                    help="print a text summary of rocprofv3 databases of a --profile run")
    args = ap.parse_args()
    if args.rocpd_summary:
        print(f"source_hash: {kernel_source_hash(args.sources)} (sources: "
              f"{', '.join(SOURCE_GROUPS[args.sources])})")
        rocpd_summary(args.rocpd_summary)
        return
    if args.gpus != 1:
        print(f"bench.py: the benchmark runs on one GPU only (asked for --gpus {args.gpus}); "
              "the quantizer has no multi-GPU path.", file=sys.stderr)
        sys.exit(2)

    import torch

    import microscaling_fp4_block_amd as nv
    import workloads

    nv.load()
    if args.workloads:
        workloads_table(torch, nv, workloads)
        return
    if args.kv_append:
        kv_append_table(torch, nv, workloads)
        return
    if args.formats:
        formats_table(torch, nv, workloads)
        return
    if args.attention:
        attention_table(torch, nv, workloads)
        return
    if args.decode_profile:
        decode_profile(torch, nv, workloads, split=args.decode_split)
        return
    if args.attention_profile:
        attention_profile(torch, nv, workloads)
        return
    if args.hadamard_profile:
        hadamard_profile(torch, nv, workloads)
        return
    dev = torch.device("cuda:0")
    print(f"[bench] generating workload 4 ({ROWS}x{COLS} bf16)", file=sys.stderr, flush=True)
    xh = workloads.workload(4)
    x = torch.from_numpy(xh.view(np.int16)).view(torch.bfloat16).to(dev)
    n = x.numel()
    ws = torch.empty(nv.workspace_bytes(ROWS, COLS), dtype=torch.uint8, device=dev)
    stream = torch.cuda.current_stream(dev)
    codes = torch.empty(ROWS, COLS // 2, dtype=torch.uint8, device=dev)
    scales = torch.empty(ROWS, COLS // 16, dtype=torch.uint8, device=dev)
    g = torch.empty(1, dtype=torch.float32, device=dev)
    y = torch.empty_like(x)
    out = (codes, scales, g)

    def step():  # the whole quantize call: amax pass, tensor scale, search, pack
        nv.quantize(x, OFFSETS, workspace=ws, out=out)

    step()
    torch.cuda.synchronize()
    gfix = g.clone()

    def search_only():
        nv.quantize(x, OFFSETS, global_scale=gfix, workspace=ws, out=out)

    def amax_only():
        nv.global_scale(x, workspace=ws)

    def control_only():
        nv.quantize(x, (0, 0), global_scale=gfix, workspace=ws, out=out)

    def dequant_only():
        nv.dequantize(codes, scales, g, torch.bfloat16, out=y)

    def quant_dequant():
        step()
        dequant_only()

    if args.profile:
        # Fixed launch order: a warm-up step, then 5 launches of each pass, then the
        # 1 GiB copies that calibrate the byte counters.
        for fn in (search_only, control_only, amax_only, dequant_only):
            for _ in range(5):
                fn()
        src = torch.empty(1 << 30, dtype=torch.uint8, device=dev)
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        print("[bench] profile run done", file=sys.stderr, flush=True)
        return

    # Per-pass breakdown first, each pass timed over its own launches on the same stream
    # (kernel durations settle over the first ~20 ms of GPU work of a process).
    print("[bench] timing the passes", file=sys.stderr, flush=True)
    t0 = time.perf_counter()
    while time.perf_counter() - t0 < 0.1:
        step()
    torch.cuda.synchronize()
    iters = max(args.steps, 20)
    ms_search = event_time_ms(torch, search_only, iters, stream)
    ms_amax = event_time_ms(torch, amax_only, iters, stream)
    ms_ctrl = event_time_ms(torch, control_only, iters, stream)
    ms_deq = event_time_ms(torch, dequant_only, iters, stream)
    ms_qdq = event_time_ms(torch, quant_dequant, iters, stream)
    s10, s50, s90 = percentiles(launch_times_ms(torch, search_only, iters, stream))

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    print(f"[bench] timing {args.steps} steps", file=sys.stderr, flush=True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    ms_step = event_time_ms(torch, step, args.steps, stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    # the 1 GiB reference copies run after the timed steps: right before them they
    # left the clocks low for the first milliseconds of a short run (20 steps after
    # 5 warm-up steps measured 8% slow)
    copy_rate = copy_gbs(torch, dev, stream)

    qbytes = quantize_bytes(n, 2)
    value = qbytes / (ms_step * 1e-3) / 1e9
    amax_bytes = n * 2
    # the whole call reads the input twice (amax pass, then search pass): at the HBM peak
    # it could reach qbytes / (qbytes + amax_bytes) of the peak in qbytes-per-second terms
    two_pass_ceiling = qbytes / (qbytes + amax_bytes)
    search_gbs = search_pass_bytes(n, 2) / (ms_search * 1e-3) / 1e9
    ncand = OFFSETS[1] - OFFSETS[0] + 1
    alg_flops = OPS_PER_ELEMENT_CANDIDATE * ncand * n
    alg_tflops = alg_flops / (ms_search * 1e-3) / 1e12
    # VALU check: the kernel's own wave-instructions per launch (committed counters,
    # fixed for given sources and input) x 64 lanes over the live launch time
    valu_waves = committed_figure("valu_wave_instructions_per_launch", SEARCH_KERNEL)
    lane_rate = None if valu_waves is None else valu_waves * 64 / (ms_search * 1e-3) / 1e12
    qdq_bytes = qbytes + dequantize_bytes(n, 2)
    out = {
        "metric": METRIC,
        "value": round(value, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {
            "workload": "bf16 weight 8192x28672 N(0,0.02^2) seed 3: the whole nvfp4_quantize "
                        "call, ScaleSearch offsets [-2,6] (global amax pass, tensor scale, "
                        "candidate search, pack); inputs resident in HBM",
            "rows": ROWS, "cols": COLS, "block": 16, "offsets": list(OFFSETS),
            "bytes_per_step": qbytes,
        },
        "pct_hbm_peak": round(100 * value / HBM_PEAK_GBS, 2),
        "two_pass_ceiling_pct_hbm_peak": round(100 * two_pass_ceiling, 1),
        "roofline": {
            "bound": "hbm",
            "achieved": round(search_gbs, 2),
            "peak": HBM_PEAK_GBS,
            "unit": "GB/s",
            "frac": round(search_gbs / HBM_PEAK_GBS, 4),
            "traffic": committed_traffic(SEARCH_KERNEL),
            "kernel": SEARCH_KERNEL,
            "kernel_ms": round(ms_search, 4),
            "bytes_per_launch": search_pass_bytes(n, 2),
            "valu_check": {
                "limit": "VALU issue (the kernel's binding limit)",
                "lane_instructions_per_launch": None if valu_waves is None
                else int(valu_waves * 64),
                "achieved": None if lane_rate is None else round(lane_rate, 2),
                "peak": round(VALU_PEAK_TLANE, 2),
                "unit": "T lane-instructions/s",
                "frac": None if lane_rate is None else round(lane_rate / VALU_PEAK_TLANE, 4),
                "issue_frac_counters": committed_valu_issue(SEARCH_KERNEL),
            },
            "exact_search_fp32_ops_per_launch": alg_flops,
            "exact_search_fp32_tops": round(alg_tflops, 2),
        },
        "breakdown": {
            "search_pass_ms": round(ms_search, 4),
            "search_pass_gbs": round(search_gbs, 2),
            "search_pass_per_launch_ms_p10_p50_p90": [round(s10, 4), round(s50, 4), round(s90, 4)],
            "amax_pass_ms": round(ms_amax, 4),
            "amax_pass_gbs": round(amax_bytes / (ms_amax * 1e-3) / 1e9, 2),
            "amax_plus_search_ms": round(ms_amax + ms_search, 4),
            "max_scaling_control_ms": round(ms_ctrl, 4),
            "scalesearch_over_max_scaling": round(ms_search / ms_ctrl, 3),
            "dequantize_bf16_ms": round(ms_deq, 4),
            "dequantize_bf16_gbs": round(dequantize_bytes(n, 2) / (ms_deq * 1e-3) / 1e9, 2),
            "quantize_then_dequantize_ms": round(ms_qdq, 4),
            "quantize_then_dequantize_gbs": round(qdq_bytes / (ms_qdq * 1e-3) / 1e9, 2),
            "hip_d2d_copy_gbs": round(copy_rate, 1),
            "wall_s_timed_region": round(wall, 3),
        },
        "profiles": profile_status(),
    }
    if not args.no_cpu:
        print("[bench] timing the CPU oracle on a sample", file=sys.stderr, flush=True)
        out["cpu_baseline"] = cpu_baseline(xh)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
