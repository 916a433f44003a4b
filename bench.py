#!/usr/bin/env python3
"""Throughput of the weight-only-quantized decode GEMV on one MI355X.

Headline workload: Q2_0 ternary GEMV, M=1, N=K=5120 (an attention qkv/o-sized
projection), weights cold-cycled through a ring of distinct copies larger than
the 256 MB Infinity Cache.  One step = one q2_0_gemv call on the next ring
copy, with the activations and every weight copy already resident in HBM.

Metric: effective weight-stream bandwidth = packed weight bytes per call
(N*(K/128)*34) / time per call, and its fraction of the 8 TB/s HBM peak.

Prints one JSON line (rank 0, N=1).  Extra keys: ``roofline`` (the kernel's
own average duration from HIP events on its stream, against HBM peak),
``cpu_baseline`` (the CPU oracle timed on host cores over a bounded sample)
and ``sweep`` (the other synthetic workloads: Q2_0 batched M, W8A16, FFN
shapes), unless ``--no-sweep``.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import re
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0
METRIC = "effective weight-stream GB/s & % HBM peak, Q2_0/FP8 GEMV N=K=5120, M=1..16"
RING_BYTES = 512 * 1024 * 1024


def parse_args():
    p = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=2000)
    p.add_argument("--warmup", type=int, default=200)
    p.add_argument("--no-sweep", action="store_true", help="headline workload only")
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--cpu-seconds", type=float, default=10.0)
    p.add_argument("--only", default=None, help="run a single sweep entry by name (profiling)")
    p.add_argument("--copy-probe", action="store_true",
                   help="also run a plain 256 MiB device copy (reference for counter scaling)")
    return p.parse_args()


def log(msg: str) -> None:
    print(msg, file=sys.stderr, flush=True)


def ring_size(nbytes: int) -> int:
    if nbytes < (1 << 20):  # the small correctness workload is latency-bound; no cold ring
        return 8
    return max(8, math.ceil(RING_BYTES / nbytes))


def q2_0_bytes(N, K):
    return N * (K // 128) * 34


def fp8_bytes(N, K):
    return N * K + ((N + 127) // 128) * (K // 128) * 4


# ------------------------------------------------------------------ workloads
class Q2Workload:
    fmt = "q2_0"

    def __init__(self, name, wid, N, K, M):
        self.name, self.wid, self.N, self.K, self.M = name, wid, N, K, M
        self.bytes = q2_0_bytes(N, K)
        self.dispatches = (M + 7) // 8

    def setup(self, torch, gen, wqd):
        N, K, M = self.N, self.K, self.M
        A = gen.activations(self.wid, K, M)
        codes, d = gen.q2_0_weights(self.wid, N, K)
        packed = wqd.q2_0_pack(codes, d)
        self.host = (A, codes, d)
        row = (K // 128) * 34
        base = torch.from_numpy(packed).to("cuda").view(N, row)
        self.R = ring_size(self.bytes)
        # copy i = copy 0 with its weight rows rotated by i (distinct bytes and addresses)
        self.ring = [torch.roll(base, shifts=i, dims=0).contiguous().view(-1) for i in range(self.R)]
        del base
        self.A = torch.from_numpy(A.view("int16")).to("cuda")
        self.C = torch.empty((M, N), dtype=torch.int16, device="cuda")

    def call(self, wqd, i):
        B = self.ring[i % self.R]
        if self.M == 1:
            wqd.q2_0_gemv(self.A, B, self.C, self.N, self.K)
        else:
            wqd.q2_0_gemv_batchm(self.A, B, self.C, self.N, self.K, 128, self.M)

    def check(self, torch, np, oracle, check_fn, copy_idx):
        A, codes, d = self.host
        self.call(self._wqd, copy_idx)
        torch.cuda.synchronize()
        got = self.C.cpu().numpy().view(np.uint16)
        cols = np.arange(self.N) if self.N * self.M <= 5120 * 16 else \
            np.sort(np.random.Generator(np.random.PCG64(copy_idx)).choice(self.N, 1024, replace=False))
        src = (cols - copy_idx) % self.N  # rolled rows
        ref = oracle.q2_0_gemv(A, codes[src], d[src])
        check_fn(got[:, cols], ref)

    def oracle_call(self, oracle, nthreads):
        A, codes, d = self.host
        oracle.q2_0_gemv(A, codes, d, nthreads=nthreads)

    def free(self):
        self.ring = self.A = self.C = None


class Fp8Workload:
    fmt = "w8a16"
    entry = "w8a16_gemm_m16"  # the matrix-core GEMM; Fp8ValuWorkload times the vector-ALU GEMV

    def __init__(self, name, wid, N, K, M):
        self.name, self.wid, self.N, self.K, self.M = name, wid, N, K, M
        self.bytes = fp8_bytes(N, K)
        self.dispatches = (M + 15) // 16

    def setup(self, torch, gen, wqd):
        N, K, M = self.N, self.K, self.M
        A = gen.activations(self.wid, K, M)
        W, S = gen.w8a16_weights(self.wid, N, K)
        self.host = (A, W, S)
        base = torch.from_numpy(W).to("cuda")
        self.R = ring_size(self.bytes)
        self.ring = [torch.roll(base, shifts=i, dims=0).contiguous() for i in range(self.R)]
        del base
        self.S = torch.from_numpy(S).to("cuda")
        self.A = torch.from_numpy(A.view("int16")).to("cuda")
        self.C = torch.empty((M, N), dtype=torch.int16, device="cuda")

    def call(self, wqd, i):
        W = self.ring[i % self.R]
        fn = getattr(wqd, self.entry)
        for r0 in range(0, self.M, 16):  # 17..32 rows: two calls on contiguous halves
            rows = min(16, self.M - r0)
            fn(self.A[r0:r0 + rows], W, self.S, self.C[r0:r0 + rows], rows, self.N, self.K)

    def check(self, torch, np, oracle, check_fn, copy_idx):
        A, W, S = self.host
        self.call(self._wqd, copy_idx)
        torch.cuda.synchronize()
        got = self.C.cpu().numpy().view(np.uint16)
        cols = np.sort(np.random.Generator(np.random.PCG64(copy_idx)).choice(self.N, 256, replace=False))
        src = (cols - copy_idx) % self.N
        ref = np.concatenate([oracle.w8a16_gemm(A, W[s:s + 1], S[c // 128:c // 128 + 1])
                              for s, c in zip(src, cols)], axis=1)
        check_fn(got[:, cols], ref)

    def oracle_call(self, oracle, nthreads):
        A, W, S = self.host
        oracle.w8a16_gemm(A, W, S, nthreads=nthreads)

    def free(self):
        self.ring = self.A = self.C = self.S = None


class Fp8ValuWorkload(Fp8Workload):
    fmt = "w8a16-valu"
    entry = "w8a16_gemv_batch16"

    def __init__(self, name, wid, N, K, M):
        super().__init__(name, wid, N, K, M)
        rows = 8 if K <= 10240 else max(1, (160 * 1024) // (((K + 1023) // 1024) * 2048))  # rows per launch
        self.dispatches = sum((min(16, M - r0) + rows - 1) // rows for r0 in range(0, M, 16))


class ReadProbe:
    """The workload's weight ring read by a plain coalesced kernel (no
    arithmetic, no stores): the single-launch HBM read ceiling for the same
    bytes, cold-cycled the same way, timed like the workload."""

    def __init__(self, torch, lib, wl):
        import ctypes
        self.torch, self.lib, self.ring, self.R = torch, lib, wl.ring, wl.R
        self.nbytes = (wl.ring[0].numel() * wl.ring[0].element_size()) // 16 * 16
        self.sink = torch.zeros(1, dtype=torch.int32, device="cuda")
        lib.wqd_bench_read.argtypes = [ctypes.c_void_p, ctypes.c_uint64, ctypes.c_void_p, ctypes.c_void_p]
        lib.wqd_bench_read.restype = ctypes.c_int

    def call(self, wqd, i):
        t = self.ring[i % self.R]
        rc = self.lib.wqd_bench_read(t.data_ptr(), self.nbytes, self.sink.data_ptr(),
                                     self.torch.cuda.current_stream().cuda_stream)
        if rc != 0:
            raise RuntimeError(f"wqd_bench_read failed with hipError {rc}")


HEADLINE = ("q2_0 M=1 N=5120 K=5120", Q2Workload, 2, 5120, 5120, 1)


def sweep_list():
    out = [("q2_0 M=1 N=256 K=1024", Q2Workload, 1, 256, 1024, 1)]
    for M in (2, 4, 5, 8, 16):
        out.append((f"q2_0 M={M} N=5120 K=5120", Q2Workload, 3, 5120, 5120, M))
    for M in (1, 8, 16):
        out.append((f"w8a16 M={M} N=5120 K=5120", Fp8Workload, 4, 5120, 5120, M))
    for M in (1, 2, 4, 8):
        out.append((f"w8a16-valu M={M} N=5120 K=5120", Fp8ValuWorkload, 4, 5120, 5120, M))
    for (N, K) in ((17408, 5120), (5120, 17408)):
        for M in (1, 8, 16, 32):
            out.append((f"q2_0 M={M} N={N} K={K}", Q2Workload, 5, N, K, M))
            out.append((f"w8a16 M={M} N={N} K={K}", Fp8Workload, 5, N, K, M))
        out.append((f"w8a16-valu M=1 N={N} K={K}", Fp8ValuWorkload, 5, N, K, 1))
    return out


# ------------------------------------------------------------------- timing
# Fewest launches in one captured graph: a graph of a small ring (8 copies of
# a small matrix) replays faster than the host enqueues the next replay.
MIN_GRAPH_STEPS = 64


def graph_len(R: int) -> int:
    """Steps in the full graph: the ring walked whole, as many times as needed
    to reach MIN_GRAPH_STEPS (step i reads copy i mod R)."""
    return R * max(1, math.ceil(MIN_GRAPH_STEPS / R))


def timed_plan(R: int, steps: int):
    """How the timed region walks the ring of R weight copies: `full` replays
    of a graph over steps 0..L-1 (L = graph_len(R), step i on copy i mod R),
    then one graph over steps 0..rest-1 (steps = full * L + rest, exactly).
    An untimed replay of the full graph runs just before, so every timed step
    reads the copy that was last read R steps earlier: R - 1 other copies in
    between."""
    full, rest = divmod(steps, graph_len(R))
    return full, rest


def timed_traffic(R: int, nbytes: int, steps: int):
    """Weight bytes of the timed region: distinct copies touched, and the
    fewest bytes of other weight copies read between two reads of one copy
    (the reuse distance; above the 256 MB on-die cache it is a cold read)."""
    distinct = min(steps, R)
    return {"distinct_copies": distinct, "distinct_bytes": distinct * nbytes,
            "reuse_distance_bytes": (R - 1) * nbytes}


def _capture(torch, wqd, wl, copies):
    stream = torch.cuda.current_stream()
    side = torch.cuda.Stream()
    side.wait_stream(stream)
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.stream(side):
        with torch.cuda.graph(graph, stream=side):
            for i in copies:
                wl.call(wqd, i)
    torch.cuda.synchronize()
    return graph


_SLEEP_CYCLES = None


def _gpu_pre_delay(torch):
    """Keep the GPU busy for about 0.3 ms before the timed region opens, so
    that the host has enqueued the timed launches by then and the host's
    launch cost stays out of the measured device time.  The spin kernel is
    torch's own bounded one; its length is calibrated once with events."""
    global _SLEEP_CYCLES
    if _SLEEP_CYCLES is None:
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        probe = 1_000_000
        torch.cuda._sleep(probe)  # first launch loads the kernel
        torch.cuda.synchronize()
        e0.record()
        torch.cuda._sleep(probe)
        e1.record()
        torch.cuda.synchronize()
        ms = max(e0.elapsed_time(e1), 1e-3)
        _SLEEP_CYCLES = int(min(probe * 0.3 / ms, 2e9))
    torch.cuda._sleep(_SLEEP_CYCLES)


def time_workload(torch, wqd, wl, steps, warmup):
    """Milliseconds per step over the timed region, HIP events recorded on the
    stream the kernels run on.

    Returns (graph, eager).  graph: `steps` steps replayed from captured HIP
    graphs that walk the weight ring in order (timed_plan), which is how a
    decode loop issues fixed-shape launches and leaves only the GPU's own
    per-dispatch cost between kernels; every timed step reads a copy last read
    R steps before, whatever `steps` is.  eager: the same number of steps
    launched one by one from Python, continuing around the ring, which adds
    the host's launch cost (several microseconds per call) whenever that
    exceeds the kernel."""
    R = wl.R
    for i in range(warmup):
        wl.call(wqd, i)
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream()
    t0, t1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t0.record(stream)
    for i in range(steps):
        wl.call(wqd, warmup + i)
    t1.record(stream)
    torch.cuda.synchronize()
    eager = t0.elapsed_time(t1) / steps

    full, rest = timed_plan(R, steps)
    g_full = _capture(torch, wqd, wl, range(graph_len(R)))
    g_rest = _capture(torch, wqd, wl, range(rest)) if rest else None
    g_full.replay()  # untimed: the whole ring, ending at copy R - 1
    _gpu_pre_delay(torch)
    t0.record(stream)
    for _ in range(full):
        g_full.replay()
    if g_rest is not None:
        g_rest.replay()
    t1.record(stream)
    torch.cuda.synchronize()
    del g_full, g_rest
    return t0.elapsed_time(t1) / steps, eager


def cpu_info():
    """Host facts reported beside the CPU baseline."""
    model = None
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                model = line.split(":", 1)[1].strip()
                break
    except OSError:
        pass
    try:
        usable = len(os.sched_getaffinity(0))
    except Exception:
        usable = os.cpu_count() or 1
    return {"cpu_model": model, "nproc": os.cpu_count(), "usable_cpus": usable}


# CPU threads of one GPU's share of the GPU host: the oracle's worker threads
# are capped there, whatever the host's core count.
GPU_SHARE_CPUS = 16


def cpu_threads() -> int:
    return max(1, min(GPU_SHARE_CPUS, cpu_info()["usable_cpus"]))


# The headline's kernel and the committed rocprofv3 summary that covers it.
HEADLINE_KERNEL = {"name": "q2_0_pairs_kernel<1, 8, 3, 2, 1, 0>", "source": "q2_0_mfma.hip",
                   "profile": "q2_0_gemv_kernel_m1_5120x5120"}


def profile_facts(kernel_src: str, name: str) -> dict:
    """HBM bytes per launch and kernel-trace average from the committed
    rocprofv3 summary, if it was taken on the current kernel source (else
    empty)."""
    prof = os.path.join(ROOT, "profiles", f"{name}.md")
    if not os.path.exists(prof):
        return {}
    text = open(prof).read()
    sha = hashlib.sha256(open(kernel_src, "rb").read()).hexdigest()
    m_sha = re.search(r"kernel_source_sha256:\s*([0-9a-f]{64})", text)
    if not m_sha or m_sha.group(1) != sha:
        return {}
    out = {}
    m_t = re.search(r"traffic_bytes_per_launch:\s*([0-9.]+)", text)
    if m_t:
        out["traffic"] = float(m_t.group(1))
    m_u = re.search(r"trace_avg_us:\s*([0-9.]+)", text)
    if m_u:
        out["trace_us"] = float(m_u.group(1))
    return out


def main():
    args = parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print("bench.py measures one GPU only: this library has no multi-GPU path "
              "(the kernels would shard by output rows; see the design notes). Run with --gpus 1.",
              file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    from weight_quantized_decode_block_amd import inputs as gen
    from weight_quantized_decode_block_amd import wqd

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    torch.cuda.set_device(0)
    wqd.lib()

    import ctypes
    from weight_quantized_decode_block_amd import build as hip_build
    if not os.path.exists(hip_build.BENCH_LIB):
        sys.exit(f"{hip_build.BENCH_LIB} is missing: build first (python -m weight_quantized_decode_block_amd.build)")
    read_lib = ctypes.CDLL(hip_build.BENCH_LIB)

    import oracle  # parity checks and the CPU baseline only
    sys.path.insert(0, os.path.join(ROOT, "tests"))
    from parity import check_parity

    def run(entry, steps, warmup):
        name, cls, wid, N, K, M = entry
        wl = cls(name, wid, N, K, M)
        wl._wqd = wqd
        t = time.time()
        wl.setup(torch, gen, wqd)
        log(f"[bench] {name}: ring of {wl.R} copies x {wl.bytes} B set up in {time.time() - t:.1f}s")
        wl.check(torch, np, oracle, lambda g, r: check_parity(g, r, name), 0)
        wl.check(torch, np, oracle, lambda g, r: check_parity(g, r, name), wl.R // 2 + 1)
        step_ms, eager_ms = time_workload(torch, wqd, wl, steps, warmup)
        probe = ReadProbe(torch, read_lib, wl)
        read_ms, _ = time_workload(torch, wqd, probe, steps, warmup)
        res = {"workload": name, "format": wl.fmt, "N": N, "K": K, "M": M, "ring": wl.R,
               "dispatches": wl.dispatches, "bytes_per_call": wl.bytes,
               "us_per_call": round(step_ms * 1e3, 3),
               "gbs": round(wl.bytes / (step_ms * 1e-3) / 1e9, 1),
               "us_per_call_eager": round(eager_ms * 1e3, 3),
               "read_ceiling_us": round(read_ms * 1e3, 3),
               "read_ceiling_gbs": round(probe.nbytes / (read_ms * 1e-3) / 1e9, 1)}
        res["frac_hbm"] = round(res["gbs"] / HBM_PEAK_GBS, 4)
        res["frac_read_ceiling"] = round(read_ms / step_ms, 4)
        res["timed"] = timed_traffic(wl.R, wl.bytes, steps)
        log(f"[bench] {name}: {res['us_per_call']} us/call, {res['gbs']} GB/s, "
            f"{100 * res['frac_hbm']:.1f}% of HBM peak (eager launches: {res['us_per_call_eager']} us/call); "
            f"plain read of the same ring {res['read_ceiling_us']} us ({res['read_ceiling_gbs']} GB/s)")
        return wl, res

    if args.copy_probe:
        # a plain device-to-device copy of known size: 256 MiB read + 256 MiB
        # written per launch, the reference for scaling traffic counters
        src = torch.empty(256 << 20, dtype=torch.uint8, device="cuda").fill_(1)
        dst = torch.empty_like(src)
        for _ in range(5):
            dst.copy_(src)
        torch.cuda.synchronize()
        log("[bench] copy probe: 5 copies of 268435456 B done")
        del src, dst
        torch.cuda.empty_cache()

    if args.only:
        entries = [e for e in [HEADLINE] + sweep_list() if e[0] == args.only]
        if not entries:
            sys.exit(f"unknown workload {args.only!r}")
        wl, res = run(entries[0], args.steps, args.warmup)
        print(json.dumps({"only": res}))
        return

    wl, head = run(HEADLINE, args.steps, args.warmup)

    cpu = None
    if not args.no_cpu_baseline:
        def oracle_rate(nthr, seconds):
            calls, t0 = 0, time.perf_counter()
            while True:
                wl.oracle_call(oracle, nthr)
                calls += 1
                el = time.perf_counter() - t0
                if el >= seconds:
                    return calls, el

        info = cpu_info()
        nthr = cpu_threads()
        calls, el = oracle_rate(nthr, args.cpu_seconds)
        calls1, el1 = oracle_rate(1, max(1.0, args.cpu_seconds / 3))
        cpu = {"value": round(wl.bytes * calls / el / 1e9, 4), "unit": "GB/s", "cores": nthr,
               "kind": "oracle",
               "sample": f"oracle_q2_0_gemv over the whole N=K=5120 M=1 workload (ring copy 0), "
                         f"{calls} calls in {el:.2f} s on {nthr} threads (one GPU's share of the host's CPUs); "
                         f"1 thread: {calls1} calls in {el1:.2f} s",
               "value_1_core": round(wl.bytes * calls1 / el1 / 1e9, 4),
               "us_per_call": round(el / calls * 1e6, 1), "us_per_call_1_core": round(el1 / calls1 * 1e6, 1),
               **info}
        log(f"[bench] cpu oracle: {cpu['value']} GB/s ({calls} calls, {el:.1f}s, {nthr} threads); "
            f"1 thread {cpu['value_1_core']} GB/s; {info}")
    wl.free()
    torch.cuda.empty_cache()

    sweep = []
    if not args.no_sweep:
        for entry in sweep_list():
            w2, r2 = run(entry, min(args.steps, 1000), min(args.warmup, 100))
            w2.free()
            torch.cuda.empty_cache()
            sweep.append(r2)

    kern_src = os.path.join(ROOT, "weight_quantized_decode_block_amd", "csrc", HEADLINE_KERNEL["source"])
    prof = profile_facts(kern_src, HEADLINE_KERNEL["profile"])
    achieved = head["gbs"]  # one dispatch per step, back to back: step time = average launch duration
    tt = head["timed"]
    line = {
        "metric": METRIC,
        "value": head["gbs"],
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(head["us_per_call"] / 1e3, 6),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": "Q2_0 ternary GEMV M=1 N=5120 K=5120 group=128, bf16 activations, "
                               f"weights cycled in order through a ring of {head['ring']} distinct copies "
                               f"({head['ring'] * head['bytes_per_call'] / 2**20:.0f} MiB); the timed "
                               f"{args.steps} steps touch {tt['distinct_copies']} distinct copies "
                               f"({tt['distinct_bytes'] / 2**20:.0f} MiB) and every timed read of a copy comes "
                               f"{tt['reuse_distance_bytes'] / 2**20:.0f} MiB of other weight copies after its "
                               f"previous read (above the 256 MB on-die cache); launches replayed from HIP graphs",
                   "bytes_per_call": head["bytes_per_call"], "frac_hbm_peak": head["frac_hbm"],
                   "us_per_call": head["us_per_call"], "us_per_call_eager": head["us_per_call_eager"],
                   "timed": tt},
        "roofline": {"bound": "hbm", "achieved": achieved, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(achieved / HBM_PEAK_GBS, 4),
                     "traffic": prof.get("traffic"),
                     "kernel": HEADLINE_KERNEL["name"],
                     "launch_us_avg_events": head["us_per_call"],
                     "trace_us_avg": prof.get("trace_us"),
                     "note": "achieved = algorithmic weight bytes per launch / average launch duration from HIP "
                             "events around graph-replayed launches on the kernel's stream; trace_us_avg is the "
                             "rocprofv3 kernel-trace average of the committed profile (null if the kernel source "
                             "changed since)"},
        "cpu_baseline": cpu,
        "read_ceiling": {"us_per_call": head["read_ceiling_us"], "gbs": head["read_ceiling_gbs"],
                         "frac": head["frac_read_ceiling"],
                         "kernel": "plain coalesced read of the same weight ring copies, graph-replayed "
                                   "(libwqd_bench.so); frac = its time / the GEMV's time"},
    }
    if sweep:
        line["sweep"] = sweep
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
