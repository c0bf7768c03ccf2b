#!/usr/bin/env python3
"""Benchmark of the KDA chunk solver on one MI355X.

Metric: 64x64 tril inverses per second, plus the achieved HBM bandwidth of
the solver kernel as a fraction of the 8 TB/s peak, on the packed workload
of 16 requests x 512 tokens with 64 heads (8192 chunk-head matrices, fp32 A
in, fp32 X out). One step is one solver call over the whole batch: chunk
map, tile loads, the four diagonal inverses, the block merge and the stores
all run inside it. Inputs are resident in HBM before the timed region, and
the steps rotate over several independently generated buffer sets (more
bytes than the 256 MB Infinity Cache) so that no step reads its input from
the cache.

Other workloads (--workload) are diagnostics: the other batch shapes, the
16- and 32-token branches, the path that builds A from keys, decays and
write strengths inside the solver (timed beside the unfused pair: A stored,
then solved), and the fused KDA decode core. --oracle-table times the CPU
oracle alone on the five solver batch shapes.

Prints one JSON line on stdout; diagnostics go to stderr.
"""
from __future__ import annotations

import argparse
import ctypes
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, AMD published peak
MFMA_F32_PEAK_TFLOPS = 157.3   # MI355X dense FP32 matrix peak, AMD published
# The pages' H200 solver times after the change they describe (context: a
# different GPU, dtypes not stated), as inverses per second:
#   8192 tokens x 64 heads (8192 matrices): 0.476 ms;  64 tokens x 64 heads: 0.0254 ms.
H200_INV_PER_S = {"packed_16x512_h64_f32": 8192 / 0.476e-3, "packed_1x64_h64_f32": 64 / 0.0254e-3}
SOLVE_WORKLOADS = ["packed_1x64_h64_f32", "dense_b4_t512_h16_bf16_f32", "packed_16x512_h64_f32",
                   "packed_ragged48_h64_f32_bf16", "packed_1x131072_h64_f32",
                   "packed_16x512_h64_c16_f32", "packed_16x512_h64_c32_f32"]
KKT_WORKLOADS = ["packed_16x512_h64_k128_kkt_bf16_f32", "packed_16x512_h64_k128_kkt_f32_f32"]
DECODE_WORKLOADS = [f"decode_b{B}_h32_d128_w4_bf16" for B in (2, 4, 8, 16, 32)]
WORKLOADS = SOLVE_WORKLOADS + KKT_WORKLOADS + DECODE_WORKLOADS
# The decode page's per-layer medians of its fused GFX950 kernel, by batch
# size (graph replay; model shapes not stated): context, not a target.
DECODE_PAGES_US = {2: 11.19, 4: 11.78, 8: 13.30, 16: 15.25, 32: 22.14}
MAIN_WORKLOAD = "packed_16x512_h64_f32"
METRIC = "64x64 tril inverses/sec + achieved HBM GB/s (% peak), 8192 tok x 64 heads"
COPY_KERNEL = "kda_probe_copy_kernel"


def dtype_bytes(name: str) -> int:
    return 2 if name in ("bf16", "f16") else 4


def kernel_of(workload: str):
    """(kernel name pattern, sources its code comes from) of the kernel a
    workload times; a counter summary taken on other sources is not used.
    The pattern is matched against rocprofv3's demangled kernel names."""
    if workload in KKT_WORKLOADS:  # the fused kernel, not the matrix-only one
        return r"tril_kkt<.*, true>", ["tril_device.h", "tril_kkt.hip", "tril_launch.h"]
    if workload in DECODE_WORKLOADS:
        return r"kda_decode_step_kernel<", ["tril_device.h", "kda_decode.hip", "tril_launch.h"]
    import synth
    C = synth.CONFIGS[workload].get("chunk", 64)
    if C == 64:  # the column kernel (few chunk-heads), the per-wavefront kernel or, for
        # long launches with 9+ heads, the 4-head one
        return r"tril_inv_fused_(heads4|mfma|cols)<", ["tril_device.h", "tril_group.h",
                                                  "tril_fused.hip", "tril_launch.h",
                                                  "launch_common.cpp"]
    if C == 32:  # the per-wavefront kernel or, for long launches with 32+ heads, the group one
        return r"tril_inv_c32(_group)?<", ["tril_device.h", "tril_small.hip", "tril_launch.h",
                                           "launch_common.cpp"]
    return rf"tril_inv_c{C}<", ["tril_device.h", "tril_small.hip", "tril_launch.h"]


def copy_bytes_of(workload: str) -> int:
    """Bytes the copy probe moves each way for a workload: A's size, or the
    decays' size for the path that builds A from keys."""
    import synth
    if workload in KKT_WORKLOADS:
        cfg = synth.KKT_CONFIGS[workload]
        return int(sum(synth.config_lengths(cfg))) * cfg["H"] * cfg["K"] * 4
    if workload in DECODE_WORKLOADS:  # the state pool of one set
        cfg = synth.DECODE_CONFIGS[workload]
        return cfg["slots"] * cfg["H"] * cfg["d"] * cfg["d"] * 4
    cfg = synth.CONFIGS[workload]
    return (int(sum(synth.config_lengths(cfg))) * cfg["H"] * cfg.get("chunk", 64) *
            dtype_bytes(cfg["a_dtype"]))


def traffic_file(workload: str) -> str:
    return os.path.join(ROOT, "profiles", f"traffic_{workload}.json")


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def load_copy_probe():
    lib = ctypes.CDLL(os.path.join(ROOT, "tril_solve_amd", "libkda_bench_probe.so"))
    lib.kda_probe_copy_f32.restype = ctypes.c_int
    lib.kda_probe_copy_f32.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int64,
                                       ctypes.c_void_p]
    lib.kda_probe_stream.restype = ctypes.c_int
    lib.kda_probe_stream.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_void_p,
                                     ctypes.c_void_p, ctypes.c_int64, ctypes.c_int64,
                                     ctypes.c_int64, ctypes.c_void_p]
    return lib


PROBE_KINDS = {"copy": 0, "read": 1, "fill": 2}
PROBE_POLICIES = {"default": 0, "nontemporal": 1, "nt_stores": 2}


def probe_bytes(kind: str, nbytes: int) -> int:
    """HBM bytes one streaming probe moves over a buffer of nbytes: a copy
    reads and writes it, a read or a fill touches it once."""
    return 2 * nbytes if kind == "copy" else nbytes


def probe_sweep(torch, stream, dev, tensors, reps=20):
    """Streaming probes (copy, read-only, write-only) over the rotation of
    `tensors` (each a source of the same size, with a destination of its
    own), every unroll, cache policy and grid size; prints one JSON line per
    setting to stdout and returns the fastest setting per kind."""
    lib = load_copy_probe()
    n = tensors[0].numel() * tensors[0].element_size() // 4
    cus = torch.cuda.get_device_properties(dev).multi_processor_count
    dsts = [torch.empty(n, dtype=torch.float32, device=dev) for _ in tensors]
    best = {}
    grids = [cus * k for k in (1, 2, 4, 8, 16, 32)] + [min(n // 4 // 256, 1 << 20)]
    for kind, kc in PROBE_KINDS.items():
        for pol, pc in PROBE_POLICIES.items():
            if kind == "read" and pc == 2:
                continue  # no stores to make nontemporal
            for unroll in (1, 2, 4, 8):
                for blocks in grids:
                    args = [(kc, unroll, pc, ctypes.c_void_p(t.data_ptr()),
                             ctypes.c_void_p(d.data_ptr()), n, d.numel(), blocks,
                             ctypes.c_void_p(stream.cuda_stream))
                            for t, d in zip(tensors, dsts)]
                    for a in args[:2]:
                        if lib.kda_probe_stream(*a) != 0:
                            raise RuntimeError(f"probe {kind} failed")
                    e0 = torch.cuda.Event(enable_timing=True)
                    e1 = torch.cuda.Event(enable_timing=True)
                    e0.record(stream)
                    for i in range(reps):
                        lib.kda_probe_stream(*args[i % len(args)])
                    e1.record(stream)
                    torch.cuda.synchronize()
                    us = e0.elapsed_time(e1) * 1e3 / reps
                    gbs = probe_bytes(kind, 4 * n) / (us * 1e-6) / 1e9
                    row = {"probe": kind, "policy": pol, "unroll": unroll, "blocks": blocks,
                           "blocks_per_cu": round(blocks / cus, 2), "us": round(us, 2),
                           "gbs": round(gbs, 1), "frac_of_8tbs": round(gbs / HBM_PEAK_GBS, 4)}
                    print(json.dumps(row), flush=True)
                    if kind not in best or gbs > best[kind]["gbs"]:
                        best[kind] = row
    return best


def _code_only(text: str) -> str:
    """C++ source without comments and with whitespace runs collapsed, so a
    comment edit leaves the kernel hash unchanged (the sources hold no string
    literals with comment markers)."""
    import re
    text = re.sub(r"/\*.*?\*/", " ", text, flags=re.S)
    text = re.sub(r"//[^\n]*", " ", text)
    return " ".join(text.split())


def kernel_hash(workload: str) -> str:
    """Hash of the code (comments aside) of the sources a workload's kernel
    is built from."""
    h = hashlib.sha256()
    for f in kernel_of(workload)[1]:
        with open(os.path.join(ROOT, "tril_solve_amd", "csrc", f), encoding="utf-8") as fh:
            h.update(_code_only(fh.read()).encode())
    return h.hexdigest()[:16]


def algorithmic_bytes(lengths, H, a_bytes, x_bytes, C=64) -> int:
    """Full C-wide rows of A read and X written: rows x H x C x (in + out)."""
    return int(sum(lengths)) * H * C * (a_bytes + x_bytes)


def kkt_algorithmic_bytes(lengths, H, K, k_bytes, x_bytes) -> int:
    """Keys, decays (FP32) and write strengths read, full 64-wide rows of X
    written: rows x H x (K (k + 4) + k + 64 x)."""
    return int(sum(lengths)) * H * (K * (k_bytes + 4) + k_bytes + 64 * x_bytes)


def load_traffic(workload: str):
    """HBM bytes per launch from the committed rocprofv3 counter summary, or
    None when it is missing or was taken on other kernel sources."""
    try:
        with open(traffic_file(workload)) as f:
            t = json.load(f)
    except (OSError, ValueError):
        return None
    if t.get("kernel_hash") != kernel_hash(workload):
        return None
    return int(t["hbm_bytes_per_launch"])


def _counter_mean(csv_path: str, kernel: str, counter: str) -> tuple[float, int]:
    """Mean value of `counter` (KiB per dispatch) over the dispatches of the
    kernels whose name matches the pattern `kernel`, from a rocprofv3 counter
    CSV."""
    import csv
    import re
    pat = re.compile(kernel)
    vals = []
    with open(csv_path, newline="") as f:
        for row in csv.DictReader(f):
            if pat.search(row["Kernel_Name"]) and row["Counter_Name"] == counter:
                vals.append(float(row["Counter_Value"]))
    if not vals:
        raise SystemExit(f"{csv_path}: no {counter} rows for {kernel}")
    return sum(vals) / len(vals), len(vals)


def record_traffic(workload: str, csvs, out_path: str) -> dict:
    """Counter summary of a workload's kernel: FETCH_SIZE and WRITE_SIZE (KiB
    per dispatch) each scaled by what the same counter reads for the copy
    probe moving a known byte count each way."""
    fetch_csv, write_csv, copy_fetch_csv, copy_write_csv = csvs
    k = kernel_of(workload)[0]
    fetch, nf = _counter_mean(fetch_csv, k, "FETCH_SIZE")
    write, nw = _counter_mean(write_csv, k, "WRITE_SIZE")
    cfetch, _ = _counter_mean(copy_fetch_csv, COPY_KERNEL, "FETCH_SIZE")
    cwrite, _ = _counter_mean(copy_write_csv, COPY_KERNEL, "WRITE_SIZE")
    known = copy_bytes_of(workload) / 1024.0
    fs, ws = known / cfetch, known / cwrite
    rd, wr = int(fetch * fs * 1024), int(write * ws * 1024)
    t = {"kernel": k, "workload": workload, "kernel_hash": kernel_hash(workload),
         "dispatches": {"fetch": nf, "write": nw},
         "fetch_size_kib_raw": round(fetch, 1), "write_size_kib_raw": round(write, 1),
         "copy_fetch_size_kib_raw": round(cfetch, 1), "copy_write_size_kib_raw": round(cwrite, 1),
         "copy_known_kib_each_way": round(known, 1),
         "fetch_scale": round(fs, 5), "write_scale": round(ws, 5),
         "hbm_read_bytes_per_launch": rd, "hbm_write_bytes_per_launch": wr,
         "hbm_bytes_per_launch": rd + wr,
         "commands": [
             f"rocprofv3 --pmc {c} -f csv -d <out> -o run -- python3 bench.py --workload "
             f"{workload} {extra}"
             for extra in ("--steps 10 --warmup 2 --no-cpu-baseline",
                           "--probe copy --steps 3 --warmup 1")
             for c in ("FETCH_SIZE", "WRITE_SIZE")]}
    with open(out_path, "w") as f:
        json.dump(t, f, indent=1)
    return t


def cpu_baseline(d, budget_s=12.0):
    import oracle
    n = 0
    t0 = time.perf_counter()
    while True:
        oracle.tril_inv_packed(d["A"], d["cu_seqlens"], d["a_dtype"])
        n += 1
        el = time.perf_counter() - t0
        if el >= budget_s:
            break
    mats = d["num_chunks"] * d["H"] * n
    return {"value": mats / el, "unit": "inverses/s", "cores": oracle.num_threads(),
            "kind": "oracle",
            "sample": f"whole workload ({d['num_chunks'] * d['H']} matrices) solved {n}x "
                      f"by the fp64 oracle in {el:.1f} s",
            "cpu_model": _cpu_model(), "nproc": os.cpu_count()}


def oracle_table(budget_s: float = 3.0) -> int:
    """Times the fp64 oracle on the five solver configurations (the same
    inputs the GPU legs use), with all host threads and with one, and prints
    one JSON line per configuration. No GPU use."""
    import oracle
    import synth
    for name in SOLVE_WORKLOADS[:5]:
        log(f"[oracle] {name}")
        d = synth.make(name)
        mats = d["num_chunks"] * d["H"]
        row = {"workload": name, "matrices": mats, "cpu_model": _cpu_model(),
               "nproc": os.cpu_count()}
        for label, nth in (("all_threads", 0), ("one_thread", 1)):
            n, t0 = 0, time.perf_counter()
            while True:
                if d["layout"] == "dense":
                    oracle.tril_inv_dense(d["A"], d["a_dtype"], nthreads=nth)
                else:
                    oracle.tril_inv_packed(d["A"], d["cu_seqlens"], d["a_dtype"], nthreads=nth)
                n += 1
                el = time.perf_counter() - t0
                if el >= budget_s:
                    break
            row[label] = {"threads": oracle.num_threads() if nth == 0 else 1, "calls": n,
                          "ms_per_call": 1e3 * el / n, "inverses_per_s": mats * n / el}
        print(json.dumps(row), flush=True)
        del d
    return 0


def _cpu_model() -> str:
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def describe(d) -> str:
    if d["layout"] == "dense":
        shape = f"dense B={d['B']} x T={d['T']}"
    elif len(set(d["lengths"])) == 1:
        shape = f"packed {len(d['lengths'])} x {d['lengths'][0]} tokens"
    else:
        shape = f"packed {len(d['lengths'])} ragged requests, {d['T_total']} tokens"
    if "K" in d:
        return (f"{shape}, {d['H']} heads, A built from {d['k_dtype']} keys (K={d['K']}), "
                f"fp32 decays and {d['k_dtype']} write strengths -> {d['x_dtype']} X "
                f"({d['num_chunks'] * d['H']} chunk-head 64x64 matrices)")
    C = d.get("chunk", 64)
    return (f"{shape}, {d['H']} heads, {d['a_dtype']} A -> {d['x_dtype']} X "
            f"({d['num_chunks'] * d['H']} chunk-head {C}x{C} matrices)")


class Timer:
    """Launch timing on one stream: K back-to-back calls bracketed by HIP
    events on that stream and by device synchronisation, plus a per-launch
    distribution from individually bracketed calls (after the timed region)."""

    def __init__(self, torch, stream):
        self.torch, self.stream = torch, stream

    def run(self, calls, steps, warmup):
        torch, stream = self.torch, self.stream
        for i in range(warmup):
            calls[i % len(calls)]()
        torch.cuda.synchronize()
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        e0.record(stream)
        for i in range(steps):
            calls[i % len(calls)]()
        e1.record(stream)
        torch.cuda.synchronize()
        el = time.perf_counter() - t0
        avg = e0.elapsed_time(e1) * 1e-3 / steps  # seconds per call
        reps = min(50, steps)
        ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
              for _ in range(reps)]
        for i, (a, b) in enumerate(ev):
            a.record(stream)
            calls[i % len(calls)]()
            b.record(stream)
        torch.cuda.synchronize()
        per = sorted(a.elapsed_time(b) * 1e3 for a, b in ev)  # microseconds
        dist = {"median": per[len(per) // 2], "min": per[0],
                "p90": per[int(0.9 * (len(per) - 1))], "launches": reps}
        return el, avg, dist


def graph_replay(torch, launch_all, n_calls, replays=50):
    """Per-call time of n_calls launches captured once into a HIP graph (the
    graph-replay setting) and replayed: launch_all() issues the calls on the
    current stream. Returns (average over back-to-back replays, median of
    individually bracketed replays), both in microseconds per call."""
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    g = torch.cuda.CUDAGraph()
    with torch.cuda.stream(side):
        launch_all()  # warm-up outside the graph
    side.synchronize()
    with torch.cuda.graph(g):
        launch_all()
    torch.cuda.synchronize()
    for _ in range(3):
        g.replay()
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for _ in range(replays):
        g.replay()
    e1.record(stream)
    torch.cuda.synchronize()
    avg = e0.elapsed_time(e1) * 1e3 / (replays * n_calls)
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
          for _ in range(replays)]
    for a, b in ev:
        a.record(stream)
        g.replay()
        b.record(stream)
    torch.cuda.synchronize()
    per = sorted(a.elapsed_time(b) * 1e3 / n_calls for a, b in ev)
    return avg, per[len(per) // 2]


class CopyProbe:
    """Streaming copies of a tensor's bytes into a destination of its own
    (one per source): the plain copy (counter calibration) and the fastest
    copy of the probe sweep (the measured ceiling)."""

    def __init__(self, torch, stream, dev):
        self.torch, self.stream, self.dev = torch, stream, dev
        self.lib = load_copy_probe()
        self.dst = {}

    def _dst(self, A):
        D = self.dst.get(A.data_ptr())
        if D is None:
            nbytes = A.numel() * A.element_size()
            D = self.torch.empty(nbytes // 4, dtype=self.torch.float32, device=self.dev)
            if nbytes % 16 or D.numel() * 4 != nbytes:
                raise RuntimeError("copy probe: source and destination sizes differ")
            self.dst[A.data_ptr()] = D
        return D

    def __call__(self, A):
        """The plain copy (one thread per 16 bytes, default cache policy)."""
        D = self._dst(A)
        if self.lib.kda_probe_copy_f32(ctypes.c_void_p(A.data_ptr()), ctypes.c_void_p(D.data_ptr()),
                                       D.numel(), ctypes.c_void_p(self.stream.cuda_stream)) != 0:
            raise RuntimeError("copy probe failed")

    def tuned(self, A):
        """The fastest copy of the probe sweep: one nontemporal 16-byte load
        and store per thread."""
        D = self._dst(A)
        n = D.numel()
        st = self.lib.kda_probe_stream(PROBE_KINDS["copy"], 1, PROBE_POLICIES["nontemporal"],
                                       ctypes.c_void_p(A.data_ptr()),
                                       ctypes.c_void_p(D.data_ptr()), n, n,
                                       max(1, min(n // 4 // 256, 1 << 20)),
                                       ctypes.c_void_p(self.stream.cuda_stream))
        if st != 0:
            raise RuntimeError("tuned copy probe failed")

    def ceiling_gbs(self, tensors):
        """(measured copy ceiling, plain copy rate): the faster of the sweep's
        fastest copy (nontemporal; best on buffers far past the 256 MB cache)
        and the plain copy (default policy; faster on buffers of a few tens of
        MB), both on the rotation, and the plain one alone."""
        tuned = self.rate_gbs(tensors)
        plain = self.rate_gbs(tensors, tuned=False)
        return max(tuned, plain), plain

    def rate_gbs(self, tensors, ncopy=40, tuned=True):
        """Read + write bytes per second of a copy over the rotation: the
        fastest streaming copy of the probe sweep (one nontemporal 16-byte
        load and store per thread) when `tuned`, else the plain copy."""
        torch = self.torch
        fn = self.tuned if tuned else self
        for i in range(4):
            fn(tensors[i % len(tensors)])
        c0 = torch.cuda.Event(enable_timing=True)
        c1 = torch.cuda.Event(enable_timing=True)
        c0.record(self.stream)
        for i in range(ncopy):
            fn(tensors[i % len(tensors)])
        c1.record(self.stream)
        torch.cuda.synchronize()
        copy_s = c0.elapsed_time(c1) * 1e-3 / ncopy
        t = tensors[0]
        return 2 * t.numel() * t.element_size() / copy_s / 1e9

    def only(self, tensors, args):
        """--probe copy: copies only (counter calibration runs)."""
        for _ in range(args.warmup + args.steps):
            for t in tensors:
                self(t)
        self.torch.cuda.synchronize()
        log(f"copy probe: {args.warmup + args.steps} x {len(tensors)} copies of "
            f"{tensors[0].numel() * tensors[0].element_size()} bytes read + written")
        return 0


def base_line(args, el, k_avg, dist, mats, bytes_alg, nsets, metric, vs_baseline, config,
              io_dtype):
    """The JSON line's common fields. `dtype` is the arithmetic type of every
    kernel (FP32); `io_dtype` names the element types of the inputs and the
    output. roofline.achieved counts algorithmic bytes (what the operation
    must move by definition); the measured HBM rate, from the committed
    counter summary, is added by with_measured_hbm."""
    achieved = bytes_alg / k_avg / 1e9
    return {
        "metric": metric,
        "value": mats * args.steps / el,
        "unit": "inverses/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": el / args.steps * 1e3,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": vs_baseline,
        "dtype": "f32",
        "io_dtype": io_dtype,
        "data": f"synthetic (seeded delta-rule generator, {nsets} rotating buffer sets)",
        "config": config,
        "roofline": {"bound": "hbm", "achieved": achieved, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": achieved / HBM_PEAK_GBS, "traffic": None,
                     "bytes": "algorithmic"},
        "kernel_us_avg": k_avg * 1e6,
        "kernel_us_per_launch": dist,
        "algorithmic_bytes_per_launch": bytes_alg,
    }


def with_measured_hbm(out, traffic):
    """Sets roofline.traffic and, when it is known, the HBM rate the kernel
    achieves in measured bytes (counter bytes per launch / kernel time)."""
    out["roofline"]["traffic"] = traffic
    if traffic:
        gbs = traffic / (out["kernel_us_avg"] * 1e-6) / 1e9
        out["hbm_measured"] = {"bytes_per_launch": traffic, "achieved": gbs,
                               "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": gbs / HBM_PEAK_GBS}
    return out


def run_solve(args, torch, np, dev, stream):
    import synth
    import tril_solve_amd as kt

    cfg = synth.CONFIGS[args.workload]
    d0 = synth.make(cfg)
    C = d0["chunk"]
    if C != 64 and args.algo not in ("auto", "fused"):
        log(f"bench.py: the {C}-token branch has a single kernel (algo auto or fused)")
        return 2
    a_bytes, x_bytes = dtype_bytes(cfg["a_dtype"]), dtype_bytes(cfg["x_dtype"])
    H = cfg["H"]
    T = d0["T_total"]
    mats = d0["num_chunks"] * H
    bytes_alg = algorithmic_bytes(d0["lengths"], H, a_bytes, x_bytes, C)
    nsets = args.sets or max(1, min(16, -(-(1 << 30) // bytes_alg)))
    x_dt = {"bf16": torch.bfloat16, "f16": torch.float16}.get(cfg["x_dtype"], torch.float32)

    def to_dev(d):
        if cfg["a_dtype"] in ("bf16", "f16"):
            dt = torch.bfloat16 if cfg["a_dtype"] == "bf16" else torch.float16
            return torch.from_numpy(d["A"].view(np.int16)).view(dt).to(dev)
        return torch.from_numpy(d["A"]).to(dev)

    sets = []
    for i in range(nsets):
        d = d0
        if i:
            c = dict(cfg)
            c["seed"] = cfg["seed"] + 100 * i
            d = synth.make(c)
        A = to_dev(d)
        sets.append((A, torch.empty(A.shape, dtype=x_dt, device=dev)))
    dense = cfg["layout"] == "dense"
    cu = None if dense else torch.from_numpy(d0["cu_seqlens"]).to(dev)
    if C != 64:
        nbytes, chosen = 0, "fused"
    elif dense:
        nbytes, chosen = kt.kda_tril_inv_workspace_size(T, cfg["B"], d0["num_chunks"], H,
                                                        args.algo)
    else:
        nbytes, chosen = kt.kda_tril_inv_workspace_size(T, len(d0["lengths"]), 0, H, args.algo)
    ws = torch.empty(max(nbytes // 4, 1), dtype=torch.float32, device=dev) if nbytes else None
    torch.cuda.synchronize()

    copy = CopyProbe(torch, stream, dev)
    if args.probe == "copy":
        return copy.only([A for A, _ in sets], args)
    if args.probe == "sweep":
        best = probe_sweep(torch, stream, dev, [A for A, _ in sets])
        print(json.dumps({"best": best, "buffer_bytes": A.numel() * A.element_size(),
                          "rotation": len(sets)}), flush=True)
        return 0

    cmap = None
    if args.chunk_map and not dense:  # built once on the host, reused by every call
        cmap = torch.tensor([(s, c) for s, L in enumerate(d0["lengths"])
                             for c in range(-(-int(L) // C))], dtype=torch.int32, device=dev)
    if dense:
        calls = [kt.prepare_dense(A, X, workspace=ws, algo=args.algo) for A, X in sets]
    else:
        calls = [kt.prepare_packed(A, X, cu, workspace=ws, algo=args.algo, chunk_indices=cmap)
                 for A, X in sets]
    el, k_avg, dist = Timer(torch, stream).run(calls, args.steps, args.warmup)

    # measured copy roofline: a plain streaming copy of A's byte count, read
    # and written, same buffer rotation, events over the region
    copy_gbs, copy_plain = (copy.ceiling_gbs([A for A, _ in sets]) if a_bytes == 4
                            else (None, None))

    h200 = H200_INV_PER_S.get(args.workload)
    metric = METRIC if C == 64 else f"{C}x{C} tril inverses/sec + achieved HBM GB/s (% peak)"
    value = mats * args.steps / el
    out = base_line(args, el, k_avg, dist, mats, bytes_alg, len(sets), metric,
                    (value / h200) if h200 else None,
                    {"workload": describe(d0), "tokens": T, "heads": H,
                     "requests": len(d0["lengths"]), "matrices": mats,
                     "a_dtype": cfg["a_dtype"], "x_dtype": cfg["x_dtype"],
                     "algo": args.algo, "plan": chosen,
                     "chunks_from": "caller chunk map" if cmap is not None else "cu_seqlens scan"},
                    f"{cfg['a_dtype']} A -> {cfg['x_dtype']} X")
    if args.algo in ("auto", "fused") and chosen == "fused":
        with_measured_hbm(out, load_traffic(args.workload))
    out["copy_roofline_gbs"] = copy_gbs
    out["copy_plain_gbs"] = copy_plain
    if not args.no_cpu_baseline and args.workload == MAIN_WORKLOAD:
        log("timing the CPU oracle ...")
        out["cpu_baseline"] = cpu_baseline(d0)
    else:
        out["cpu_baseline"] = None
    print(json.dumps(out), flush=True)
    return 0


def run_kkt(args, torch, np, dev, stream):
    """The path that builds A from keys k, decays g and write strengths beta
    inside the solver; also times the unfused pair (A stored in FP32 by the
    matrix-only kernel, then the 64-token solver) on the same inputs."""
    import synth
    import tril_solve_amd as kt

    cfg = synth.KKT_CONFIGS[args.workload]
    d0 = synth.make_kkt(cfg)
    kb, xb = dtype_bytes(cfg["k_dtype"]), dtype_bytes(cfg["x_dtype"])
    H, K, T = cfg["H"], cfg["K"], d0["T_total"]
    mats = d0["num_chunks"] * H
    bytes_alg = kkt_algorithmic_bytes(d0["lengths"], H, K, kb, xb)
    nsets = args.sets or max(1, min(16, -(-(1 << 30) // bytes_alg)))
    x_dt = {"bf16": torch.bfloat16, "f16": torch.float16}.get(cfg["x_dtype"], torch.float32)
    k_dt = {"bf16": torch.bfloat16, "f16": torch.float16}.get(cfg["k_dtype"], torch.float32)

    def to_dev(a):
        if k_dt != torch.float32:
            return torch.from_numpy(a.view(np.int16)).view(k_dt).to(dev)
        return torch.from_numpy(a).to(dev)

    sets = []
    for i in range(nsets):
        d = d0
        if i:
            c = dict(cfg)
            c["seed"] = cfg["seed"] + 100 * i
            d = synth.make_kkt(c)
        kd, gd, bd = to_dev(d["k"]), torch.from_numpy(d["g"]).to(dev), to_dev(d["beta"])
        sets.append((kd, gd, bd, torch.empty((T, H, 64), dtype=x_dt, device=dev)))
    cu = torch.from_numpy(d0["cu_seqlens"]).to(dev)
    torch.cuda.synchronize()

    copy = CopyProbe(torch, stream, dev)
    if args.probe == "copy":
        return copy.only([s[1] for s in sets], args)

    calls = [kt.prepare_kkt(k, g, b, X, cu, solve=True) for k, g, b, X in sets]
    timer = Timer(torch, stream)
    el, k_avg, dist = timer.run(calls, args.steps, args.warmup)

    # the unfused pair on the same inputs: FP32 A written, then read back
    A32 = torch.empty((T, H, 64), dtype=torch.float32, device=dev)
    pairs = []
    for k, g, b, X in sets:
        build = kt.prepare_kkt(k, g, b, A32, cu, solve=False)
        solve = kt.prepare_packed(A32, X, cu, algo="fused")
        pairs.append(lambda build=build, solve=solve: (build(), solve()))
    _, pair_avg, _ = timer.run(pairs, max(10, args.steps // 4), min(args.warmup, 5))

    copy_gbs, copy_plain = copy.ceiling_gbs([s[1] for s in sets])
    flops = 10 * 2 * 16 * 16 * K * mats  # the ten 16 x 16 blocks of A, K-long products
    out = base_line(args, el, k_avg, dist, mats, bytes_alg, len(sets),
                    f"delta-rule 64x64 chunk inverses/sec with A built in-kernel from keys "
                    f"(K={K}) + achieved HBM GB/s (% peak)", None,
                    {"workload": describe(d0), "tokens": T, "heads": H, "key_dim": K,
                     "requests": len(d0["lengths"]), "matrices": mats,
                     "k_dtype": cfg["k_dtype"], "x_dtype": cfg["x_dtype"], "plan": "fused"},
                    f"{cfg['k_dtype']} k and beta, f32 g -> {cfg['x_dtype']} X")
    with_measured_hbm(out, load_traffic(args.workload))
    out["mfma_fp32"] = {"tflops": flops / k_avg / 1e12, "peak": MFMA_F32_PEAK_TFLOPS,
                        "frac": flops / k_avg / 1e12 / MFMA_F32_PEAK_TFLOPS}
    out["unfused_pair_us_avg"] = pair_avg * 1e6
    out["unfused_over_fused"] = pair_avg / k_avg
    out["copy_roofline_gbs"] = copy_gbs
    out["copy_plain_gbs"] = copy_plain
    out["cpu_baseline"] = None
    print(json.dumps(out), flush=True)
    return 0


def decode_algorithmic_bytes(B, H, d, W, in_bytes, out_bytes, padding=0) -> int:
    """One decode step: per non-padding (sequence, head) the d x d FP32 state
    and the three (W - 1) x d conv windows read and written, the new q, k, v,
    gate, decays, write strength read and the output written; per head the
    conv taps, and once the norm weights."""
    per = (2 * d * d * 4 + 2 * 3 * (W - 1) * d * 4 + 3 * d * in_bytes + d * in_bytes + d * 4 +
           4 + d * out_bytes)
    return (B - padding) * H * per + H * 3 * W * d * 4 + d * 4


def run_decode(args, torch, np, dev, stream):
    """The fused KDA decode core: one step for B sequences, rotating over
    several state pools (one per layer) so that the states come from HBM."""
    import synth
    import tril_solve_amd as kt

    cfg = synth.DECODE_CONFIGS[args.workload]
    B, H, d, W = cfg["B"], cfg["H"], cfg["d"], cfg["W"]
    ib, ob = dtype_bytes(cfg["in_dtype"]), dtype_bytes(cfg["out_dtype"])
    bytes_alg = decode_algorithmic_bytes(B, H, d, W, ib, ob)
    touched = B * H * d * d * 4  # state bytes one step touches
    nsets = args.sets or max(2, min(64, -(-(1 << 30) // touched)))
    x_dt = {"bf16": torch.bfloat16, "f16": torch.float16}.get(cfg["out_dtype"], torch.float32)
    in_dt = {"bf16": torch.bfloat16, "f16": torch.float16}.get(cfg["in_dtype"], torch.float32)

    def to_in(a):
        if in_dt != torch.float32:
            return torch.from_numpy(a.view(np.int16)).view(in_dt).to(dev)
        return torch.from_numpy(a).to(dev)

    sets = []
    for i in range(nsets):
        inp = synth.decode_inputs(B, H, d, W, cfg["slots"], cfg["seed"] + 1000 * i,
                                  cfg["in_dtype"])
        t = {k: torch.from_numpy(np.ascontiguousarray(inp[k])).to(dev)
             for k in ("g", "beta", "norm_w", "conv_w", "slot", "state", "conv_state")}
        t["qkv"], t["z"] = to_in(inp["qkv"]), to_in(inp["z"])
        t["out"] = torch.empty((B, H, d), dtype=x_dt, device=dev)
        sets.append(t)
    torch.cuda.synchronize()

    copy = CopyProbe(torch, stream, dev)
    if args.probe == "copy":
        return copy.only([t["state"] for t in sets], args)

    calls = [kt.prepare_decode(t["qkv"], t["z"], t["g"], t["beta"], t["norm_w"], t["conv_w"],
                               t["slot"], t["state"], t["conv_state"], t["out"]) for t in sets]
    el, k_avg, dist = Timer(torch, stream).run(calls, args.steps, args.warmup)
    copy_gbs, copy_plain = copy.ceiling_gbs([t["state"] for t in sets[:4]])

    def launch_all():  # one step per state pool, on the current stream
        for t in sets:
            kt.kda_decode_step(t["qkv"], t["z"], t["g"], t["beta"], t["norm_w"], t["conv_w"],
                               t["slot"], t["state"], t["conv_state"], t["out"])
    graph_avg, graph_median = graph_replay(torch, launch_all, len(sets))
    out = base_line(args, el, k_avg, dist, B, bytes_alg, len(sets),
                    "fused KDA decode core: sequences decoded per second through one layer "
                    "+ achieved HBM GB/s (% peak)", None,
                    {"workload": f"decode step, {B} sequences, {H} heads of dim {d}, conv width "
                                 f"{W}, {cfg['in_dtype']} activations -> {cfg['out_dtype']} "
                                 f"output, FP32 state pools of {cfg['slots']} slots",
                     "batch": B, "heads": H, "head_dim": d, "conv_width": W,
                     "in_dtype": cfg["in_dtype"], "out_dtype": cfg["out_dtype"]},
                    f"{cfg['in_dtype']} activations, f32 state -> {cfg['out_dtype']} output")
    out["unit"] = "sequences/s"
    with_measured_hbm(out, load_traffic(args.workload))
    # the same steps captured once in a HIP graph (one per pool) and replayed
    out["graph_replay_us_per_launch"] = {"avg": graph_avg, "median_of_replays": graph_median}
    out["pages_gfx950_fused_us_context"] = DECODE_PAGES_US.get(B)
    out["copy_roofline_gbs"] = copy_gbs
    out["copy_plain_gbs"] = copy_plain
    out["cpu_baseline"] = None
    print(json.dumps(out), flush=True)
    return 0


def main() -> int:
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--algo", default="auto", choices=["auto", "fused", "split", "fused_valu"])
    ap.add_argument("--workload", default=MAIN_WORKLOAD, choices=WORKLOADS,
                    help="the default is the metric's workload; the others are diagnostics")
    ap.add_argument("--sets", type=int, default=0,
                    help="rotating input/output buffer sets (default: enough for >= 1 GB)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--probe", choices=["copy", "sweep"], default=None,
                    help="copy: run only a plain copy of the input's byte count (counter "
                         "calibration); sweep: streaming copy / read / fill probes over the "
                         "input rotation at every unroll, cache policy and grid size (one JSON "
                         "line each, then the fastest per kind)")
    ap.add_argument("--record-traffic", nargs=5, default=None,
                    metavar=("FETCH_CSV", "WRITE_CSV", "COPY_FETCH_CSV", "COPY_WRITE_CSV", "OUT"),
                    help="write the HBM-traffic summary of --workload from rocprofv3 counter "
                         "CSVs (no GPU use)")
    ap.add_argument("--chunk-map", action="store_true",
                    help="packed solver workloads: pass a chunk map built once on the host "
                         "instead of letting the kernels scan cu_seqlens")
    ap.add_argument("--oracle-table", action="store_true",
                    help="time the CPU oracle on the five solver configurations, all host "
                         "threads and one (no GPU use)")
    args = ap.parse_args()

    if args.oracle_table:
        return oracle_table()
    if args.record_traffic:
        t = record_traffic(args.workload, args.record_traffic[:4], args.record_traffic[4])
        log(json.dumps(t))
        return 0

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) > 1:
        log("bench.py: this solver is measured on one GPU only (--gpus 1). Every chunk-head "
            "is independent, so a multi-GPU run would shard heads or chunks with no "
            "communication; that is not implemented.")
        return 2

    import numpy as np
    import torch

    dev = torch.device("cuda:0")
    stream = torch.cuda.current_stream()
    if args.workload in KKT_WORKLOADS or args.workload in DECODE_WORKLOADS:
        if args.algo not in ("auto", "fused"):
            log("bench.py: this workload has a single kernel (algo auto or fused)")
            return 2
        if args.workload in DECODE_WORKLOADS:
            return run_decode(args, torch, np, dev, stream)
        return run_kkt(args, torch, np, dev, stream)
    return run_solve(args, torch, np, dev, stream)


if __name__ == "__main__":
    sys.exit(main())
