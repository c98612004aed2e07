"""Benchmark of the RT-Lynx sparse + LoRA linear layer on one MI355X.

    python bench.py [--steps K] [--warmup W] [--workload mlp_up] [--no-cpu]

A step is one call of lynx_linear_sparse_lora (sparsify + 2:4 sparse-MFMA GEMM
with the LoRA epilogue) per layer of the workload on one batch of synthetic
input already resident in HBM.  The default workload is the DiT MLP
up-projection, X [4096 x 3072] -> Y [4096 x 12288], rank-64 LoRA; `block` is
the CFG-batched DiT block's four linears (M = 9216: QKV, attention-out, MLP-up,
MLP-down) in sequence.  Inputs rotate over three independent sets
(X, W, LA, LB, Y, workspace) so the working set (> 600 MB) exceeds the 256 MB
last-level cache.

First the sparse layer, the dense bf16 MFMA layer (lynx_linear_dense, the
speedup baseline), the sparsifier alone and the GEMM alone (split of the sparse
layer's time) and torch.matmul (hipBLASLt, a reference the library never calls)
take turns in rounds of --calls calls; each reports the median over --rounds
rounds, so all of them are timed under the same clock and power state.  Then
the headline: --warmup untimed steps and --steps timed steps, back to back,
while the clock is settled from that load; the same steps started after half a
second of idle are reported beside it (ms_per_step_after_idle).  The CPU oracle
is timed on a bounded sample on the host (cpu_baseline).  Prints ONE JSON line.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import re
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_DENSE_BF16_TFLOPS = 2516.6    # MI355X dense bf16 MFMA, AMD published
PEAK_SPARSE_BF16_TFLOPS = 5033.2   # 2:4 structured-sparse bf16 (dense-equivalent), AMD published
PEAK_HBM_GBS = 8000.0
METRIC = "dense-equiv TFLOP/s + % sparse-MFMA peak; speedup vs dense bf16 GEMM, M4096 K3072"


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=50)
    p.add_argument("--warmup", type=int, default=10)
    p.add_argument("--workload", default="mlp_up",
                   choices=["tiny", "qkv", "mlp_up", "mlp_down", "block"])
    p.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle baseline")
    p.add_argument("--sets", type=int, default=3)
    p.add_argument("--skip", default="",
                   help="block workload: comma-separated layer names (qkv, attn_out, mlp_up, "
                        "mlp_down) run as the dense layer (selective layer skipping)")
    p.add_argument("--rounds", type=int, default=7,
                   help="rounds of the interleaved comparison timing")
    p.add_argument("--calls", type=int, default=20,
                   help="calls per function and round in the comparison timing")
    p.add_argument("--copy-calibration", action="store_true",
                   help="after timing, run a plain 256 MiB streaming kernel (torch.neg) three "
                        "times, the reference for HBM byte counters")
    p.add_argument("--summarize-mfma", metavar="SQ_DIR",
                   help="write profiles/mfma_busy_<workload>.json from a rocprofv3 --pmc run of "
                        "SQ_VALU_MFMA_BUSY_CYCLES SQ_BUSY_CYCLES GRBM_GUI_ACTIVE and exit")
    p.add_argument("--mfma-peak", action="store_true",
                   help="measure the bf16 matrix-instruction issue rates and the clock under "
                        "that load (lynx_probe_mfma_rate, one wave per SIMD on every compute unit) "
                        "and exit")
    p.add_argument("--cpu-table", action="store_true",
                   help="CPU baseline per workload: the oracle on bounded row samples of every "
                        "workload, BLAS at one thread and at all cores, median of 3; print one "
                        "JSON line and exit (no GPU)")
    p.add_argument("--summarize-trace", metavar="TRACE_DIR",
                   help="no GPU: write profiles/trace_<workload>.md from a rocprofv3 --kernel-trace "
                        "run of this benchmark and exit")
    p.add_argument("--fusion-prototype", action="store_true",
                   help="time the fused-sparsifier GEMM prototype (tests/proto) against the "
                        "library's sparsifier + sparse GEMM pair on the MLP-up, MLP-down and QKV "
                        "shapes (interleaved, --rounds x --calls) and exit")
    p.add_argument("--sustained", type=float, metavar="SECONDS",
                   help="after 1 s of idle, run the workload's step back to back for SECONDS and "
                        "print the time per step over elapsed time, with the board power sampled "
                        "meanwhile (one JSON line) and exit")
    p.add_argument("--sustained-op", choices=("layer", "dense", "torch"), default="layer",
                   help="with --sustained: the sparse + LoRA layer (default), the library's dense "
                        "layer, or torch.matmul (hipBLASLt)")
    p.add_argument("--report", nargs="+", metavar="JSON",
                   help="no GPU: render the JSON lines of earlier runs of this benchmark (one or "
                        "more files) as one Markdown table and exit")
    p.add_argument("--summarize-traffic", nargs=2, metavar=("FETCH_DIR", "WRITE_DIR"),
                   help="no GPU: turn two rocprofv3 --pmc outputs (FETCH_SIZE, WRITE_SIZE) of a "
                        "--copy-calibration run into profiles/traffic_<workload>.json")
    return p.parse_args()


def time_region(fn, steps, warmup, stream):
    """Average ms per call of fn(i) over `steps` calls, HIP events on `stream`."""
    import torch
    for i in range(warmup):
        fn(i)
    torch.cuda.synchronize()
    start = torch.cuda.Event(enable_timing=True)
    end = torch.cuda.Event(enable_timing=True)
    start.record(stream)
    for i in range(steps):
        fn(i)
    end.record(stream)
    torch.cuda.synchronize()
    return start.elapsed_time(end) / steps


def time_interleaved(fns: dict, rounds: int, calls: int, stream) -> dict:
    """Median over `rounds` of the average ms per call of each fn, the fns
    taking turns (`calls` calls each per round) so that all of them run under
    the same clock and power state; HIP events on `stream`."""
    import statistics

    import torch
    per = {name: [] for name in fns}
    start = torch.cuda.Event(enable_timing=True)
    end = torch.cuda.Event(enable_timing=True)
    for _ in range(rounds):
        for name, fn in fns.items():
            torch.cuda.synchronize()
            start.record(stream)
            for i in range(calls):
                fn(i)
            end.record(stream)
            torch.cuda.synchronize()
            per[name].append(start.elapsed_time(end) / calls)
    def pct(v, q):  # nearest-rank percentile of the per-round averages
        v = sorted(v)
        return v[min(len(v) - 1, max(0, int(round(q * (len(v) - 1)))))]
    return {name: (statistics.median(v), pct(v, 0.1), pct(v, 0.9)) for name, v in per.items()}


SUSTAINED_MARKS_MS = (1, 2, 5, 10, 20, 50, 100, 200, 500, 1000, 2000, 5000, 10000, 20000, 60000)


class PowerSampler:
    """Samples the GPU's board power (hwmon power1_input, µW) and, where the
    driver exposes it, the current shader clock level (pp_dpm_sclk) on a
    background thread; reads nothing else and writes nothing."""

    def __init__(self, period_s: float = 0.02):
        import glob
        self.period = period_s
        hw = sorted(glob.glob("/sys/class/drm/card*/device/hwmon/hwmon*/power1_input"))
        self.power_path = hw[0] if hw else None
        cap = os.path.join(os.path.dirname(hw[0]), "power1_cap") if hw else None
        self.cap_w = self._read_w(cap) if cap and os.path.exists(cap) else None
        sclk = sorted(glob.glob("/sys/class/drm/card*/device/pp_dpm_sclk"))
        self.sclk_path = sclk[0] if sclk else None
        self.power, self.sclk, self._stop, self._thread = [], [], False, None

    @staticmethod
    def _read_w(path):
        try:
            with open(path) as f:
                return int(f.read().strip()) / 1e6
        except (OSError, ValueError):
            return None

    def _sclk_mhz(self):
        try:
            with open(self.sclk_path) as f:
                for line in f:
                    if line.rstrip().endswith("*"):
                        m = re.search(r"(\d+)\s*[Mm]hz", line)
                        return int(m.group(1)) if m else None
        except (OSError, TypeError):
            return None
        return None

    def _run(self):
        while not self._stop:
            if self.power_path:
                w = self._read_w(self.power_path)
                if w is not None:
                    self.power.append(w)
            if self.sclk_path:
                c = self._sclk_mhz()
                if c is not None:
                    self.sclk.append(c)
            time.sleep(self.period)

    def start(self):
        import threading
        self._thread = threading.Thread(target=self._run, daemon=True)
        self._thread.start()

    def stop(self) -> dict:
        self._stop = True
        if self._thread:
            self._thread.join()

        def summ(v, nd):
            if not v:
                return None
            v = sorted(v)
            return {"mean": round(sum(v) / len(v), nd), "p10": round(v[len(v) // 10], nd),
                    "p90": round(v[(9 * len(v)) // 10], nd), "samples": len(v)}
        return {"power_w": summ(self.power, 1), "power_cap_w": self.cap_w,
                "sclk_mhz": summ(self.sclk, 0)}


def sustained(step, seconds: float, stream, chunk: int = 10, idle_s: float = 1.0) -> dict:
    """Time per step over `seconds` of back-to-back steps that start after
    `idle_s` of idle: one value per chunk of `chunk` steps (HIP events on
    `stream`), reported at log-spaced elapsed times, and the mean of the run;
    the board power over the second half of the run (PowerSampler)."""
    import torch
    torch.cuda.synchronize()
    time.sleep(idle_s)
    sampler, sampling = PowerSampler(), False
    series, elapsed, i, nxt = [], 0.0, 0, 0
    while elapsed < seconds * 1e3:
        if not sampling and elapsed >= seconds * 500:   # the settled second half
            sampler.start()
            sampling = True
        evs = [torch.cuda.Event(enable_timing=True) for _ in range(21)]
        evs[0].record(stream)
        for b in range(20):
            for _ in range(chunk):
                step(i)
                i += 1
            evs[b + 1].record(stream)
        torch.cuda.synchronize()
        for b in range(20):
            per = evs[b].elapsed_time(evs[b + 1]) / chunk
            elapsed += per * chunk
            while nxt < len(SUSTAINED_MARKS_MS) and elapsed >= SUSTAINED_MARKS_MS[nxt]:
                series.append({"elapsed_ms": round(elapsed, 1), "us_per_step": round(per * 1e3, 1)})
                nxt += 1
    power = sampler.stop() if sampling else None
    return {"steps": i, "seconds": round(elapsed / 1e3, 3), "idle_s_before": idle_s,
            "chunk_steps": chunk, "mean_us_per_step": round(elapsed / i * 1e3, 2), "series": series,
            "second_half": power}


def cpu_model() -> str:
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:  # pragma: no cover
        pass
    return "unknown"


def cpu_baseline(L, min_s=10.0, max_rows_growth=8.0, one_thread_s=6.0):
    """The fp64 oracle, as it stands, on a bounded sample of the same workload.

    The row count grows until one call takes about four seconds or covers the
    whole layer; calls at that size then repeat until min_s seconds of CPU work
    have been timed.  Each call includes the oracle's own decode of W, LA, LB.
    The same is then repeated with the BLAS pool limited to one thread (about
    one_thread_s seconds), reported beside it."""
    from oracle import lynx_oracle as orc
    try:
        import threadpoolctl
        info = threadpoolctl.threadpool_info()
        cores = max((i.get("num_threads", 1) for i in info), default=os.cpu_count())
        blas = ", ".join(sorted({f"{i.get('internal_api', '?')} {i.get('version', '')}".strip()
                                 for i in info if i.get("user_api") == "blas"})) or "unknown"
    except Exception:  # pragma: no cover
        threadpoolctl, cores, blas = None, os.cpu_count(), "unknown"

    def run(rows):
        t0 = time.perf_counter()
        orc.linear_sparse_lora(L.X[:rows], L.W, L.LA, L.LB)
        return time.perf_counter() - t0

    def measure(target_call_s, budget_s):
        rows = min(L.M, 16)
        dt = run(rows)
        while dt < target_call_s and rows < L.M:
            rows = min(L.M, int(rows * min(max_rows_growth, max(2.0, target_call_s / max(dt, 1e-3)))))
            dt = run(rows)
        total, calls = 0.0, 0
        while total < budget_s:
            total += run(rows)
            calls += 1
        flops = calls * (2 * rows * L.N * L.K + 2 * rows * L.R * (L.K + L.N))
        return flops / total / 1e12, total, calls, rows

    value, total, calls, rows = measure(4.0, min_s)
    rec = {"value": round(value, 6), "unit": "TFLOP/s (dense-equivalent)",
           "cores": cores, "kind": "oracle", "seconds": round(total, 2),
           "sample": f"{calls} call(s) on the first {rows} of {L.M} rows of the {L.name} layer "
                     f"(full W, LA, LB): fp64 NumPy oracle with selection, norms and both "
                     f"contractions",
           "cpu_model": cpu_model(), "os_cpu_count": os.cpu_count(), "blas": blas}
    if threadpoolctl is not None:
        with threadpoolctl.threadpool_limits(1):
            v1, t1, c1, r1 = measure(2.0, one_thread_s)
        rec["one_thread"] = {"value": round(v1, 6), "seconds": round(t1, 2),
                             "sample": f"{c1} call(s) on the first {r1} rows, BLAS limited to 1 thread"}
    return rec


def cpu_table(target_s=0.5, repeats=3) -> dict:
    """The oracle (as it stands) on every workload, once with BLAS limited to
    one thread and once with all cores.  A call costs a fixed part (decoding
    the layer's W, LA, LB) plus a part linear in the rows of X (the layer is
    row-independent), so each layer is timed on r and 2 r rows (median of
    `repeats` calls each, r sized so the row part of a call is about
    target_s) and the whole layer's time is fixed + M x per-row."""
    import statistics

    import threadpoolctl

    from oracle import lynx_oracle as orc
    from workloads import CONFIGS, make_config
    info = threadpoolctl.threadpool_info()
    blas = ", ".join(sorted({f"{i.get('internal_api', '?')} {i.get('version', '')}".strip()
                             for i in info if i.get("user_api") == "blas"})) or "unknown"
    all_threads = max((i.get("num_threads", 1) for i in info), default=os.cpu_count())
    out = {"cpu_model": cpu_model(), "os_cpu_count": os.cpu_count(), "blas": blas,
           "threads_all": all_threads, "repeats": repeats, "workloads": {}}

    def call(L, rows):
        t0 = time.perf_counter()
        orc.linear_sparse_lora(L.X[:rows], L.W, L.LA, L.LB)
        return time.perf_counter() - t0

    for name in CONFIGS:
        layers = make_config(name)
        flops = sum(L.dense_equiv_flops for L in layers)
        rec = {"layers": [f"{L.M}x{L.K}->{L.N}" for L in layers],
               "dense_equiv_gflop": round(flops / 1e9, 2)}
        for label, limit in (("one_thread", 1), ("all_cores", all_threads)):
            with threadpoolctl.threadpool_limits(limit):
                total_s, sample = 0.0, []
                for L in layers:
                    r0 = min(64, max(1, L.M // 2))
                    t1, t2 = call(L, r0), call(L, 2 * r0)
                    per_row = max((t2 - t1) / r0, 1e-9)
                    r = int(min(L.M // 2, max(r0, target_s / per_row)))
                    a = statistics.median(call(L, r) for _ in range(repeats))
                    b = statistics.median(call(L, 2 * r) for _ in range(repeats))
                    per_row = max((b - a) / r, 0.0)
                    fixed = max(a - r * per_row, 0.0)
                    total_s += fixed + L.M * per_row
                    sample.append(f"{r} and {2 * r} of {L.M} rows")
            rec[label] = {"seconds_whole_workload": round(total_s, 3),
                          "tflops": round(flops / total_s / 1e12, 5), "threads": limit,
                          "sample": "; ".join(sample)}
            print(f"cpu table: {name} {label}: {total_s:.2f} s", file=sys.stderr, flush=True)
        out["workloads"][name] = rec
    return out


CSRC = os.path.join(ROOT, "activation_sparse_gemm_amd", "csrc")
# the source files each profiled kernel is built from (its .hip and the
# internal headers it includes): a counter record is used only while their
# hash matches the one it was taken on
KERNEL_SOURCES = {
    "gemm_sparse32": ("k_gemm.hip", "lynx_tile.h", "lynx_dma.h", "lynx_internal.h"),
    "gemm_dense32": ("k_gemm_dense.hip", "lynx_tile.h", "lynx_dma.h", "lynx_internal.h"),
    "sparsify_kernel": ("k_sparsify.hip", "lynx_internal.h"),
}
COPY_MIB = 256
IDLE_S = 0.5   # idle before the from-idle repeat of the headline steps


def source_sha(kernel: str) -> str:
    """Hash of the sources `kernel` is built from (None for a library kernel)."""
    files = KERNEL_SOURCES.get(kernel)
    if files is None:
        return None
    h = hashlib.sha256()
    for name in files:
        with open(os.path.join(CSRC, name), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def per_dispatch_kib(run_dir: str, counter: str) -> dict:
    """Mean value of `counter` per dispatch, by kernel name, from rocprofv3
    output under run_dir (rocpd SQLite database or counter_collection.csv)."""
    import csv
    import glob
    import sqlite3
    vals = {}
    for path in glob.glob(os.path.join(run_dir, "**", "*_results.db"), recursive=True):
        con = sqlite3.connect(path)
        for name, value in con.execute(
                "select kernel_name, value from counters_collection where counter_name = ?",
                (counter,)):
            vals.setdefault(name, []).append(float(value))
        con.close()
    for path in glob.glob(os.path.join(run_dir, "**", "*counter_collection.csv"), recursive=True):
        with open(path) as f:
            for row in csv.DictReader(f):
                if row.get("Counter_Name") == counter:
                    vals.setdefault(row["Kernel_Name"], []).append(float(row["Counter_Value"]))
    return {k: sum(v) / len(v) for k, v in vals.items()}


def summarize_traffic(fetch_dir: str, write_dir: str, workload: str) -> dict:
    """HBM bytes per K2 launch: FETCH_SIZE and WRITE_SIZE (KiB per dispatch),
    each scaled by what the same counter reads for the plain streaming kernel
    of known size (reads COPY_MIB MiB, writes COPY_MIB MiB)."""
    fetch = per_dispatch_kib(fetch_dir, "FETCH_SIZE")
    write = per_dispatch_kib(write_dir, "WRITE_SIZE")

    def pick(d, key):
        hits = [k for k in d if key in k]
        if len(hits) != 1:
            raise SystemExit(f"expected one kernel matching {key!r}, found {hits}")
        return d[hits[0]]

    def mean_over(d, key):
        # mean per dispatch over every instantiation matching key (each layer
        # of a workload is launched once per step)
        hits = [k for k in d if key in k]
        if not hits:
            raise SystemExit(f"no kernel matching {key!r}")
        return sum(d[k] for k in hits) / len(hits)

    from workloads import CONFIGS
    per_step = len(CONFIGS[workload]) if workload in CONFIGS else 1
    known_kib = COPY_MIB * 1024.0
    f_factor = known_kib / pick(fetch, "neg")
    w_factor = known_kib / pick(write, "neg")
    f_bytes = mean_over(fetch, "gemm_sparse32") * 1024.0 * f_factor * per_step
    w_bytes = mean_over(write, "gemm_sparse32") * 1024.0 * w_factor * per_step
    rec = {"workload": workload, "kernel": "gemm_sparse32", "kernel_sha": source_sha("gemm_sparse32"),
           "launches_per_step": per_step,
           "fetch_bytes_per_launch": round(f_bytes / per_step),
           "write_bytes_per_launch": round(w_bytes / per_step),
           "bytes_per_launch": round((f_bytes + w_bytes) / per_step),
           "bytes_per_step": round(f_bytes + w_bytes),
           "copy_factor_fetch": round(f_factor, 4), "copy_factor_write": round(w_factor, 4),
           "commands": [f"rocprofv3 --pmc {c} -d <dir> -o run -- python3 bench.py --steps 3 "
                        f"--warmup 1 --no-cpu --sets 1 --copy-calibration --workload {workload}"
                        for c in ("FETCH_SIZE", "WRITE_SIZE")],
           "raw_kib_per_dispatch": {"fetch": {k[:60]: round(v, 1) for k, v in fetch.items()},
                                    "write": {k[:60]: round(v, 1) for k, v in write.items()}}}
    out = os.path.join(ROOT, "profiles", f"traffic_{workload}.json")
    with open(out, "w") as f:
        json.dump(rec, f, indent=1)
    return rec


# shader engines and SIMDs of the MI355X (8 XCDs x 4 SEs, 256 CUs x 4 SIMDs):
# SQ_BUSY_CYCLES is summed over the shader engines, SQ_VALU_MFMA_BUSY_CYCLES
# over every SIMD's matrix core
N_SE, N_SIMD = 32, 1024


def summarize_mfma(sq_dir: str, workload: str) -> dict:
    """Matrix-core busy fraction per kernel: SQ_VALU_MFMA_BUSY_CYCLES over
    (kernel cycles x SIMDs), the kernel cycles being SQ_BUSY_CYCLES per shader
    engine (means per dispatch)."""
    busy = per_dispatch_kib(sq_dir, "SQ_VALU_MFMA_BUSY_CYCLES")
    sq = per_dispatch_kib(sq_dir, "SQ_BUSY_CYCLES")
    grbm = per_dispatch_kib(sq_dir, "GRBM_GUI_ACTIVE")
    kernels = {}
    for name, b in busy.items():
        if b <= 0 or name not in sq:
            continue
        cycles = sq[name] / N_SE
        base = next((k for k in KERNEL_SOURCES if k in name), None)
        inst = re.search(r"(gemm_sparse32|gemm_dense32|sparsify_kernel)<[^>]*>", name)
        key = (inst.group(0).replace(" ", "") if inst is not None else base if base is not None else
               "torch.matmul (hipBLASLt " + name[:48] + ")" if "Cijk" in name else name[:60])
        kernels[key] = {"mfma_busy_cycles": round(b), "sq_busy_cycles": round(sq[name]),
                        "grbm_gui_active": round(grbm.get(name, 0.0)),
                        "kernel_cycles": round(cycles),
                        "mfma_busy": round(b / (cycles * N_SIMD), 4),
                        "source_sha": source_sha(base) if base is not None else None}
    rec = {"workload": workload, "kernels": kernels,
           "command": "rocprofv3 --pmc SQ_VALU_MFMA_BUSY_CYCLES SQ_BUSY_CYCLES GRBM_GUI_ACTIVE "
                      f"-d <dir> -o run -- python3 bench.py --steps 3 --warmup 1 --no-cpu --sets 1 "
                      f"--rounds 1 --calls 3 --workload {workload}"}
    out = os.path.join(ROOT, "profiles", f"mfma_busy_{workload}.json")
    with open(out, "w") as f:
        json.dump(rec, f, indent=1)
    return rec


TRACE_CALLS = ("over every call bench.py makes: the interleaved rounds of the sparse layer, the "
               "dense layer, the GEMM alone, the sparsifier alone and torch.matmul (hipBLASLt), "
               "then the consecutive timed steps, then the same steps after half a second of idle.")
FUSION_CALLS = ("over every call bench.py --fusion-prototype makes: per shape (MLP-up, "
                "MLP-down, QKV), interleaved rounds of the library's layer (sparsifier + "
                "sparse GEMM with the rank-64 LoRA), the sparsifier alone, the sparse GEMM alone "
                "and the fused prototype (gemm_fused32: selection inside the GEMM's operand "
                "load, no LoRA).")


def summarize_trace(trace_dir: str, workload: str, command: str, calls: str = TRACE_CALLS,
                    out_name: str | None = None, timeline: int = 0) -> str:
    """Per-kernel dispatch times (µs) and resources from a rocprofv3
    --kernel-trace results database, as profiles/trace_<out_name or workload>.md."""
    import collections
    import glob
    import sqlite3
    dbs = glob.glob(os.path.join(trace_dir, "**", "*_results.db"), recursive=True)
    if len(dbs) != 1:
        raise SystemExit(f"expected one results database under {trace_dir}, found {dbs}")
    con = sqlite3.connect(dbs[0])
    syms = {}
    for kid, dem, kn, av, acv, sg, lds in con.execute(
            "select id, demangled_kernel_name, kernel_name, arch_vgpr_count, accum_vgpr_count, "
            "sgpr_count, group_segment_size from kernel_symbols"):
        name = (dem or kn).replace("lynx::(anonymous namespace)::", "")
        name = name[5:] if name.startswith("void ") else name
        if not name.startswith("at::") and "(" in name:
            name = name[:name.index("(")]
        syms[kid] = (re.sub(r"\.kd$", "", name)[:70], av, acv, sg, lds)
    times, wgs = collections.defaultdict(list), {}
    order = []
    for kid, t0, t1, gx, wx in con.execute(
            "select kernel_id, start, end, grid_size_x, workgroup_size_x from rocpd_kernel_dispatch "
            "order by start"):
        times[kid].append((t1 - t0) / 1000.0)
        wgs[kid] = gx // wx
        order.append((kid, (t1 - t0) / 1000.0))
    con.close()
    total = sum(sum(v) for v in times.values())
    title = f"{workload} workload, bench.py" if out_name is None else out_name.replace("_", " ")
    lines = [f"# Kernel trace: {title}", "",
             "Command (on one MI355X, from the repository root, with `TMPDIR=/tmp`):", "", "```",
             command, "```", "",
             "Durations are per dispatch under the profiler (µs), from the run's results database, "
             + calls, "",
             "| kernel | calls | avg µs | median µs | total µs | % of GPU time |",
             "|---|---|---|---|---|---|"]
    for kid, v in sorted(times.items(), key=lambda kv: -sum(kv[1])):
        med = sorted(v)[len(v) // 2]
        lines.append(f"| `{syms[kid][0]}` | {len(v)} | {sum(v) / len(v):.1f} | {med:.1f} | "
                     f"{sum(v):.0f} | {100 * sum(v) / total:.1f} |")
    lines += ["", "Per-kernel dispatch statistics (µs) and resources:", "",
              "| kernel | n | avg | min | max | arch VGPR | acc VGPR | SGPR | LDS B | workgroups |",
              "|---|---|---|---|---|---|---|---|---|---|"]
    for kid, v in sorted(times.items(), key=lambda kv: syms[kv[0]][0]):
        n, av, acv, sg, lds = syms[kid]
        lines.append(f"| `{n}` | {len(v)} | {sum(v) / len(v):.1f} | {min(v):.1f} | {max(v):.1f} | "
                     f"{av} | {acv} | {sg} | {lds} | {wgs[kid]} |")
    if timeline:
        # from the sparsifier launch before the first sparse GEMM (the first
        # step; bench.py's set-up calls only the sparsifier before it)
        first = next((i for i, (kid, _) in enumerate(order) if "gemm_sparse32" in syms[kid][0]), 1)
        first = max(first - 1, 0)
        lines += ["", f"{timeline} dispatches in time order from the first step (µs):", "",
                  "| # | kernel | µs |", "|---|---|---|"]
        lines += [f"| {i} | `{syms[kid][0]}` | {d:.1f} |"
                  for i, (kid, d) in enumerate(order[first:first + timeline], start=first)]
    text = "\n".join(lines) + "\n"
    with open(os.path.join(ROOT, "profiles", f"trace_{out_name or workload}.md"), "w") as f:
        f.write(text)
    return text


def mfma_busy_for(workload: str):
    """Matrix-core busy fractions from the committed counter summary, for the
    kernels whose sources are unchanged since it was taken (library kernels
    always); None if there is no summary or nothing in it is current."""
    path = os.path.join(ROOT, "profiles", f"mfma_busy_{workload}.json")
    if not os.path.exists(path):
        return None
    rec = json.load(open(path))
    out = {}
    for k, v in rec.get("kernels", {}).items():
        base = next((b for b in KERNEL_SOURCES if k.startswith(b)), None)
        if base is None or v.get("source_sha") == source_sha(base):
            out[k] = v["mfma_busy"]
    return out or None


def traffic_for(workload: str):
    """HBM bytes per K2 launch from the committed rocprofv3 counter summary,
    if it was taken on the current sources; else None."""
    path = os.path.join(ROOT, "profiles", f"traffic_{workload}.json")
    if not os.path.exists(path):
        return None
    rec = json.load(open(path))
    ok = rec.get("kernel_sha") == source_sha("gemm_sparse32")
    return rec.get("bytes_per_step", rec.get("bytes_per_launch")) if ok else None


def mfma_peak() -> dict:
    """Measured peak of each bf16 matrix instruction the kernels use: every
    compute unit runs 4 waves (one per SIMD) of back-to-back instructions.
    Reports cycles per instruction and the shader clock from the waves' own
    counters, and the chip-wide dense-equivalent TFLOP/s from HIP events."""
    import numpy as np
    import torch

    from activation_sparse_gemm_amd import _abi
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    out = {"cus": cus, "simds": 4 * cus, "instructions": {}}
    for which, name in enumerate(_abi.PROBE_NAMES):
        iters = 4096 if which in (0, 2) else 2048
        _abi.probe_mfma_rate(which, 64, cus)          # warm-up
        runs = [_abi.probe_mfma_rate(which, iters, cus) for _ in range(5)]
        ms = float(np.median([r["ms"] for r in runs]))
        st = np.concatenate([r["stamps"] for r in runs]).astype(np.float64)
        cpi = float(np.median(st[:, 0])) / (16 * iters)
        mhz = float(np.median(100.0 * st[:, 0] / np.maximum(st[:, 1], 1)))
        n_instr = 4 * cus * 16 * iters
        tf = n_instr * _abi.PROBE_FLOPS[which] / (ms * 1e-3) / 1e12
        out["instructions"][name] = {
            "cycles_per_instruction": round(cpi, 2), "clock_mhz": round(mhz, 1),
            "tflops_dense_equiv": round(tf, 1),
            "tflops_at_2400mhz": round(4 * cus * _abi.PROBE_FLOPS[which] / cpi * 2.4e9 / 1e12, 1),
            "ms": round(ms, 4), "iters": iters}
    return out


def fusion_prototype(rounds: int, calls: int, nsets: int) -> dict:
    """The fused-sparsifier GEMM prototype against the library's pair: per
    shape, the layer (sparsifier + sparse GEMM, rank-64 LoRA), each of its two
    kernels alone and the prototype (no LoRA) take turns; medians in ms."""
    import numpy as np
    import torch

    import activation_sparse_gemm_amd as lynx
    from tests.proto import fused_proto
    from workloads import make_config, make_layer

    dev = torch.device("cuda:0")
    stream = torch.cuda.current_stream(dev)

    def to_dev(b):
        return torch.from_numpy(np.ascontiguousarray(b).view(np.int16)).view(torch.bfloat16).to(dev)

    out = {}
    for wl in ("mlp_up", "mlp_down", "qkv"):
        base = make_config(wl)[0]
        sets = []
        for s in range(nsets):
            L = base if s == 0 else make_layer(base.M, base.K, base.N, base.kind,
                                               seed=100 + 10 * s, R=base.R, name=base.name)
            d = dict(X=to_dev(L.X), W=to_dev(L.W), LA=to_dev(L.LA), LB=to_dev(L.LB))
            d["Y"] = torch.empty((L.M, L.N), dtype=torch.bfloat16, device=dev)
            d["ws"] = torch.empty(lynx.workspace_bytes(L.M, L.K, L.R), dtype=torch.uint8,
                                  device=dev)
            d["packed"] = lynx.sparsify(d["X"], d["LB"])
            sets.append(d)
        S = len(sets)

        def layer(i):
            d = sets[i % S]
            lynx.linear_sparse_lora(d["X"], d["W"], d["LA"], d["LB"], Y=d["Y"], workspace=d["ws"])

        def sparsify(i):
            d = sets[i % S]
            v, m, sc, T = d["packed"]
            lynx.sparsify(d["X"], d["LB"], out=dict(values=v, meta=m, scale=sc, T=T))

        def gemm(i):
            d = sets[i % S]
            v, m, sc, T = d["packed"]
            lynx.linear_sparse_lora_packed(v, m, sc, T, d["W"], d["LA"], Y=d["Y"])

        def fused(i):
            d = sets[i % S]
            fused_proto.gemm_fused(d["X"], d["W"], Y=d["Y"])

        fns = {"layer": layer, "sparsify": sparsify, "gemm": gemm, "fused": fused}
        for fn in fns.values():
            fn(0)
        torch.cuda.synchronize()
        med = time_interleaved(fns, rounds=rounds, calls=calls, stream=stream)
        rec = {k: round(v[0], 5) for k, v in med.items()}
        rec["fused_over_layer"] = round(med["fused"][0] / med["layer"][0], 3)
        rec["fused_over_gemm"] = round(med["fused"][0] / med["gemm"][0], 3)
        rec["shape"] = {"M": base.M, "K": base.K, "N": base.N, "R": base.R}
        out[wl] = rec
        print(f"fusion prototype {wl}: {rec}", file=sys.stderr, flush=True)
        del sets
        torch.cuda.synchronize()
    return {"ms": out, "rounds": rounds, "calls": calls, "sets": nsets}


REPORT_COLUMNS = (
    ("workload", None), ("TFLOP/s (steps)", None), ("ms/step", None), ("ms/step after idle", None),
    ("sparse layer µs", None), ("dense (K3) µs", None), ("hipBLASLt µs", None),
    ("vs K3", None), ("vs hipBLASLt", None), ("vs best dense", None),
    ("K1 µs", None), ("K2 µs", None), ("K2 roofline", None), ("K2 MFMA busy", None),
    ("K1 HBM frac", None), ("CPU oracle TFLOP/s", None))


REPORT_HEAD = """# Benchmark report: RT-Lynx sparse + LoRA linear on one MI355X

Rendered by `python bench.py --report` from the JSON lines that `python bench.py` (MLP-up, with the CPU
baseline) and `python bench.py --workload W --steps 30 --warmup 5 --no-cpu` (the other workloads) printed:
{files}.
"""

REPORT_LEGEND = """Columns:
- **TFLOP/s (steps), ms/step**: the benchmark's `value` and `ms_per_step`, dense-equivalent flops
  (2·M·N·K plus the LoRA flops) over consecutive steps at the settled clock; **after idle**: the same steps
  started after half a second of idle (the clock's transient).
- **sparse layer, dense (K3), hipBLASLt**: interleaved medians of the sparse + LoRA layer, the library's dense
  bf16 layer and `torch.matmul`.
- **vs K3, vs hipBLASLt, vs best dense**: their ratios to the sparse layer; the last is against the faster of
  the two dense layers.
- **K1, K2**: the sparsifier and the sparse GEMM with its LoRA epilogue, timed on their own.
- **K2 roofline**: K2's flops per second over the dense bf16 peak ({peak_mfma} TFLOP/s).
- **K2 MFMA busy**: matrix-core busy fraction from the committed rocprofv3 counters (a dash where none were
  taken).
- **K1 HBM frac**: K1's algorithmic bytes per second over {peak_hbm:.0f} GB/s.
- **CPU oracle**: the fp64 oracle on the host cores, on a bounded sample.
"""


def render_report(records: list) -> str:
    """One Markdown table row per benchmark record (the JSON line main() prints)."""
    def us(ms):
        return "—" if ms is None else f"{ms * 1e3:.1f}"

    def x(v):
        return "—" if v is None else f"{v:.2f}×"

    lines = ["| " + " | ".join(c for c, _ in REPORT_COLUMNS) + " |",
             "|" + "---|" * len(REPORT_COLUMNS)]
    for r in records:
        inter, split = r.get("interleaved_ms", {}), r.get("split_ms", {})
        busy = r.get("mfma_busy") or {}
        k2_busy = next((v for k, v in busy.items() if k.startswith("gemm_sparse32")), None)
        cpu = r.get("cpu_baseline")
        roof, k1roof = r.get("roofline") or {}, r.get("sparsify_roofline") or {}
        idle = r.get("ms_per_step_after_idle")
        cells = [r["config"]["workload"].split(":")[0], f"{r['value']:.0f}", f"{r['ms_per_step']:.4f}",
                 "—" if idle is None else f"{idle:.4f}",
                 us(inter.get("sparse_layer")), us(inter.get("dense_layer")), us(inter.get("torch_matmul")),
                 x(r.get("speedup_vs_dense")), x(r.get("speedup_vs_torch_matmul")),
                 x(r.get("speedup_vs_best_dense")), us(split.get("sparsify")),
                 us(split.get("sparse_gemm_lora")),
                 "—" if roof.get("frac") is None else f"{roof['frac']:.3f}",
                 "—" if k2_busy is None else f"{k2_busy:.2f}",
                 "—" if k1roof.get("frac") is None else f"{k1roof['frac']:.3f}",
                 "—" if cpu is None else f"{cpu['value']:.3f} ({cpu['cores']} threads)"]
        lines.append("| " + " | ".join(cells) + " |")
    return "\n".join(lines) + "\n"


def read_records(paths: list) -> list:
    """The last JSON line with a "metric" key of each file."""
    out = []
    for path in paths:
        with open(path) as f:
            recs = [json.loads(t) for t in f.read().splitlines() if t.startswith("{")]
        recs = [r for r in recs if "metric" in r]
        if not recs:
            raise SystemExit(f"{path}: no benchmark record")
        out.append(recs[-1])
    return out


def main():
    args = parse()
    if args.report:
        print(REPORT_HEAD.format(files=", ".join(f"`{os.path.basename(f)}`" for f in args.report)))
        print(render_report(read_records(args.report)))
        print(REPORT_LEGEND.format(peak_mfma=PEAK_DENSE_BF16_TFLOPS, peak_hbm=PEAK_HBM_GBS), end="")
        return
    if args.mfma_peak:
        print(json.dumps(mfma_peak()))
        return
    if args.summarize_mfma:
        print(json.dumps(summarize_mfma(args.summarize_mfma, args.workload)))
        return
    if args.summarize_traffic:
        print(json.dumps(summarize_traffic(*args.summarize_traffic, args.workload)))
        return
    if args.cpu_table:
        print(json.dumps(cpu_table()))
        return
    if args.fusion_prototype:
        if args.summarize_trace:
            cmd = (f"rocprofv3 --kernel-trace --stats -d <dir> -o run -- python3 bench.py "
                   f"--fusion-prototype --rounds {args.rounds} --calls {args.calls}")
            print(summarize_trace(args.summarize_trace, "fusion", cmd, FUSION_CALLS,
                                  out_name="fusion_prototype"))
            return
        print(json.dumps(fusion_prototype(args.rounds, args.calls, args.sets)))
        return
    if args.summarize_trace:
        cmd = (f"rocprofv3 --kernel-trace --stats -d <dir> -o run -- python3 bench.py "
               f"--workload {args.workload} --steps {args.steps} --warmup {args.warmup} --no-cpu")
        print(summarize_trace(args.summarize_trace, args.workload, cmd))
        return
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only; --gpus {args.gpus} is not supported "
              f"(the layer shards by rows with no communication; see the design notes)",
              file=sys.stderr)
        sys.exit(2)
    import numpy as np
    import torch

    import activation_sparse_gemm_amd as lynx
    from workloads import BLOCK_LAYER_NAMES, make_config, make_layer

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    dev = torch.device("cuda:0")
    layers = make_config(args.workload)   # one layer, or the block's four in sequence
    skip = [x for x in args.skip.split(",") if x]
    if skip and args.workload != "block":
        sys.exit("--skip applies to the block workload")
    unknown = set(skip) - set(BLOCK_LAYER_NAMES)
    if unknown:
        sys.exit(f"--skip: unknown layers {sorted(unknown)}")
    skipped = [len(layers) > 1 and BLOCK_LAYER_NAMES[j] in skip for j in range(len(layers))]

    def to_dev(b):
        return torch.from_numpy(np.ascontiguousarray(b).view(np.int16)).view(torch.bfloat16).to(dev)

    # sets[s][j]: device tensors of layer j in input set s (set 0 = the seeded
    # workload itself, the others independent draws of the same shapes)
    sets, seq_workspaces = [], []
    for s in range(args.sets):
        row = []
        for j, base in enumerate(layers):
            L = base if s == 0 else make_layer(base.M, base.K, base.N, base.kind,
                                               seed=100 + 10 * s + j, R=base.R, name=base.name)
            X, W, LA, LB = to_dev(L.X), to_dev(L.W), to_dev(L.LA), to_dev(L.LB)
            M, K, N, R = L.M, L.K, L.N, L.R
            ws = torch.empty(lynx.workspace_bytes(M, K, R), dtype=torch.uint8, device=dev)
            Y = torch.empty((M, N), dtype=torch.bfloat16, device=dev)
            Yd = torch.empty((M, N), dtype=torch.bfloat16, device=dev)
            packed = lynx.sparsify(X, LB)
            row.append(dict(X=X, W=W, LA=LA, LB=LB, ws=ws, Y=Y, Yd=Yd, packed=packed,
                            dense=skipped[j]))
        seq_ws = torch.empty((max(lynx.sequence_workspace_bytes(row), 1),), dtype=torch.uint8,
                             device=dev)
        sets.append(row)
        seq_workspaces.append(seq_ws)
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream(dev)
    S = len(sets)

    def step(i):
        if len(layers) > 1:   # the block: one lynx_linear_sequence call
            lynx.linear_sequence(sets[i % S], workspace=seq_workspaces[i % S])
            return
        for d in sets[i % S]:
            lynx.linear_sparse_lora(d["X"], d["W"], d["LA"], d["LB"], Y=d["Y"],
                                    workspace=d["ws"])

    def dense(i):
        for d in sets[i % S]:
            lynx.linear_dense(d["X"], d["W"], Y=d["Yd"])

    def gemm_only(i):
        for d in sets[i % S]:
            if d["dense"]:
                continue
            v, m, sc, T = d["packed"]
            lynx.linear_sparse_lora_packed(v, m, sc, T, d["W"], d["LA"], Y=d["Y"])

    def sparsify_only(i):
        for d in sets[i % S]:
            if d["dense"]:
                continue
            v, m, sc, T = d["packed"]
            lynx.sparsify(d["X"], d["LB"], out=dict(values=v, meta=m, scale=sc, T=T))

    def torch_mm(i):
        for d in sets[i % S]:
            torch.matmul(d["X"], d["W"].t(), out=d["Yd"])

    torch.cuda.synchronize()
    if args.sustained:
        fn = {"layer": step, "dense": dense, "torch": torch_mm}[args.sustained_op]
        print(json.dumps(dict(sustained(fn, args.sustained, stream), workload=args.workload,
                              op=args.sustained_op)))
        return
    # comparisons: the sparse layer, the dense layer, the split of the sparse
    # layer and hipBLASLt take turns, so each sees the same clock and power
    # state
    med = time_interleaved({"sparse": step, "dense": dense, "gemm": gemm_only,
                            "sparsify": sparsify_only, "torch": torch_mm},
                           rounds=args.rounds, calls=args.calls, stream=stream)
    # the headline: K consecutive steps after W warm-up steps, right after the
    # comparisons.  Coming out of idle (input set-up), the first ~20 ms of
    # back-to-back steps run through a power-management transient, up to 25%
    # slower than the rate the chip then holds for seconds (--sustained); after
    # the comparisons' GPU load the clock has settled.  The same W + K steps
    # started after IDLE_S of idle are reported beside it.
    ms = time_region(step, args.steps, args.warmup, stream)
    torch.cuda.synchronize()
    time.sleep(IDLE_S)
    ms_idle = time_region(step, args.steps, args.warmup, stream)
    ms_sparse_i, ms_dense = med["sparse"][0], med["dense"][0]
    ms_gemm, ms_k1, ms_torch = med["gemm"][0], med["sparsify"][0], med["torch"][0]

    # dense-equivalent flops of a step (all layers)
    flops = sum(2 * L.M * L.N * L.K + (0 if sk else 2 * L.M * L.R * (L.K + L.N))
                for L, sk in zip(layers, skipped))
    dense_flops = sum(2 * L.M * L.N * L.K for L in layers)
    tflops = flops / (ms * 1e-3) / 1e12
    # dominant kernel: the 2:4 GEMM; algorithmic flops = products on kept values
    # (M N K/2 multiply-adds) + LoRA up-projection (M R N multiply-adds)
    k2_alg_flops = sum(L.M * L.N * L.K + 2 * L.M * L.R * L.N
                       for L, sk in zip(layers, skipped) if not sk)
    k2_tflops = k2_alg_flops / (ms_gemm * 1e-3) / 1e12
    traffic = traffic_for(args.workload)
    # the sparsifier's algorithmic HBM bytes: read X and LB, write the packed
    # values and meta, s and T (2MK + 2RK + MK + MK/8 + 4M + 2MR per layer)
    k1_bytes = sum(2 * L.M * L.K + 2 * L.R * L.K + L.M * L.K + L.M * L.K // 8 + 4 * L.M
                   + 2 * L.M * L.R for L, sk in zip(layers, skipped) if not sk)
    k1_gbs = k1_bytes / (ms_k1 * 1e-3) / 1e9
    if args.copy_calibration:
        src = torch.ones(COPY_MIB << 19, dtype=torch.bfloat16, device=dev)
        dst = torch.empty_like(src)
        for _ in range(3):
            torch.neg(src, out=dst)
        torch.cuda.synchronize()
        del src, dst
    cpu = None if args.no_cpu else cpu_baseline(layers[-1] if len(layers) == 1 else layers[2])

    shapes = [(f"{L.name}: " if len(layers) > 1 else "") + f"X[{L.M}x{L.K}] -> Y[{L.M}x{L.N}]"
              + (" (skipped: dense)" if sk else "") for L, sk in zip(layers, skipped)]
    kinds = sorted({L.kind for L in layers})
    first = layers[0]
    config = {"workload": f"{args.workload}: " + "; ".join(shapes) +
                          f"; bf16, rank-{first.R} LoRA, {'/'.join(kinds)} activations, "
                          f"{S} rotating input sets",
              "layers": [{"M": L.M, "K": L.K, "N": L.N, "R": L.R, "skipped": sk}
                         for L, sk in zip(layers, skipped)]}
    if len(layers) == 1:
        config.update({"M": first.M, "K": first.K, "N": first.N, "R": first.R})
    rec = {
        "metric": METRIC,
        "value": round(tflops, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms, 5),
        "ms_per_step_after_idle": round(ms_idle, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": config,
        "pct_sparse_peak": round(100 * tflops / PEAK_SPARSE_BF16_TFLOPS, 2),
        "pct_dense_peak": round(100 * tflops / PEAK_DENSE_BF16_TFLOPS, 2),
        "speedup_vs_dense": round(ms_dense / ms_sparse_i, 3),
        "speedup_vs_torch_matmul": round(ms_torch / ms_sparse_i, 3),
        # against the faster of the two dense layers (the library's and hipBLASLt)
        "speedup_vs_best_dense": round(min(ms_dense, ms_torch) / ms_sparse_i, 3),
        "interleaved_ms": {"sparse_layer": round(ms_sparse_i, 5), "dense_layer": round(ms_dense, 5),
                           "torch_matmul": round(ms_torch, 5)},
        # p10 / p90 of the per-round averages behind each median
        "interleaved_p10_p90_ms": {k: [round(v[1], 5), round(v[2], 5)] for k, v in med.items()},
        "dense_tflops": round(dense_flops / (ms_dense * 1e-3) / 1e12, 2),
        "split_ms": {"sparsify": round(ms_k1, 5), "sparse_gemm_lora": round(ms_gemm, 5)},
        "roofline": {"bound": "mfma", "kernel": "gemm_sparse32 (2:4 SMFMAC + LoRA up-projection)",
                     "achieved": round(k2_tflops, 2), "peak": PEAK_DENSE_BF16_TFLOPS,
                     "unit": "TFLOP/s", "frac": round(k2_tflops / PEAK_DENSE_BF16_TFLOPS, 4),
                     "traffic": traffic},
        # the sparsifier against the HBM bound (algorithmic bytes over its
        # interleaved median time)
        "sparsify_roofline": {"bound": "hbm", "kernel": "sparsify_kernel (select, norms, pack, LoRA down)",
                              "achieved": round(k1_gbs, 1), "peak": PEAK_HBM_GBS, "unit": "GB/s",
                              "frac": round(k1_gbs / PEAK_HBM_GBS, 4), "bytes": k1_bytes},
        # HBM bytes of the profiled K2 launch over its measured time, and the
        # matrix-core busy fractions of the profiled kernels (rocprofv3
        # counters committed under profiles/, null once the kernel changed)
        "k2_hbm_gbps": None if traffic is None else round(traffic / (ms_gemm * 1e-3) / 1e9, 1),
        "mfma_busy": mfma_busy_for(args.workload),
        "cpu_baseline": cpu,
    }
    print(json.dumps(rec))


if __name__ == "__main__":
    main()
