#!/usr/bin/env python3
"""Benchmark of one MLA tree-verify attention step on one MI355X.

A step is one verify_attn_run over the whole batch (split-K partial kernel + combine). The
default workload is the long-context one: 1 request, H=64 heads, a 23,000-key prefix and a
16-node random draft tree, bf16 q [16,64,576] and a bf16 latent cache scattered over a
1,048,576-slot pool. Inputs are resident in HBM before timing starts.

Prints ONE JSON line on stdout. Everything else goes to stderr.
"""
from __future__ import annotations

import argparse
import ctypes
import hashlib
import json
import math
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "verify-attn µs/step + effective HBM GB/s at P=23k, T=16, H=64 (% roofline)"
PEAK_HBM_GBS = 8000.0          # MI355X HBM3E
PEAK_MFMA_TFLOPS = 2500.0      # MI355X dense bf16/fp16 MFMA


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def algorithmic_work(w, out_bytes=4):
    """Bytes the method must move and flops it must do (one step)."""
    e_in = 2 if w.in_dtype == "bf16" else 4
    by = 0
    fl = 0
    for r in range(w.bs):
        t, p = int(w.tree_lens[r]), int(w.prefix_lens[r])
        l = t + p
        by += l * (576 * e_in + 8) + t * w.num_heads * (576 * e_in + 512 * out_bytes) + t * t
        m = w.custom_mask[w.mask_indptr[r]:w.mask_indptr[r + 1]].reshape(t, l)
        vis_tree = int((m[:, p:] != 0).sum())
        fl += 2 * (576 + 512) * w.num_heads * (t * p + vis_tree)
    by += (w.bs + 1) * 20
    return by, fl


def counter_traffic(kernel_file_stem, workload, sources):
    """HBM bytes per dispatch from the committed rocprofv3 byte-counter summary of this kernel
    and workload, or None when there is none or the kernel's sources changed since."""
    path = os.path.join(ROOT, "profiles", f"{kernel_file_stem}_{workload}.txt")
    if not os.path.exists(path):
        return None
    traffic = digest = None
    for line in open(path):
        line = line.strip()
        if line.startswith("traffic per dispatch:"):
            traffic = int(line.split(":")[1].split()[0])
        elif line.startswith("kernel sources sha256"):
            digest = line.rsplit(":", 1)[1].strip()
    h = hashlib.sha256()
    for f in sources:
        h.update(open(os.path.join(ROOT, "mla_tree_verify_paged_amd", "csrc", f), "rb").read())
    return traffic if digest == h.hexdigest() else None


class HipEvents:
    """hipEvent_t handles from the HIP runtime torch uses (same process-wide copy)."""

    def __init__(self):
        import torch  # noqa: F401  (loads the runtime)
        self.rt = ctypes.CDLL("libamdhip64.so.7")
        self.rt.hipEventCreateWithFlags.argtypes = [ctypes.POINTER(ctypes.c_void_p),
                                                    ctypes.c_uint]
        self.rt.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.c_void_p,
                                                ctypes.c_void_p]
        self.rt.hipEventDestroy.argtypes = [ctypes.c_void_p]
        self.rt.hipEventRecord.argtypes = [ctypes.c_void_p, ctypes.c_void_p]

    # timing-only events: no system-scope fence when recorded (its cache writeback would be
    # charged to the kernel being timed); the host synchronises the device before reading them
    DISABLE_SYSTEM_FENCE = 0x20000000

    def create(self):
        e = ctypes.c_void_p()
        rc = self.rt.hipEventCreateWithFlags(ctypes.byref(e), self.DISABLE_SYSTEM_FENCE)
        if rc != 0:
            raise RuntimeError(f"hipEventCreateWithFlags failed: {rc}")
        return e.value

    def elapsed_ms(self, a, b):
        f = ctypes.c_float()
        rc = self.rt.hipEventElapsedTime(ctypes.byref(f), a, b)
        if rc != 0:
            raise RuntimeError(f"hipEventElapsedTime failed: {rc}")
        return float(f.value)

    def record(self, e, stream_handle):
        rc = self.rt.hipEventRecord(e, stream_handle)
        if rc != 0:
            raise RuntimeError(f"hipEventRecord failed: {rc}")

    def destroy(self, e):
        self.rt.hipEventDestroy(e)


def cpu_model():
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def oracle_us_per_step(w, pool, cores, budget_s, reps=3):
    """Median over `reps` runs of the oracle on an evenly spaced sample of the workload's
    rows sized to about budget_s / reps seconds per run, scaled to all rows (us per step).
    Returns (us_per_step, rows_in_sample, median_run_seconds)."""
    import oracle
    total = w.num_tokens * w.num_heads
    probe = np.arange(0, total, max(1, total // 16))[:16]
    t0 = time.perf_counter()
    oracle.run_workload(w, rows=probe, nthreads=cores, pool=pool)
    per_row = (time.perf_counter() - t0) / len(probe)
    n = int(min(total, max(len(probe), budget_s / reps / max(per_row, 1e-9))))
    rows = np.unique(np.linspace(0, total - 1, n).round().astype(np.int64))
    runs = []
    for _ in range(reps):
        t0 = time.perf_counter()
        oracle.run_workload(w, rows=rows, nthreads=cores, pool=pool)
        runs.append(time.perf_counter() - t0)
    dt = float(np.median(runs))
    return dt / len(rows) * total * 1e6, len(rows), dt


def cpu_baseline(w, budget_s=15.0):
    """The fp64 oracle on the host cores: a bounded, deterministic sample of rows of the
    bench's workload (median of 3 runs, scaled to a whole step), plus single-threaded timings
    of the tiny and short workloads."""
    import workloads
    cores = int(os.environ.get("OMP_NUM_THREADS", os.cpu_count() or 1))
    total = w.num_tokens * w.num_heads
    us_step, n_rows, dt = oracle_us_per_step(w, w.pool_np(), cores, budget_s)
    single = {}
    for name, budget in (("tiny", 0.3), ("short", 4.0)):
        sw = workloads.make(name)
        us, rows, sdt = oracle_us_per_step(sw, sw.pool_np(), 1, budget)
        single[name] = {"us_per_step": round(us, 1), "rows_in_sample": rows,
                        "rows_total": sw.num_tokens * sw.num_heads,
                        "median_run_s": round(sdt, 3)}
    return {"value": us_step, "unit": "us/step", "cores": cores, "kind": "oracle",
            "cpu_model": cpu_model(), "host_cpus": os.cpu_count(),
            "sample": f"{n_rows} of {total} (token, head) rows of the same workload, evenly "
                      f"spaced; fp64 two-pass C loop with OpenMP on {cores} threads; median of "
                      f"3 runs ({dt:.2f} s each), scaled to all rows",
            "single_thread": single}


def time_tree_ops(w, va, steps):
    """Times the two tree kernels on the workload's trees: the mask build (with mask_indptr)
    and greedy acceptance (synthetic draft / target tokens that accept about half the time).
    The mask build is priced against HBM: its algorithmic bytes are the mask it writes plus
    the parents and index tables it reads."""
    import torch
    parents = torch.from_numpy(np.concatenate(w.parents).astype(np.int64)).cuda()
    qo = torch.from_numpy(w.qo_indptr).cuda()
    kv = torch.from_numpy(w.kv_indptr).cuda()
    mask = torch.empty(int(w.mask_indptr[-1]), dtype=torch.uint8, device="cuda")
    ind = torch.empty(w.bs + 1, dtype=torch.int64, device="cuda")
    rng = np.random.default_rng(1)
    draft = rng.integers(0, 4, w.num_tokens).astype(np.int64)
    target = rng.integers(0, 4, w.num_tokens).astype(np.int64)
    d_draft, d_target = torch.from_numpy(draft).cuda(), torch.from_numpy(target).cuda()
    acc = torch.empty(w.bs, dtype=torch.int32, device="cuda")
    path = torch.empty((w.bs, max(1, w.max_q_per_req)), dtype=torch.int64, device="cuda")
    nxt = torch.empty(w.bs, dtype=torch.int64, device="cuda")

    def timed(fn):
        # the calls are recorded into a graph and replayed, so host time per call (argument
        # marshalling) cannot enter the figure: it is the GPU time of back-to-back launches
        fn(True)
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        s = torch.cuda.Stream()
        s.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(s):
            fn(False)
        torch.cuda.current_stream().wait_stream(s)
        torch.cuda.synchronize()
        with torch.cuda.graph(g):
            for _ in range(steps):
                fn(False)
        g.replay()
        torch.cuda.synchronize()
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        g.replay()
        b.record()
        b.synchronize()
        return a.elapsed_time(b) * 1e3 / steps

    mask_us = timed(lambda c: va.build_mask(parents, qo, kv, mask, ind, check=c))
    accept_us = timed(lambda c: va.accept(parents, d_draft, d_target, qo, acc, path, nxt,
                                          check=c))
    ok = bool(torch.equal(mask.cpu(), torch.from_numpy(w.custom_mask)))
    mask_bytes = int(w.mask_indptr[-1]) + 8 * w.num_tokens + 20 * (w.bs + 1)
    return {"mask_build_us": round(mask_us, 3), "mask_bytes": mask_bytes,
            "mask_build_GBps": round(mask_bytes / (mask_us * 1e-6) / 1e9, 2),
            "mask_build_frac_hbm": round(mask_bytes / (mask_us * 1e-6) / 1e9 / PEAK_HBM_GBS, 4),
            "mask_matches_workload": ok, "accept_us": round(accept_us, 3),
            "timing": "back-to-back launches recorded in a graph, replay time per launch"}


def single_launch_ab(partial_us, combine_us, step_us):
    """The fixed costs of a single-launch merge on this GPU (csrc/single_launch_ab.hip):
    a cooperative launch and one grid barrier, against the measured two-launch step. The
    fused step cannot take less than the partial kernel plus those two costs (its merge
    reads the same partials the combine reads)."""
    lib_path = os.path.join(ROOT, "mla_tree_verify_paged_amd", "libsingle_launch_ab.so")
    lib = ctypes.CDLL(lib_path)
    lib.single_launch_ab.argtypes = [ctypes.POINTER(ctypes.c_double)]
    lib.single_launch_ab.restype = ctypes.c_int
    out = (ctypes.c_double * 8)()
    rc = lib.single_launch_ab(out)
    if rc != 0:
        return {"error": f"hip error {rc}"}
    plain, coop, coop1, coop33, graph1, timeouts, mismatches, captured = list(out)
    barrier_us = (coop33 - coop1) / 64.0          # 33 barrier pairs against 1
    coop_overhead_us = coop - plain
    bound = partial_us + coop_overhead_us + barrier_us
    return {
        "plain_launch_us": round(plain, 2), "cooperative_launch_us": round(coop, 2),
        "cooperative_overhead_us": round(coop_overhead_us, 2),
        "grid_barrier_us": round(barrier_us, 2),
        "cooperative_graph_replay_1_barrier_pair_us": round(graph1, 2),
        "cooperative_capture_ok": bool(captured), "barrier_timeouts": int(timeouts),
        "visibility_mismatches": int(mismatches),
        "two_launch_step_us": round(step_us, 2), "two_launch_combine_us": round(combine_us, 2),
        "fused_step_lower_bound_us": round(bound, 2),
        "fused_wins": bool(bound < step_us),
        "method": "fused >= partial kernel + (cooperative - plain launch) + one grid barrier; "
                  "1 vs 33 barrier pairs on 1 workgroup per CU with 150 KB LDS",
    }


def lds_probe():
    """How fast LDS feeds the matrix cores at one and two wavefronts per SIMD, per operand read
    form, and what a dependent accumulation chain costs (csrc/lds_mfma_probe.hip)."""
    lib = ctypes.CDLL(os.path.join(ROOT, "mla_tree_verify_paged_amd", "liblds_mfma_probe.so"))
    lib.lds_mfma_probe.argtypes = [ctypes.POINTER(ctypes.c_double)]
    lib.lds_mfma_probe.restype = ctypes.c_int
    out = (ctypes.c_double * 28)()
    rc = lib.lds_mfma_probe(out)
    if rc != 0:
        return {"error": f"hip error {rc}"}
    forms = ["b128 (K fragment)", "two tr_b64 (V^T fragment)", "alternating",
             "b128 + two tr_b64 (2 KB per product)", "two b128 (2 KB per product)",
             "four tr_b64 (2 KB per product)"]
    nf = len(forms)
    feed = {}
    for w in range(2):
        for f, name in enumerate(forms):
            feed.setdefault(name, {})[f"{w + 1} wave/SIMD"] = {
                "mfma_util_pct": round(out[2 * nf * w + 2 * f], 1),
                "lds_bytes_per_clk_per_cu": round(out[2 * nf * w + 2 * f + 1], 1)}
    return {"feed": feed,
            "cycles_per_32x32x16_product": {"1 chain": round(out[4 * nf], 2),
                                            "2 chains": round(out[4 * nf + 1], 2),
                                            "4 chains": round(out[4 * nf + 2], 2)},
            "clock_ghz": round(out[4 * nf + 3], 2),
            "method": "one 256- or 512-thread workgroup per CU (96 KB LDS), each product's 1 KB "
                      "operand read 4 products ahead; utilisation = matrix cycles / elapsed "
                      "cycles"}


SWEEP_P = (1024, 5700, 23000, 65536, 131072)
SWEEP_T = (1, 4, 16, 64)
SWEEP_BS = (1, 8, 32)


def sweep(heads=64, budget_s=0.2, seed=0):
    """Step time over prefix length x tree size x batch size (H = 64, one GPU): where the path
    is bound by HBM bytes and where by matrix work. Inputs are drawn on the device (seeded
    standard normal bf16 q and key rows, key rows scattered over a pool with one ninth of its
    slots unused, random draft trees per request whose mask the library's own mask build
    writes); each case is captured in a graph and replayed."""
    import torch
    import workloads
    from mla_tree_verify_paged_amd import VerifyAttn
    gen = torch.Generator(device="cuda")
    gen.manual_seed(seed)
    rng = np.random.default_rng(seed)
    out_rows = []
    for P in SWEEP_P:
        for T in SWEEP_T:
            for bs in SWEEP_BS:
                L = P + T
                n_keys, n_tok = bs * L, bs * T
                slots = n_keys + n_keys // 8
                q = torch.randn((n_tok, heads, 576), generator=gen, device="cuda").bfloat16()
                pool = torch.empty((slots, 576), dtype=torch.bfloat16, device="cuda")
                for a in range(0, slots, 1 << 20):  # in chunks: bounded fp32 temporaries
                    b = min(slots, a + (1 << 20))
                    pool[a:b] = torch.randn((b - a, 576), generator=gen, device="cuda").bfloat16()
                kvi = torch.randperm(slots, generator=gen, device="cuda")[:n_keys].contiguous()
                kvp = (torch.arange(bs + 1, device="cuda", dtype=torch.int64) * L).int()
                qo = torch.arange(bs + 1, device="cuda", dtype=torch.int64) * T
                trees = [workloads.random_tree(T, rng) for _ in range(bs)]
                par = torch.from_numpy(np.concatenate(trees)).cuda()
                va = VerifyAttn(heads, max_batch=bs, max_q_per_req=T, max_q_tokens=n_tok)
                mask = torch.empty(bs * T * L, dtype=torch.uint8, device="cuda")
                mind = torch.empty(bs + 1, dtype=torch.int64, device="cuda")
                va.build_mask(par, qo, kvp, mask, mind)
                out = torch.empty((n_tok, heads, 512), dtype=torch.float32, device="cuda")
                lse = torch.empty((n_tok, heads), dtype=torch.float32, device="cuda")

                def step(check=False):
                    va.run(q, pool, kvi, kvp, qo, mask, mind, workloads.DEFAULT_SCALE, out, lse,
                           None, bs=bs, num_tokens=n_tok, check=check)

                step(True)
                torch.cuda.synchronize()
                status = va.read_device_status()
                g = torch.cuda.CUDAGraph()
                st = torch.cuda.Stream()
                st.wait_stream(torch.cuda.current_stream())
                with torch.cuda.stream(st):
                    step()
                torch.cuda.current_stream().wait_stream(st)
                torch.cuda.synchronize()
                with torch.cuda.graph(g):
                    step()
                ev0 = torch.cuda.Event(enable_timing=True)
                ev1 = torch.cuda.Event(enable_timing=True)
                g.replay()
                ev0.record()
                g.replay()
                ev1.record()
                ev1.synchronize()
                est = ev0.elapsed_time(ev1) * 1e-3
                reps = int(min(50, max(3, budget_s / max(est, 1e-6))))
                ev0.record()
                for _ in range(reps):
                    g.replay()
                ev1.record()
                ev1.synchronize()
                us = ev0.elapsed_time(ev1) * 1e3 / reps
                vis = sum(int(workloads.tree_depths(t).sum()) + T for t in trees)
                fl = 2 * (576 + 512) * heads * (bs * T * P + vis)
                by = bs * (L * (576 * 2 + 8) + T * heads * (576 * 2 + 512 * 4) + T * T) + \
                    (bs + 1) * 20
                f_mfma = fl / (us * 1e-6) / 1e12 / PEAK_MFMA_TFLOPS
                f_hbm = by / (us * 1e-6) / 1e9 / PEAK_HBM_GBS
                hbm_bound = by / (PEAK_HBM_GBS * 1e9) > fl / (PEAK_MFMA_TFLOPS * 1e12)
                out_rows.append({
                    "P": P, "T": T, "bs": bs, "us": round(us, 2), "status": status,
                    "TFLOPs": round(fl / (us * 1e-6) / 1e12, 1),
                    "GBps": round(by / (us * 1e-6) / 1e9, 1),
                    "flop_per_byte": round(fl / by, 1),
                    "bound": "hbm" if hbm_bound else "mfma",
                    "frac": round(f_hbm if hbm_bound else f_mfma, 4), "replays": reps})
                log(f"sweep P={P} T={T} bs={bs}: {us:.1f} us, "
                    f"{'hbm' if hbm_bound else 'mfma'} frac "
                    f"{f_hbm if hbm_bound else f_mfma:.3f}")
                va.close()
                del q, pool, kvi, mask, out, lse, g
                torch.cuda.empty_cache()
    return out_rows


# ---- rocprofv3 summaries (profiles/*.txt), written from the csv output of these commands,
# run from a scratch folder <out> on an MI355X (the profiler wants TMPDIR on a local disk):
PROFILE_KERNELS = {
    # file stem: (kernel-name fragment, sources whose sha256 the summary records)
    "mfma_partial_kernel": ("mfma_partial_kernel<", ["verify_mfma.hip", "va_internal.h"]),
    "mfma_partial_ws_kernel": ("mfma_partial_ws_kernel<", ["verify_mfma.hip", "va_internal.h"]),
    "simple_partial_kernel": ("simple_partial_kernel", ["verify_simple.hip", "va_internal.h"]),
    "combine_kernel": ("combine_kernel<", ["verify_combine.hip", "va_internal.h"]),
    "combine_rows_kernel": ("combine_rows_kernel<", ["verify_combine.hip", "va_internal.h"]),
    "combine_few_rows_kernel": ("combine_few_rows_kernel", ["verify_combine.hip",
                                                            "va_internal.h"]),
    "build_mask_kernel": ("build_mask_kernel<", ["tree_ops.hip", "va_internal.h"]),
    "accept_kernel": ("accept_kernel", ["tree_ops.hip", "va_internal.h"]),
}
PROFILE_BENCH_ARGS = "--steps 20 --warmup 5 --cold-steps 5 --no-cpu-baseline --copy-calibration"
PROFILE_PASSES = (("trace", "--kernel-trace --stats"), ("fetch", "--pmc FETCH_SIZE"),
                  ("write", "--pmc WRITE_SIZE"))
WAVE_BENCH_ARGS = "--steps 10 --warmup 2 --cold-steps 2 --no-cpu-baseline"
WAVE_PASSES = (
    ("a", "SQ_VALU_MFMA_BUSY_CYCLES SQ_VALU_MFMA_COEXEC_CYCLES SQ_BUSY_CU_CYCLES "
          "SQ_INSTS_VALU_MFMA_MOPS_BF16 SQ_INSTS_VALU_MFMA_MOPS_F16 SQ_ACTIVE_INST_VALU "
          "SQ_WAVE_CYCLES SQ_LDS_BANK_CONFLICT GRBM_GUI_ACTIVE"),
    ("b", "SQ_ACTIVE_INST_LDS SQ_WAIT_INST_ANY SQ_ACTIVE_INST_ANY SQ_INSTS_LDS SQ_INSTS_VALU "
          "SQ_INSTS_MFMA SQ_WAIT_ANY SQ_ACTIVE_INST_MISC GRBM_GUI_ACTIVE"),
    ("c", "SQ_LDS_IDX_ACTIVE SQ_LDS_DATA_FIFO_FULL SQ_LDS_CMD_FIFO_FULL SQ_WAIT_INST_LDS "
          "SQ_INST_LEVEL_LDS SQ_INSTS_LDS_LOAD_BANDWIDTH SQ_LDS_ADDR_CONFLICT "
          "SQ_INSTS_LDS_STORE_BANDWIDTH GRBM_GUI_ACTIVE"),
)


def profile_commands(workload):
    """The commands whose output --summarize-profile reads (run in <out>, repository at <repo>)."""
    cmds = ["cd <out> && export TMPDIR=/tmp"]
    for sub, flags in PROFILE_PASSES:
        cmds.append(f"rocprofv3 {flags} --output-format csv -d <out>/{sub} -o run -- python3 "
                    f"<repo>/bench.py --workload {workload} {PROFILE_BENCH_ARGS} > "
                    f"<out>/{sub}.json")
    cmds.append(f"python3 <repo>/bench.py --workload {workload} --summarize-profile <out>")
    return cmds


def wave_commands(workload):
    cmds = ["cd <out> && export TMPDIR=/tmp"]
    for sub, counters in WAVE_PASSES:
        cmds.append(f"rocprofv3 --pmc {counters} --output-format csv -d <out>/{sub} -o run -- "
                    f"python3 <repo>/bench.py --workload {workload} {WAVE_BENCH_ARGS} > "
                    f"<out>/{sub}.json")
    cmds.append(f"python3 <repo>/bench.py --workload {workload} --summarize-wave-counters <out>")
    return cmds


def _csv_rows(path):
    import csv
    with open(path) as f:
        return list(csv.DictReader(f))


def _per_dispatch(rows, counter, fragment):
    """Counter summed over its instances for each dispatch of kernels matching `fragment`."""
    per = {}
    for r in rows:
        if r["Counter_Name"] == counter and fragment in r["Kernel_Name"]:
            k = int(r["Dispatch_Id"])
            per[k] = per.get(k, 0.0) + float(r["Counter_Value"])
    return per


def _sources_sha(sources):
    h = hashlib.sha256()
    for f in sources:
        h.update(open(os.path.join(ROOT, "mla_tree_verify_paged_amd", "csrc", f), "rb").read())
    return h.hexdigest()


def _bench_line(path):
    lines = [ln for ln in open(path).read().splitlines() if ln.startswith("{")]
    return json.loads(lines[-1]) if lines else {}


def _timed_dispatches(d, bench, stem):
    """The trace average over the traced run's timed steps alone, for the kernels every step
    launches once (the partial and combine kernels): the dispatches after the checked call,
    the settle steps and the warm-up. The all-dispatch average above mixes the clock's ramp
    and the graph and cold replays in."""
    if not bench or not ("partial" in stem or "combine" in stem):
        return []
    s0 = 1 + int(bench.get("settle_steps", 0)) + int(bench.get("warmup", 0))
    k = int(bench.get("steps", 0))
    if k <= 0 or len(d) < s0 + k:
        return []
    t = d[s0:s0 + k]
    return [f"  the {k} timed steps (dispatches {s0}..{s0 + k - 1}): average "
            f"{sum(t) / k:.3f} us, min {min(t):.3f} us, max {max(t):.3f} us"]


def summarize_profile(out_dir, workload, dest=None):
    """Writes profiles/<kernel>_<workload>.txt for every profiled kernel that ran: its kernel
    trace and --stats row, and its HBM bytes per dispatch from FETCH_SIZE and WRITE_SIZE
    (KiB per dispatch), each scaled by what the same counter reads for the calibration kernel
    (one fp32 elementwise multiply over 64 Mi elements: 256 MiB read, 256 MiB written)."""
    import statistics
    trace = _csv_rows(os.path.join(out_dir, "trace", "run_kernel_trace.csv"))
    stats = _csv_rows(os.path.join(out_dir, "trace", "run_kernel_stats.csv"))
    fetch = _csv_rows(os.path.join(out_dir, "fetch", "run_counter_collection.csv"))
    write = _csv_rows(os.path.join(out_dir, "write", "run_counter_collection.csv"))
    bench = _bench_line(os.path.join(out_dir, "trace.json"))

    def calibration(rows, counter):
        per = _per_dispatch(rows, counter, "MulFunctor")
        return per[max(per)]  # the last elementwise multiply: the 256 MiB calibration kernel

    cf, cw = calibration(fetch, "FETCH_SIZE"), calibration(write, "WRITE_SIZE")
    ff = round(262144.0 / cf * 1000) / 1000
    fw = round(262144.0 / cw * 1000) / 1000
    written = []
    for stem, (frag, sources) in PROFILE_KERNELS.items():
        ks = [r for r in trace if frag in r["Kernel_Name"]]
        if not ks:
            continue
        d = [(int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3 for r in ks]
        r0 = ks[-1]
        names = sorted({r["Kernel_Name"].split("namespace)::")[-1].split("(va::")[0]
                        for r in ks})
        fpd = _per_dispatch(fetch, "FETCH_SIZE", frag)
        wpd = _per_dispatch(write, "WRITE_SIZE", frag)
        f_kib = statistics.mean(fpd.values())
        w_kib = statistics.mean(wpd.values())
        rd, wr = f_kib * ff * 1024, w_kib * fw * 1024
        o = [f"# {stem} - workload '{workload}' (bench.py's '{workload}' configuration)", "",
             "Commands (<repo> is the repository root, <out> a scratch folder):"]
        o += ["  " + c for c in profile_commands(workload)]
        what = ("checked call, settle and warm-up steps, timed steps, graph replays and cold "
                "replays" if ("partial" in stem or "combine" in stem) else
                "the tree-op timing's checked calls, warm-up and graph replays")
        o += ["", f"Kernel trace ({len(d)} dispatches: {what}):",
              "  instantiations: " + ", ".join(names),
              f"  average {statistics.mean(d):.3f} us, median {statistics.median(d):.3f} us, "
              f"min {min(d):.3f} us, max {max(d):.3f} us",
              *_timed_dispatches(d, bench, stem),
              f"  grid {r0['Grid_Size_X']} work-items, workgroup {r0['Workgroup_Size_X']}, LDS "
              f"{r0['LDS_Block_Size']} B, VGPR {r0['VGPR_Count']}, AGPR "
              f"{r0['Accum_VGPR_Count']}, SGPR {r0['SGPR_Count']}, scratch {r0['Scratch_Size']} B",
              "", "rocprofv3 --stats (run_kernel_stats.csv):"]
        for r in stats:
            if frag in r["Name"]:
                nm = r["Name"].split("namespace)::")[-1].split("(va::")[0]
                o.append(f"  {nm}: calls {r['Calls']}, average {float(r['AverageNs']) / 1e3:.3f}"
                         f" us, min {float(r['MinNs']) / 1e3:.3f} us, max "
                         f"{float(r['MaxNs']) / 1e3:.3f} us, {r['Percentage']}% of kernel time")
        o += ["", f"Byte counters (KiB per dispatch, mean over {len(fpd)} and {len(wpd)} "
                  "dispatches):",
              f"  FETCH_SIZE {f_kib:.1f}  x {ff:.3f} (calibration) = {rd / 2**20:.2f} MiB read",
              f"  WRITE_SIZE {w_kib:.1f}  x {fw:.3f} (calibration) = {wr / 2**20:.2f} MiB written",
              f"  calibration: the elementwise fp32 kernel that reads and writes 256 MiB reads "
              f"FETCH_SIZE {cf:.1f} KiB and WRITE_SIZE {cw:.1f} KiB", "",
              f"  traffic per dispatch: {int(round(rd + wr))} bytes",
              f"  kernel sources sha256 ({' + '.join(sources)}): {_sources_sha(sources)}"]
        if bench:
            o += ["", "bench.py line of the traced run (its own HIP-event timing, under the "
                      "profiler):",
                  f"  partial_kernel_us {bench.get('partial_kernel_us')}, combine_kernel_us "
                  f"{bench.get('combine_kernel_us')}, value {bench.get('value')} us/step"]
        path = os.path.join(dest or os.path.join(ROOT, "profiles"), f"{stem}_{workload}.txt")
        with open(path, "w") as f:
            f.write("\n".join(o) + "\n")
        written.append(path)
    return written


def summarize_wave_counters(out_dir, workload, dest=None):
    """Writes profiles/<partial kernel>_<workload>_wave_counters.txt from the three SQ counter
    passes: matrix-core busy time, issue and wait fractions, LDS traffic. The partial kernel is
    the 8-wavefront variant when it ran, else the 4-wavefront one."""
    import statistics
    rows_by = {sub: _csv_rows(os.path.join(out_dir, sub, "run_counter_collection.csv"))
               for sub, _ in WAVE_PASSES}
    ws = any("mfma_partial_ws_kernel<" in r["Kernel_Name"] for r in rows_by[WAVE_PASSES[0][0]])
    stem = "mfma_partial_ws_kernel" if ws else "mfma_partial_kernel"
    waves_per_simd = 2 if ws else 1
    vals = {}
    for sub, _ in WAVE_PASSES:
        rows = rows_by[sub]
        names = {r["Counter_Name"] for r in rows}
        for c in names:
            per = _per_dispatch(rows, c, stem + "<")
            if per:
                vals[c] = (statistics.mean(per.values()), len(per))
    simds = 256 * 4
    v = {k: x[0] for k, x in vals.items()}
    n = vals["SQ_WAVE_CYCLES"][1]
    # SQ_WAVE_CYCLES counts 4-cycle units and sums over the wavefronts a SIMD holds
    life = v["SQ_WAVE_CYCLES"] * 4 / simds / waves_per_simd
    busy = v["SQ_VALU_MFMA_BUSY_CYCLES"] / simds
    co = v["SQ_VALU_MFMA_COEXEC_CYCLES"] / simds
    mops = v["SQ_INSTS_VALU_MFMA_MOPS_BF16"] + v["SQ_INSTS_VALU_MFMA_MOPS_F16"]

    def pct(counter):  # per SIMD (both wavefronts together when there are two)
        return 100 * v[counter] * 4 / simds / life

    srcs = PROFILE_KERNELS[stem][1]
    o = [f"# {stem} - workload '{workload}': wave-level counters", "",
         "Commands (<repo> is the repository root, <out> a scratch folder):"]
    o += ["  " + c for c in wave_commands(workload)]
    o += ["", f"Raw counters (mean per dispatch over {n} dispatches; SQ_* summed over the chip):"]
    o += [f"  {k:32s} {v[k]:.1f}" for k in sorted(v)]
    o += ["", f"Derived (1024 SIMDs, {waves_per_simd} wavefront(s) per SIMD for the whole "
              "kernel; SQ_WAVE_CYCLES and SQ_ACTIVE_*/SQ_WAIT_* count 4-cycle units summed over "
              "wavefronts, SQ_VALU_MFMA_* cycles; issue and wait fractions are per SIMD):",
          f"  matrix work: (MOPS_BF16 + MOPS_F16) x 512 = {mops * 512 / 1e9:.2f} GFLOP per "
          "dispatch",
          f"  wavefront lifetime: {life:.0f} cycles per SIMD",
          f"  matrix core busy: {busy:.0f} cycles per SIMD = {100 * busy / life:.1f}% of the "
          "lifetime",
          f"  VALU issuing while the matrix core is busy: {co:.0f} cycles per SIMD "
          f"({100 * co / busy:.1f}% of its busy time)",
          f"  VALU issue {pct('SQ_ACTIVE_INST_VALU'):.1f}%, LDS issue "
          f"{pct('SQ_ACTIVE_INST_LDS'):.1f}%, any issue {pct('SQ_ACTIVE_INST_ANY'):.1f}%, "
          f"waiting on a dependency {pct('SQ_WAIT_INST_ANY'):.1f}% of the lifetime",
          f"  instructions per SIMD: {v['SQ_INSTS_MFMA'] / simds:.0f} matrix, "
          f"{v['SQ_INSTS_VALU'] / simds:.0f} VALU (matrix included), "
          f"{v['SQ_INSTS_LDS'] / simds:.0f} LDS",
          f"  LDS bank conflicts: {v['SQ_LDS_BANK_CONFLICT']:.0f} cycles",
          f"  LDS bytes read by LDS instructions (64-byte units): "
          f"{v['SQ_INSTS_LDS_LOAD_BANDWIDTH'] * 64 / 1e9:.2f} GB per dispatch, "
          f"{v['SQ_INSTS_LDS_LOAD_BANDWIDTH'] * 64 / 256 / life:.0f} B per cycle per compute "
          "unit over the lifetime (direct-to-LDS tile loads come on top)",
          f"  waiting to issue an LDS instruction: {pct('SQ_WAIT_INST_LDS'):.1f}% of the lifetime",
          "", f"  kernel sources sha256 ({' + '.join(srcs)}): {_sources_sha(srcs)}"]
    path = os.path.join(dest or os.path.join(ROOT, "profiles"),
                        f"{stem}_{workload}_wave_counters.txt")
    with open(path, "w") as f:
        f.write("\n".join(o) + "\n")
    return [path]


def workload_names():
    import workloads
    return workloads.CONFIGS.keys()


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=100)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--settle-ms", type=float, default=50.0,
                    help="untimed steps for at least this long before the warm-up steps: the "
                         "GPU's clock takes about 15-20 ms of load to reach its steady value "
                         "(reported as settle_steps)")
    ap.add_argument("--workload", default="long", choices=sorted(workload_names()))
    ap.add_argument("--kernel", default="auto", choices=["auto", "simple", "mfma"])
    ap.add_argument("--splits", type=int, default=0)
    ap.add_argument("--layout", default="combined", choices=["combined", "split"],
                    help="key slots: tree slots at the tail of each kv_indices segment, or "
                         "prefix-only kv_indices plus out_cache_loc")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cold-steps", type=int, default=200,
                    help="graph replays timed cold, each after a 512 MB flush (median, p10, p90)")
    ap.add_argument("--single-launch-ab", action="store_true",
                    help="also measure the fixed costs a single-launch (fused) merge would pay: "
                         "cooperative launch overhead and one grid barrier, against this step's "
                         "two-launch time (extra key single_launch_ab)")
    ap.add_argument("--lds-probe", action="store_true",
                    help="also measure how fast LDS feeds the matrix cores at one and two "
                         "wavefronts per SIMD (extra key lds_probe)")
    ap.add_argument("--sweep", action="store_true",
                    help="also time the step over P x T x bs (extra key sweep)")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="also run one elementwise kernel that reads and writes 256 MiB (for "
                         "scaling hardware byte counters)")
    ap.add_argument("--summarize-profile", metavar="OUT",
                    help="write profiles/<kernel>_<workload>.txt from the rocprofv3 output in OUT "
                         "(kernel trace with --stats, then FETCH_SIZE, then WRITE_SIZE); no GPU")
    ap.add_argument("--summarize-wave-counters", metavar="OUT",
                    help="write profiles/<partial kernel>_<workload>_wave_counters.txt from "
                         "the three SQ counter passes in OUT; no GPU")
    args = ap.parse_args()

    if args.summarize_profile or args.summarize_wave_counters:
        paths = (summarize_profile(args.summarize_profile, args.workload)
                 if args.summarize_profile else
                 summarize_wave_counters(args.summarize_wave_counters, args.workload))
        for p in paths:
            log(p)
        return

    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py measures one GPU only: the verify path is a single-GPU kernel library; "
              "run with --gpus 1", file=sys.stderr)
        sys.exit(2)

    import torch
    import workloads
    from mla_tree_verify_paged_amd import VerifyAttn
    from mla_tree_verify_paged_amd.binding import verify_attn_set_profiling_events
    from mla_tree_verify_paged_amd.device_inputs import to_device

    w = workloads.make(args.workload)
    log(f"workload {w.name}: bs={w.bs} H={w.num_heads} P={w.prefix_lens.tolist()} "
        f"T={w.tree_lens.tolist()} in={w.in_dtype}")
    dev = to_device(w)
    va = VerifyAttn(w.num_heads, in_dtype=w.in_dtype, out_dtype="fp32", max_batch=w.bs,
                    max_q_per_req=w.max_q_per_req, max_q_tokens=w.num_tokens,
                    num_splits=args.splits, kernel=args.kernel)
    info = va.info
    kernel_name = {1: "simple", 2: "mfma"}[info.kernel]
    # the MFMA partial kernel's variant: 8 wavefronts per workgroup (two per SIMD) or 4
    part_stem = "mfma_partial_ws_kernel" if info.partial_waves == 8 else "mfma_partial_kernel"
    log(f"kernel={kernel_name} splits={info.num_splits} workspace={info.workspace_bytes} "
        f"partial waves={info.partial_waves}")
    out = torch.empty((w.num_tokens, w.num_heads, 512), dtype=torch.float32, device="cuda")
    lse = torch.empty((w.num_tokens, w.num_heads), dtype=torch.float32, device="cuda")
    stream = torch.cuda.current_stream()

    split = args.layout == "split"
    kvi = dev["kv_indices_prefix"] if split else dev["kv_indices"]
    kvp = dev["kv_indptr_prefix"] if split else dev["kv_indptr"]
    ocl = dev["out_cache_loc"] if split else None

    def run_on(stream_handle, check=False):
        # the buffers are checked once (first warm-up call); the timed calls skip the host-side
        # layout checks, whose Python cost would otherwise enter short steps
        va.run(dev["q"], dev["kv_buffer"], kvi, kvp, dev["qo_indptr"], dev["custom_mask"],
               dev["mask_indptr"], w.scale, out, lse, None, bs=w.bs, num_tokens=w.num_tokens,
               stream=stream_handle, out_cache_loc=ocl, check=check)

    def step():
        run_on(stream.cuda_stream)

    run_on(stream.cuda_stream, check=True)
    # settle: untimed steps until the clock has had settle_ms of load (in batches of 16 steps,
    # each batch waited for, so the count reflects device time)
    settle_steps = 0
    t_settle = time.perf_counter()
    while (time.perf_counter() - t_settle) * 1e3 < args.settle_ms:
        for _ in range(16):
            step()
        settle_steps += 16
        torch.cuda.synchronize()
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    status = va.read_device_status()
    if status != 0 or not torch.isfinite(out).all():
        log(f"bad output: status={status}")
        sys.exit(1)

    # ---- timed region: K eager steps, per-kernel HIP events recorded by the library on the
    # launch stream: step i records edge[i] ahead of its partial kernel and mid[i] between its
    # two kernels; edge[i + 1] (the next step's, or one recorded after the last step) ends
    # its combine. Two events per step rather than three: each recorded event is a queue
    # packet that costs the step about 1.5 us.
    hev = HipEvents()
    edge = [hev.create() for _ in range(args.steps + 1)]
    mid = [hev.create() for _ in range(args.steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        verify_attn_set_profiling_events(va.ctx, edge[i], mid[i], None)
        step()
    hev.record(edge[args.steps], stream.cuda_stream)
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    verify_attn_set_profiling_events(va.ctx, None, None, None)
    part_ms = np.array([hev.elapsed_ms(edge[i], mid[i]) for i in range(args.steps)])
    comb_ms = np.array([hev.elapsed_ms(mid[i], edge[i + 1]) for i in range(args.steps)])
    for x in edge + mid:
        hev.destroy(x)
    ms_per_step = (t1 - t0) * 1e3 / args.steps
    log(f"eager: {ms_per_step * 1e3:.2f} us/step; partial {part_ms.mean() * 1e3:.2f} us, "
        f"combine {comb_ms.mean() * 1e3:.2f} us")

    # ---- graph replays (capture-safe path), warm and cold
    g = torch.cuda.CUDAGraph()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        run_on(s.cuda_stream)
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    with torch.cuda.graph(g):
        run_on(torch.cuda.current_stream().cuda_stream)
    for _ in range(20):  # warm-up replays
        g.replay()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        g.replay()
    torch.cuda.synchronize()
    graph_us = (time.perf_counter() - t0) * 1e6 / args.steps
    flush = torch.empty(512 * 1024 * 1024 // 4, dtype=torch.float32, device="cuda")
    cold = []
    for _ in range(args.cold_steps):
        flush.fill_(1.0)
        a = torch.cuda.Event(enable_timing=True)
        b = torch.cuda.Event(enable_timing=True)
        a.record()
        g.replay()
        b.record()
        b.synchronize()
        cold.append(a.elapsed_time(b) * 1e3)
    cold = np.array(cold)
    del flush
    log(f"graph warm {graph_us:.2f} us/step; cold median {np.median(cold):.2f} us")

    if args.copy_calibration:
        # one elementwise kernel that reads 256 MiB and writes 256 MiB (fp32 x 1.0): the
        # reference for scaling the hardware byte counters of the kernels above
        src = torch.ones(64 * 1024 * 1024, dtype=torch.float32, device="cuda")
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        torch.mul(src, 1.0, out=dst)
        torch.cuda.synchronize()
        del src, dst

    single_launch = None
    if args.single_launch_ab:
        single_launch = single_launch_ab(part_ms.mean() * 1e3, comb_ms.mean() * 1e3,
                                         ms_per_step * 1e3)
        log(f"single-launch A/B: {single_launch}")

    tree_ops = time_tree_ops(w, va, args.steps)
    log(f"tree ops: {tree_ops}")

    by, fl = algorithmic_work(w)
    traffic = (counter_traffic(part_stem, w.name, ["verify_mfma.hip", "va_internal.h"])
               if kernel_name == "mfma" else None)
    part_s = part_ms.mean() * 1e-3
    us = ms_per_step * 1e3
    # the binding roofline of the step: matrix work, or the bytes when few query rows share
    # each key row; the partial kernel moves everything but the output, which the combine
    # writes
    hbm_bound = by / (PEAK_HBM_GBS * 1e9) > fl / (PEAK_MFMA_TFLOPS * 1e12)
    part_bytes = by - w.num_tokens * w.num_heads * 512 * 4
    if hbm_bound:
        achieved, peak, unit = part_bytes / part_s / 1e9, PEAK_HBM_GBS, "GB/s"
    else:
        achieved, peak, unit = fl / part_s / 1e12, PEAK_MFMA_TFLOPS, "TFLOP/s"
    result = {
        "metric": METRIC,
        "value": round(us, 3),
        "unit": "us/step",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "settle_steps": settle_steps,
        "ms_per_step": round(ms_per_step, 6),
        "higher_is_better": False,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": w.in_dtype,
        "data": "synthetic",
        "config": {
            "workload": f"{w.name}: bs={w.bs}, H={w.num_heads}, P={w.prefix_lens.tolist()}, "
                        f"T={w.tree_lens.tolist()} random draft trees, {w.in_dtype} absorbed q "
                        f"[num_tok,H,576] and paged latent KV [{w.num_slots},576]",
            "kernel": kernel_name,
            "num_splits": int(info.num_splits),
            "slot_layout": args.layout,
            "out_dtype": "fp32",
        },
        "effective_GBps": round(by / (us * 1e-6) / 1e9, 2),
        "frac_hbm": round(by / (us * 1e-6) / 1e9 / PEAK_HBM_GBS, 4),
        "frac_mfma_step": round(fl / (us * 1e-6) / 1e12 / PEAK_MFMA_TFLOPS, 4),
        "algorithmic_bytes": int(by),
        "algorithmic_flops": int(fl),
        "partial_kernel_us": round(part_ms.mean() * 1e3, 3),
        "combine_kernel_us": round(comb_ms.mean() * 1e3, 3),
        "graph_warm_us_per_step": round(graph_us, 3),
        "graph_cold_us": {"median": round(float(np.median(cold)), 3),
                          "p10": round(float(np.percentile(cold, 10)), 3),
                          "p90": round(float(np.percentile(cold, 90)), 3)},
        "roofline": {
            "bound": "hbm" if hbm_bound else "mfma",
            "achieved": round(achieved, 3),
            "peak": peak,
            "unit": unit,
            "frac": round(achieved / peak, 4),
            "traffic": traffic,
            "kernel": (f"{part_stem} (split-K partial)" if kernel_name == "mfma"
                       else "simple_partial_kernel (split-K partial)"),
        },
        "tree_ops": tree_ops,
        "cpu_baseline": None,
    }
    if single_launch is not None:
        result["single_launch_ab"] = single_launch
    if args.sweep:
        result["sweep"] = sweep()
    if args.lds_probe:
        result["lds_probe"] = lds_probe()
        log(f"lds probe: {result['lds_probe']}")
    if not args.no_cpu_baseline:
        log("cpu baseline (oracle) ...")
        result["cpu_baseline"] = cpu_baseline(w)
        log(f"cpu baseline: {result['cpu_baseline']['value']:.0f} us/step")
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
