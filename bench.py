#!/usr/bin/env python3
"""Benchmark of the MLA decode hot path on one MI355X.

One step = one pass of the whole path over one batch of synthetic input:
  1. fused dual RMSNorm + per-1x128 FP8 group quant of M tokens (q latent
     [M, 1536] and kv latent [M, 512], strided split views of one [M, 2048]
     bf16 projection buffer), scales in the layout both consumers agreed on;
  2. the block-scaled FP8 GEMMs of the quantised q with W_a [24576, 1536]
     (attention wq_b) and W_b [8192, 1536] (indexer wq_b), sharing the pair;
through mi_fused_normquant_gemm_pair (the default ``--step``): one launch of
both for decode batches up to 16 rows, above that the norm-quant launch
followed by one launch of both GEMMs; ``--step two-launch`` calls the two
entry points (the other form is timed too and reported beside).
Default M = 64 (a decode batch).  Inputs are resident in HBM before the
timed region; every step uses the next of several buffer sets (weights,
activations, outputs) whose total exceeds the 256 MB Infinity Cache, so the
weights stream from HBM as they do in a real decode step ("cold").  The step
is captured once as a HIP graph and replayed.

Prints ONE JSON line.  ``value`` is microseconds per step (lower is better).
``roofline`` is for the kernel that dominates the step, from HIP events
around back-to-back launches of that kernel on the stream it runs on.
``cpu_baseline`` is the CPU oracle timed on this host on one full step.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "norm+FP8-quant µs/call & HBM GB/s (% peak) at M=1/64/8192; FP8 GEMM % MFMA"
HBM_PEAK_GBS = 8000.0          # MI355X HBM3E
FP8_MFMA_PEAK_TFLOPS = 5000.0  # MI355X dense FP8
MALL_BYTES = 256 << 20
COLD_BYTES = 1 << 30           # rotate buffer sets past 1 GiB
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic.json")
# the sources each kernel's code comes from (their hash keys the committed
# counter figures)
NORMQUANT_SOURCES = ("normquant.hip", "normquant_row.h", "device.h", "launch.h")
GEMM_SOURCES = ("gemm_fp8_bs.hip", "normquant_row.h", "device.h", "launch.h")


def parse():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=2000)
    ap.add_argument("--warmup", type=int, default=400)
    ap.add_argument("--M", type=int, default=64, help="tokens per step")
    ap.add_argument("--scale-layout", choices=("row", "col"), default="col")
    ap.add_argument("--weight-layout", choices=("preferred", "row", "tiled"), default="preferred",
                    help="weight byte order (preferred: what mi_preferred_weight_layout says)")
    ap.add_argument("--step", choices=("library", "two-launch"), default="library",
                    help="library: mi_fused_normquant_gemm_pair (one launch where the library takes one); "
                         "two-launch: the norm-quant call, then the GEMM pair call")
    ap.add_argument("--warm", action="store_true", help="reuse one buffer set (cache-warm numbers)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-sweep", action="store_true", help="skip the M=1 / M=8192 / M=256 extras")
    ap.add_argument("--no-warm", action="store_true", help="skip the labelled warm-cache figures")
    ap.add_argument("--kernel-loop", default="", help="only launch this kernel in a loop (profiling)")
    ap.add_argument("--profile-loop", default="",
                    help="comma-separated profiling loops (" + ", ".join(PROFILE_LOOPS) + "), run in turn")
    ap.add_argument("--flush", action="store_true", help="profiling loop nq1: evict the caches between launches")
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="only run a plain 64 MiB device copy in a loop (scales the HBM byte counters)")
    return ap.parse_args()


# --------------------------------------------------------------- helpers

def algorithmic_bytes_normquant(M, Nq=1536, Nkv=512):
    """Bytes the fused norm-quant must move: read q and kv rows (bf16) and
    both gammas once; write codes (1 B), scales (4 B per 128) and kv (bf16)."""
    G = Nq // 128
    return M * (2 * Nq + 2 * Nkv + Nq + 4 * G + 2 * Nkv) + 2 * (Nq + Nkv)


def algorithmic_bytes_single(M, N, normalize):
    """Single-input quant: read x (+ gamma), write codes and scales."""
    return M * N * 2 + M * N + M * (N // 128) * 4 + (N * 2 if normalize else 0)


def algorithmic_bytes_gemm(M, N, K):
    """Weight codes + weight scales + activation codes + activation scales +
    bf16 output, each moved once."""
    return N * K + 4 * (N // 128) * (K // 128) + M * K + 4 * M * (K // 128) + 2 * M * N


def algorithmic_bytes_gemm_pair(M, N1, N2, K):
    """Both weights and their scales, the shared activation pair once, both
    bf16 outputs."""
    return (N1 + N2) * K + 4 * ((N1 + N2) // 128) * (K // 128) + M * K + 4 * M * (K // 128) + 2 * M * (N1 + N2)


def gemm_flops(M, N, K):
    return 2 * M * N * K


def source_sha(*names):
    h = hashlib.sha256()
    for n in names:
        with open(os.path.join(ROOT, "rmsnorm_fp8_block_amd", "csrc", n), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


MEDIANS_FILE = os.path.join(ROOT, "profiles", "kernel_medians.json")
MFMA_FILE = os.path.join(ROOT, "profiles", "mfma_counters.json")


def roofline_frac(flops, nbytes, us):
    """Achieved / min(FP8 MFMA peak, arithmetic intensity x HBM peak), i.e.
    the larger of the two ideal times over the measured time."""
    t_ideal = max(flops / (FP8_MFMA_PEAK_TFLOPS * 1e6), nbytes / (HBM_PEAK_GBS * 1e3))
    return round(t_ideal / us, 4)


def mfma_counters(M, N, e8m0=False):
    """MFMA-busy figures committed under profiles/ (rocprofv3 --pmc
    SQ_VALU_MFMA_BUSY_CYCLES, SQ_INSTS_VALU_MFMA_MOPS_F8, GRBM_GUI_ACTIVE) for
    the GEMM at this shape, if taken on the current kernel source."""
    try:
        with open(MFMA_FILE) as f:
            t = json.load(f)
    except (OSError, ValueError):
        return None
    sha = source_sha(*GEMM_SOURCES)
    for e in t.values():
        if e.get("M") == M and e.get("N") == N and bool(e.get("e8m0")) == e8m0 and e.get("source_sha") == sha:
            return {k: e[k] for k in ("mfma_busy_frac", "mfma_busy_frac_trace", "mfma_busy_cycles",
                                      "gui_active_cycles_per_xcd", "mops_f8") if k in e}
    return None


def kernel_medians(sources):
    """rocprofv3 kernel-trace medians committed under profiles/ for the
    kernel built from these sources (None when the source has changed since
    they were taken)."""
    try:
        with open(MEDIANS_FILE) as f:
            t = json.load(f)
    except (OSError, ValueError):
        return None
    sha = source_sha(*sources)
    out = {k: v for k, v in t.items() if isinstance(v, dict) and v.get("source_sha") == sha}
    return out or None


def measured_traffic(kernel, sha, M):
    """HBM bytes per launch from committed rocprofv3 counter runs, if they
    were taken on the current kernel source at this batch size; else None."""
    try:
        with open(TRAFFIC_FILE) as f:
            t = json.load(f)
    except (OSError, ValueError):
        return None
    for key, e in t.items():
        if e.get("kernel", key) == kernel and e.get("M") == M and e.get("source_sha") == sha:
            return e.get("bytes_per_launch")
    return None


class Timer:
    """HIP events on torch's current stream (the stream every launch below
    goes to)."""

    def __init__(self, torch):
        self.t = torch
        self.a = torch.cuda.Event(enable_timing=True)
        self.b = torch.cuda.Event(enable_timing=True)

    def start(self):
        self.a.record()

    def stop_ms(self):
        self.b.record()
        self.b.synchronize()
        return self.a.elapsed_time(self.b)


def make_graph(torch, fns):
    """Capture the given launches once (warm-up run first, on a side stream
    as torch requires) and return the replayable graph."""
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        for f in fns:
            f()
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for f in fns:
            f()
    torch.cuda.synchronize()
    return g


CHUNK = 2000  # steps per captured graph in the timed region


def capture(torch, fns):
    """Capture the given launches as a graph, with no eager run first (the
    kernels' device set-up is done by mi_init before any capture)."""
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=s):
        for f in fns:
            f()
    torch.cuda.synchronize()
    return g


def time_graph(torch, g, launches_per_replay, replays, warmup=2):
    for _ in range(warmup):
        g.replay()
    torch.cuda.synchronize()
    tm = Timer(torch)
    tm.start()
    for _ in range(replays):
        g.replay()
    ms = tm.stop_ms()
    return 1000.0 * ms / (replays * launches_per_replay)


def time_eager(torch, fns, reps, warmup=3):
    """Back-to-back eager launches cycling through ``fns``; us per launch."""
    for i in range(warmup * len(fns)):
        fns[i % len(fns)]()
    torch.cuda.synchronize()
    tm = Timer(torch)
    tm.start()
    for i in range(reps):
        fns[i % len(fns)]()
    ms = tm.stop_ms()
    return 1000.0 * ms / reps


# ----------------------------------------------------------- workloads

def bf16_dev(torch, np, a, dev):
    return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).to(dev)


def build_sets(torch, np, mi, W, M, layout, wa, wb, nsets, dev, tiled):
    """``nsets`` independent buffer sets for the full step (device copies of
    the same seeded inputs), each with its own outputs.  ``tiled``: the
    weights are stored in the library's tiled layout (the load-time
    relayout, done here once, outside any timed region)."""
    case = W.producer_activations(M) if M <= 256 else W.strided_batch(M)
    buf0 = bf16_dev(torch, np, case.buffer, dev)
    gq = bf16_dev(torch, np, case.gamma_q, dev)
    gk = bf16_dev(torch, np, case.gamma_kv, dev)
    wa_c0 = torch.from_numpy(wa.codes).to(dev)
    wa_s0 = torch.from_numpy(wa.scale).to(dev)
    wb_c0 = torch.from_numpy(wb.codes).to(dev)
    wb_s0 = torch.from_numpy(wb.scale).to(dev)
    if tiled:
        wa_c0, wb_c0 = mi.relayout_weight(wa_c0), mi.relayout_weight(wb_c0)

    def copy_weight(w):
        return mi.TiledWeight(w.data.clone(), w.N, w.K) if tiled else w.clone()

    G = W.NQ // 128
    sets = []
    for i in range(nsets):
        buf = buf0 if i == 0 else buf0.clone()
        q, kv = buf[:, :W.NQ], buf[:, W.NQ:]
        oq = torch.empty((M, W.NQ), dtype=torch.uint8, device=dev)
        osc = torch.empty(M * G, dtype=torch.float32, device=dev)
        okv = torch.empty((M, W.NKV), dtype=torch.bfloat16, device=dev)
        scale = osc.as_strided((M, G), (1, M)) if layout else osc.view(M, G)
        wa_c = wa_c0 if i == 0 else copy_weight(wa_c0)
        wb_c = wb_c0 if i == 0 else copy_weight(wb_c0)
        oa = torch.empty((M, wa.codes.shape[0]), dtype=torch.bfloat16, device=dev)
        ob = torch.empty((M, wb.codes.shape[0]), dtype=torch.bfloat16, device=dev)
        sets.append({
            "nq": mi.prepare_fused_dual_rmsnorm_group_quant(q, kv, gq, gk, W.EPS, layout, oq, osc, okv),
            "gp": mi.prepare_block_scaled_fp8_gemm_pair(oq, scale, wa_c, wa_s0, oa, wb_c, wb_s0, ob),
            "ga": mi.prepare_block_scaled_fp8_gemm(oq, scale, wa_c, wa_s0, oa),
            "gb": mi.prepare_block_scaled_fp8_gemm(oq, scale, wb_c, wb_s0, ob),
            "fs": mi.prepare_fused_normquant_gemm_pair(q, kv, gq, gk, W.EPS, layout, wa_c, wa_s0, wb_c, wb_s0,
                                                       oq, osc, okv, oa, ob),
            "out": (oq, osc, okv, oa, ob),
        })
    return sets


def cpu_model():
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def cpu_baseline(np, W, M, layout, wa, wb):
    """The oracle as it stands, on this host, in the same run.
    - Norm-quant legs at M = 1 (decode_single), 64 (strided batch) and 8192
      (prefill): single-threaded and on every core this process may use,
      median of 100 runs (M <= 256) or 5 (M = 8192), as us/call and the
      equivalent GB/s of the same algorithmic bytes as the GPU kernel.
    - The step (``value``): the norm-quant of the step's M rows and both GEMMs
      over all their columns, once, on every core.
    Returns the bench entry and the step's oracle outputs (q codes, scales in
    storage order, kv bf16 bits, both GEMM outputs in fp64)."""
    import ctypes
    import oracle
    oracle.lib()
    try:  # the oracle's OpenMP runtime (gcc's libgomp, loaded with it)
        gomp = ctypes.CDLL("libgomp.so.1")
        set_threads = gomp.omp_set_num_threads
    except OSError:
        set_threads = None
    cores = len(os.sched_getaffinity(0)) if hasattr(os, "sched_getaffinity") else (os.cpu_count() or 1)
    if os.environ.get("OMP_NUM_THREADS", "").isdigit():  # the host's share of CPUs, where it is set
        cores = max(1, min(cores, int(os.environ["OMP_NUM_THREADS"])))
    legs = {}
    for Mx, reps in ((1, 100), (64, 100), (8192, 5)):
        case = W.decode_single() if Mx == 1 else W.strided_batch(Mx) if Mx == 64 else W.prefill(Mx)
        for threads in ((1, cores) if set_threads else (None,)):
            if set_threads:
                set_threads(threads)
            ts = []
            for _ in range(reps):
                t0 = time.perf_counter()
                oracle.dual_rmsnorm_group_quant(case.q, case.kv, case.gamma_q, case.gamma_kv, W.EPS, layout)
                ts.append(time.perf_counter() - t0)
            us = float(np.median(ts)) * 1e6
            legs[f"normquant_M{Mx}_{oracle.num_threads()}t"] = {
                "us_median": round(us, 1), "runs": reps,
                "GB/s": round(algorithmic_bytes_normquant(Mx) / us / 1e3, 3)}
    if set_threads:
        set_threads(cores)
    case = W.producer_activations(M) if M <= 256 else W.strided_batch(M)
    t0 = time.perf_counter()
    r = oracle.dual_rmsnorm_group_quant(case.q, case.kv, case.gamma_q, case.gamma_kv, W.EPS, layout)
    o1 = oracle.block_scaled_fp8_gemm(r["q"], r["scale"], layout, wa.codes, wa.scale)
    o2 = oracle.block_scaled_fp8_gemm(r["q"], r["scale"], layout, wb.codes, wb.scale)
    dt = time.perf_counter() - t0
    flops = gemm_flops(M, wa.codes.shape[0] + wb.codes.shape[0], W.NQ)
    entry = {"value": round(dt * 1e6, 1), "unit": "µs/step", "cores": oracle.num_threads(), "kind": "oracle",
             "sample": f"one full step at M={M}: fp64 norm-quant of {M} rows + both GEMMs over all "
                       f"{wa.codes.shape[0] + wb.codes.shape[0]} output columns ({dt:.1f} s wall, "
                       f"{flops / dt / 1e9:.2f} GFLOP/s), on {oracle.num_threads()} threads; norm-quant legs "
                       "below: median of 100 runs (M <= 64) or 5 (M = 8192), 1 thread and all threads",
             "cpu_model": cpu_model(), "host_cpus_usable": cores, "legs": legs}
    return entry, (r["q"], r["scale"], r["kv"], o1, o2)


def sign_magnitude_ord(bits, np, sign_bit):
    """Signed-magnitude bit patterns (e4m3 codes, bf16 bits) mapped to
    integers in value order, so that neighbouring representable values
    differ by 1 (+0 and -0 both map to 0)."""
    b = bits.astype(np.int64)
    mag = b & (sign_bit - 1)
    return np.where(b & sign_bit, -mag, mag)


def parity_stats(np, got, ref):
    """The step's outputs on the device (buffer set 0, the same inputs as
    the oracle's) against the oracle's: fraction of identical q codes and
    the largest e4m3 step between them, the largest relative scale error,
    the largest kv difference in bf16 steps, and each GEMM output's relative
    Frobenius and max errors (max |out - ref| / max |ref|)."""
    gq, gs, gkv, g1, g2 = got
    rq, rs, rkv, r1, r2 = ref
    dq = np.abs(sign_magnitude_ord(gq, np, 0x80) - sign_magnitude_ord(rq, np, 0x80))
    dk = np.abs(sign_magnitude_ord(gkv, np, 0x8000) - sign_magnitude_ord(rkv, np, 0x8000))
    rel = np.abs(gs.astype(np.float64) / rs.astype(np.float64) - 1.0)
    out = {"q_codes_exact": round(float((dq == 0).mean()), 6), "q_codes_max_ulp": int(dq.max()),
           "scale_max_rel": float(rel.max()), "kv_exact": round(float((dk == 0).mean()), 6),
           "kv_max_ulp": int(dk.max())}
    for name, o, r in (("W_a", g1, r1), ("W_b", g2, r2)):
        fro = float(np.linalg.norm(o - r) / max(np.linalg.norm(r), 1e-300))
        mx = float(np.abs(o - r).max() / max(np.abs(r).max(), 1e-300))
        out[f"gemm_{name}_rel_fro"] = float(f"{fro:.3e}")
        out[f"gemm_{name}_rel_max"] = float(f"{mx:.3e}")
    return out


def sweep(torch, np, mi, W, wa, wb, dev, cold, tiled):
    """Extra figures of the metric: norm-quant at M=1 and M=256 (us/call) and
    M=8192 (GB/s, both layouts); the single-input quantisations at [8192, 1536] and
    [256, 7168] (GB/s); the GEMMs at M=256 (TFLOP/s, % of FP8 MFMA peak) and at
    tensor-parallel shard shapes, with the step's weight layout (``tiled``),
    and the pair / W_a in both layouts, timed back to back."""
    res = {}
    gq = bf16_dev(torch, np, W.gammas()[0], dev)
    gk = bf16_dev(torch, np, W.gammas()[1], dev)
    # M = 1: latency.  Many tiny buffer sets, one launch each, in a graph.
    one = W.decode_single()
    q1 = bf16_dev(torch, np, one.q, dev)
    k1 = bf16_dev(torch, np, one.kv, dev)
    fns = []
    for i in range(64):
        q = q1.clone()
        k = k1.clone()
        fns.append(mi.prepare_fused_dual_rmsnorm_group_quant(
            q, k, gq, gk, W.EPS, False, torch.empty(1536, dtype=torch.uint8, device=dev),
            torch.empty(12, dtype=torch.float32, device=dev),
            torch.empty(512, dtype=torch.bfloat16, device=dev)))
    g = make_graph(torch, fns)
    res["normquant_M1"] = {
        "us_per_call_graph": round(time_graph(torch, g, len(fns), 20), 3),
        "us_per_call_eager": round(time_eager(torch, fns, 2000), 3),
        "cache": "warm (64 sets of 10.8 KB: Infinity Cache and L2 resident, as the decode step's freshly "
                 "written latents are)",
        "rocprof_median_us": kernel_medians(NORMQUANT_SOURCES)}
    del g, fns
    # M = 256 (a batch of 256 tokens: the outlier workload's rows),
    # column-major scales, many buffer sets in one graph
    case = W.outlier_stress(256)
    b256 = bf16_dev(torch, np, np.concatenate([case.q, case.kv], axis=1), dev)
    fns = []
    for i in range(32):
        b = b256 if i == 0 else b256.clone()
        fns.append(mi.prepare_fused_dual_rmsnorm_group_quant(
            b[:, :W.NQ], b[:, W.NQ:], gq, gk, W.EPS, True,
            torch.empty((256, 1536), dtype=torch.uint8, device=dev),
            torch.empty(256 * 12, dtype=torch.float32, device=dev),
            torch.empty((256, 512), dtype=torch.bfloat16, device=dev)))
    g = make_graph(torch, fns)
    us = time_graph(torch, g, len(fns), 20)
    res["normquant_M256_col"] = {"us": round(us, 3), "GB/s": round(algorithmic_bytes_normquant(256) / us / 1e3, 1),
                                 "cache": "warm (32 sets of 1.7 MB: Infinity Cache resident)"}
    del g, fns, b256
    # M = 8192 prefill, both layouts
    pre = W.prefill(8192)
    bufp = bf16_dev(torch, np, pre.buffer, dev)
    nbytes = algorithmic_bytes_normquant(8192)
    nsets = max(1, COLD_BYTES // nbytes + 1) if cold else 1
    for layout in (0, 1):
        fns = []
        for i in range(nsets):
            b = bufp if i == 0 else bufp.clone()
            fns.append(mi.prepare_fused_dual_rmsnorm_group_quant(
                b[:, :W.NQ], b[:, W.NQ:], gq, gk, W.EPS, layout,
                torch.empty((8192, 1536), dtype=torch.uint8, device=dev),
                torch.empty(8192 * 12, dtype=torch.float32, device=dev),
                torch.empty((8192, 512), dtype=torch.bfloat16, device=dev)))
        g = make_graph(torch, fns)
        us = time_graph(torch, g, len(fns), max(1, 200 // len(fns)))
        gbs = nbytes / us / 1e3
        lay = "col" if layout else "row"
        res[f"normquant_M8192_{lay}"] = {
            "us": round(us, 3), "GB/s": round(gbs, 1), "frac_hbm": round(gbs / HBM_PEAK_GBS, 4),
            "traffic": measured_traffic(f"fused_dual_rmsnorm_group_quant_{lay}", source_sha(*NORMQUANT_SOURCES),
                                        8192)}
        del g, fns
        torch.cuda.empty_cache()
    del bufp
    # single-input forms: RMSNorm + quant and the norm-less quant, column-major scales
    for M, N in ((8192, 1536), (256, 7168)):
        x0, gam = W.single_input(M, N)
        xd0 = bf16_dev(torch, np, x0, dev)
        gd = bf16_dev(torch, np, gam, dev)
        for normalize in (True, False):
            nbytes = algorithmic_bytes_single(M, N, normalize)
            nsets = max(1, COLD_BYTES // nbytes + 1) if cold else 1
            fns = []
            for i in range(nsets):
                xd = xd0 if i == 0 else xd0.clone()
                oq = torch.empty((M, N), dtype=torch.uint8, device=dev)
                osc = torch.empty(M * (N // 128), dtype=torch.float32, device=dev)
                fns.append(mi.prepare_rmsnorm_group_quant(xd, gd, W.EPS, True, oq, osc) if normalize
                           else mi.prepare_group_quant_1x128(xd, True, oq, osc))
            g = make_graph(torch, fns)
            us = time_graph(torch, g, len(fns), max(1, 200 // len(fns)))
            gbs = nbytes / us / 1e3
            res[f"{'rmsnorm_quant' if normalize else 'quant_1x128'}_M{M}_N{N}_col"] = {
                "us": round(us, 3), "GB/s": round(gbs, 1), "frac_hbm": round(gbs / HBM_PEAK_GBS, 4)}
            del g, fns
            torch.cuda.empty_cache()
    # weights in the given layout (tiled: the load-time relayout, done once here)
    def dev_weight(codes, as_tiled):
        w = torch.from_numpy(np.ascontiguousarray(codes)).to(dev)
        return mi.relayout_weight(w) if as_tiled else w

    def copy_weight(w):
        return mi.TiledWeight(w.data.clone(), w.N, w.K) if isinstance(w, mi.TiledWeight) else w.clone()

    # both weight layouts back to back at the same point of the run (timings
    # drift with the position in a long run, so only adjacent figures are
    # compared): the pair at M = 1 / 64 and W_a at M = 256
    was_d, wbs_d = torch.from_numpy(wa.scale).to(dev), torch.from_numpy(wb.scale).to(dev)
    NA, NB = wa.codes.shape[0], wb.codes.shape[0]
    for M in (1, 64, 256):
        a = torch.randint(0, 0x78, (M, 1536), dtype=torch.uint8, device=dev)
        asc = (torch.rand((12, M), dtype=torch.float32, device=dev) + 0.5).T
        per = algorithmic_bytes_gemm_pair(M, NA, NB, 1536) if M <= 64 else algorithmic_bytes_gemm(M, NA, 1536)
        nsets = max(1, COLD_BYTES // per + 1) if cold else 1
        for lay in ("rowmajor", "tiled"):
            wat0 = dev_weight(wa.codes, lay == "tiled")
            wbt0 = dev_weight(wb.codes, lay == "tiled") if M <= 64 else None
            fns = []
            for i in range(nsets):
                wat = wat0 if i == 0 else copy_weight(wat0)
                oa = torch.empty((M, NA), dtype=torch.bfloat16, device=dev)
                if M <= 64:
                    wbt = wbt0 if i == 0 else copy_weight(wbt0)
                    ob = torch.empty((M, NB), dtype=torch.bfloat16, device=dev)
                    fns.append(mi.prepare_block_scaled_fp8_gemm_pair(a, asc, wat, was_d, oa, wbt, wbs_d, ob))
                else:
                    fns.append(mi.prepare_block_scaled_fp8_gemm(a, asc, wat, was_d, oa))
            g = make_graph(torch, fns)
            us = time_graph(torch, g, len(fns), max(1, 200 // len(fns)))
            key = f"{lay}_pair_M{M}" if M <= 64 else f"{lay}_W_a_M{M}"
            res[key] = {"us": round(us, 3), "GB/s": round(per / us / 1e3, 1),
                        "frac_hbm": round(per / us / 1e3 / HBM_PEAK_GBS, 4)}
            del g, fns, wat0, wbt0
            torch.cuda.empty_cache()
    # tensor-parallel shards: rank r holds N/TP rows of W_a and W_b; the pair
    # launch at decode sizes and at M = 256, and the W_a shard alone at M = 256
    for tp in (2, 4, 8):
        na, nb = wa.codes.shape[0] // tp, wb.codes.shape[0] // tp
        wac0, was = dev_weight(wa.codes[:na], tiled), torch.from_numpy(wa.scale[:na // 128]).to(dev)
        wbc0, wbs = dev_weight(wb.codes[:nb], tiled), torch.from_numpy(wb.scale[:nb // 128]).to(dev)
        for M, pair in ((1, True), (16, True), (64, True), (256, False), (256, True)):
            a = torch.randint(0, 0x78, (M, 1536), dtype=torch.uint8, device=dev)
            asc = (torch.rand((12, M), dtype=torch.float32, device=dev) + 0.5).T   # column-major
            per = (algorithmic_bytes_gemm_pair(M, na, nb, 1536) if pair
                   else algorithmic_bytes_gemm(M, na, 1536))
            nsets = max(1, COLD_BYTES // per + 1) if cold else 1
            fns = []
            for i in range(nsets):
                wac = wac0 if i == 0 else copy_weight(wac0)
                oa = torch.empty((M, na), dtype=torch.bfloat16, device=dev)
                if pair:
                    wbc = wbc0 if i == 0 else copy_weight(wbc0)
                    ob = torch.empty((M, nb), dtype=torch.bfloat16, device=dev)
                    fns.append(mi.prepare_block_scaled_fp8_gemm_pair(a, asc, wac, was, oa, wbc, wbs, ob))
                else:
                    fns.append(mi.prepare_block_scaled_fp8_gemm(a, asc, wac, was, oa))
            g = make_graph(torch, fns)
            us = time_graph(torch, g, len(fns), max(1, 200 // len(fns)))
            key = f"tp{tp}_pair_M{M}" if pair else f"tp{tp}_W_a_M{M}"
            res[key] = {"N": [na, nb] if pair else na, "us": round(us, 3), "GB/s": round(per / us / 1e3, 1),
                        "frac_hbm": round(per / us / 1e3 / HBM_PEAK_GBS, 4)}
            if pair and M > 64:   # the pair's own launches (the step's count less the norm-quant's)
                res[key]["launches"] = mi.mi_fused_normquant_gemm_pair_launches(M, W.NQ, W.NKV, na, nb) - 1
            del g, fns
        del wac0, wbc0
        torch.cuda.empty_cache()
    # e8m0 (power-of-two) scales: the whole step at M = 64 (norm-quant + pair),
    # and the GEMMs at M = 256, weights tiled
    ea = W.block_fp8_weight_e8m0(*W.W_A_SHAPE, W.W_A_SEED)
    eb = W.block_fp8_weight_e8m0(*W.W_B_SHAPE, W.W_B_SEED)
    eac0, ebc0 = dev_weight(ea.codes, True), dev_weight(eb.codes, True)
    eas, ebs = torch.from_numpy(ea.scale).to(dev), torch.from_numpy(eb.scale).to(dev)
    NA, NB = ea.codes.shape[0], eb.codes.shape[0]
    M = 64
    case = W.producer_activations(M)
    buf0 = bf16_dev(torch, np, case.buffer, dev)
    gq, gk = bf16_dev(torch, np, case.gamma_q, dev), bf16_dev(torch, np, case.gamma_kv, dev)
    per = algorithmic_bytes_normquant(M) - 3 * M * 12 + algorithmic_bytes_gemm_pair(M, NA, NB, 1536) - \
        3 * (M * 12 + (NA + NB) // 128 * 12)   # 1-byte scales instead of 4-byte ones
    nsets = max(1, COLD_BYTES // per + 1) if cold else 1
    step_fns, pair_fns = [], []
    for i in range(nsets):
        b = buf0 if i == 0 else buf0.clone()
        oq = torch.empty((M, W.NQ), dtype=torch.uint8, device=dev)
        osc = torch.empty(M * 12, dtype=torch.uint8, device=dev)
        okv = torch.empty((M, W.NKV), dtype=torch.bfloat16, device=dev)
        nq = mi.prepare_fused_dual_rmsnorm_group_quant_e8m0(b[:, :W.NQ], b[:, W.NQ:], gq, gk, W.EPS, True, oq, osc, okv)
        wac = eac0 if i == 0 else copy_weight(eac0)
        wbc = ebc0 if i == 0 else copy_weight(ebc0)
        oa = torch.empty((M, NA), dtype=torch.bfloat16, device=dev)
        ob = torch.empty((M, NB), dtype=torch.bfloat16, device=dev)
        gp = mi.prepare_block_scaled_fp8_gemm_pair(oq, osc.as_strided((M, 12), (1, M)), wac, eas, oa, wbc, ebs, ob)
        step_fns += [nq, gp]
        pair_fns.append(gp)
    g = make_graph(torch, step_fns)
    res["e8m0_step_M64_us"] = round(time_graph(torch, g, nsets, max(1, 200 // nsets)), 3)
    del g
    g = make_graph(torch, pair_fns)
    us = time_graph(torch, g, nsets, max(1, 200 // nsets))
    pb = algorithmic_bytes_gemm_pair(M, NA, NB, 1536) - 3 * (M * 12 + (NA + NB) // 128 * 12)
    res["e8m0_pair_M64"] = {"us": round(us, 3), "GB/s": round(pb / us / 1e3, 1),
                            "frac_hbm": round(pb / us / 1e3 / HBM_PEAK_GBS, 4)}
    del g, step_fns, pair_fns
    torch.cuda.empty_cache()
    # ... and at M = 16 through the one-call step (one launch) and as the two calls
    M = 16
    case = W.producer_activations(M)
    buf0 = bf16_dev(torch, np, case.buffer, dev)
    per = algorithmic_bytes_normquant(M) - 3 * M * 12 + algorithmic_bytes_gemm_pair(M, NA, NB, 1536) - \
        3 * (M * 12 + (NA + NB) // 128 * 12)
    nsets = max(2, COLD_BYTES // per + 1) if cold else 1
    one_fns, two_fns = [], []
    for i in range(nsets):
        b = buf0 if i == 0 else buf0.clone()
        oq = torch.empty((M, W.NQ), dtype=torch.uint8, device=dev)
        osc = torch.empty(M * 12, dtype=torch.uint8, device=dev)
        okv = torch.empty((M, W.NKV), dtype=torch.bfloat16, device=dev)
        wac = eac0 if i == 0 else copy_weight(eac0)
        wbc = ebc0 if i == 0 else copy_weight(ebc0)
        oa = torch.empty((M, NA), dtype=torch.bfloat16, device=dev)
        ob = torch.empty((M, NB), dtype=torch.bfloat16, device=dev)
        one_fns.append(mi.prepare_fused_normquant_gemm_pair(b[:, :W.NQ], b[:, W.NQ:], gq, gk, W.EPS, True, wac, eas,
                                                            wbc, ebs, oq, osc, okv, oa, ob))
        two_fns += [mi.prepare_fused_dual_rmsnorm_group_quant_e8m0(b[:, :W.NQ], b[:, W.NQ:], gq, gk, W.EPS, True,
                                                                   oq, osc, okv),
                    mi.prepare_block_scaled_fp8_gemm_pair(oq, osc.as_strided((M, 12), (1, M)), wac, eas, oa, wbc,
                                                          ebs, ob)]
    entry = {"launches": mi.mi_fused_normquant_gemm_pair_launches(M, W.NQ, W.NKV, NA, NB)}
    for name, fns in (("us", one_fns), ("two_calls_us", two_fns)):
        g = make_graph(torch, fns)
        entry[name] = round(time_graph(torch, g, nsets, max(1, 200 // nsets)), 3)
        del g
    res["e8m0_step_M16"] = entry
    del one_fns, two_fns
    torch.cuda.empty_cache()
    M = 256
    a = torch.randint(0, 0x78, (M, 1536), dtype=torch.uint8, device=dev)
    asc = torch.randint(118, 127, (12, M), dtype=torch.uint8, device=dev).T
    for name, wc0, ws, N in (("W_a", eac0, eas, NA), ("W_b", ebc0, ebs, NB)):
        perg = algorithmic_bytes_gemm(M, N, 1536) - 3 * (M * 12 + N // 128 * 12)
        nsets = max(1, COLD_BYTES // perg + 1) if cold else 1
        fns = []
        for i in range(nsets):
            wc = wc0 if i == 0 else copy_weight(wc0)
            fns.append(mi.prepare_block_scaled_fp8_gemm(a, asc, wc, ws, torch.empty((M, N), dtype=torch.bfloat16,
                                                                                      device=dev)))
        g = make_graph(torch, fns)
        us = time_graph(torch, g, len(fns), max(1, 200 // len(fns)))
        tf = gemm_flops(M, N, 1536) / us / 1e6
        res[f"e8m0_gemm_{name}_M256"] = {"us": round(us, 3), "TFLOP/s": round(tf, 1),
                                         "frac_fp8_mfma": round(tf / FP8_MFMA_PEAK_TFLOPS, 4),
                                         "GB/s": round(perg / us / 1e3, 1),
                                         "roofline_frac": roofline_frac(gemm_flops(M, N, 1536), perg, us),
                                         "mfma_counters": mfma_counters(M, N, e8m0=True),
                                         "traffic": measured_traffic(f"block_scaled_fp8_gemm_{name}_e8m0",
                                                                     source_sha(*GEMM_SOURCES), M)}
        del g, fns
    del eac0, ebc0
    torch.cuda.empty_cache()
    # GEMMs at M = 256
    M = 256
    a = torch.randint(0, 0x78, (M, 1536), dtype=torch.uint8, device=dev)
    asc = torch.rand((M, 12), dtype=torch.float32, device=dev) + 0.5
    for name, wt in (("W_a", wa), ("W_b", wb)):
        N, K = wt.codes.shape
        wc0 = dev_weight(wt.codes, tiled)
        ws = torch.from_numpy(wt.scale).to(dev)
        per = algorithmic_bytes_gemm(M, N, K)
        nsets = max(1, COLD_BYTES // per + 1) if cold else 1
        fns = []
        for i in range(nsets):
            wc = wc0 if i == 0 else copy_weight(wc0)
            fns.append(mi.prepare_block_scaled_fp8_gemm(
                a, asc, wc, ws, torch.empty((M, N), dtype=torch.bfloat16, device=dev)))
        g = make_graph(torch, fns)
        us = time_graph(torch, g, len(fns), max(1, 200 // len(fns)))
        tf = gemm_flops(M, N, K) / us / 1e6
        res[f"gemm_{name}_M256"] = {"us": round(us, 3), "TFLOP/s": round(tf, 1),
                                    "frac_fp8_mfma": round(tf / FP8_MFMA_PEAK_TFLOPS, 4),
                                    "GB/s": round(per / us / 1e3, 1),
                                    "roofline_frac": roofline_frac(gemm_flops(M, N, K), per, us),
                                    "mfma_counters": mfma_counters(M, N),
                                    "traffic": measured_traffic(f"block_scaled_fp8_gemm_{name}",
                                                                source_sha(*GEMM_SOURCES), M)}
        del g, fns
        torch.cuda.empty_cache()

    # the step at other batch sizes, in the form the library picks (one
    # launch up to 16 rows) and as the two calls, back to back
    for M in (1, 16, 256):
        per = algorithmic_bytes_normquant(M) + algorithmic_bytes_gemm_pair(M, W.W_A_SHAPE[0], W.W_B_SHAPE[0], W.NQ)
        nsets = max(2, COLD_BYTES // per + 1) if cold else 1
        sets = build_sets(torch, np, mi, W, M, 1, wa, wb, nsets, dev, tiled)
        entry = {"launches": mi.mi_fused_normquant_gemm_pair_launches(M, W.NQ, W.NKV, W.W_A_SHAPE[0],
                                                                      W.W_B_SHAPE[0])}
        for name, keys in (("us", ["fs"]), ("two_calls_us", ["nq", "gp"])):
            g = make_graph(torch, [st[k] for st in sets for k in keys])
            entry[name] = round(time_graph(torch, g, nsets, max(1, 200 // nsets)), 3)
            del g
        res[f"step_M{M}"] = entry
        del sets
        torch.cuda.empty_cache()
    return res


def time_ceiling(torch, fns, replays=20):
    """A ceiling timed like the kernels it bounds: its launches captured in
    one graph (after an eager warm-up), us per launch over the replays."""
    g = make_graph(torch, fns)
    us = time_graph(torch, g, len(fns), replays)
    del g
    return us


def ceilings(torch, np, W):
    """Measured data-movement ceilings of this GPU for the kernels' access
    patterns (libmi_ceiling.so: hand-written skeletons that move the same
    bytes with no arithmetic), cold (buffer sets rotated past 2x the Infinity
    Cache), HIP events around graph replays (as the kernels are timed):
      normquant_M8192: the dual norm-quant's reads and writes at 8192 rows;
      weight_stream_{W_a,W_b,pair}: every weight byte of the GEMM read once
      from HBM into LDS by 256 workgroups (the floor of any GEMM kernel
      that streams that weight, before activations and outputs);
      mfma[_fold]_{W_a,W_b}_M256: the GEMM's 16x16x128 FP8 MFMAs at M = 256
      (W_a: 256 workgroups x 12 waves x 96, W_b: 256 x 4 x 96) on register
      operands, no memory traffic, with the fp32-scale fold or accumulating
      in place (e8m0): the matrix-core floor at the clock the chip holds,
      whose waves' shader-clock / real-time counters give that clock
      (`shader_clock_GHz`: 5th, 50th, 95th percentile over the waves)."""
    import ctypes
    lib = ctypes.CDLL(os.path.join(ROOT, "rmsnorm_fp8_block_amd", "libmi_ceiling.so"))
    p, i64 = ctypes.c_void_p, ctypes.c_int64
    lib.mi_ceiling_normquant_skeleton.argtypes = [p, i64, p, p, p, i64, p]
    lib.mi_ceiling_weight_stream.argtypes = [p, i64, i64, p, p]
    lib.mi_ceiling_mfma.argtypes = [i64, ctypes.c_int, i64, ctypes.c_int, ctypes.c_float, p, p, p]
    dev = torch.device("cuda:0")
    stream = lambda: ctypes.c_void_p(torch.cuda.current_stream(dev).cuda_stream)
    res = {}
    M = 8192
    nbytes = algorithmic_bytes_normquant(M)
    sets = []
    for _ in range(2 * MALL_BYTES // nbytes + 2):
        sets.append((torch.empty((M, 2048), dtype=torch.bfloat16, device=dev).normal_(),
                     torch.empty((M, 1536), dtype=torch.uint8, device=dev),
                     torch.empty(M * 12, dtype=torch.float32, device=dev),
                     torch.empty((M, 512), dtype=torch.bfloat16, device=dev)))

    def nq(i):
        b, q, sc, kv = sets[i % len(sets)]
        st = lib.mi_ceiling_normquant_skeleton(b.data_ptr(), 2048, q.data_ptr(), sc.data_ptr(), kv.data_ptr(), M,
                                               stream())
        if st != 0:
            raise RuntimeError(f"mi_ceiling_normquant_skeleton: hip error {st}")
    fns = [lambda i=i: nq(i) for i in range(len(sets))]
    us = time_ceiling(torch, fns)
    res["normquant_M8192"] = {"us": round(us, 3), "GB/s": round(nbytes / us / 1e3, 1),
                              "frac_hbm": round(nbytes / us / 1e3 / HBM_PEAK_GBS, 4),
                              "what": "dual norm-quant data movement at 8192 rows (reads 4096 B and writes 2608 B "
                                      "per row, the kernel's launch shape and store widths, no arithmetic)"}
    del sets, fns
    torch.cuda.empty_cache()
    sink = torch.zeros(4, dtype=torch.int32, device=dev)
    for name, n in (("W_a", W.W_A_SHAPE[0]), ("W_b", W.W_B_SHAPE[0]), ("pair", W.W_A_SHAPE[0] + W.W_B_SHAPE[0]),
                    ("tp8_pair", (W.W_A_SHAPE[0] + W.W_B_SHAPE[0]) // 8), ("tp8_W_a", W.W_A_SHAPE[0] // 8)):
        wbytes = n * W.NQ
        # the most workgroups (at most one per CU) that split the weight into
        # whole 4 KB stages
        blocks = next(b for b in range(256, 0, -1) if wbytes % (b * 4096) == 0)
        slab = wbytes // blocks
        bufs = [torch.empty(wbytes, dtype=torch.uint8, device=dev).fill_(1)
                for _ in range(2 * MALL_BYTES // wbytes + 2)]

        def ws(i, bufs=bufs, slab=slab, blocks=blocks):
            st = lib.mi_ceiling_weight_stream(bufs[i % len(bufs)].data_ptr(), slab, blocks, sink.data_ptr(), stream())
            if st != 0:
                raise RuntimeError(f"mi_ceiling_weight_stream: hip error {st}")
        fns = [lambda i=i: ws(i) for i in range(len(bufs))]
        us = time_ceiling(torch, fns)
        res[f"weight_stream_{name}"] = {"us": round(us, 3), "bytes": wbytes, "workgroups": blocks,
                                        "GB/s": round(wbytes / us / 1e3, 1),
                                        "frac_hbm": round(wbytes / us / 1e3 / HBM_PEAK_GBS, 4)}
        del bufs, fns
        torch.cuda.empty_cache()
    msink = torch.zeros(1024, dtype=torch.float32, device=dev)
    for name, blocks, waves, per_wave in (("W_a_M256", 256, 12, 96), ("W_b_M256", 256, 4, 96)):
        for fold in (True, False):
            def mf(blocks=blocks, waves=waves, per_wave=per_wave, fold=fold, clocks=None):
                st = lib.mi_ceiling_mfma(blocks, waves, per_wave, int(fold), 1.0, msink.data_ptr(),
                                         None if clocks is None else clocks.data_ptr(), stream())
                if st != 0:
                    raise RuntimeError(f"mi_ceiling_mfma: hip error {st}")
            us = time_ceiling(torch, [mf] * 20)
            flops = blocks * waves * per_wave * 16 * 16 * 128 * 2
            entry = {"us": round(us, 3), "mfmas": blocks * waves * per_wave, "launch": [blocks, waves, per_wave],
                     "TFLOP/s": round(flops / us / 1e6, 1),
                     "frac_fp8_peak": round(flops / us / 1e6 / FP8_MFMA_PEAK_TFLOPS, 4)}
            # one more launch (eager, after the timed ones) with the waves' clock
            # counters: shader cycles over 100 MHz real time
            clocks = torch.zeros(4 * blocks * waves, dtype=torch.int64, device=dev)
            mf(clocks=clocks)
            torch.cuda.synchronize()
            c = clocks.view(-1, 4).cpu().numpy().astype(np.float64)
            ok = c[:, 3] > c[:, 1]
            if ok.any():
                ghz = (c[ok, 2] - c[ok, 0]) / (c[ok, 3] - c[ok, 1]) * 0.1
                entry["shader_clock_GHz"] = [round(float(np.percentile(ghz, q)), 3) for q in (5, 50, 95)]
            res[f"mfma{'_fold' if fold else ''}_{name}"] = entry
    return res


PROFILE_LOOPS = ("nq1", "nq8192_row", "nq8192_col", "gemm_a256", "gemm_b256", "gemm_a256_e8m0",
                 "gemm_b256_e8m0", "pair64", "tp8pair1")


def profile_loops(torch, np, mi, W, names, steps, tiled, flush):
    """Profiling aid: for each named loop in turn, ``steps`` back-to-back
    launches of one kernel over buffer sets rotated past twice the Infinity
    Cache (cold), after 3 untimed rounds; prints one JSON line per loop with
    its launch order, so a rocprofv3 trace of the run splits by position.
      nq1           dual norm-quant, M = 1 (decode_single); with ``flush`` a
                    512 MiB fill runs between launches so every launch finds
                    its input and weights of RMSNorm out of the caches
      nq8192_row/col  dual norm-quant of the prefill batch, both layouts
      gemm_{a,b}256[_e8m0]  W_a / W_b GEMM at M = 256, fp32 or e8m0 scales
      pair64        both GEMMs at M = 64 (the decode step's pair launch)
      tp8pair1      both GEMMs' tensor-parallel shards at TP = 8 (the last
                    rank's 3072 + 1024 rows), M = 1, one pair launch"""
    dev = torch.device("cuda:0")
    gq = bf16_dev(torch, np, W.gammas()[0], dev)
    gk = bf16_dev(torch, np, W.gammas()[1], dev)

    def cold_sets(nbytes):
        return max(2, (2 * MALL_BYTES) // nbytes + 1)

    def dev_weight(codes):
        w = torch.from_numpy(np.ascontiguousarray(codes)).to(dev)
        return mi.relayout_weight(w) if tiled else w

    def copy_weight(w):
        return mi.TiledWeight(w.data.clone(), w.N, w.K) if isinstance(w, mi.TiledWeight) else w.clone()

    order = 0
    for name in names:
        fns, extra = [], None
        if name == "nq1":
            one = W.decode_single()
            q0, k0 = bf16_dev(torch, np, one.q, dev), bf16_dev(torch, np, one.kv, dev)
            for i in range(64):
                fns.append(mi.prepare_fused_dual_rmsnorm_group_quant(
                    q0.clone(), k0.clone(), gq.clone(), gk.clone(), W.EPS, False,
                    torch.empty(1536, dtype=torch.uint8, device=dev), torch.empty(12, dtype=torch.float32, device=dev),
                    torch.empty(512, dtype=torch.bfloat16, device=dev)))
            if flush:
                junk = torch.empty(512 << 20, dtype=torch.uint8, device=dev)
                extra = lambda: junk.fill_(1)
        elif name.startswith("nq8192"):
            pre = W.prefill(8192)
            b0 = bf16_dev(torch, np, pre.buffer, dev)
            layout = 1 if name.endswith("col") else 0
            for i in range(cold_sets(algorithmic_bytes_normquant(8192))):
                b = b0 if i == 0 else b0.clone()
                fns.append(mi.prepare_fused_dual_rmsnorm_group_quant(
                    b[:, :W.NQ], b[:, W.NQ:], gq, gk, W.EPS, layout,
                    torch.empty((8192, 1536), dtype=torch.uint8, device=dev),
                    torch.empty(8192 * 12, dtype=torch.float32, device=dev),
                    torch.empty((8192, 512), dtype=torch.bfloat16, device=dev)))
        elif name.startswith("gemm_"):
            M = 256
            e8m0 = name.endswith("e8m0")
            shape, seed = (W.W_A_SHAPE, W.W_A_SEED) if name.startswith("gemm_a") else (W.W_B_SHAPE, W.W_B_SEED)
            wt = (W.block_fp8_weight_e8m0 if e8m0 else W.block_fp8_weight)(*shape, seed)
            N, K = shape
            a = torch.randint(0, 0x78, (M, K), dtype=torch.uint8, device=dev)
            asc = (torch.randint(118, 127, (K // 128, M), dtype=torch.uint8, device=dev) if e8m0 else
                   torch.rand((K // 128, M), dtype=torch.float32, device=dev) + 0.5).T
            w0 = dev_weight(wt.codes)
            ws = torch.from_numpy(wt.scale).to(dev)
            for i in range(cold_sets(algorithmic_bytes_gemm(M, N, K))):
                fns.append(mi.prepare_block_scaled_fp8_gemm(
                    a, asc, w0 if i == 0 else copy_weight(w0), ws,
                    torch.empty((M, N), dtype=torch.bfloat16, device=dev)))
        elif name == "pair64":
            sets = build_sets(torch, np, mi, W, 64, 1, W.block_fp8_weight(*W.W_A_SHAPE, W.W_A_SEED),
                              W.block_fp8_weight(*W.W_B_SHAPE, W.W_B_SEED),
                              cold_sets(algorithmic_bytes_gemm_pair(64, W.W_A_SHAPE[0], W.W_B_SHAPE[0], W.NQ)), dev,
                              tiled)
            fns = [st["gp"] for st in sets]
        elif name == "tp8pair1":
            M, K = 1, W.NQ
            wa_full = W.block_fp8_weight(*W.W_A_SHAPE, W.W_A_SEED)
            wb_full = W.block_fp8_weight(*W.W_B_SHAPE, W.W_B_SEED)
            na, nb = W.W_A_SHAPE[0] // 8, W.W_B_SHAPE[0] // 8
            wa0, wb0 = dev_weight(wa_full.codes[-na:]), dev_weight(wb_full.codes[-nb:])
            sa = torch.from_numpy(np.ascontiguousarray(wa_full.scale[-na // 128:])).to(dev)
            sb = torch.from_numpy(np.ascontiguousarray(wb_full.scale[-nb // 128:])).to(dev)
            a = torch.randint(0, 0x78, (M, K), dtype=torch.uint8, device=dev)
            asc = (torch.rand((K // 128, M), dtype=torch.float32, device=dev) + 0.5).T
            for i in range(cold_sets(algorithmic_bytes_gemm_pair(M, na, nb, K))):
                fns.append(mi.prepare_block_scaled_fp8_gemm_pair(
                    a, asc, wa0 if i == 0 else copy_weight(wa0), sa, torch.empty((M, na), dtype=torch.bfloat16,
                                                                                   device=dev),
                    wb0 if i == 0 else copy_weight(wb0), sb, torch.empty((M, nb), dtype=torch.bfloat16, device=dev)))
        else:
            raise SystemExit(f"unknown profile loop {name!r}; known: {', '.join(PROFILE_LOOPS)}")
        seq = []
        for f in fns:
            seq += [extra, f] if extra else [f]
        for i in range(3 * len(seq)):          # untimed rounds
            seq[i % len(seq)]()
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for i in range(steps * (2 if extra else 1)):
            seq[i % len(seq)]()
        torch.cuda.synchronize()
        dt = time.perf_counter() - t0
        print(json.dumps({"profile_loop": name, "first_launch": order, "warmup_launches": 3 * len(fns),
                          "launches": steps, "sets": len(fns), "interleaved_flush": bool(extra),
                          "wall_us_per_launch": round(1e6 * dt / steps, 3)}), flush=True)
        order += 3 * len(fns) + steps
        del fns, seq
        torch.cuda.empty_cache()


def calibrate_copy(torch, steps):
    """A plain device-to-device copy of a known size (64 MiB, rotating over
    16 buffer pairs = 2 GiB so every copy streams from HBM).  Run under
    rocprofv3 --pmc, FETCH_SIZE / WRITE_SIZE per copy divided by 64 MiB give
    the factors that turn those counters into HBM bytes."""
    dev = torch.device("cuda:0")
    n = 64 << 20
    srcs = [torch.empty(n, dtype=torch.uint8, device=dev).random_() for _ in range(16)]
    dsts = [torch.empty(n, dtype=torch.uint8, device=dev) for _ in range(16)]
    fns = [lambda i=i: dsts[i].copy_(srcs[i]) for i in range(16)]
    us = time_eager(torch, fns, steps)
    print(json.dumps({"calibrate_copy_bytes": n, "us_per_copy": round(us, 3),
                      "GB/s(read+write)": round(2 * n / us / 1e3, 1)}), flush=True)


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only (got --gpus {args.gpus}): the path has no cross-GPU step "
              "to measure (norm-quant rows and GEMM columns shard with no exchange)", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    if args.calibrate_copy:
        calibrate_copy(torch, args.steps)
        return

    import rmsnorm_fp8_block_amd as mi
    from rmsnorm_fp8_block_amd import workloads as W

    mi.lib()  # fails loudly if the HIP library is missing
    mi.mi_init()
    if args.profile_loop:
        tiled = args.weight_layout != "row"
        profile_loops(torch, np, mi, W, args.profile_loop.split(","), args.steps, tiled, args.flush)
        return
    dev = torch.device("cuda:0")
    props = torch.cuda.get_device_properties(dev)
    layout = 1 if args.scale_layout == "col" else 0
    M = args.M

    wa = W.block_fp8_weight(*W.W_A_SHAPE, W.W_A_SEED)
    wb = W.block_fp8_weight(*W.W_B_SHAPE, W.W_B_SEED)
    step_bytes = (algorithmic_bytes_normquant(M)
                  + algorithmic_bytes_gemm_pair(M, W.W_A_SHAPE[0], W.W_B_SHAPE[0], W.NQ))
    nsets = 1 if args.warm else max(2, COLD_BYTES // step_bytes + 1)
    if args.weight_layout == "preferred":
        prefs = {mi.mi_preferred_weight_layout(*W.W_A_SHAPE), mi.mi_preferred_weight_layout(*W.W_B_SHAPE)}
        tiled = prefs == {1}
    else:
        tiled = args.weight_layout == "tiled"
    sets = build_sets(torch, np, mi, W, M, layout, wa, wb, nsets, dev, tiled)
    torch.cuda.synchronize()

    if args.kernel_loop:
        # profiling aid: only the named kernel, back to back over the sets
        key = {"normquant": "nq", "gemm_pair": "gp", "gemm_a": "ga", "gemm_b": "gb",
               "step": "fs"}[args.kernel_loop]
        fns = [s[key] for s in sets]
        us = time_eager(torch, fns, args.steps)
        print(json.dumps({"kernel_loop": args.kernel_loop, "M": M, "warmup_launches": 3 * len(fns),
                          "launches": args.steps, "sets": len(fns), "us_per_launch": us}))
        return

    # ---- the timed region: exactly K steps after exactly W untimed ones,
    # step i on buffer set i mod nsets, captured as HIP graphs (at most
    # CHUNK steps per graph) and replayed ----
    def step_graphs(one_launch, n, first):
        """Graphs covering n steps starting at step `first`: (graph, replays)."""
        out, done = [], 0
        while done < n:
            c = min(CHUNK, n - done)
            fns = []
            for i in range(c):
                st = sets[(first + done + i) % nsets]
                fns += [st["fs"]] if one_launch else [st["nq"], st["gp"]]
            out.append(capture(torch, fns))
            done += c
        return out

    def time_steps(one_launch, K, Wm):
        warm = step_graphs(one_launch, Wm, 0)
        timed = step_graphs(one_launch, K, Wm)
        for g in warm:
            g.replay()
        torch.cuda.synchronize()
        tm = Timer(torch)
        tm.start()
        for g in timed:
            g.replay()
        ms = tm.stop_ms()
        torch.cuda.synchronize()
        del warm, timed
        return 1000.0 * ms / K

    launches = mi.mi_fused_normquant_gemm_pair_launches(M, W.NQ, W.NKV, W.W_A_SHAPE[0], W.W_B_SHAPE[0])
    library = args.step == "library"
    steps, warmup_steps = max(1, args.steps), max(0, args.warmup)
    us_step = time_steps(library, steps, warmup_steps)
    us_other = time_steps(not library, steps, warmup_steps)
    one_launch = library and launches == 1

    # ---- per-kernel average launch duration (events around back-to-back
    # launches of one kernel over the same buffer sets, same stream) ----
    kernels = {}
    NA, NB = W.W_A_SHAPE[0], W.W_B_SHAPE[0]
    specs = {
        "fused_dual_rmsnorm_group_quant": ("nq", algorithmic_bytes_normquant(M), None, NORMQUANT_SOURCES),
        "block_scaled_fp8_gemm_pair": ("gp", algorithmic_bytes_gemm_pair(M, NA, NB, W.NQ),
                                       gemm_flops(M, NA + NB, W.NQ), GEMM_SOURCES),
        "block_scaled_fp8_gemm_W_a": ("ga", algorithmic_bytes_gemm(M, *W.W_A_SHAPE),
                                      gemm_flops(M, *W.W_A_SHAPE), GEMM_SOURCES),
        "block_scaled_fp8_gemm_W_b": ("gb", algorithmic_bytes_gemm(M, *W.W_B_SHAPE),
                                      gemm_flops(M, *W.W_B_SHAPE), GEMM_SOURCES),
        "normquant_gemm_pair": ("fs", algorithmic_bytes_normquant(M) + algorithmic_bytes_gemm_pair(M, NA, NB, W.NQ),
                                gemm_flops(M, NA + NB, W.NQ), GEMM_SOURCES),
    }
    if launches != 1:
        del specs["normquant_gemm_pair"]  # the call is the two kernels above
    for name, (key, nbytes, flops, src) in specs.items():
        fns = [s[key] for s in sets]
        gk = make_graph(torch, fns)
        us = time_graph(torch, gk, len(fns), max(2, 400 // len(fns)))
        del gk
        gbs = nbytes / us / 1e3
        k = {"us": round(us, 3), "bytes": nbytes, "GB/s": round(gbs, 1),
             "frac_hbm": round(gbs / HBM_PEAK_GBS, 4), "source_sha": source_sha(*src)}
        # what this loop's rotation touches: under the Infinity Cache size,
        # its operands stay cache-resident (the step itself stays cold: the
        # weights rotate past 1 GiB)
        footprint = len(fns) * nbytes
        rotation = f"{len(fns)} sets, {footprint / 2**20:.1f} MiB in all"
        k["cache"] = ("cold" if footprint > 2 * MALL_BYTES else
                      f"partly warm ({rotation}: within twice the 256 MiB Infinity Cache)" if footprint > MALL_BYTES
                      else f"warm ({rotation}: Infinity Cache resident)")
        if flops:
            k["TFLOP/s"] = round(flops / us / 1e6, 2)
        k["traffic"] = measured_traffic(name, k["source_sha"], M)
        kernels[name] = k
    # the dominant kernel of the step (the single-consumer GEMMs are listed
    # for reference only: the step runs the pair)
    dom = ("normquant_gemm_pair" if one_launch else
           max(("fused_dual_rmsnorm_group_quant", "block_scaled_fp8_gemm_pair"), key=lambda n: kernels[n]["us"]))
    dk = kernels[dom]
    roofline = {"bound": "hbm", "achieved": dk["GB/s"], "peak": HBM_PEAK_GBS, "unit": "GB/s",
                "frac": dk["frac_hbm"], "traffic": dk["traffic"],
                "kernel": dom, "bytes_per_launch": dk["bytes"], "us_per_launch": dk["us"]}
    # the committed rocprofv3 kernel-trace median of the same kernel source
    # and launch (profile loop pair64: the pair at 64 rows, cold), beside the
    # events figure, which also holds the gap between back-to-back launches
    med = kernel_medians(GEMM_SOURCES) if dom == "block_scaled_fp8_gemm_pair" and M == 64 else None
    if med and "pair64" in med:
        roofline["rocprof_median_us"] = med["pair64"]["median_us"]
        roofline["frac_rocprof_median"] = round(dk["bytes"] / med["pair64"]["median_us"] / 1e3 / HBM_PEAK_GBS, 4)

    line = {
        "metric": METRIC,
        "value": round(us_step, 3),
        "unit": "µs/call",
        "n_gpus": 1,
        "steps": steps,
        "warmup": warmup_steps,
        "ms_per_step": round(us_step / 1000.0, 6),
        "higher_is_better": False,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32 norm, e4m3 x e4m3 -> f32 MFMA",
        "data": "synthetic",
        "config": {
            "workload": f"mla_decode_step: fused dual RMSNorm + 1x128 FP8 group quant of M={M} tokens "
                        f"(q [M,1536] and kv [M,512] as strided views of a [M,2048] bf16 buffer), then "
                        f"block-scaled FP8 GEMMs with W_a [24576,1536] and W_b [8192,1536] sharing "
                        f"the (q_fp8, scale) pair, through mi_fused_normquant_gemm_pair: "
                        + ("all in one launch" if launches == 1 else
                           "the norm-quant launch then one launch of both GEMMs (its form above 16 rows)"),
            "step": args.step,
            "launches": launches if library else 2,   # kernel launches per step
            "other_step_us": {"two-launch" if library else "library": round(us_other, 3)},
            "M": M, "scale_layout": "column-major" if layout else "row-major",
            "weight_layout": "tiled (relaid out once at load time)" if tiled else "row-major",
            "cache": "warm" if args.warm else f"cold ({nsets} rotating buffer sets, "
                                              f"{nsets * step_bytes / 2**30:.2f} GiB)",
            "timing": "exactly `warmup` untimed steps, then `steps` timed steps (step i on buffer set "
                      "i mod sets), as HIP graphs of up to 2000 steps, replayed; HIP events around the timed "
                      "replays",
            "parallelism": "single GPU",
        },
        "roofline": roofline,
        "kernels": kernels,
        "device": {"name": props.name, "arch": getattr(props, "gcnArchName", "?"),
                   "cus": props.multi_processor_count},
    }
    if not args.warm and not args.no_warm:
        # labelled warm figures: one buffer set reused, so the weights come
        # from the Infinity Cache / L2 instead of HBM (not the headline)
        warm = {"cache": "warm (buffer set 0 reused every step)"}
        for name, keys, nbytes in (("step", ["fs"] if library else ["nq", "gp"], step_bytes),
                                   ("pair", ["gp"], kernels["block_scaled_fp8_gemm_pair"]["bytes"])):
            gw = make_graph(torch, [sets[0][k] for k in keys] * 20)   # 20 steps per replay
            us = time_graph(torch, gw, 20, 20)
            del gw
            warm[f"{name}_us"] = round(us, 3)
            warm[f"{name}_GB/s"] = round(nbytes / us / 1e3, 1)
        line["warm"] = warm
    if not args.no_sweep:
        sw = sweep(torch, np, mi, W, wa, wb, dev, cold=not args.warm, tiled=tiled)
        ceil = ceilings(torch, np, W)
        # the kernels against the measured data-movement ceilings of the same
        # access pattern (fraction = ceiling time / kernel time)
        for lay in ("row", "col"):
            e = sw.get(f"normquant_M8192_{lay}")
            if e:
                e["frac_ceiling"] = round(ceil["normquant_M8192"]["us"] / e["us"], 4)
        for name in ("W_a", "W_b"):
            for key, mf in ((f"gemm_{name}_M256", f"mfma_fold_{name}_M256"), (f"e8m0_gemm_{name}_M256",
                                                                             f"mfma_{name}_M256")):
                e = sw.get(key)
                if e:
                    e["frac_weight_stream_floor"] = round(ceil[f"weight_stream_{name}"]["us"] / e["us"], 4)
                    e["frac_mfma_floor"] = round(ceil[mf]["us"] / e["us"], 4)
        line["sweep"] = sw
        line["ceilings"] = ceil
    if not args.no_cpu_baseline:
        # set 0 once more through the library's step (its outputs were last
        # written by the single-GEMM timing loops), then to the host
        sets[0]["fs"]()
        torch.cuda.synchronize()
        oq, osc, okv, oa, ob = sets[0]["out"]
        got = (oq.cpu().numpy(), osc.cpu().numpy(), okv.view(torch.int16).cpu().numpy().view(np.uint16),
               oa.float().cpu().numpy().astype(np.float64), ob.float().cpu().numpy().astype(np.float64))
        line["cpu_baseline"], ref = cpu_baseline(np, W, M, layout, wa, wb)
        line["parity"] = parity_stats(np, got, ref)
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
