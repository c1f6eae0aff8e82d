"""Benchmark: W4A16 g128 decode GEMV on Llama-3-8B-shaped linear layers, 1 GPU.

One step = one decode pass (M = 1) through the four weight matrices of a
Llama-3-8B decoder layer -- fused QKV (6144x4096), O (4096x4096), fused
gate+up (28672x4096), down (4096x14336) -- each a W4A16 group-128 asymmetric
GEMV through the C ABI (qgemv_w4a16).  Inputs are seeded synthetic tensors of
those shapes (x ~ N(0,1), codes U{0..15}, scales U(0.001,0.02), zeros
U{0..15}); each layer rotates over R copies of its weight tensors (R * bytes
>= 1 GiB, above the 256 MB Infinity Cache and the 8 x 4 MB L2), so every call
reads its weights from HBM.

Timing: W eager warm-up steps; then the GPU is kept busy by a device-side
sleep while the host enqueues exactly K steps (4K kernel launches) between two
HIP events on the launch stream, so the measured region holds GPU time only
(the host finishes enqueueing before the sleep ends -- checked, else the run
aborts).  Synchronized on both sides.  value = algorithmic bytes of the K steps
/ elapsed time.

Printed: ONE JSON line (rank 0).  Extra objects:
  roofline      the dominant kernel (gate+up, the largest matrix): average
                launch duration over K back-to-back launches of that layer alone,
                timed the same way; against the 8 TB/s HBM peak and against the
                achievable peak (the best plain streaming read of 4 GiB through
                qgemv_stream_read); traffic = HBM bytes per launch from rocprofv3
                FETCH_SIZE / WRITE_SIZE (scaled by a device copy of known size),
                read from profiles/, null when the kernel sources changed since
  layers        per-layer us/call, with the streaming read of the same byte
                count (cache-cold slices) beside it
  stream_read   the streaming-read measurements
  variants      W2, W8, W4 at M = 4 and 16, LUT4, outliers, codebooks, W4A8,
                prefill, unfused baselines on the same layers (sampled rows
                checked against the oracle first; not part of `value`)
  skinny_70b    W4 and W2 on the Llama-70B-shaped layers at M = 1, 2, 4, 8, 16
                on both dot engines (VALU and MFMA): the batch-size crossover
  cpu_baseline  the plain C float64 oracle on a bounded row sample, one thread
                and all host cores, CPU model recorded

Profiling helpers (used under rocprofv3):
  --only LAYER          run only that layer in every step (skips the extras)
  --no-variants         skip the variants and the 70B skinny workload
  --copy-calibration    also time a device copy of known size (for scaling
                        FETCH_SIZE / WRITE_SIZE counters)
  --summarize-trace CSV print per-kernel, per-grid duration statistics of a
                        rocprofv3 --kernel-trace CSV and exit
  --traffic-from FETCH_CSV WRITE_CSV
                        write the gate_up traffic record (profiles/) from the
                        two counter passes' CSVs and exit
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

import synth  # noqa: E402

PEAK_HBM_GBS = 8000.0
METRIC = "W4A16 g128 decode GEMV µs/call and effective HBM GB/s (% of peak), 1 GPU"
BITS, M, G = 4, 1, 128


def alg_bytes(N, K, bits=BITS, m=M):
    Gn = K // G
    return N * K * bits // 8 + N * Gn * 2 + N * ((Gn * bits + 31) // 32) * 4 + m * K * 2 + m * N * 2


def build_inputs(torch, q, dev):
    layers = []
    for idx, (name, (N, K)) in enumerate(synth.LLAMA3_8B_LAYERS.items()):
        c = synth.uniform_case(synth.seed_for(1, idx), M, N, K, BITS)
        wq = q.pack(torch.from_numpy(c["codes"]).to(dev), BITS)
        zq = q.pack_zeros(torch.from_numpy(c["zeros"]).to(dev), BITS)
        s = torch.from_numpy(c["scales"]).to(dev)
        x = torch.from_numpy(c["x"]).to(dev)
        layers.append(dict(name=name, N=N, K=K, x=x, wq=[wq], s=[s], z=[zq], host=c,
                           y=torch.empty((M, N), dtype=torch.float16, device=dev),
                           bytes=alg_bytes(N, K)))
    step_bytes = sum(L["bytes"] for L in layers)
    # each layer rotates over its own R copies, R * bytes >= 1 GiB (above the
    # 256 MB Infinity Cache), so every call -- in a step or timed alone --
    # reads its weights from HBM
    for L in layers:
        L["R"] = max(2, -(-(1 << 30) // L["bytes"]))
        for _ in range(L["R"] - 1):
            L["wq"].append(L["wq"][0].clone())
            L["s"].append(L["s"][0].clone())
            L["z"].append(L["z"][0].clone())
    torch.cuda.synchronize()
    return layers, step_bytes


def spot_check(q, layers):
    """Sampled rows of every layer against the float64 oracle (a guard that the
    timed kernels compute the right thing; the full parity suite is in tests/)."""
    from oracle import reference as ref

    for L in layers:
        y = q.w4a16(L["x"], L["wq"][0], L["s"][0], L["z"][0]).cpu().numpy()
        rows = np.linspace(0, L["N"] - 1, 16).astype(np.int64)
        c = L["host"]
        y_ref, A = ref.gemv_uniform(c["x"], c["codes"], c["scales"], c["zeros"], rows=rows)
        ok = ref.within_tolerance(y[:, rows], y_ref, A)
        if not ok.all():
            raise SystemExit(f"bench: {L['name']} outside tolerance on sampled rows")


class Timer:
    """GPU-time regions of back-to-back launches: a device sleep keeps the
    stream busy while the host enqueues the region, so the two events bracket
    GPU execution only."""

    def __init__(self, torch):
        self.torch = torch
        # calibrate the sleep primitive (cycles -> seconds) once
        cyc = 10_000_000
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        e0.record()
        torch.cuda._sleep(cyc)
        e1.record()
        torch.cuda.synchronize()
        self.s_per_cycle = e0.elapsed_time(e1) * 1e-3 / cyc

    host_bound = False

    def region_us(self, fn, n, host_s_per_call):
        torch = self.torch
        sleep_s = max(0.005, 3.0 * n * host_s_per_call)
        for attempt in range(4):
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            torch.cuda.synchronize()
            t0 = time.perf_counter()
            torch.cuda._sleep(int(sleep_s / self.s_per_cycle))
            e0.record()
            for i in range(n):
                fn(i)
            e1.record()
            host = time.perf_counter() - t0
            torch.cuda.synchronize()
            if host <= 0.8 * sleep_s:
                return e0.elapsed_time(e1) * 1000.0
            sleep_s = 2.0 * host  # the host was slower than estimated (e.g. under a profiler)
        print(f"bench: warning: host enqueue ({host * 1e3:.1f} ms) did not stay ahead of the GPU",
              file=sys.stderr)
        Timer.host_bound = True
        return e0.elapsed_time(e1) * 1000.0


def host_cost(torch, fn, n=20):
    """Host seconds per fn call (to size the covering sleep)."""
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(n):
        fn(i)
    dt = (time.perf_counter() - t0) / n
    torch.cuda.synchronize()
    return dt


def summarize_trace(path):
    """Per kernel name and grid: count, mean/median/p10/p90 duration (us)."""
    import csv
    from collections import defaultdict

    import re

    d = defaultdict(list)
    with open(path) as f:
        for r in csv.DictReader(f):
            name = re.sub(r"^(void )?qg::\(anonymous namespace\)::", "", r["Kernel_Name"]).split("(")[0]
            key = (name.replace(" ", ""), int(r["Grid_Size_X"]), int(r["Workgroup_Size_X"]))
            d[key].append((int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1000.0)
    print(f"{'kernel':72s} {'grid':>8s} {'wg':>5s} {'n':>5s} {'mean':>8s} {'median':>8s} {'p10':>8s} {'p90':>8s}")
    for (name, gx, wx), v in sorted(d.items(), key=lambda kv: -sum(kv[1])):
        v.sort()
        n = len(v)
        print(f"{name[:72]:72s} {gx:8d} {wx:5d} {n:5d} {sum(v) / n:8.3f} {v[n // 2]:8.3f} "
              f"{v[n // 10]:8.3f} {v[(9 * n) // 10]:8.3f}")


# HBM traffic of the dominant kernel, from two rocprofv3 --pmc passes
# (FETCH_SIZE, WRITE_SIZE) scaled by the same counters on a device copy of
# known size; valid only for the kernel sources it was measured on.
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "gemv_w4a16_gate_up_28672x4096_m1_hbm_traffic.json")


KERNEL_SOURCES = ["gemm_unpack_bit_amd/csrc/gemv_tiles.hip", "gemm_unpack_bit_amd/csrc/dequant.hpp",
                  "gemm_unpack_bit_amd/csrc/common.hpp", "gemm_unpack_bit_amd/csrc/kernels.hpp",
                  "gemm_unpack_bit_amd/csrc/api.cpp"]
GEMV_KERNELS = ("gemv_tiles_kernel",)


def sources_sha256(paths):
    import hashlib

    h = hashlib.sha256()
    for src in paths:
        with open(os.path.join(ROOT, src), "rb") as f:
            h.update(f.read())
    return h.hexdigest()


def traffic_from(fetch_csv, write_csv):
    """The traffic record from two rocprofv3 --pmc runs of
    `bench.py --only gate_up --copy-calibration` (FETCH_SIZE, then WRITE_SIZE):
    the GEMV's KiB per dispatch, each scaled by what the same counter reads for
    the 256 MiB calibration copy, stamped with the current kernel sources'
    SHA-256.  Written to TRAFFIC_FILE and printed."""
    import csv

    copy_bytes = 256 << 20

    def read(path, counter):
        gemv, copy, names = [], [], set()
        for r in csv.DictReader(open(path)):
            if r["Counter_Name"] != counter:
                continue
            v = float(r["Counter_Value"])
            if any(k in r["Kernel_Name"] for k in GEMV_KERNELS):
                gemv.append(v)
                names.add((r["Kernel_Name"], r["Grid_Size"], r["Workgroup_Size"]))
            elif "copyBuffer" in r["Kernel_Name"]:
                copy.append(v)
        if not gemv or not copy or len(names) != 1:
            raise SystemExit(f"traffic: expected one GEMV kernel and the calibration copy in {path}")
        return sum(gemv) / len(gemv), max(copy), len(gemv), names.pop()

    f_kib, f_copy, n, (kname, grid, wg) = read(fetch_csv, "FETCH_SIZE")
    w_kib, w_copy, _, _ = read(write_csv, "WRITE_SIZE")
    ff, wf = copy_bytes / 1024 / f_copy, copy_bytes / 1024 / w_copy
    import re

    m = re.search(r"gemv_tiles_kernel<[^>]*>", kname)
    kshort = m.group(0).replace(" ", "") if m else kname
    N, K = synth.LLAMA3_8B_LAYERS["gate_up"]
    rec = {
        "kernel": f"{kshort} (gate_up {N}x{K}, W4A16 g128, M=1, grid {grid} threads x {wg}/wg)",
        "kernel_sources": KERNEL_SOURCES,
        "kernel_src_sha256": sources_sha256(KERNEL_SOURCES),
        "fetch_size_kib_per_dispatch": round(f_kib, 3),
        "write_size_kib_per_dispatch": round(w_kib, 3),
        "dispatches": n,
        "copy_bytes": copy_bytes,
        "copy_fetch_kib": round(f_copy, 3),
        "copy_write_kib": round(w_copy, 3),
        "fetch_factor": round(ff, 5),
        "write_factor": round(wf, 5),
        "traffic_bytes_per_launch": int(round((f_kib * ff + w_kib * wf) * 1024)),
        "algorithmic_bytes_per_launch": alg_bytes(N, K),
    }
    with open(TRAFFIC_FILE, "w") as f:
        json.dump(rec, f, indent=1)
    print(json.dumps(rec, indent=1))


def measured_traffic():
    try:
        with open(TRAFFIC_FILE) as f:
            rec = json.load(f)
        digest = sources_sha256(rec["kernel_sources"])
    except (OSError, KeyError, ValueError):
        return None
    if digest != rec.get("kernel_src_sha256"):
        return None  # the kernel changed since the counters were taken
    return int(rec["traffic_bytes_per_launch"])


# ---------------------------------------------------------------------------
# the other variants on the same four layers, and the codebook on the 70B
# layers (reported beside the headline,
# not part of `value`): each layer's cache-cold launch time, algorithmic bytes
# per launch, sampled rows checked against the oracle first
# ---------------------------------------------------------------------------
VARIANTS = {
    "w2a16_m1": dict(kind="uniform", bits=2, m=1),
    "w8a16_m1": dict(kind="uniform", bits=8, m=1),
    "w4a16_m4": dict(kind="uniform", bits=4, m=4),
    "w4a16_m16": dict(kind="uniform", bits=4, m=16),
    "lut4_m1": dict(kind="lut4", bits=4, m=1),
    "outlier_m1": dict(kind="outlier", bits=4, m=1),
    "codebook_m1": dict(kind="codebook", bits=2, m=1),
    # the codebook workload's own shapes: the 70B layers at M = 1 and 4
    "codebook_70b_m1": dict(kind="codebook", bits=2, m=1, layers="70b"),
    "codebook_70b_m4": dict(kind="codebook", bits=2, m=4, layers="70b"),
    # the general codebook kernel on two ~2-bit formats of the family the
    # CodeGEMM notes compare: (m, v, g) = (3, 16, 32) and (2, 8, 64)
    "codebook_m3v16g32_m1": dict(kind="codebook_gen", bits=2, m=1, cb=(3, 16, 32)),
    "codebook_m2v8g64_m1": dict(kind="codebook_gen", bits=2, m=1, cb=(2, 8, 64)),
    # W4A8 (int8 activations, padding strategy, int8 matrix cores)
    "w4a8_m1": dict(kind="w4a8", bits=4, m=1),
    "w4a8_m16": dict(kind="w4a8", bits=4, m=16),
    # W4A8 by the split strategy (fp8 matrix cores) and with asymmetric activations
    "w4a8_split_m1": dict(kind="w4a8_split", bits=4, m=1),
    "w4a8_split_m16": dict(kind="w4a8_split", bits=4, m=16),
    "w4a8_asym_m1": dict(kind="w4a8_asym", bits=4, m=1),
    "w4a8_asym_m16": dict(kind="w4a8_asym", bits=4, m=16),
    # prefill: the GEMM path at M = 512 (compute-bound; TFLOP/s reported)
    "w4a16_prefill_m512": dict(kind="gemm", bits=4, m=512),
    # unfused baselines: what fusion buys.  fp16 weights (no quantization),
    # eager dequantization + dense GEMV, and the dense W4 kernel + separate SpMV
    "f16_dense_m1": dict(kind="dense", bits=16, m=1),
    "eager_w4a16_m1": dict(kind="eager", bits=4, m=1),
    "eager_lut4_m1": dict(kind="eager_lut4", bits=4, m=1),
    "outlier_unfused_m1": dict(kind="outlier_unfused", bits=4, m=1),
}


def variant_layer(torch, q, dev, kind, bits, m, idx, N, K, cb=None):
    """Host case, device inputs (one copy), launch function, algorithmic bytes
    and, for the two-kernel baselines, each kernel alone with its bytes."""
    from oracle import reference as ref

    seed = synth.seed_for(2, 16 * idx + bits + 4 * m)
    up = lambda a: torch.from_numpy(np.ascontiguousarray(a)).to(dev)
    y = torch.empty((m, N), dtype=torch.float16, device=dev)
    io = 2 * m * K + 2 * m * N
    parts = None
    if kind == "dense":
        c = synth.dense_case(seed, m, N, K)
        t = dict(x=up(c["x"]), w=up(c["w"]))
        call = lambda t: q.gemv_f16(t["x"], t["w"], out=y)
        oracle = lambda rows: ref.gemv_dense(c["x"], c["w"], rows=rows)
        nbytes = 2 * N * K + io
    elif kind == "codebook_gen":
        ncb, v, g = cb
        c = synth.codebook_additive_case(seed, m, N, K, ncb, v, g)
        ws = torch.zeros(max(q.codebook_gen_workspace_bytes(m, N, K, ncb, v, g), 4) // 4, dtype=torch.int32,
                         device=dev)
        t = dict(x=up(c["x"]), codes=q.pack_codebook_planes(up(c["codes"])), cb=up(c["codebooks"]),
                 s=up(c["scales"]))
        call = lambda t: q.codebook_gen(t["x"], t["codes"], t["cb"], t["s"], g, ws=ws, out=y)
        oracle = lambda rows: ref.gemv_codebook_additive(c["x"], c["codes"], c["codebooks"], c["scales"], g,
                                                         rows=rows)
        nbytes = ncb * N * K // v + N * (K // g) * 2 + ncb * 256 * v * 2 + io
    elif kind == "eager":
        c = synth.uniform_case(seed, m, N, K, bits)
        t = dict(x=up(c["x"]), wq=q.pack(up(c["codes"]), bits), s=up(c["scales"]),
                 z=q.pack_zeros(up(c["zeros"]), bits), w=torch.empty((N, K), dtype=torch.float16, device=dev))
        deq = lambda t: q.dequant(t["wq"], t["s"], t["z"], bits, K, out=t["w"])
        mv = lambda t: q.gemv_f16(t["x"], t["w"], out=y)
        call = lambda t: (deq(t), mv(t))
        oracle = lambda rows: ref.gemv_uniform(c["x"], c["codes"], c["scales"], c["zeros"], rows=rows)
        b_deq = alg_bytes(N, K, bits, 0) + 2 * N * K
        parts = {"dequant": (deq, b_deq), "gemv_f16": (mv, 2 * N * K + io)}
        nbytes = b_deq + 2 * N * K + io
    elif kind == "eager_lut4":
        c = synth.lut4_case(seed, m, N, K)
        t = dict(x=up(c["x"]), wq=q.pack(up(c["codes"]), 4), a=up(c["absmax"]), lut=up(c["lut"]),
                 w=torch.empty((N, K), dtype=torch.float16, device=dev))
        deq = lambda t: q.dequant_lut4(t["wq"], t["a"], t["lut"], K, out=t["w"])
        mv = lambda t: q.gemv_f16(t["x"], t["w"], out=y)
        call = lambda t: (deq(t), mv(t))
        oracle = lambda rows: ref.gemv_lut4(c["x"], c["codes"], c["absmax"], c["lut"], rows=rows)
        b_deq = N * K // 2 + N * (K // 64) * 2 + 32 + 2 * N * K
        parts = {"dequant_lut4": (deq, b_deq), "gemv_f16": (mv, 2 * N * K + io)}
        nbytes = b_deq + 2 * N * K + io
    elif kind == "outlier_unfused":
        c = synth.outlier_case(seed, m, N, K)
        ptr, rec = q.tilecoo_encode(N, K, c["o_rows"], c["o_cols"], c["o_vals"])
        t = dict(x=up(c["x"]), wq=q.pack(up(c["codes"]), 4), s=up(c["scales"]),
                 z=q.pack_zeros(up(c["zeros"]), 4), p=up(ptr.view(np.int32)), r=up(rec.view(np.int32)))
        dense = lambda t: q.w4a16(t["x"], t["wq"], t["s"], t["z"], out=y)
        sp = lambda t: q.spmv_tilecoo(t["x"], t["p"], t["r"], y)
        call = lambda t: (dense(t), sp(t))
        oracle = lambda rows: ref.gemv_outlier(c["x"], c["codes"], c["scales"], c["zeros"], c["o_rows"],
                                               c["o_cols"], c["o_vals"], rows=rows)
        b_sp = 4 * rec.size + 4 * ptr.size + 2 * m * K + 4 * m * N
        parts = {"w4a16": (dense, alg_bytes(N, K, 4, m)), "spmv_tilecoo": (sp, b_sp)}
        nbytes = alg_bytes(N, K, 4, m) + 4 * rec.size + 4 * ptr.size
    elif kind in ("w4a8", "w4a8_split", "w4a8_asym"):
        c = synth.uniform_case(seed, m, N, K, bits)
        fn, wsb, ofn = {"w4a8": (q.w4a8, q.w4a8_workspace_bytes, ref.gemv_w4a8),
                        "w4a8_split": (q.w4a8_split, q.w4a8_split_workspace_bytes, ref.gemv_w4a8_split),
                        "w4a8_asym": (q.w4a8_asym, q.w4a8_asym_workspace_bytes, ref.gemv_w4a8_asym)}[kind]
        ws = torch.zeros(wsb(m, K), dtype=torch.uint8, device=dev)
        t = dict(x=up(c["x"]), wq=q.pack(up(c["codes"]), bits), s=up(c["scales"]),
                 z=q.pack_zeros(up(c["zeros"]), bits))
        call = lambda t: fn(t["x"], t["wq"], t["s"], t["z"], ws, out=y)
        oracle = lambda rows: ofn(c["x"], c["codes"], c["scales"], c["zeros"], rows=rows)
        nbytes = alg_bytes(N, K, bits, m)
    elif kind == "gemm":
        c = synth.uniform_case(seed, m, N, K, bits)
        t = dict(x=up(c["x"]), wq=q.pack(up(c["codes"]), bits), s=up(c["scales"]),
                 z=q.pack_zeros(up(c["zeros"]), bits))
        call = lambda t: q.gemm_uniform(t["x"], t["wq"], t["s"], t["z"], bits, out=y)
        oracle = lambda rows: ref.gemv_uniform(c["x"], c["codes"], c["scales"], c["zeros"], rows=rows)
        nbytes = alg_bytes(N, K, bits, m)
    elif kind == "uniform":
        c = synth.uniform_case(seed, m, N, K, bits)
        t = dict(x=up(c["x"]), wq=q.pack(up(c["codes"]), bits), s=up(c["scales"]),
                 z=q.pack_zeros(up(c["zeros"]), bits))
        call = lambda t: q.uniform(t["x"], t["wq"], t["s"], t["z"], bits, out=y)
        oracle = lambda rows: ref.gemv_uniform(c["x"], c["codes"], c["scales"], c["zeros"], rows=rows)
        nbytes = alg_bytes(N, K, bits, m)
    elif kind == "lut4":
        c = synth.lut4_case(seed, m, N, K)
        t = dict(x=up(c["x"]), wq=q.pack(up(c["codes"]), 4), a=up(c["absmax"]), lut=up(c["lut"]))
        call = lambda t: q.lut4(t["x"], t["wq"], t["a"], t["lut"], out=y)
        oracle = lambda rows: ref.gemv_lut4(c["x"], c["codes"], c["absmax"], c["lut"], rows=rows)
        nbytes = N * K // 2 + N * (K // 64) * 2 + 32 + io
    elif kind == "outlier":
        c = synth.outlier_case(seed, m, N, K)
        ptr, rec = q.tilecoo_encode(N, K, c["o_rows"], c["o_cols"], c["o_vals"])
        t = dict(x=up(c["x"]), wq=q.pack(up(c["codes"]), 4), s=up(c["scales"]),
                 z=q.pack_zeros(up(c["zeros"]), 4), p=up(ptr.view(np.int32)), r=up(rec.view(np.int32)))
        call = lambda t: q.outlier(t["x"], t["wq"], t["s"], t["z"], t["p"], t["r"], out=y)
        oracle = lambda rows: ref.gemv_outlier(c["x"], c["codes"], c["scales"], c["zeros"], c["o_rows"],
                                               c["o_cols"], c["o_vals"], rows=rows)
        nbytes = alg_bytes(N, K, 4, m) + 4 * rec.size + 4 * ptr.size
    else:
        c = synth.codebook_case(seed, m, N, K)
        ws = torch.zeros(max(q.codebook_workspace_bytes(m, N, K), 4) // 4, dtype=torch.int32, device=dev)
        t = dict(x=up(c["x"]), codes=q.pack(up(c["codes"]), 8, q.LAYOUT_ROWS64), cb=up(c["codebook"]),
                 s=up(c["scales"]))
        call = lambda t: q.codebook(t["x"], t["codes"], t["cb"], t["s"], ws=ws, out=y)
        oracle = lambda rows: ref.gemv_codebook(c["x"], c["codes"], c["codebook"], c["scales"], rows=rows)
        nbytes = N * K // 4 + N * (K // 128) * 2 + 256 * 4 * 2 + io
    return t, call, oracle, y, nbytes, parts


def measure_variants(torch, q, dev, timer, n):
    from oracle import reference as ref

    out = {}
    for vname, v in VARIANTS.items():
        layers, total_us, total_bytes = {}, 0.0, 0
        shapes = synth.LLAMA_70B_LAYERS if v.get("layers") == "70b" else synth.LLAMA3_8B_LAYERS
        for idx, (name, (N, K)) in enumerate(shapes.items()):
            t, call, oracle, y, nbytes, parts = variant_layer(torch, q, dev, v["kind"], v["bits"], v["m"], idx,
                                                              N, K, v.get("cb"))
            call(t)
            rows = np.linspace(0, N - 1, 8).astype(np.int64)
            y_ref, A = oracle(rows)
            if not ref.within_tolerance(y.cpu().numpy()[:, rows], y_ref, A).all():
                raise SystemExit(f"bench: variant {vname} {name} outside tolerance on sampled rows")
            R = max(2, -(-(1 << 30) // nbytes))
            copies = [t] + [{k: (a.clone() if k not in ("x", "lut", "cb") else a) for k, a in t.items()}
                            for _ in range(R - 1)]
            fn = lambda i: call(copies[i % R])
            for i in range(8):
                fn(i)
            us = timer.region_us(fn, n, host_cost(torch, fn)) / n
            layers[name] = {"us_per_call": round(us, 3), "GBps": round(nbytes / us / 1e3, 1),
                            "pct_peak": round(nbytes / us / 1e3 / PEAK_HBM_GBS * 100, 1), "bytes": nbytes}
            if v["kind"] == "gemm":  # compute-bound: fp16 matrix-core peak 2.5 PFLOP/s
                layers[name]["TFLOPs"] = round(2.0 * v["m"] * N * K / us / 1e6, 1)
            for pname, (pcall, pbytes) in (parts or {}).items():  # each kernel of the sequence alone
                pfn = lambda i, pcall=pcall: pcall(copies[i % R])
                pus = timer.region_us(pfn, n, host_cost(torch, pfn)) / n
                layers[name][pname] = {"us_per_call": round(pus, 3), "GBps": round(pbytes / pus / 1e3, 1),
                                       "bytes": pbytes}
            total_us += us
            total_bytes += nbytes
            del copies, t
            torch.cuda.empty_cache()
        out[vname] = {"m": v["m"], "layers": layers, "us_per_step": round(total_us, 3),
                      "GBps": round(total_bytes / total_us / 1e3, 1)}
    return out


def profile_variant(torch, q, dev, vname, only, calls):
    """Run one entry of the variants table (one layer with `only`) `calls`
    times on cache-cold copies, for counter collection; prints one line."""
    v = VARIANTS[vname]
    shapes = synth.LLAMA_70B_LAYERS if v.get("layers") == "70b" else synth.LLAMA3_8B_LAYERS
    done = []
    for idx, (name, (N, K)) in enumerate(shapes.items()):
        if only and name != only:
            continue
        t, call, _, _, nbytes, _ = variant_layer(torch, q, dev, v["kind"], v["bits"], v["m"], idx, N, K, v.get("cb"))
        R = max(2, -(-(1 << 30) // nbytes))
        copies = [t] + [{k: (a.clone() if k not in ("x", "lut", "cb") else a) for k, a in t.items()}
                        for _ in range(R - 1)]
        for i in range(calls):
            call(copies[i % R])
        torch.cuda.synchronize()
        done.append({"layer": name, "N": N, "K": K, "bytes_per_call": nbytes, "calls": calls})
        del copies, t
        torch.cuda.empty_cache()
    print(json.dumps({"profile_variant": vname, "m": v["m"], "layers": done}), flush=True)


def cpu_model():
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def cpu_baseline(layers, budget_s=8.0):
    """The plain C oracle (oracle/cref.c: unpack -> dequantize -> float64
    matvec) on rows [0, N/8) of every layer: single-threaded, then with one
    thread per host core available to this process, each repeated until
    about `budget_s` of wall time.  Packing the sample (plain layout) is done
    once, outside the timed region."""
    from oracle import cref, formats

    sample = []
    for L in layers:
        c, n8 = L["host"], L["N"] // 8
        packed = (formats.pack_plain(c["codes"][:n8], BITS), formats.pack_plain(c["zeros"][:n8], BITS))
        sample.append((c, n8, packed, alg_bytes(n8, L["K"])))
    sample_bytes = sum(sb for *_, sb in sample)
    cores = len(os.sched_getaffinity(0)) if hasattr(os, "sched_getaffinity") else (os.cpu_count() or 1)

    def timed(threads, budget):
        reps, t0 = 0, time.perf_counter()
        while True:
            for c, n8, packed, _ in sample:
                cref.gemv_uniform(c["x"], None, c["scales"][:n8], None, BITS, packed=packed, threads=threads)
            reps += 1
            el = time.perf_counter() - t0
            if el >= budget:
                return reps, el

    r1, e1 = timed(1, budget_s / 2)
    rn, en = timed(cores, budget_s / 2)
    step_us = lambda reps, el: el / reps * 8 * 1e6
    return {
        "value": round(sample_bytes * rn / en / 1e9, 4),
        "unit": "GB/s",
        "cores": int(cores),
        "kind": "oracle",
        "sample": f"plain C float64 oracle (oracle/cref.c, OpenMP over rows) on rows [0, N/8) of each of the "
                  f"4 layers: {rn} passes in {en:.1f} s on {cores} threads, {r1} passes in {e1:.1f} s on one; "
                  f"extrapolated {step_us(rn, en):.0f} us ({cores} threads) and {step_us(r1, e1):.0f} us "
                  f"(1 thread) per full 4-layer step",
        "single_thread_GBps": round(sample_bytes * r1 / e1 / 1e9, 4),
        "us_per_step": round(step_us(rn, en), 1),
        "us_per_step_single_thread": round(step_us(r1, e1), 1),
        "cpu_model": cpu_model(),
    }


# ---------------------------------------------------------------------------
# achievable peak: a plain streaming read (qgemv_stream_read) of a 4 GiB
# buffer, the best of a few launch shapes; and reads of each layer's byte
# count from rotating slices of the same buffer (cache-cold)
# ---------------------------------------------------------------------------
READ_SHAPES = [(wg, th) for wg in (256, 512, 1024, 2048, 4096) for th in (256, 512, 1024)]


def achievable_peak(torch, q, timer, sizes):
    GiB = 1 << 30
    buf = torch.empty(4 * GiB, dtype=torch.uint8, device="cuda")
    buf.fill_(0x5A)
    sink = torch.zeros(4, dtype=torch.int32, device="cuda")

    def best_read(nbytes, n):
        nbytes = nbytes // 16 * 16
        slices = max(1, (4 * GiB) // nbytes)
        best = None
        for wg, th in READ_SHAPES:
            fn = lambda i, wg=wg, th=th: q.stream_read(buf, sink, nbytes, wg, th, (i % slices) * nbytes)
            for i in range(2):
                fn(i)
            us = timer.region_us(fn, n, host_cost(torch, fn)) / n
            if best is None or us < best[0]:
                best = (us, wg, th)
        return {"bytes": nbytes, "us": round(best[0], 3), "GBps": round(nbytes / best[0] / 1e3, 1),
                "workgroups": best[1], "threads": best[2]}

    out = {"read_4GiB": best_read(4 * GiB, 3)}
    out["per_size"] = {name: best_read(nb, 40) for name, nb in sizes.items()}
    del buf
    torch.cuda.empty_cache()
    return out


# ---------------------------------------------------------------------------
# the 70B skinny-GEMM workload: W4 and W2 on the four Llama-70B-shaped layers
# at M = 1, 2, 4, 8, 16, each on both dot engines (the batch-size crossover)
# ---------------------------------------------------------------------------
SKINNY_M = (1, 2, 4, 8, 16)


def measure_skinny(torch, q, timer, n):
    from oracle import reference as ref

    up = lambda a: torch.from_numpy(np.ascontiguousarray(a)).cuda()
    out = {}
    for bits in (4, 2):
        per_m = {M: {"valu": 0.0, "mfma": 0.0, "bytes": 0, "layers": {}} for M in SKINNY_M}
        for idx, (name, (N, K)) in enumerate(synth.LLAMA_70B_LAYERS.items()):
            c = synth.uniform_case(synth.seed_for(3, idx), 16, N, K, bits)
            t0 = dict(wq=q.pack(up(c["codes"]), bits), s=up(c["scales"]), z=q.pack_zeros(up(c["zeros"]), bits))
            x16 = up(c["x"])
            rows = np.linspace(0, N - 1, 8).astype(np.int64)
            y_ref, A = ref.gemv_uniform(c["x"], c["codes"], c["scales"], c["zeros"], rows=rows)
            for path in (q.PATH_VALU, q.PATH_MFMA):
                for M in (1, 16):
                    y = q.uniform(x16[:M], t0["wq"], t0["s"], t0["z"], bits, path).cpu().numpy()
                    if not ref.within_tolerance(y[:, rows], y_ref[:M], A[:M]).all():
                        raise SystemExit(f"bench: skinny W{bits} {name} M={M} path={path} outside tolerance")
            R = max(2, -(-(1 << 30) // alg_bytes(N, K, bits, 0)))
            copies = [t0] + [{k: a.clone() for k, a in t0.items()} for _ in range(R - 1)]
            for M in SKINNY_M:
                x = x16[:M].contiguous()
                y = torch.empty((M, N), dtype=torch.float16, device="cuda")
                rec = {}
                for eng, path in (("valu", q.PATH_VALU), ("mfma", q.PATH_MFMA)):
                    fn = lambda i, path=path: q.uniform(x, copies[i % R]["wq"], copies[i % R]["s"],
                                                        copies[i % R]["z"], bits, path, out=y)
                    for i in range(4):
                        fn(i)
                    us = timer.region_us(fn, n, host_cost(torch, fn)) / n
                    rec[eng] = round(us, 3)
                    per_m[M][eng] += us
                nb = alg_bytes(N, K, bits, M)
                per_m[M]["bytes"] += nb
                rec["GBps_best"] = round(nb / min(rec["valu"], rec["mfma"]) / 1e3, 1)
                per_m[M]["layers"][name] = rec
            del copies, t0
            torch.cuda.empty_cache()
        res = {}
        for M, v in per_m.items():
            auto = "valu" if M <= 1 else "mfma"  # the engine the library picks (qgemv_uniform, PATH_AUTO)
            res[f"m{M}"] = {"auto_engine": auto, "us_per_step_valu": round(v["valu"], 3),
                            "us_per_step_mfma": round(v["mfma"], 3), "bytes": v["bytes"],
                            "GBps_auto": round(v["bytes"] / v[auto] / 1e3, 1),
                            "pct_peak_auto": round(v["bytes"] / v[auto] / 1e3 / PEAK_HBM_GBS * 100, 1),
                            "faster_engine": "valu" if v["valu"] < v["mfma"] else "mfma", "layers": v["layers"]}
        out[f"w{bits}a16"] = res
    return out


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=50)
    ap.add_argument("--no-cpu", action="store_true", help="skip the cpu_baseline leg")
    ap.add_argument("--no-variants", action="store_true", help="skip the other variants' measurements")
    ap.add_argument("--only", default=None, help="run only this layer (profiling)")
    ap.add_argument("--variant", default=None,
                    help="profiling: run only this entry of the variants table (with --only: one layer), "
                         "--steps calls per layer, and exit")
    ap.add_argument("--copy-calibration", action="store_true")
    ap.add_argument("--summarize-trace", default=None)
    ap.add_argument("--traffic-from", nargs=2, metavar=("FETCH_CSV", "WRITE_CSV"), default=None)
    args = ap.parse_args()
    if args.summarize_trace:
        summarize_trace(args.summarize_trace)
        return
    if args.traffic_from:
        traffic_from(*args.traffic_from)
        return
    if args.gpus != 1:
        print(f"bench.py: the GEMV runs and is measured on one GPU; --gpus {args.gpus} is not supported "
              "(a multi-GPU run would give each GPU its own slice of the weight rows)", file=sys.stderr)
        sys.exit(2)

    import torch

    import gemm_unpack_bit_amd as q

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    dev = torch.device("cuda:0")
    if args.variant:
        profile_variant(torch, q, dev, args.variant, args.only, args.steps)
        return
    layers, step_bytes = build_inputs(torch, q, dev)

    run = [L for L in layers if args.only in (None, L["name"])]
    if not run:
        raise SystemExit(f"bench: no layer named {args.only}")
    spot_check(q, run)
    if args.only:
        step_bytes = sum(L["bytes"] for L in run)

    def step(i):
        for L in run:
            r = i % L["R"]
            q.w4a16(L["x"], L["wq"][r], L["s"][r], L["z"][r], out=L["y"])

    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()

    timer = Timer(torch)
    K = args.steps
    total_us = timer.region_us(step, K, host_cost(torch, step))
    ms_per_step = total_us / K / 1000.0
    value = step_bytes * K / (total_us * 1e-6) / 1e9

    if args.copy_calibration:
        src = torch.empty(256 << 20, dtype=torch.uint8, device=dev)
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()

    per_layer = {}
    for L in run:
        def one(i, L=L):
            r = i % L["R"]
            q.w4a16(L["x"], L["wq"][r], L["s"][r], L["z"][r], out=L["y"])

        us = timer.region_us(one, K, host_cost(torch, one)) / K
        per_layer[L["name"]] = {
            "N": L["N"], "K": L["K"], "us_per_call": round(us, 3),
            "GBps": round(L["bytes"] / us / 1e3, 1), "pct_peak": round(L["bytes"] / us / 1e3 / PEAK_HBM_GBS * 100, 1),
            "bytes": L["bytes"],
        }
    dom = max(run, key=lambda L: L["bytes"])
    dom_us = per_layer[dom["name"]]["us_per_call"]
    achieved = dom["bytes"] / dom_us / 1e3
    peak = None
    if not args.only:
        peak = achievable_peak(torch, q, timer, {L["name"]: L["bytes"] for L in run})
        for L in run:
            rd = peak["per_size"][L["name"]]
            per_layer[L["name"]]["stream_read_us"] = rd["us"]
            per_layer[L["name"]]["vs_stream_read"] = round(rd["us"] / per_layer[L["name"]]["us_per_call"], 3)

    out = {
        "metric": METRIC,
        "value": round(value, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 6),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f16",
        "data": "synthetic",
        "config": {
            "workload": "Llama-3-8B decoder-layer linear GEMVs (qkv 6144x4096, o 4096x4096, gate_up 28672x4096, "
                        "down 4096x14336), W4A16 asymmetric g128, M=1, cache-cold rotated weights",
            "batch_m": M, "bits": BITS, "group": G, "rotated_copies": {L["name"]: L["R"] for L in layers},
            "step_bytes": step_bytes,
            "us_per_step": round(ms_per_step * 1000, 3), "pct_peak": round(value / PEAK_HBM_GBS * 100, 2),
            "timing": "GPU-time region of back-to-back launches behind a device sleep"
                      + (" (host-bound: numbers unreliable)" if Timer.host_bound else ""),
        },
        "roofline": {
            "bound": "hbm",
            "kernel": f"qgemv W4A16 GEMV gate_up {dom['N']}x{dom['K']} M=1",
            "achieved": round(achieved, 1),
            "peak": PEAK_HBM_GBS,
            "unit": "GB/s",
            "frac": round(achieved / PEAK_HBM_GBS, 4),
            "traffic": measured_traffic() if dom["name"] == "gate_up" else None,
            "us_per_launch": dom_us,
            "bytes_per_launch": dom["bytes"],
        },
        "layers": per_layer,
    }
    if peak:
        ap = peak["read_4GiB"]["GBps"]
        out["roofline"]["achievable_peak"] = ap
        out["roofline"]["frac_achievable"] = round(achieved / ap, 4)
        out["roofline"]["achievable_peak_from"] = (
            f"qgemv_stream_read of a 4 GiB buffer, best of {len(READ_SHAPES)} launch shapes "
            f"({peak['read_4GiB']['workgroups']} x {peak['read_4GiB']['threads']})")
        out["stream_read"] = peak
    if not (args.no_variants or args.only):
        out["variants"] = measure_variants(torch, q, dev, timer, max(20, min(K, 100)))
        out["skinny_70b"] = measure_skinny(torch, q, timer, max(20, min(K, 60)))
    if not args.no_cpu:
        out["cpu_baseline"] = cpu_baseline(layers)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
