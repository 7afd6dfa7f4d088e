"""Benchmark: one GPTQ layer (H from calibration tokens, damping, inverse
factor, blocked sweep) on one MI355X.

Default workload: the attention-projection layer (W 4096x4096 fp16 with 0.1 %
outliers x10; X = 262144 tokens x 4096 fp16, lognormal channel scales, 8
outlier channels x20; 4-bit, group 128, block 128, damp 0.01), inputs drawn by
synth/ and resident in HBM before timing.  A step is the whole path:
restore W, zero H, gptq_hessian_accumulate, gptq_prepare_hinv,
gptq_quantize_layer (with the dequantized weights written back).

--workload picks another layer shape: tiny (64x128 fp32), mlp_up / mlp_down
(11008x4096 / 4096x11008, 3-bit per row, 262144 tokens), qkv / o / gate_up /
down7b (a 7B block's jobs over 65536 tokens: q/k/v stacked to 12288 rows and
gate/up to 22016 rows, each on one shared Hessian), fc1 / fc2 (a 175B-class
FFN shard, 3-bit g128, 262144 tokens).

Beside the whole-step time the line carries, per phase, the median and the
minimum of the HIP-event times over the timed steps and the phase's roofline
fraction from its algorithmic work: SYRK n(n+1)T flops against dense fp16
MFMA; the inverse factor 4n^3/3 flops (the route run here executes 2n^3/3)
against fp32 MFMA; the trailing update's GEMM kernels the flops they perform of
m n (n - B) against fp32 MFMA; the sweep kernel m n (4 + 4 + b/8) + 8 m G +
4 n B bytes against HBM.  The two quantize-phase splits come from GPU kernel
durations recorded by torch.profiler over one further step.

Prints one JSON line (rank 0).  Multi-GPU runs are not supported.

--kernel w4a16 instead times the runtime use of a packed layer,
gptq_dequant_matmul (Y = X What^T with 4-bit g128 codes unpacked next to fp16
activations), on an MLP-shaped layer (28672 x 8192) for one decode token; its
line carries the same keys, with GB/s of the packed layer as the metric.

--kernel rotate times gptq_rotate_hadamard on the attention-projection
calibration activations (262144 x 4096 fp16, one 4096-wide Hadamard block per
row, in place): the fixed rotation applied before GPTQ; GB/s of HBM traffic.

--kernel stack times the network-level loop (quantize_mlp_stack) over two
7B-shaped MLP blocks (d 4096, f 11008, 4-bit g128) with 8192 calibration
tokens: per block, H, factor and sweep for gate/up (shared H) and down, the
quantized forward through gptq_dequant_matmul, SwiGLU and the residual.

--kernel obq times OBQ's greedy-order quantization (gptq_quantize_greedy)
of a 4096 x n fp16 layer (n = 256 by default, --obq-n), 4-bit: every row
picks its weights in order of least added loss on its own copy of H^-1.

--kernel peaks measures the chip's attainable peaks with kernels that do
nothing else (libgptq_peaks.so): dense fp16 and fp32 MFMA streams, an HBM
read stream and an HBM copy; the line gives each beside the published peak.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_TF16 = 2500.0     # MI355X dense fp16 MFMA, TFLOP/s
PEAK_TF32 = 157.3      # MI355X fp32 MFMA, TFLOP/s
PEAK_HBM = 8000.0      # GB/s
# measured on one MI355X by `bench.py --kernel peaks` (profiles/attainable_peaks.md):
# fp16 MFMA stream with random operands, fp32 MFMA stream, HBM read stream
ATTAIN_TF16 = 1726.4
ATTAIN_TF32 = 155.0
ATTAIN_HBM_READ = 6390.2

# --workload name -> (synth workload, job index)
LAYERS = {
    "tiny": ("tiny", 0), "attn": ("attn", 0), "mlp_up": ("mlp", 0), "mlp_down": ("mlp", 1),
    "qkv": ("block7b", 0), "o": ("block7b", 1), "gate_up": ("block7b", 2), "down7b": ("block7b", 3),
    "fc1": ("ffn175b", 0), "fc2": ("ffn175b", 1),
}


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", default="attn", choices=sorted(LAYERS))
    ap.add_argument("--kernel", default="layer",
                    choices=["layer", "w4a16", "rotate", "stack", "tstack", "peaks", "obq"],
                    help="layer: the quantization path (default); w4a16: the packed layer at run time; "
                         "rotate: the Hadamard rotation before GPTQ; stack / tstack: the network-level loop over "
                         "MLP / transformer blocks; peaks: measured attainable MFMA and HBM rates")
    ap.add_argument("--bits", type=int, default=4, choices=[3, 4], help="code width for --kernel w4a16")
    ap.add_argument("--obq-n", type=int, default=256, help="row length for --kernel obq (m = 4096 rows)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--traffic", default=os.path.join(ROOT, "profiles", "syrk_attn_4096x262144_traffic.json"),
                    help="JSON with rocprofv3 FETCH/WRITE bytes per SYRK launch (optional)")
    return ap.parse_args()


def host_info():
    """CPU model, memory and the BLAS numpy calls, for the CPU-baseline record."""
    import platform

    import numpy as np
    cpu = platform.processor() or ""
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    cpu = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    ram = None
    try:
        with open("/proc/meminfo") as f:
            for line in f:
                if line.startswith("MemTotal"):
                    ram = round(int(line.split()[1]) / 2 ** 20, 1)
                    break
    except OSError:
        pass
    blas = None
    try:
        b = np.show_config(mode="dicts").get("Build Dependencies", {}).get("blas", {})
        blas = f"{b.get('name')} {b.get('version')}"
    except Exception:  # noqa: BLE001 - older numpy: no dict form
        pass
    return {"cpu": cpu, "logical_cpus": os.cpu_count(), "ram_gib": ram, "blas": blas}


def cpu_baseline(W16, X16, job, U_gpu):
    """The fp64 oracle timed on a bounded sample of the same layer, scaled to
    one full layer: H over a whole number of 2048-token chunks (about 65536
    tokens at n = 4096, fewer for wider layers), the inverse factor at full
    size, the sweep over a subset of rows (about 4 M weights)."""
    import numpy as np

    import oracle as O
    T = X16.shape[0]
    n = W16.shape[1]
    m = W16.shape[0]
    tok = max(2048, min(T, int(65536 * (4096 / n) ** 2) // 2048 * 2048))
    rows = max(8, min(m, int(4 * 2 ** 20 // n)))
    t0 = time.perf_counter()
    H = O.hessian([X16[c:c + 2048] for c in range(0, tok, 2048)])
    t1 = time.perf_counter()
    Hd, _ = O.damp(H * (T / tok), job.damp)
    U, info = O.inverse_cholesky_upper(Hd)
    t2 = time.perf_counter()
    Ug = U_gpu.astype(np.float64)
    O.gptq_quantize(W16[:rows].astype(np.float64), Ug, job.bits, job.group, job.block)
    t3 = time.perf_counter()
    est = (t1 - t0) * (T / tok) + (t2 - t1) + (t3 - t2) * (m / rows)
    threads = int(os.environ.get("OMP_NUM_THREADS", os.cpu_count() or 1))
    return {"value": round(est * 1e3, 1), "unit": "ms per layer (estimated from the sample)", "cores": threads,
            "kind": "oracle", "host": host_info(),
            "sample": f"fp64 oracle: Hessian over {tok} of {T} tokens (x{T / tok:g}), full {n}x{n} inverse factor, "
                      f"sweep of {rows} of {m} rows (x{m / rows:.2f}); stage seconds "
                      f"{t1 - t0:.2f}/{t2 - t1:.2f}/{t3 - t2:.2f}"}


def pack_rows(q, bits: int):
    """Codes [m x n] (0 <= q < 2^bits) as per-row little-endian bit-streams of
    uint32 words (code j at bits [bits j, bits j + bits) of the row's stream),
    the layout gptq_quantize_layer writes; built on the host before timing."""
    import numpy as np
    m, n = q.shape
    W = (n * bits + 31) // 32
    out = np.zeros((m, W), dtype=np.uint32)
    for r0 in range(0, m, 2048):
        qb = q[r0:r0 + 2048].astype(np.uint8)
        bitsarr = ((qb[:, :, None] >> np.arange(bits, dtype=np.uint8)) & 1).reshape(qb.shape[0], n * bits)
        pad = np.zeros((qb.shape[0], W * 32 - n * bits), dtype=np.uint8)
        packed = np.packbits(np.concatenate([bitsarr, pad], axis=1), axis=1, bitorder="little")
        out[r0:r0 + 2048] = packed.view("<u4")
    return out


def bench_w4a16(args):
    """gptq_dequant_matmul on a 28672 x 8192 4-bit g128 layer (MLP up/gate
    projection shape), one fp16 decode token; synthetic packed layer (codes,
    scales, zero points) and activations from synth/.  A step is one call.
    Bytes counted: codes m n / 2, scales and zeros 8 m G, X and Y."""
    import numpy as np
    import torch

    import post_weight_quantization_10_amd as pw
    import synth
    m, n, T, group = 28672, 8192, 1, 128
    dev = torch.device("cuda:0")
    bits = args.bits
    q, s, z = synth.packed_layer(m, n, bits, group, seed=7)
    words = pack_rows(q, bits)
    qw = torch.from_numpy(words.view(np.int32)).to(dev)
    sd, zd = torch.from_numpy(s).to(dev), torch.from_numpy(z).to(dev)
    X = torch.from_numpy(synth.activations(T, n, "f16", seed=8)).to(dev)
    Y = torch.empty((T, m), dtype=torch.float16, device=dev)
    ws = torch.empty(max(pw.dequant_matmul_workspace_bytes(T, m, n), 1), dtype=torch.uint8, device=dev)
    for _ in range(max(args.warmup, 1) * 10):
        pw.dequant_matmul(X, qw, sd, zd, bits, group, Y=Y, workspace=ws)
    reps = 20 * args.steps
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(reps):
        pw.dequant_matmul(X, qw, sd, zd, bits, group, Y=Y, workspace=ws)
    torch.cuda.synchronize()
    us = (time.perf_counter() - t0) * 1e6 / reps
    # the same calls timed with HIP events on the stream the kernels run on
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record()
    for _ in range(reps):
        pw.dequant_matmul(X, qw, sd, zd, bits, group, Y=Y, workspace=ws)
    b.record()
    torch.cuda.synchronize()
    us_ev = a.elapsed_time(b) * 1e3 / reps
    G = n // group
    nbytes = m * n * bits / 8 + 8.0 * m * G + 2.0 * T * n + 2.0 * T * m
    gbs = nbytes / (us * 1e-6) / 1e9
    gbs_ev = nbytes / (us_ev * 1e-6) / 1e9
    res = {
        "metric": f"GB/s of the packed {bits}-bit layer, W{bits}A16 dequant-matmul (28672x8192 g128, 1 fp16 token)",
        "value": round(gbs, 1), "unit": "GB/s", "n_gpus": 1, "steps": reps, "warmup": args.warmup,
        "ms_per_step": round(us / 1e3, 5), "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": f"fp16 x u{bits} -> fp32 sums", "data": "synthetic",
        "config": {"workload": f"w{bits}a16 decode: W {m}x{n} {bits}-bit g{group} packed, X {T}x{n} fp16, "
                               f"Y {T}x{m} fp16",
                   "tokens": T, "m": m, "n": n, "bits": bits, "group": group, "parallelism": "single GPU"},
        "roofline": {"kernel": "gptq_dequant_matmul: dqmm4_task_kernel + dqmm_reduce_kernel", "bound": "hbm",
                     "achieved": round(gbs_ev, 1), "peak": PEAK_HBM, "unit": "GB/s",
                     "frac": round(gbs_ev / PEAK_HBM, 4), "traffic": None,
                     "attainable": {"peak": ATTAIN_HBM_READ, "frac": round(gbs_ev / ATTAIN_HBM_READ, 4),
                                    "source": "bench.py --kernel peaks (HBM read stream)"}},
    }
    if not args.no_cpu_baseline:
        import oracle as O
        rows = 1024
        t1 = time.perf_counter()
        O.dequant_matmul(synth.as_float64(X.cpu().numpy(), "f16"), words[:rows], s[:rows], z[:rows], bits, group, n)
        dt = time.perf_counter() - t1
        threads = int(os.environ.get("OMP_NUM_THREADS", os.cpu_count() or 1))
        res["cpu_baseline"] = {"value": round(nbytes / (dt * m / rows) / 1e9, 3),
                               "unit": "GB/s (estimated from the sample)", "cores": threads, "kind": "oracle",
                               "sample": f"fp64 oracle unpack + dequantize + matmul of {rows} of {m} rows "
                                         f"({dt:.2f} s), scaled x{m // rows}"}
    print(json.dumps(res), flush=True)


def traffic_bytes(path):
    """HBM bytes per Hessian launch from the committed rocprofv3 counter
    summary, or None when there is none or the kernel source has changed
    since the counters were taken."""
    import hashlib
    if not os.path.exists(path):
        return None
    with open(path) as f:
        js = json.load(f)
    src = os.path.join(ROOT, js.get("source", ""))
    if not os.path.isfile(src):
        return None
    with open(src, "rb") as f:
        if hashlib.sha256(f.read()).hexdigest() != js.get("source_sha256"):
            return None
    return js.get("bytes_per_launch")


def bench_rotate(args):
    """gptq_rotate_hadamard on 262144 x 4096 fp16 activations (block 4096), in
    place; a step is one call.  Bytes counted: every element read and written
    once (2 x 2 bytes)."""
    import numpy as np
    import torch

    import post_weight_quantization_10_amd as pw
    import synth
    T, n = 262144, 4096
    dev = torch.device("cuda:0")
    wl = synth.workloads()["attn"]
    job = wl.jobs[0]
    X = torch.from_numpy(synth.x_full(job.x, wl.seed, wl.wid)).to(dev)
    for _ in range(max(args.warmup, 1)):
        pw.rotate_hadamard(X)
    torch.cuda.synchronize()
    reps = 2 * max(args.steps, 1)
    t0 = time.perf_counter()
    for _ in range(reps):
        pw.rotate_hadamard(X)
    torch.cuda.synchronize()
    ms = (time.perf_counter() - t0) * 1e3 / reps
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record()
    for _ in range(reps):
        pw.rotate_hadamard(X)
    b.record()
    torch.cuda.synchronize()
    ms_ev = a.elapsed_time(b) / reps
    nbytes = 2.0 * 2.0 * T * n
    gbs, gbs_ev = nbytes / (ms * 1e-3) / 1e9, nbytes / (ms_ev * 1e-3) / 1e9
    res = {
        "metric": "GB/s of the Hadamard rotation before GPTQ (262144 x 4096 fp16 activations, block 4096)",
        "value": round(gbs, 1), "unit": "GB/s", "n_gpus": 1, "steps": reps, "warmup": args.warmup,
        "ms_per_step": round(ms, 4), "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "fp16 in/out, fp32 butterflies", "data": "synthetic",
        "config": {"workload": f"rotate X {T}x{n} fp16 in place, Hadamard block {n}", "tokens": T, "n": n,
                   "block": n, "parallelism": "single GPU"},
        "roofline": {"kernel": "gptq_rotate_hadamard: hadamard_rows_kernel", "bound": "hbm",
                     "achieved": round(gbs_ev, 1), "peak": PEAK_HBM, "unit": "GB/s",
                     "frac": round(gbs_ev / PEAK_HBM, 4), "traffic": None,
                     "attainable": {"peak": 4943.7, "frac": round(gbs_ev / 4943.7, 4),
                                    "source": "bench.py --kernel peaks (HBM copy stream)"}},
    }
    if not args.no_cpu_baseline:
        import oracle as O
        rows = 256
        sample = X[:rows].float().cpu().numpy().astype(np.float64)
        t1 = time.perf_counter()
        O.hadamard_rotate(sample)
        dt = time.perf_counter() - t1
        threads = int(os.environ.get("OMP_NUM_THREADS", os.cpu_count() or 1))
        res["cpu_baseline"] = {"value": round(nbytes / (dt * T / rows) / 1e9, 3),
                               "unit": "GB/s (estimated from the sample)", "cores": threads, "kind": "oracle",
                               "sample": f"fp64 oracle hadamard_rotate of {rows} of {T} rows ({dt:.2f} s), scaled"}
    print(json.dumps(res), flush=True)


def bench_obq(args):
    """gptq_quantize_greedy (OBQ's greedy order) on a 4096 x n fp16 layer,
    4-bit g128 (per-row grid when n < 128), against the factor U of a
    lognormal-input Hessian prepared on the GPU beforehand; a step is one
    call (H^-1 = U^T U packed, then every row's greedy sweep).  Flops
    counted per row: the rank-one downdates, sum over R of R (R - 1) (one
    multiply-add per entry of the (R-1)-triangle) ~ n^3 / 3."""
    import numpy as np
    import torch

    import post_weight_quantization_10_amd as pw
    import synth
    m, n, bits = 4096, args.obq_n, 4
    group = 128 if n >= 128 else 0
    dev = torch.device("cuda:0")
    W, X = synth.small_layer(m, n, 4 * 2048, seed=41, law="lognormal", w_dtype="f16", x_dtype="f16",
                             outlier_channels=2)
    Wd = torch.from_numpy(W).to(dev)
    H = torch.zeros((n, n), dtype=torch.float32, device=dev)
    pw.hessian_accumulate(H, torch.from_numpy(X).to(dev))
    U, lam, info = pw.prepare_hinv(H, 0.01)
    torch.cuda.synchronize()
    if int(info.item()) != 0:
        raise SystemExit("damped Hessian not positive definite")
    ws = torch.empty(max(pw.greedy_workspace_bytes(m, n), 1), dtype=torch.uint8, device=dev)
    out = pw.quantize_greedy(Wd, U, bits, group, workspace=ws)
    for _ in range(max(args.warmup, 1)):
        pw.quantize_greedy(Wd, U, bits, group, workspace=ws, out=out)
    torch.cuda.synchronize()
    reps = max(args.steps, 1)
    t0 = time.perf_counter()
    for _ in range(reps):
        pw.quantize_greedy(Wd, U, bits, group, workspace=ws, out=out)
    torch.cuda.synchronize()
    ms = (time.perf_counter() - t0) * 1e3 / reps
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record()
    for _ in range(reps):
        pw.quantize_greedy(Wd, U, bits, group, workspace=ws, out=out)
    b.record()
    torch.cuda.synchronize()
    ms_ev = a.elapsed_time(b) / reps
    flops = 2.0 * m * sum(R * (R - 1) / 2 for R in range(1, n + 1))
    tf_ev = flops / (ms_ev * 1e-3) / 1e12
    path = ("deferred downdates, base H^-1 in LDS, four rows per CU" if n <= 128 else
            "deferred downdates, base H^-1 in LDS" if n <= 256 else
            "deferred downdates, base H^-1 in the workspace" if n <= 1024 else "workspace-resident H^-1")
    if n <= 256:     # per 8 downdates of an entry (16 flops): 8 B of LDS for the base, under the ALU peak
        bound = {"peak": 157.3, "unit": "TFLOP/s",
                 "source": "fp32 vector peak: base and deferred columns in LDS, 0.5 B of LDS per flop "
                           "(78.6 TB/s of LDS would allow 157 TFLOP/s)"}
    elif n <= 1024:  # the base entry (8 B read + written) crosses HBM once per 16 downdates: 0.25 B per flop
        bound = {"peak": round(PEAK_HBM / 0.25 / 1e3, 2), "unit": "TFLOP/s",
                 "source": "HBM 8 TB/s, base H^-1 read and written once per 16 deferred downdates (0.25 B per flop)"}
    else:            # every downdate reads and writes the base entry: 4 B per flop
        bound = {"peak": round(PEAK_HBM / 4.0 / 1e3, 2), "unit": "TFLOP/s",
                 "source": "HBM 8 TB/s, base H^-1 read and written every downdate (4 B per flop)"}
    bound["frac"] = round(tf_ev / bound["peak"], 4)
    res = {
        "metric": f"ms per layer, OBQ greedy-order quantization ({m}x{n} fp16, 4-bit g{group or n})",
        "value": round(ms, 3), "unit": "ms", "n_gpus": 1, "steps": reps, "warmup": args.warmup,
        "ms_per_step": round(ms, 3), "higher_is_better": False, "scaling": "weak", "vs_baseline": None,
        "dtype": "f32", "data": "synthetic",
        "config": {"workload": f"OBQ greedy: W {m}x{n} fp16, H from 8192 lognormal-input tokens, "
                               f"4-bit g{group or n}, {path}",
                   "m": m, "n": n, "bits": bits, "group": group, "parallelism": "single GPU"},
        "roofline": {"kernel": "gptq_quantize_greedy: " + ("greedy_kernel" if n > 1024 else "greedy_lazy_kernel") +
                               " (+ hinv_pack_kernel)",
                     "bound": "alu",
                     "achieved": round(tf_ev, 3), "peak": 157.3, "unit": "TFLOP/s",
                     "frac": round(tf_ev / 157.3, 4), "traffic": None, "attainable": bound},
    }
    if not args.no_cpu_baseline:
        import oracle as O
        rows = 96
        Ucpu = U.cpu().numpy().astype(np.float64)
        t1 = time.perf_counter()
        O.obq_greedy(W[:rows].astype(np.float64), Ucpu, bits, group)
        dt = time.perf_counter() - t1
        threads = int(os.environ.get("OMP_NUM_THREADS", os.cpu_count() or 1))
        res["cpu_baseline"] = {"value": round(dt * m / rows * 1e3, 1), "unit": "ms per layer (estimated from the sample)",
                               "cores": threads, "kind": "oracle",
                               "sample": f"fp64 oracle obq_greedy of {rows} of {m} rows ({dt:.2f} s), "
                                         f"scaled x{m / rows:.1f}"}
    print(json.dumps(res), flush=True)


def bench_stack(args):
    """quantize_mlp_stack over 2 MLP blocks of a 7B shape (d 4096, f 11008,
    weights N(0, 0.02^2) with 0.1 % x10 outliers, fp16), 8192 calibration
    tokens of the attention-projection recipe; a step is the whole loop.
    Phase times from HIP events on the stream, one block traced by hand:
    hessian (both), prepare (both), sweeps (three), forward (three products,
    SwiGLU, residual)."""
    import numpy as np
    import torch

    import post_weight_quantization_10_amd as pw
    import synth
    d, f, T, L, bits, group, B = 4096, 11008, 8192, 2, 4, 128, 128
    dev = torch.device("cuda:0")
    blocks = []
    for l in range(L):
        ws = [synth.small_layer(r, c, 16, seed=300 + 3 * l + k, w_dtype="f16", outlier_frac=0.001)[0]
              for k, (r, c) in enumerate([(f, d), (f, d), (d, f)])]
        blocks.append(tuple(torch.from_numpy(w).to(dev) for w in ws))
    X0 = torch.from_numpy(synth.activations(T, d, "f16", seed=301)).to(dev)
    for _ in range(max(args.warmup, 1)):
        pw.quantize_mlp_stack(blocks, X0, bits, group, B, 0.01)
    torch.cuda.synchronize()
    steps = max(args.steps, 1)
    t0 = time.perf_counter()
    for _ in range(steps):
        pw.quantize_mlp_stack(blocks, X0, bits, group, B, 0.01)
    torch.cuda.synchronize()
    ms = (time.perf_counter() - t0) * 1e3 / steps
    # phases of one block, HIP events between the same calls quantize_mlp_stack makes
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(9)]
    Wg, Wu, Wd = blocks[0]
    X = X0.clone()
    ev[0].record()
    H = torch.zeros((d, d), dtype=torch.float32, device=dev)
    pw.hessian_accumulate(H, X)
    ev[1].record()
    U, _, _ = pw.prepare_hinv(H, 0.01)
    ev[2].record()
    rg = pw.quantize_layer(Wg.clone(), U, bits, group, B, write_dequant=False)
    ru = pw.quantize_layer(Wu.clone(), U, bits, group, B, write_dequant=False)
    ev[3].record()
    G = pw.dequant_matmul(X, rg["qcodes"], rg["scales"], rg["zeros"], bits, group)
    Uo = pw.dequant_matmul(X, ru["qcodes"], ru["scales"], ru["zeros"], bits, group)
    A = pw.swiglu(G, Uo)
    ev[4].record()
    H2 = torch.zeros((f, f), dtype=torch.float32, device=dev)
    pw.hessian_accumulate(H2, A)
    ev[5].record()
    U2, _, _ = pw.prepare_hinv(H2, 0.01)
    ev[6].record()
    rd = pw.quantize_layer(Wd.clone(), U2, bits, group, B, write_dequant=False)
    ev[7].record()
    Y = pw.dequant_matmul(A, rd["qcodes"], rd["scales"], rd["zeros"], bits, group)
    pw.residual_add(X, Y)
    ev[8].record()
    torch.cuda.synchronize()
    t = [ev[i].elapsed_time(ev[i + 1]) for i in range(8)]
    phases = {"hessian": round(t[0] + t[4], 3), "prepare": round(t[1] + t[5], 3), "sweeps": round(t[2] + t[6], 3),
              "forward": round(t[3] + t[7], 3)}
    fwd_flops = 2.0 * T * d * f * 3
    fwd_ms = t[3] + t[7]
    res = {
        "metric": "ms per 7B-shaped MLP block of the network-level loop (d 4096, f 11008, 8192 tokens, 4-bit g128)",
        "value": round(ms / L, 3), "unit": "ms", "n_gpus": 1, "steps": steps, "warmup": args.warmup,
        "ms_per_step": round(ms, 3), "higher_is_better": False, "scaling": "weak", "vs_baseline": None,
        "dtype": "fp16 MFMA (H, forward) / fp32", "data": "synthetic",
        "config": {"workload": f"{L} MLP blocks d {d} f {f}, X0 {T}x{d} fp16, {bits}-bit g{group} B{B}",
                   "tokens": T, "d": d, "f": f, "blocks": L, "parallelism": "single GPU"},
        "phases_ms_one_block": phases,
        "roofline": {"kernel": "gptq_dequant_matmul (many tokens: dqmm4_gemm_kernel), the block's forward products",
                     "bound": "mfma", "achieved": round(fwd_flops / (fwd_ms * 1e-3) / 1e12, 2), "peak": PEAK_TF16,
                     "unit": "TFLOP/s", "frac": round(fwd_flops / (fwd_ms * 1e-3) / 1e12 / PEAK_TF16, 4),
                     "traffic": None},
    }
    print(json.dumps(res), flush=True)


def bench_tstack(args):
    """quantize_transformer_stack over 2 transformer blocks of a 7B shape
    (d 4096, f 11008, 32 heads of 128, no normalisation; weights N(0, 1/fan-in)
    with 0.1 % x10 outliers, fp16), 8192 calibration tokens of the
    attention-projection recipe in sequences of 2048; a step is the whole loop.
    Phase times of one block from HIP events between the same calls the loop
    makes: hessian (four), prepare (four), sweeps (q/k/v stacked, o, gate/up
    stacked, down), attention, the rest of the forward (the quantized
    products, SwiGLU, the residuals)."""
    import torch

    import post_weight_quantization_10_amd as pw
    import synth
    d, f, heads, seq, T, L, bits, group, B = 4096, 11008, 32, 2048, 8192, 2, 4, 128, 128
    dev = torch.device("cuda:0")
    blocks = []
    # weights of std 1/sqrt(fan-in): with no normalisation between blocks,
    # 0.02 (the single-layer recipe) grows the residual stream ~50x a block
    # and overflows fp16 in the second block's SwiGLU
    for l in range(L):
        shapes = [(d, d)] * 4 + [(f, d), (f, d), (d, f)]
        ws = [synth.small_layer(r, c, 16, seed=400 + 7 * l + k, w_dtype="f16", sigma=c ** -0.5,
                                outlier_frac=0.001)[0]
              for k, (r, c) in enumerate(shapes)]
        blocks.append(tuple(torch.from_numpy(w).to(dev) for w in ws))
    X0 = torch.from_numpy(synth.activations(T, d, "f16", seed=401)).to(dev)
    for _ in range(max(args.warmup, 1)):
        pw.quantize_transformer_stack(blocks, X0, seq, heads, bits, group, B, 0.01)
    torch.cuda.synchronize()
    steps = max(args.steps, 1)
    t0 = time.perf_counter()
    for _ in range(steps):
        pw.quantize_transformer_stack(blocks, X0, seq, heads, bits, group, B, 0.01)
    torch.cuda.synchronize()
    ms = (time.perf_counter() - t0) * 1e3 / steps

    # one block by hand, HIP events between the calls the loop makes
    Wq, Wk, Wv, Wo, Wg, Wu, Wd = blocks[0]
    acc = {"hessian": 0.0, "prepare": 0.0, "sweeps": 0.0, "attention": 0.0, "forward": 0.0}
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(2)]

    def timed(key, fn):
        ev[0].record()
        r = fn()
        ev[1].record()
        torch.cuda.synchronize()
        acc[key] += ev[0].elapsed_time(ev[1])
        return r

    def factor(Xa):
        n = Xa.shape[1]
        H = torch.zeros((n, n), dtype=torch.float32, device=dev)
        timed("hessian", lambda: pw.hessian_accumulate(H, Xa))
        return timed("prepare", lambda: pw.prepare_hinv(H, 0.01))[0]

    def product(Xa, r):
        return pw.dequant_matmul(Xa, r["qcodes"], r["scales"], r["zeros"], bits, group)

    X = X0.clone()
    U1 = factor(X)
    Wqkv = torch.cat([Wq, Wk, Wv], dim=0)
    rqkv = timed("sweeps", lambda: pw.quantize_layer(Wqkv, U1, bits, group, B, write_dequant=False))
    qkv = timed("forward", lambda: product(X, rqkv))
    A = timed("attention", lambda: pw.attention(qkv[:, :d], qkv[:, d:2 * d], qkv[:, 2 * d:], seq, heads))
    U2 = factor(A)
    ro = timed("sweeps", lambda: pw.quantize_layer(Wo.clone(), U2, bits, group, B, write_dequant=False))
    timed("forward", lambda: pw.residual_add(X, product(A, ro)))
    U3 = factor(X)
    Wgu = torch.cat([Wg, Wu], dim=0)
    rgu = timed("sweeps", lambda: pw.quantize_layer(Wgu, U3, bits, group, B, write_dequant=False))
    A2 = timed("forward", lambda: (lambda GU: pw.swiglu(GU[:, :f], GU[:, f:]))(product(X, rgu)))
    U4 = factor(A2)
    rd = timed("sweeps", lambda: pw.quantize_layer(Wd.clone(), U4, bits, group, B, write_dequant=False))
    timed("forward", lambda: pw.residual_add(X, product(A2, rd)))
    att_flops = 4.0 * d * T * (seq + 1) / 2  # QK and PV, causal: (seq + 1) / 2 keys per query on average
    att_ms = acc["attention"]
    res = {
        "metric": "ms per 7B-shaped transformer block of the network-level loop (d 4096, f 11008, 32 heads, "
                  "8192 tokens in sequences of 2048, 4-bit g128)",
        "value": round(ms / L, 3), "unit": "ms", "n_gpus": 1, "steps": steps, "warmup": args.warmup,
        "ms_per_step": round(ms, 3), "higher_is_better": False, "scaling": "weak", "vs_baseline": None,
        "dtype": "fp16 MFMA (H, products) / fp32", "data": "synthetic",
        "config": {"workload": f"{L} transformer blocks d {d} f {f} heads {heads}, X0 {T}x{d} fp16 "
                               f"(sequences of {seq}), {bits}-bit g{group} B{B}",
                   "tokens": T, "d": d, "f": f, "heads": heads, "seq_len": seq, "blocks": L,
                   "parallelism": "single GPU"},
        "phases_ms_one_block": {k: round(v, 3) for k, v in acc.items()},
        "roofline": {"kernel": "gptq_attention (attention_kernel: causal softmax attention, fp32 VALU)",
                     "bound": "alu", "achieved": round(att_flops / (att_ms * 1e-3) / 1e12, 2), "peak": PEAK_TF32,
                     "unit": "TFLOP/s", "frac": round(att_flops / (att_ms * 1e-3) / 1e12 / PEAK_TF32, 4),
                     "traffic": None},
    }
    print(json.dumps(res), flush=True)


def bench_peaks(args):
    """Attainable peaks, each the best of a few timed launches on the current
    stream (HIP events): MFMA streams of 1024 workgroups x 4 waves, eight
    independent accumulators per wave; HBM read of 4 GiB and copy of 2 GiB,
    grid 4096 x 256 threads."""
    import ctypes

    import torch

    from post_weight_quantization_10_amd import build as B
    if not os.path.exists(B.PROBE_PATH):
        raise RuntimeError(f"{B.PROBE_PATH} is missing: build it with python -m post_weight_quantization_10_amd.build")
    L = ctypes.CDLL(B.PROBE_PATH)
    L.gptq_peaks_launch.argtypes = [ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_size_t, ctypes.c_int,
                                    ctypes.c_int, ctypes.c_void_p]
    L.gptq_peaks_launch.restype = ctypes.c_int
    dev = torch.device("cuda:0")
    st = torch.cuda.current_stream().cuda_stream
    reps = max(3, args.steps)

    def best(fn):
        fn()
        torch.cuda.synchronize()
        ts = []
        for _ in range(reps):
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record()
            fn()
            b.record()
            torch.cuda.synchronize()
            ts.append(a.elapsed_time(b) * 1e-3)
        return min(ts)

    out = {}
    g_mfma, iters = 1024, 2048
    bits = torch.randint(-2 ** 31, 2 ** 31 - 1, (g_mfma * 256 * 4,), dtype=torch.int32, device=dev)
    sink = torch.empty(g_mfma * 256, dtype=torch.float32, device=dev)
    for which, key, flop in ((0, "mfma_fp16", 2 * 32 * 32 * 16), (1, "mfma_fp32", 2 * 32 * 32 * 2)):
        def run(which=which):
            assert L.gptq_peaks_launch(which, bits.data_ptr(), sink.data_ptr(), 0, iters, g_mfma, st) == 0
        t = best(run)
        out[key] = g_mfma * 4 * iters * 16 * flop / t / 1e12
    nbytes = 4 << 30
    src = torch.empty(nbytes // 4, dtype=torch.int32, device=dev).random_()
    words = torch.empty(4096 * 256, dtype=torch.int32, device=dev)
    t = best(lambda: L.gptq_peaks_launch(2, src.data_ptr(), words.data_ptr(), nbytes, 0, 4096, st))
    out["hbm_read"] = nbytes / t / 1e9
    half = nbytes // 2
    dst = torch.empty(half // 4, dtype=torch.int32, device=dev)
    t = best(lambda: L.gptq_peaks_launch(3, src.data_ptr(), dst.data_ptr(), half, 0, 4096, st))
    out["hbm_copy"] = 2 * half / t / 1e9
    assert torch.equal(dst, src[: half // 4])
    spec = {"mfma_fp16": PEAK_TF16, "mfma_fp32": PEAK_TF32, "hbm_read": PEAK_HBM, "hbm_copy": PEAK_HBM}
    units = {"mfma_fp16": "TFLOP/s", "mfma_fp32": "TFLOP/s", "hbm_read": "GB/s", "hbm_copy": "GB/s (read + write)"}
    res = {"metric": "measured attainable peaks (MFMA streams, HBM streams)", "value": round(out["mfma_fp16"], 1),
           "unit": "TFLOP/s (fp16 MFMA)", "n_gpus": 1, "steps": reps, "warmup": 1, "higher_is_better": True,
           "scaling": "weak", "vs_baseline": None, "dtype": "fp16/fp32 MFMA, u32 loads", "data": "synthetic",
           "config": {"workload": "peak probes: MFMA 1024 workgroups x 4 waves x 2048 x 16 instructions; "
                                  "HBM read 4 GiB, copy 2 GiB"},
           "peaks": {k: {"measured": round(v, 1), "published": spec[k], "unit": units[k],
                         "frac": round(v / spec[k], 4)} for k, v in out.items()}}
    print(json.dumps(res), flush=True)


def main():
    args = parse()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py runs on one GPU only: the quantizer's data-parallel path here is a single-GPU build "
              "(multi-GPU sharding is a design note, not implemented)", file=sys.stderr)
        sys.exit(2)
    if args.kernel == "w4a16":
        bench_w4a16(args)
        return
    if args.kernel == "peaks":
        bench_peaks(args)
        return
    if args.kernel == "rotate":
        bench_rotate(args)
        return
    if args.kernel == "stack":
        bench_stack(args)
        return
    if args.kernel == "tstack":
        bench_tstack(args)
        return
    if args.kernel == "obq":
        bench_obq(args)
        return
    bench_layer(args)


def trailing_schedule(m: int, n: int, B: int, group: int, cus: int = 256):
    """Flops of the trailing update m n (n - B) split as gptq_quantize_layer
    runs it: (flops in the GEMM kernels, flops applied inside the sweep
    kernel).  With B a multiple of 64 and groups no wider than a block:
    while the rows fit one 16-row workgroup per CU, one launch sweeps a whole
    1024-column superblock, every block taking the superblock's earlier errors
    inside the kernel, and a GEMM with K = 1024 updates the rest of the row
    after each superblock; otherwise the blocks go in pairs: the second block
    of a pair takes the first one's errors on its own columns inside the
    sweep, then GEMMs update the columns after the pair (those of its
    1024-column superblock at once, the rest after the superblock with
    K = 1024; the same flops either way)."""
    look = B % 64 == 0 and (group <= 0 or group <= B) and n % 4 == 0
    gemm = in_sweep = 0.0
    if look and -(-m // 16) <= cus:
        for s0 in range(0, n, 1024):
            s1 = min(s0 + 1024, n)
            for i in range(s0, s1, B):
                in_sweep += 2.0 * m * (i - s0) * min(B, s1 - i)
            gemm += 2.0 * m * (s1 - s0) * (n - s1)
    elif look:
        g0 = 0
        while g0 < n:
            w1 = min(B, n - g0)
            w2 = min(B, n - g0 - w1)
            in_sweep += 2.0 * m * w1 * w2
            i = g0 + w1 + w2
            gemm += 2.0 * m * (i - g0) * (n - i)
            g0 = i
    else:
        for i in range(0, n, B):
            w = min(B, n - i)
            gemm += 2.0 * m * w * (n - i - w)
    return gemm, in_sweep


def kernel_ms(fn, groups):
    """GPU durations (ms) of the kernels fn() launches, summed per group of
    kernel-name substrings, from torch.profiler's device activity; None when
    the profiler gives no device events."""
    import torch
    from torch.profiler import ProfilerActivity, profile
    torch.cuda.synchronize()
    with profile(activities=[ProfilerActivity.CUDA]) as prof:
        fn()
        torch.cuda.synchronize()
    tot = {g: 0.0 for g in groups}
    seen = 0
    for e in prof.key_averages():
        us = getattr(e, "device_time_total", None)
        if us is None:
            us = getattr(e, "cuda_time_total", 0.0)
        if not us:
            continue
        for g, subs in groups.items():
            if any(k in e.key for k in subs):
                tot[g] += us / 1e3
                seen += 1
                break
    return tot if seen else None


def _phase(ms_list, work, unit, peak, attain=None, attain_src=None, scale=1e12):
    import numpy as np
    med, mn = float(np.median(ms_list)), float(np.min(ms_list))
    rate = work / (med * 1e-3) / scale
    d = {"ms_median": round(med, 4), "ms_min": round(mn, 4), "work": work, "achieved": round(rate, 2),
         "unit": unit, "peak": peak, "frac": round(rate / peak, 4)}
    if attain:
        d["attainable"] = {"peak": attain, "frac": round(rate / attain, 4), "source": attain_src}
    return d


def bench_layer(args):
    import numpy as np
    import torch

    import post_weight_quantization_10_amd as pw
    import synth

    dev = torch.device("cuda:0")
    wkey, jidx = LAYERS[args.workload]
    wl = synth.workloads()[wkey]
    job = wl.jobs[jidx]
    t_gen = time.perf_counter()
    W_np = synth.stacked_weight(job, wl.seed, wl.wid)
    X_np = synth.x_full(job.x, wl.seed, wl.wid)
    t_gen = time.perf_counter() - t_gen
    m, n = W_np.shape
    T = X_np.shape[0]
    B, bits, group = job.block, job.bits, job.group
    W0 = torch.from_numpy(W_np).to(dev)
    X = torch.from_numpy(X_np).to(dev)
    keep_host = not args.no_cpu_baseline
    if not keep_host:
        del X_np
    Wk = W0.clone()
    H = torch.zeros((n, n), dtype=torch.float32, device=dev)
    U = torch.empty_like(H)
    hws = torch.empty(max(pw.hessian_workspace_bytes(n, T), 1), dtype=torch.uint8, device=dev)
    pws = torch.empty(pw.prepare_workspace_bytes(n), dtype=torch.uint8, device=dev)
    qws = torch.empty(pw.quantize_workspace_bytes(m, n, B), dtype=torch.uint8, device=dev)
    G = pw.n_groups(n, group)
    out = {
        "qcodes": torch.empty((m, pw.packed_words(n, bits)), dtype=torch.int32, device=dev),
        "scales": torch.empty((m, G), dtype=torch.float32, device=dev),
        "zeros": torch.empty((m, G), dtype=torch.int32, device=dev),
        "err_sq": torch.empty((m,), dtype=torch.float32, device=dev),
    }
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(4)]
    phase = {"hessian": [], "prepare": [], "quantize": []}
    info_t = None

    def hess():
        pw.hessian_accumulate(H, X, workspace=hws)

    def prep():
        nonlocal info_t
        _, _, info_t = pw.prepare_hinv(H, job.damp, U=U, workspace=pws)

    def quant():
        pw.quantize_layer(Wk, U, bits, group, B, write_dequant=True, workspace=qws, out=out)

    def step(record: bool):
        Wk.copy_(W0)
        H.zero_()
        ev[0].record()
        hess()
        ev[1].record()
        prep()
        ev[2].record()
        quant()
        ev[3].record()
        if record:
            torch.cuda.synchronize()
            phase["hessian"].append(ev[0].elapsed_time(ev[1]))
            phase["prepare"].append(ev[1].elapsed_time(ev[2]))
            phase["quantize"].append(ev[2].elapsed_time(ev[3]))

    for _ in range(args.warmup):
        step(False)
    torch.cuda.synchronize()
    print(f"# {args.workload}: inputs generated in {t_gen:.1f}s; warmup done", file=sys.stderr, flush=True)
    # timed region: exactly K steps, synchronized on both sides
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        step(False)
    torch.cuda.synchronize()
    ms_step = (time.perf_counter() - t0) * 1e3 / args.steps
    # per-phase HIP-event timings over max(K, 20) further steps (same stream as the kernels)
    for _ in range(max(args.steps, 20)):
        step(True)
    assert int(info_t.item()) == 0, "damped Hessian not positive definite"
    print("# timed; splitting the quantize phase", file=sys.stderr, flush=True)

    # the quantize phase's kernels, by GPU duration (one further step of it)
    split = None
    try:
        Wk.copy_(W0)
        split = kernel_ms(quant, {"sweep": ("sweep_block_kernel", "sweep_superblock_kernel"),
                                  "trailing_gemm": ("gemm_nn_dma_kernel", "gemm_nn_dma64_kernel", "gemm_f32_kernel",
                                                    "gemm_split_reduce", "gemm_x3_kernel", "split_t_kernel"),
                                  "other": ("to_f32", "diag_blocks", "row_params", "pack_kernel", "dequant",
                                            "zero_f32")})
    except Exception as exc:  # noqa: BLE001 - the split is reported as missing, the rest stands
        print(f"# quantize-phase split unavailable: {exc}", file=sys.stderr, flush=True)
    if split:
        # the kernel durations of one quantize step must add up to about the
        # event-timed phase; under an outside profiler torch's own can attribute
        # them wrongly, and then no split is reported
        q_med = float(np.median(phase["quantize"]))
        tot = sum(split.values())
        if not 0.6 * q_med <= tot <= 1.3 * q_med:
            print(f"# quantize-phase split dropped: kernels sum to {tot:.3f} ms against a {q_med:.3f} ms phase",
                  file=sys.stderr, flush=True)
            split = None

    syrk_flop = float(n) * (n + 1) * T
    prep_flop = 4.0 * n ** 3 / 3
    gemm_flop, in_sweep_flop = trailing_schedule(m, n, B, group,
                                                 torch.cuda.get_device_properties(dev).multi_processor_count)
    sweep_bytes = m * n * (4 + 4 + bits / 8) + 8.0 * m * G + 4.0 * n * B
    ph = {
        "syrk": _phase(phase["hessian"], syrk_flop, "TFLOP/s", PEAK_TF16, ATTAIN_TF16,
                       "bench.py --kernel peaks (fp16 MFMA stream, random operands)"),
        "prepare": _phase(phase["prepare"], prep_flop, "TFLOP/s", PEAK_TF32, ATTAIN_TF32,
                          "bench.py --kernel peaks (fp32 MFMA stream)"),
        "quantize": {"ms_median": round(float(np.median(phase["quantize"])), 4),
                     "ms_min": round(float(np.min(phase["quantize"])), 4)},
    }
    ph["prepare"]["work_note"] = (f"4n^3/3 algorithmic flops; the route run here executes 2n^3/3 "
                                  f"({2.0 * n ** 3 / 3:.4g}), frac on that basis "
                                  f"{ph['prepare']['frac'] / 2:.4f}")
    if split:
        g_ms, s_ms = split["trailing_gemm"], split["sweep"]
        # the flushes run as three bf16 products (fp32 operands split hi / lo)
        # on the look-ahead paths for rows up to 16384 columns
        x3 = B % 64 == 0 and (group <= 0 or group <= B) and n % 4 == 0 and n <= 16384
        if g_ms > 0:
            rate = gemm_flop / (g_ms * 1e-3) / 1e12
            note = (f"flops the GEMM kernels perform of m n (n - B) = {float(m) * n * (n - B):.4g}; "
                    f"{in_sweep_flop:.4g} more are applied inside the sweep kernel")
            if x3:
                ex = 3.0 * rate  # executed on the 16-bit matrix cores
                ph["trailing_gemm"] = {"ms": round(g_ms, 4), "work": gemm_flop, "algorithmic_tflops": round(rate, 2),
                                       "achieved": round(ex, 2), "unit": "TFLOP/s (bf16 MFMA, 3 products per fp32 "
                                       "product)", "peak": PEAK_TF16, "frac": round(ex / PEAK_TF16, 4),
                                       "attainable": {"peak": ATTAIN_TF16, "frac": round(ex / ATTAIN_TF16, 4),
                                                      "source": "bench.py --kernel peaks (fp16 MFMA stream, random operands)"},
                                       "work_note": note + "; each fp32 product runs as E_hi U_hi + E_hi U_lo + "
                                                           "E_lo U_hi in bf16 with fp32 accumulation (the split "
                                                           "and transpose of U included in the time)"}
            else:
                ph["trailing_gemm"] = {"ms": round(g_ms, 4), "work": gemm_flop, "achieved": round(rate, 2),
                                       "unit": "TFLOP/s", "peak": PEAK_TF32, "frac": round(rate / PEAK_TF32, 4),
                                       "attainable": {"peak": ATTAIN_TF32, "frac": round(rate / ATTAIN_TF32, 4),
                                                      "source": "bench.py --kernel peaks (fp32 MFMA stream)"},
                                       "work_note": note}
        if s_ms > 0:
            rate = sweep_bytes / (s_ms * 1e-3) / 1e9
            ph["sweep"] = {"ms": round(s_ms, 4), "work": sweep_bytes, "achieved": round(rate, 1), "unit": "GB/s",
                           "peak": PEAK_HBM, "frac": round(rate / PEAK_HBM, 4),
                           "attainable": {"peak": ATTAIN_HBM_READ, "frac": round(rate / ATTAIN_HBM_READ, 4),
                                          "source": "bench.py --kernel peaks (HBM read stream)"},
                           "latency_floor_us": [round(n * c / 2.4e3, 1) for c in (20, 50)],
                           "work_note": "m n (4 + 4 + b/8) + 8 m G + 4 n B bytes: V read, E written, codes, "
                                        "scales and zeros, the factor's diagonal blocks; the sweep kernels "
                                        f"also apply {in_sweep_flop:.4g} flops of the trailing update on MFMA"}
        ph["quantize"]["other_ms"] = round(split["other"], 4)
    achieved = ph["syrk"]["achieved"]
    traffic = traffic_bytes(args.traffic) if args.workload == "attn" else None
    med_total = sum(ph[k]["ms_median"] for k in ("syrk", "prepare", "quantize"))
    res = {
        "metric": "ms per 4096x4096 4-bit g128 GPTQ layer (incl. H^-1) + % MFMA/HBM roofline"
                  if args.workload == "attn" else f"ms per GPTQ layer ({args.workload}, incl. H and H^-1)",
        "value": round(ms_step, 3),
        "unit": "ms",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 3),
        "higher_is_better": False,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "fp16 MFMA (H) / fp32 (trailing products as 3 bf16 MFMA products up to 16384 columns)",
        "data": "synthetic",
        "config": {
            "workload": f"{args.workload}: W {m}x{n} {job.weights[0].dtype}, X {T} tokens x {n} {job.x.dtype}, "
                        f"{bits}-bit, group {group}, block {B}, damp {job.damp}",
            "tokens": T, "m": m, "n": n, "bits": bits, "group": group, "block": B,
            "parallelism": "single GPU",
        },
        "phases_ms": {"hessian": ph["syrk"]["ms_median"], "prepare": ph["prepare"]["ms_median"],
                      "quantize": ph["quantize"]["ms_median"]},
        "ms_layer_incl_hinv": round(ph["prepare"]["ms_median"] + ph["quantize"]["ms_median"], 4),
        "ms_layer_incl_hinv_min": round(ph["prepare"]["ms_min"] + ph["quantize"]["ms_min"], 4),
        "ms_step_event_median": round(med_total, 4),
        "roofline": {
            "kernel": "gptq_hessian_accumulate, H += 2 X^T X: syrk16_dma_kernel (MFMA fp16) + syrk_reduce_kernel",
            "bound": "mfma",
            "achieved": achieved,
            "peak": PEAK_TF16,
            "unit": "TFLOP/s",
            "frac": ph["syrk"]["frac"],
            "traffic": traffic,
            "attainable": ph["syrk"]["attainable"],
            "phases": ph,
        },
    }
    if not args.no_cpu_baseline:
        res["cpu_baseline"] = cpu_baseline(W_np, X_np, job, U.cpu().numpy())
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
