"""Seeded synthetic workloads for GPTQ layer quantization.

This module only draws random numbers and arranges them into the shapes the
quantizer consumes; it holds none of the method's arithmetic.  Both the fp64
oracle and the GPU path read the bytes produced here, so the two sides see
identical inputs.

Streams: every tensor (and every 2048-token chunk of an activation matrix) has
its own numpy PCG64 stream seeded by
``SeedSequence(seed, spawn_key=(workload_id, tensor_tag, chunk))``, so any
chunk can be regenerated on its own, in any order, from any thread.

Layouts: W is ``[m x n]`` row-major (output features x input features).
Calibration activations are token-major ``[tokens x n]``: one row per token,
so a chunk of 2048 tokens is a contiguous slab.

Workloads (shapes and laws of the five layer configurations this library is
measured on):

* ``tiny``      W 64x128 fp32 ~N(0, 0.02^2); X: 2048 tokens of x = L z with L
                unit lower-triangular, off-diagonal ~N(0, 0.1^2); 4-bit per-row,
                block 32.
* ``attn``      W 4096x4096 fp16 ~N(0, 0.02^2), 0.1 % of entries x10;
                X 262144 x 4096 fp16, x = z * s_c, s_c ~ LogNormal(0, 1), 8
                channels x20; 4-bit, group 128, block 128.
* ``mlp``       up 11008x4096 with X as ``attn``; down 4096x11008 with
                X = SiLU(z * s_c); fp16; 3-bit per-row, block 128.
* ``block7b``   q/k/v stacked 12288x4096 (one Hessian), o 4096x4096,
                gate/up stacked 22016x4096 (one Hessian), down 4096x11008;
                65536 tokens; 4-bit, group 128, block 128.
* ``ffn175b``   fc1 49152x12288, fc2 12288x49152, fp16 ~N(0, 0.01^2) with
                0.05 % of entries x10; X 262144 tokens, x = z * |t_4|_c
                (Student-t, 4 degrees of freedom); 3-bit, group 128, block 128.
"""
from __future__ import annotations

import concurrent.futures as _cf
import dataclasses
import os
from typing import Dict, List, Optional, Sequence, Tuple

import numpy as np

CHUNK = 2048  # tokens per calibration sequence / generation chunk

_TAGS = {"W": 1, "Xscale": 2, "Xz": 3, "Wout": 4, "L": 5, "P": 6, "A": 7}


def _rng(seed: int, workload_id: int, tensor: str, chunk: int = 0, sub: int = 0) -> np.random.Generator:
    tag = _TAGS[tensor.split(":")[0]]
    name_key = sum(ord(c) * (i + 1) for i, c in enumerate(tensor)) % 100003
    ss = np.random.SeedSequence(seed, spawn_key=(workload_id, tag, name_key, chunk, sub))
    return np.random.Generator(np.random.PCG64(ss))


@dataclasses.dataclass(frozen=True)
class XSpec:
    """How one calibration-activation matrix is drawn."""
    name: str          # stream name (distinct matrices get distinct names)
    n: int             # features (columns of W that consume it)
    tokens: int
    law: str           # "corr" | "lognormal" | "silu" | "student_t"
    dtype: str         # "f32" | "f16" | "bf16"
    outlier_channels: int = 0
    outlier_mult: float = 1.0
    corr_sigma: float = 0.1


@dataclasses.dataclass(frozen=True)
class WSpec:
    """How one weight matrix is drawn."""
    name: str
    m: int
    n: int
    sigma: float
    dtype: str
    outlier_frac: float = 0.0
    outlier_mult: float = 1.0


@dataclasses.dataclass(frozen=True)
class Job:
    """One Hessian and the (row-stacked) weights quantized against it."""
    x: XSpec
    weights: Tuple[WSpec, ...]
    bits: int
    group: int      # <= 0: one scale/zero per row
    block: int
    damp: float = 0.01


@dataclasses.dataclass(frozen=True)
class Workload:
    key: str
    wid: int
    jobs: Tuple[Job, ...]
    seed: int = 0


def _attn_x(name, n, tokens):
    return XSpec(name, n, tokens, "lognormal", "f16", outlier_channels=8, outlier_mult=20.0)


def workloads() -> Dict[str, Workload]:
    T = 128 * CHUNK
    tiny = Workload("tiny", 1, (Job(XSpec("x", 128, CHUNK, "corr", "f32"),
                                    (WSpec("w", 64, 128, 0.02, "f32"),), bits=4, group=0, block=32),))
    attn = Workload("attn", 2, (Job(_attn_x("x", 4096, T),
                                    (WSpec("w", 4096, 4096, 0.02, "f16", 0.001, 10.0),),
                                    bits=4, group=128, block=128),))
    mlp = Workload("mlp", 3, (
        Job(_attn_x("x_up", 4096, T), (WSpec("up", 11008, 4096, 0.02, "f16"),), bits=3, group=0, block=128),
        Job(XSpec("x_down", 11008, T, "silu", "f16"), (WSpec("down", 4096, 11008, 0.02, "f16"),),
            bits=3, group=0, block=128),
    ))
    T4 = 32 * CHUNK
    blk = Workload("block7b", 4, (
        Job(_attn_x("x_qkv", 4096, T4), tuple(WSpec(nm, 4096, 4096, 0.02, "f16") for nm in ("q", "k", "v")),
            bits=4, group=128, block=128),
        Job(_attn_x("x_o", 4096, T4), (WSpec("o", 4096, 4096, 0.02, "f16"),), bits=4, group=128, block=128),
        Job(_attn_x("x_gu", 4096, T4), (WSpec("gate", 11008, 4096, 0.02, "f16"), WSpec("up", 11008, 4096, 0.02, "f16")),
            bits=4, group=128, block=128),
        Job(XSpec("x_down", 11008, T4, "silu", "f16"), (WSpec("down", 4096, 11008, 0.02, "f16"),),
            bits=4, group=128, block=128),
    ))
    ffn = Workload("ffn175b", 5, (
        Job(XSpec("x_fc1", 12288, T, "student_t", "f16"), (WSpec("fc1", 49152, 12288, 0.01, "f16", 0.0005, 10.0),),
            bits=3, group=128, block=128),
        Job(XSpec("x_fc2", 49152, T, "student_t", "f16"), (WSpec("fc2", 12288, 49152, 0.01, "f16", 0.0005, 10.0),),
            bits=3, group=128, block=128),
    ))
    return {w.key: w for w in (tiny, attn, mlp, blk, ffn)}


_NP = {"f32": np.float32, "f16": np.float16, "bf16": None}


def _cast(a: np.ndarray, dtype: str) -> np.ndarray:
    if dtype == "f32":
        return np.ascontiguousarray(a, dtype=np.float32)
    if dtype == "f16":
        return np.ascontiguousarray(a, dtype=np.float16)
    if dtype == "bf16":
        # round-to-nearest-even to bfloat16, returned as the raw uint16 bit pattern
        f = np.ascontiguousarray(a, dtype=np.float32).view(np.uint32)
        r = ((f >> 16) & 1) + 0x7FFF
        return ((f + r) >> 16).astype(np.uint16)
    raise ValueError(dtype)


def bf16_bits_to_f32(u16: np.ndarray) -> np.ndarray:
    return (u16.astype(np.uint32) << 16).view(np.float32)


# ----------------------------------------------------------------------------- weights

def weight(spec: WSpec, seed: int = 0, wid: int = 0, row_block: int = 1024) -> np.ndarray:
    """W [m x n] in spec.dtype: ~N(0, sigma^2); a fraction of entries (drawn
    without replacement) multiplied by outlier_mult."""
    out = np.empty((spec.m, spec.n), dtype=np.float32)
    for r0 in range(0, spec.m, row_block):
        r1 = min(spec.m, r0 + row_block)
        g = _rng(seed, wid, "W:" + spec.name, chunk=r0 // row_block)
        out[r0:r1] = g.standard_normal((r1 - r0, spec.n), dtype=np.float32) * np.float32(spec.sigma)
    k = int(round(spec.outlier_frac * spec.m * spec.n))
    if k > 0:
        g = _rng(seed, wid, "Wout:" + spec.name)
        idx = g.choice(spec.m * spec.n, size=k, replace=False)
        flat = out.reshape(-1)
        flat[idx] *= np.float32(spec.outlier_mult)
    return _cast(out, spec.dtype)


def stacked_weight(job: Job, seed: int = 0, wid: int = 0) -> np.ndarray:
    """Rows of every layer that shares the job's Hessian, stacked along m."""
    ws = [weight(s, seed, wid) for s in job.weights]
    return ws[0] if len(ws) == 1 else np.concatenate(ws, axis=0)


# ----------------------------------------------------------------------------- activations

def channel_scales(x: XSpec, seed: int = 0, wid: int = 0) -> np.ndarray:
    """Per-channel multipliers (float32, length n) for the lognormal / silu /
    student_t laws; ones for 'corr'."""
    g = _rng(seed, wid, "Xscale:" + x.name)
    if x.law in ("lognormal", "silu"):
        s = g.lognormal(0.0, 1.0, size=x.n)
    elif x.law == "student_t":
        s = np.abs(g.standard_t(4.0, size=x.n))
    elif x.law == "corr":
        return np.ones(x.n, dtype=np.float32)
    else:
        raise ValueError(x.law)
    if x.outlier_channels:
        idx = g.choice(x.n, size=x.outlier_channels, replace=False)
        s[idx] *= x.outlier_mult
    return s.astype(np.float32)


def corr_factor(x: XSpec, seed: int = 0, wid: int = 0) -> np.ndarray:
    """Unit lower-triangular L (float64) for the 'corr' law."""
    g = _rng(seed, wid, "L:" + x.name)
    L = np.tril(g.standard_normal((x.n, x.n)) * x.corr_sigma, k=-1)
    L[np.diag_indices(x.n)] = 1.0
    return L


def x_chunk(x: XSpec, chunk: int, seed: int = 0, wid: int = 0, scales: Optional[np.ndarray] = None,
            L: Optional[np.ndarray] = None) -> np.ndarray:
    """Tokens [chunk*2048, ...) of X as a [rows x n] array in x.dtype (bf16 as raw uint16)."""
    rows = min(CHUNK, x.tokens - chunk * CHUNK)
    if rows <= 0:
        raise IndexError(chunk)
    g = _rng(seed, wid, "Xz:" + x.name, chunk=chunk)
    if x.law == "corr":
        z = g.standard_normal((rows, x.n))
        if L is None:
            L = corr_factor(x, seed, wid)
        return _cast(z @ L.T, x.dtype)
    z = g.standard_normal((rows, x.n), dtype=np.float32)
    if scales is None:
        scales = channel_scales(x, seed, wid)
    v = z * scales[None, :]
    if x.law == "silu":
        with np.errstate(over="ignore"):
            v = v / (np.float32(1.0) + np.exp(-v))
    return _cast(v, x.dtype)


def n_chunks(x: XSpec) -> int:
    return (x.tokens + CHUNK - 1) // CHUNK


def x_range(x: XSpec, c0: int, c1: int, seed: int = 0, wid: int = 0, threads: Optional[int] = None,
            out: Optional[np.ndarray] = None) -> np.ndarray:
    """Chunks [c0, c1) stacked into one token-major array (generated in parallel)."""
    scales = channel_scales(x, seed, wid)
    L = corr_factor(x, seed, wid) if x.law == "corr" else None
    rows = [min(CHUNK, x.tokens - c * CHUNK) for c in range(c0, c1)]
    npdt = np.uint16 if x.dtype == "bf16" else _NP[x.dtype]
    if out is None:
        out = np.empty((sum(rows), x.n), dtype=npdt)
    offs = np.concatenate([[0], np.cumsum(rows)])

    def work(i):
        out[offs[i]:offs[i + 1]] = x_chunk(x, c0 + i, seed, wid, scales, L)

    threads = threads or min(16, os.cpu_count() or 1)
    with _cf.ThreadPoolExecutor(threads) as ex:
        list(ex.map(work, range(c1 - c0)))
    return out


def x_full(x: XSpec, seed: int = 0, wid: int = 0, threads: Optional[int] = None) -> np.ndarray:
    return x_range(x, 0, n_chunks(x), seed, wid, threads)


# ----------------------------------------------------------------------------- small generic layers

def small_layer(m: int, n: int, tokens: int, seed: int, law: str = "lognormal", w_dtype: str = "f32",
                x_dtype: str = "f32", sigma: float = 0.02, outlier_frac: float = 0.0,
                outlier_channels: int = 0) -> Tuple[np.ndarray, np.ndarray]:
    """A (W, X) pair of arbitrary small shape for parity sweeps over sizes."""
    wid = 1000 + (seed % 1000)
    ws = WSpec(f"w{m}x{n}", m, n, sigma, w_dtype, outlier_frac, 10.0)
    xs = XSpec(f"x{n}x{tokens}:{law}", n, tokens, law, x_dtype, outlier_channels=outlier_channels,
               outlier_mult=20.0)
    return weight(ws, seed, wid), x_full(xs, seed, wid)


def as_float64(a: np.ndarray, dtype: str) -> np.ndarray:
    """Exact fp64 view of generated values (bf16 arrive as raw uint16)."""
    if dtype == "bf16":
        return bf16_bits_to_f32(a).astype(np.float64)
    return a.astype(np.float64)


# ----------------------------------------------------------------------------- packed layers at run time

def packed_layer(m: int, n: int, bits: int, group: int, seed: int = 0) -> Tuple[np.ndarray, np.ndarray, np.ndarray]:
    """Codes q [m x n] uniform on 0..2^bits-1, zero points z [m x G] uniform on
    the same range, scales s [m x G] log-normal around 0.01 (the size of
    4-bit scales of weights with std 0.02): the structure of a quantized
    layer's outputs, without running the quantizer."""
    G = 1 if group <= 0 else (n + group - 1) // group
    rng = _rng(seed, 0, f"P:{m}x{n}:{bits}:{group}")
    q = rng.integers(0, 1 << bits, (m, n), dtype=np.int64)
    z = rng.integers(0, 1 << bits, (m, G), dtype=np.int64).astype(np.int32)
    s = (0.01 * rng.lognormal(0.0, 0.5, (m, G))).astype(np.float32)
    return q, s, z


def activations(tokens: int, n: int, dtype: str = "f16", seed: int = 0) -> np.ndarray:
    """Token-major activations [tokens x n]: normal with log-normal per-channel
    scales (a few channels much larger, as in transformer layers); fp16, or
    bf16 as raw uint16."""
    rng = _rng(seed, 0, f"A:{tokens}x{n}")
    ch = rng.lognormal(0.0, 0.75, n)
    X = (rng.standard_normal((tokens, n)) * ch).astype(np.float32)
    return _cast(X, dtype)
