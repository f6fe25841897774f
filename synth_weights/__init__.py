"""Seeded synthetic BF16 (and FP8) weight generators.

This module produces the uint16 bit patterns that both the CPU oracle and the
HIP library are fed.  It holds no part of the codec (no histogram, no code
construction, no bit packing): it only draws random numbers and rounds them to
BF16.  Real checkpoints (Llama 3.3, Qwen 3, Mistral 3, FLUX.1, named in the
abstract of "70% Size, 100% Accuracy: Lossless LLM Compression for Efficient
GPU Inference via Dynamic-Length Float (DFloat11)") are not available, so
these Gaussian-like stand-ins take their place.

Recipe (every draw is reproducible from the integers below):

* fp32 -> bf16 is round-to-nearest-even on the bit pattern:
  ``b = (u + 0x7FFF + ((u >> 16) & 1)) >> 16``.
* A tensor of shape [rows, cols] is filled in row chunks of about
  ``CHUNK_ELEMS`` elements.  Chunk c of tensor t of unit u in config k draws
  from ``numpy.random.default_rng([k_seed, u, t, 0, c])``; per-row scales draw
  from ``default_rng([k_seed, u, t, 1])``.  Chunks are independent, so the
  fill runs on a thread pool (numpy releases the GIL while filling).
* "lognormal rows": s_r = exp(N(ln 0.02, 0.3^2)) drawn in float64 and cast to
  fp32; w = bf16(s_r * z) with z ~ N(0, 1) in fp32.
* FP8 variants of a unit: each BF16 tensor scaled so that its largest
  magnitude maps to the format's largest finite value (448 for E4M3, 57344
  for E5M2), then rounded to nearest, ties to even, saturating.
"""

from __future__ import annotations

import math
import os
from concurrent.futures import ThreadPoolExecutor
from dataclasses import dataclass, field

import numpy as np

CHUNK_ELEMS = 1 << 22

LLAMA3_8B_BLOCK = [
    ("q_proj", (4096, 4096)),
    ("k_proj", (1024, 4096)),
    ("v_proj", (1024, 4096)),
    ("o_proj", (4096, 4096)),
    ("gate_proj", (14336, 4096)),
    ("up_proj", (14336, 4096)),
    ("down_proj", (4096, 14336)),
]

LLAMA3_70B_BLOCK = [
    ("q_proj", (8192, 8192)),
    ("k_proj", (1024, 8192)),
    ("v_proj", (1024, 8192)),
    ("o_proj", (8192, 8192)),
    ("gate_proj", (28672, 8192)),
    ("up_proj", (28672, 8192)),
    ("down_proj", (8192, 28672)),
]

# One GPU's share of the 70B-shaped block under 8-way tensor parallelism in
# the usual layout: the projections that feed a nonlinearity or attention (q,
# k, v, gate, up) split their output rows, the two that feed the residual
# stream (o, down) split their input columns.  Each shard row is drawn with the
# full block's per-row recipe, which is what slicing the full matrix would give.
LLAMA3_70B_BLOCK_TP8 = [
    ("q_proj", (1024, 8192)),
    ("k_proj", (128, 8192)),
    ("v_proj", (128, 8192)),
    ("o_proj", (8192, 1024)),
    ("gate_proj", (3584, 8192)),
    ("up_proj", (3584, 8192)),
    ("down_proj", (8192, 3584)),
]

# The same share of a Llama-3.1-405B-shaped block (hidden 16384, intermediate
# 53248, 8 key/value heads of 128), the largest model the pages name.
LLAMA31_405B_BLOCK_TP8 = [
    ("q_proj", (2048, 16384)),
    ("k_proj", (128, 16384)),
    ("v_proj", (128, 16384)),
    ("o_proj", (16384, 2048)),
    ("gate_proj", (6656, 16384)),
    ("up_proj", (6656, 16384)),
    ("down_proj", (16384, 6656)),
]

VOCAB_SHAPE = (128256, 4096)
STRESS_SHAPE = (4096, 14336)


@dataclass
class Unit:
    """One launch's worth of tensors sharing one exponent codebook."""

    name: str
    tensors: list  # list of (name, (rows, cols))
    dist: str  # "gauss", "lognormal_rows", "student_t_outliers", "one_exponent", "uniform_bits"
    seed: int
    index: int = 0

    @property
    def numel(self) -> int:
        return sum(r * c for _, (r, c) in self.tensors)


@dataclass
class Config:
    index: int
    name: str
    units: list = field(default_factory=list)

    @property
    def numel(self) -> int:
        return sum(u.numel for u in self.units)


def config(k: int | str) -> Config:
    """The five workloads: 0 small tensor, 1 8B block, 2 70B block,
    3 distribution stress (3a/3b/3c as units), 4 full 8B model; and 2tp8 and
    405tp8, one GPU's share of the 70B and of a 405B-shaped block under 8-way
    tensor parallelism."""
    k = str(k)
    if k == "0":
        return Config(0, "tensor_1024x1024_gauss",
                      [Unit("w", [("w", (1024, 1024))], "gauss", 0)])
    if k == "1":
        return Config(1, "llama3_8b_block",
                      [Unit("block", LLAMA3_8B_BLOCK, "lognormal_rows", 1)])
    if k == "2":
        return Config(2, "llama3_70b_block",
                      [Unit("block", LLAMA3_70B_BLOCK, "lognormal_rows", 2)])
    if k == "2tp8":
        return Config(2, "llama3_70b_block_tp8_shard",
                      [Unit("block_tp8_rank0", LLAMA3_70B_BLOCK_TP8, "lognormal_rows", 22)])
    if k == "405tp8":
        return Config(2, "llama31_405b_block_tp8_shard",
                      [Unit("block_tp8_rank0", LLAMA31_405B_BLOCK_TP8, "lognormal_rows", 23)])
    if k in ("3", "3a", "3b", "3c"):
        units = [
            Unit("3a_student_t_outliers", [("w", STRESS_SHAPE)], "student_t_outliers", 30),
            Unit("3b_one_exponent", [("w", STRESS_SHAPE)], "one_exponent", 31),
            Unit("3c_uniform_bits", [("w", STRESS_SHAPE)], "uniform_bits", 32),
        ]
        if k != "3":
            units = [u for u in units if u.name.startswith(k)]
        return Config(3, "distribution_stress" if k == "3" else units[0].name, units)
    if k == "4":
        units = [Unit("embedding", [("embed_tokens", VOCAB_SHAPE)], "lognormal_rows", 4, 0)]
        for b in range(32):
            units.append(Unit(f"block{b:02d}", LLAMA3_8B_BLOCK, "lognormal_rows", 4, 1 + b))
        units.append(Unit("lm_head", [("lm_head", VOCAB_SHAPE)], "lognormal_rows", 4, 33))
        return Config(4, "llama3_8b_full_model", units)
    raise ValueError(f"unknown config {k!r}")


def bf16_from_f32(x: np.ndarray) -> np.ndarray:
    """Round fp32 to bf16 (nearest, ties to even) and return the uint16 bit patterns."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    r = (u + np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1))) >> np.uint32(16)
    return r.astype(np.uint16)


# OCP 8-bit floating point formats: exponent bits, mantissa bits, bias, largest finite value
FP8_FORMATS = {"e4m3": (4, 3, 7, 448.0), "e5m2": (5, 2, 15, 57344.0)}


def fp8_from_f32(x: np.ndarray, fmt: str) -> np.ndarray:
    """Round fp32 values to an FP8 format (nearest, ties to even, saturating at
    the largest finite value) and return the uint8 bit patterns.  Computed in
    float64, where every step below is exact for fp32 inputs."""
    e_bits, m_bits, bias, max_finite = FP8_FORMATS[fmt]
    x = np.asarray(x, dtype=np.float32).astype(np.float64)
    sign = np.signbit(x).astype(np.uint8)
    a = np.abs(x)
    emin = 1 - bias  # exponent of the smallest normal
    _, e = np.frexp(a)  # a = f * 2^e with f in [0.5, 1): floor(log2 a) = e - 1
    e = np.maximum(e.astype(np.int64) - 1, emin)
    q = np.ldexp(1.0, e - m_bits)  # spacing of representable values around a
    r = np.minimum(np.round(a / q) * q, max_finite)  # numpy rounds halves to even
    _, er = np.frexp(r)
    er = er.astype(np.int64) - 1
    normal = r >= np.ldexp(1.0, emin)
    field = np.where(normal, er + bias, 0)
    mant = np.where(normal, r / np.ldexp(1.0, np.where(normal, er, 0) - m_bits) - (1 << m_bits),
                    r / np.ldexp(1.0, emin - m_bits))
    return ((sign << 7) | (field.astype(np.uint8) << m_bits) | mant.astype(np.uint8)).astype(np.uint8)


def gen_unit_fp8(unit: "Unit", fmt: str, threads: int | None = None) -> list:
    """The unit's tensors quantized to FP8: each BF16 tensor from gen_unit is
    scaled so its largest magnitude maps to the format's largest finite value
    (a per-tensor scale, as FP8 checkpoints store one) and rounded."""
    max_finite = FP8_FORMATS[fmt][3]
    out = []
    with ThreadPoolExecutor(_threads(threads)) as pool:
        for w in gen_unit(unit, threads):
            v = (w.astype(np.uint32) << np.uint32(16)).view(np.float32)
            amax = float(np.max(np.abs(v))) if v.size else 0.0
            scale = np.float32(max_finite / amax) if amax > 0 else np.float32(1.0)
            q = np.empty(v.size, dtype=np.uint8)

            def conv(lo, v=v, q=q, scale=scale):
                q[lo:lo + CHUNK_ELEMS] = fp8_from_f32(v[lo:lo + CHUNK_ELEMS] * scale, fmt)

            list(pool.map(conv, range(0, v.size, CHUNK_ELEMS)))
            out.append(q)
    return out


def _threads(threads: int | None) -> int:
    if threads is not None:
        return max(1, threads)
    return max(1, min(16, os.cpu_count() or 1))


def _fill_chunk(dist: str, seed: int, unit_idx: int, t_idx: int, c_idx: int,
                rows: slice, cols: int, row_scale: np.ndarray | None,
                out: np.ndarray) -> None:
    rng = np.random.default_rng([seed, unit_idx, t_idx, 0, c_idx])
    nrows = rows.stop - rows.start
    n = nrows * cols
    if dist == "uniform_bits":
        out[:] = rng.integers(0, 65536, size=n, dtype=np.uint16)
        return
    if dist == "student_t_outliers":
        t = rng.standard_t(3.0, size=n) * 0.02
        mask = rng.random(n) < 0.001
        t[mask] *= 100.0
        out[:] = bf16_from_f32(t.astype(np.float32))
        return
    z = rng.standard_normal(size=n, dtype=np.float32)
    if dist == "lognormal_rows":
        z = z.reshape(nrows, cols)
        z *= row_scale[rows.start:rows.stop, None]
        out[:] = bf16_from_f32(z.reshape(-1))
        return
    z *= np.float32(0.02)
    w = bf16_from_f32(z)
    if dist == "one_exponent":
        mask = rng.random(n) < 0.99
        w[mask] = (w[mask] & np.uint16(0x807F)) | np.uint16(121 << 7)
    elif dist != "gauss":
        raise ValueError(dist)
    out[:] = w


def gen_tensor(unit: Unit, t_idx: int, threads: int | None = None,
               pool: ThreadPoolExecutor | None = None) -> np.ndarray:
    """Flattened uint16 bit patterns of tensor ``t_idx`` of ``unit``."""
    _, (rows, cols) = unit.tensors[t_idx]
    out = np.empty(rows * cols, dtype=np.uint16)
    row_scale = None
    if unit.dist == "lognormal_rows":
        srng = np.random.default_rng([unit.seed, unit.index, t_idx, 1])
        row_scale = np.exp(srng.normal(math.log(0.02), 0.3, size=rows)).astype(np.float32)
    rows_per_chunk = max(1, CHUNK_ELEMS // cols)
    jobs = []
    for c, r0 in enumerate(range(0, rows, rows_per_chunk)):
        r1 = min(rows, r0 + rows_per_chunk)
        jobs.append((c, slice(r0, r1)))
    own = pool is None
    if own:
        pool = ThreadPoolExecutor(_threads(threads))
    try:
        futs = [pool.submit(_fill_chunk, unit.dist, unit.seed, unit.index, t_idx, c,
                            sl, cols, row_scale, out[sl.start * cols:sl.stop * cols])
                for c, sl in jobs]
        for f in futs:
            f.result()
    finally:
        if own:
            pool.shutdown()
    return out


def gen_unit(unit: Unit, threads: int | None = None) -> list:
    """All tensors of a unit, each a flattened uint16 array, in listed order."""
    with ThreadPoolExecutor(_threads(threads)) as pool:
        return [gen_tensor(unit, t, pool=pool) for t in range(len(unit.tensors))]
