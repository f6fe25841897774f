"""CPU oracle for DFloat11-style lossless BF16 compression.

TEST INFRASTRUCTURE ONLY: the test suite, the smoke check and the benchmark's
CPU-baseline leg are its only users.  The product library never imports,
links or calls anything here, and this package never imports the product.

The arithmetic lives in ``df11_oracle.c`` (plain bit-serial C, built with gcc
into ``libdf11_oracle.so``); this module only marshals numpy arrays into it and
adds the closed-form quantities the checks need (entropy, Kraft sum, mean
code length).  What each step follows on the pages is cited in the C file.
"""

from __future__ import annotations

import ctypes
import math
import os
import subprocess
from dataclasses import dataclass

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "df11_oracle.c")
_LIB = os.path.join(_HERE, "libdf11_oracle.so")

MAX_LEN = 32


def build(force: bool = True) -> str:
    """Compile the oracle with gcc (-O2, no fast-math, nothing vectorised by hand)."""
    if force or not os.path.exists(_LIB):
        tmp = _LIB + ".tmp"
        subprocess.check_call(["gcc", "-O2", "-std=c99", "-Wall", "-Wextra", "-fPIC", "-shared",
                               _SRC, "-o", tmp])
        os.replace(tmp, _LIB)
    return _LIB


_lib = None


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB):
            build()
        L = ctypes.CDLL(_LIB)
        u8p = ctypes.POINTER(ctypes.c_uint8)
        u16p = ctypes.POINTER(ctypes.c_uint16)
        u32p = ctypes.POINTER(ctypes.c_uint32)
        u64p = ctypes.POINTER(ctypes.c_uint64)
        u64 = ctypes.c_uint64
        u32 = ctypes.c_uint32
        L.oracle_histogram.argtypes = [u16p, u64, u64p]
        L.oracle_histogram.restype = None
        L.oracle_huffman_lengths.argtypes = [u64p, u8p]
        L.oracle_huffman_lengths.restype = ctypes.c_int
        L.oracle_limited_lengths.argtypes = [u64p, ctypes.c_int, u8p]
        L.oracle_limited_lengths.restype = ctypes.c_int
        L.oracle_code_lengths.argtypes = [u64p, u8p]
        L.oracle_code_lengths.restype = ctypes.c_int
        L.oracle_canonical_codes.argtypes = [u8p, u32p]
        L.oracle_canonical_codes.restype = None
        L.oracle_encode.argtypes = [u16p, u64, u8p, u32p, u8p, u64, u8p, u64p]
        L.oracle_encode.restype = ctypes.c_int
        for name in ("oracle_aux", "oracle_aux_fast"):
            f = getattr(L, name)
            f.argtypes = [u16p, u64, u8p, u32, u32, u8p, u64, u32p, u64]
            f.restype = ctypes.c_int
        L.oracle_decode.argtypes = [u8p, u64, u64, u8p, u8p, u64, u16p]
        L.oracle_decode.restype = ctypes.c_int
        L.oracle_fp8_split.argtypes = [u8p, u64, ctypes.c_int, u8p, u8p]
        L.oracle_fp8_split.restype = ctypes.c_int
        L.oracle_fp8_merge.argtypes = [u8p, u8p, u64, ctypes.c_int, u8p]
        L.oracle_fp8_merge.restype = ctypes.c_int
        L.oracle_histogram_symbols.argtypes = [u8p, u64, u64p]
        L.oracle_histogram_symbols.restype = None
        L.oracle_encode_symbols.argtypes = [u8p, u64, u8p, u32p, u8p, u64, u64p]
        L.oracle_encode_symbols.restype = ctypes.c_int
        L.oracle_aux_symbols.argtypes = [u8p, u64, u8p, u32, u32, u8p, u64, u32p, u64]
        L.oracle_aux_symbols.restype = ctypes.c_int
        L.oracle_decode_symbols.argtypes = [u8p, u64, u64, u8p, u64, u8p]
        L.oracle_decode_symbols.restype = ctypes.c_int
        _lib = L
    return _lib


def _p(a: np.ndarray, ct):
    assert a.flags["C_CONTIGUOUS"]
    return a.ctypes.data_as(ctypes.POINTER(ct))


def _cat(tensors) -> np.ndarray:
    if isinstance(tensors, np.ndarray):
        tensors = [tensors]
    parts = [np.ascontiguousarray(t, dtype=np.uint16).reshape(-1) for t in tensors]
    if len(parts) == 1:
        return parts[0]
    return np.concatenate(parts)


# ---------------------------------------------------------------- codebook


def histogram(tensors) -> np.ndarray:
    w = _cat(tensors)
    c = np.zeros(256, dtype=np.uint64)
    lib().oracle_histogram(_p(w, ctypes.c_uint16), w.size, _p(c, ctypes.c_uint64))
    return c


def huffman_lengths(counts) -> np.ndarray:
    c = np.ascontiguousarray(counts, dtype=np.uint64)
    assert c.size == 256
    lens = np.zeros(256, dtype=np.uint8)
    lib().oracle_huffman_lengths(_p(c, ctypes.c_uint64), _p(lens, ctypes.c_uint8))
    return lens


def limited_lengths(counts, limit: int) -> np.ndarray:
    c = np.ascontiguousarray(counts, dtype=np.uint64)
    assert c.size == 256
    lens = np.zeros(256, dtype=np.uint8)
    r = lib().oracle_limited_lengths(_p(c, ctypes.c_uint64), int(limit), _p(lens, ctypes.c_uint8))
    if r < 0:
        raise ValueError("more symbols than codes of the given limit")
    return lens


def code_lengths(counts) -> np.ndarray:
    c = np.ascontiguousarray(counts, dtype=np.uint64)
    lens = np.zeros(256, dtype=np.uint8)
    lib().oracle_code_lengths(_p(c, ctypes.c_uint64), _p(lens, ctypes.c_uint8))
    return lens


def canonical_codes(lens) -> np.ndarray:
    lens = np.ascontiguousarray(lens, dtype=np.uint8)
    codes = np.zeros(256, dtype=np.uint32)
    lib().oracle_canonical_codes(_p(lens, ctypes.c_uint8), _p(codes, ctypes.c_uint32))
    return codes


@dataclass
class Codebook:
    counts: np.ndarray
    lens: np.ndarray
    codes: np.ndarray


def codebook(tensors) -> Codebook:
    counts = histogram(tensors)
    lens = code_lengths(counts)
    return Codebook(counts, lens, canonical_codes(lens))


# ---------------------------------------------------------------- stream


@dataclass
class Encoded:
    stream: np.ndarray        # uint8, ceil(total_bits / 8) bytes
    sm: np.ndarray            # uint8, one per weight
    total_bits: int
    tensor_start_bits: list   # start bit of each input tensor, plus total_bits
    numel: list


def encode(tensors, cb: Codebook) -> Encoded:
    if isinstance(tensors, np.ndarray):
        tensors = [tensors]
    w = _cat(tensors)
    lens = np.ascontiguousarray(cb.lens, dtype=np.uint8)
    codes = np.ascontiguousarray(cb.codes, dtype=np.uint32)
    total = int(sum(int(lens[(int(e))]) * int(c) for e, c in enumerate(histogram(w))))
    stream = np.zeros(max(1, (total + 7) // 8), dtype=np.uint8)
    sm = np.zeros(w.size, dtype=np.uint8)
    tb = np.zeros(1, dtype=np.uint64)
    r = lib().oracle_encode(_p(w, ctypes.c_uint16), w.size, _p(lens, ctypes.c_uint8),
                            _p(codes, ctypes.c_uint32), _p(stream, ctypes.c_uint8), stream.size,
                            _p(sm, ctypes.c_uint8), _p(tb, ctypes.c_uint64))
    if r != 0:
        raise ValueError(f"oracle_encode failed ({r})")
    assert int(tb[0]) == total
    starts = [0]
    numel = []
    for t in tensors:
        t = np.ascontiguousarray(t, dtype=np.uint16).reshape(-1)
        h = histogram(t)
        starts.append(starts[-1] + int(sum(int(lens[e]) * int(c) for e, c in enumerate(h))))
        numel.append(t.size)
    return Encoded(stream[: (total + 7) // 8], sm, total, starts, numel)


def aux(tensors, cb: Codebook, tile_windows: int, window_bytes: int, fast: bool = True):
    """(gaps uint8[n_tiles*tile_windows], block_out_pos uint32[n_tiles+1]) from the definitions."""
    w = _cat(tensors)
    lens = np.ascontiguousarray(cb.lens, dtype=np.uint8)
    total = int(sum(int(lens[e]) * int(c) for e, c in enumerate(histogram(w))))
    window_bits = 8 * window_bytes
    tile_bits = window_bits * tile_windows
    n_tiles = (total + tile_bits - 1) // tile_bits
    gaps = np.zeros(n_tiles * tile_windows, dtype=np.uint8)
    bop = np.zeros(n_tiles + 1, dtype=np.uint32)
    f = lib().oracle_aux_fast if fast else lib().oracle_aux
    r = f(_p(w, ctypes.c_uint16), w.size, _p(lens, ctypes.c_uint8), window_bits, tile_windows,
          _p(gaps, ctypes.c_uint8), gaps.size, _p(bop, ctypes.c_uint32), n_tiles)
    if r != 0:
        raise ValueError(f"oracle_aux failed ({r})")
    return gaps, bop


def window_counts(sym: np.ndarray, lens, n_windows: int, window_bytes: int = 8) -> np.ndarray:
    """count_j = number of codes whose first bit lies in window j (bits
    [8 B j, 8 B (j+1))), for the symbol sequence sym coded with lengths lens.
    Code i starts at the sum of the lengths of codes 0 .. i-1 (DFloat11
    abstract: the first of the two phases counts each thread's codes)."""
    sym = np.ascontiguousarray(sym).reshape(-1)
    ln = np.asarray(lens, dtype=np.int64)[sym]
    starts = np.cumsum(ln) - ln
    return np.bincount(starts // (8 * window_bytes), minlength=n_windows).astype(np.uint32)


def decode(stream: np.ndarray, start_bit: int, end_bit: int, lens, sm: np.ndarray,
           n: int | None = None) -> np.ndarray:
    """Bit-serial decode of n symbols from start_bit; returns uint16 BF16 bit patterns."""
    stream = np.ascontiguousarray(stream, dtype=np.uint8)
    lens = np.ascontiguousarray(lens, dtype=np.uint8)
    sm = np.ascontiguousarray(sm, dtype=np.uint8)
    if n is None:
        n = sm.size
    assert sm.size >= n
    out = np.zeros(n, dtype=np.uint16)
    if n == 0:
        return out
    r = lib().oracle_decode(_p(stream, ctypes.c_uint8), start_bit, end_bit,
                            _p(lens, ctypes.c_uint8), _p(sm, ctypes.c_uint8), n,
                            _p(out, ctypes.c_uint16))
    if r != 0:
        raise ValueError(f"oracle_decode failed ({r})")
    return out


# ---------------------------------------------------------------- closed forms


def entropy_bits(counts) -> float:
    """Shannon entropy H = -sum p log2 p of the exponent histogram, in float64."""
    c = np.asarray(counts, dtype=np.float64)
    n = c.sum()
    if n == 0:
        return 0.0
    p = c[c > 0] / n
    return float(-(p * np.log2(p)).sum())


def mean_code_length(counts, lens) -> float:
    c = np.asarray(counts, dtype=np.float64)
    n = c.sum()
    return float((c * np.asarray(lens, dtype=np.float64)).sum() / n) if n else 0.0


def total_code_bits(counts, lens) -> int:
    return int(sum(int(c) * int(l) for c, l in zip(np.asarray(counts), np.asarray(lens))))


def kraft_numerator(lens) -> int:
    """sum over coded symbols of 2^(32 - l): equals 2^32 exactly for a complete code."""
    return int(sum(1 << (MAX_LEN - int(l)) for l in np.asarray(lens) if int(l) > 0))


def sign_mantissa(w: np.ndarray) -> np.ndarray:
    w = np.asarray(w, dtype=np.uint16)
    return (((w >> 8) & 0x80) | (w & 0x7F)).astype(np.uint8)


def exponents(w: np.ndarray) -> np.ndarray:
    return ((np.asarray(w, dtype=np.uint16) >> 7) & 0xFF).astype(np.uint8)


def gaussian_exponent_probs(sigma: float) -> np.ndarray:
    """Closed-form probability that a N(0, sigma^2) value lands in BF16 binade e.

    For normal binades, |x| in [2^(e-127), 2^(e-126)) has probability
    2 * (Phi(2^(e-126)/sigma) - Phi(2^(e-127)/sigma)); e = 0 (zero and
    subnormals) takes |x| < 2^-126.  Rounding at binade edges is ignored.
    """
    phi = lambda x: 0.5 * (1.0 + math.erf(x / math.sqrt(2.0)))
    p = np.zeros(256)
    p[0] = 2.0 * (phi(2.0 ** -126 / sigma) - 0.5)
    for e in range(1, 255):
        lo, hi = 2.0 ** (e - 127), 2.0 ** (e - 126)
        p[e] = 2.0 * (phi(hi / sigma) - phi(lo / sigma))
    return p


# ---------------------------------------------------------------- GEMV consumer


def bf16_to_f64(w: np.ndarray) -> np.ndarray:
    """Exact values of BF16 bit patterns: the pattern is the top half of an fp32."""
    w = np.ascontiguousarray(w, dtype=np.uint16)
    return (w.astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def gemv(w_flat: np.ndarray, shapes, x_flat: np.ndarray) -> np.ndarray:
    """y = W_k x_k for row-major BF16 matrices stored back to back in w_flat
    (shapes: (rows, cols) each), x slices back to back in x_flat; float64.

    Products of a BF16 and an fp32 value are exact in float64, and a row of at
    most 2^20 terms sums with relative error below 2^-32, far inside any fp32
    tolerance.
    """
    w = bf16_to_f64(np.asarray(w_flat).reshape(-1))
    x = np.asarray(x_flat, dtype=np.float64).reshape(-1)
    ys, wo, xo = [], 0, 0
    for rows, cols in shapes:
        W = w[wo:wo + rows * cols].reshape(rows, cols)
        ys.append(W @ x[xo:xo + cols])
        wo += rows * cols
        xo += cols
    return np.concatenate(ys) if ys else np.zeros(0)


def gemm(w_flat: np.ndarray, shapes, x_flat: np.ndarray, n_tokens: int) -> np.ndarray:
    """Y_k = X_k W_k^T for row-major BF16 matrices W_k stored back to back in
    w_flat, with token-major BF16 activations X_k (n_tokens x cols_k) back to
    back in x_flat; returns the token-major Y_k (n_tokens x rows_k) back to
    back, float64.  Products of two BF16 values are exact in float64; sums of
    at most 2^20 terms keep a relative error below 2^-32."""
    w = bf16_to_f64(np.asarray(w_flat).reshape(-1))
    x = bf16_to_f64(np.asarray(x_flat).reshape(-1))
    ys, wo, xo = [], 0, 0
    for rows, cols in shapes:
        W = w[wo:wo + rows * cols].reshape(rows, cols)
        X = x[xo:xo + n_tokens * cols].reshape(n_tokens, cols)
        ys.append((X @ W.T).reshape(-1))
        wo += rows * cols
        xo += n_tokens * cols
    return np.concatenate(ys) if ys else np.zeros(0)


# ---------------------------------------------------------------- FP8 weights
# (the C file's FP8 section gives the formats and the readings)

FP8_FORMATS = {"e4m3": 1, "e5m2": 2}


def fp8_split(b: np.ndarray, fmt: str):
    """(symbols uint8[n], packed sign+mantissa nibbles uint8[ceil(n/2)])."""
    b = np.ascontiguousarray(b, dtype=np.uint8).reshape(-1)
    sym = np.zeros(b.size, dtype=np.uint8)
    sm = np.zeros((b.size + 1) // 2, dtype=np.uint8)
    if b.size:
        r = lib().oracle_fp8_split(_p(b, ctypes.c_uint8), b.size, FP8_FORMATS[fmt],
                                   _p(sym, ctypes.c_uint8), _p(sm, ctypes.c_uint8))
        assert r == 0
    return sym, sm


def fp8_merge(sym: np.ndarray, sm: np.ndarray, fmt: str) -> np.ndarray:
    sym = np.ascontiguousarray(sym, dtype=np.uint8)
    sm = np.ascontiguousarray(sm, dtype=np.uint8)
    out = np.zeros(sym.size, dtype=np.uint8)
    if sym.size:
        r = lib().oracle_fp8_merge(_p(sym, ctypes.c_uint8), _p(sm, ctypes.c_uint8), sym.size,
                                   FP8_FORMATS[fmt], _p(out, ctypes.c_uint8))
        assert r == 0
    return out


def histogram_symbols(sym: np.ndarray) -> np.ndarray:
    sym = np.ascontiguousarray(sym, dtype=np.uint8).reshape(-1)
    c = np.zeros(256, dtype=np.uint64)
    lib().oracle_histogram_symbols(_p(sym, ctypes.c_uint8), sym.size, _p(c, ctypes.c_uint64))
    return c


def codebook_symbols(sym: np.ndarray) -> Codebook:
    counts = histogram_symbols(sym)
    lens = code_lengths(counts)
    return Codebook(counts, lens, canonical_codes(lens))


def encode_symbols(sym: np.ndarray, cb: Codebook):
    """(stream bytes, total_bits) of the symbol sequence."""
    sym = np.ascontiguousarray(sym, dtype=np.uint8).reshape(-1)
    lens = np.ascontiguousarray(cb.lens, dtype=np.uint8)
    codes = np.ascontiguousarray(cb.codes, dtype=np.uint32)
    total = total_code_bits(histogram_symbols(sym), lens)
    stream = np.zeros(max(1, (total + 7) // 8), dtype=np.uint8)
    tb = np.zeros(1, dtype=np.uint64)
    r = lib().oracle_encode_symbols(_p(sym, ctypes.c_uint8), sym.size, _p(lens, ctypes.c_uint8),
                                    _p(codes, ctypes.c_uint32), _p(stream, ctypes.c_uint8),
                                    stream.size, _p(tb, ctypes.c_uint64))
    if r != 0:
        raise ValueError(f"oracle_encode_symbols failed ({r})")
    assert int(tb[0]) == total
    return stream[: (total + 7) // 8], total


def aux_symbols(sym: np.ndarray, cb: Codebook, tile_windows: int, window_bytes: int):
    sym = np.ascontiguousarray(sym, dtype=np.uint8).reshape(-1)
    lens = np.ascontiguousarray(cb.lens, dtype=np.uint8)
    total = total_code_bits(histogram_symbols(sym), lens)
    window_bits = 8 * window_bytes
    n_tiles = (total + window_bits * tile_windows - 1) // (window_bits * tile_windows)
    gaps = np.zeros(n_tiles * tile_windows, dtype=np.uint8)
    bop = np.zeros(n_tiles + 1, dtype=np.uint32)
    r = lib().oracle_aux_symbols(_p(sym, ctypes.c_uint8), sym.size, _p(lens, ctypes.c_uint8),
                                 window_bits, tile_windows, _p(gaps, ctypes.c_uint8), gaps.size,
                                 _p(bop, ctypes.c_uint32), n_tiles)
    if r != 0:
        raise ValueError(f"oracle_aux_symbols failed ({r})")
    return gaps, bop


def decode_symbols(stream: np.ndarray, start_bit: int, end_bit: int, lens, n: int) -> np.ndarray:
    stream = np.ascontiguousarray(stream, dtype=np.uint8)
    lens = np.ascontiguousarray(lens, dtype=np.uint8)
    out = np.zeros(n, dtype=np.uint8)
    if n == 0:
        return out
    r = lib().oracle_decode_symbols(_p(stream, ctypes.c_uint8), start_bit, end_bit,
                                    _p(lens, ctypes.c_uint8), n, _p(out, ctypes.c_uint8))
    if r != 0:
        raise ValueError(f"oracle_decode_symbols failed ({r})")
    return out
