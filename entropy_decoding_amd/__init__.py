"""Python binding of libdf11 (DFloat11-style lossless BF16 compression on MI355X).

Argument marshalling only: every step of compression runs in the library's
C++ host code and every step of decompression in its HIP kernels.  PyTorch is
used for device memory and streams (``tensor.data_ptr()``,
``torch.cuda.current_stream().cuda_stream``).  The functions keep the C names:
``df11_build_codebook``, ``df11_encode_size``, ``df11_encode``,
``df11_decompress_block``, ``df11_decompress_tensor``.

The library must be built (``entropy_decoding_amd.build.build_library()``);
importing this module without it raises ImportError.  There is no fallback.
"""

from __future__ import annotations

import ctypes
import os
from dataclasses import dataclass

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libdf11.so")

DF11_MAX_CODE_LEN = 32
DF11_MAX_LUTS = 64
DF11_STREAM_PAD = 16
DF11_MULTI_BITS = 10
DF11_COUNT_BITS = 12

DF11_OK = 0
DF11_E_INVALID = 1
DF11_E_LUT_BUDGET = 2
DF11_E_SYMBOL = 3
DF11_E_CAPACITY = 4
DF11_E_HIP = 5
DF11_E_CORRUPT = 6

DEFAULT_TILE_WINDOWS = 64
DEFAULT_WINDOW_BYTES = 8


class Df11Error(RuntimeError):
    def __init__(self, fn: str, status: int):
        super().__init__(f"{fn}: {status_string(status)} ({status})")
        self.status = status


_u8p = ctypes.POINTER(ctypes.c_uint8)
_u16p = ctypes.POINTER(ctypes.c_uint16)
_u32p = ctypes.POINTER(ctypes.c_uint32)
_u64p = ctypes.POINTER(ctypes.c_uint64)


class df11_codebook(ctypes.Structure):
    _fields_ = [
        ("code_len", ctypes.c_uint8 * 256),
        ("code", ctypes.c_uint32 * 256),
        ("n_luts", ctypes.c_uint32),
        ("max_len", ctypes.c_uint32),
        ("multi", ctypes.c_uint32 * (1 << DF11_MULTI_BITS)),
        ("count", ctypes.c_uint16 * (1 << DF11_COUNT_BITS)),
        ("lut", (ctypes.c_uint16 * 256) * DF11_MAX_LUTS),
    ]


class df11_sizes(ctypes.Structure):
    _fields_ = [(n, ctypes.c_uint64) for n in (
        "n_weights", "total_bits", "n_tiles", "n_windows", "stream_bytes", "sm_bytes",
        "bop_entries")]


class df11_host_stream(ctypes.Structure):
    _fields_ = [
        ("stream", _u8p),
        ("sm", _u8p),
        ("gaps", _u8p),
        ("block_out_pos", _u32p),
        ("tensor_offsets", _u64p),
        ("tensor_tiles", _u64p),
        ("stream_capacity", ctypes.c_uint64),
        ("sm_capacity", ctypes.c_uint64),
        ("gaps_capacity", ctypes.c_uint64),
        ("bop_capacity", ctypes.c_uint64),
        ("n_tensors", ctypes.c_uint32),
        ("tile_windows", ctypes.c_uint32),
        ("window_bytes", ctypes.c_uint32),
        ("max_tile_symbols", ctypes.c_uint32),
        ("n_weights", ctypes.c_uint64),
        ("total_bits", ctypes.c_uint64),
        ("n_tiles", ctypes.c_uint64),
        ("format", ctypes.c_uint32),
    ]


class df11_device_stream(ctypes.Structure):
    _fields_ = [
        ("stream", ctypes.c_void_p),
        ("sm", ctypes.c_void_p),
        ("gaps", ctypes.c_void_p),
        ("block_out_pos", ctypes.c_void_p),
        ("tables", ctypes.c_void_p),
        ("tensor_offsets", _u64p),
        ("tensor_tiles", _u64p),
        ("n_weights", ctypes.c_uint64),
        ("total_bits", ctypes.c_uint64),
        ("n_tiles", ctypes.c_uint64),
        ("n_luts", ctypes.c_uint32),
        ("tile_windows", ctypes.c_uint32),
        ("window_bytes", ctypes.c_uint32),
        ("max_tile_symbols", ctypes.c_uint32),
        ("n_tensors", ctypes.c_uint32),
        ("format", ctypes.c_uint32),
    ]


class df11_gemv_tensor(ctypes.Structure):
    _fields_ = [
        ("w_offset", ctypes.c_uint64),
        ("x_offset", ctypes.c_uint64),
        ("y_offset", ctypes.c_uint64),
        ("rows", ctypes.c_uint32),
        ("cols", ctypes.c_uint32),
    ]


class df11_device_encode(ctypes.Structure):
    _fields_ = [
        ("stream", ctypes.c_void_p),
        ("sm", ctypes.c_void_p),
        ("gaps", ctypes.c_void_p),
        ("block_out_pos", ctypes.c_void_p),
        ("d_max_tile_symbols", ctypes.c_void_p),
        ("scratch", ctypes.c_void_p),
        ("scratch_bytes", ctypes.c_uint64),
    ]


DF11_PIPELINE_MAX_SLOTS = 4
# df11_format; the names are what the binding's ``fmt`` arguments accept
FORMATS = {"bf16": 0, "fp8_e4m3": 1, "fp8_e5m2": 2}
DF11_GEMV_MAX_TENSORS = 16


def _load():
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"{LIB_PATH} is not built; run python entropy_decoding_amd/build.py")
    # PyTorch ships its own libamdhip64 (soname libamdhip64.so.7).  Loading torch
    # first lets the dynamic loader satisfy libdf11's dependency with that same
    # runtime; loading libdf11 first would bring in a second HIP runtime, whose
    # streams and launches are invisible to torch's.
    import torch  # noqa: F401

    L = ctypes.CDLL(LIB_PATH)
    tens = ctypes.POINTER(ctypes.c_void_p)
    L.df11_build_codebook.argtypes = [tens, _u64p, ctypes.c_uint32, ctypes.POINTER(df11_codebook)]
    L.df11_build_codebook_fmt.argtypes = [ctypes.c_uint32, tens, _u64p, ctypes.c_uint32,
                                          ctypes.POINTER(df11_codebook)]
    L.df11_encode_size_fmt.argtypes = [ctypes.c_uint32, ctypes.POINTER(df11_codebook), tens, _u64p,
                                       ctypes.c_uint32, ctypes.c_uint32, ctypes.c_uint32,
                                       ctypes.POINTER(df11_sizes)]
    L.df11_encode_fmt.argtypes = [ctypes.c_uint32, ctypes.POINTER(df11_codebook), tens, _u64p,
                                  ctypes.c_uint32, ctypes.c_uint32, ctypes.c_uint32,
                                  ctypes.POINTER(df11_host_stream)]
    L.df11_encode_size.argtypes = [ctypes.POINTER(df11_codebook), tens, _u64p, ctypes.c_uint32,
                                   ctypes.c_uint32, ctypes.c_uint32, ctypes.POINTER(df11_sizes)]
    L.df11_encode.argtypes = [ctypes.POINTER(df11_codebook), tens, _u64p, ctypes.c_uint32,
                              ctypes.c_uint32, ctypes.c_uint32, ctypes.POINTER(df11_host_stream)]
    L.df11_decompress_block.argtypes = [ctypes.POINTER(df11_device_stream), ctypes.c_void_p,
                                        ctypes.c_void_p, ctypes.c_void_p]
    L.df11_decompress_tensor.argtypes = [ctypes.POINTER(df11_device_stream), ctypes.c_uint32,
                                         ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p]
    L.df11_window_counts.argtypes = [ctypes.POINTER(df11_device_stream), ctypes.c_void_p,
                                     ctypes.c_void_p]
    L.df11_status_string.argtypes = [ctypes.c_int]
    L.df11_status_string.restype = ctypes.c_char_p
    vp = ctypes.c_void_p
    L.df11_pipeline_create.argtypes = [vp, ctypes.c_uint32, ctypes.POINTER(vp)]
    L.df11_pipeline_destroy.argtypes = [vp]
    L.df11_pipeline_decompress.argtypes = [vp, ctypes.c_uint32, ctypes.POINTER(df11_device_stream),
                                           vp, vp]
    L.df11_pipeline_acquire.argtypes = [vp, ctypes.c_uint32, vp]
    L.df11_pipeline_release.argtypes = [vp, ctypes.c_uint32, vp]
    L.df11_pipeline_set_decode_share.argtypes = [vp, ctypes.c_uint32]
    L.df11_gemv_bf16.argtypes = [vp, ctypes.POINTER(df11_gemv_tensor), ctypes.c_uint32, vp, vp, vp]
    L.df11_build_codebook_from_counts.argtypes = [_u64p, ctypes.POINTER(df11_codebook)]
    L.df11_decompress_gemv_scratch_bytes.argtypes = [ctypes.POINTER(df11_device_stream)]
    L.df11_decompress_gemv_scratch_bytes.restype = ctypes.c_uint64
    L.df11_decompress_gemv.argtypes = [ctypes.POINTER(df11_device_stream),
                                       ctypes.POINTER(df11_gemv_tensor), ctypes.c_uint32, vp, vp,
                                       vp, ctypes.c_uint64, vp, vp]
    L.df11_decompress_gemv_noalloc.argtypes = [ctypes.POINTER(df11_device_stream),
                                               ctypes.POINTER(df11_gemv_tensor), ctypes.c_uint32,
                                               vp, vp, vp, vp]
    L.df11_gemm_order.argtypes = [_u16p, ctypes.c_uint32, ctypes.c_uint32, _u16p]
    L.df11_decompress_gemm_scratch_bytes.argtypes = [ctypes.POINTER(df11_gemv_tensor),
                                                     ctypes.c_uint32, ctypes.c_uint32]
    L.df11_decompress_gemm_scratch_bytes.restype = ctypes.c_uint64
    L.df11_decompress_gemm.argtypes = [ctypes.POINTER(df11_device_stream),
                                       ctypes.POINTER(df11_gemv_tensor), ctypes.c_uint32,
                                       ctypes.c_uint32, vp, vp, vp, ctypes.c_uint64, vp, vp]
    L.df11_encode_size_from_counts.argtypes = [ctypes.c_uint32, ctypes.POINTER(df11_codebook),
                                               _u64p, ctypes.c_uint64, ctypes.c_uint32,
                                               ctypes.c_uint32, ctypes.POINTER(df11_sizes)]
    L.df11_histogram_device.argtypes = [ctypes.c_uint32, vp, ctypes.c_uint64, vp, vp]
    L.df11_tensor_ranges_from_counts.argtypes = [ctypes.c_uint32, ctypes.POINTER(df11_codebook),
                                                 _u64p, _u32p, ctypes.c_uint32, ctypes.c_uint32,
                                                 ctypes.c_uint32, _u64p, _u64p]
    L.df11_encode_device_scratch_bytes.argtypes = [ctypes.c_uint64]
    L.df11_encode_device_scratch_bytes.restype = ctypes.c_uint64
    L.df11_encode_device.argtypes = [ctypes.c_uint32, ctypes.POINTER(df11_codebook), vp,
                                     ctypes.c_uint64, ctypes.c_uint32, ctypes.c_uint32,
                                     ctypes.POINTER(df11_sizes), ctypes.POINTER(df11_device_encode),
                                     vp]
    for f in (L.df11_build_codebook, L.df11_encode_size, L.df11_encode,
              L.df11_build_codebook_fmt, L.df11_encode_size_fmt, L.df11_encode_fmt,
              L.df11_decompress_block, L.df11_decompress_tensor, L.df11_pipeline_create,
              L.df11_pipeline_destroy, L.df11_pipeline_decompress, L.df11_pipeline_acquire,
              L.df11_pipeline_release, L.df11_pipeline_set_decode_share, L.df11_gemv_bf16,
              L.df11_build_codebook_from_counts,
              L.df11_encode_size_from_counts, L.df11_histogram_device, L.df11_encode_device,
              L.df11_decompress_gemv, L.df11_gemm_order, L.df11_decompress_gemm,
              L.df11_window_counts, L.df11_tensor_ranges_from_counts,
              L.df11_decompress_gemv_noalloc):
        f.restype = ctypes.c_int
    return L


LIB = _load()


def status_string(status: int) -> str:
    return LIB.df11_status_string(int(status)).decode()


def _check(fn: str, rc: int):
    if rc != DF11_OK:
        raise Df11Error(fn, rc)


def _format(fmt: str) -> int:
    if fmt not in FORMATS:
        raise ValueError(f"fmt must be one of {sorted(FORMATS)}")
    return FORMATS[fmt]


def _tensor_args(tensors, fmt: str = "bf16"):
    if isinstance(tensors, np.ndarray):
        tensors = [tensors]
    want = np.uint16 if fmt == "bf16" else np.uint8
    arrs = []
    for t in tensors:
        a = np.asarray(t)
        if a.dtype != want:
            raise TypeError(f"{fmt} tensors must be {np.dtype(want).name} bit patterns")
        arrs.append(np.ascontiguousarray(a).reshape(-1))
    n = len(arrs)
    ptrs = (ctypes.c_void_p * max(n, 1))(*[a.ctypes.data for a in arrs])
    numel = (ctypes.c_uint64 * max(n, 1))(*[a.size for a in arrs])
    return arrs, ptrs, numel, n


# ---------------------------------------------------------------- host calls


def df11_build_codebook(tensors, fmt: str = "bf16") -> df11_codebook:
    """Histogram + Huffman (+ package-merge at 32 bits) + canonical codes + LUTs.
    BF16 tensors are uint16 arrays (df11_build_codebook); FP8 ones uint8
    arrays (df11_build_codebook_fmt)."""
    arrs, ptrs, numel, n = _tensor_args(tensors, fmt)
    cb = df11_codebook()
    if fmt == "bf16":
        _check("df11_build_codebook", LIB.df11_build_codebook(ptrs, numel, n, ctypes.byref(cb)))
    else:
        _check("df11_build_codebook_fmt",
               LIB.df11_build_codebook_fmt(_format(fmt), ptrs, numel, n, ctypes.byref(cb)))
    return cb


def df11_encode_size(cb: df11_codebook, tensors, tile_windows: int = DEFAULT_TILE_WINDOWS,
                     window_bytes: int = DEFAULT_WINDOW_BYTES, fmt: str = "bf16") -> df11_sizes:
    arrs, ptrs, numel, n = _tensor_args(tensors, fmt)
    sz = df11_sizes()
    if fmt == "bf16":
        _check("df11_encode_size", LIB.df11_encode_size(ctypes.byref(cb), ptrs, numel, n,
                                                        tile_windows, window_bytes,
                                                        ctypes.byref(sz)))
    else:
        _check("df11_encode_size_fmt",
               LIB.df11_encode_size_fmt(_format(fmt), ctypes.byref(cb), ptrs, numel, n,
                                        tile_windows, window_bytes, ctypes.byref(sz)))
    return sz


@dataclass
class HostStream:
    """A compressed unit in host memory (numpy arrays owned by this object)."""

    stream: np.ndarray
    sm: np.ndarray
    gaps: np.ndarray
    block_out_pos: np.ndarray
    tensor_offsets: np.ndarray
    tensor_tiles: np.ndarray
    tile_windows: int
    window_bytes: int
    max_tile_symbols: int
    n_weights: int
    total_bits: int
    n_tiles: int
    format: int = 0

    @property
    def n_tensors(self) -> int:
        return self.tensor_offsets.size - 1

    def compressed_bytes(self, cb: df11_codebook | None = None) -> dict:
        """Bytes of every array a decompression reads (payload and auxiliary)."""
        d = {
            "stream": (self.total_bits + 7) // 8,
            "sm": self.n_weights if self.format == 0 else (self.n_weights + 1) // 2,
            "gaps": self.gaps.size,
            "block_out_pos": 4 * self.block_out_pos.size,
        }
        if cb is not None:
            d["tables"] = table_bytes(cb)
        return d


def df11_encode(cb: df11_codebook, tensors, tile_windows: int = DEFAULT_TILE_WINDOWS,
                window_bytes: int = DEFAULT_WINDOW_BYTES, fmt: str = "bf16") -> HostStream:
    arrs, ptrs, numel, n = _tensor_args(tensors, fmt)
    sz = df11_encode_size(cb, arrs, tile_windows, window_bytes, fmt)
    stream = np.empty(sz.stream_bytes, dtype=np.uint8)
    sm = np.empty(sz.sm_bytes, dtype=np.uint8)
    gaps = np.empty(max(1, sz.n_windows), dtype=np.uint8)
    bop = np.empty(sz.bop_entries, dtype=np.uint32)
    offs = np.empty(n + 1, dtype=np.uint64)
    tiles = np.empty(max(1, 2 * n), dtype=np.uint64)
    hs = df11_host_stream()
    hs.stream = stream.ctypes.data_as(_u8p)
    hs.sm = sm.ctypes.data_as(_u8p)
    hs.gaps = gaps.ctypes.data_as(_u8p)
    hs.block_out_pos = bop.ctypes.data_as(_u32p)
    hs.tensor_offsets = offs.ctypes.data_as(_u64p)
    hs.tensor_tiles = tiles.ctypes.data_as(_u64p)
    hs.stream_capacity = stream.size
    hs.sm_capacity = sm.size
    hs.gaps_capacity = sz.n_windows
    hs.bop_capacity = bop.size
    hs.n_tensors = n
    if fmt == "bf16":
        _check("df11_encode", LIB.df11_encode(ctypes.byref(cb), ptrs, numel, n, tile_windows,
                                              window_bytes, ctypes.byref(hs)))
    else:
        _check("df11_encode_fmt", LIB.df11_encode_fmt(_format(fmt), ctypes.byref(cb), ptrs, numel,
                                                      n, tile_windows, window_bytes,
                                                      ctypes.byref(hs)))
    return HostStream(stream, sm, gaps[: sz.n_windows], bop, offs, tiles[: 2 * n],
                      hs.tile_windows, hs.window_bytes, hs.max_tile_symbols, hs.n_weights,
                      hs.total_bits, hs.n_tiles, hs.format)


# ---------------------------------------------------------------- device side


class DeviceStream:
    """A compressed unit resident in device memory (torch uint8/int32 tensors).

    Holds the ctypes descriptor passed to df11_decompress_*; the host-side
    tensor metadata (offsets, tile ranges) stays in numpy arrays it owns.
    Built from a HostStream (uploaded) or, by encode_on_device, from arrays
    written on the device.
    """

    def __init__(self, hs: HostStream, cb: df11_codebook, device="cuda", arrays=None):
        import torch

        def up(a):
            t = torch.from_numpy(np.ascontiguousarray(a).view(np.uint8).reshape(-1))
            return t.to(device)

        self.host = hs
        if arrays is None:
            self.stream = up(hs.stream)
            self.sm = up(hs.sm)
            self.gaps = up(hs.gaps if hs.gaps.size else np.zeros(1, np.uint8))
            self.block_out_pos = up(hs.block_out_pos)
        else:
            self.stream, self.sm, self.gaps, self.block_out_pos = arrays
        self.tables = up(table_image(cb))
        self.tensor_offsets = np.ascontiguousarray(hs.tensor_offsets, dtype=np.uint64)
        self.tensor_tiles = np.ascontiguousarray(
            hs.tensor_tiles if hs.tensor_tiles.size else np.zeros(2, np.uint64), dtype=np.uint64)
        d = df11_device_stream()
        d.stream = self.stream.data_ptr()
        d.sm = self.sm.data_ptr()
        d.gaps = self.gaps.data_ptr()
        d.block_out_pos = self.block_out_pos.data_ptr()
        d.tables = self.tables.data_ptr()
        d.tensor_offsets = self.tensor_offsets.ctypes.data_as(_u64p)
        d.tensor_tiles = self.tensor_tiles.ctypes.data_as(_u64p)
        d.n_weights = hs.n_weights
        d.total_bits = hs.total_bits
        d.n_tiles = hs.n_tiles
        d.n_luts = cb.n_luts
        d.tile_windows = hs.tile_windows
        d.window_bytes = hs.window_bytes
        d.max_tile_symbols = hs.max_tile_symbols
        d.n_tensors = hs.n_tensors
        d.format = hs.format
        self.desc = d

    @property
    def n_weights(self) -> int:
        return int(self.desc.n_weights)

    def device_bytes(self) -> int:
        return sum(t.numel() for t in (self.stream, self.sm, self.gaps, self.block_out_pos,
                                       self.tables))


def _stream_handle(stream):
    import torch

    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream))


def _check_out(ds: DeviceStream, out, n: int) -> None:
    size = 2 if ds.desc.format == 0 else 1
    if out.numel() < n or out.element_size() != size or not out.is_contiguous():
        raise ValueError(f"out must be a contiguous device tensor of {n} {8 * size}-bit elements")


def df11_decompress_block(ds: DeviceStream, out, status=None, stream=None) -> None:
    """One launch decompressing the whole unit into ``out`` (a device tensor of
    n_weights elements: 16-bit (torch.bfloat16, torch.int16) for BF16 units,
    8-bit (torch.uint8, torch.float8_*) for FP8 units)."""
    _check_out(ds, out, ds.n_weights)
    sp = ctypes.c_void_p(status.data_ptr()) if status is not None else ctypes.c_void_p(0)
    _check("df11_decompress_block",
           LIB.df11_decompress_block(ctypes.byref(ds.desc), ctypes.c_void_p(out.data_ptr()), sp,
                                     _stream_handle(stream)))


def df11_decompress_tensor(ds: DeviceStream, k: int, out, status=None, stream=None) -> None:
    """Decompress tensor k of the unit into ``out`` (its numel 16-bit elements)."""
    n = 0
    if 0 <= k < ds.tensor_offsets.size - 1:
        n = int(ds.tensor_offsets[k + 1] - ds.tensor_offsets[k])
    _check_out(ds, out, n)
    sp = ctypes.c_void_p(status.data_ptr()) if status is not None else ctypes.c_void_p(0)
    _check("df11_decompress_tensor",
           LIB.df11_decompress_tensor(ctypes.byref(ds.desc), int(k),
                                      ctypes.c_void_p(out.data_ptr()), sp,
                                      _stream_handle(stream)))


def df11_window_counts(ds: DeviceStream, counts, stream=None) -> None:
    """Phase 1 of the decode on its own: ``counts`` (a device int32 tensor of
    n_tiles * tile_windows elements) receives each stream window's number of
    code starts."""
    n = int(ds.desc.n_tiles) * int(ds.desc.tile_windows)
    if counts.numel() != n or counts.element_size() != 4 or not counts.is_contiguous():
        raise Df11Error(f"df11_window_counts: counts must be {n} contiguous 4-byte elements")
    _check("df11_window_counts",
           LIB.df11_window_counts(ctypes.byref(ds.desc), ctypes.c_void_p(counts.data_ptr()),
                                  _stream_handle(stream)))


# ---------------------------------------------------------------- block pipeline


class Pipeline:
    """df11_pipeline_*: a ring of n_slots output buffers decompressed on
    ``decode_stream`` and read by consumer streams, ordered by events."""

    def __init__(self, decode_stream, n_slots: int = 2):
        self._p = ctypes.c_void_p(0)
        self.decode_stream = decode_stream
        _check("df11_pipeline_create",
               LIB.df11_pipeline_create(_stream_handle(decode_stream), int(n_slots),
                                        ctypes.byref(self._p)))

    def decompress(self, slot: int, ds: DeviceStream, out, status=None) -> None:
        _check_out(ds, out, ds.n_weights)
        sp = ctypes.c_void_p(status.data_ptr()) if status is not None else ctypes.c_void_p(0)
        _check("df11_pipeline_decompress",
               LIB.df11_pipeline_decompress(self._p, int(slot), ctypes.byref(ds.desc),
                                            ctypes.c_void_p(out.data_ptr()), sp))

    def set_decode_share(self, workgroups_per_cu: int) -> None:
        """Cap the decode at this many workgroups per compute unit (0: full grid)."""
        _check("df11_pipeline_set_decode_share",
               LIB.df11_pipeline_set_decode_share(self._p, int(workgroups_per_cu)))

    def acquire(self, slot: int, consumer_stream) -> None:
        _check("df11_pipeline_acquire",
               LIB.df11_pipeline_acquire(self._p, int(slot), _stream_handle(consumer_stream)))

    def release(self, slot: int, consumer_stream) -> None:
        _check("df11_pipeline_release",
               LIB.df11_pipeline_release(self._p, int(slot), _stream_handle(consumer_stream)))

    def close(self) -> None:
        if self._p:
            _check("df11_pipeline_destroy", LIB.df11_pipeline_destroy(self._p))
            self._p = ctypes.c_void_p(0)

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass


def gemv_layout(shapes):
    """df11_gemv_tensor descriptors for row-major matrices stored back to back
    (one decompressed unit), with x and y slices also back to back."""
    descs, w, x, y = [], 0, 0, 0
    for rows, cols in shapes:
        descs.append((w, x, y, rows, cols))
        w += rows * cols
        x += cols
        y += rows
    arr = (df11_gemv_tensor * max(len(descs), 1))()
    for i, (wo, xo, yo, r, c) in enumerate(descs):
        arr[i].w_offset, arr[i].x_offset, arr[i].y_offset, arr[i].rows, arr[i].cols = wo, xo, yo, r, c
    return arr, len(descs), x, y


def df11_gemv_bf16(w, layout, x, y, stream=None) -> None:
    """y = W x per tensor of ``layout`` (from gemv_layout) over the 16-bit
    device tensor ``w``; x and y are float32 device tensors."""
    arr, n, nx, ny = layout
    if w.element_size() != 2 or x.dtype.itemsize != 4 or y.dtype.itemsize != 4:
        raise ValueError("w must be 16-bit, x and y float32")
    if x.numel() < nx or y.numel() < ny:
        raise ValueError("x or y too small for the layout")
    _check("df11_gemv_bf16",
           LIB.df11_gemv_bf16(ctypes.c_void_p(w.data_ptr()), arr, n, ctypes.c_void_p(x.data_ptr()),
                              ctypes.c_void_p(y.data_ptr()), _stream_handle(stream)))


def df11_gemm_order(w, rows: int, cols: int) -> np.ndarray:
    """The host permutation df11_decompress_gemm expects (see include/df11.h):
    16-row blocks of 32-column sub-blocks, each in the matrix cores' lane
    order (four 8-column quarters of 16 rows of 8 weights)."""
    src = np.ascontiguousarray(np.asarray(w).reshape(-1)).view(np.uint16)
    if src.size != rows * cols:
        raise ValueError("w must hold rows * cols weights")
    out = np.empty(rows * cols, dtype=np.uint16)
    _check("df11_gemm_order", LIB.df11_gemm_order(src.ctypes.data_as(_u16p), rows, cols,
                                                  out.ctypes.data_as(_u16p)))
    return out


def gemm_layout(shapes, n_tokens: int):
    """df11_gemv_tensor descriptors for df11_decompress_gemm: matrices back to
    back in the unit, and for each a token-major x slice (n_tokens x cols,
    BF16) and y slice (n_tokens x rows, float32), also back to back."""
    descs, w, x, y = [], 0, 0, 0
    for rows, cols in shapes:
        descs.append((w, x, y, rows, cols))
        w += rows * cols
        x += n_tokens * cols
        y += n_tokens * rows
    arr = (df11_gemv_tensor * max(len(descs), 1))()
    for i, (wo, xo, yo, r, c) in enumerate(descs):
        arr[i].w_offset, arr[i].x_offset, arr[i].y_offset, arr[i].rows, arr[i].cols = wo, xo, yo, r, c
    return arr, len(descs), x, y


def df11_decompress_gemm_scratch_bytes(layout, n_tokens: int) -> int:
    arr, n, _, _ = layout
    return int(LIB.df11_decompress_gemm_scratch_bytes(arr, n, n_tokens))


def df11_decompress_gemm(ds: DeviceStream, layout, n_tokens: int, x, y, scratch=None,
                         status=None, stream=None) -> None:
    """y = W x for n_tokens tokens per matrix of ``layout`` (from gemm_layout)
    on the matrix cores, straight from the compressed unit ``ds`` (encoded
    from df11_gemm_order weights).  x: 16-bit device tensor (BF16 bits), y:
    float32 device tensor; ``scratch``: a device uint8 tensor of
    df11_decompress_gemm_scratch_bytes bytes, allocated here when not given."""
    import torch

    arr, n, nx, ny = layout
    if x.element_size() != 2 or y.dtype.itemsize != 4 or x.numel() < nx or y.numel() < ny:
        raise ValueError("x must be a 16-bit and y a float32 device tensor covering the layout")
    need = df11_decompress_gemm_scratch_bytes(layout, n_tokens)
    if scratch is None:
        scratch = torch.empty(max(need, 16), dtype=torch.uint8, device=x.device)
    sp = ctypes.c_void_p(status.data_ptr()) if status is not None else ctypes.c_void_p(0)
    _check("df11_decompress_gemm",
           LIB.df11_decompress_gemm(ctypes.byref(ds.desc), arr, n, n_tokens,
                                    ctypes.c_void_p(x.data_ptr()), ctypes.c_void_p(y.data_ptr()),
                                    ctypes.c_void_p(scratch.data_ptr()), scratch.numel(), sp,
                                    _stream_handle(stream)))


# ---------------------------------------------------------------- device encoder


def df11_histogram_device(w, fmt: str = "bf16", stream=None, counts=None):
    """Exponent histogram of the device tensor ``w`` (uint64[256] on its device;
    written into ``counts``, a 256-element 8-byte device tensor, when given)."""
    import torch

    if counts is None:
        counts = torch.empty(256, dtype=torch.int64, device=w.device)
    elif counts.numel() != 256 or counts.element_size() != 8 or not counts.is_contiguous():
        raise ValueError("counts must be 256 contiguous 8-byte elements")
    _check("df11_histogram_device",
           LIB.df11_histogram_device(_format(fmt), ctypes.c_void_p(w.data_ptr()), w.numel(),
                                     ctypes.c_void_p(counts.data_ptr()), _stream_handle(stream)))
    return counts


def df11_build_codebook_from_counts(counts) -> df11_codebook:
    c = np.ascontiguousarray(np.asarray(counts), dtype=np.uint64)
    cb = df11_codebook()
    _check("df11_build_codebook_from_counts",
           LIB.df11_build_codebook_from_counts(c.ctypes.data_as(_u64p), ctypes.byref(cb)))
    return cb


def df11_tensor_ranges_from_counts(cb: df11_codebook, counts, last_weights, fmt: str = "bf16",
                                   tile_windows: int = DEFAULT_TILE_WINDOWS,
                                   window_bytes: int = DEFAULT_WINDOW_BYTES):
    """(tensor_offsets uint64[n+1], tensor_tiles uint64[2n]) from per-tensor
    histograms ``counts`` (n x 256) and the tensors' last weights (n bit patterns)."""
    c = np.ascontiguousarray(np.asarray(counts), dtype=np.uint64).reshape(-1, 256)
    n = c.shape[0]
    last = np.ascontiguousarray(np.asarray(last_weights), dtype=np.uint32).reshape(-1)
    if last.size != n:
        raise ValueError("one last weight per tensor")
    offs = np.zeros(n + 1, dtype=np.uint64)
    tiles = np.zeros(max(2 * n, 1), dtype=np.uint64)
    _check("df11_tensor_ranges_from_counts",
           LIB.df11_tensor_ranges_from_counts(_format(fmt), ctypes.byref(cb), c.ctypes.data_as(_u64p),
                                              last.ctypes.data_as(_u32p), n, tile_windows,
                                              window_bytes, offs.ctypes.data_as(_u64p),
                                              tiles.ctypes.data_as(_u64p)))
    return offs, tiles[: 2 * n]


def encode_on_device(tensors, fmt: str = "bf16", tile_windows: int = DEFAULT_TILE_WINDOWS,
                     window_bytes: int = DEFAULT_WINDOW_BYTES, stream=None):
    """Compress device tensors (16-bit for BF16, 8-bit for FP8) into a
    DeviceStream without moving the weights to the host: per-tensor device
    histograms, the codebook built on the host from them, then
    df11_encode_device on the concatenated unit.  Every allocation, copy and
    launch is ordered on ``stream`` (a torch stream or a raw hipStream_t; the
    current stream when None), and the call returns once that stream has
    finished the encoding.  Returns (DeviceStream, codebook)."""
    import torch

    if stream is None:
        st = torch.cuda.current_stream()
    elif isinstance(stream, torch.cuda.Stream):
        st = stream
    else:
        st = torch.cuda.ExternalStream(int(getattr(stream, "cuda_stream", stream)))
    size = 2 if fmt == "bf16" else 1
    for t in tensors:
        if t.element_size() != size:
            raise TypeError(f"{fmt} tensors must have {8 * size}-bit elements")
    cur = torch.cuda.current_stream()
    with torch.cuda.stream(st):
        if st != cur:
            st.wait_stream(cur)  # the work that wrote the tensors comes first
        flat = [t.reshape(-1).view(torch.int16 if size == 2 else torch.uint8).contiguous()
                for t in tensors]
        unit = torch.cat(flat) if len(flat) != 1 else flat[0]
        n = unit.numel()
        dev = unit.device
        per = torch.zeros((max(len(flat), 1), 256), dtype=torch.int64, device=dev)
        lasts = torch.zeros(max(len(flat), 1), dtype=torch.int32, device=dev)
        for k, t in enumerate(flat):
            if t.numel():
                df11_histogram_device(t, fmt, st, per[k])
                lasts[k] = t[-1].to(torch.int32)
        per_h = per.cpu().numpy().view(np.uint64)[: len(flat)]  # waits for st
        lasts_h = lasts.cpu().numpy().view(np.uint32)[: len(flat)] & (0xFFFF if size == 2 else 0xFF)
        counts = per_h.sum(axis=0, dtype=np.uint64) if len(flat) else np.zeros(256, np.uint64)
        cb = df11_build_codebook_from_counts(counts)
        sz = df11_sizes()
        _check("df11_encode_size_from_counts",
               LIB.df11_encode_size_from_counts(_format(fmt), ctypes.byref(cb),
                                                counts.ctypes.data_as(_u64p), n, tile_windows,
                                                window_bytes, ctypes.byref(sz)))
        offs, tiles = df11_tensor_ranges_from_counts(cb, per_h, lasts_h, fmt, tile_windows,
                                                     window_bytes)
        stm = torch.empty(sz.stream_bytes, dtype=torch.uint8, device=dev)
        sm = torch.empty(sz.sm_bytes, dtype=torch.uint8, device=dev)
        gaps = torch.empty(max(16, sz.n_windows), dtype=torch.uint8, device=dev)
        bop = torch.empty(sz.bop_entries, dtype=torch.int32, device=dev)
        mx = torch.empty(4, dtype=torch.int32, device=dev)
        nbytes = int(LIB.df11_encode_device_scratch_bytes(n))
        scratch = torch.empty(nbytes + 256, dtype=torch.uint8, device=dev)
        sp = scratch.data_ptr()
        out = df11_device_encode(stm.data_ptr(), sm.data_ptr(), gaps.data_ptr(), bop.data_ptr(),
                                 mx.data_ptr(), (sp + 255) // 256 * 256, nbytes)
        _check("df11_encode_device",
               LIB.df11_encode_device(_format(fmt), ctypes.byref(cb),
                                      ctypes.c_void_p(unit.data_ptr()), n, tile_windows,
                                      window_bytes, ctypes.byref(sz), ctypes.byref(out),
                                      _stream_handle(st)))
        max_tile = int(mx.cpu()[0])  # waits for st: the arrays are complete
    hs = HostStream(np.zeros(0, np.uint8), np.zeros(0, np.uint8), np.zeros(sz.n_windows, np.uint8),
                    np.zeros(sz.bop_entries, np.uint32), offs, tiles, tile_windows, window_bytes,
                    max_tile, n, int(sz.total_bits), int(sz.n_tiles), _format(fmt))
    ds = DeviceStream(hs, cb, dev, arrays=(stm, sm, gaps, bop))
    return ds, cb


def df11_decompress_gemv(ds: DeviceStream, layout, x, y, scratch=None, status=None,
                         stream=None) -> None:
    """y = W x per matrix of ``layout`` (from gemv_layout, matching the unit's
    tensors) computed straight from the compressed unit ``ds``.  ``scratch``: a
    device uint8 tensor of df11_decompress_gemv_scratch_bytes bytes, allocated
    here when not given."""
    import torch

    arr, n, nx, ny = layout
    if x.dtype.itemsize != 4 or y.dtype.itemsize != 4 or x.numel() < nx or y.numel() < ny:
        raise ValueError("x and y must be float32 device tensors covering the layout")
    need = int(LIB.df11_decompress_gemv_scratch_bytes(ctypes.byref(ds.desc)))
    if scratch is None:
        scratch = torch.empty(need, dtype=torch.uint8, device=x.device)
    sp = ctypes.c_void_p(status.data_ptr()) if status is not None else ctypes.c_void_p(0)
    _check("df11_decompress_gemv",
           LIB.df11_decompress_gemv(ctypes.byref(ds.desc), arr, n, ctypes.c_void_p(x.data_ptr()),
                                    ctypes.c_void_p(y.data_ptr()),
                                    ctypes.c_void_p(scratch.data_ptr()), scratch.numel(), sp,
                                    _stream_handle(stream)))


DF11_GEMV_NOALLOC_MAX_TILES = 786432


def df11_decompress_gemv_noalloc(ds: DeviceStream, layout, x, y, status=None,
                                 stream=None) -> None:
    """df11_decompress_gemv on the library's static per-GPU workspace (no
    allocation anywhere in the call; units of at most
    DF11_GEMV_NOALLOC_MAX_TILES tiles; calls on one GPU must not overlap)."""
    arr, n, nx, ny = layout
    if x.dtype.itemsize != 4 or y.dtype.itemsize != 4 or x.numel() < nx or y.numel() < ny:
        raise ValueError("x and y must be float32 device tensors covering the layout")
    sp = ctypes.c_void_p(status.data_ptr()) if status is not None else ctypes.c_void_p(0)
    _check("df11_decompress_gemv_noalloc",
           LIB.df11_decompress_gemv_noalloc(ctypes.byref(ds.desc), arr, n,
                                            ctypes.c_void_p(x.data_ptr()),
                                            ctypes.c_void_p(y.data_ptr()), sp,
                                            _stream_handle(stream)))


def table_bytes(cb: df11_codebook) -> int:
    """df11_table_bytes(): multi-symbol, count and n_luts hierarchical tables."""
    return ctypes.sizeof(cb.multi) + ctypes.sizeof(cb.count) + 512 * int(cb.n_luts)


def table_image(cb: df11_codebook) -> np.ndarray:
    """The device copy of the codebook's tables (bytes from cb.multi onward)."""
    start = df11_codebook.multi.offset
    raw = ctypes.string_at(ctypes.addressof(cb) + start, table_bytes(cb))
    return np.frombuffer(raw, dtype=np.uint8).copy()


def codebook_arrays(cb: df11_codebook):
    """(code_len uint8[256], code uint32[256]) views of a codebook."""
    return (np.ctypeslib.as_array(cb.code_len).copy(), np.ctypeslib.as_array(cb.code).copy())
