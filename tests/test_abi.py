"""The C-ABI library loads and exports every function include/df11.h declares.

No compute call runs here (that needs a GPU); the host calls are covered by
test_host_codec.py.
"""

import ctypes
import os
import re
import subprocess
import sys

import entropy_decoding_amd as ed

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "df11.h")


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:const\s+)?\w+\s*\*?\s*(df11_\w+)\s*\(", text, flags=re.M)))


def test_header_declares_the_boundary():
    names = declared_functions()
    for n in ("df11_build_codebook", "df11_encode_size", "df11_encode",
              "df11_decompress_tensor", "df11_decompress_block", "df11_status_string"):
        assert n in names


def test_library_exports_every_declared_symbol():
    lib = ctypes.CDLL(ed.LIB_PATH)
    for n in declared_functions():
        assert hasattr(lib, n), n
    out = subprocess.run(["nm", "-D", "--defined-only", ed.LIB_PATH], capture_output=True,
                         text=True, check=True).stdout
    exported = set(re.findall(r"\bT (df11_\w+)", out))
    assert set(declared_functions()) <= exported


def test_struct_sizes_match_the_header():
    src = f'''
#include <stdio.h>
#include <stddef.h>
#include "df11.h"
int main(void) {{
  printf("%zu %zu %zu %zu\\n", sizeof(df11_codebook), sizeof(df11_sizes),
         sizeof(df11_host_stream), sizeof(df11_device_stream));
  printf("%zu %zu %zu\\n", offsetof(df11_codebook, lut), offsetof(df11_host_stream, n_weights),
         offsetof(df11_device_stream, n_luts));
  printf("%zu %zu %zu %d %d\\n", sizeof(df11_gemv_tensor), offsetof(df11_gemv_tensor, rows),
         offsetof(df11_gemv_tensor, cols), DF11_PIPELINE_MAX_SLOTS, DF11_GEMV_MAX_TENSORS);
  printf("%zu %zu %d %d %d\\n", offsetof(df11_host_stream, format),
         offsetof(df11_device_stream, format), DF11_FORMAT_BF16, DF11_FORMAT_FP8_E4M3,
         DF11_FORMAT_FP8_E5M2);
  return 0;
}}
'''
    import tempfile

    with tempfile.TemporaryDirectory() as d:
        c = os.path.join(d, "s.c")
        exe = os.path.join(d, "s")
        open(c, "w").write(src)
        subprocess.check_call(["gcc", "-I", os.path.join(ROOT, "include"), c, "-o", exe])
        lines = subprocess.check_output([exe], text=True).split("\n")
    sizes = [int(x) for x in lines[0].split()]
    offs = [int(x) for x in lines[1].split()]
    assert sizes == [ctypes.sizeof(ed.df11_codebook), ctypes.sizeof(ed.df11_sizes),
                     ctypes.sizeof(ed.df11_host_stream), ctypes.sizeof(ed.df11_device_stream)]
    assert offs == [ed.df11_codebook.lut.offset, ed.df11_host_stream.n_weights.offset,
                    ed.df11_device_stream.n_luts.offset]
    g = [int(x) for x in lines[2].split()]
    assert g == [ctypes.sizeof(ed.df11_gemv_tensor), ed.df11_gemv_tensor.rows.offset,
                 ed.df11_gemv_tensor.cols.offset, ed.DF11_PIPELINE_MAX_SLOTS,
                 ed.DF11_GEMV_MAX_TENSORS]
    f = [int(x) for x in lines[3].split()]
    assert f == [ed.df11_host_stream.format.offset, ed.df11_device_stream.format.offset,
                 ed.FORMATS["bf16"], ed.FORMATS["fp8_e4m3"], ed.FORMATS["fp8_e5m2"]]


def test_status_strings():
    for s in range(7):
        assert ed.status_string(s)
    assert ed.status_string(ed.DF11_E_CORRUPT).startswith("compressed stream")


def test_one_hip_runtime_per_process():
    """libdf11 must share PyTorch's HIP runtime (streams and launches are per runtime)."""
    code = ("import entropy_decoding_amd, torch\n"
            "maps = open('/proc/self/maps').read().split('\\n')\n"
            "paths = {l.split()[-1] for l in maps if 'libamdhip64' in l}\n"
            "print(len(paths), sorted(paths))\n")
    out = subprocess.run([sys.executable, "-c", code], capture_output=True, text=True, cwd=ROOT,
                         check=True).stdout
    assert out.startswith("1 "), out


def test_empty_unit_claiming_tiles_is_rejected_before_any_launch():
    """A descriptor with no weights but tiles or bits is inconsistent: every
    device entry point rejects it on the host (its pointers are null, so a
    launch would read through them)."""
    import ctypes

    import entropy_decoding_amd as ed

    for n_tiles, total_bits in ((1, 0), (1, 64), (0, 8)):
        d = ed.df11_device_stream()
        d.n_weights, d.n_tiles, d.total_bits = 0, n_tiles, total_bits
        d.tile_windows, d.window_bytes, d.n_luts = 64, 8, 1
        counts = ctypes.c_void_p(0x1000)  # never dereferenced: the call returns first
        assert ed.LIB.df11_window_counts(ctypes.byref(d), counts, None) == ed.DF11_E_INVALID
        assert ed.LIB.df11_decompress_block(ctypes.byref(d), counts, None, None) == ed.DF11_E_INVALID
    # more weights than bits, or more bits than 32 per weight, cannot be a valid unit
    for n, bits in ((100, 99), (2, 65)):
        d = ed.df11_device_stream()
        d.n_weights, d.total_bits, d.n_tiles = n, bits, 1
        d.tile_windows, d.window_bytes, d.n_luts = 64, 8, 1
        assert ed.LIB.df11_decompress_block(ctypes.byref(d), ctypes.c_void_p(0x1000), None,
                                            None) == ed.DF11_E_INVALID
