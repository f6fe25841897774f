"""The oracle's pins against planted mistakes.

Each case plants one plausible mistake in a copy of the oracle (a wrong
shift, index, comparison, bit order, term or operand layout), lets the copy
rebuild itself with gcc, and runs the pin suite (tests/test_oracle_pins.py)
against it in a fresh process: the case passes when a pin fails.  The
unmodified copy must pass every pin.  The copies live in a temporary
directory; nothing here touches the GPU, the product library or the oracle
in the repository.
"""

import concurrent.futures
import os
import re
import shutil
import subprocess
import sys
import tempfile
from dataclasses import dataclass

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
C = "oracle/df11_oracle.c"
PY = "oracle/__init__.py"

# (name, file, anchor, old, new): in `file`, the first `old` after the one
# place where `anchor` occurs becomes `new`.
MUTANTS = [
    # histogram and Huffman lengths
    ("histogram reads the wrong exponent bits", C, "void oracle_histogram(const uint16_t",
     "(w[i] >> 7) & 0xFF", "(w[i] >> 8) & 0xFF"),
    ("Huffman tie-break reversed", C, "int oracle_huffman_lengths",
     "tiebreak[i] < tiebreak[best]", "tiebreak[i] > tiebreak[best]"),
    ("Huffman takes the later of equal weights", C, "int oracle_huffman_lengths",
     "weight[i] < weight[best] ||", "weight[i] <= weight[best] ||"),
    ("single symbol coded without its dummy", C, "int oracle_huffman_lengths",
     "lens[dummy] = 1;", "(void)dummy;"),
    ("internal nodes tie-broken before leaves", C, "int oracle_huffman_lengths",
     "(uint32_t)(NSYM + k)", "(uint32_t)k"),
    ("code length counted one too long", C, "int oracle_huffman_lengths",
     "int depth = 0;", "int depth = 1;"),
    # package-merge
    ("package-merge leaves in descending symbol order on equal weight", C,
     "int oracle_limited_lengths", "sym[j] > s", "sym[j] < s"),
    ("package-merge puts packages before equal leaves", C, "int oracle_limited_lengths",
     "counts[sym[li]] <= pw", "counts[sym[li]] < pw"),
    ("package-merge pairs an item with itself", C, "int oracle_limited_lengths",
     "lists[level + 1][2 * pi + 1].w", "lists[level + 1][2 * pi].w"),
    ("package-merge takes one item too few", C, "int oracle_limited_lengths",
     "i < 2 * n - 2", "i < 2 * n - 3"),
    ("length limit applied one bit late", C, "int oracle_code_lengths",
     "m > MAXLEN", "m > MAXLEN + 1"),
    # canonical codes
    ("canonical code incremented after the shift", C, "void oracle_canonical_codes",
     "code = (code + 1) << (lens[order[i]] - lens[order[i - 1]]);",
     "code = (code << (lens[order[i]] - lens[order[i - 1]])) + 1;"),
    ("canonical codes of one length in descending value order", C,
     "void oracle_canonical_codes", "order[j] > s", "order[j] < s"),
    # encoder
    ("stream bits least significant first", C, "int oracle_encode(const uint16_t",
     "0x80u >> (pos % 8)", "1u << (pos % 8)"),
    ("code bits written lowest first", C, "int oracle_encode(const uint16_t",
     "for (int k = l - 1; k >= 0; k--)", "for (int k = 0; k < l; k++)"),
    ("sm byte keeps the exponent's low bit", C, "int oracle_encode(const uint16_t",
     "(w[i] & 0x7F)", "(w[i] & 0xFF)"),
    ("sm sign taken from the wrong bit", C, "int oracle_encode(const uint16_t",
     "((w[i] >> 8) & 0x80)", "((w[i] >> 9) & 0x80)"),
    # auxiliary arrays
    ("gap one bit late", C, "int oracle_aux_fast(",
     "gaps[j] = (uint8_t)(start - j * window_bits);",
     "gaps[j] = (uint8_t)(start - j * window_bits + 1);"),
    ("block_out_pos counts its own tile", C, "int oracle_aux_fast(",
     "block_out_pos[t] = (uint32_t)acc;\n        if (t < n_tiles)\n            acc += starts_in_tile[t];",
     "if (t < n_tiles)\n            acc += starts_in_tile[t];\n        block_out_pos[t] = (uint32_t)acc;"),
    ("code assigned to the window where it ends", C, "int oracle_aux_fast(",
     "uint64_t j = start / window_bits;",
     "uint64_t j = (start + lens[(w[i] >> 7) & 0xFF] - 1) / window_bits;"),
    ("plain block_out_pos counts a code in its own tile", C, "int oracle_aux(const",
     "t = start / tile_bits + 1;", "t = start / tile_bits;"),
    # decoder
    ("decoder accepts one code past a length's range", C, "int oracle_decode(const",
     "v - first[l] < count[l]", "v - first[l] <= count[l]"),
    ("decoder places the exponent one bit high", C, "int oracle_decode(const",
     "((uint32_t)sym << 7)", "((uint32_t)sym << 8)"),
    ("decoder's first codes built without the carry", C, "int oracle_decode(const",
     "code = (code + count[l]) << 1;", "code = (code << 1) + count[l];"),
    ("decoder reads bits least significant first", C, "int oracle_decode(const",
     "(7 - pos % 8)", "(pos % 8)"),
    ("decoder puts the sign one bit low", C, "int oracle_decode(const",
     "((sm[i] & 0x80u) << 8)", "((sm[i] & 0x80u) << 7)"),
    ("decoder keeps the sm byte's top bit in the mantissa", C, "int oracle_decode(const",
     "(sm[i] & 0x7Fu)", "(sm[i] & 0xFFu)"),
    ("gap from the last code start in the window", C, "int oracle_aux_fast(",
     "if (gaps[j] == 255)", "if (1)"),
    ("plain gap one bit late", C, "int oracle_aux(const",
     "gaps[j] = (uint8_t)(start - j * window_bits);",
     "gaps[j] = (uint8_t)(start - j * window_bits + 1);"),
    ("encoder reports one bit too many", C, "int oracle_encode(const uint16_t",
     "*total_bits = pos;", "*total_bits = pos + 1;"),
    ("single symbol's dummy is the largest absent symbol", C, "int oracle_huffman_lengths",
     "for (int s = 0; s < NSYM && dummy < 0; s++)", "for (int s = NSYM - 1; s >= 0 && dummy < 0; s--)"),
    # FP8
    ("FP8 nibbles in the wrong half of the byte", C, "int oracle_fp8_split(",
     "nib << (4 * (i % 2))", "nib << (4 * (1 - i % 2))"),
    ("FP8 sign placed above bit 2 for every format", C, "int oracle_fp8_split(",
     "unsigned nib = (s << mb) | m;", "unsigned nib = (s << 3) | m;"),
    ("E4M3 mantissa one bit wide too many", C, "static int fp8_fields(",
     "*ebits = 4; *mbits = 3;", "*ebits = 4; *mbits = 4;"),
    ("FP8 exponent field one bit narrow", C, "int oracle_fp8_split(",
     "((1u << eb) - 1u)", "((1u << (eb - 1)) - 1u)"),
    ("E5M2 exponent field four bits wide", C, "static int fp8_fields(",
     "*ebits = 5; *mbits = 2;", "*ebits = 4; *mbits = 2;"),
    ("FP8 merge takes the sign from bit 3 in every format", C, "int oracle_fp8_merge(",
     "unsigned s = (nib >> mb) & 1u;", "unsigned s = (nib >> 3) & 1u;"),
    ("FP8 merge shifts the exponent one bit high", C, "int oracle_fp8_merge(",
     "((unsigned)sym[i] << mb)", "((unsigned)sym[i] << (mb + 1))"),
    ("symbol stream bits least significant first", C, "int oracle_encode_symbols(",
     "0x80u >> (pos % 8)", "1u << (pos % 8)"),
    ("symbol gaps one bit late", C, "int oracle_aux_symbols(",
     "gaps[j] = (uint8_t)(start - j * window_bits);",
     "gaps[j] = (uint8_t)(start - j * window_bits + 1);"),
    ("symbol block_out_pos counts its own tile", C, "int oracle_aux_symbols(",
     "block_out_pos[t] = (uint32_t)acc;\n        if (t < n_tiles)\n            acc += starts_in_tile[t];",
     "if (t < n_tiles)\n            acc += starts_in_tile[t];\n        block_out_pos[t] = (uint32_t)acc;"),
    ("symbol decoder accepts one code past a length's range", C, "int oracle_decode_symbols(",
     "v - first[l] < count[l]", "v - first[l] <= count[l]"),
    ("symbol decoder reads bits least significant first", C, "int oracle_decode_symbols(",
     "(7 - pos % 8)", "(pos % 8)"),
    # the Python side: wrappers, closed forms and the matrix products
    ("codebook without the 32-bit limit", PY, "def codebook(tensors)",
     "lens = code_lengths(counts)", "lens = huffman_lengths(counts)"),
    ("encoded stream loses its last partial byte", PY, "def encode(tensors",
     "return Encoded(stream[: (total + 7) // 8]", "return Encoded(stream[: total // 8]"),
    ("aux adds a tile when the stream fills its last one", PY, "def aux(tensors",
     "n_tiles = (total + tile_bits - 1) // tile_bits", "n_tiles = total // tile_bits + 1"),
    ("symbol aux adds a tile when the stream fills its last one", PY, "def aux_symbols(",
     "n_tiles = (total + window_bits * tile_windows - 1) // (window_bits * tile_windows)",
     "n_tiles = total // (window_bits * tile_windows) + 1"),
    ("window counts from code ends", PY, "def window_counts(",
     "starts = np.cumsum(ln) - ln", "starts = np.cumsum(ln)"),
    ("entropy in nats", PY, "def entropy_bits(", "np.log2(p)", "np.log(p)"),
    ("Kraft numerator doubled", PY, "def kraft_numerator(",
     "1 << (MAX_LEN - int(l))", "1 << (MAX_LEN - int(l) + 1)"),
    ("total code bits adds instead of multiplying", PY, "def total_code_bits(",
     "int(c) * int(l)", "int(c) + int(l)"),
    ("sign+mantissa helper takes the sign from the exponent", PY, "def sign_mantissa(",
     "((w >> 8) & 0x80)", "((w >> 7) & 0x80)"),
    ("exponent helper one bit off", PY, "def exponents(", ">> 7) & 0xFF", ">> 8) & 0xFF"),
    ("Gaussian binade edges one binade high", PY, "def gaussian_exponent_probs(",
     "lo, hi = 2.0 ** (e - 127), 2.0 ** (e - 126)", "lo, hi = 2.0 ** (e - 126), 2.0 ** (e - 125)"),
    ("BF16 value from a 15-bit shift", PY, "def bf16_to_f64(", "<< 16", "<< 15"),
    ("GEMV x slices advance by rows", PY, "def gemv(", "xo += cols", "xo += rows"),
    ("GEMV reads x backwards", PY, "def gemv(", "W @ x[xo:xo + cols]", "W @ x[xo:xo + cols][::-1]"),
    ("GEMM activations read transposed", PY, "def gemm(",
     ".reshape(n_tokens, cols)", ".reshape(cols, n_tokens).T"),
    ("GEMM with W untransposed and X transposed", PY, "def gemm(",
     "(X @ W.T).reshape(-1)", "(W @ X.T).reshape(-1)"),
]


def _copy_tree(dst):
    for d in ("oracle", "synth_weights", "tests", "tests/golden"):
        os.makedirs(os.path.join(dst, d), exist_ok=True)
    for f in (C, PY, "pytest.ini", "tests/conftest.py", "tests/test_oracle_pins.py"):
        shutil.copy(os.path.join(ROOT, f), os.path.join(dst, f))
    for d in ("synth_weights", "tests/golden"):
        for f in os.listdir(os.path.join(ROOT, d)):
            if f.endswith((".py", ".txt")):
                shutil.copy(os.path.join(ROOT, d, f), os.path.join(dst, d, f))


def _plant(dst, file, anchor, old, new):
    path = os.path.join(dst, file)
    src = open(path).read()
    assert src.count(anchor) == 1, f"anchor {anchor!r} must occur once in {file}"
    i = src.find(old, src.index(anchor))
    assert i >= 0, f"{old!r} not found after {anchor!r} in {file}"
    with open(path, "w") as f:
        f.write(src[:i] + new + src[i + len(old):])


NOT_BUILT, TIMED_OUT = -1000, -999


@dataclass
class Outcome:
    returncode: int
    first_failure: str
    tail: str


def _run_pins(dst) -> Outcome:
    env = dict(os.environ, PYTHONDONTWRITEBYTECODE="1", PYTHONPATH="")
    try:
        r = subprocess.run([sys.executable, "-m", "pytest", "-x", "-q", "-p", "no:cacheprovider",
                            "tests/test_oracle_pins.py"], cwd=dst, env=env, capture_output=True,
                           text=True, timeout=240)
    except subprocess.TimeoutExpired as e:
        return Outcome(TIMED_OUT, "timed out", str(e.stdout)[-2000:])
    m = re.search(r"FAILED (\S+)", r.stdout)
    return Outcome(r.returncode, m.group(1) if m else "", (r.stdout + r.stderr)[-2000:])


def _case(args):
    name, planted = args
    dst = tempfile.mkdtemp(prefix="df11_oracle_mutant_")
    try:
        _copy_tree(dst)
        if planted is not None:
            _plant(dst, *planted)
        # build the copy's library here, so that a planted mistake that does
        # not compile is reported as such rather than as a failing pin
        r = subprocess.run(["gcc", "-O2", "-std=c99", "-fPIC", "-shared", os.path.join(dst, C),
                            "-o", os.path.join(dst, "oracle", "libdf11_oracle.so")],
                           capture_output=True, text=True)
        if r.returncode != 0:
            return name, Outcome(NOT_BUILT, "", r.stderr[-2000:])
        return name, _run_pins(dst)
    finally:
        shutil.rmtree(dst, ignore_errors=True)


@pytest.fixture(scope="module")
def outcomes():
    cases = [("unmodified", None)] + [(m[0], m[1:]) for m in MUTANTS]
    workers = max(1, min(8, os.cpu_count() or 1))
    with concurrent.futures.ThreadPoolExecutor(workers) as ex:
        return dict(ex.map(_case, cases))


def test_mutant_names_are_distinct():
    assert len({m[0] for m in MUTANTS}) == len(MUTANTS)


def test_the_unmodified_copy_passes_every_pin(outcomes):
    o = outcomes["unmodified"]
    assert o.returncode == 0, o.tail


@pytest.mark.parametrize("name", [m[0] for m in MUTANTS])
def test_a_planted_mistake_fails_a_pin(outcomes, name):
    o = outcomes[name]
    assert o.returncode != NOT_BUILT, f"the planted copy does not compile: {name}\n{o.tail}"
    # pytest exits with 1 when a test failed; a crash of the planted copy
    # (a signal) or a hang also means the mistake was caught, while 2-5
    # (interrupted, internal or usage error, nothing collected) do not
    assert o.returncode != 0 and o.returncode not in (2, 3, 4, 5), \
        f"no pin caught: {name}\n{o.tail}"
