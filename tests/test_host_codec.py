"""Host half of the library (codebook + encoder) against the oracle, on CPU.

The library and the oracle follow the same tie-break and canonical rules, so
code lengths, codes, stream bytes, sm bytes, gaps and block_out_pos must be
equal byte for byte; where package-merge limits lengths, several optimal
codes exist and only the total size is unique.
"""

import numpy as np
import pytest

import entropy_decoding_amd as ed
import oracle
import synth_weights as sw


def _compare(tensors, threads=512, bpt=8, expect_same_lengths=True):
    cb = ed.df11_build_codebook(tensors)
    lens, codes = ed.codebook_arrays(cb)
    ocb = oracle.codebook(tensors)
    assert oracle.kraft_numerator(lens) == 1 << 32
    assert oracle.total_code_bits(ocb.counts, lens) == oracle.total_code_bits(ocb.counts, ocb.lens)
    if expect_same_lengths:
        assert np.array_equal(lens, ocb.lens)
        assert np.array_equal(codes, ocb.codes)
    else:
        ocb = oracle.Codebook(ocb.counts, lens, oracle.canonical_codes(lens))
        assert np.array_equal(codes, ocb.codes)
    hs = ed.df11_encode(cb, tensors, threads, bpt)
    enc = oracle.encode(tensors, ocb)
    nb = (enc.total_bits + 7) // 8
    assert hs.total_bits == enc.total_bits
    assert np.array_equal(hs.stream[:nb], enc.stream)
    assert not hs.stream[nb:].any()
    assert hs.stream.size == hs.n_tiles * threads * bpt + ed.DF11_STREAM_PAD
    n = sum(np.asarray(t).size for t in tensors)
    assert np.array_equal(hs.sm[:n], enc.sm)
    assert not hs.sm[n:].any()
    gaps, bop = oracle.aux(tensors, ocb, threads, bpt)
    assert np.array_equal(hs.gaps, gaps)
    assert np.array_equal(hs.block_out_pos, bop)
    assert hs.max_tile_symbols == (int(np.diff(bop.astype(np.int64)).max()) if bop.size > 1 else 0)
    # tensor offsets and tile ranges from the oracle's per-tensor start bits
    assert hs.tensor_offsets.tolist() == [0, *np.cumsum(enc.numel).tolist()]
    tile_bits = 8 * bpt * threads
    for k, t in enumerate(tensors):
        t = np.asarray(t).reshape(-1)
        if t.size == 0:
            assert hs.tensor_tiles[2 * k] == hs.tensor_tiles[2 * k + 1]
            continue
        first = enc.tensor_start_bits[k] // tile_bits
        last_len = int(lens[(int(t[-1]) >> 7) & 0xFF])
        last = (enc.tensor_start_bits[k + 1] - last_len) // tile_bits + 1
        assert (hs.tensor_tiles[2 * k], hs.tensor_tiles[2 * k + 1]) == (first, last)
    return cb, hs, ocb, enc


def test_config0_matches_oracle(unit_tensors):
    _compare(unit_tensors("0"))


@pytest.mark.parametrize("cfg", ["3a", "3b", "3c"])
def test_stress_configs_match_oracle(unit_tensors, cfg):
    (w,) = unit_tensors(cfg)
    _compare([w[: 1 << 22]])


@pytest.mark.parametrize("tw", [64, 256])
def test_smaller_tiles_match_oracle(unit_tensors, tw):
    _compare(unit_tensors("0"), threads=tw)


def test_multi_tensor_unit_with_ragged_and_empty_tensors():
    rng = np.random.default_rng(11)
    ts = []
    for n in (4097, 0, 1, 333_333, 8, 5_000_001 % 700_000):
        z = (rng.standard_normal(n).astype(np.float32) * 0.02).view(np.uint32) >> 16
        ts.append(z.astype(np.uint16))
    _compare(ts)


def test_pieces_larger_than_one_encoder_work_item():
    # > 4 Mi weights per tensor exercises the parallel pieces and their stitching
    rng = np.random.default_rng(12)
    z = (rng.standard_normal((1 << 22) + 12345).astype(np.float32) * 0.05).view(np.uint32) >> 16
    _compare([z.astype(np.uint16), z[:777].astype(np.uint16)])


@pytest.mark.parametrize("n", [1, 2, 7, 64, 2047, 2048, 2049])
def test_tiny_units(n):
    rng = np.random.default_rng(n)
    w = rng.integers(0, 1 << 16, size=n, dtype=np.uint16)
    w[::3] = 0x3F80
    _compare([w])


def test_single_exponent_unit():
    w = (np.arange(50_000, dtype=np.uint16) & np.uint16(0x807F)) | np.uint16(121 << 7)
    cb, hs, ocb, _ = _compare([w])
    lens, _ = ed.codebook_arrays(cb)
    assert lens[121] == 1 and lens[0] == 1 and cb.n_luts == 1
    assert hs.total_bits == w.size


def test_every_bf16_bit_pattern():
    w = np.arange(1 << 16, dtype=np.uint16)
    np.random.default_rng(13).shuffle(w)
    cb, hs, _, _ = _compare([w])
    assert cb.max_len == 8 and cb.n_luts == 1


def _fib_unit(nsym=36):
    f = [1, 1]
    while len(f) < nsym:
        f.append(f[-1] + f[-2])
    sym = np.repeat(np.arange(nsym, dtype=np.uint16) + 90, f)
    np.random.default_rng(14).shuffle(sym)
    return ((sym << 7) | (np.arange(sym.size) & 0x807F)).astype(np.uint16)


def test_length_limited_codebook_forced_by_fibonacci_counts():
    w = _fib_unit()
    cb, hs, _, _ = _compare([w], expect_same_lengths=False)
    assert cb.max_len == 32
    assert cb.n_luts >= 4


def test_lut_entries_resolve_every_code():
    """Walk the library's tables for every code, as a decoder would."""
    w = _fib_unit()
    cb = ed.df11_build_codebook([w])
    lens, codes = ed.codebook_arrays(cb)
    lut = np.ctypeslib.as_array(cb.lut)
    for s in np.nonzero(lens)[0]:
        l = int(lens[s])
        v = int(codes[s]) << (32 - l)
        table, lvl = 0, 0
        while True:
            e = int(lut[table][(v >> (24 - 8 * lvl)) & 0xFF])
            if e & 0x8000:
                table, lvl = e & 0x7FFF, lvl + 1
                assert table < cb.n_luts and lvl < 4
                continue
            assert (e >> 8) & 0x3F == l and e & 0xFF == s
            break


def test_errors():
    w = np.zeros(10, dtype=np.uint16) | np.uint16(100 << 7)
    cb = ed.df11_build_codebook([w])
    other = np.full(4, 50 << 7, dtype=np.uint16)
    with pytest.raises(ed.Df11Error) as e:
        ed.df11_encode(cb, [other])
    assert e.value.status == ed.DF11_E_SYMBOL
    with pytest.raises(ed.Df11Error) as e:
        ed.df11_encode(cb, [w], tile_windows=128)
    assert e.value.status == ed.DF11_E_INVALID
    with pytest.raises(ed.Df11Error) as e:
        ed.df11_build_codebook([np.zeros(0, dtype=np.uint16)])
    assert e.value.status == ed.DF11_E_INVALID


def test_lut_budget_error():
    # dyadic counts force the lengths: 64 symbols of 7 bits, 64 of 8, 128 of 9.
    # The 9-bit codes fill 64 distinct 8-bit prefixes, so the root needs 64
    # second-level tables: 65 in all, one over the budget.
    counts = np.zeros(256, dtype=np.int64)
    counts[:64], counts[64:128], counts[128:] = 4, 2, 1
    w = np.repeat(np.arange(256, dtype=np.uint16) << 7, counts)
    ocb = oracle.codebook(w)
    assert sorted(set(ocb.lens.tolist())) == [7, 8, 9]
    with pytest.raises(ed.Df11Error) as e:
        ed.df11_build_codebook([w])
    assert e.value.status == ed.DF11_E_LUT_BUDGET
    # one 9-bit prefix fewer fits: merge two 9-bit pairs into 8-bit codes
    counts[128:] = 1
    counts[126:128] = 0
    counts[128:130] = 2
    w = np.repeat(np.arange(256, dtype=np.uint16) << 7, counts)
    cb = ed.df11_build_codebook([w])
    assert cb.n_luts <= ed.DF11_MAX_LUTS


def _greedy_codes(bits: str, table):
    """Codes decoded from the front of a bit string until one does not fit."""
    out, pos = [], 0
    while True:
        for l in range(1, len(bits) - pos + 1):
            s = table.get((l, bits[pos:pos + l]))
            if s is not None:
                out.append((pos, l, s))
                pos += l
                break
        else:
            return out


@pytest.mark.parametrize("which", ["cfg0", "one_exponent", "fibonacci", "uniform"])
def test_fast_tables_match_a_brute_force_decode(which, unit_tensors):
    if which == "cfg0":
        w = unit_tensors("0")[0]
    elif which == "one_exponent":
        w = (np.arange(5000, dtype=np.uint16) & np.uint16(0x807F)) | np.uint16(121 << 7)
        w[::50] = 0x3F80
    elif which == "fibonacci":
        w = _fib_unit()
    else:
        w = np.arange(1 << 16, dtype=np.uint16)
    cb = ed.df11_build_codebook([w])
    ocb = oracle.codebook([w])
    lens, codes = ed.codebook_arrays(cb)
    assert np.array_equal(lens, ocb.lens) or which == "fibonacci"
    table = {(int(l), format(int(codes[s]), f"0{int(l)}b")): s for s, l in enumerate(lens) if l}
    multi = np.ctypeslib.as_array(cb.multi)
    count = np.ctypeslib.as_array(cb.count)
    root = np.ctypeslib.as_array(cb.lut)[0]
    kM, kC = ed.DF11_MULTI_BITS, ed.DF11_COUNT_BITS
    n_long = 0
    for x in range(1 << kM):
        got = _greedy_codes(format(x, f"0{kM}b"), table)[:3]
        e = int(multi[x])
        assert e >> 30 == len(got), x
        if not got:
            # first code longer than the index: the entry names the level-1
            # table that the root entry for the top 8 bits points at
            r = int(root[x >> (kM - 8)])
            assert r & 0x8000 and e == r & 0x7FFF and e >= 1, x
            n_long += 1
            continue
        assert (e >> 24) & 0x3F == sum(l for _, l, _ in got), x
        for i, (_, _, s) in enumerate(got):
            assert (e >> (8 * i)) & 0xFF == s, x
        for i in range(len(got), 3):
            assert (e >> (8 * i)) & 0xFF == 0
    for x in range(1 << kC):
        got = _greedy_codes(format(x, f"0{kC}b"), table)
        e = int(count[x])
        assert e >> 12 == sum(l for _, l, _ in got), x
        if not got:
            r = int(root[x >> (kC - 8)])
            assert r & 0x8000 and e == r & 0x7FFF and e >= 1, x
            continue
        assert e & 0xFFF == sum(1 << pos for pos, _, _ in got), x
    assert (n_long > 0) == (int(lens.max()) > kM)


# ------------------------------------------------------------------ FP8 units


def _fp8(w16, fmt, scale=20000.0):
    return sw.fp8_from_f32((w16.astype(np.uint32) << 16).view(np.float32) * np.float32(scale), fmt)


def _compare_fp8(tensors, fmt):
    """Library FP8 encoding vs the oracle, byte for byte."""
    of = fmt.split("_")[1]
    cb = ed.df11_build_codebook(tensors, fmt)
    hs = ed.df11_encode(cb, tensors, 64, 8, fmt)
    allb = np.concatenate([np.asarray(t, np.uint8).reshape(-1) for t in tensors])
    sym, sm = oracle.fp8_split(allb, of)
    ocb = oracle.codebook_symbols(sym)
    lens, codes = ed.codebook_arrays(cb)
    assert np.array_equal(lens, ocb.lens) and np.array_equal(codes[lens > 0], ocb.codes[lens > 0])
    stream, total = oracle.encode_symbols(sym, ocb)
    assert hs.total_bits == total and hs.format == ed.FORMATS[fmt]
    assert np.array_equal(hs.stream[:stream.size], stream) and not hs.stream[stream.size:].any()
    assert np.array_equal(hs.sm[:sm.size], sm) and not hs.sm[sm.size:].any()
    gaps, bop = oracle.aux_symbols(sym, ocb, 64, 8)
    assert np.array_equal(hs.gaps, gaps) and np.array_equal(hs.block_out_pos, bop)
    assert hs.max_tile_symbols == int(np.diff(bop.astype(np.int64)).max())
    return cb, hs


@pytest.mark.parametrize("fmt", ["fp8_e4m3", "fp8_e5m2"])
def test_fp8_units_match_oracle(fmt, unit_tensors):
    (w,) = unit_tensors("0")
    b = _fp8(w, fmt.split("_")[1])
    _compare_fp8([b], fmt)
    # odd-sized tensors: sign+mantissa bytes shared by two tensors, and pieces of
    # more than 4 Mi weights starting at odd indices
    rng = np.random.default_rng(21)
    big = rng.integers(0, 256, (1 << 22) + 5001, dtype=np.uint8) & np.uint8(0xC7) | np.uint8(0x30)
    _compare_fp8([b[:333_333], b[333_333:], big, b[:7]], fmt)


@pytest.mark.parametrize("fmt", ["fp8_e4m3", "fp8_e5m2"])
def test_fp8_every_byte_value(fmt):
    b = np.tile(np.arange(256, dtype=np.uint8), 50)
    np.random.default_rng(4).shuffle(b)
    _compare_fp8([b], fmt)


def test_fp8_argument_errors():
    b = np.arange(256, dtype=np.uint8)
    cb = ed.df11_build_codebook([b], "fp8_e4m3")
    with pytest.raises(ed.Df11Error) as e:
        ed.df11_encode(cb, [b], 256, 8, "fp8_e4m3")  # FP8 units use 64-window tiles
    assert e.value.status == ed.DF11_E_INVALID
    with pytest.raises(TypeError):
        ed.df11_build_codebook([b.astype(np.uint16)], "fp8_e4m3")
    with pytest.raises(ValueError):
        ed.df11_build_codebook([b], "fp8_e3m4")
    ptrs = (ed.ctypes.c_void_p * 1)(b.ctypes.data)
    numel = (ed.ctypes.c_uint64 * 1)(b.size)
    rc = ed.LIB.df11_build_codebook_fmt(7, ptrs, numel, 1, ed.ctypes.byref(ed.df11_codebook()))
    assert rc == ed.DF11_E_INVALID


def test_gemm_order_is_the_documented_permutation():
    # out[(((m * cols/32 + kb) * 4 + q) * 16 + i) * 8 + e] = w[(16 m + i) * cols + 32 kb + 8 q + e]
    rows, cols = 48, 96
    w = np.arange(rows * cols, dtype=np.uint32).astype(np.uint16)
    out = ed.df11_gemm_order(w, rows, cols)
    for m, kb, q, i, e in [(0, 0, 0, 0, 0), (0, 0, 0, 1, 0), (0, 0, 1, 0, 0), (0, 1, 0, 0, 0),
                           (1, 0, 3, 0, 7), (2, 2, 3, 15, 7), (1, 2, 2, 9, 3)]:
        assert (out[(((m * (cols // 32) + kb) * 4 + q) * 16 + i) * 8 + e]
                == w[(16 * m + i) * cols + 32 * kb + 8 * q + e])
    # the same permutation by array reshapes
    ref = w.reshape(rows // 16, 16, cols // 32, 4, 8).transpose(0, 2, 3, 1, 4).reshape(-1)
    assert np.array_equal(out, ref)
    with pytest.raises(ed.Df11Error):
        ed.df11_gemm_order(w[:40 * cols], 40, cols)  # rows not a multiple of 16
    with pytest.raises(ed.Df11Error):
        ed.df11_gemm_order(w[:48 * 80], 48, 80)  # cols not a multiple of 32


def test_fused_workspace_sizes():
    """Host-only size queries of the fused entry points (no device call)."""
    shapes = [(64, 1024), (32, 4096)]
    lay = ed.gemm_layout(shapes, 48)
    assert ed.df11_decompress_gemm_scratch_bytes(lay, 48) == 2 * 48 * (1024 + 4096)
    assert ed.LIB.df11_decompress_gemm_scratch_bytes(None, 0, 16) == 0
    # 12288 and 8224 columns against the narrowest 4096: three K segments
    # each, whose float32 partial sums follow the activations
    lay = ed.gemm_layout([(16, 4096), (32, 12288), (48, 8224)], 16)
    assert ed.df11_decompress_gemm_scratch_bytes(lay, 16) == (
        2 * 16 * (4096 + 12288 + 8224) + 4 * 3 * 16 * (32 + 48))
    # the narrowest counts as 4096 at least: 1024 is not split, 8192 has two
    # segments, 12288 three
    lay = ed.gemm_layout([(16, 1024), (16, 8192), (16, 12288)], 32)
    assert ed.df11_decompress_gemm_scratch_bytes(lay, 32) == (
        2 * 32 * (1024 + 8192 + 12288) + 4 * (2 + 3) * 32 * 16)
    rng = np.random.default_rng(3)
    w = (rng.standard_normal(64 * 1024).astype(np.float32).view(np.uint32) >> 16).astype(np.uint16)
    cb = ed.df11_build_codebook([w])
    hs = ed.df11_encode(cb, [w], 64, 8)
    desc = ed.df11_device_stream()
    desc.n_tiles = hs.n_tiles
    # four row sums and a first-row index per tile, plus alignment slack
    assert ed.LIB.df11_decompress_gemv_scratch_bytes(ed.ctypes.byref(desc)) == hs.n_tiles * 20 + 256
    assert ed.LIB.df11_decompress_gemv_scratch_bytes(None) == 0


def test_random_units_match_oracle_property():
    """Generated units (sizes, tensor splits, value spreads, raw bit patterns,
    few-exponent data, tile sizes): the library's codebook, stream and
    auxiliary arrays equal the oracle's byte for byte."""
    from hypothesis import HealthCheck, given, settings
    from hypothesis import strategies as st

    @settings(max_examples=60, deadline=None, derandomize=True,
              suppress_health_check=[HealthCheck.too_slow])
    @given(data=st.data())
    def check(data):
        rng = np.random.default_rng(data.draw(st.integers(0, 2 ** 32 - 1), label="seed"))
        mode = data.draw(st.sampled_from(["gauss", "bits", "few"]), label="mode")
        tensors = []
        for _ in range(data.draw(st.integers(1, 4), label="tensors")):
            n = data.draw(st.integers(0, 6000), label="numel")
            if mode == "gauss":
                sigma = data.draw(st.sampled_from([1e-3, 0.02, 1.0, 300.0]), label="sigma")
                v = (rng.standard_normal(n) * sigma).astype(np.float32)
                t = ((v.view(np.uint32) + 0x7FFF + ((v.view(np.uint32) >> 16) & 1)) >> 16).astype(np.uint16)
            elif mode == "bits":
                t = rng.integers(0, 1 << 16, n, dtype=np.uint32).astype(np.uint16)
            else:
                exps = rng.choice(256, size=int(rng.integers(1, 4)), replace=False)
                t = ((rng.choice(exps, n).astype(np.uint32) << 7)
                     | rng.integers(0, 128, n).astype(np.uint32)
                     | (rng.integers(0, 2, n).astype(np.uint32) << 15)).astype(np.uint16)
            tensors.append(t)
        if sum(t.size for t in tensors) == 0:
            tensors.append(np.array([0x3F80], dtype=np.uint16))
        _compare(tensors, data.draw(st.sampled_from([64, 256, 512]), label="tile windows"), 8)

    check()


# ------------------------------------------------- tensor ranges from histograms


def _oracle_ranges(tensors, lens, tile_bits, fmt):
    """Element offsets and tile ranges from the oracle's code start bits."""
    offs = [0]
    tiles = []
    bit = 0
    for t in tensors:
        t = np.asarray(t).reshape(-1)
        if fmt == "bf16":
            sym = oracle.exponents(t)
        else:
            sym = oracle.fp8_split(t, fmt.split("_")[1])[0]
        ln = lens[sym].astype(np.int64)
        if t.size:
            last_start = bit + int(ln.sum()) - int(ln[-1])
            tiles += [bit // tile_bits, last_start // tile_bits + 1]
        else:
            tiles += [bit // tile_bits, bit // tile_bits]
        bit += int(ln.sum())
        offs.append(offs[-1] + t.size)
    return offs, tiles


@pytest.mark.parametrize("seed", range(6))
def test_tensor_ranges_from_counts_match_the_oracle(seed):
    rng = np.random.default_rng(700 + seed)
    fmt = ["bf16", "bf16", "fp8_e4m3", "bf16", "fp8_e5m2", "bf16"][seed]
    tw = 64 if fmt != "bf16" else int(rng.choice([64, 256, 512]))
    tensors = []
    for _ in range(int(rng.integers(1, 7))):
        n = int(rng.choice([0, 1, 7, 4095, 4096, int(rng.integers(1, 90_000))]))
        w = ((rng.standard_normal(n).astype(np.float32) * float(rng.choice([0.02, 3.0])))
             .view(np.uint32) >> 16).astype(np.uint16)
        tensors.append(w if fmt == "bf16" else _fp8(w, fmt.split("_")[1]))
    if not any(np.asarray(t).size for t in tensors):  # a codebook needs one weight
        tensors.append(np.full(3, 0x3C00, np.uint16) if fmt == "bf16" else np.full(3, 0x38, np.uint8))
    cb = ed.df11_build_codebook(tensors, fmt)
    hs = ed.df11_encode(cb, tensors, tw, 8, fmt)
    if fmt == "bf16":
        counts = [oracle.histogram(t) for t in tensors]
    else:
        counts = [oracle.histogram_symbols(oracle.fp8_split(t, fmt.split("_")[1])[0]) for t in tensors]
    last = [int(np.asarray(t).reshape(-1)[-1]) if np.asarray(t).size else 0 for t in tensors]
    offs, tiles = ed.df11_tensor_ranges_from_counts(cb, np.array(counts), last, fmt, tw, 8)
    lens = ed.codebook_arrays(cb)[0]
    o_offs, o_tiles = _oracle_ranges(tensors, lens, 64 * tw, fmt)
    assert offs.tolist() == o_offs and tiles.tolist() == o_tiles
    assert np.array_equal(offs, hs.tensor_offsets) and np.array_equal(tiles, hs.tensor_tiles)


def test_tensor_ranges_from_counts_errors():
    w = np.arange(0x3C00, 0x3C40, dtype=np.uint16)
    cb = ed.df11_build_codebook([w])
    c = oracle.histogram(w)
    with pytest.raises(ed.Df11Error) as e:  # the last weight's symbol is not counted
        ed.df11_tensor_ranges_from_counts(cb, c[None, :], [0x7F80])
    assert e.value.status == ed.DF11_E_INVALID
    bad = c.copy()
    bad[200] = 5  # a symbol without a code
    with pytest.raises(ed.Df11Error) as e:
        ed.df11_tensor_ranges_from_counts(cb, bad[None, :], [int(w[-1])])
    assert e.value.status == ed.DF11_E_SYMBOL
    with pytest.raises(ed.Df11Error):
        ed.df11_tensor_ranges_from_counts(cb, c[None, :], [int(w[-1])], "bf16", 100, 8)
    offs, tiles = ed.df11_tensor_ranges_from_counts(cb, np.zeros((0, 256), np.uint64), [])
    assert offs.tolist() == [0] and tiles.size == 0
