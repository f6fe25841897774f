"""GPU parity: the HIP decoder against the oracle and against the original bits.

Every comparison is on 16-bit patterns (int16 views), never on float values.
Small cases compare every output with the oracle's bit-serial decode; the full
workloads compare every output with the original tensor (the method is
lossless: decompressed == original, bit for bit) and sampled tiles with the
oracle's decode of those tiles.
"""

import numpy as np
import pytest

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")

import entropy_decoding_amd as ed  # noqa: E402
import oracle  # noqa: E402
import synth_weights as sw  # noqa: E402

B = 8  # window bytes


def say(msg):
    print(msg, flush=True)


@pytest.fixture(scope="module", autouse=True)
def _device():
    assert torch.cuda.is_available(), "GPU tests need a ROCm device"
    torch.cuda.init()
    yield
    torch.cuda.synchronize()


def _cat(tensors):
    return np.concatenate([np.asarray(t, dtype=np.uint16).reshape(-1) for t in tensors])


def _dev_i16(a):
    return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).cuda()


class Unit:
    """Library-compressed unit resident on the GPU."""

    def __init__(self, tensors, tw=ed.DEFAULT_TILE_WINDOWS):
        self.tensors = [np.asarray(t, dtype=np.uint16).reshape(-1) for t in tensors]
        self.cb = ed.df11_build_codebook(self.tensors)
        self.hs = ed.df11_encode(self.cb, self.tensors, tw, B)
        self.ds = ed.DeviceStream(self.hs, self.cb, "cuda")
        self.n = self.hs.n_weights
        self.tw = tw

    def decompress(self, poison=-1, label=""):
        out = torch.full((max(self.n, 1),), poison, dtype=torch.int16, device="cuda")
        status = torch.zeros(1, dtype=torch.int32, device="cuda")
        say(f"[gpu] df11_decompress_block {label} N={self.n} tiles={self.hs.n_tiles} "
            f"T={self.tw} luts={self.cb.n_luts} max_len={self.cb.max_len}")
        ed.df11_decompress_block(self.ds, out, status)
        torch.cuda.synchronize()
        return out[: self.n], int(status.item())

    def decompress_tensor(self, k, poison=-1, label=""):
        nk = self.tensors[k].size
        out = torch.full((max(nk, 1),), poison, dtype=torch.int16, device="cuda")
        status = torch.zeros(1, dtype=torch.int32, device="cuda")
        say(f"[gpu] df11_decompress_tensor {label} k={k} numel={nk}")
        ed.df11_decompress_tensor(self.ds, k, out, status)
        torch.cuda.synchronize()
        return out[:nk], int(status.item())

    def tile_start_bit(self, t):
        g = self.hs.gaps[t * self.tw:(t + 1) * self.tw]
        j = int(np.argmax(g != 255))
        assert g[j] != 255
        return (t * self.tw + j) * 8 * B + int(g[j])

    def oracle_tile(self, t):
        """The oracle's bit-serial decode of tile t of the library's stream."""
        lens, _ = ed.codebook_arrays(self.cb)
        p0, p1 = int(self.hs.block_out_pos[t]), int(self.hs.block_out_pos[t + 1])
        if p1 == p0:
            return p0, np.zeros(0, np.uint16)
        return p0, oracle.decode(self.hs.stream, self.tile_start_bit(t), self.hs.total_bits, lens,
                                 self.hs.sm[p0:p1], p1 - p0)


def check_identity(u, label, poisons=(-1, 0)):
    ref = _dev_i16(_cat(u.tensors))
    for p in poisons:
        out, st = u.decompress(p, label)
        assert st == 0
        assert torch.equal(out, ref), f"{label}: mismatches={int((out != ref).sum())}"
    return out


def check_sampled_tiles(u, out, n_samples=24, seed=0):
    rng = np.random.default_rng(seed)
    nt = int(u.hs.n_tiles)
    tiles = sorted(set([0, nt - 1, nt // 2, *rng.integers(0, nt, size=n_samples).tolist()]))
    host = out.cpu().numpy().view(np.uint16)
    for t in tiles:
        p0, dec = u.oracle_tile(t)
        assert np.array_equal(host[p0:p0 + dec.size], dec), t


# ------------------------------------------------------------------ small, exhaustive


@pytest.mark.parametrize("tw", [64, 256, 512])
def test_config0_every_output_equals_the_oracle(tw, unit_tensors):
    (w,) = unit_tensors("0")
    ocb = oracle.codebook(w)
    enc = oracle.encode(w, ocb)
    odec = oracle.decode(enc.stream, 0, enc.total_bits, ocb.lens, enc.sm)
    u = Unit([w], tw)
    assert u.hs.n_tiles > 1 and u.hs.total_bits % (8 * B * tw) != 0  # ragged last tile
    out, st = u.decompress(-1, f"cfg0 T={tw}")
    assert st == 0
    got = out.cpu().numpy().view(np.uint16)
    assert np.array_equal(got, odec)
    assert np.array_equal(got, w)


@pytest.mark.parametrize("seed", range(12))
def test_random_multi_tensor_units(seed):
    rng = np.random.default_rng(1000 + seed)
    ntens = int(rng.integers(1, 6))
    tensors = []
    for _ in range(ntens):
        n = int(rng.integers(0, 200_000)) // 8 * 8 if seed % 2 else int(rng.integers(0, 200_000))
        sigma = float(rng.choice([0.02, 0.002, 1.0]))
        z = (rng.standard_normal(n).astype(np.float32) * sigma).view(np.uint32) >> 16
        tensors.append(z.astype(np.uint16))
    if sum(t.size for t in tensors) == 0:
        tensors.append(np.array([0x3F80], dtype=np.uint16))
    u = Unit(tensors, (64, 256, 512)[seed % 3])
    out = check_identity(u, f"random seed={seed}")
    check_sampled_tiles(u, out, 8, seed)
    check_window_counts(u, oracle.exponents(_cat(tensors)), f"random seed={seed}")
    offs = u.hs.tensor_offsets
    for k in range(len(tensors)):
        if offs[k] % 8:
            with pytest.raises(ed.Df11Error) as e:
                ed.df11_decompress_tensor(u.ds, k, torch.empty(max(1, tensors[k].size),
                                                              dtype=torch.int16, device="cuda"))
            assert e.value.status == ed.DF11_E_INVALID
            continue
        got, st = u.decompress_tensor(k, -1, f"random seed={seed}")
        assert st == 0 and torch.equal(got, _dev_i16(tensors[k]))


@pytest.mark.parametrize("n", [1, 2, 7, 8, 9, 2047, 2048 * 8 + 3])
def test_tiny_and_ragged_sizes(n):
    rng = np.random.default_rng(n)
    w = ((rng.standard_normal(n).astype(np.float32) * 0.02).view(np.uint32) >> 16).astype(np.uint16)
    u = Unit([w])
    check_identity(u, f"n={n}")
    check_window_counts(u, oracle.exponents(w), f"n={n}")


def test_single_exponent_one_bit_codes():
    # every code is 1 bit: 64 symbols per window, the staging buffer's worst case
    w = (np.arange(300_000, dtype=np.uint32) * 2654435761 % 65536).astype(np.uint16)
    w = (w & np.uint16(0x807F)) | np.uint16(121 << 7)
    u = Unit([w])
    assert u.hs.max_tile_symbols == 8 * B * u.tw
    check_identity(u, "single exponent")


def test_every_bit_pattern_including_nan_inf_subnormal():
    w = np.tile(np.arange(1 << 16, dtype=np.uint16), 3)
    np.random.default_rng(7).shuffle(w)
    check_identity(Unit([w]), "all bit patterns")


def test_special_values():
    specials = np.array([0x0000, 0x8000, 0x7F80, 0xFF80, 0x7FC0, 0xFFC1, 0x7F81, 0x0001, 0x807F,
                         0x0080, 0x3F80, 0xBF80], dtype=np.uint16)
    rng = np.random.default_rng(8)
    w = ((rng.standard_normal(100_000).astype(np.float32) * 0.02).view(np.uint32) >> 16)
    w = w.astype(np.uint16)
    w[rng.integers(0, w.size, 5000)] = rng.choice(specials, 5000)
    check_identity(Unit([w]), "specials")


def test_32_bit_codes_walk_four_table_levels():
    f = [1, 1]
    while len(f) < 36:
        f.append(f[-1] + f[-2])
    sym = np.repeat(np.arange(36, dtype=np.uint16) + 90, f)
    np.random.default_rng(9).shuffle(sym)
    w = ((sym << 7) | (np.arange(sym.size) & 0x807F)).astype(np.uint16)
    u = Unit([w])
    assert u.cb.max_len == 32
    out = check_identity(u, "fibonacci 32-bit codes")
    check_sampled_tiles(u, out, 8)


# ------------------------------------------------------------------ phase 1 alone


def check_window_counts(u, sym, label):
    """df11_window_counts (the decode's first phase, window by window) against
    the oracle's count of code starts per window, with the oracle's lengths."""
    ocb_lens = oracle.code_lengths(oracle.histogram_symbols(sym))
    lens, _ = ed.codebook_arrays(u.cb)
    assert np.array_equal(np.asarray(lens), ocb_lens)
    n = int(u.hs.n_tiles) * u.tw
    c = torch.full((n,), -1, dtype=torch.int32, device="cuda")
    say(f"[gpu] df11_window_counts {label} windows={n}")
    ed.df11_window_counts(u.ds, c)
    torch.cuda.synchronize()
    ref = oracle.window_counts(sym, ocb_lens, n)
    got = c.cpu().numpy().view(np.uint32)
    assert np.array_equal(got, ref), np.flatnonzero(got != ref)[:10]


@pytest.mark.parametrize("tw", [64, 256, 512])
def test_phase1_window_counts_config0(tw, unit_tensors):
    (w,) = unit_tensors("0")
    check_window_counts(Unit([w], tw), oracle.exponents(w), f"cfg0 T={tw}")


def test_phase1_window_counts_32_bit_codes_and_one_bit_codes():
    f = [1, 1]
    while len(f) < 36:
        f.append(f[-1] + f[-2])
    sym = np.repeat(np.arange(36, dtype=np.uint16) + 90, f)
    np.random.default_rng(9).shuffle(sym)
    w = ((sym << 7) | (np.arange(sym.size) & 0x807F)).astype(np.uint16)
    u = Unit([w])
    assert u.cb.max_len == 32
    check_window_counts(u, oracle.exponents(w), "fibonacci 32-bit codes")
    w1 = np.full(100003, 0x3F80, dtype=np.uint16)  # one exponent: one-bit codes
    check_window_counts(Unit([w1]), oracle.exponents(w1), "single exponent")


def test_phase1_window_counts_8b_block_full_size():
    tensors = sw.gen_unit(sw.config("1").units[0])
    u = Unit(tensors)
    check_window_counts(u, oracle.exponents(_cat(tensors)), "cfg1 block")


def _corrupt_level_tables(u):
    """Replace the unit's device tables by an image whose hierarchical tables
    1.. hold only pointers back to table 1, so that no code longer than the
    fast tables' index reaches a leaf."""
    bad = ed.df11_codebook.from_buffer_copy(u.cb)
    for k in range(1, int(bad.n_luts)):
        for b in range(256):
            bad.lut[k][b] = 0x8001
    u.ds.tables.copy_(torch.from_numpy(ed.table_image(bad)))


def test_phase1_flags_windows_whose_codes_reach_no_leaf(unit_tensors):
    """A code that the tables cannot resolve adds 2^20 to its window's count:
    exactly the windows where a code longer than the 12-bit count table starts
    are flagged, the others keep the oracle's counts, and a flagged window's
    low bits count the codes before its first long one."""
    (w,) = unit_tensors("0")
    u = Unit([w])
    assert u.cb.n_luts > 1 and u.cb.max_len > ed.DF11_COUNT_BITS
    _corrupt_level_tables(u)
    n = int(u.hs.n_tiles) * u.tw
    c = torch.full((n,), -1, dtype=torch.int32, device="cuda")
    say(f"[gpu] df11_window_counts with unresolvable long codes windows={n}")
    ed.df11_window_counts(u.ds, c)
    torch.cuda.synchronize()
    got = c.cpu().numpy().view(np.uint32)
    sym = oracle.exponents(w)
    lens = oracle.code_lengths(oracle.histogram_symbols(sym))
    ln = lens[sym].astype(np.int64)
    win = (np.cumsum(ln) - ln) // 64  # window of every code start
    ref = np.bincount(win, minlength=n).astype(np.uint32)
    longw = np.unique(win[ln > ed.DF11_COUNT_BITS])
    flagged = np.flatnonzero(got >= (1 << 20))
    assert longw.size > 0 and np.array_equal(flagged, longw)
    ok = np.setdiff1d(np.arange(n), longw)
    assert np.array_equal(got[ok], ref[ok])
    first_code = np.searchsorted(win, longw)
    first_long = np.array([int(np.flatnonzero((win == j) & (ln > ed.DF11_COUNT_BITS))[0]) for j in longw])
    assert np.array_equal(got[longw] - (1 << 20), first_long - first_code)


def test_unresolvable_codes_are_reported_by_the_decoder(unit_tensors):
    """The same tables in a decompression: the flagged tiles fail their count
    check (DF11_E_CORRUPT) and write nothing; tiles without codes longer than
    the 10-bit multi-symbol index never use those tables and stay exact."""
    (w,) = unit_tensors("0")
    u = Unit([w])
    _corrupt_level_tables(u)
    out, st = u.decompress(-1, "unresolvable long codes")
    assert st == ed.DF11_E_CORRUPT
    got = out.cpu().numpy().view(np.uint16)
    sym = oracle.exponents(w)
    lens = oracle.code_lengths(oracle.histogram_symbols(sym))
    ln = lens[sym].astype(np.int64)
    tile = (np.cumsum(ln) - ln) // (64 * u.tw)
    bop = u.hs.block_out_pos.astype(np.int64)
    long_tiles = set(np.unique(tile[ln > ed.DF11_MULTI_BITS]).tolist())
    clean = [t for t in range(int(u.hs.n_tiles)) if t not in long_tiles]
    assert len(clean) > 0
    for t in clean:  # a tile writes only its own outputs [bop[t], bop[t+1])
        assert np.array_equal(got[bop[t]:bop[t + 1]], w[bop[t]:bop[t + 1]]), t


# ------------------------------------------------------------------ failure paths


def test_corrupt_block_out_pos_is_reported_and_tiles_left_unwritten(unit_tensors):
    (w,) = unit_tensors("0")
    u = Unit([w])
    bop = u.hs.block_out_pos.copy()
    bad = bop.copy()
    bad[5] += 1  # tiles 4 and 5 now disagree with their decoded counts
    u.ds.block_out_pos.copy_(torch.from_numpy(bad.view(np.uint8)))
    out, st = u.decompress(-1, "corrupt bop")
    assert st == ed.DF11_E_CORRUPT
    got = out.cpu().numpy().view(np.uint16)
    # tiles 4, 5 wrote nothing; every other tile is exact
    lo, hi = int(bad[4]), int(bad[6])
    assert (got[lo + 8:hi - 8] == 0xFFFF).all()
    assert np.array_equal(got[: int(bop[4])], w[: int(bop[4])])
    assert np.array_equal(got[int(bop[6]):], w[int(bop[6]):])


def test_corrupt_gap_is_reported(unit_tensors):
    (w,) = unit_tensors("0")
    u = Unit([w])
    gaps = u.hs.gaps.copy()
    gaps[3 * u.tw + 17] = 255  # a window whose codes are now skipped
    u.ds.gaps.copy_(torch.from_numpy(gaps))
    _, st = u.decompress(-1, "corrupt gap")
    assert st == ed.DF11_E_CORRUPT


def test_invalid_arguments_are_rejected_before_launch(unit_tensors):
    (w,) = unit_tensors("0")
    u = Unit([w])
    buf = torch.empty(u.n + 8, dtype=torch.int16, device="cuda")
    with pytest.raises(ed.Df11Error) as e:
        ed.df11_decompress_block(u.ds, buf[1:])  # 2-byte aligned only
    assert e.value.status == ed.DF11_E_INVALID
    d = u.ds.desc
    saved = d.n_tiles
    d.n_tiles = saved + 1
    with pytest.raises(ed.Df11Error):
        ed.df11_decompress_block(u.ds, buf)
    d.n_tiles = saved
    with pytest.raises(ed.Df11Error):
        ed.df11_decompress_tensor(u.ds, 1, buf)


def test_empty_unit_launches_nothing():
    d = ed.df11_device_stream()
    d.tile_windows, d.window_bytes = 512, 8
    rc = ed.LIB.df11_decompress_block(ed.ctypes.byref(d), None, None, None)
    assert rc == ed.DF11_OK


def test_launch_on_a_side_stream(unit_tensors):
    (w,) = unit_tensors("0")
    u = Unit([w])
    s = torch.cuda.Stream()
    out = torch.zeros(u.n, dtype=torch.int16, device="cuda")
    torch.cuda.synchronize()
    say("[gpu] df11_decompress_block on a side stream")
    with torch.cuda.stream(s):
        ed.df11_decompress_block(u.ds, out, stream=s)
    s.synchronize()
    assert torch.equal(out, _dev_i16(w))


def test_concurrent_launches_on_two_streams(unit_tensors):
    # the library holds no state between calls: two units decoded on two
    # streams at once, launches interleaved, each equal to its original
    (w0,) = unit_tensors("0")
    rng = np.random.default_rng(21)
    w1 = ((rng.standard_normal(700_001).astype(np.float32) * 0.05).view(np.uint32) >> 16).astype(np.uint16)
    units = [Unit([w0]), Unit([w1])]
    refs = [_dev_i16(w0), _dev_i16(w1)]
    streams = [torch.cuda.Stream(), torch.cuda.Stream()]
    outs = [[torch.zeros(u.n, dtype=torch.int16, device="cuda") for _ in range(4)] for u in units]
    status = [torch.zeros(1, dtype=torch.int32, device="cuda") for _ in units]
    torch.cuda.synchronize()
    say("[gpu] two units decoded concurrently on two streams")
    for i in range(4):
        for k in (0, 1):
            with torch.cuda.stream(streams[k]):
                ed.df11_decompress_block(units[k].ds, outs[k][i], status[k], stream=streams[k])
    torch.cuda.synchronize()
    for k in (0, 1):
        assert int(status[k].item()) == 0
        for i in range(4):
            assert torch.equal(outs[k][i], refs[k]), f"unit {k} launch {i}"


# ------------------------------------------------------------------ full workloads


@pytest.mark.parametrize("cfg", ["3a", "3b", "3c"])
def test_stress_config_full_size(cfg, unit_tensors):
    u = Unit(unit_tensors(cfg))
    out = check_identity(u, f"cfg{cfg}", poisons=(-1,))
    check_sampled_tiles(u, out)


@pytest.mark.parametrize("cfg,tw", [("1", 64), ("1", 256), ("2", 64), ("2tp8", 64), ("405tp8", 64)])
def test_block_config_full_size(cfg, tw):
    unit = sw.config(cfg).units[0]
    tensors = sw.gen_unit(unit)
    u = Unit(tensors, tw)
    out = check_identity(u, f"cfg{cfg} block T={tw}", poisons=(-1,))
    check_sampled_tiles(u, out, 16)
    del out
    for k in (0, 6):
        got, st = u.decompress_tensor(k, 0, f"cfg{cfg} T={tw}")
        assert st == 0 and torch.equal(got, _dev_i16(tensors[k]))


@pytest.mark.parametrize("group", range(6))
def test_full_model_units(group):
    """Config 4 (embedding, 32 blocks, lm_head), six units per test case."""
    cfg = sw.config("4")
    units = cfg.units[group * 6:(group + 1) * 6]
    for unit in units:
        tensors = sw.gen_unit(unit)
        u = Unit(tensors)
        check_identity(u, f"cfg4 {unit.name}", poisons=(-1,))
        del u
