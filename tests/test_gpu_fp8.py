"""GPU parity for FP8 units (E4M3 and E5M2): the HIP decoder against the
oracle's bit-serial decode and against the original bytes."""

import numpy as np
import pytest

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")

import entropy_decoding_amd as ed  # noqa: E402
import oracle  # noqa: E402
import synth_weights as sw  # noqa: E402

FMTS = ["fp8_e4m3", "fp8_e5m2"]


def say(msg):
    print(msg, flush=True)


@pytest.fixture(scope="module", autouse=True)
def _device():
    assert torch.cuda.is_available(), "GPU tests need a ROCm device"
    torch.cuda.init()
    yield
    torch.cuda.synchronize()


def _fp8(w16, fmt, scale=20000.0):
    return sw.fp8_from_f32((w16.astype(np.uint32) << 16).view(np.float32) * np.float32(scale),
                           fmt.split("_")[1])


class Unit:
    def __init__(self, tensors, fmt):
        self.tensors = [np.asarray(t, dtype=np.uint8).reshape(-1) for t in tensors]
        self.fmt = fmt
        self.cb = ed.df11_build_codebook(self.tensors, fmt)
        self.hs = ed.df11_encode(self.cb, self.tensors, 64, 8, fmt)
        self.ds = ed.DeviceStream(self.hs, self.cb, "cuda")
        self.n = self.hs.n_weights

    def decompress(self, poison=0xA5, label=""):
        out = torch.full((max(self.n, 1),), poison, dtype=torch.uint8, device="cuda")
        status = torch.zeros(1, dtype=torch.int32, device="cuda")
        say(f"[gpu] df11_decompress_block {self.fmt} {label} N={self.n} tiles={self.hs.n_tiles}")
        ed.df11_decompress_block(self.ds, out, status)
        torch.cuda.synchronize()
        return out[: self.n], int(status.item())

    def original(self):
        return np.concatenate(self.tensors) if self.tensors else np.zeros(0, np.uint8)


def check_identity(u, label, poisons=(0xA5, 0x5A)):
    ref = torch.from_numpy(u.original()).cuda()
    for p in poisons:
        out, st = u.decompress(p, label)
        assert st == 0
        assert torch.equal(out, ref), f"{label}: mismatches={int((out != ref).sum())}"
    return out


@pytest.mark.parametrize("fmt", FMTS)
def test_fp8_phase1_window_counts(fmt, unit_tensors):
    """The first decode phase, window by window, against the oracle's count of
    code starts on the FP8 exponent symbols."""
    (w,) = unit_tensors("0")
    b = _fp8(w, fmt)
    sym, _ = oracle.fp8_split(b, fmt.split("_")[1])
    lens = oracle.code_lengths(oracle.histogram_symbols(sym))
    u = Unit([b], fmt)
    n = int(u.hs.n_tiles) * 64
    c = torch.full((n,), -1, dtype=torch.int32, device="cuda")
    say(f"[gpu] df11_window_counts {fmt} cfg0 windows={n}")
    ed.df11_window_counts(u.ds, c)
    torch.cuda.synchronize()
    assert np.array_equal(c.cpu().numpy().view(np.uint32), oracle.window_counts(sym, lens, n))


@pytest.mark.parametrize("fmt", FMTS)
def test_fp8_config0_every_output_equals_the_oracle(fmt, unit_tensors):
    (w,) = unit_tensors("0")
    b = _fp8(w, fmt)
    of = fmt.split("_")[1]
    sym, sm = oracle.fp8_split(b, of)
    ocb = oracle.codebook_symbols(sym)
    stream, total = oracle.encode_symbols(sym, ocb)
    odec = oracle.fp8_merge(oracle.decode_symbols(stream, 0, total, ocb.lens, sym.size), sm, of)
    u = Unit([b], fmt)
    assert u.hs.n_tiles > 1 and u.hs.total_bits % (64 * 64) != 0
    out, st = u.decompress(0xA5, "cfg0")
    assert st == 0
    got = out.cpu().numpy()
    assert np.array_equal(got, odec) and np.array_equal(got, b)


@pytest.mark.parametrize("fmt", FMTS)
def test_fp8_every_byte_value_and_ragged_sizes(fmt):
    b = np.tile(np.arange(256, dtype=np.uint8), 300)
    np.random.default_rng(5).shuffle(b)
    check_identity(Unit([b], fmt), "all bytes")
    for n in (1, 2, 15, 16, 17, 4097, 70001):
        check_identity(Unit([b[:n]], fmt), f"n={n}", poisons=(0xA5,))


@pytest.mark.parametrize("seed", range(6))
def test_fp8_random_multi_tensor_units(seed):
    fmt = FMTS[seed % 2]
    rng = np.random.default_rng(2000 + seed)
    tensors = []
    for _ in range(int(rng.integers(1, 6))):
        n = int(rng.integers(0, 150_000))
        if seed % 3 == 0:
            n = n // 16 * 16
        z = (rng.standard_normal(n).astype(np.float32) * float(rng.choice([0.02, 1.0])))
        tensors.append(sw.fp8_from_f32(z * np.float32(100.0), fmt.split("_")[1]))
    if sum(t.size for t in tensors) == 0:
        tensors.append(np.array([0x38], dtype=np.uint8))
    u = Unit(tensors, fmt)
    check_identity(u, f"random seed={seed}")
    offs = u.hs.tensor_offsets
    for k, t in enumerate(tensors):
        out = torch.full((max(1, t.size),), 0xA5, dtype=torch.uint8, device="cuda")
        if offs[k] % 16:
            with pytest.raises(ed.Df11Error) as e:
                ed.df11_decompress_tensor(u.ds, k, out)
            assert e.value.status == ed.DF11_E_INVALID
            continue
        st = torch.zeros(1, dtype=torch.int32, device="cuda")
        say(f"[gpu] df11_decompress_tensor {fmt} seed={seed} k={k} numel={t.size}")
        ed.df11_decompress_tensor(u.ds, k, out, st)
        torch.cuda.synchronize()
        assert int(st.item()) == 0
        assert np.array_equal(out[: t.size].cpu().numpy(), t)


def test_fp8_corrupt_block_out_pos_is_reported_and_tiles_left_unwritten(unit_tensors):
    (w,) = unit_tensors("0")
    b = _fp8(w, "fp8_e4m3")
    u = Unit([b], "fp8_e4m3")
    bop = u.hs.block_out_pos.copy()
    bad = bop.copy()
    bad[9] += 1  # tiles 8 and 9 now disagree with their decoded counts
    u.ds.block_out_pos.copy_(torch.from_numpy(bad.view(np.uint8)))
    out, st = u.decompress(0xA5, "corrupt bop")
    assert st == ed.DF11_E_CORRUPT
    got = out.cpu().numpy()
    # tiles 8, 9 wrote nothing (away from the chunks they share with 7 and 10);
    # every other tile is exact
    lo, hi = int(bad[8]), int(bad[10])
    assert (got[lo + 16:hi - 16] == 0xA5).all()
    assert np.array_equal(got[: int(bop[8])], b[: int(bop[8])])
    assert np.array_equal(got[int(bop[10]):], b[int(bop[10]):])


@pytest.mark.parametrize("fmt", FMTS)
def test_fp8_long_tiles_take_the_general_store_path(fmt):
    # Nearly every weight shares one exponent: codes of about one bit, so a
    # 64-window tile holds up to ~4000 outputs, more than the two prefetched
    # chunk slots of the fixed-store kernel cover (2033); the library then
    # uses the kernel with the general store loop.  Short-code and ordinary
    # units must both come back bit-exact.
    rng = np.random.default_rng(77)
    n = 300_000
    b = np.full(n, 0x38 if fmt == "fp8_e4m3" else 0x3C, dtype=np.uint8)
    b ^= rng.integers(0, 2, n, dtype=np.uint8) << 7  # random signs
    b[rng.integers(0, n, 300)] = rng.integers(0, 256, 300, dtype=np.uint8)
    u = Unit([b], fmt)
    assert u.hs.max_tile_symbols > 2033
    check_identity(u, "long tiles")
    z = sw.fp8_from_f32(rng.standard_normal(n).astype(np.float32) * 100.0, fmt.split("_")[1])
    v = Unit([z], fmt)
    assert v.hs.max_tile_symbols <= 2033
    check_identity(v, "ordinary tiles")


def test_fp8_e5m2_long_codes_walk_four_table_levels():
    # Fibonacci counts over the 32 E5M2 exponent values give the most skewed
    # code, 31 bits long at the deepest, resolved through four table levels
    f = [1, 1]
    while len(f) < 32:
        f.append(f[-1] + f[-2])
    rng = np.random.default_rng(31)
    e = np.repeat(np.arange(32, dtype=np.uint8), f)
    rng.shuffle(e)
    b = ((e << 2) | rng.integers(0, 4, e.size, dtype=np.uint8)
         | (rng.integers(0, 2, e.size, dtype=np.uint8) << 7)).astype(np.uint8)
    u = Unit([b], "fp8_e5m2")
    assert u.cb.max_len == 31 and u.cb.n_luts == 4
    check_identity(u, "31-bit codes")


def test_fp8_requires_64_window_tiles_and_8_bit_outputs(unit_tensors):
    (w,) = unit_tensors("0")
    u = Unit([_fp8(w, "fp8_e5m2")], "fp8_e5m2")
    with pytest.raises(ValueError):
        ed.df11_decompress_block(u.ds, torch.empty(u.n, dtype=torch.int16, device="cuda"))
    u.ds.desc.tile_windows = 256  # FP8 units decode with 64-window tiles only
    rc = ed.LIB.df11_decompress_block(ed.ctypes.byref(u.ds.desc), None, None, None)
    assert rc == ed.DF11_E_INVALID


@pytest.mark.parametrize("fmt", FMTS)
def test_fp8_70b_block_full_size(fmt):
    tensors = sw.gen_unit_fp8(sw.config("2").units[0], fmt.split("_")[1])
    u = Unit(tensors, fmt)
    out = check_identity(u, "70B block", poisons=(0xA5,))
    host = out.cpu().numpy()
    lens, _ = ed.codebook_arrays(u.cb)
    of = fmt.split("_")[1]
    rng = np.random.default_rng(0)
    nt = int(u.hs.n_tiles)
    for t in sorted(set([0, nt - 1, *rng.integers(0, nt, 12).tolist()])):
        g = u.hs.gaps[t * 64:(t + 1) * 64]
        j = int(np.argmax(g != 255))
        p0, p1 = int(u.hs.block_out_pos[t]), int(u.hs.block_out_pos[t + 1])
        syms = oracle.decode_symbols(u.hs.stream, (t * 64 + j) * 64 + int(g[j]), u.hs.total_bits,
                                     lens, p1 - p0)
        # the tile's sign+mantissa nibbles, repacked to start at weight p0
        packed = u.hs.sm[p0 // 2:(p1 + 1) // 2 + 1]
        nib = np.stack([packed & 0xF, packed >> 4], axis=1).reshape(-1)[p0 % 2:p0 % 2 + p1 - p0]
        nib = np.r_[nib, np.zeros(nib.size % 2, np.uint8)]
        sm = (nib[0::2] | (nib[1::2] << 4)).astype(np.uint8)
        assert np.array_equal(host[p0:p1], oracle.fp8_merge(syms, sm, of)), t
