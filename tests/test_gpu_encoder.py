"""GPU-side encoder: every array it writes must equal, byte for byte, what the
host encoder (itself checked against the oracle) writes for the same weights,
and the device-encoded unit must decompress to the original bits."""

import numpy as np
import pytest

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")

import entropy_decoding_amd as ed  # noqa: E402
import oracle  # noqa: E402
import synth_weights as sw  # noqa: E402


def say(msg):
    print(msg, flush=True)


@pytest.fixture(scope="module", autouse=True)
def _device():
    assert torch.cuda.is_available(), "GPU tests need a ROCm device"
    torch.cuda.init()
    yield
    torch.cuda.synchronize()


def _dev(a):
    a = np.ascontiguousarray(a)
    return torch.from_numpy(a.view(np.int16) if a.dtype == np.uint16 else a).cuda()


def check_against_host(tensors, fmt, tw, label, decode=True):
    say(f"[gpu] encode_on_device {fmt} T={tw} {label} sizes={[t.size for t in tensors][:8]}")
    ds, cb = ed.encode_on_device([_dev(t) for t in tensors], fmt, tw)
    hcb = ed.df11_build_codebook(tensors, fmt)
    hs = ed.df11_encode(hcb, tensors, tw, 8, fmt)
    assert np.array_equal(np.ctypeslib.as_array(cb.code_len), np.ctypeslib.as_array(hcb.code_len))
    d = ds.desc
    assert (d.n_weights, d.total_bits, d.n_tiles, d.max_tile_symbols, d.format) == \
        (hs.n_weights, hs.total_bits, hs.n_tiles, hs.max_tile_symbols, hs.format)
    assert np.array_equal(ds.stream.cpu().numpy(), hs.stream)
    assert np.array_equal(ds.sm.cpu().numpy(), hs.sm)
    assert np.array_equal(ds.gaps.cpu().numpy()[: hs.gaps.size], hs.gaps)
    assert np.array_equal(ds.block_out_pos.cpu().numpy().view(np.uint32), hs.block_out_pos)
    assert np.array_equal(ds.tensor_offsets, hs.tensor_offsets)
    assert np.array_equal(ds.tensor_tiles, hs.tensor_tiles)
    if decode:
        ref = np.concatenate([t.reshape(-1) for t in tensors])
        out = torch.empty(max(1, ref.size), dtype=torch.int16 if fmt == "bf16" else torch.uint8,
                          device="cuda")
        st = torch.zeros(1, dtype=torch.int32, device="cuda")
        ed.df11_decompress_block(ds, out, st)
        torch.cuda.synchronize()
        assert int(st.item()) == 0
        got = out[: ref.size].cpu().numpy()
        assert np.array_equal(got.view(np.uint16) if fmt == "bf16" else got, ref)
    return ds


def _bf16(rng, n, sigma=0.02):
    return ((rng.standard_normal(n).astype(np.float32) * sigma).view(np.uint32) >> 16).astype(np.uint16)


def test_device_histogram_equals_the_oracle(unit_tensors):
    (w,) = unit_tensors("0")
    c = ed.df11_histogram_device(_dev(w)).cpu().numpy().view(np.uint64)
    assert np.array_equal(c, oracle.histogram(w))
    b = np.arange(256, dtype=np.uint8).repeat(7)
    for fmt, of in (("fp8_e4m3", "e4m3"), ("fp8_e5m2", "e5m2")):
        c = ed.df11_histogram_device(_dev(b), fmt).cpu().numpy().view(np.uint64)
        assert np.array_equal(c, oracle.histogram_symbols(oracle.fp8_split(b, of)[0]))


@pytest.mark.parametrize("tw", [64, 256, 512])
def test_bf16_config0(tw, unit_tensors):
    (w,) = unit_tensors("0")
    check_against_host([w], "bf16", tw, "cfg0")


@pytest.mark.parametrize("n", [1, 15, 4095, 4096, 4097, 100_003])
def test_bf16_ragged_sizes(n):
    rng = np.random.default_rng(n)
    check_against_host([_bf16(rng, n)], "bf16", 64, f"n={n}")


@pytest.mark.parametrize("seed", range(4))
def test_multi_tensor_units(seed):
    rng = np.random.default_rng(300 + seed)
    fmt = ["bf16", "fp8_e4m3", "bf16", "fp8_e5m2"][seed]
    tensors = []
    for _ in range(int(rng.integers(1, 6))):
        n = int(rng.integers(1, 120_000))
        t = _bf16(rng, n, float(rng.choice([0.02, 1.0])))
        if fmt != "bf16":
            t = sw.fp8_from_f32((t.astype(np.uint32) << 16).view(np.float32) * np.float32(100),
                                fmt.split("_")[1])
        tensors.append(t)
    check_against_host(tensors, fmt, 64 if fmt != "bf16" else (64, 256)[seed % 2], f"seed={seed}")


def test_every_bit_pattern_and_long_codes():
    w = np.tile(np.arange(1 << 16, dtype=np.uint16), 2)
    np.random.default_rng(1).shuffle(w)
    check_against_host([w], "bf16", 64, "all patterns")
    f = [1, 1]
    while len(f) < 36:
        f.append(f[-1] + f[-2])
    sym = np.repeat(np.arange(36, dtype=np.uint16) + 90, f)
    np.random.default_rng(9).shuffle(sym)
    w = ((sym << 7) | (np.arange(sym.size) & 0x807F)).astype(np.uint16)
    check_against_host([w[:3_000_000]], "bf16", 64, "32-bit codes")


def test_encoder_argument_errors():
    w = _dev(np.arange(64, dtype=np.uint16))
    cb = ed.df11_build_codebook([np.arange(64, dtype=np.uint16)])
    sz = ed.df11_sizes()
    out = ed.df11_device_encode()
    rc = ed.LIB.df11_encode_device(0, ed.ctypes.byref(cb), ed.ctypes.c_void_p(w.data_ptr()), 0, 64, 8,
                                   ed.ctypes.byref(sz), ed.ctypes.byref(out), None)
    assert rc == ed.DF11_E_INVALID  # n == 0 and nothing allocated
    with pytest.raises(ed.Df11Error):
        ed.df11_histogram_device(w[1:])  # misaligned
    with pytest.raises(ed.Df11Error):
        ed.encode_on_device([_dev(np.arange(256, dtype=np.uint8))], "fp8_e4m3", 256)


def test_70b_block_full_size():
    tensors = sw.gen_unit(sw.config("2").units[0])
    check_against_host(tensors, "bf16", 64, "70B block")
