"""GPU tests of the fused decode + GEMV (df11_decompress_gemv): results against
the oracle's float64 product within the rounding bound of the kernel's
summation order, determinism, and the argument checks."""

import numpy as np
import pytest

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")

import entropy_decoding_amd as ed  # noqa: E402
import oracle  # noqa: E402
import synth_weights as sw  # noqa: E402

U = 2.0 ** -24


def say(msg):
    print(msg, flush=True)


@pytest.fixture(scope="module", autouse=True)
def _device():
    assert torch.cuda.is_available(), "GPU tests need a ROCm device"
    torch.cuda.init()
    yield
    torch.cuda.synchronize()


def _bf16(rng, n, sigma=0.02):
    return ((rng.standard_normal(n).astype(np.float32) * sigma).view(np.uint32) >> 16).astype(np.uint16)


def _depth_per_row(hs, shapes):
    """Roundings on the longest path into each output.  In a tile a lane's
    64-chunk passes number at most P = ceil(chunks per tile / 64); it chains
    fused multiply-adds over its whole 8-weight chunks of a row (at most 8P),
    and the row's accumulator receives at most P + 2 additions (the running
    sum, chunk sums of passes that cross a row start, one edge weight).  A
    tile spanning two matrices chains at most ceil(weights / 64) <= 8P
    products per lane.  Then 7 levels of the wave sum (4 within rows of 16
    lanes, 3 over the row sums) and one addition per tile holding the row."""
    bop = hs.block_out_pos.astype(np.int64)
    passes = -(-(int(hs.max_tile_symbols) // 8 + 2) // 64)
    per_lane = 9 * passes + 2
    out, off = [], 0
    for rows, cols in shapes:
        starts = off + np.arange(rows, dtype=np.int64) * cols
        t0 = np.searchsorted(bop, starts, side="right") - 1
        t1 = np.searchsorted(bop, starts + cols - 1, side="right") - 1
        out.append(per_lane + 7 + (t1 - t0 + 1))
        off += rows * cols
    return np.concatenate(out)


def _check(tensors, shapes, label, rows_subset=None, seed=0, hs=None, cb=None):
    rng = np.random.default_rng(seed)
    if hs is None:
        cb = ed.df11_build_codebook(tensors)
        hs = ed.df11_encode(cb, tensors, 64, 8)
    ds = ed.DeviceStream(hs, cb, "cuda")
    layout = ed.gemv_layout(shapes)
    x = rng.standard_normal(layout[2]).astype(np.float32)
    xd = torch.from_numpy(x).cuda()
    y = torch.full((layout[3],), float("nan"), device="cuda")
    st = torch.zeros(1, dtype=torch.int32, device="cuda")
    say(f"[gpu] df11_decompress_gemv {label} N={hs.n_weights} shapes={shapes[:3]}...")
    ed.df11_decompress_gemv(ds, layout, xd, y, status=st)
    y2 = torch.full_like(y, float("nan"))
    ed.df11_decompress_gemv(ds, layout, xd, y2, status=st)
    torch.cuda.synchronize()
    assert int(st.item()) == 0
    assert torch.equal(y, y2)  # deterministic
    got = y.cpu().numpy().astype(np.float64)
    d = _depth_per_row(hs, shapes)
    g = d * U / (1 - d * U)
    wo = xo = yo = 0
    for (rows, cols), w in zip(shapes, tensors):
        r = np.arange(rows) if rows_subset is None else \
            np.unique(np.linspace(0, rows - 1, rows_subset).astype(np.int64))
        W = w.reshape(rows, cols)[r]
        ref = oracle.gemv(W.reshape(-1), [(r.size, cols)], x[xo:xo + cols])
        absum = np.abs(oracle.bf16_to_f64(W.reshape(-1))).reshape(r.size, cols) @ np.abs(x[xo:xo + cols])
        err = np.abs(got[yo + r] - ref)
        assert np.all(err <= g[yo + r] * absum + 1e-30), (label, np.max(err - g[yo + r] * absum))
        wo += rows * cols
        xo += cols
        yo += rows
    return got


@pytest.mark.parametrize("seed", range(3))
def test_fused_gemv_matches_the_oracle(seed):
    rng = np.random.default_rng(40 + seed)
    shapes = [(int(rng.integers(1, 50)), int(rng.integers(128, 700)) * 8) for _ in range(int(rng.integers(1, 6)))]
    tensors = [_bf16(rng, r * c, float(rng.choice([0.02, 0.5]))) for r, c in shapes]
    _check(tensors, shapes, f"random seed={seed}", seed=seed)


def test_fused_gemv_8b_block():
    unit = sw.config("1").units[0]
    tensors = sw.gen_unit(unit)
    _check(tensors, [s for _, s in unit.tensors], "8B block", rows_subset=48)


def test_fused_gemv_argument_errors():
    rng = np.random.default_rng(3)
    w = _bf16(rng, 64 * 1024)
    cb = ed.df11_build_codebook([w])
    ds = ed.DeviceStream(ed.df11_encode(cb, [w], 64, 8), cb, "cuda")
    x = torch.zeros(8192, device="cuda")
    y = torch.zeros(8192, device="cuda")
    with pytest.raises(ed.Df11Error):
        ed.df11_decompress_gemv(ds, ed.gemv_layout([(32, 1024)]), x, y)  # covers half the unit
    with pytest.raises(ed.Df11Error):
        ed.df11_decompress_gemv(ds, ed.gemv_layout([(4096, 16)]), x, y)  # too many rows per tile
    ds256 = ed.DeviceStream(ed.df11_encode(cb, [w], 256, 8), cb, "cuda")
    with pytest.raises(ed.Df11Error):
        ed.df11_decompress_gemv(ds256, ed.gemv_layout([(64, 1024)]), x, y)
    ed.df11_decompress_gemv(ds, ed.gemv_layout([(64, 1024)]), x, y)


def test_fused_gemv_small_and_ragged_units():
    rng = np.random.default_rng(11)
    for shapes in ([(1, 8)], [(2, 8)], [(3, 1024), (1, 2048)], [(5, 1040), (7, 2080), (2, 8192)]):
        tensors = [_bf16(rng, r * c) for r, c in shapes]
        _check(tensors, shapes, f"shapes={shapes}")


def test_fused_gemv_last_tile_inside_one_chunk():
    """A unit whose last tile holds fewer than 8 weights, all in one chunk
    that starts in the previous tile: the edge pass of that tile must count
    each weight once."""
    rng = np.random.default_rng(12)
    for _ in range(4000):
        rows, cols = int(rng.integers(1, 12)), int(rng.integers(128, 512)) * 8
        w = _bf16(rng, rows * cols)
        cb = ed.df11_build_codebook([w])
        hs = ed.df11_encode(cb, [w], 64, 8)
        p0, p1 = int(hs.block_out_pos[-2]), int(hs.block_out_pos[-1])
        if hs.n_tiles > 1 and 0 < p1 - p0 < 8 and p0 % 8 and (p0 // 8) == ((p1 - 1) // 8):
            _check([w], [(rows, cols)], f"last tile [{p0},{p1})", hs=hs, cb=cb)
            return
    pytest.fail("no unit with such a last tile among the sizes tried")


def test_fused_gemv_corrupt_unit_is_reported():
    rng = np.random.default_rng(13)
    shapes = [(64, 2048)]
    w = _bf16(rng, 64 * 2048)
    cb = ed.df11_build_codebook([w])
    hs = ed.df11_encode(cb, [w], 64, 8)
    ds = ed.DeviceStream(hs, cb, "cuda")
    bad = hs.block_out_pos.copy()
    bad[5] += 3
    ds.block_out_pos.copy_(torch.from_numpy(bad.view(np.uint8)))
    layout = ed.gemv_layout(shapes)
    x = torch.ones(layout[2], device="cuda")
    y = torch.zeros(layout[3], device="cuda")
    st = torch.zeros(1, dtype=torch.int32, device="cuda")
    say("[gpu] df11_decompress_gemv corrupt block_out_pos")
    ed.df11_decompress_gemv(ds, layout, x, y, status=st)
    torch.cuda.synchronize()
    assert int(st.item()) == ed.DF11_E_CORRUPT


def test_fused_gemv_scratch_needs_no_initialisation():
    """The workspace's previous contents (any bytes, or another unit's
    indices) do not change the results."""
    rng = np.random.default_rng(14)
    shapes = [(40, 4096), (24, 2048)]
    tensors = [_bf16(rng, r * c) for r, c in shapes]
    cb = ed.df11_build_codebook(tensors)
    ds = ed.DeviceStream(ed.df11_encode(cb, tensors, 64, 8), cb, "cuda")
    layout = ed.gemv_layout(shapes)
    x = torch.from_numpy(rng.standard_normal(layout[2]).astype(np.float32)).cuda()
    need = int(ed.LIB.df11_decompress_gemv_scratch_bytes(ed.ctypes.byref(ds.desc)))
    ys = []
    for fill in ("zeros", "ones", "random"):
        if fill == "zeros":
            scr = torch.zeros(need, dtype=torch.uint8, device="cuda")
        elif fill == "ones":
            scr = torch.full((need,), 0xFF, dtype=torch.uint8, device="cuda")
        else:
            scr = torch.from_numpy(rng.integers(0, 256, need, dtype=np.uint8)).cuda()
        y = torch.full((layout[3],), float("nan"), device="cuda")
        st = torch.zeros(1, dtype=torch.int32, device="cuda")
        say(f"[gpu] df11_decompress_gemv scratch={fill}")
        ed.df11_decompress_gemv(ds, layout, x, y, scr, st)
        torch.cuda.synchronize()
        assert int(st.item()) == 0
        ys.append(y)
    assert torch.equal(ys[0], ys[1]) and torch.equal(ys[0], ys[2])
    with pytest.raises(ed.Df11Error):  # one byte short
        ed.df11_decompress_gemv(ds, layout, x, ys[0], torch.zeros(need - 1, dtype=torch.uint8,
                                                                  device="cuda"))
