"""GPU tests of the fused decode + GEMM on the matrix cores
(df11_decompress_gemm).

With small integer weights and activations every partial sum is an integer
below 2^24, so any float32 summation order is exact and the results must
equal the oracle's float64 product bit for bit; this pins the sub-block
order, the lane mapping, the masking of shared chunks and the cross-wave sum.
On Gaussian data the results must lie within a rounding bound that assumes
nothing about the matrix cores' internal order: at most one rounding of at
most 2u per addition, K + K/32 + 3 additions per output, plus one per extra
K segment of a split matrix (at most ceil(K / 4096) segments).
"""

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


def _bf16(a):
    return (np.asarray(a, dtype=np.float32).view(np.uint32) >> 16).astype(np.uint16)


class GemmUnit:
    """Matrices (row-major BF16) compressed in GEMM order, one unit."""

    def __init__(self, tensors, shapes):
        self.tensors, self.shapes = tensors, shapes
        ordered = [ed.df11_gemm_order(t, r, c) for t, (r, c) in zip(tensors, shapes)]
        self.cb = ed.df11_build_codebook(ordered)
        self.hs = ed.df11_encode(self.cb, ordered, 64, 8)
        self.ds = ed.DeviceStream(self.hs, self.cb, "cuda")
        self.ordered = ordered

    def run(self, x, n, label, status=None):
        layout = ed.gemm_layout(self.shapes, n)
        y = torch.full((layout[3],), float("nan"), device="cuda")
        st = torch.zeros(1, dtype=torch.int32, device="cuda") if status is None else status
        say(f"[gpu] df11_decompress_gemm {label} n={n} N={self.hs.n_weights} tiles={self.hs.n_tiles}")
        ed.df11_decompress_gemm(self.ds, layout, n, torch.from_numpy(x.view(np.int16)).cuda(), y,
                                status=st)
        torch.cuda.synchronize()
        return y.cpu().numpy().astype(np.float64), int(st.item())


def _int_unit(rng, shapes, scale_exp=0):
    tensors = [_bf16(rng.integers(-4, 5, r * c).astype(np.float32) * 2.0 ** scale_exp)
               for r, c in shapes]
    return GemmUnit(tensors, shapes)


@pytest.mark.parametrize("n", [16, 32, 48, 64])
def test_gemm_integer_data_is_exact(n):
    rng = np.random.default_rng(100 + n)
    shapes = [(16, 32), (48, 96), (32, 1024), (64, 2080)]
    u = _int_unit(rng, shapes)
    x = _bf16(rng.integers(-3, 4, sum(n * c for _, c in shapes)).astype(np.float32))
    y, st = u.run(x, n, "integers")
    assert st == 0
    ref = oracle.gemm(np.concatenate(u.tensors), shapes, x, n)
    assert np.array_equal(y, ref), np.flatnonzero(y != ref)[:10]


@pytest.mark.parametrize("seed", range(4))
def test_gemm_integer_random_units(seed):
    """Random shapes and value spreads: tile and row-block boundaries fall
    anywhere (value spreads change the code lengths and tile sizes)."""
    rng = np.random.default_rng(200 + seed)
    shapes = [(16 * int(rng.integers(1, 9)), 32 * int(rng.integers(1, 40)))
              for _ in range(int(rng.integers(1, 6)))]
    u = _int_unit(rng, shapes, scale_exp=int(rng.integers(-8, 8)))
    n = 16 * int(rng.integers(1, 5))
    x = _bf16(rng.integers(-3, 4, sum(n * c for _, c in shapes)).astype(np.float32))
    y, st = u.run(x, n, f"random seed={seed} shapes={shapes}")
    assert st == 0
    assert np.array_equal(y, oracle.gemm(np.concatenate(u.tensors), shapes, x, n))


def _bound(tensors, shapes, x, n):
    w = np.abs(oracle.bf16_to_f64(np.concatenate(tensors)))
    xa = np.abs(oracle.bf16_to_f64(x))
    out, wo, xo = [], 0, 0
    for r, c in shapes:
        d = c + c // 32 + 3 + (c + 4095) // 4096 - 1
        g = 2 * d * U / (1 - 2 * d * U)
        W = w[wo:wo + r * c].reshape(r, c)
        X = xa[xo:xo + n * c].reshape(n, c)
        out.append((g * (X @ W.T)).reshape(-1))
        wo += r * c
        xo += n * c
    return np.concatenate(out)


def test_gemm_gaussian_data_within_the_bound_and_deterministic():
    rng = np.random.default_rng(7)
    shapes = [(64, 4096), (32, 1024), (48, 2048)]
    tensors = [_bf16(rng.standard_normal(r * c) * 0.02) for r, c in shapes]
    u = GemmUnit(tensors, shapes)
    n = 32
    x = _bf16(rng.standard_normal(sum(n * c for _, c in shapes)))
    y1, st1 = u.run(x, n, "gaussian")
    y2, st2 = u.run(x, n, "gaussian again")
    assert st1 == 0 and st2 == 0
    assert np.array_equal(y1, y2)
    ref = oracle.gemm(np.concatenate(tensors), shapes, x, n)
    err = np.abs(y1 - ref)
    assert np.all(err <= _bound(tensors, shapes, x, n) + 1e-30)


@pytest.mark.parametrize("n", [16, 32, 48, 64])
def test_gemm_split_rows_integer_exact_and_gaussian_bound(n):
    """Matrices 3.25 and 2.02 times wider than the narrowest (4096 columns)
    are split into K segments of 104 and 87/87/85 sub-blocks: integer data
    stays exact, Gaussian data within the bound, and repeated calls agree."""
    rng = np.random.default_rng(300 + n)
    shapes = [(32, 4096), (16, 13312), (48, 8288)]
    u = _int_unit(rng, shapes)
    x = _bf16(rng.integers(-3, 4, sum(n * c for _, c in shapes)).astype(np.float32))
    y, st = u.run(x, n, "split integers")
    assert st == 0
    ref = oracle.gemm(np.concatenate(u.tensors), shapes, x, n)
    assert np.array_equal(y, ref), np.flatnonzero(y != ref)[:10]

    tensors = [_bf16(rng.standard_normal(r * c) * 0.02) for r, c in shapes]
    g = GemmUnit(tensors, shapes)
    x = _bf16(rng.standard_normal(sum(n * c for _, c in shapes)))
    y1, st1 = g.run(x, n, "split gaussian")
    y2, st2 = g.run(x, n, "split gaussian again")
    assert st1 == st2 == 0
    assert np.array_equal(y1, y2)
    ref = oracle.gemm(np.concatenate(tensors), shapes, x, n)
    assert np.all(np.abs(y1 - ref) <= _bound(tensors, shapes, x, n))


def test_gemm_8b_block_sampled():
    unit = sw.config("1").units[0]
    shapes = [s for _, s in unit.tensors]
    tensors = sw.gen_unit(unit)
    u = GemmUnit(tensors, shapes)
    n = 16
    rng = np.random.default_rng(8)
    x = _bf16(rng.standard_normal(sum(n * c for _, c in shapes)))
    y, st = u.run(x, n, "8B block")
    assert st == 0
    yo = xo = 0
    for (r, c), w in zip(shapes, tensors):
        rows = np.unique(np.linspace(0, r - 1, 24).astype(np.int64))
        W = w.reshape(r, c)[rows]
        X = x[xo:xo + n * c]
        ref = oracle.gemm(W.reshape(-1), [(rows.size, c)], X, n).reshape(n, rows.size)
        got = y[yo:yo + n * r].reshape(n, r)[:, rows]
        b = _bound([W.reshape(-1)], [(rows.size, c)], X, n).reshape(n, rows.size)
        assert np.all(np.abs(got - ref) <= b + 1e-30)
        yo += n * r
        xo += n * c


def test_gemm_order_unit_decompresses_to_the_ordered_weights():
    rng = np.random.default_rng(9)
    shapes = [(32, 256), (16, 64)]
    u = _int_unit(rng, shapes)
    out = torch.empty(u.hs.n_weights, dtype=torch.int16, device="cuda")
    ed.df11_decompress_block(u.ds, out)
    torch.cuda.synchronize()
    assert np.array_equal(out.cpu().numpy().view(np.uint16), np.concatenate(u.ordered))


def test_gemm_argument_errors_and_corruption():
    rng = np.random.default_rng(10)
    shapes = [(32, 512)]
    u = _int_unit(rng, shapes)
    x = torch.zeros(80 * 1024, dtype=torch.int16, device="cuda")
    y = torch.zeros(80 * 32, dtype=torch.float32, device="cuda")
    lay = ed.gemm_layout(shapes, 16)
    for n in (0, 8, 80):
        with pytest.raises(ed.Df11Error):
            ed.df11_decompress_gemm(u.ds, ed.gemm_layout(shapes, max(n, 16)), n, x, y)
    with pytest.raises(ed.Df11Error):  # rows not a multiple of 16 (the layout no longer tiles)
        ed.df11_decompress_gemm(u.ds, ed.gemm_layout([(16, 512), (8, 1024)], 16), 16, x, y)
    with pytest.raises(ed.Df11Error):  # misaligned x
        ed.df11_decompress_gemm(u.ds, lay, 16, x[1:], y)
    u256 = ed.DeviceStream(ed.df11_encode(u.cb, u.ordered, 256, 8), u.cb, "cuda")
    with pytest.raises(ed.Df11Error):  # 256-window tiles
        ed.df11_decompress_gemm(u256, lay, 16, x, y)
    bad = u.hs.block_out_pos.copy()
    if bad.size > 3:
        bad[1] += 1
        u.ds.block_out_pos.copy_(torch.from_numpy(bad.view(np.uint8)))
        st = torch.zeros(1, dtype=torch.int32, device="cuda")
        say("[gpu] df11_decompress_gemm corrupt block_out_pos")
        ed.df11_decompress_gemm(u.ds, lay, 16, x, y, status=st)
        torch.cuda.synchronize()
        assert int(st.item()) == ed.DF11_E_CORRUPT


def test_gemm_split_matrix_corruption_is_reported_and_other_matrices_exact():
    """A corrupt block_out_pos entry inside a matrix split into three K
    segments is reported; the unsplit matrix before it, whose tiles are
    intact, keeps its exact products."""
    rng = np.random.default_rng(12)
    shapes = [(16, 4096), (16, 12288)]
    u = _int_unit(rng, shapes)
    n = 16
    x = _bf16(rng.integers(-3, 4, sum(n * c for _, c in shapes)).astype(np.float32))
    bad = u.hs.block_out_pos.copy()
    t = int(np.searchsorted(bad, 16 * 4096 + 16 * 6000))  # a tile boundary in the split matrix
    assert bad[t - 1] > 16 * 4096 + 512
    bad[t] += 3
    u.ds.block_out_pos.copy_(torch.from_numpy(bad.view(np.uint8)))
    st = torch.zeros(1, dtype=torch.int32, device="cuda")
    y, code = u.run(x, n, "split corrupt", status=st)
    assert code == ed.DF11_E_CORRUPT
    ref = oracle.gemm(np.concatenate(u.tensors), shapes, x, n)
    first = ref.reshape(-1)[: n * 16]  # y of the first matrix (token-major, 16 rows)
    assert np.array_equal(y[: n * 16], first)


@pytest.mark.parametrize("shapes,split", [([(32, 512), (16, 256)], 0),
                                          ([(16, 4096), (16, 8224)], 3)])
def test_gemm_scratch_needs_no_initialisation_and_is_checked(shapes, split):
    """Neither the reordered activations nor the K segments' partial sums
    (8224 columns against 4096: three segments) need clearing."""
    rng = np.random.default_rng(11)
    u = _int_unit(rng, shapes)
    n = 32
    layout = ed.gemm_layout(shapes, n)
    x = torch.from_numpy(_bf16(rng.integers(-3, 4, layout[2]).astype(np.float32)).view(np.int16)).cuda()
    need = ed.df11_decompress_gemm_scratch_bytes(layout, n)
    assert need == 2 * n * sum(c for _, c in shapes) + 4 * split * n * shapes[-1][0]
    ys = []
    for fill in (0x00, 0xFF):
        scr = torch.full((need,), fill, dtype=torch.uint8, device="cuda")
        y = torch.full((layout[3],), float("nan"), device="cuda")
        ed.df11_decompress_gemm(u.ds, layout, n, x, y, scr)
        torch.cuda.synchronize()
        ys.append(y)
    assert torch.equal(ys[0], ys[1])
    ref = oracle.gemm(np.concatenate(u.tensors), shapes, x.cpu().numpy().view(np.uint16), n)
    assert np.array_equal(ys[0].cpu().numpy().astype(np.float64), ref)
    with pytest.raises(ed.Df11Error):
        ed.df11_decompress_gemm(u.ds, layout, n, x, ys[0],
                                torch.zeros(need - 16, dtype=torch.uint8, device="cuda"))
