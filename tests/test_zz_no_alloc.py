"""df11_decompress_gemv_noalloc: the fused decode + GEMV on the library's
static per-GPU workspace, called through the C ABI, must give exactly the
products of df11_decompress_gemv (same kernels and summation order) on two
calls in a row, the second on a smaller unit; units beyond the workspace are
refused before anything is launched."""

import ctypes

import numpy as np
import pytest

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")

import entropy_decoding_amd as ed  # noqa: E402
import synth_weights as sw  # noqa: E402


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


def _both(tensors, shapes, label, seed):
    cb = ed.df11_build_codebook(tensors)
    hs = ed.df11_encode(cb, tensors, 64, 8)
    ds = ed.DeviceStream(hs, cb, "cuda")
    layout = ed.gemv_layout(shapes)
    arr, n, nx, ny = layout
    x = torch.from_numpy(np.random.default_rng(seed).standard_normal(nx).astype(np.float32)).cuda()
    y_ref = torch.full((ny,), float("nan"), device="cuda")
    y = torch.full((ny,), float("nan"), device="cuda")
    st_ref = torch.zeros(1, dtype=torch.int32, device="cuda")
    st = torch.zeros(1, dtype=torch.int32, device="cuda")
    say(f"[gpu] df11_decompress_gemv vs _noalloc {label} N={hs.n_weights} tiles={hs.n_tiles}")
    ed.df11_decompress_gemv(ds, layout, x, y_ref, status=st_ref)
    stream = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    rc = ed.LIB.df11_decompress_gemv_noalloc(ctypes.byref(ds.desc), arr, n,
                                             ctypes.c_void_p(x.data_ptr()),
                                             ctypes.c_void_p(y.data_ptr()),
                                             ctypes.c_void_p(st.data_ptr()), stream)
    assert rc == ed.DF11_OK
    torch.cuda.synchronize()
    assert int(st_ref.item()) == 0 and int(st.item()) == 0
    assert torch.equal(y, y_ref), f"{label}: {int((y != y_ref).sum())} outputs differ"
    assert not torch.isnan(y).any()


def test_two_calls_in_a_row_second_smaller():
    unit = sw.config("1").units[0]
    shapes = [s for _, s in unit.tensors]
    _both(sw.gen_unit(unit), shapes, "8B block", 1)
    rng = np.random.default_rng(77)
    shapes2 = [(96, 1024), (40, 2048), (130, 1536)]  # wide enough for the 4-row tile rule
    _both([_bf16(rng, r * c) for r, c in shapes2], shapes2, "small unit", 2)


def test_a_unit_beyond_the_workspace_is_refused():
    d = ed.df11_device_stream()
    d.tile_windows, d.window_bytes, d.n_luts = 64, 8, 1
    d.n_tiles = ed.DF11_GEMV_NOALLOC_MAX_TILES + 1
    d.total_bits = d.n_tiles * 4096
    d.n_weights = d.total_bits // 3
    arr, n, _, _ = ed.gemv_layout([(1, 8)])
    rc = ed.LIB.df11_decompress_gemv_noalloc(ctypes.byref(d), arr, n, None, None, None, None)
    assert rc == ed.DF11_E_CAPACITY
