"""The decode under HIP graph capture: the library allocates nothing, clears
nothing with memsets and never synchronises, so a captured launch replays
as is.  Each graph is replayed several times with the program's own eager
work (a fill of the output) and a synchronisation between replays, and every
replay must equal the eager result bit for bit."""

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


def _replays(graph, out, ref, fill, label, n=4):
    for i in range(n):
        out.fill_(fill)
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(out, ref), f"{label}: replay {i}: {int((out != ref).sum())} outputs differ"


def test_decompress_block_replays_from_a_graph():
    rng = np.random.default_rng(11)
    tensors = [((rng.standard_normal(n).astype(np.float32) * 0.02).view(np.uint32) >> 16)
               .astype(np.uint16) for n in (300_001, 4096, 77_777)]
    cb = ed.df11_build_codebook(tensors)
    hs = ed.df11_encode(cb, tensors, 64, 8)
    ds = ed.DeviceStream(hs, cb, "cuda")
    original = torch.from_numpy(np.concatenate(tensors).view(np.int16)).cuda()
    out = torch.empty(hs.n_weights, dtype=torch.int16, device="cuda")
    status = torch.zeros(1, dtype=torch.int32, device="cuda")
    say(f"[gpu] df11_decompress_block captured in a graph, N={hs.n_weights} tiles={hs.n_tiles}")
    ed.df11_decompress_block(ds, out, status)  # eager, before the capture
    torch.cuda.synchronize()
    assert int(status.item()) == 0 and torch.equal(out, original)
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        ed.df11_decompress_block(ds, out, status)
    _replays(graph, out, original, -1, "df11_decompress_block")
    assert int(status.item()) == 0


def test_noalloc_gemv_replays_from_a_graph():
    unit = sw.config("0").units[0]
    tensors = sw.gen_unit(unit)
    shapes = [shape for _, shape in unit.tensors]
    cb = ed.df11_build_codebook(tensors)
    hs = ed.df11_encode(cb, tensors, 64, 8)
    ds = ed.DeviceStream(hs, cb, "cuda")
    layout = ed.gemv_layout(shapes)
    x = torch.from_numpy(np.random.default_rng(12).standard_normal(layout[2]).astype(np.float32)).cuda()
    y_ref = torch.full((layout[3],), float("nan"), device="cuda")
    y = torch.full((layout[3],), float("nan"), device="cuda")
    status = torch.zeros(1, dtype=torch.int32, device="cuda")
    say(f"[gpu] df11_decompress_gemv_noalloc captured in a graph, N={hs.n_weights}")
    # eager calls first: the reference, and the first call on this device,
    # which looks up the static workspace's address
    ed.df11_decompress_gemv(ds, layout, x, y_ref, status=status)
    ed.df11_decompress_gemv_noalloc(ds, layout, x, y, status=status)
    torch.cuda.synchronize()
    assert int(status.item()) == 0 and torch.equal(y, y_ref)
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        ed.df11_decompress_gemv_noalloc(ds, layout, x, y, status=status)
    _replays(graph, y, y_ref, float("nan"), "df11_decompress_gemv_noalloc")
    assert int(status.item()) == 0
