"""GPU tests of the overlapped block pipeline and its GEMV consumer.

The GEMV is checked against the oracle's float64 product within the rounding
bound of the kernel's fixed summation order; the pipeline is checked by
comparing, bit for bit, the consumer's results under overlap with the results
of the same kernels run one after another on one stream (a missing wait would
let the consumer read a half-written buffer, or a decompression overwrite a
buffer still being read).
"""

import numpy as np
import pytest

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")

import entropy_decoding_amd as ed  # noqa: E402
import oracle  # noqa: E402

U = 2.0 ** -24  # unit roundoff of float32


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


def _gemv_bound(w_flat, shapes, x):
    """Per-row bound on |y - y_exact|.  Each row is a sum formed by a chain of
    at most ceil(cols / 64) fused multiply-adds per lane followed by 6 levels of
    a butterfly, so every term passes through at most d = ceil(cols/64) + 6
    roundings: |error| <= gamma_d * sum |w x| with gamma_d = d u / (1 - d u)."""
    w = np.abs(oracle.bf16_to_f64(w_flat))
    xa = np.abs(np.asarray(x, dtype=np.float64))
    out, wo, xo = [], 0, 0
    for rows, cols in shapes:
        d = -(-cols // 64) + 6
        g = d * U / (1 - d * U)
        out.append(g * (w[wo:wo + rows * cols].reshape(rows, cols) @ xa[xo:xo + cols]))
        wo += rows * cols
        xo += cols
    return np.concatenate(out)


def _check_gemv(shapes, seed):
    rng = np.random.default_rng(seed)
    n = sum(r * c for r, c in shapes)
    w = _bf16(rng, n)
    layout = ed.gemv_layout(shapes)
    x = rng.standard_normal(layout[2]).astype(np.float32)
    wd = torch.from_numpy(w.view(np.int16)).cuda()
    xd = torch.from_numpy(x).cuda()
    yd = torch.full((layout[3],), float("nan"), dtype=torch.float32, device="cuda")
    say(f"[gpu] df11_gemv_bf16 shapes={shapes}")
    ed.df11_gemv_bf16(wd, layout, xd, yd)
    torch.cuda.synchronize()
    y = yd.cpu().numpy().astype(np.float64)
    ref = oracle.gemv(w, shapes, x)
    bound = _gemv_bound(w, shapes, x)
    assert np.all(np.abs(y - ref) <= bound + 1e-30), np.max(np.abs(y - ref) - bound)
    return y


@pytest.mark.parametrize("seed", range(3))
def test_gemv_matches_the_oracle_within_the_rounding_bound(seed):
    shapes = [(7, 8), (33, 520), (4, 512), (130, 1024), (5, 4096), (1, 8), (3, 14336)]
    _check_gemv(shapes[seed:] + shapes[:seed], seed)


def test_gemv_exact_cases():
    # all-ones weights and small integer x: every partial sum is an exact integer
    rows, cols = 9, 1032
    w = np.full(rows * cols, 0x3F80, dtype=np.uint16)
    x = (np.arange(cols) % 7).astype(np.float32)
    layout = ed.gemv_layout([(rows, cols)])
    yd = torch.zeros(rows, dtype=torch.float32, device="cuda")
    ed.df11_gemv_bf16(torch.from_numpy(w.view(np.int16)).cuda(), layout,
                      torch.from_numpy(x).cuda(), yd)
    torch.cuda.synchronize()
    assert np.array_equal(yd.cpu().numpy(), np.full(rows, x.sum(), dtype=np.float32))


def test_gemv_rejects_misaligned_layouts():
    w = torch.zeros(64, dtype=torch.int16, device="cuda")
    x = torch.zeros(16, dtype=torch.float32, device="cuda")
    y = torch.zeros(16, dtype=torch.float32, device="cuda")
    with pytest.raises(ed.Df11Error):
        ed.df11_gemv_bf16(w, ed.gemv_layout([(2, 12)]), x, y)  # cols not a multiple of 8
    lay = ed.gemv_layout([(2, 8)])
    with pytest.raises(ed.Df11Error):
        ed.df11_gemv_bf16(w[1:], lay, x, y)  # w not 16-byte aligned


def _blocks(seed, n_blocks):
    rng = np.random.default_rng(seed)
    blocks = []
    for i in range(n_blocks):
        shapes = [(int(rng.integers(1, 400)) * 4, int(rng.integers(1, 96)) * 64) for _ in range(3)]
        if i % 3 == 1:
            shapes.append((4096, 2048))  # a large one: decompression of it overlaps more work
        tensors = [_bf16(rng, r * c, float(rng.choice([0.02, 0.005]))) for r, c in shapes]
        cb = ed.df11_build_codebook(tensors)
        hs = ed.df11_encode(cb, tensors)
        blocks.append((shapes, tensors, ed.DeviceStream(hs, cb, "cuda")))
    return blocks


@pytest.mark.parametrize("n_slots,share", [(2, 0), (3, 0), (2, 1), (3, 2)])
def test_pipelined_results_equal_sequential_results(n_slots, share):
    """(share: the decode's workgroups per compute unit; 0 is the full grid)"""
    blocks = _blocks(100 + n_slots, 7)
    nmax = max(ds.n_weights for _, _, ds in blocks)
    bufs = [torch.empty(nmax, dtype=torch.int16, device="cuda") for _ in range(n_slots)]
    layouts = [ed.gemv_layout(shapes) for shapes, _, _ in blocks]
    rng = np.random.default_rng(7)
    xs = [torch.from_numpy(rng.standard_normal(lay[2]).astype(np.float32)).cuda() for lay in layouts]
    y_pipe = [torch.full((lay[3],), float("nan"), device="cuda") for lay in layouts]
    y_seq = [torch.full((lay[3],), float("nan"), device="cuda") for lay in layouts]
    status = torch.zeros(1, dtype=torch.int32, device="cuda")
    torch.cuda.synchronize()

    decode, compute = torch.cuda.Stream(), torch.cuda.Stream()
    p = ed.Pipeline(decode, n_slots)
    p.set_decode_share(share)
    say(f"[gpu] pipeline n_slots={n_slots} share={share} blocks={len(blocks)}")
    for i in range(min(n_slots - 1, len(blocks))):
        p.decompress(i % n_slots, blocks[i][2], bufs[i % n_slots], status)
    for i in range(len(blocks)):
        j = i + n_slots - 1
        if j < len(blocks):
            p.decompress(j % n_slots, blocks[j][2], bufs[j % n_slots], status)
        p.acquire(i % n_slots, compute)
        ed.df11_gemv_bf16(bufs[i % n_slots], layouts[i], xs[i], y_pipe[i], stream=compute)
        p.release(i % n_slots, compute)
    compute.synchronize()
    decode.synchronize()
    p.close()

    say("[gpu] the same work on one stream")
    for i, (shapes, tensors, ds) in enumerate(blocks):
        ed.df11_decompress_block(ds, bufs[0], status)
        ed.df11_gemv_bf16(bufs[0], layouts[i], xs[i], y_seq[i])
    torch.cuda.synchronize()
    assert int(status.item()) == 0
    for i, (shapes, tensors, _) in enumerate(blocks):
        assert torch.equal(y_pipe[i], y_seq[i]), i
        w = np.concatenate(tensors)
        x = xs[i].cpu().numpy()
        err = np.abs(y_seq[i].cpu().numpy().astype(np.float64) - oracle.gemv(w, shapes, x))
        assert np.all(err <= _gemv_bound(w, shapes, x) + 1e-30), i


def test_pipeline_argument_errors():
    s = torch.cuda.Stream()
    with pytest.raises(ed.Df11Error):
        ed.Pipeline(s, 0)
    with pytest.raises(ed.Df11Error):
        ed.Pipeline(s, ed.DF11_PIPELINE_MAX_SLOTS + 1)
    p = ed.Pipeline(s, 2)
    with pytest.raises(ed.Df11Error):
        p.acquire(0, s)  # never filled
    with pytest.raises(ed.Df11Error):
        p.release(1, s)
    with pytest.raises(ed.Df11Error):
        p.acquire(2, s)  # no such slot
    with pytest.raises(ed.Df11Error):
        p.set_decode_share(65)  # more workgroups per compute unit than can be resident
    p.close()
    p.close()  # idempotent
