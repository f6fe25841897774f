"""Decompression throughput of the DFloat11-style BF16 decoder on one MI355X.

One step = one df11_decompress_block launch over a whole unit (by default the
Llama-3-70B-shaped transformer block: 855,638,016 BF16 weights, one codebook,
one launch), with the compressed unit already resident in HBM.

Prints one JSON line: value = decompressed BF16 GB/s (2 bytes per weight
written, whole job over K steps), plus the dominant kernel's HBM roofline
fraction from algorithmic bytes (compressed arrays read once + BF16 written)
and the CPU oracle's bit-serial decode timed on this host as a baseline.

  python bench.py [--steps K] [--warmup W] [--config 2|1|0|2tp8|405tp8|3a|3b|3c|4] [--tile-windows 64|256|512]
  python bench.py --pipeline     # 8B model blocks, next block decompressed while a GEMV reads this one
  python bench.py --fused        # y = W x straight from the compressed block vs decompress + GEMV
  python bench.py --fused-gemm   # Y = X W^T for 16-64 tokens on the matrix cores, same comparison
"""

from __future__ import annotations

import argparse
import hashlib
import json
import os
import platform
import subprocess
import sys
import threading
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0
KERNEL_SOURCE = os.path.join(ROOT, "entropy_decoding_amd", "csrc", "df11_device.hip")
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic.json")


def log(msg):
    print(msg, file=sys.stderr, flush=True)


def kernel_hash() -> str:
    return hashlib.sha256(open(KERNEL_SOURCE, "rb").read()).hexdigest()[:16]


def algorithmic_bytes(hs, cb) -> int:
    """Compressed arrays read once (stream payload, sign+mantissa array, gaps,
    block_out_pos, tables) plus the output written: 2 bytes per BF16 weight, 1
    per FP8 weight."""
    import entropy_decoding_amd as ed

    sm = hs.n_weights if hs.format == 0 else (hs.n_weights + 1) // 2
    read = (hs.total_bits + 7) // 8 + sm + hs.gaps.size + 4 * hs.block_out_pos.size \
        + ed.table_bytes(cb)
    return int(read + (2 if hs.format == 0 else 1) * hs.n_weights)


def measured_traffic(workload: str, tile_windows: int):
    """HBM bytes per launch from the committed rocprofv3 counter runs, if they were
    taken on the current kernel source; else None."""
    try:
        rec = json.load(open(TRAFFIC_FILE))
    except (OSError, ValueError):
        return None
    r = rec.get(f"{workload}/T{tile_windows}")
    if not r or r.get("kernel_sha") != kernel_hash():
        return None
    return r.get("bytes_per_launch")


def cpu_name() -> str:
    try:
        out = subprocess.run(["lscpu"], capture_output=True, text=True).stdout
        for line in out.splitlines():
            if line.startswith("Model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return platform.processor() or "unknown"


def cpu_baseline(tensors):
    """The oracle as it stands, on this host's cores, after the GPU timing.

    Three figures from one oracle encoding of the whole unit (the unit's
    codebook, the plain bit-serial encoder): the encode itself on one thread,
    a bit-serial decode of the whole unit on one thread, and one thread per
    tensor decoding from the tensor start bits the oracle's encoder records.
    GB/s are BF16 bytes (2 per weight) per second.  `value` is the
    thread-per-tensor decode."""
    import oracle

    n = sum(t.size for t in tensors)
    ocb = oracle.codebook(tensors)
    t0 = time.perf_counter()
    enc = oracle.encode(tensors, ocb)
    t_enc = time.perf_counter() - t0
    t0 = time.perf_counter()
    whole = oracle.decode(enc.stream, 0, enc.total_bits, ocb.lens, enc.sm)
    t_one = time.perf_counter() - t0
    flat = np.concatenate([np.asarray(t).reshape(-1) for t in tensors])
    assert np.array_equal(whole, flat), "oracle decode is not lossless"
    del whole
    outs = [None] * len(tensors)
    offs = np.cumsum([0] + [t.size for t in tensors])

    def dec(i):
        outs[i] = oracle.decode(enc.stream, enc.tensor_start_bits[i], enc.tensor_start_bits[i + 1],
                                ocb.lens, enc.sm[offs[i]:offs[i + 1]])

    ths = [threading.Thread(target=dec, args=(i,)) for i in range(len(tensors))]
    t0 = time.perf_counter()
    for t in ths:
        t.start()
    for t in ths:
        t.join()
    t_par = time.perf_counter() - t0
    for o, t in zip(outs, tensors):
        assert np.array_equal(o, np.asarray(t).reshape(-1)), "oracle decode is not lossless"
    host, nproc = cpu_name(), os.cpu_count()
    gbs = lambda dt: round(2 * n / dt / 1e9, 4)
    return {"value": gbs(t_par), "unit": "GB/s", "cores": len(tensors), "kind": "oracle",
            "sample": f"host {host}, nproc {nproc}, {len(tensors)} threads: the whole unit "
                      f"({n} weights, {len(tensors)} tensors), one thread per tensor decoding "
                      f"bit-serially from the oracle's tensor start bits, {t_par:.2f} s wall; "
                      f"one thread over the whole unit {t_one:.2f} s; oracle encode on one "
                      f"thread {t_enc:.2f} s",
            "host": host, "nproc": nproc,
            "decode_one_thread": {"value": gbs(t_one), "unit": "GB/s", "cores": 1,
                                  "seconds": round(t_one, 3)},
            "encode_one_thread": {"value": gbs(t_enc), "unit": "GB/s of BF16 input", "cores": 1,
                                  "seconds": round(t_enc, 3)}}


def settle(step, torch, ms: float = 100.0, max_launches: int = 5000):
    """Runs step() until the GPU has been kept busy for `ms` milliseconds.

    An idle MI355X sits at a low shader clock (157 MHz read by rocm-smi before
    a run) and ramps up only over tens of milliseconds of work: on the 70B
    block, five warm-up launches left the first timed launches at 0.63-0.65 ms
    against 0.537 ms once settled.  This runs before the warm-up steps, untimed,
    and its length is reported."""
    t0 = time.perf_counter()
    n = 0
    while n < max_launches:
        for _ in range(8):
            step()
        n += 8
        torch.cuda.synchronize()
        if (time.perf_counter() - t0) * 1e3 >= ms:
            break
    return {"launches": n, "ms": round((time.perf_counter() - t0) * 1e3, 1)}


def log_steps(name, kms):
    """Per-step kernel times on stderr: the first and last steps, so that a
    run whose early steps are slower than its late ones shows it."""
    k = np.asarray(kms)
    head = " ".join(f"{v:.4f}" for v in k[:8])
    tail = " ".join(f"{v:.4f}" for v in k[-8:])
    log(f"[bench] {name}: step ms first [{head}] last [{tail}] "
        f"min {k.min():.4f} p50 {np.percentile(k, 50):.4f} max {k.max():.4f}")


def run_unit(name, tensors, args, torch, ed):
    dev = torch.device("cuda:0")
    t0 = time.perf_counter()
    cb = ed.df11_build_codebook(tensors, args.format)
    hs = ed.df11_encode(cb, tensors, args.tile_windows, 8, args.format)
    log(f"[bench] {name}: encoded {hs.n_weights} weights in {time.perf_counter() - t0:.1f} s, "
        f"{hs.n_tiles} tiles, luts={cb.n_luts}, max_len={cb.max_len}")
    ds = ed.DeviceStream(hs, cb, dev)
    n = hs.n_weights
    out = torch.empty(n, dtype=torch.bfloat16 if args.format == "bf16" else torch.uint8,
                      device=dev)
    status = torch.zeros(1, dtype=torch.int32, device=dev)
    stream = torch.cuda.current_stream()
    alg = algorithmic_bytes(hs, cb)
    # a unit under 1 GiB could be served partly from the 256 MB last-level
    # cache on the next step: evict it between steps by READING 1 GiB (a
    # write would leave dirty lines for the timed kernel to write back)
    small = alg < (1 << 30)
    flush = torch.zeros(1 << 28, dtype=torch.int32, device=dev) if small else None
    sink = torch.zeros((), dtype=torch.int32, device=dev)

    settled = settle(lambda: ed.df11_decompress_block(ds, out, status, stream), torch,
                     args.settle_ms)
    for _ in range(args.warmup):
        ed.df11_decompress_block(ds, out, status, stream)
    torch.cuda.synchronize()

    starts = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps)]
    ends = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        if flush is not None:
            torch.amax(flush, dim=0, out=sink)
        starts[i].record(stream)
        ed.df11_decompress_block(ds, out, status, stream)
        ends[i].record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    kms = np.array([s.elapsed_time(e) for s, e in zip(starts, ends)])
    log_steps(name, kms)

    st = int(status.item())
    if args.format == "bf16":
        ref = torch.from_numpy(np.concatenate([np.asarray(t).reshape(-1) for t in tensors])
                               .view(np.int16)).to(dev)
        exact = st == 0 and torch.equal(out.view(torch.int16), ref)
    else:
        ref = torch.from_numpy(np.concatenate([np.asarray(t).reshape(-1) for t in tensors])).to(dev)
        exact = st == 0 and torch.equal(out, ref)
    del ref
    payload = (8 if args.format == "bf16" else 4) + hs.total_bits / n
    total_bits = 8 * (sum(hs.compressed_bytes(cb).values())) / n
    return {
        "name": name, "n": n, "hs": hs, "cb": cb, "kernel_ms": kms, "wall_s": wall,
        "alg_bytes": alg, "exact": exact, "status": st, "payload_bpw": payload,
        "total_bpw": total_bits, "flushed": small, "settle": settled,
    }


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=100)
    ap.add_argument("--config", default="2")
    ap.add_argument("--tile-windows", type=int, default=64, choices=(64, 256, 512))
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--settle-ms", type=float, default=100.0,
                    help="keep the GPU busy this long before the warm-up steps (clock ramp)")
    ap.add_argument("--no-extra-configs", dest="extra_configs", action="store_false",
                    help="skip timing configs 0, 1, 2tp8, 405tp8, 3a-c after the 70B block")
    ap.add_argument("--copy-bytes", type=int, default=0,
                    help="time a plain device-to-device copy of this many bytes instead "
                         "(the achievable-bandwidth reference and the counter calibration)")
    ap.add_argument("--format", default="bf16", choices=("bf16", "fp8_e4m3", "fp8_e5m2"),
                    help="weight format of the workload (FP8: the BF16 workload quantized "
                         "with a per-tensor scale)")
    ap.add_argument("--encode", action="store_true",
                    help="time the GPU-side encoder (and the host encoder) on the workload instead")
    ap.add_argument("--pipeline", action="store_true",
                    help="time the overlapped block pipeline with a GEMV consumer over the "
                         "32 blocks of the 8B model instead")
    ap.add_argument("--fused", action="store_true",
                    help="time the fused decode + GEMV on the workload's block against "
                         "decompression followed by a GEMV, and a GEMV on resident BF16")
    ap.add_argument("--fused-gemm", action="store_true",
                    help="time the fused decode + GEMM (matrix cores) on the workload's block "
                         "against decompression followed by a library GEMM")
    ap.add_argument("--tokens", type=int, default=64, choices=(16, 32, 48, 64),
                    help="tokens for --fused-gemm")
    ap.add_argument("--batch", type=int, default=512,
                    help="vectors of the --pipeline GEMM consumer")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py measures one GPU: the decoder needs no cross-GPU exchange (each GPU "
              f"decompresses its own shard); --gpus {args.gpus} is not supported.",
              file=sys.stderr)
        sys.exit(2)

    import torch

    import entropy_decoding_amd as ed
    import synth_weights as sw

    assert torch.cuda.is_available(), "bench.py needs a ROCm GPU"
    if args.copy_bytes:
        return copy_reference(args, torch)
    if args.pipeline:
        return pipeline_bench(args, torch, ed, sw)
    if args.encode:
        return encode_bench(args, torch, ed, sw)
    if args.fused:
        return fused_bench(args, torch, ed, sw)
    if args.fused_gemm:
        return fused_gemm_bench(args, torch, ed, sw)
    if args.format != "bf16" and (args.tile_windows != 64 or args.config in ("4",)):
        print("FP8 workloads use 64-window tiles and single-unit configs", file=sys.stderr)
        sys.exit(2)
    cfg = sw.config(args.config)
    if len(cfg.units) != 1:
        return stream_units(cfg, args, torch, ed, sw)
    unit = cfg.units[0]
    tensors, workload = gen_workload(unit, cfg, args, sw)
    r = run_unit(workload, tensors, args, torch, ed)
    out_bytes = 2 if args.format == "bf16" else 1
    kms = r["kernel_ms"]
    avg_ms = float(kms.mean())
    n = r["n"]
    achieved = r["alg_bytes"] / (avg_ms * 1e-3) / 1e9
    if r["flushed"]:
        value = out_bytes * n * args.steps / (kms.sum() * 1e-3) / 1e9  # flush kernels excluded
    else:
        value = out_bytes * n * args.steps / r["wall_s"] / 1e9
    traffic = measured_traffic(workload, args.tile_windows)
    line = {
        "metric": "decompressed BF16 GB/s" if args.format == "bf16" else "decompressed FP8 GB/s",
        "value": round(value, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(r["wall_s"] * 1e3 / args.steps if not r["flushed"] else avg_ms, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": args.format,
        "data": "synthetic",
        "config": {
            "workload": workload,
            "n_weights": n,
            "layout": f"T{args.tile_windows}xB8",
            "arithmetic": "integer (bit-exact decode; no floating point)",
            "bit_exact": bool(r["exact"]),
            "bits_per_weight_payload": round(r["payload_bpw"], 4),
            "bits_per_weight_total": round(r["total_bpw"], 4),
            "size_vs_original": round(r["total_bpw"] / (8 * out_bytes), 4),
            "kernel_ms_p50": round(float(np.percentile(kms, 50)), 4),
            "kernel_ms_p99": round(float(np.percentile(kms, 99)), 4),
            "caches_flushed_between_steps": r["flushed"],
            "settle_before_warmup": r["settle"],
        },
        "roofline": {
            "bound": "hbm",
            "achieved": round(achieved, 1),
            "peak": HBM_PEAK_GBS,
            "unit": "GB/s",
            "frac": round(achieved / HBM_PEAK_GBS, 4),
            "traffic": traffic,
        },
        "system": system_info(torch),
    }
    line["copy_reference"] = copy_context(torch, int(r["alg_bytes"]), achieved)
    del r
    if args.extra_configs and args.config == "2" and args.format == "bf16":
        line["other_configs"] = other_configs(args, torch, ed, sw)
    if not args.no_cpu_baseline and args.format == "bf16":
        log("[bench] timing the CPU oracle")
        line["cpu_baseline"] = cpu_baseline(tensors)
    print(json.dumps(line), flush=True)
    if not line["config"]["bit_exact"] or not all(
            c["bit_exact"] for c in line.get("other_configs", {}).values()):
        sys.exit(1)


def gen_workload(unit, cfg, args, sw):
    t0 = time.perf_counter()
    if args.format == "bf16":
        tensors = sw.gen_unit(unit)
        workload = cfg.name
    else:
        tensors = sw.gen_unit_fp8(unit, args.format.split("_")[1])
        workload = f"{cfg.name}_{args.format}"
    log(f"[bench] generated {workload} ({unit.numel} weights) in {time.perf_counter() - t0:.1f} s")
    return tensors, workload


def system_info(torch) -> dict:
    p = torch.cuda.get_device_properties(0)
    return {"gpu": p.name, "arch": getattr(p, "gcnArchName", ""), "cus": p.multi_processor_count,
            "torch": torch.__version__, "hip": getattr(torch.version, "hip", None)}


def other_configs(args, torch, ed, sw) -> dict:
    """The single-unit configurations besides the 70B block, in the same
    process after it: each timed like the headline (settle, warm-up, timed
    steps with the caches evicted between steps) and compared with the
    original bits."""
    res = {}
    for k in ("0", "1", "2tp8", "405tp8", "3a", "3b", "3c"):
        cfg = sw.config(k)
        unit = cfg.units[0]
        tensors, name = gen_workload(unit, cfg, args, sw)
        r = run_unit(name, tensors, args, torch, ed)
        kms = r["kernel_ms"]
        ach = r["alg_bytes"] / (float(kms.mean()) * 1e-3) / 1e9
        res[name] = {
            "n_weights": r["n"], "bit_exact": bool(r["exact"]),
            "bf16_out_gbs": round(2 * r["n"] / (float(kms.mean()) * 1e-3) / 1e9, 1),
            "kernel_ms_p50": round(float(np.percentile(kms, 50)), 4),
            "kernel_ms_p99": round(float(np.percentile(kms, 99)), 4),
            "frac": round(ach / HBM_PEAK_GBS, 4),
            "bits_per_weight_payload": round(r["payload_bpw"], 4),
            "bits_per_weight_total": round(r["total_bpw"], 4),
            "caches_flushed_between_steps": r["flushed"],
        }
        del r, tensors
        torch.cuda.empty_cache()
    return res


def copy_context(torch, alg_bytes: int, achieved_gbs: float, steps: int = 20) -> dict:
    """Context for the roofline: a plain device-to-device copy (torch's copy
    kernel) that moves the decoder's algorithmic bytes per launch, half read
    and half written, timed with HIP events in the same process.  The
    denominator of `frac` stays the 8 TB/s peak."""
    n = alg_bytes // 8  # int32 elements per buffer: 4 B read + 4 B written each
    src = torch.ones(n, dtype=torch.int32, device="cuda")
    dst = torch.empty_like(src)
    stream = torch.cuda.current_stream()
    for _ in range(5):
        dst.copy_(src)
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
          for _ in range(steps)]
    for a, b in ev:
        a.record(stream)
        dst.copy_(src)
        b.record(stream)
    torch.cuda.synchronize()
    ms = np.array([a.elapsed_time(b) for a, b in ev])
    gbs = 8 * n / (float(ms.mean()) * 1e-3) / 1e9
    del src, dst
    torch.cuda.empty_cache()
    return {"bytes_moved": 8 * n, "ms_mean": round(float(ms.mean()), 4), "gbs": round(gbs, 1),
            "decoder_vs_copy": round(achieved_gbs / gbs, 4)}


def copy_reference(args, torch):
    """A plain copy: reads and writes copy_bytes each launch."""
    n = args.copy_bytes // 4
    src = torch.ones(n, dtype=torch.int32, device="cuda")
    dst = torch.empty_like(src)
    stream = torch.cuda.current_stream()
    for _ in range(args.warmup):
        dst.copy_(src)
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
          for _ in range(args.steps)]
    torch.cuda.synchronize()
    for a, b in ev:
        a.record(stream)
        dst.copy_(src)
        b.record(stream)
    torch.cuda.synchronize()
    ms = np.array([a.elapsed_time(b) for a, b in ev])
    moved = 2 * 4 * n
    print(json.dumps({"metric": "device copy GB/s (read + write)",
                      "value": round(moved / (ms.mean() * 1e-3) / 1e9, 1), "unit": "GB/s",
                      "bytes_read_per_launch": 4 * n, "bytes_written_per_launch": 4 * n,
                      "ms_mean": round(float(ms.mean()), 4), "steps": args.steps}), flush=True)


def stream_units(cfg, args, torch, ed, sw):
    """Several units: each compressed unit resident in HBM, decompressed in
    order into one reused output buffer; per-unit latency from HIP events."""
    dev = torch.device("cuda:0")
    units = []
    t0 = time.perf_counter()
    for unit in cfg.units:
        tensors = sw.gen_unit(unit)
        cb = ed.df11_build_codebook(tensors)
        hs = ed.df11_encode(cb, tensors, args.tile_windows, 8)
        ds = ed.DeviceStream(hs, cb, dev)
        ref_hash = None
        units.append((unit, ds, hs, cb, tensors if cfg.index != 4 else None))
        log(f"[bench] {unit.name}: {hs.n_weights} weights resident "
            f"({time.perf_counter() - t0:.0f} s)")
        del tensors, ref_hash
    nmax = max(u[2].n_weights for u in units)
    out = torch.empty(nmax, dtype=torch.bfloat16, device=dev)
    status = torch.zeros(1, dtype=torch.int32, device=dev)
    stream = torch.cuda.current_stream()
    # a unit is read again only after the rest of the pass: when a whole pass
    # moves under 1 GiB, its data could still sit in the 256 MB last-level
    # cache, so the caches are evicted before every launch by reading 1 GiB
    # (outside the timed events), as for the single-unit configs
    pass_bytes = sum(algorithmic_bytes(u[2], u[3]) for u in units)
    flush = torch.zeros(1 << 28, dtype=torch.int32, device=dev) if pass_bytes < (1 << 30) else None
    sink = torch.zeros((), dtype=torch.int32, device=dev)
    settled = settle(lambda: ed.df11_decompress_block(units[0][1], out, status, stream), torch,
                     args.settle_ms)
    for _ in range(args.warmup):
        for u in units:
            ed.df11_decompress_block(u[1], out, status, stream)
    torch.cuda.synchronize()
    passes = max(1, args.steps)
    # the whole job: passes of back-to-back launches, nothing recorded between
    # them (events between launches add a few microseconds each)
    wall = None
    if flush is None:
        t0 = time.perf_counter()
        for p in range(passes):
            for u in units:
                ed.df11_decompress_block(u[1], out, status, stream)
        torch.cuda.synchronize()
        wall = time.perf_counter() - t0
    # per-unit latency: the same passes with HIP events around every launch
    ev = [[(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
           for _ in units] for _ in range(passes)]
    t0 = time.perf_counter()
    for p in range(passes):
        for i, u in enumerate(units):
            if flush is not None:
                torch.amax(flush, dim=0, out=sink)
            ev[p][i][0].record(stream)
            ed.df11_decompress_block(u[1], out, status, stream)
            ev[p][i][1].record(stream)
    torch.cuda.synchronize()
    instrumented_wall = time.perf_counter() - t0
    lat = np.array([[a.elapsed_time(b) for a, b in row] for row in ev])
    n_total = sum(u[2].n_weights for u in units)
    alg = sum(algorithmic_bytes(u[2], u[3]) for u in units)
    # bit-exactness: every unit once more, compared with regenerated originals
    exact = int(status.item()) == 0
    for unit, ds, hs, cb, tensors in units:
        if tensors is None:
            tensors = sw.gen_unit(unit)
        ed.df11_decompress_block(ds, out, status, stream)
        ref = torch.from_numpy(np.concatenate([t.reshape(-1) for t in tensors]).view(np.int16))
        exact &= torch.equal(out[: hs.n_weights].view(torch.int16).cpu(), ref)
    exact &= int(status.item()) == 0
    blocks = lat[:, [i for i, u in enumerate(units) if u[0].name.startswith("block")]]
    avg_pass_ms = float(lat.sum(axis=1).mean())
    achieved = alg / (avg_pass_ms * 1e-3) / 1e9
    # with flushes in between, the job's time is the sum of the launches' times
    job_s = float(lat.sum()) * 1e-3 if flush is not None else wall
    line = {
        "metric": "decompressed BF16 GB/s",
        "value": round(2 * n_total * passes / job_s / 1e9, 2),
        "unit": "GB/s", "n_gpus": 1, "steps": passes, "warmup": args.warmup,
        "ms_per_step": round(job_s * 1e3 / passes, 4), "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
        "config": {
            "workload": cfg.name, "n_weights": n_total, "units": len(units),
            "layout": f"T{args.tile_windows}xB8", "bit_exact": bool(exact),
            "unit_ms_p50": round(float(np.percentile(lat, 50)), 4),
            "unit_ms_p99": round(float(np.percentile(lat, 99)), 4),
            "block_ms_p50": round(float(np.percentile(blocks, 50)), 4) if blocks.size else None,
            "block_ms_p99": round(float(np.percentile(blocks, 99)), 4) if blocks.size else None,
            "per_unit_ms_mean": {u[0].name: round(float(lat[:, i].mean()), 4)
                                 for i, u in enumerate(units)},
            "caches_flushed_between_steps": flush is not None,
            "settle_before_warmup": settled,
            "ms_per_pass_with_events": round(instrumented_wall * 1e3 / passes, 4),
        },
        "roofline": {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS,
                     "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": None},
    }
    print(json.dumps(line), flush=True)
    if not exact:
        sys.exit(1)


def encode_bench(args, torch, ed, sw):
    """The GPU-side encoder on a single-unit workload: device histogram, host
    codebook from it, device encode; timed with HIP events on one stream, the
    host encoder timed beside it.  Output arrays are compared with the host's."""
    import ctypes

    dev = torch.device("cuda:0")
    cfg = sw.config(args.config)
    unit = cfg.units[0]
    fmt = args.format
    tensors = sw.gen_unit(unit) if fmt == "bf16" else sw.gen_unit_fp8(unit, fmt.split("_")[1])
    flat = np.concatenate([t.reshape(-1) for t in tensors])
    n = flat.size
    w = torch.from_numpy(flat.view(np.int16) if fmt == "bf16" else flat).to(dev)
    stream = torch.cuda.current_stream()
    # sizes and buffers once (the codebook is the same for every step)
    counts = ed.df11_histogram_device(w, fmt).cpu().numpy().view(np.uint64)
    t0 = time.perf_counter()
    cb = ed.df11_build_codebook_from_counts(counts)
    codebook_ms = (time.perf_counter() - t0) * 1e3
    sz = ed.df11_sizes()
    ed._check("df11_encode_size_from_counts", ed.LIB.df11_encode_size_from_counts(
        ed.FORMATS[fmt], ctypes.byref(cb), counts.ctypes.data_as(ctypes.POINTER(ctypes.c_uint64)),
        n, args.tile_windows, 8, ctypes.byref(sz)))
    bufs = [torch.empty(x, dtype=torch.uint8, device=dev)
            for x in (sz.stream_bytes, sz.sm_bytes, max(16, sz.n_windows), 4 * sz.bop_entries, 16)]
    nscratch = int(ed.LIB.df11_encode_device_scratch_bytes(n))
    scratch = torch.empty(nscratch, dtype=torch.uint8, device=dev)
    out = ed.df11_device_encode(*[b.data_ptr() for b in bufs], scratch.data_ptr(), nscratch)
    cnt = torch.empty(256, dtype=torch.int64, device=dev)
    sh = ctypes.c_void_p(stream.cuda_stream)

    def hist():
        ed._check("df11_histogram_device", ed.LIB.df11_histogram_device(
            ed.FORMATS[fmt], ctypes.c_void_p(w.data_ptr()), n, ctypes.c_void_p(cnt.data_ptr()), sh))

    def enc():
        ed._check("df11_encode_device", ed.LIB.df11_encode_device(
            ed.FORMATS[fmt], ctypes.byref(cb), ctypes.c_void_p(w.data_ptr()), n, args.tile_windows,
            8, ctypes.byref(sz), ctypes.byref(out), sh))

    settle(lambda: (hist(), enc()), torch, args.settle_ms)
    for _ in range(max(1, min(args.warmup, 10))):
        hist()
        enc()
    torch.cuda.synchronize()
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(args.steps)]
    for a, b, c in ev:
        a.record(stream)
        hist()
        b.record(stream)
        enc()
        c.record(stream)
    torch.cuda.synchronize()
    h_ms = np.array([a.elapsed_time(b) for a, b, _ in ev])
    e_ms = np.array([b.elapsed_time(c) for _, b, c in ev])
    t0 = time.perf_counter()
    hcb = ed.df11_build_codebook(tensors, fmt)
    hs = ed.df11_encode(hcb, tensors, args.tile_windows, 8, fmt)
    host_ms = (time.perf_counter() - t0) * 1e3
    exact = (np.array_equal(bufs[0].cpu().numpy(), hs.stream)
             and np.array_equal(bufs[1].cpu().numpy(), hs.sm)
             and np.array_equal(bufs[2].cpu().numpy()[: hs.gaps.size], hs.gaps)
             and np.array_equal(bufs[3].cpu().numpy().view(np.uint32), hs.block_out_pos)
             and int(bufs[4][:4].cpu().numpy().view(np.uint32)[0]) == hs.max_tile_symbols)
    total_ms = float(h_ms.mean() + e_ms.mean())
    in_bytes = n * (2 if fmt == "bf16" else 1)
    # the encode call (the larger share): weights read once, compressed arrays
    # (stream, sign+mantissa, gaps, block_out_pos) written once
    enc_alg = in_bytes + (hs.total_bits + 7) // 8 + hs.sm.size + hs.gaps.size + 4 * hs.block_out_pos.size
    enc_ach = enc_alg / (float(e_ms.mean()) * 1e-3) / 1e9
    line = {
        "metric": "GPU encode GB/s (input weights)", "value": round(in_bytes / (total_ms * 1e-3) / 1e9, 2),
        "unit": "GB/s", "n_gpus": 1, "steps": args.steps, "higher_is_better": True,
        "dtype": fmt, "data": "synthetic",
        "config": {"workload": cfg.name if fmt == "bf16" else f"{cfg.name}_{fmt}", "n_weights": n,
                   "layout": f"T{args.tile_windows}xB8", "byte_exact_vs_host_encoder": bool(exact)},
        "device_ms": {"histogram": round(float(h_ms.mean()), 4), "encode": round(float(e_ms.mean()), 4),
                      "codebook_on_host": round(codebook_ms, 3)},
        "host_encoder_ms": round(host_ms, 1),
        "roofline": {"bound": "hbm", "achieved": round(enc_ach, 1), "peak": HBM_PEAK_GBS,
                     "unit": "GB/s", "frac": round(enc_ach / HBM_PEAK_GBS, 4),
                     "bytes_per_launch": int(enc_alg), "kernel": "df11_encode_device (all launches)"},
    }
    print(json.dumps(line), flush=True)
    if not exact:
        sys.exit(1)


def pipeline_bench(args, torch, ed, sw):
    """The 32 transformer blocks of the 8B model, each consumed by the model's
    matrix products on its 7 weight matrices, with the next block decompressed
    on a second stream into the other of two buffers (df11_pipeline_*).

    Two consumers: this library's BF16 GEMV (one fp32 vector, memory-bound like
    decoding one token) and a plain library BF16 GEMM over --batch vectors
    (torch.mm, compute-bound like a prefill chunk).  Times per block:
    decompression alone, the consumer alone on resident BF16 weights, both in
    sequence on one stream, and both overlapped."""
    import oracle

    dev = torch.device("cuda:0")
    cfg = sw.config("4")
    units = [u for u in cfg.units if u.name.startswith("block")]
    shapes = [shape for _, shape in units[0].tensors]
    blocks = []
    t0 = time.perf_counter()
    for unit in units:
        tensors = sw.gen_unit(unit)
        cb = ed.df11_build_codebook(tensors)
        hs = ed.df11_encode(cb, tensors, args.tile_windows, 8)
        blocks.append((unit, ed.DeviceStream(hs, cb, dev), hs, cb))
        del tensors
    log(f"[bench] pipeline: {len(blocks)} blocks resident ({time.perf_counter() - t0:.0f} s)")
    n = blocks[0][2].n_weights
    nb = len(blocks)
    bufs = [torch.empty(n, dtype=torch.bfloat16, device=dev) for _ in range(2)]
    status = torch.zeros(1, dtype=torch.int32, device=dev)
    main_s = torch.cuda.current_stream()
    decode_s, compute_s = torch.cuda.Stream(), torch.cuda.Stream()
    rng = np.random.default_rng(4)
    offs = np.cumsum([0] + [r * c for r, c in shapes])

    # consumer 1: GEMV, y = W x in fp32
    layout = ed.gemv_layout(shapes)
    x = torch.from_numpy(rng.standard_normal(layout[2]).astype(np.float32)).to(dev)
    y_pipe = [torch.zeros(layout[3], dtype=torch.float32, device=dev) for _ in blocks]
    y_seq = [torch.zeros(layout[3], dtype=torch.float32, device=dev) for _ in blocks]

    def gemv(buf, i, out):
        ed.df11_gemv_bf16(buf, layout, x, out[i], torch.cuda.current_stream())

    # consumer 2: GEMM over a batch of BF16 vectors (library GEMM; 512 by default)
    batch = args.batch
    xb = [torch.from_numpy(rng.standard_normal((c, batch)).astype(np.float32)).to(dev)
          .to(torch.bfloat16).contiguous() for _, c in shapes]
    ob = [torch.empty((r, batch), dtype=torch.bfloat16, device=dev) for r, _ in shapes]

    def gemm(buf, i, out):
        for k, (r, c) in enumerate(shapes):
            torch.mm(buf[offs[k]:offs[k + 1]].view(r, c), xb[k], out=ob[k])

    def run(consumer, out, pipelined, pipe=None):
        if not pipelined:
            for i, (_, ds, _, _) in enumerate(blocks):
                ed.df11_decompress_block(ds, bufs[0], status, main_s)
                consumer(bufs[0], i, out)
            return
        pipe.decompress(0, blocks[0][1], bufs[0], status)
        for i in range(nb):
            if i + 1 < nb:
                pipe.decompress((i + 1) % 2, blocks[i + 1][1], bufs[(i + 1) % 2], status)
            pipe.acquire(i % 2, compute_s)
            with torch.cuda.stream(compute_s):
                consumer(bufs[i % 2], i, out)
            pipe.release(i % 2, compute_s)

    def timed(fn, passes):
        for _ in range(max(1, min(args.warmup, 3))):
            fn()
        torch.cuda.synchronize()
        t = time.perf_counter()
        for _ in range(passes):
            fn()
        torch.cuda.synchronize()
        return (time.perf_counter() - t) * 1e3 / (passes * nb)

    passes = max(1, args.steps // 5)
    settle(lambda: ed.df11_decompress_block(blocks[0][1], bufs[0], status, main_s), torch,
           args.settle_ms)
    pipe = ed.Pipeline(decode_s, 2)
    for _, ds, _, _ in blocks[:2]:
        ed.df11_decompress_block(ds, bufs[0], status, main_s)
    ms_decode = timed(lambda: [ed.df11_decompress_block(b[1], bufs[0], status, main_s)
                               for b in blocks], passes)
    results = {}
    shares = (0, 1, 2, 3, 4)  # decode workgroups per compute unit (0: the full grid)
    for name, consumer in (("gemv_b1", gemv), (f"gemm_b{batch}", gemm)):
        alone = timed(lambda: [consumer(bufs[i % 2], i, y_seq) for i in range(nb)], passes)
        seq = timed(lambda: run(consumer, y_seq, False), passes)
        by_share = {}
        for sh in shares:
            pipe.set_decode_share(sh)
            by_share[sh] = timed(lambda: run(consumer, y_pipe, True, pipe), passes)
        best = min(by_share, key=by_share.get)
        pip = by_share[best]
        results[name] = {"decode_ms": round(ms_decode, 4), "consumer_ms": round(alone, 4),
                         "sequential_ms": round(seq, 4), "pipelined_ms": round(pip, 4),
                         "decode_share_best": best,
                         "pipelined_ms_by_decode_share": {str(k): round(v, 4) for k, v in by_share.items()},
                         "pipelined_vs_slower_kernel": round(pip / max(ms_decode, alone), 4),
                         "overlap_saving": round(1 - pip / seq, 4),
                         "hidden_fraction_of_decode": round((ms_decode + alone - pip) / ms_decode, 4)}
        log(f"[bench] pipeline {name}: decode {ms_decode:.4f} consumer {alone:.4f} sequential "
            f"{seq:.4f} pipelined by share {by_share}")
    pipe.set_decode_share(0)
    pipe.close()

    # the pipelined GEMV results equal the one-stream results bit for bit, and
    # sampled rows of block 0 agree with the oracle's float64 product
    run(gemv, y_seq, False)
    torch.cuda.synchronize()  # the pipelined run below reuses bufs[0] from other streams
    exact = int(status.item()) == 0
    for sh in sorted({0, results[f"gemm_b{batch}"]["decode_share_best"]}):
        for y in y_pipe:
            y.zero_()
        pipe = ed.Pipeline(decode_s, 2)
        pipe.set_decode_share(sh)
        run(gemv, y_pipe, True, pipe)
        torch.cuda.synchronize()
        pipe.close()
        exact &= int(status.item()) == 0 and all(torch.equal(a, b) for a, b in zip(y_pipe, y_seq))
    tensors = sw.gen_unit(units[0])
    xh = x.cpu().numpy()
    y0 = y_seq[0].cpu().numpy().astype(np.float64)
    xo = yo = 0
    for (rows, cols), w in zip(shapes, tensors):
        r = np.unique(np.linspace(0, rows - 1, 64).astype(np.int64))
        W = w.reshape(rows, cols)[r]
        ref = oracle.gemv(W.reshape(-1), [(r.size, cols)], xh[xo:xo + cols])
        d = -(-cols // 64) + 6
        bound = d * 2.0 ** -24 / (1 - d * 2.0 ** -24) * (
            np.abs(oracle.bf16_to_f64(W.reshape(-1))).reshape(r.size, cols) @ np.abs(xh[xo:xo + cols]))
        exact &= bool(np.all(np.abs(y0[yo + r] - ref) <= bound + 1e-30))
        xo += cols
        yo += rows
    dec_bytes = algorithmic_bytes(blocks[0][2], blocks[0][3])
    gemv_bytes = 2 * n + 4 * (layout[2] + layout[3])
    g = results["gemv_b1"]
    achieved = (dec_bytes + gemv_bytes) / (g["pipelined_ms"] * 1e-3) / 1e9
    gm = results[f"gemm_b{batch}"]
    line = {
        "metric": f"pipelined block time (decompress the next block while a GEMM over {batch} "
                  "vectors reads this one)",
        "value": gm["pipelined_ms"], "unit": "ms per block", "n_gpus": 1,
        "steps": passes, "warmup": max(1, min(args.warmup, 3)), "higher_is_better": False,
        "vs_baseline": None, "dtype": "bf16 decode + f32 GEMV", "data": "synthetic",
        "config": {"workload": "llama3_8b_32_blocks", "blocks": nb, "n_weights_per_block": n,
                   "slots": 2, "layout": f"T{args.tile_windows}xB8", "bit_exact": bool(exact)},
        "consumers": results,
        "roofline": {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS,
                     "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4),
                     "bytes_per_block": dec_bytes + gemv_bytes},
    }
    print(json.dumps(line), flush=True)
    if not exact:
        sys.exit(1)


def fused_bench(args, torch, ed, sw):
    """One block's matrix-vector products y = W x (fp32 x and y) three ways:
    the fused kernel reading only the compressed block (df11_decompress_gemv),
    decompression to BF16 followed by the GEMV (two launches), and the GEMV on
    resident BF16 weights.  Times are HIP events on the launch stream; caches
    are evicted between steps when the block fits in them."""
    import oracle

    if args.format != "bf16" or args.tile_windows != 64:
        print("the fused GEMV takes BF16 units with 64-window tiles", file=sys.stderr)
        sys.exit(2)
    dev = torch.device("cuda:0")
    cfg = sw.config(args.config)
    unit = cfg.units[0]
    shapes = [shape for _, shape in unit.tensors]
    tensors = sw.gen_unit(unit)
    cb = ed.df11_build_codebook(tensors)
    hs = ed.df11_encode(cb, tensors, 64, 8)
    ds = ed.DeviceStream(hs, cb, dev)
    n = hs.n_weights
    layout = ed.gemv_layout(shapes)
    rng = np.random.default_rng(5)
    xh = rng.standard_normal(layout[2]).astype(np.float32)
    x = torch.from_numpy(xh).to(dev)
    y_f = torch.zeros(layout[3], dtype=torch.float32, device=dev)
    y_s = torch.zeros_like(y_f)
    y_r = torch.zeros_like(y_f)
    w_res = torch.from_numpy(np.concatenate(tensors).view(np.int16)).to(dev)
    buf = torch.empty(n, dtype=torch.int16, device=dev)
    status = torch.zeros(1, dtype=torch.int32, device=dev)
    scratch = torch.empty(int(ed.LIB.df11_decompress_gemv_scratch_bytes(ed.ctypes.byref(ds.desc))),
                          dtype=torch.uint8, device=dev)
    stream = torch.cuda.current_stream()
    dec_bytes = algorithmic_bytes(hs, cb)
    read_bytes = dec_bytes - 2 * n
    vec_bytes = 4 * (layout[2] + layout[3])
    small = dec_bytes < (1 << 30)
    flush = torch.zeros(1 << 28, dtype=torch.int32, device=dev) if small else None
    sink = torch.zeros((), dtype=torch.int32, device=dev)

    def fused():
        ed.df11_decompress_gemv(ds, layout, x, y_f, scratch, status, stream)

    def sequential():
        ed.df11_decompress_block(ds, buf, status, stream)
        ed.df11_gemv_bf16(buf, layout, x, y_s, stream)

    def resident():
        ed.df11_gemv_bf16(w_res, layout, x, y_r, stream)

    def timed(fn):
        for _ in range(args.warmup):
            fn()
        torch.cuda.synchronize()
        ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
              for _ in range(args.steps)]
        for a, b in ev:
            if flush is not None:
                torch.amax(flush, dim=0, out=sink)
            a.record(stream)
            fn()
            b.record(stream)
        torch.cuda.synchronize()
        return np.array([a.elapsed_time(b) for a, b in ev])

    settle(fused, torch, args.settle_ms)
    res = {name: timed(fn) for name, fn in
           (("fused", fused), ("decompress_then_gemv", sequential), ("bf16_gemv", resident))}
    ok = int(status.item()) == 0 and torch.equal(buf, w_res)
    # sampled rows of every matrix against the oracle's float64 product, within
    # the rounding bound of each kernel's summation order
    yf, ys = y_f.cpu().numpy().astype(np.float64), y_s.cpu().numpy().astype(np.float64)
    bop = hs.block_out_pos.astype(np.int64)
    passes = -(-(int(hs.max_tile_symbols) // 8 + 2) // 64)
    u = 2.0 ** -24
    off = xo = yo = 0
    for (rows, cols), w in zip(shapes, tensors):
        r = np.unique(np.linspace(0, rows - 1, 64).astype(np.int64))
        W = w.reshape(rows, cols)[r].reshape(-1)
        ref = oracle.gemv(W, [(r.size, cols)], xh[xo:xo + cols])
        absum = np.abs(oracle.bf16_to_f64(W)).reshape(r.size, cols) @ np.abs(xh[xo:xo + cols])
        starts = off + r * cols
        tiles = (np.searchsorted(bop, starts + cols - 1, side="right")
                 - np.searchsorted(bop, starts, side="right") + 1)
        df = 9 * passes + 2 + 7 + tiles  # the fused kernel's summation depth
        ds_ = -(-cols // 64) + 6
        ok &= bool(np.all(np.abs(yf[yo + r] - ref) <= df * u / (1 - df * u) * absum + 1e-30))
        ok &= bool(np.all(np.abs(ys[yo + r] - ref) <= ds_ * u / (1 - ds_ * u) * absum + 1e-30))
        off += rows * cols
        xo += cols
        yo += rows
    f = res["fused"]
    achieved = (read_bytes + vec_bytes) / (f.mean() * 1e-3) / 1e9
    line = {
        "metric": "fused decompress+GEMV time per block",
        "value": round(float(f.mean()), 4), "unit": "ms per block", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "higher_is_better": False,
        "vs_baseline": None, "dtype": "bf16 x f32 -> f32", "data": "synthetic",
        "config": {"workload": cfg.name, "n_weights": n, "layout": "T64xB8",
                   "within_rounding_bound": bool(ok), "caches_flushed_between_steps": small},
        "ms": {k: {"mean": round(float(v.mean()), 4), "p50": round(float(np.percentile(v, 50)), 4)}
               for k, v in res.items()},
        "speedup_vs_decompress_then_gemv": round(float(res["decompress_then_gemv"].mean() / f.mean()), 3),
        "speedup_vs_bf16_gemv": round(float(res["bf16_gemv"].mean() / f.mean()), 3),
        "roofline": {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS,
                     "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4),
                     "bytes_per_launch": read_bytes + vec_bytes},
    }
    print(json.dumps(line), flush=True)
    if not ok:
        sys.exit(1)


def fused_gemm_bench(args, torch, ed, sw):
    """One block's products Y_k = X_k W_k^T for n tokens (BF16 X, float32 Y)
    three ways: the fused kernel on the matrix cores reading only the
    compressed block (encoded in GEMM order), decompression to BF16 followed by
    a library GEMM per matrix (torch.mm, BF16 out), and that GEMM on resident
    BF16 weights.  HIP events on the launch stream; caches evicted between
    steps when the block fits in them."""
    import oracle

    dev = torch.device("cuda:0")
    n = args.tokens
    cfg = sw.config(args.config)
    unit = cfg.units[0]
    shapes = [shape for _, shape in unit.tensors]
    tensors = sw.gen_unit(unit)
    t0 = time.perf_counter()
    ordered = [ed.df11_gemm_order(t, r, c) for t, (r, c) in zip(tensors, shapes)]
    cbg = ed.df11_build_codebook(ordered)
    hsg = ed.df11_encode(cbg, ordered, 64, 8)
    dsg = ed.DeviceStream(hsg, cbg, dev)
    del ordered
    cb = ed.df11_build_codebook(tensors)
    hs = ed.df11_encode(cb, tensors, 64, 8)
    ds = ed.DeviceStream(hs, cb, dev)
    log(f"[bench] fused gemm: {cfg.name} encoded twice (GEMM and row order) in "
        f"{time.perf_counter() - t0:.1f} s, {hsg.n_tiles} tiles")
    nw = hs.n_weights
    layout = ed.gemm_layout(shapes, n)
    rng = np.random.default_rng(6)
    xh = ((rng.standard_normal(layout[2]).astype(np.float32).view(np.uint32) >> 16)
          .astype(np.uint16))
    x = torch.from_numpy(xh.view(np.int16)).to(dev)
    y_f = torch.zeros(layout[3], dtype=torch.float32, device=dev)
    status = torch.zeros(1, dtype=torch.int32, device=dev)
    buf = torch.empty(nw, dtype=torch.bfloat16, device=dev)
    w_res = torch.from_numpy(np.concatenate(tensors).view(np.int16)).to(dev).view(torch.bfloat16)
    offs = np.cumsum([0] + [r * c for r, c in shapes])
    xoffs = np.cumsum([0] + [n * c for _, c in shapes])
    xb = x.view(torch.bfloat16)
    xs = [xb[xoffs[k]:xoffs[k + 1]].view(n, c) for k, (_, c) in enumerate(shapes)]
    outs = [torch.empty((n, r), dtype=torch.bfloat16, device=dev) for r, _ in shapes]
    stream = torch.cuda.current_stream()
    # compressed unit read once, activations read once, products written once
    alg = algorithmic_bytes(hsg, cbg) - 2 * nw + 2 * layout[2] + 4 * layout[3]
    small = algorithmic_bytes(hs, cb) < (1 << 30)
    flush = torch.zeros(1 << 28, dtype=torch.int32, device=dev) if small else None
    sink = torch.zeros((), dtype=torch.int32, device=dev)

    scratch = torch.empty(ed.df11_decompress_gemm_scratch_bytes(layout, n), dtype=torch.uint8,
                          device=dev)

    def fused():
        ed.df11_decompress_gemm(dsg, layout, n, x, y_f, scratch, status, stream)

    def mm(wbuf):
        for k, (r, c) in enumerate(shapes):
            torch.mm(xs[k], wbuf[offs[k]:offs[k + 1]].view(r, c).t(), out=outs[k])

    def sequential():
        ed.df11_decompress_block(ds, buf, status, stream)
        mm(buf)

    def resident():
        mm(w_res)

    def timed(fn):
        for _ in range(args.warmup):
            fn()
        torch.cuda.synchronize()
        ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
              for _ in range(args.steps)]
        for a, b in ev:
            if flush is not None:
                torch.amax(flush, dim=0, out=sink)
            a.record(stream)
            fn()
            b.record(stream)
        torch.cuda.synchronize()
        return np.array([a.elapsed_time(b) for a, b in ev])

    settle(fused, torch, args.settle_ms)
    res = {name: timed(fn) for name, fn in
           (("fused", fused), ("decompress_then_gemm", sequential), ("bf16_gemm", resident))}
    ok = int(status.item()) == 0 and torch.equal(buf.view(torch.int16), w_res.view(torch.int16))
    # sampled rows of every matrix against the oracle's float64 product, within
    # a bound that assumes nothing about the matrix cores' order of additions
    yf = y_f.cpu().numpy().astype(np.float64)
    u = 2.0 ** -24
    yo = 0
    for k, ((r, c), w) in enumerate(zip(shapes, tensors)):
        rows = np.unique(np.linspace(0, r - 1, 32).astype(np.int64))
        W = w.reshape(r, c)[rows]
        X = xh[xoffs[k]:xoffs[k + 1]]
        ref = oracle.gemm(W.reshape(-1), [(rows.size, c)], X, n).reshape(n, rows.size)
        d = c + c // 32 + 3
        bound = 2 * d * u / (1 - 2 * d * u) * (
            np.abs(oracle.bf16_to_f64(X)).reshape(n, c) @ np.abs(oracle.bf16_to_f64(W.reshape(-1)))
            .reshape(rows.size, c).T)
        got = yf[yo:yo + n * r].reshape(n, r)[:, rows]
        ok &= bool(np.all(np.abs(got - ref) <= bound + 1e-30))
        yo += n * r
    f = res["fused"]
    achieved = alg / (f.mean() * 1e-3) / 1e9
    flops = 2.0 * nw * n
    line = {
        "metric": "fused decompress+GEMM time per block",
        "value": round(float(f.mean()), 4), "unit": "ms per block", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "higher_is_better": False,
        "vs_baseline": None, "dtype": "bf16 x bf16 -> f32", "data": "synthetic",
        "config": {"workload": cfg.name, "n_weights": nw, "tokens": n, "layout": "T64xB8, GEMM order",
                   "within_rounding_bound": bool(ok), "caches_flushed_between_steps": small},
        "ms": {k: {"mean": round(float(v.mean()), 4), "p50": round(float(np.percentile(v, 50)), 4)}
               for k, v in res.items()},
        "speedup_vs_decompress_then_gemm": round(float(res["decompress_then_gemm"].mean() / f.mean()), 3),
        "speedup_vs_bf16_gemm": round(float(res["bf16_gemm"].mean() / f.mean()), 3),
        "matrix_core_tflops": round(flops / (f.mean() * 1e-3) / 1e12, 1),
        "roofline": {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS,
                     "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4),
                     "bytes_per_launch": int(alg)},
    }
    print(json.dumps(line), flush=True)
    if not ok:
        sys.exit(1)


if __name__ == "__main__":
    main()
