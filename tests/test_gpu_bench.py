"""bench.py on the GPU: the JSON line the benchmark prints keeps its contract
(the keys a reader of the line relies on, a bit-exact result, a roofline
fraction that the algorithmic bytes and the kernel time give), on the small
1024 x 1024 workload in BF16 and FP8."""

import json
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

pytestmark = pytest.mark.gpu


def _bench(*args):
    p = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--config", "0",
                        "--steps", "5", "--warmup", "2", "--settle-ms", "5", "--no-cpu-baseline",
                        *args], capture_output=True, text=True, timeout=300)
    assert p.returncode == 0, p.stderr[-3000:]
    lines = [l for l in p.stdout.splitlines() if l.startswith("{")]
    assert len(lines) == 1, p.stdout
    return json.loads(lines[0])


@pytest.mark.parametrize("fmt", ["bf16", "fp8_e4m3"])
def test_json_line_contract(fmt):
    print(f"[gpu] bench.py --config 0 --format {fmt}", flush=True)
    d = _bench("--format", fmt)
    for key in ("metric", "value", "unit", "n_gpus", "steps", "warmup", "ms_per_step",
                "higher_is_better", "scaling", "vs_baseline", "dtype", "data", "config",
                "roofline", "copy_reference", "system"):
        assert key in d, key
    assert d["n_gpus"] == 1 and d["steps"] == 5 and d["warmup"] == 2
    assert d["dtype"] == fmt and d["higher_is_better"] is True and d["value"] > 0
    c = d["config"]
    assert c["workload"].startswith("tensor_1024x1024") and c["bit_exact"] is True
    raw = 8 if fmt == "bf16" else 4  # sign and mantissa bits stored as they are
    assert c["n_weights"] == 1 << 20 and raw < c["bits_per_weight_payload"] < 2 * raw
    r = d["roofline"]
    assert r["bound"] == "hbm" and r["peak"] == 8000.0 and r["unit"] == "GB/s"
    assert 0 < r["frac"] < 1 and abs(r["frac"] - r["achieved"] / r["peak"]) < 1e-3
    cr = d["copy_reference"]
    assert cr["gbs"] > 0 and cr["bytes_moved"] > 0
    assert abs(cr["decoder_vs_copy"] - r["achieved"] / cr["gbs"]) < 1e-2 * cr["decoder_vs_copy"] + 1e-3
