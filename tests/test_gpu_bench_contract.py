"""bench.py's one JSON line, on a small workload: every field the contract
names is there with its type, the roofline object is complete, the CPU
baseline names its threads and host, and the numbers agree with each other
(value = shard elements / ms_per_step, frac = achieved / peak)."""

from __future__ import annotations

import json
import os
import subprocess
import sys

import pytest

pytestmark = pytest.mark.gpu

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.fixture(autouse=True)
def _need_gpu():
    import torch

    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def test_bench_line_contract():
    print("case bench contract gpt2-small-flat", flush=True)
    p = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--config",
                        "gpt2-small-flat", "--no-extra-configs", "--steps", "5", "--warmup", "2"],
                       capture_output=True, text=True, timeout=300, cwd=ROOT)
    assert p.returncode == 0, p.stderr[-2000:]
    lines = [ln for ln in p.stdout.splitlines() if ln.startswith("{")]
    assert len(lines) == 1, p.stdout
    d = json.loads(lines[0])
    for k, t in (("metric", str), ("value", float), ("unit", str), ("n_gpus", int),
                 ("steps", int), ("warmup", int), ("ms_per_step", float),
                 ("higher_is_better", bool), ("scaling", str), ("dtype", str), ("data", str),
                 ("config", dict), ("roofline", dict), ("cpu_baseline", dict)):
        assert isinstance(d[k], t), (k, d[k])
    assert "vs_baseline" in d and d["vs_baseline"] is None
    assert d["n_gpus"] == 1 and d["steps"] == 5 and d["warmup"] == 2
    assert d["higher_is_better"] is True and d["scaling"] in ("weak", "strong")
    assert d["config"]["workload"] == "gpt2-small-flat"
    n = d["config"]["shard_len"]
    assert abs(d["value"] - n / (d["ms_per_step"] * 1e-3)) <= 1e-6 * d["value"]
    r = d["roofline"]
    assert r["bound"] == "hbm" and r["unit"] == "GB/s" and r["peak"] == 8000.0
    assert 0.0 < r["achieved"] and abs(r["frac"] - r["achieved"] / r["peak"]) < 1e-4
    assert "traffic" in r
    c = d["cpu_baseline"]
    assert c["kind"] == "oracle" and c["value"] > 0 and c["cores"] >= 1
    assert c["host"]["nproc"] >= 1 and isinstance(c["sample"], str)
