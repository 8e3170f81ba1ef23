"""The boundary from plain C: tests/native/c_abi_step (built by
__graft_entry__.build(); no Python or PyTorch in its process) allocates with
hipMalloc, calls zero_shard_init / zero_shard_gnorm / zero_shard_step /
zero_shard_free (or captures zero_shard_gnorm_noalloc and
zero_shard_step_dev into one HIP graph and replays it), and writes its
outputs; they are compared with the oracle
on the same seeded inputs, to the parity tolerances."""

from __future__ import annotations

import os
import subprocess
import sys

import numpy as np
import pytest

import oracle as O
import seeded_inputs as S
from tests import _parity as P

pytestmark = pytest.mark.gpu

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
EXE = os.path.join(ROOT, "tests", "native", "c_abi_step")


@pytest.fixture(autouse=True)
def _need_gpu():
    import torch

    if not torch.cuda.is_available():
        pytest.skip("no GPU")


@pytest.mark.parametrize("mode", ["eager", "graph"])
@pytest.mark.parametrize("name,n,nd,qb,clip,steps", [
    ("tiny-zero1", 4099, 4, 256, 0.0, 3),
    ("13B-nd16-clip-int8", 100_003, 16, 256, 0.05, 3),
    ("gpt2-small-flat", 65_536 + 7, 8, 0, 0.0, 2),
])
def test_c_program_matches_oracle(tmp_path, name, n, nd, qb, clip, steps, mode):
    """eager: gnorm (with the spill) and step at every step; graph: one HIP
    graph captured from C (allocation-free norm pass without a spill, the
    step re-reading the contributions with its constants read on the
    device), replayed at every step."""
    if not os.path.exists(EXE):
        pytest.fail("tests/native/c_abi_step is not built (run __graft_entry__.build())")
    w = S.by_name(name)
    lr, wd = np.float32(w.lr), np.float32(w.weight_decay)
    master, m, v = S.host_state(w, 0, n)
    assert nd <= w.n_d
    rows = [S.host_contrib(w, s, 0, n)[:nd] for s in range(1, steps + 1)]
    src, dst = tmp_path / "in.bin", tmp_path / "out.bin"
    with open(src, "wb") as f:
        f.write(np.array([n], np.int64).tobytes())
        f.write(np.array([nd, qb, steps], np.int32).tobytes())
        f.write(np.array([lr, wd, clip], np.float32).tobytes())
        for a in (master, m, v):
            f.write(a.tobytes())
        for r in rows:
            f.write(np.ascontiguousarray(r).tobytes())
    print(f"case c abi {mode} {name} n={n} nd={nd} qb={qb} clip={clip}", flush=True)
    sys.stdout.flush()
    argv = [EXE, str(src), str(dst)] + (["graph"] if mode == "graph" else [])
    r = subprocess.run(argv, capture_output=True, text=True, timeout=120)
    assert r.returncode == 0, r.stderr
    out = np.fromfile(dst, dtype=np.uint8)
    off = 0

    def take(dtype, count):
        nonlocal off
        nbytes = np.dtype(dtype).itemsize * count
        a = out[off:off + nbytes].view(dtype)
        off += nbytes
        return a

    g_master, g_m, g_v = take(np.float32, n), take(np.float32, n), take(np.float32, n)
    g_p = take(np.uint16, n)
    nb = -(-n // qb) if qb else 0
    g_codes, g_scales = (take(np.int8, n), take(np.float32, nb)) if qb else (None, None)
    g_ssq = take(np.float64, steps) if clip > 0 else None
    assert off == out.size

    for s, rr in enumerate(rows, 1):
        h = O.Hyper(lr=float(lr), beta1=0.9, beta2=0.999, eps=1e-8, weight_decay=float(wd),
                    t=s, max_norm=float(np.float32(clip)), quant_block=qb)
        o = O.step(list(rr), master, m, v, h)
        if clip > 0:
            assert abs(g_ssq[s - 1] - o.sumsq) <= P.sumsq_tolerance(n, o.sumsq)
    P.f32_close("master", g_master, master)
    P.f32_close("m", g_m, m)
    P.f32_close("v", g_v, v)
    P.bf16_close("bf16", g_p, o.p)
    if qb:
        diff = P.int8_exact("int8", g_codes, g_scales, o.codes, o.scales, g_p, o.p, qb)
        if diff.any():
            c2, _ = O.quant_int8(g_p, qb)
            blk = np.repeat(diff, qb)[:n]
            assert np.array_equal(g_codes[blk], c2[blk])
