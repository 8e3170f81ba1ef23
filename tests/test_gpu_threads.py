"""Several host threads driving the library at once, each with its own
handle on its own stream (handles created, stepped and freed concurrently):
every shard's result equals the same shard stepped alone, bit for bit.  The
library's process-wide state (the live-handle set, the per-device caches
of the architecture check and of the allocation-free scratch address) is
shared by these threads."""

from __future__ import annotations

import dataclasses
import threading

import numpy as np
import pytest

import seeded_inputs as S
from tests._gpu import GpuShard, log

pytestmark = pytest.mark.gpu

CASES = [  # (base workload, shard length, overrides)
    ("13B-nd16-clip-int8", 300_007, {}),
    ("tiny-zero1", 262_144, {}),
    ("gpt2-small-flat", 200_003, {"quant_block": 64}),
    ("7.5B-nd64", 50_011, {}),
    ("13B-nd16-clip-int8", 123_457, {"max_norm": 0.05, "quant_block": 512}),
    ("7.5B-nd64-zeropp", 65_536 + 8, {}),
]


@pytest.fixture(autouse=True)
def _gpu_cleanup():
    import torch

    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    yield
    torch.cuda.synchronize()
    torch.cuda.empty_cache()


def _run(case, stream, steps: int = 3) -> dict:
    import torch

    base, n, kw = case
    w = dataclasses.replace(S.by_name(base), **kw)
    with torch.cuda.stream(stream):
        g = GpuShard(w, n=n, stream=stream)
        g.init_state()
        for s in range(1, steps + 1):
            g.fill_grads(s)
            g.step(s)
        stream.synchronize()
        out = g.host()
        g.free()
    return out


def test_concurrent_handles_equal_sequential():
    import torch

    log(f"case {len(CASES)} threads, one handle and stream each")
    ref = [_run(c, torch.cuda.current_stream()) for c in CASES]
    streams = [torch.cuda.Stream() for _ in CASES]
    got: list = [None] * len(CASES)
    errors: list = []

    def worker(i):
        try:
            got[i] = _run(CASES[i], streams[i])
        except Exception as e:  # reported below, with the case
            errors.append((i, repr(e)))

    threads = [threading.Thread(target=worker, args=(i,)) for i in range(len(CASES))]
    for t in threads:
        t.start()
    for t in threads:
        t.join()
    assert not errors, errors
    for i, (a, b) in enumerate(zip(ref, got)):
        for k in a:
            if a[k] is None:
                continue
            assert np.array_equal(a[k].view(np.uint8), b[k].view(np.uint8)), (CASES[i], k)
