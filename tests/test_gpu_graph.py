"""The shard step captured in a HIP graph: zero_shard_gnorm and
zero_shard_step queue only kernel launches on the handle's stream (no
allocation, no memset), so a graph of one clipped, quantized step can be
captured and replayed.  Every replay is checked against the same step run
eagerly, with eager work and synchronisations between the replays.  The
step counter and learning rate are baked into the captured launches, so
each replay repeats step t."""

from __future__ import annotations

import dataclasses

import numpy as np
import pytest

import seeded_inputs as S
from tests._gpu import GpuShard, log

pytestmark = pytest.mark.gpu


@pytest.fixture(autouse=True)
def _gpu_cleanup():
    import torch

    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    yield
    torch.cuda.synchronize()
    torch.cuda.empty_cache()


@pytest.mark.parametrize("name,n", [("13B-nd16-clip-int8", 300_001), ("tiny-zero1", 262_144)])
def test_captured_step_replays_match_eager(name, n):
    import torch

    w = dataclasses.replace(S.by_name(name), max_norm=0.05) if "clip" in name else S.by_name(name)
    side = torch.cuda.Stream()
    log(f"case graph {name} n={n}")
    eager = GpuShard(w, n=n)
    graphed = GpuShard(w, n=n, stream=side)
    for g in (eager, graphed):
        g.init_state()
        g.fill_grads(1)
    torch.cuda.synchronize()
    t = 5
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph, stream=side):
        graphed.step(t)
    torch.cuda.synchronize()  # capture ran nothing: both shards still at their start
    for rep in range(3):
        eager.step(t)
        graph.replay()
        torch.cuda.synchronize()
        a, b = eager.host(), graphed.host()
        for k in a:
            assert np.array_equal(a[k].view(np.uint8), b[k].view(np.uint8)), (rep, k)
        eager.fill_grads(2 + rep)  # eager work between replays, same inputs on both
        with torch.cuda.stream(side):
            graphed.fill_grads(2 + rep)
        torch.cuda.synchronize()
    eager.free()
    graphed.free()
