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


@pytest.mark.parametrize("name,n", [("tiny-zero1", 262_144), ("13B-nd16-clip-int8", 300_001)])
def test_one_graph_serves_every_step(name, n):
    """zero_shard_step_dev reads lr, lr*wd and the bias corrections from a
    device array when the kernel runs: one captured step (norm pass and
    update when clipping) replayed for t = 1..6, the step's constants copied
    into that array before each replay, outside the graph, equals the eager
    zero_shard_step at (lr, t) bit for bit; then a graph of 3 steps reading
    rows of a constants table, replayed twice, equals 6 eager steps."""
    import torch

    w = dataclasses.replace(S.by_name(name), max_norm=0.05) if "clip" in name else S.by_name(name)
    side = torch.cuda.Stream()
    log(f"case graph every step {name} n={n}")
    eager = GpuShard(w, n=n)
    graphed = GpuShard(w, n=n, stream=side)
    for g in (eager, graphed):
        g.init_state()
        g.fill_grads(1)
    torch.cuda.synchronize()
    consts = torch.zeros(4, dtype=torch.float64, device="cuda")
    host = torch.zeros(4, dtype=torch.float64).pin_memory()
    spill = graphed.clip and graphed.gbar_ws is not None

    def graphed_step(cdev):
        if graphed.clip:
            graphed.norm()
        graphed.shard.step_dev(None if spill else graphed.tab, cdev,
                               graphed.sumsq if graphed.clip else None)

    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph, stream=side):
        graphed_step(consts)
    torch.cuda.synchronize()
    for t in range(1, 7):
        eager.step(t)
        host.copy_(torch.tensor(graphed.shard.consts(w.lr, w.t_of(t)), dtype=torch.float64))
        # the copy and the replay on one stream: replay() launches on the
        # current stream, so it is entered here to follow the copy
        with torch.cuda.stream(side):
            consts.copy_(host, non_blocking=True)
            graph.replay()
        torch.cuda.synchronize()
        a, b = eager.host(), graphed.host()
        for k in a:
            assert np.array_equal(a[k].view(np.uint8), b[k].view(np.uint8)), (t, k)
        eager.fill_grads(t + 1)  # eager work between replays, same inputs on both
        with torch.cuda.stream(side):
            graphed.fill_grads(t + 1)
        torch.cuda.synchronize()
    # a 3-step graph over a table of constants
    table = torch.zeros(3, 4, dtype=torch.float64, device="cuda")
    graph3 = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph3, stream=side):
        for j in range(3):
            graphed_step(table[j])
    torch.cuda.synchronize()
    for base in (7, 10):
        rows = [graphed.shard.consts(w.lr, w.t_of(base + j)) for j in range(3)]
        with torch.cuda.stream(side):
            table.copy_(torch.tensor(rows, dtype=torch.float64).pin_memory(), non_blocking=True)
            graph3.replay()
        for j in range(3):
            eager.step(base + j)
        torch.cuda.synchronize()
        a, b = eager.host(), graphed.host()
        for k in a:
            assert np.array_equal(a[k].view(np.uint8), b[k].view(np.uint8)), (base, k)
    eager.free()
    graphed.free()
