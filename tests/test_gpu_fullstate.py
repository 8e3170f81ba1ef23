"""Full final state at full size: after the steps of a large workload the
GPU's whole shard (master, m, v, the bf16 copy, int8 codes and scales) is
compared with the oracle's, chunk by chunk, to the parity tolerances.  The
window tests follow more steps on sampled windows; this covers every
element.  The oracle runs over 2^24-element chunks on a pool of host
threads (each chunk's work is plain C, outside the interpreter lock), with
the clipping S summed over the chunks in chunk order."""

from __future__ import annotations

from concurrent.futures import ThreadPoolExecutor

import numpy as np
import pytest

import oracle as O
import seeded_inputs as S
from tests import _parity as P
from tests._gpu import GpuShard, log

pytestmark = pytest.mark.gpu

CHUNK = 1 << 24


@pytest.fixture(autouse=True)
def _gpu_cleanup():
    import torch

    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    yield
    torch.cuda.synchronize()
    torch.cuda.empty_cache()


class FullOracle:
    """The oracle's state for a whole shard, stepped chunk by chunk."""

    def __init__(self, w: S.Workload, pool: ThreadPoolExecutor):
        self.w, self.pool, self.n = w, pool, w.shard_len
        self.chunks = [(lo, min(self.n, lo + CHUNK)) for lo in range(0, self.n, CHUNK)]
        states = list(pool.map(lambda c: S.host_state(w, c[0], c[1] - c[0]), self.chunks))
        self.master = np.concatenate([s[0] for s in states])
        self.m = np.concatenate([s[1] for s in states])
        self.v = np.concatenate([s[2] for s in states])
        del states
        self.out = [None] * len(self.chunks)

    def _hyper(self, s: int):
        w = self.w
        return O.Hyper(lr=w.lr, beta1=w.beta1, beta2=w.beta2, eps=w.eps,
                       weight_decay=w.weight_decay, t=w.t_of(s), quant_block=w.quant_block)

    def _inputs(self, s, lo, hi):
        if self.w.contrib_block:
            codes, scales = S.host_contrib_q8(self.w, s, lo, hi - lo)
            return list(codes), list(scales)
        return list(S.host_contrib(self.w, s, lo, hi - lo)), None

    def step(self, s: int) -> float | None:
        w, h = self.w, self._hyper(s)
        cb = w.contrib_block

        def gbar_of(j):
            lo, hi = self.chunks[j]
            a, b = self._inputs(s, lo, hi)
            return O.gbar_sumsq_q8(a, b, cb, threads=2) if cb else O.gbar_sumsq(a, threads=2)

        if w.max_norm > 0:  # two passes: S over every chunk, then the update
            parts = list(self.pool.map(gbar_of, range(len(self.chunks))))
            total = 0.0
            for _, sj in parts:
                total += sj
            coef = O.clip_coef(total, float(np.float32(w.max_norm)))

            def upd(j):
                lo, hi = self.chunks[j]
                sl = slice(lo, hi)
                O.adam(self.master[sl], self.m[sl], self.v[sl], parts[j][0], coef, h)
                p = O.f32_to_bf16(self.master[sl])
                codes = scales = None
                if w.quant_block:
                    codes, scales = O.quant_int8(p, w.quant_block)
                self.out[j] = O.StepOut(p, codes, scales, parts[j][1])

            list(self.pool.map(upd, range(len(self.chunks))))
            return total

        def one(j):
            lo, hi = self.chunks[j]
            sl = slice(lo, hi)
            a, b = self._inputs(s, lo, hi)
            if cb:
                self.out[j] = O.step_q8(a, b, cb, self.master[sl], self.m[sl], self.v[sl], h,
                                        threads=2)
            else:
                self.out[j] = O.step(a, self.master[sl], self.m[sl], self.v[sl], h, threads=2)

        list(self.pool.map(one, range(len(self.chunks))))
        return None


def run_and_compare(name: str, steps: int) -> None:
    """Steps 1..steps of workload `name` on the GPU and in the oracle (fresh
    seeded gradients every step, S compared at every clipped step), then
    the whole final shard compared chunk by chunk."""
    import time

    import torch

    w = S.by_name(name)
    n = w.shard_len
    log(f"case full state {name}: n={n} n_d={w.n_d}, {steps} steps")
    g = GpuShard(w)
    g.init_state()
    t0 = time.time()
    with ThreadPoolExecutor(max_workers=8) as pool:
        orc = FullOracle(w, pool)
        for s in range(1, steps + 1):
            g.fill_grads(s)
            g.step(s)
            total = orc.step(s)
            if total is not None:
                torch.cuda.synchronize()
                got = float(g.sumsq.item())
                assert abs(got - total) <= P.sumsq_tolerance(n, total), (s, got, total)
            log(f"  step {s} done ({time.time() - t0:.0f} s)")
    torch.cuda.synchronize()
    worst = 0
    for j, (lo, hi) in enumerate(orc.chunks):
        got = g.host(lo, hi)
        o = orc.out[j]
        sl = slice(lo, hi)
        name_j = f"{name} [{lo},{hi})"
        P.f32_close(f"{name_j} master", got["master"], orc.master[sl])
        P.f32_close(f"{name_j} m", got["m"], orc.m[sl])
        P.f32_close(f"{name_j} v", got["v"], orc.v[sl])
        P.bf16_close(f"{name_j} bf16", got["p"], o.p)
        if w.quant_block:
            diff = P.int8_exact(f"{name_j} int8", got["codes"], got["scales"], o.codes,
                                o.scales, got["p"], o.p, w.quant_block)
            worst = max(worst, int(diff.sum()))
            if diff.any():  # other correct codes: those of the GPU's own bf16
                c2, _ = O.quant_int8(got["p"], w.quant_block)
                blk = np.repeat(diff, w.quant_block)[:hi - lo]
                assert np.array_equal(got["codes"][blk], c2[blk])
    log(f"  all {len(orc.chunks)} chunks within tolerance after {steps} steps; int8 blocks "
        f"with differing input in a chunk: at most {worst}")
    g.free()


@pytest.mark.parametrize("name,steps", [("7.5B-nd64", 2), ("7.5B-nd64-zeropp", 2),
                                        ("13B-nd16-clip-int8", 10)])
def test_full_final_state(name, steps):
    """The 13B clipped workload through all its 10 steps (about a minute);
    the 7.5B workloads after 2 of their 50 (all 50 take 2.5 minutes each:
    tests/test_gpu_long_parity.py)."""
    run_and_compare(name, steps)


def stage0_streamed(steps: int) -> None:
    """The 13B stage-0 flat buffer (12,851,609,600 elements, N_d = 1,
    unclipped) after `steps` steps: every element against the oracle.  An
    unclipped step is elementwise, so each 2^24-element chunk is regenerated
    from its seeds (initial state, every step's contributions) and stepped by
    the oracle on its own, on a pool of host threads, then compared with the
    GPU's chunk; host memory stays bounded by the chunks in flight."""
    import time

    import torch

    w = S.by_name("13B-nd1-stage0")
    n = w.shard_len
    log(f"case full state streamed {w.name}: n={n} (205.6 GB resident), {steps} steps")
    g = GpuShard(w)
    g.init_state()
    for s in range(1, steps + 1):
        g.fill_grads(s)
        g.step(s)
    torch.cuda.synchronize()
    chunks = [(lo, min(n, lo + CHUNK)) for lo in range(0, n, CHUNK)]
    hyper = {s: O.Hyper(lr=w.lr, beta1=w.beta1, beta2=w.beta2, eps=w.eps,
                        weight_decay=w.weight_decay, t=w.t_of(s)) for s in range(1, steps + 1)}

    def one(j):
        lo, hi = chunks[j]
        master, m, v = S.host_state(w, lo, hi - lo)
        for s in range(1, steps + 1):
            out = O.step(list(S.host_contrib(w, s, lo, hi - lo)), master, m, v, hyper[s])
        got = g.host(lo, hi)
        nm = f"{w.name} [{lo},{hi})"
        st = P.f32_close(f"{nm} master", got["master"], master)
        P.f32_close(f"{nm} m", got["m"], m)
        P.f32_close(f"{nm} v", got["v"], v)
        P.bf16_close(f"{nm} bf16", got["p"], out.p)
        return st["bitwise"]

    t0 = time.time()
    bitwise = []
    with ThreadPoolExecutor(max_workers=16) as pool:
        for i, b in enumerate(pool.map(one, range(len(chunks))), 1):
            bitwise.append(b)
            if i % 64 == 0 or i == len(chunks):
                log(f"  {i}/{len(chunks)} chunks within tolerance ({time.time() - t0:.0f} s)")
    log(f"  every element of the 13B stage-0 buffer within tolerance after {steps} steps; "
        f"master bitwise fraction min {min(bitwise):.6f}")
    g.free()


def test_13b_stage0_full_final_state_streamed():
    """Two of the buffer's 20 steps (all 20: tests/test_gpu_long_parity.py)."""
    stage0_streamed(2)
