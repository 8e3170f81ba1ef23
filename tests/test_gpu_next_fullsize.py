"""The bucketed step and the offloaded step at the workloads' full sizes, in
the launch configuration the benchmark times (buckets of 5e8 gradient
elements on 2 worker streams; offload with 16 host threads and the one-step
delayed update).  Both are scheduling variants of the same definition, so
their outputs are compared with the on-device unbucketed step over the
whole shard (bit for bit, given the same S), and the bucketed S with the
unbucketed S within the bound for two binary64 summation orders.  The
bucketed outputs are also compared with the oracle directly on windows
across bucket boundaries (the head, the tail, the first boundaries, one in
the middle, the last), clipped by the oracle's own S."""

from __future__ import annotations

import numpy as np
import pytest

import seeded_inputs as S
import oracle as O
from tests import _parity as P
from tests._gpu import GpuShard, OffloadShard, OracleWindow, log, oracle_global_sumsq

pytestmark = pytest.mark.gpu


@pytest.fixture(autouse=True)
def _gpu_cleanup():
    import torch

    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    yield
    torch.cuda.synchronize()
    torch.cuda.empty_cache()


def _bucket_len(w, elems: float = 5e8) -> int:
    per = -(-int(elems) // w.n_d)
    return -(-per // 512) * 512


def _dev_equal(a: GpuShard, b: GpuShard) -> None:
    import torch

    pairs = [("master", a.master, b.master), ("m", a.m, b.m), ("v", a.v, b.v), ("p", a.p, b.p)]
    if a.qb:
        pairs += [("codes", a.codes, b.codes), ("scales", a.scales, b.scales)]
    for name, x, y in pairs:
        same = torch.equal(x.view(torch.int32) if x.dtype == torch.float32 else x,
                           y.view(torch.int32) if y.dtype == torch.float32 else y)
        assert same, name


@pytest.mark.parametrize("name", ["13B-nd16-clip-int8", "7.5B-nd64"])
def test_bucketed_full_size(name):
    import torch

    w = S.by_name(name)
    bl = _bucket_len(w)
    log(f"case bucketed full size {name} bucket_len={bl}")
    a, b = GpuShard(w), GpuShard(w)
    a.init_state()
    b.init_state()
    n, nb = w.shard_len, -(-w.shard_len // bl)
    half = 8192  # windows straddle bucket boundaries by this much on each side
    cuts = sorted({1, 2, nb // 2, nb - 1})
    wins = [(0, 2 * half)] + [(j * bl - half, j * bl + half) for j in cuts if 0 < j < nb]
    wins.append(((n - 2 * half) // 256 * 256, n))
    ows = [OracleWindow(w, lo, hi - lo) for lo, hi in wins]
    for s in range(1, 3):
        a.fill_grads(s)
        b.fill_grads(s)
        if w.max_norm > 0:
            a.norm()
            b.shard.gnorm_bucketed(b.rows, bl, b.sumsq, streams=2)
            torch.cuda.synchronize()
            sa, sb = float(a.sumsq.item()), float(b.sumsq.item())
            tol = 2 * P.sumsq_tolerance(w.shard_len, sa, buckets=-(-w.shard_len // bl))
            assert abs(sa - sb) <= tol, (sa, sb, tol)
            a.sumsq.copy_(b.sumsq)
            a.update(s)
            b.shard.step_bucketed(None, bl, w.lr, w.t_of(s), b.sumsq, streams=2)
        else:
            a.step(s)
            b.shard.step_bucketed(b.rows, bl, w.lr, w.t_of(s), streams=2)
        torch.cuda.synchronize()
        _dev_equal(a, b)
        s_orc = oracle_global_sumsq(w, s) if w.max_norm > 0 else None
        if s_orc is not None:
            sb = float(b.sumsq.item())
            tol = P.sumsq_tolerance(n, s_orc, buckets=nb)
            assert abs(sb - s_orc) <= tol, (sb, s_orc, tol)
        for (lo, hi), ow in zip(wins, ows):
            o = ow.step(s, sumsq_total=s_orc)
            got = b.host(lo, hi)
            nm = f"{name} bucketed step {s} [{lo},{hi})"
            P.f32_close(f"{nm} master", got["master"], ow.master)
            P.f32_close(f"{nm} m", got["m"], ow.m)
            P.f32_close(f"{nm} v", got["v"], ow.v)
            P.bf16_close(f"{nm} bf16", got["p"], o.p)
            if w.quant_block:
                c_own, _ = O.quant_int8(got["p"], w.quant_block)
                assert np.array_equal(got["codes"], c_own), nm
                P.int8_exact(f"{nm} int8", got["codes"], got["scales"], o.codes, o.scales,
                             got["p"], o.p, w.quant_block)
        log(f"  step {s}: bitwise equal to the unbucketed step; {len(wins)} windows across "
            f"bucket boundaries within tolerance of the oracle")
    a.free()
    b.free()


def test_offload_full_size():
    import torch

    w = S.by_name("13B-nd16-clip-int8")
    log(f"case offload full size {w.name} n={w.shard_len}")
    g = GpuShard(w)
    g.init_state()
    off = OffloadShard(w, threads=16)
    for s in range(1, 3):
        g.fill_grads(s)
        off.fill_grads(s)
        g.step(s)
        off.step(s, delayed=True)
    off.finish()
    torch.cuda.synchronize()
    for name, dev, host in (("master", g.master, off.master), ("m", g.m, off.m),
                            ("v", g.v, off.v)):
        assert np.array_equal(dev.cpu().numpy().view(np.uint32), host.view(np.uint32)), name
    assert torch.equal(g.p, off.params())
    assert np.array_equal(g.codes.cpu().numpy(), off.codes)
    assert np.array_equal(g.scales.cpu().numpy().view(np.uint32), off.scales.view(np.uint32))
    off.free()
    g.free()
