"""Bucketed step (zero_shard_gnorm_bucketed / zero_shard_step_bucketed):
the shard processed bucket by bucket on several worker streams, each bucket
waiting for its own arrival event.  Every element's update is the same
definition as the unbucketed step, so the outputs must be bit-identical to
zero_shard_step's given the same S; the bucketed S differs from the
unbucketed one only in the association of a binary64 sum and is checked
against the oracle's S within the rounding bound of that sum."""

from __future__ import annotations

import dataclasses

import numpy as np
import pytest

import oracle as O
import seeded_inputs as S
import sharded_mixed_precision_zero_amd as Z
from tests import _parity as P
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


def _same(a: dict, b: dict) -> None:
    for k in a:
        x, y = a[k], b[k]
        assert np.array_equal(x.view(np.uint8), y.view(np.uint8)), k


@pytest.mark.parametrize("name,n,bucket,streams,qb", [
    ("gpt2-small-flat", 300_001, 65_536, 2, 0),     # ragged last bucket
    ("gpt2-small-flat", 300_001, 512, 4, 256),      # many small buckets
    ("7.5B-nd64", 100_000, 40_960, 3, 512),
    ("tiny-zero1", 262_144, 262_144, 1, 64),        # one bucket
    ("tiny-zero1", 1000, 1024, 2, 0),               # bucket longer than the shard
])
def test_bucketed_step_bitwise_equals_step(name, n, bucket, streams, qb):
    import torch

    w = dataclasses.replace(S.by_name(name), quant_block=qb)
    log(f"case bucketed {name} n={n} bucket={bucket} streams={streams} qb={qb}")
    a, b = GpuShard(w, n=n), GpuShard(w, n=n)
    a.init_state()
    b.init_state()
    for s in range(1, 4):
        a.fill_grads(s)
        b.fill_grads(s)
        a.step(s)
        b.shard.step_bucketed(b.rows, bucket, w.lr, w.t_of(s), streams=streams)
    torch.cuda.synchronize()
    _same(a.host(), b.host())
    a.free()
    b.free()


@pytest.mark.parametrize("bucket,streams", [(65_536, 2), (131_072, 4), (512 * 97, 1)])
def test_bucketed_clipped_step(bucket, streams):
    """Clipping with the spill: bucketed norm then bucketed step; S against
    the oracle's, outputs bitwise against the unbucketed step run with the
    same S."""
    import torch

    w = dataclasses.replace(S.by_name("13B-nd16-clip-int8"), max_norm=0.05)
    n = 300_001
    log(f"case bucketed clip n={n} bucket={bucket} streams={streams}")
    a, b = GpuShard(w, n=n), GpuShard(w, n=n)
    a.init_state()
    b.init_state()
    for s in range(1, 4):
        a.fill_grads(s)
        b.fill_grads(s)
        b.shard.gnorm_bucketed(b.rows, bucket, b.sumsq, streams=streams)
        a.norm()
        torch.cuda.synchronize()
        s_b, s_a = float(b.sumsq.item()), float(a.sumsq.item())
        rows = list(S.host_contrib(w, s, 0, n))
        _, s_o = O.gbar_sumsq(rows)
        tol = P.sumsq_tolerance(n, s_o, buckets=-(-n // bucket))
        assert abs(s_b - s_o) <= tol, (s_b, s_o, tol)
        assert abs(s_a - s_o) <= tol
        a.sumsq.copy_(b.sumsq)  # the unbucketed step clips by the same S
        a.update(s)
        b.shard.step_bucketed(None, bucket, w.lr, w.t_of(s), b.sumsq, streams=streams)
    torch.cuda.synchronize()
    _same(a.host(), b.host())
    a.free()
    b.free()


def test_bucketed_waits_for_arrival_events():
    """Each bucket's contributions are written on a separate stream (the
    stand-in for its reduce-scatter) and announced by an event; the bucketed
    norm and step wait for them."""
    import torch

    w = dataclasses.replace(S.by_name("13B-nd16-clip-int8"), max_norm=0.05)
    n, bucket = 1_000_003, 131_072
    nb = -(-n // bucket)
    log(f"case bucketed events n={n} buckets={nb}")
    a, b = GpuShard(w, n=n), GpuShard(w, n=n)
    a.init_state()
    b.init_state()
    comm = torch.cuda.Stream()
    for s in range(1, 3):
        a.fill_grads(s)
        a.norm()
        # the previous step's work on b's stream has read the rows before
        # the new ones arrive
        comm.wait_stream(torch.cuda.current_stream())
        events = []
        for j in range(nb):
            lo, hi = j * bucket, min(n, (j + 1) * bucket)
            view = b.rows_buf[lo:]
            S.dev_contrib(w, s, view, hi - lo, b.stride, i0=lo, stream=comm)
            e = torch.cuda.Event()
            e.record(comm)
            events.append(e)
        b.shard.gnorm_bucketed(b.rows, bucket, b.sumsq, streams=2, ready=events)
        a.sumsq.copy_(b.sumsq)
        a.update(s)
        b.shard.step_bucketed(None, bucket, w.lr, w.t_of(s), b.sumsq, streams=2, ready=events)
    torch.cuda.synchronize()
    _same(a.host(), b.host())
    a.free()
    b.free()


def test_bucketed_unclipped_with_events_and_reuse():
    """Unclipped: the fused step per bucket as each arrives; then the same
    handle with fewer and with more buckets (scratch regrown)."""
    import torch

    w = S.by_name("gpt2-small-flat")
    n = 500_000
    a, b = GpuShard(w, n=n), GpuShard(w, n=n)
    a.init_state()
    b.init_state()
    comm = torch.cuda.Stream()
    for s, bucket in ((1, 100_352), (2, 250_368), (3, 25_088)):
        log(f"case bucketed unclipped reuse step={s} bucket={bucket}")
        a.fill_grads(s)
        a.step(s)
        nb = -(-n // bucket)
        comm.wait_stream(torch.cuda.current_stream())
        events = []
        for j in range(nb):
            lo, hi = j * bucket, min(n, (j + 1) * bucket)
            S.dev_contrib(w, s, b.rows_buf[lo:], hi - lo, b.stride, i0=lo, stream=comm)
            e = torch.cuda.Event()
            e.record(comm)
            events.append(e if j % 3 else None)  # NULL entries: no wait
        if any(e is None for e in events):
            comm.synchronize()  # buckets announced by NULL have arrived
        b.shard.step_bucketed(b.rows, bucket, w.lr, w.t_of(s), streams=3, ready=events)
    torch.cuda.synchronize()
    _same(a.host(), b.host())
    a.free()
    b.free()


def test_bucketed_empty_shard_and_errors():
    import torch

    w = S.by_name("tiny-zero1")
    g = GpuShard(w, n=0, phi=3, r=3)
    g.sumsq.fill_(7.0)
    g.shard.gnorm_bucketed(g.rows, 512, g.sumsq)
    g.shard.step_bucketed(g.rows, 512, 1e-3, 1)
    torch.cuda.synchronize()
    assert float(g.sumsq.item()) == 0.0
    g.free()

    w = dataclasses.replace(S.by_name("13B-nd16-clip-int8"), max_norm=0.05)
    g = GpuShard(w, n=10_000)
    g.init_state()
    g.fill_grads(1)
    before = g.host()
    h = g.shard.h
    assert Z.zero_shard_gnorm_bucketed(h, g.rows, 1000, 2, None, g.sumsq) == Z.ZS_EINVAL
    assert Z.zero_shard_gnorm_bucketed(h, g.rows, 0, 2, None, g.sumsq) == Z.ZS_EINVAL
    assert Z.zero_shard_gnorm_bucketed(h, g.rows, 512, 0, None, g.sumsq) == Z.ZS_EINVAL
    assert Z.zero_shard_gnorm_bucketed(h, g.rows, 512, 5, None, g.sumsq) == Z.ZS_EINVAL
    assert Z.zero_shard_gnorm_bucketed(h, g.rows, 512, 2, None, None) == Z.ZS_EINVAL
    # the spill is not valid before a norm pass
    assert Z.zero_shard_step_bucketed(h, None, 512, 2, None, 1e-3, 1, g.sumsq) == Z.ZS_ESTATE
    assert Z.zero_shard_step_bucketed(h, g.rows, 512, 2, None, 1e-3, 1, None) == Z.ZS_EINVAL
    bad = [r[1:] for r in g.rows]
    assert Z.zero_shard_gnorm_bucketed(h, bad, 512, 2, None, g.sumsq) == Z.ZS_EALIGN
    torch.cuda.synchronize()
    _same(before, g.host())
    g.free()
    assert Z.zero_shard_gnorm_bucketed(h, g.rows, 512, 2, None, g.sumsq) == Z.ZS_ESTATE


@pytest.mark.parametrize("clip,bucket,streams", [
    (0.0, 65_536, 2),
    (0.0, 512 * 37, 3),
    (0.05, 65_536, 2),
    (0.05, 131_072, 4),
])
def test_bucketed_q8_equals_step_q8(clip, bucket, streams):
    """int8 contributions (qgZ) bucket by bucket: bitwise equal to the
    unbucketed _q8 step given the same S; S against the oracle's."""
    import torch

    w = dataclasses.replace(S.by_name("7.5B-nd64-zeropp"), n_d=16, max_norm=clip)
    n, cb = 300_001, w.contrib_block
    log(f"case bucketed q8 n={n} clip={clip} bucket={bucket} streams={streams}")
    a, b = GpuShard(w, n=n), GpuShard(w, n=n)
    a.init_state()
    b.init_state()
    for s in range(1, 4):
        a.fill_grads(s)
        b.fill_grads(s)
        if clip > 0:
            a.norm()
            b.shard.gnorm_bucketed_q8(b.qrows, b.srows, cb, bucket, b.sumsq, streams=streams)
            torch.cuda.synchronize()
            codes, scales = S.host_contrib_q8(w, s, 0, n)
            _, s_o = O.gbar_sumsq_q8(codes, scales, cb)
            tol = P.sumsq_tolerance(n, s_o, buckets=-(-n // bucket))
            assert abs(float(b.sumsq.item()) - s_o) <= tol
            a.sumsq.copy_(b.sumsq)
            a.update(s)
            b.shard.step_bucketed_q8(None, None, cb, bucket, w.lr, w.t_of(s), b.sumsq,
                                     streams=streams)
        else:
            a.step(s)
            b.shard.step_bucketed_q8(b.qrows, b.srows, cb, bucket, w.lr, w.t_of(s),
                                     streams=streams)
    torch.cuda.synchronize()
    _same(a.host(), b.host())
    a.free()
    b.free()


def test_bucketed_q8_errors():
    w = dataclasses.replace(S.by_name("7.5B-nd64-zeropp"), n_d=4)
    g = GpuShard(w, n=4096)
    h = g.shard.h
    assert Z.zero_shard_step_bucketed_q8(h, g.qrows, g.srows, 100, 512, 2, None, 1e-3,
                                         1) == Z.ZS_EINVAL
    assert Z.zero_shard_step_bucketed_q8(h, g.qrows, g.srows, 256, 768, 2, None, 1e-3,
                                         1) == Z.ZS_EINVAL
    assert Z.zero_shard_gnorm_bucketed_q8(h, g.qrows, None, 256, 512, 2, None,
                                          g.sumsq) == Z.ZS_EINVAL
    g.free()


def test_arrival_delay_waits_and_bucketed_step_waits_for_it():
    """The arrival stand-in (a bounded wait on the wall clock) takes about
    the time asked for, and a bucketed step that waits on events recorded
    after such waits gives the unbucketed step's bits."""
    import torch

    comm = torch.cuda.Stream()
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record(comm)
    S.dev_delay(2000.0, comm)
    b.record(comm)
    torch.cuda.synchronize()
    ms = a.elapsed_time(b)
    assert 1.9 <= ms <= 4.0, ms

    w = dataclasses.replace(S.by_name("13B-nd16-clip-int8"), max_norm=0.05)
    n, bucket = 300_001, 65_536
    g1, g2 = GpuShard(w, n=n), GpuShard(w, n=n)
    g1.init_state()
    g2.init_state()
    for s in (1, 2):
        g1.fill_grads(s)
        g2.fill_grads(s)
        g1.norm()
        comm.wait_stream(torch.cuda.current_stream())
        evs = []
        for _ in range(-(-n // bucket)):
            S.dev_delay(300.0, comm)
            e = torch.cuda.Event()
            e.record(comm)
            evs.append(e)
        g2.shard.gnorm_bucketed(g2.rows, bucket, g2.sumsq, streams=2, ready=evs)
        g1.sumsq.copy_(g2.sumsq)
        g1.update(s)
        g2.shard.step_bucketed(None, bucket, w.lr, w.t_of(s), g2.sumsq, streams=2)
    torch.cuda.synchronize()
    _same(g1.host(), g2.host())
    g1.free()
    g2.free()


def test_bucketed_sum_independent_of_stream_count():
    """The bucketed S adds the bucket sums in bucket order, so it is the same
    double whatever the number of worker streams, call after call."""
    import torch

    w = dataclasses.replace(S.by_name("13B-nd16-clip-int8"), max_norm=0.05)
    n, bucket = 1_000_003, 65_536
    g = GpuShard(w, n=n)
    g.init_state()
    g.fill_grads(1)
    got = []
    for streams in (1, 2, 3, 4, 2, 1):
        g.shard.gnorm_bucketed(g.rows, bucket, g.sumsq, streams=streams)
        torch.cuda.synchronize()
        got.append(g.sumsq.cpu().numpy().view(np.uint64)[0])
    assert len(set(got)) == 1, got
    g.free()


@pytest.mark.parametrize("contrib,clip,bucket,streams", [
    ("bf16", 0.05, 65_536, 2),    # ragged last bucket (300,001 = 4 x 65,536 + 37,857)
    ("bf16", 0.05, 512 * 37, 3),
    ("bf16", 0.0, 65_536, 2),
    ("q8", 0.05, 65_536, 2),
    ("q8", 0.05, 131_072, 4),
    ("q8", 0.0, 512 * 37, 3),
])
def test_bucketed_against_oracle(contrib, clip, bucket, streams):
    """The bucketed step's outputs against the oracle directly, element by
    element, at every step: master, m, v within the fp32 tolerance, bf16
    within 1 ulp, int8 codes and scales exact (on the GPU's own bf16, and on
    every block whose bf16 input equals the oracle's).  With clipping the
    oracle takes its own S over the whole shard; the GPU's bucketed S is
    checked against it within the bound for the two summation orders.  This
    pins the bucket offsets (rows, scales of int8 contributions, int8 output
    scales) and the ragged last bucket to the definition, not to the
    unbucketed kernel."""
    import torch

    if contrib == "bf16":
        w = dataclasses.replace(S.by_name("13B-nd16-clip-int8"), max_norm=clip)
    else:
        w = dataclasses.replace(S.by_name("7.5B-nd64-zeropp"), n_d=16, max_norm=clip,
                                weight_decay=0.1, warm=False, t0=0)
    n, cb = 300_001, w.contrib_block
    log(f"case bucketed vs oracle {contrib} clip={clip} bucket={bucket} streams={streams}")
    g = GpuShard(w, n=n)
    g.init_state()
    master, m, v = S.host_state(w, 0, n)
    for s in range(1, 4):
        g.fill_grads(s)
        if cb:
            codes, scales = S.host_contrib_q8(w, s, 0, n)
            if clip > 0:
                g.shard.gnorm_bucketed_q8(g.qrows, g.srows, cb, bucket, g.sumsq,
                                          streams=streams)
                g.shard.step_bucketed_q8(None, None, cb, bucket, w.lr, w.t_of(s), g.sumsq,
                                         streams=streams)
            else:
                g.shard.step_bucketed_q8(g.qrows, g.srows, cb, bucket, w.lr, w.t_of(s),
                                         streams=streams)
        else:
            rows = list(S.host_contrib(w, s, 0, n))
            if clip > 0:
                g.shard.gnorm_bucketed(g.rows, bucket, g.sumsq, streams=streams)
                g.shard.step_bucketed(None, bucket, w.lr, w.t_of(s), g.sumsq, streams=streams)
            else:
                g.shard.step_bucketed(g.rows, bucket, w.lr, w.t_of(s), streams=streams)
        h = O.Hyper(lr=w.lr, beta1=w.beta1, beta2=w.beta2, eps=w.eps,
                    weight_decay=w.weight_decay, t=w.t_of(s), max_norm=clip,
                    quant_block=w.quant_block)
        out = (O.step_q8(list(codes), list(scales), cb, master, m, v, h, threads=4) if cb
               else O.step(rows, master, m, v, h, threads=4))
        torch.cuda.synchronize()
        if clip > 0:
            s_gpu = float(g.sumsq.item())
            tol = P.sumsq_tolerance(n, out.sumsq, buckets=-(-n // bucket))
            assert abs(s_gpu - out.sumsq) <= tol, (s_gpu, out.sumsq, tol)
        got = g.host()
        name = f"bucketed {contrib} step {s}"
        P.f32_close(f"{name} master", got["master"], master)
        P.f32_close(f"{name} m", got["m"], m)
        P.f32_close(f"{name} v", got["v"], v)
        P.bf16_close(f"{name} bf16", got["p"], out.p)
        c_own, s_own = O.quant_int8(got["p"], w.quant_block)
        assert np.array_equal(got["codes"], c_own) and np.array_equal(
            got["scales"].view(np.uint32), s_own.view(np.uint32)), name
        P.int8_exact(f"{name} int8", got["codes"], got["scales"], out.codes, out.scales,
                     got["p"], out.p, w.quant_block)
    g.free()
