"""Calls whose work the library splits into several kernel launches: the
norm pass runs in launches of ZS_NORM_LAUNCH_LEN shard elements, an update
in its wide form (many contribution rows) in launches of ZS_WIDE_LAUNCH_LEN.
S is checked against the oracle over the whole shard, and the spill and the
updated state on windows that straddle the launch boundaries, the head and
the tail, for bf16 and int8 contributions (tolerances of tests/_parity.py).
"""

from __future__ import annotations

import dataclasses

import numpy as np
import pytest

import oracle as O
import seeded_inputs as S
import sharded_mixed_precision_zero_amd as Z
from tests import _parity as P
from tests._gpu import GpuShard, OracleWindow, log

pytestmark = pytest.mark.gpu

LN, LW = Z.ZS_NORM_LAUNCH_LEN, Z.ZS_WIDE_LAUNCH_LEN

CASES = [
    # (name, base workload, n, n_d, contribution block, int8 out block, clip,
    #  launch length, bucket length or 0)
    ("bf16 norm + clipped update", "13B-nd16-clip-int8", LN + 1029, 16, 0, 256, 1.0, LN, 0),
    ("int8-row norm + clipped update", "7.5B-nd64-zeropp", LN + 77, 4, 64, 0, 0.5, LN, 0),
    ("bf16 wide update", "7.5B-nd64", 2 * LW + 333, 24, 0, 0, 0.0, LW, 0),
    ("bf16 wide update, int8 out", "7.5B-nd64", LW + 99, 32, 0, 128, 0.0, LW, 0),
    ("int8-row wide update", "7.5B-nd64-zeropp", 2 * LW + 4099, 16, 256, 256, 0.0, LW, 0),
    # whole launches only, no ragged last one
    ("bf16 norm, two whole launches", "13B-nd16-clip-int8", 2 * LN, 8, 0, 256, 1.0, LN, 0),
    ("bf16 wide update, two whole launches", "7.5B-nd64", 2 * LW, 24, 0, 0, 0.0, LW, 0),
    # buckets longer than one launch: the first bucket's norm pass is two launches
    ("bf16 bucketed norm + clipped update", "13B-nd16-clip-int8", LN + LW + 333, 16, 0, 256, 1.0,
     LN, LN + 512),
    # the first bucket's wide update is two launches
    ("bf16 bucketed wide update", "7.5B-nd64", LW + LW // 2 + 77, 24, 0, 0, 0.0, LW, LW + 512),
]


@pytest.fixture(autouse=True)
def _gpu_cleanup():
    import torch

    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    yield
    torch.cuda.synchronize()
    torch.cuda.empty_cache()


def _rows(w, s, lo, n):
    if w.contrib_block:
        codes, scales = S.host_contrib_q8(w, s, lo, n)
        return O.gbar_sumsq_q8(list(codes), list(scales), w.contrib_block)
    return O.gbar_sumsq(list(S.host_contrib(w, s, lo, n)))


def _bounds(n: int, launch: int, bucket: int) -> list[int]:
    """Every launch boundary inside (0, n): launches restart at each bucket."""
    part = bucket or n
    out = set()
    for b0 in range(0, n, part):
        if b0:
            out.add(b0)
        for k in range(b0 + launch, min(n, b0 + part), launch):
            out.add(k)
    return sorted(out)


@pytest.mark.parametrize("name,base,n,nd,cb,qb,clip,launch,bucket", CASES,
                         ids=[c[0] for c in CASES])
def test_split_launches_against_oracle(name, base, n, nd, cb, qb, clip, launch, bucket):
    import torch

    w = dataclasses.replace(S.by_name(base), n_d=nd, contrib_block=cb, quant_block=qb,
                            max_norm=clip, weight_decay=0.1 if clip else 0.0)
    bounds = _bounds(n, launch, bucket)
    log(f"case {name}: n={n} n_d={nd} contrib_block={cb} out_block={qb} clip={clip} "
        f"bucket={bucket} launch boundaries={bounds}")
    g = GpuShard(w, n=n)
    g.init_state()
    size = 8192
    wins = [(0, size)] + [(b - size // 2, min(n, b + size // 2)) for b in bounds]
    tail = (n - size) // 256 * 256
    if tail >= wins[-1][1]:
        wins.append((tail, n))
    else:  # the last boundary window runs into the tail: take it to the end
        wins[-1] = (wins[-1][0], n)
    ows = [OracleWindow(w, lo, hi - lo) for lo, hi in wins]
    for s in (1, 2):
        g.fill_grads(s)
        if bucket:
            ssq = g.sumsq if clip else None
            if clip:
                g.shard.gnorm_bucketed(g.rows, bucket, g.sumsq, streams=2)
            g.shard.step_bucketed(None if clip else g.rows, bucket, w.lr, w.t_of(s), ssq,
                                  streams=2)
        else:
            g.step(s)
        torch.cuda.synchronize()
        s_orc = None
        if clip:
            _, s_orc = _rows(w, s, 0, n)
            s_gpu = float(g.sumsq.item())
            log(f"  step {s}: S gpu={s_gpu!r} oracle={s_orc!r}")
            nb = -(-n // bucket) if bucket else 1
            assert abs(s_gpu - s_orc) <= P.sumsq_tolerance(n, s_orc, buckets=nb)
        for (lo, hi), ow in zip(wins, ows):
            tag = f"{name} step {s} [{lo},{hi})"
            if clip:
                gbar, _ = _rows(w, s, lo, hi - lo)
                got = g.gbar_ws[lo:hi].cpu().numpy()
                assert np.array_equal(got.view(np.uint32), gbar.view(np.uint32)), f"{tag} spill"
            o = ow.step(s, sumsq_total=s_orc)
            got = g.host(lo, hi)
            P.f32_close(f"{tag} master", got["master"], ow.master)
            P.f32_close(f"{tag} m", got["m"], ow.m)
            P.f32_close(f"{tag} v", got["v"], ow.v)
            P.bf16_close(f"{tag} bf16", got["p"], o.p)
            if qb:
                P.int8_exact(f"{tag} int8", got["codes"], got["scales"], o.codes, o.scales,
                             got["p"], o.p, qb)
    g.free()
