"""GPU properties that need no oracle run: the averaging identity on exact
(dyadic) inputs, inertness of zero padding, and elastic re-sharding.

* Least squares: the mean of per-rank gradients of a dyadic linear
  least-squares problem is the full-batch gradient ("How Standard Data
  Parallelism Works": the full-data gradient is the average of the subset
  gradients); with sparse rows every addend is exact in bf16, so the averaged gradient the
  norm pass spills must equal the exact full-batch gradient bit for bit.
* Padding: elements whose gradient, master, m and v are zero stay exactly
  +0 under AdamW with decay and clipping (a flat buffer pads segments with
  zeros; the update must not move them).
* Elastic re-sharding: the update is elementwise ("Data parallelism and
  ZeRO optimization", ZeRO-1: each rank updates only its partition), so
  concatenating four shards' state after some steps, re-slicing it into two
  shards and continuing gives the same bits as never re-slicing, when the
  averaged gradients are the same (here: contributions in equal pairs, so
  the average over 4 ranks is exactly the average over 2).
"""

from __future__ import annotations

import dataclasses
from fractions import Fraction

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


def _bf16_bits(vals) -> np.ndarray:
    """Exact bf16 patterns of values that are exact in bf16."""
    f = np.asarray(vals, dtype=np.float32)
    u = f.view(np.uint32)
    assert np.all((u & 0xFFFF) == 0), "value not exact in bf16"
    return (u >> 16).astype(np.uint16)


def _put_rows(g: GpuShard, rows) -> None:
    import torch

    for k, r in enumerate(rows):
        g.rows[k].copy_(torch.from_numpy(np.ascontiguousarray(r).view(np.int16)))


@pytest.mark.parametrize("nd,b,d", [(4, 4, 4099), (16, 2, 8200), (64, 1, 2051)])
def test_least_squares_average_is_full_batch_gradient(nd, b, d):
    import torch

    rng = np.random.default_rng(11 + nd)
    B = nd * b
    # four +-1 entries per row keep every residual within +-11 and every
    # per-rank gradient an integer below 2^8 over b: exact in bf16
    X = np.zeros((B, d), dtype=np.int64)
    for i in range(B):
        X[i, rng.choice(d, size=4, replace=False)] = rng.choice([-1, 1], size=4)
    theta = rng.integers(-2, 3, size=d)
    y = rng.integers(-3, 4, size=B)
    resid = X @ theta - y
    rows = []
    for r in range(nd):
        sl = slice(r * b, (r + 1) * b)
        rows.append(_bf16_bits((X[sl].T @ resid[sl]) / b))
    full = [Fraction(int(x), B) for x in X.T @ resid]
    w = dataclasses.replace(S.by_name("tiny-zero1"), n_d=nd, max_norm=1.0)
    log(f"case least squares nd={nd} b={b} d={d}")
    g = GpuShard(w, n=d)
    g.init_state()
    _put_rows(g, rows)
    g.norm()  # spills the averaged gradient
    torch.cuda.synchronize()
    got = g.gbar_ws.cpu().numpy()
    assert [Fraction(float(x)) for x in got] == full
    g.free()


def test_zero_padding_stays_zero():
    import torch

    w = dataclasses.replace(S.by_name("13B-nd16-clip-int8"), max_norm=0.05)
    n = 70_001
    pads = [(0, 640), (33_000, 33_128), (n - 129, n)]
    log(f"case zero padding n={n}")
    g = GpuShard(w, n=n)
    g.init_state()
    for lo, hi in pads:
        for a in (g.master, g.m, g.v):
            a[lo:hi].zero_()
    for s in range(1, 4):
        g.fill_grads(s)
        for lo, hi in pads:
            for r in g.rows:
                r[lo:hi].zero_()
        g.step(s)
    torch.cuda.synchronize()
    out = g.host()
    for lo, hi in pads:
        for name in ("master", "m", "v"):
            assert np.all(out[name][lo:hi].view(np.uint32) == 0), (name, lo, hi)
        assert np.all(out["p"][lo:hi] == 0)
        assert np.all(out["codes"][lo:hi] == 0)
    g.free()


def test_elastic_reshard_four_to_two():
    import torch

    phi = 1_000_003
    base = dataclasses.replace(S.by_name("tiny-zero1"), weight_decay=0.1, phi=phi)
    steps, cut = 4, 2

    def grads(s):  # two seeded gradient vectors over the whole buffer
        return [S.host_bf16(phi, base.seed, S.GRAD, s, k, 0, base.grad_sigma) for k in (0, 1)]

    def shards(nd):
        w = dataclasses.replace(base, n_d=nd)
        per = -(-phi // nd)
        out = []
        for r in range(nd):
            n = max(0, min(per, phi - r * per))
            out.append(GpuShard(w, n=n, i0=r * per, phi=phi, r=r, n_d=nd))
        return out, per

    def run(gs, per, nd, s):
        a, b = grads(s)
        src = [a, a, b, b] if nd == 4 else [a, b]
        for r, g in enumerate(gs):
            lo, hi = r * per, r * per + g.n
            _put_rows(g, [x[lo:hi] for x in src])
            g.update(s)

    def state(gs):
        torch.cuda.synchronize()
        parts = [g.host() for g in gs]
        return {k: np.concatenate([p[k] for p in parts]) for k in ("master", "m", "v", "p")}

    log(f"case elastic reshard phi={phi}")
    ref, per4 = shards(4)
    for g in ref:
        g.init_state()
    for s in range(1, steps + 1):
        run(ref, per4, 4, s)
    want = state(ref)
    for g in ref:
        g.free()

    four, _ = shards(4)
    for g in four:
        g.init_state()
    for s in range(1, cut + 1):
        run(four, per4, 4, s)
    mid = state(four)
    for g in four:
        g.free()
    two, per2 = shards(2)
    for r, g in enumerate(two):
        lo, hi = r * per2, r * per2 + g.n
        for name, t in (("master", g.master), ("m", g.m), ("v", g.v)):
            t.copy_(torch.from_numpy(mid[name][lo:hi]))
    for s in range(cut + 1, steps + 1):
        run(two, per2, 2, s)
    got = state(two)
    for g in two:
        g.free()
    for k in want:
        assert np.array_equal(want[k].view(np.uint8), got[k].view(np.uint8)), k
