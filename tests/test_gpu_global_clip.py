"""Global-norm clipping across shards, on one GPU.

Gradient clipping ("ZeRO (딥 러닝)", "DeepSpeed에서 쓰기": gradient_clipping)
scales the whole averaged gradient by its norm over ALL shards, while each
rank updates only its own partition ("Data parallelism and ZeRO
optimization", "ZeRO-1": elementwise independence).  Here the N_d shards of
one flat buffer are N_d library handles on one GPU: each runs its norm pass
(S_r, left on the device), the host adds the S_r in shard order (the scalar
all-reduce between ranks), every shard updates with that global S, and the
concatenated shards are compared element by element with the oracle's
unpartitioned clipped step over the whole buffer, which takes its own S.

The clip threshold lies between every shard's own norm and the global norm,
so a shard that clipped by its own S alone would not clip at all: the
comparison fails unless the exchanged S is the one used.
"""

from __future__ import annotations

import dataclasses

import numpy as np
import pytest

import oracle as O
import seeded_inputs as S
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


def _workload(contrib: str, phi: int, nd: int) -> S.Workload:
    if contrib == "bf16":
        base = S.by_name("13B-nd16-clip-int8")
        return dataclasses.replace(base, phi=phi, n_d=nd)
    base = S.by_name("7.5B-nd64-zeropp")  # int8 contributions, block 256
    return dataclasses.replace(base, phi=phi, n_d=nd, weight_decay=0.1, max_norm=1.0,
                               warm=False, t0=0)


def _rows(w: S.Workload, s: int, lo: int, n: int):
    if w.contrib_block:
        codes, scales = S.host_contrib_q8(w, s, lo, n)
        return list(codes), list(scales)
    return list(S.host_contrib(w, s, lo, n)), None


def _gbar_sumsq(w, s, lo, n):
    a, b = _rows(w, s, lo, n)
    return O.gbar_sumsq_q8(a, b, w.contrib_block) if w.contrib_block else O.gbar_sumsq(a)


@pytest.mark.parametrize("contrib,phi,nd", [
    ("bf16", 1_000_003, 4),   # ragged last shard, int8 output blocks cut by the shards
    ("bf16", 600_000, 3),
    ("q8", 1_000_445, 4),     # shards of 250,112 = 977 blocks of 256 (qgZ scales align)
])
def test_exchanged_sumsq_equals_unpartitioned_clipped_step(contrib, phi, nd):
    import torch

    w0 = _workload(contrib, phi, nd)
    per = -(-phi // nd)
    bounds = [(r * per, min(phi, (r + 1) * per)) for r in range(nd)]
    # a threshold between the shards' own norms and the global norm (step 1)
    g_norm = np.sqrt(_gbar_sumsq(w0, 1, 0, phi)[1])
    local = max(np.sqrt(_gbar_sumsq(w0, 1, lo, hi - lo)[1]) for lo, hi in bounds)
    max_norm = float(np.float32(0.5 * (local + g_norm)))
    assert local < max_norm < g_norm
    w = dataclasses.replace(w0, max_norm=max_norm)
    log(f"case global clip {contrib} phi={phi} n_d={nd} per={per} max_norm={max_norm:.5g} "
        f"(shard norms <= {local:.5g} < global {g_norm:.5g})")
    shards = []
    for r, (lo, hi) in enumerate(bounds):
        g = GpuShard(w, n=hi - lo, i0=lo, phi=phi, r=r)
        g.init_state()
        shards.append(g)
    master, m, v = S.host_state(w, 0, phi)
    for s in (1, 2, 3):
        for g in shards:
            g.fill_grads(s)
            g.norm()
        torch.cuda.synchronize()
        s_r = [float(g.sumsq.item()) for g in shards]
        total = 0.0
        for x in s_r:  # the scalar exchange: shard order
            total += x
        for g in shards:
            g.sumsq.fill_(total)
            g.update(s)
        h = O.Hyper(lr=w.lr, beta1=w.beta1, beta2=w.beta2, eps=w.eps,
                    weight_decay=w.weight_decay, t=w.t_of(s), max_norm=max_norm)
        a, b = _rows(w, s, 0, phi)
        if w.contrib_block:
            out = O.step_q8(a, b, w.contrib_block, master, m, v, h, threads=4)
        else:
            out = O.step(a, master, m, v, h, threads=4)
        tol = sum(P.sumsq_tolerance(hi - lo, total) for lo, hi in bounds) + nd * 2.0**-53 * total
        assert abs(total - out.sumsq) <= tol, (total, out.sumsq, tol)
        torch.cuda.synchronize()
        for r, (g, (lo, hi)) in enumerate(zip(shards, bounds)):
            got = g.host()
            name = f"{contrib} step {s} shard {r} [{lo},{hi})"
            P.f32_close(f"{name} master", got["master"], master[lo:hi])
            P.f32_close(f"{name} m", got["m"], m[lo:hi])
            P.f32_close(f"{name} v", got["v"], v[lo:hi])
            P.bf16_close(f"{name} bf16", got["p"], out.p[lo:hi])
            # qwZ blocks start at each shard's element 0: the GPU's codes are
            # the quantizer's of its own bf16 shard, and equal the oracle's on
            # every block whose bf16 input is identical
            c_own, s_own = O.quant_int8(got["p"], w.quant_block)
            assert np.array_equal(got["codes"], c_own), name
            assert np.array_equal(got["scales"].view(np.uint32), s_own.view(np.uint32)), name
            c_o, s_o = O.quant_int8(out.p[lo:hi], w.quant_block)
            P.int8_exact(f"{name} int8", got["codes"], got["scales"], c_o, s_o, got["p"],
                         out.p[lo:hi], w.quant_block)
        log(f"  step {s}: S = {total!r} (oracle {out.sumsq!r}), coef "
            f"{O.clip_coef(total, max_norm):.6f}; every shard within tolerance")
    for g in shards:
        g.free()
