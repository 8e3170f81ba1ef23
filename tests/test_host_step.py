"""ZeRO-Offload host step (zero_shard_host_step) on the CPU against the
oracle: the same binary64 arithmetic, so every output must agree bit for
bit (the stated tolerances are the gate; bit equality is also asserted
because nothing in the definitions leaves room for a difference).  No GPU."""

from __future__ import annotations

import dataclasses

import numpy as np
import pytest

import oracle as O
import seeded_inputs as S
import sharded_mixed_precision_zero_amd as Z
from tests import _parity as P


def _run(w, n, steps, threads, clip_total=True):
    master, m, v = S.host_state(w, 0, n)
    om, mm, vm = master.copy(), m.copy(), v.copy()
    p = np.empty(n, np.uint16)
    codes = np.empty(n, np.int8) if w.quant_block else None
    scales = (np.empty(-(-n // w.quant_block), np.float32) if w.quant_block else None)
    d = Z.host_desc(phi=n, n_d=w.n_d, r=0, shard_len=n, master=master, m=m, v=v, param_out=p,
                    beta1=w.beta1, beta2=w.beta2, eps=w.eps, weight_decay=w.weight_decay,
                    max_norm=w.max_norm, quant_block=w.quant_block, q_codes=codes,
                    q_scales=scales)
    for s in range(1, steps + 1):
        rows = list(S.host_contrib(w, s, 0, n))
        gbar, ssq = O.gbar_sumsq(rows)
        rc = Z.zero_shard_host_step(d, gbar.ctypes.data, w.lr, w.t_of(s), ssq, threads)
        assert rc == Z.ZS_OK
        h = O.Hyper(lr=w.lr, beta1=w.beta1, beta2=w.beta2, eps=w.eps,
                    weight_decay=w.weight_decay, t=w.t_of(s), max_norm=w.max_norm,
                    quant_block=w.quant_block)
        o = O.step(rows, om, mm, vm, h)
        for name, a, b in (("master", master, om), ("m", m, mm), ("v", v, vm)):
            P.f32_close(f"step {s} {name}", a, b)
            assert np.array_equal(a.view(np.uint32), b.view(np.uint32)), name
        P.bf16_close(f"step {s} bf16", p, o.p)
        assert np.array_equal(p, o.p)
        if w.quant_block:
            assert np.array_equal(codes, o.codes)
            assert np.array_equal(scales.view(np.uint32), o.scales.view(np.uint32))
    return master


@pytest.mark.parametrize("name,n,threads", [
    ("tiny-zero1", 1, 1),
    ("tiny-zero1", 262_144, 3),
    ("gpt2-small-flat", 100_003, 4),
    ("7.5B-nd64", 70_001, 2),
    ("13B-nd16-clip-int8", 300_001, 8),
])
def test_host_step_matches_oracle_bitwise(name, n, threads):
    _run(S.by_name(name), n, 3, threads)


def test_host_step_thread_invariance_and_bias_off():
    w = dataclasses.replace(S.by_name("13B-nd16-clip-int8"), quant_block=64)
    a = _run(w, 200_000, 2, 1)
    b = _run(w, 200_000, 2, 7)
    assert np.array_equal(a, b)


def test_host_step_rejects_bad_arguments():
    n = 16
    x = np.zeros(n, np.float32)
    p = np.zeros(n, np.uint16)
    d = Z.host_desc(phi=n, n_d=1, r=0, shard_len=n, master=x, m=x.copy(), v=x.copy(), param_out=p)
    g = np.zeros(n, np.float32)
    assert Z.zero_shard_host_step(d, g.ctypes.data, 1e-3, 0) == Z.ZS_EINVAL
    assert Z.zero_shard_host_step(d, g.ctypes.data, -1.0, 1) == Z.ZS_EINVAL
    assert Z.zero_shard_host_step(d, None, 1e-3, 1) == Z.ZS_EINVAL
    bad = Z.host_desc(phi=n, n_d=1, r=0, shard_len=n, master=x, m=x, v=x, param_out=p,
                      quant_block=256)
    assert Z.zero_shard_host_step(bad, g.ctypes.data, 1e-3, 1) == Z.ZS_EINVAL
    empty = Z.host_desc(phi=3, n_d=4, r=3, shard_len=0, master=None, m=None, v=None,
                        param_out=None)
    assert Z.zero_shard_host_step(empty, None, 1e-3, 1) == Z.ZS_OK
