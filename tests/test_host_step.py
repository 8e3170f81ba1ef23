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


def test_host_step_thread_invariance():
    w = dataclasses.replace(S.by_name("13B-nd16-clip-int8"), quant_block=64)
    a = _run(w, 200_000, 2, 1)
    b = _run(w, 200_000, 2, 7)
    assert np.array_equal(a, b)


def _nonfinite_rows(n: int, nd: int) -> np.ndarray:
    """bf16 contributions with NaN, +-Inf and huge values planted in a few
    quantizer blocks (and one block of all zeros)."""
    rng = np.random.default_rng(7)
    x = (rng.standard_normal((nd, n)) * 1e-3).astype(np.float32)
    x[:, 64:128] = 0.0                 # zero gradient block (state moves by decay only)
    x[0, 130] = np.nan                 # NaN block
    x[1, 200] = np.inf                 # +Inf block
    x[2, 260] = -np.inf
    x[0, 300] = 3.0e38                 # large finite
    bits = x.view(np.uint32)
    rnd = 0x7FFF + ((bits >> 16) & 1)
    out = ((bits + rnd) >> 16).astype(np.uint16)
    out[np.isnan(x)] = 0x7FC0
    return out


def test_host_step_nonfinite_and_isa_equivalence(monkeypatch):
    """Non-finite gradients propagate (no step skipping) and quantize to the
    oracle's codes; the 512-bit and 256-bit host bodies give the same bits."""
    n, nd, qb = 1000, 4, 32
    rows = _nonfinite_rows(n, nd)
    w = dataclasses.replace(S.by_name("tiny-zero1"), quant_block=qb, weight_decay=0.01)
    results = []
    for no512 in (False, True):
        if no512:
            monkeypatch.setenv("ZS_HOST_NO_AVX512", "1")
        master, m, v = S.host_state(w, 0, n)
        om, mm, vm = master.copy(), m.copy(), v.copy()
        p = np.empty(n, np.uint16)
        codes = np.empty(n, np.int8)
        scales = np.empty(-(-n // qb), np.float32)
        d = Z.host_desc(phi=n, n_d=nd, r=0, shard_len=n, master=master, m=m, v=v, param_out=p,
                        weight_decay=w.weight_decay, quant_block=qb, q_codes=codes,
                        q_scales=scales)
        gbar, _ = O.gbar_sumsq(list(rows))
        assert Z.zero_shard_host_step(d, gbar.ctypes.data, w.lr, 1, 0.0, 3) == Z.ZS_OK
        h = O.Hyper(lr=w.lr, beta1=w.beta1, beta2=w.beta2, eps=w.eps,
                    weight_decay=w.weight_decay, t=1, quant_block=qb)
        o = O.step(list(rows), om, mm, vm, h)
        assert np.isnan(master).any() and np.isnan(om).any()
        for a, b in ((master, om), (m, mm), (v, vm)):
            same = (a.view(np.uint32) == b.view(np.uint32)) | (np.isnan(a) & np.isnan(b))
            assert same.all()
        assert np.array_equal(p & 0x7FFF > 0x7F80, o.p & 0x7FFF > 0x7F80)
        ok = (p == o.p) | ((p & 0x7FFF > 0x7F80) & (o.p & 0x7FFF > 0x7F80))
        assert ok.all()
        P.int8_exact("host quant", codes, scales, o.codes, o.scales, p, o.p, qb)
        assert np.array_equal(codes, o.codes)
        results.append((master.copy(), p.copy(), codes.copy(), scales.copy()))
    for a, b in zip(*results):
        assert np.array_equal(a.view(np.uint8), b.view(np.uint8))


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
