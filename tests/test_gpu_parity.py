"""GPU parity: the HIP shard step against the CPU oracle on the same seeded
inputs, through the C ABI.

Tolerances (tests/_parity.py): fp32 master/m/v within 1e-9 + 2e-6|x|,
bf16 within 1 ulp, int8 codes and scales exact on identical bf16 input.
Small workloads are compared in full at every step; the full-size ones (in
the launch configuration the benchmark times) on windows the oracle
evolves element by element, compared at every step of the workload, plus
the global norm over the whole shard at every clipped step.
"""

from __future__ import annotations

import numpy as np
import pytest

import oracle as O
import seeded_inputs as S
import sharded_mixed_precision_zero_amd as Z
from tests import _parity as P
from tests._gpu import GpuShard, OracleWindow, log, oracle_global_sumsq, windows

pytestmark = pytest.mark.gpu


@pytest.fixture(autouse=True)
def _gpu_cleanup():
    import torch

    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    yield
    torch.cuda.synchronize()
    torch.cuda.empty_cache()


def _compare(name, g: dict, o: O.StepOut, ow: OracleWindow, block: int = 0) -> dict:
    st = {
        "master": P.f32_close(f"{name} master", g["master"], ow.master),
        "m": P.f32_close(f"{name} m", g["m"], ow.m),
        "v": P.f32_close(f"{name} v", g["v"], ow.v),
        "p": P.bf16_close(f"{name} bf16", g["p"], o.p),
    }
    if block:
        diff = P.int8_exact(f"{name} int8", g["codes"], g["scales"], o.codes, o.scales,
                            g["p"], o.p, block)
        st["int8_blocks_with_differing_input"] = int(diff.sum())
        # every block, those with differing input included: the GPU's codes
        # and scales are the quantizer's of the GPU's own bf16
        c_own, s_own = O.quant_int8(g["p"], block)
        assert np.array_equal(g["codes"], c_own), f"{name} int8 codes vs own bf16"
        assert np.array_equal(g["scales"].view(np.uint32), s_own.view(np.uint32)), \
            f"{name} int8 scales vs own bf16"
    return st


# -------------------------------------------------------------- generator

def test_generator_device_equals_host():
    import torch

    w = S.by_name("gpt2-small-flat")
    for (tid, sigma, outl, kind) in [(S.MASTER, 0.02, False, S.KIND_NORMAL),
                                     (S.VAR, 1e-6, False, S.KIND_ABS),
                                     (S.GRAD, 1e-3, True, S.KIND_NORMAL)]:
        t = torch.empty(100_003, dtype=torch.float32, device="cuda")
        S.dev_f32(t, w.seed, tid, 7, 3, 12_345_678, sigma, outl, kind)
        h = S.host_f32(100_003, w.seed, tid, 7, 3, 12_345_678, sigma, outl, kind)
        assert np.array_equal(t.cpu().numpy().view(np.uint32), h.view(np.uint32))
    buf = torch.empty(w.n_d * 5000, dtype=torch.int16, device="cuda")
    S.dev_contrib(w, 4, buf, 4000, 5000, i0=999)
    hb = S.host_contrib(w, 4, 999, 4000)
    got = buf.cpu().numpy().view(np.uint16).reshape(w.n_d, 5000)[:, :4000]
    assert np.array_equal(got, hb)


# ----------------------------------------------------- the five workloads

def test_tiny_zero1_full_every_step():
    w = S.by_name("tiny-zero1")
    log(f"case {w.name}: n={w.shard_len} n_d={w.n_d} steps={w.steps}")
    g = GpuShard(w)
    g.init_state()
    ow = OracleWindow(w, 0, w.shard_len)
    for s in range(1, w.steps + 1):
        g.fill_grads(s)
        g.step(s)
        o = ow.step(s)
        st = _compare(f"{w.name} step {s}", g.host(), o, ow)
    log(f"  final bitwise fractions: {st}")
    g.free()


def test_gpt2_small_full_every_step():
    w = S.by_name("gpt2-small-flat")
    n = w.shard_len
    log(f"case {w.name}: n={n} n_d={w.n_d} steps={w.steps} (outliers), full arrays every step")
    g = GpuShard(w)
    g.init_state()
    full = OracleWindow(w, 0, n)
    for s in range(1, w.steps + 1):
        g.fill_grads(s)
        g.step(s)
        o = full.step(s)
        st = _compare(f"{w.name} step {s}", g.host(), o, full)
        if s in (1, 2, 10, 50, w.steps):
            log(f"  step {s}: {st}")
    g.free()


def test_7p5b_nd64_windows():
    w = S.by_name("7.5B-nd64")
    n = w.shard_len
    log(f"case {w.name}: n={n} n_d={w.n_d} steps={w.steps} (warm state, t0={w.t0})")
    g = GpuShard(w)
    g.init_state()
    wins = windows(n, 16, 65536, seed=2)
    ows = [OracleWindow(w, lo, hi - lo) for lo, hi in wins]
    for s in range(1, w.steps + 1):
        g.fill_grads(s)
        g.step(s)
        for (lo, hi), ow in zip(wins, ows):
            o = ow.step(s)
            _compare(f"{w.name} step {s} [{lo},{hi})", g.host(lo, hi), o, ow)
    g.free()


def test_7p5b_zeropp_windows():
    """ZeRO++ both ways at the 7.5B, N_d = 64 size: int8 contributions in
    (qgZ, block 256), int8 weights out (qwZ, block 256)."""
    w = S.by_name("7.5B-nd64-zeropp")
    n = w.shard_len
    log(f"case {w.name}: n={n} n_d={w.n_d} steps={w.steps} contrib block={w.contrib_block}")
    g = GpuShard(w)
    g.init_state()
    wins = windows(n, 16, 65536, seed=5)
    ows = [OracleWindow(w, lo, hi - lo) for lo, hi in wins]
    for s in range(1, w.steps + 1):
        g.fill_grads(s)
        g.step(s)
        for (lo, hi), ow in zip(wins, ows):
            o = ow.step(s)
            _compare(f"{w.name} step {s} [{lo},{hi})", g.host(lo, hi), o, ow, w.quant_block)
    g.free()


def test_13b_clip_int8_full_norm_and_windows():
    """Clipped steps need the norm of the whole averaged gradient: the oracle
    streams all 16 x 812.5M contributions through the host for each of the
    workload's 10 steps; S and every window are compared at every step."""
    import torch

    w = S.by_name("13B-nd16-clip-int8")
    n = w.shard_len
    steps = w.steps
    log(f"case {w.name}: n={n} n_d={w.n_d} steps={steps} clip={w.max_norm} block={w.quant_block}")
    g = GpuShard(w)
    g.init_state()
    wins = windows(n, 16, 65536, seed=3)
    ows = [OracleWindow(w, lo, hi - lo) for lo, hi in wins]
    for s in range(1, steps + 1):
        g.fill_grads(s)
        g.step(s)
        torch.cuda.synchronize()
        s_gpu = float(g.sumsq.item())
        s_orc = oracle_global_sumsq(w, s)
        log(f"  step {s}: S gpu={s_gpu!r} oracle={s_orc!r} rel={abs(s_gpu - s_orc) / s_orc:.2e} "
            f"coef={O.clip_coef(s_orc, w.max_norm):.6f}")
        assert abs(s_gpu - s_orc) <= P.sumsq_tolerance(n, s_orc)
        for (lo, hi), ow in zip(wins, ows):
            o = ow.step(s, sumsq_total=s_orc)
            _compare(f"{w.name} step {s} [{lo},{hi})", g.host(lo, hi), o, ow, w.quant_block)
    g.free()


def test_13b_stage0_nd1_windows():
    w = S.by_name("13B-nd1-stage0")
    n = w.shard_len
    log(f"case {w.name}: n={n} n_d=1 steps={w.steps} (64-bit indexing, 205.6 GB resident)")
    bounds, acc = [], 0
    for _, sz in w.segments[:6]:
        acc += sz
        bounds.append(acc - 128)
    bounds += [(1 << 31) - 4096, (1 << 32) - 4096, n // 2]
    g = GpuShard(w)
    g.init_state()
    wins = windows(n, 16, 65536, seed=4, extra=tuple(bounds))
    ows = [OracleWindow(w, lo, hi - lo) for lo, hi in wins]
    for s in range(1, w.steps + 1):
        g.fill_grads(s)
        g.step(s)
        for (lo, hi), ow in zip(wins, ows):
            o = ow.step(s)
            _compare(f"{w.name} step {s} [{lo},{hi})", g.host(lo, hi), o, ow)
    g.free()


def test_7p5b_dequant_full_size_windows():
    """qwZ receive side at the 7.5B size: 64 int8 shards of 117,187,500 back
    to a 7.5e9-element bf16 vector (15 GB); windows at shard boundaries, the
    head and the tail against the oracle."""
    import torch

    w = S.by_name("7.5B-nd64-zeropp")
    phi, nd, blk = w.phi, w.n_d, w.quant_block
    per = w.shard_len
    log(f"case dequant phi={phi} n_d={nd} block={blk}")
    stride = (per + 127) // 128 * 128 + 640
    nb = -(-per // blk)
    sstride = (nb + 63) // 64 * 64 + 64
    codes = torch.empty(nd * stride, dtype=torch.int8, device="cuda")
    scales = torch.empty(nd * sstride, dtype=torch.float32, device="cuda")
    S.dev_contrib_q8(w, 1, codes, scales, per, stride, sstride)
    out = torch.empty(phi, dtype=torch.int16, device="cuda")
    crow = [codes[r * stride: r * stride + per] for r in range(nd)]
    srow = [scales[r * sstride: r * sstride + nb] for r in range(nd)]
    assert Z.zero_shard_dequant(crow, srow, nd, phi, blk, out) == Z.ZS_OK
    torch.cuda.synchronize()
    for r in (0, 1, 31, 62, 63):
        for j0 in (0, (per // 2) // blk * blk, per - per % blk - blk * 40):
            ln = min(blk * 48, per - j0)
            c_h, s_h = S.host_contrib_q8(w, 1, j0, ln)
            want = O.dequant_bf16([c_h[r]], [s_h[r]], ln, blk)
            got = out[r * per + j0: r * per + j0 + ln].cpu().numpy().view(np.uint16)
            assert np.array_equal(got, want), (r, j0)
    del out, codes, scales


# ------------------------------------------------------------ components

def test_gnorm_and_spill_match_oracle():
    import torch

    w = S.by_name("13B-nd16-clip-int8")
    for n in (1, 7, 4096 + 3, 1_000_000 + 5):
        log(f"case gnorm n={n} n_d={w.n_d}")
        g = GpuShard(w, n=n)
        g.fill_grads(1)
        g.shard.gnorm(g.rows, g.sumsq)
        torch.cuda.synchronize()
        gbar, s = O.gbar_sumsq(list(S.host_contrib(w, 1, 0, n)))
        assert np.array_equal(g.gbar_ws.cpu().numpy().view(np.uint32), gbar.view(np.uint32))
        assert abs(g.sumsq.item() - s) <= P.sumsq_tolerance(n, s)
        g.free()


@pytest.mark.parametrize("block", Z.QUANT_BLOCKS)
def test_quant_standalone_bit_exact(block):
    import torch

    for n in (1, 31, block, block + 8, 3 * block + 17, 200_000 + 3):
        log(f"case quant block={block} n={n}")
        w = S.by_name("tiny-zero1")
        g = GpuShard(w, n=n, quant_block=block)
        p = S.host_bf16(n, 77, S.AUX, block, 0, 0, 0.02)
        p[::97] = 0  # some zeros, and one all-zero block when it fits
        if n >= 2 * block:
            p[block:2 * block] = 0
        g.p.copy_(torch.from_numpy(p.view(np.int16)))
        g.shard.quant(block)
        torch.cuda.synchronize()
        codes, scales = O.quant_int8(p, block)
        assert np.array_equal(g.codes.cpu().numpy(), codes)
        assert np.array_equal(g.scales.cpu().numpy().view(np.uint32), scales.view(np.uint32))
        g.free()
