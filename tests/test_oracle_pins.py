"""Pins of the CPU oracle to facts fixed outside it.

Each test checks one oracle routine against something it cannot simply
restate: numbers the pages print, closed forms of the mathematics, exact
rational arithmetic, exhaustive enumeration, or hand-worked tables.  Each is
chosen so that a plausible slip (a dropped term, a wrong sign, an off-by-one
step counter, a transposed operand, a wrong rounding direction) fails it.
"""

from __future__ import annotations

import json
import os
import subprocess
import tempfile
from fractions import Fraction

import numpy as np
import pytest

import oracle as O
import seeded_inputs as S

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")
ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _bf16_bits(values) -> np.ndarray:
    """bf16 patterns of values that are exactly representable in bf16."""
    f = np.asarray(values, dtype=np.float32)
    u = f.view(np.uint32)
    assert np.all((u & 0xFFFF) == 0), "value not exact in bf16"
    return (u >> 16).astype(np.uint16)


def _bf16_to_float(bits: np.ndarray) -> np.ndarray:
    return (bits.astype(np.uint32) << 16).view(np.float32)


# ------------------------------------------------------------- memory model

def test_memory_model_printed_values():
    g = json.load(open(os.path.join(GOLDEN, "memory_model.json")))
    for c in g["cases"]:
        got = O.model_state_bytes(c["psi"], c["n_d"], c["stage"]) / 1e9
        assert round(got, c["digits"]) == c["gb"], c["source"]
    # GPT-2 1.5B: at least 24 GB of model states against 3 GB of
    # half-precision weights, a ratio of (2+2+K)/2 = 8
    hw = g["half_weights"]
    assert O.model_state_bytes(hw["psi"], 1, 0) / 1e9 / hw["gb"] == 8.0


def test_memory_model_limits_and_consistency():
    lim = json.load(open(os.path.join(GOLDEN, "memory_model.json")))["limits"]
    psi = 1e9
    base = O.model_state_bytes(psi, 1, 0)
    assert base == 16 * psi
    big = 1e9  # N_d -> infinity
    assert abs(base / O.model_state_bytes(psi, big, 1) - lim["stage1"]) < 1e-6
    assert abs(base / O.model_state_bytes(psi, big, 2) - lim["stage2"]) < 1e-6
    for nd in (2, 8, 64, 1024):
        assert base / O.model_state_bytes(psi, nd, 3) == pytest.approx(nd, rel=1e-12)
        # every stage is bounded by the one before it
        s = [O.model_state_bytes(psi, nd, k) for k in range(4)]
        assert s[0] > s[1] > s[2] > s[3]
    # with one GPU every stage is plain data parallelism
    for k in range(4):
        assert O.model_state_bytes(psi, 1, k) == base


# ---------------------------------------------------------------- bf16 cast

def test_bf16_round_exhaustive():
    """All 2^32 binary32 patterns against a nearest-neighbour definition."""
    src = os.path.join(ROOT, "tests", "native", "bf16_exhaustive.c")
    so = O.LIB_PATH
    with tempfile.TemporaryDirectory() as d:
        exe = os.path.join(d, "bf16ex")
        subprocess.run(["gcc", "-O2", src, so, f"-Wl,-rpath,{os.path.dirname(so)}", "-lm",
                        "-pthread", "-o", exe], check=True)
        r = subprocess.run([exe], capture_output=True, text=True, timeout=600)
    assert r.returncode == 0, r.stdout + r.stderr
    assert "mismatches 0" in r.stdout


def test_fp32_master_keeps_small_updates():
    """fp32 master weights exist so that small updates do not vanish
    ("Memory Consumption Analysis": optimizer state in fp32 so that tiny
    updates do not underflow; "精度混合训练": the fp32 parameter is the final
    output).  theta = 1 with |step| ~ 1e-4, far below half a bf16 ulp at 1
    (2^-8): a bf16-only weight never moves, the fp32 master moves every step
    and its bf16 copy changes once the drift passes 2^-8 (rounded)."""
    n = 1
    rows = [_bf16_bits([1.0])]                   # constant gradient g = 1
    h = O.Hyper(lr=1e-4, beta1=0.9, beta2=0.999, eps=1e-8)
    master = np.ones(n, np.float32)
    m = np.zeros(n, np.float32)
    v = np.zeros(n, np.float32)
    bf16_only = np.float32(1.0)
    seen = []
    for t in range(1, 31):
        h.t = t
        out = O.step(rows, master, m, v, h)
        seen.append((float(master[0]), int(out.p[0])))
        # a bf16-only update: round(1 - 1e-4) in bf16 is 1 again
        bf16_only = _bf16_to_float(O.f32_to_bf16(np.array([bf16_only - np.float32(1e-4)])))[0]
    assert bf16_only == 1.0
    # constant g from zero state: every step is lr*g/(|g|+eps) ~ 1e-4
    assert seen[9][0] == pytest.approx(1 - 10 * 1e-4, abs=1e-6)
    assert seen[9][1] == 0x3F80                   # bf16 copy still reads 1.0
    # 1 - k*1e-4 rounds to bf16 1 - 2^-8 once k*1e-4 > 2^-9 (k >= 20)
    first = next(t for t, (_, p) in enumerate(seen, 1) if p != 0x3F80)
    assert first == 20
    assert seen[first - 1][1] == 0x3F7F           # 0.99609375 = 1 - 2^-8


# ------------------------------------------------------- a1 reduce + average

def test_reduce_average_least_squares_identity():
    """The mean of per-rank gradients equals the full-batch gradient
    ("How Standard Data Parallelism Works": the full-data gradient is the
    average of the subset gradients).  Linear least squares
    L(theta) = 1/(2B) ||X theta - y||^2 with X in {-1,0,1}, small integer y and
    theta, B = N_d * b with b a power of two: every per-rank gradient
    (1/b) X_r^T (X_r theta - y_r) is a dyadic number with <= 8 significant
    bits (exact in bf16), so the oracle's average must equal the full-batch
    gradient (1/B) X^T (X theta - y), computed exactly, bit for bit."""
    rng = np.random.default_rng(7)
    for nd, b, d in [(4, 4, 16), (8, 2, 32), (16, 4, 24), (64, 1, 24)]:
        B = nd * b
        X = rng.integers(-1, 2, size=(B, d))
        theta = rng.integers(-2, 3, size=d)
        y = rng.integers(-3, 4, size=B)
        resid = X @ theta - y
        rows = []
        for r in range(nd):
            sl = slice(r * b, (r + 1) * b)
            gr = [Fraction(int(x), b) for x in X[sl].T @ resid[sl]]
            rows.append(_bf16_bits([float(x) for x in gr]))
        full = [Fraction(int(x), B) for x in X.T @ resid]
        got = O.reduce_average(rows)
        assert [Fraction(float(x)) for x in got] == full, (nd, b, d)


def test_reduce_sum_exact_audit():
    """The fp64 rank-order sum is the exact sum of the bf16 contributions
    (exact rationals) on seeded draws, outliers included."""
    w = S.by_name("gpt2-small-flat")
    for i0 in (0, 1_000_003, w.shard_len - 4096):
        rows = S.host_contrib(w, 1, i0, 4096)
        s = O.reduce_sum(list(rows))
        vals = _bf16_to_float(rows)
        for i in range(0, 4096, 7):
            exact = sum(Fraction(float(vals[k, i])) for k in range(w.n_d))
            assert Fraction(float(s[i])) == exact
        # and the average is that exact sum / N_d rounded once to binary32
        gbar = O.reduce_average(list(rows))
        assert np.array_equal(gbar, (s / w.n_d).astype(np.float32))


def test_reduce_single_rank_is_conversion():
    bits = S.host_bf16(10_000, 99, S.GRAD, 1, 0, 0, 1e-3)
    assert np.array_equal(O.reduce_average([bits]), _bf16_to_float(bits))


def test_reduce_uses_every_rank_in_place():
    """Moving one unit between ranks keeps the mean; a unit in rank k shows
    up in the mean as 1/N_d at its own index only (no index mix-up)."""
    nd, n = 8, 64
    for k in range(nd):
        rows = [np.zeros(n, np.uint16) for _ in range(nd)]
        rows[k][k * 3] = _bf16_bits([8.0])[0]
        g = O.reduce_average(rows)
        want = np.zeros(n, np.float32)
        want[k * 3] = 1.0
        assert np.array_equal(g, want)


# ------------------------------------------------------------ a3 Adam forms

def _adam_run(g_seq, theta0, h: O.Hyper, m0=None, v0=None):
    n = len(theta0)
    master = np.array(theta0, np.float32)
    m = np.zeros(n, np.float32) if m0 is None else np.array(m0, np.float32)
    v = np.zeros(n, np.float32) if v0 is None else np.array(v0, np.float32)
    hist = []
    for t, g in enumerate(g_seq, 1):
        h.t = t
        O.adam(master, m, v, np.asarray(g, np.float32), 1.0, h)
        hist.append(master.copy())
    return hist, m, v


def test_adam_first_step_closed_form():
    """From m = v = 0, bias-corrected Adam's first step is
    -lr * g / (|g| + eps) whatever beta1, beta2 (m_hat = g, v_hat = g^2).
    Includes gradients far below eps, where the step is ~ -lr g / eps."""
    g = np.concatenate([S.host_f32(2000, 5, S.GRAD, 1, 0, 0, 1e-3),
                        np.array([1e-12, -3e-10, 5e-9, 1e-8, -2e-8, 0.0, 0.25], np.float32)])
    theta0 = S.host_f32(g.size, 5, S.MASTER, 0, 0, 0, 0.02)
    for b1, b2, lr, eps in [(0.9, 0.999, 1e-3, 1e-8), (0.5, 0.95, 1e-4, 1e-6)]:
        h = O.Hyper(lr=lr, beta1=b1, beta2=b2, eps=eps)
        (th1,), _, _ = _adam_run([g], theta0, h)
        lr64, eps64 = float(np.float32(lr)), float(np.float32(eps))
        g64 = g.astype(np.float64)
        want = theta0.astype(np.float64) - lr64 * g64 / (np.abs(g64) + eps64)
        # the oracle rounds theta' once; m_hat, v_hat carry a few binary64 ulps
        assert np.all(np.abs(th1 - want) <= np.spacing(np.abs(want).astype(np.float32)))


def test_adam_constant_gradient_closed_form():
    """Constant g from zero state: m_hat = g and v_hat = g^2 at every t (the
    bias corrections undo the geometric sums exactly), so
    theta_T = theta_0 - T lr g / (|g| + eps).  A wrong exponent in a bias
    correction, or t off by one, breaks this from step 2 on."""
    g = np.array([1e-3, -2e-4, 0.5, -7e-6, 3e-9], np.float32)
    theta0 = np.zeros(g.size, np.float32)
    h = O.Hyper(lr=1e-3, beta1=0.9, beta2=0.999, eps=1e-8)
    T = 25
    hist, _, _ = _adam_run([g] * T, theta0, h)
    lr, eps = float(np.float32(1e-3)), float(np.float32(1e-8))
    g64 = g.astype(np.float64)
    for t, th in enumerate(hist, 1):
        want = -t * lr * g64 / (np.abs(g64) + eps)
        # fp32 rounding of m, v and theta per step: a few ulps per step
        assert np.allclose(th, want, rtol=2e-6, atol=0), t


def test_adam_warm_state_against_50_digit_evaluation():
    """The general update (warm m and v, t > 1, decay, a clip coefficient)
    evaluated in 50-digit decimal arithmetic from the same binary32 inputs
    and binary32 hyper-parameters: the oracle's stored binary32 results are
    the correctly rounded exact values to within one ulp (the binary64 path
    rounds a few times before the final rounding), and almost always equal.
    A dropped term, a wrong sign or a wrong bias-correction exponent moves
    results by far more than an ulp."""
    from decimal import Decimal, getcontext

    getcontext().prec = 50
    rng = np.random.default_rng(5)
    n = 2000
    theta = rng.normal(0, 0.02, n).astype(np.float32)
    m = rng.normal(0, 1e-4, n).astype(np.float32)
    v = np.abs(rng.normal(0, 1e-6, n)).astype(np.float32)
    gbar = rng.normal(0, 1e-3, n).astype(np.float32)
    gbar[:20] = 0.0
    gbar[20:40] *= 1e-6  # |g| well below eps
    coef, t = 0.37, 7
    h = O.Hyper(lr=1e-3, beta1=0.9, beta2=0.999, eps=1e-8, weight_decay=0.1, t=t)
    f = lambda x: Decimal(float(np.float32(x)))  # noqa: E731  the binary32 value, exactly
    lr, b1, b2, eps, wd = f(h.lr), f(h.beta1), f(h.beta2), f(h.eps), f(h.weight_decay)
    bc1, bc2 = 1 - b1 ** t, 1 - b2 ** t
    c = Decimal(coef)
    want = {"theta": [], "m": [], "v": []}
    for i in range(n):
        g = c * Decimal(float(gbar[i]))
        m1 = b1 * Decimal(float(m[i])) + (1 - b1) * g
        v1 = b2 * Decimal(float(v[i])) + (1 - b2) * g * g
        th = Decimal(float(theta[i]))
        t1 = th - lr * wd * th - lr * (m1 / bc1) / ((v1 / bc2).sqrt() + eps)
        want["theta"].append(t1)
        want["m"].append(m1)
        want["v"].append(v1)
    th_o, m_o, v_o = theta.copy(), m.copy(), v.copy()
    O.adam(th_o, m_o, v_o, gbar, coef, h)
    for name, got in (("theta", th_o), ("m", m_o), ("v", v_o)):
        exact = want[name]
        nearest = np.array([float(x) for x in exact], np.float64).astype(np.float32)
        # np.float32(binary64) rounds twice; settle ties of the exact value
        # directly: the distance in ulps of the oracle's result to the exact
        ulp = np.spacing(np.abs(got)).astype(np.float64)
        err = np.array([abs(Decimal(float(got[i])) - exact[i]) / Decimal(float(ulp[i]))
                        if ulp[i] > 0 else Decimal(0) for i in range(n)], dtype=object)
        assert all(e <= 1 for e in err), name
        same = np.mean(got.view(np.uint32) == nearest.view(np.uint32))
        assert same >= 0.99, (name, same)


def test_adam_decoupled_weight_decay_alone():
    """g = 0 everywhere: m = v = 0, the Adam term is 0/(0+eps) = 0, and the
    decoupled decay gives theta_t = theta_0 (1 - lr wd)^t."""
    theta0 = np.array([0.02, -1.5, 3.0, 1e-30], np.float32)
    h = O.Hyper(lr=1e-2, weight_decay=0.1)
    T = 40
    hist, m, v = _adam_run([np.zeros(4, np.float32)] * T, theta0, h)
    assert not m.any() and not v.any()
    k = 1.0 - float(np.float32(1e-2)) * float(np.float32(0.1))
    for t, th in enumerate(hist, 1):
        assert np.allclose(th, theta0.astype(np.float64) * k**t, rtol=2e-7 * t, atol=0)


def test_adam_beta1_zero_alternating_sign():
    """beta1 = 0 and g_t = +c, -c, +c, ...: m' = g_t and v_hat = c^2 at every
    t, so theta moves by -lr c/(c+eps) then back by +lr c/(c+eps)."""
    c = np.float32(2e-3)
    theta0 = np.array([0.1], np.float32)
    h = O.Hyper(lr=1e-3, beta1=0.0, beta2=0.99, eps=1e-8)
    seq = [np.array([c if t % 2 else -c], np.float32) for t in range(1, 21)]
    hist, _, _ = _adam_run(seq, theta0, h)
    d = float(np.float32(1e-3)) * float(c) / (float(c) + float(np.float32(1e-8)))
    for t, th in enumerate(hist, 1):
        want = 0.1 - d if t % 2 else 0.1
        assert abs(float(th[0]) - want) <= 4 * np.spacing(np.float32(0.1))


# ---------------------------------------------------------- a2 norm + clip

def test_sumsq_all_equal_closed_form():
    """All ranks send c and all elements equal: gbar = c, sum of squares
    n c^2 exactly, norm |c| sqrt(n) = |c| 2^k for n = 4^k."""
    for c, k in [(0.75, 10), (-3.0, 6), (2.0**-20, 8)]:
        n = 4**k
        rows = [np.full(n, _bf16_bits([c])[0], np.uint16) for _ in range(4)]
        g, s = O.gbar_sumsq(rows, threads=3)
        assert s == n * c * c
        assert np.sqrt(s) == abs(c) * 2**k
        assert O.clip_coef(s, 1.0) == min(1.0, 1.0 / (abs(c) * 2**k + 1e-6))


def test_clip_inactive_is_unclipped_and_scaling_halves_coef():
    w = S.by_name("tiny-zero1")
    n = 50_000
    rows = S.host_contrib(w, 1, 0, n)
    g, s = O.gbar_sumsq(list(rows))
    norm = np.sqrt(s)
    base = dict(lr=1e-3, t=1)
    outs = []
    for max_norm in (0.0, norm * 1.5, norm * 100):
        master, m, v = S.host_state(w, 0, n)
        outs.append((O.step(list(rows), master, m, v, O.Hyper(max_norm=max_norm, **base)), master))
    for o, mst in outs[1:]:
        assert np.array_equal(mst, outs[0][1]) and np.array_equal(o.p, outs[0][0].p)
    # doubling every contribution (exact in bf16) quadruples the sum of squares
    rows2 = (rows.astype(np.uint32) + (1 << 7)).astype(np.uint16)  # exponent + 1
    rows2[rows == 0] = 0
    _, s2 = O.gbar_sumsq(list(rows2))
    assert s2 == 4 * s
    c1, c2 = O.clip_coef(s, norm / 4), O.clip_coef(s2, norm / 4)
    assert c1 == pytest.approx(0.25, rel=1e-4) and c2 == pytest.approx(c1 / 2, rel=1e-4)


def test_sumsq_thread_and_chunk_invariance():
    w = S.by_name("tiny-zero1")
    rows = S.host_contrib(w, 2, 0, w.shard_len)
    r = [O.gbar_sumsq(list(rows), threads=t) for t in (1, 2, 5)]
    assert r[0][1] == r[1][1] == r[2][1]
    assert np.array_equal(r[0][0], r[2][0])


# -------------------------------------------------------------- a5 quantize

def test_quant_hand_tables():
    g = json.load(open(os.path.join(GOLDEN, "quant_ties.json")))
    for c in g["cases"]:
        codes, scales = O.quant_int8(_bf16_bits(c["p"]), c["block"])
        assert codes.tolist() == c["codes"], c["why"]
        assert scales.tolist() == c["scales"], c["why"]


def test_quant_structure_on_draws():
    """On seeded bf16 shards: the absmax element of each block codes to
    +-127, every code reconstructs its value within half a step, the code
    of -p is -code(p), and a block's codes depend on that block only."""
    p = S.host_bf16(256 * 40 + 32, 11, S.AUX, 0, 0, 0, 0.02)
    codes, scales = O.quant_int8(p, 256)
    assert scales.size == 41
    x = _bf16_to_float(p).astype(np.float64)
    for b in range(41):
        blk = slice(b * 256, min((b + 1) * 256, p.size))
        a = np.abs(x[blk]).max()
        assert abs(scales[b] - a / 127) <= np.spacing(np.float32(a / 127))
        assert np.abs(codes[blk]).max() == 127
        err = np.abs(codes[blk] * float(scales[b]) - x[blk])
        assert np.all(err <= (0.5 + 1e-5) * float(scales[b]))
    neg = (p ^ np.uint16(0x8000)).astype(np.uint16)
    c2, s2 = O.quant_int8(neg, 256)
    assert np.array_equal(c2, -codes) and np.array_equal(s2, scales)
    # the tail block of 32 alone gives the same codes as inside the shard
    ct, st = O.quant_int8(p[-32:], 256)
    assert np.array_equal(ct, codes[-32:]) and st[0] == scales[-1]


# ------------------------------------------------------------- whole step

def _whole_step(w, n, steps, threads=1, quant_block=0, max_norm=0.0):
    master, m, v = S.host_state(w, 0, n)
    out = None
    for s in range(1, steps + 1):
        rows = S.host_contrib(w, s, 0, n)
        h = O.Hyper(lr=w.lr, beta1=w.beta1, beta2=w.beta2, eps=w.eps,
                    weight_decay=w.weight_decay, t=w.t_of(s), max_norm=max_norm,
                    quant_block=quant_block)
        out = O.step(list(rows), master, m, v, h, threads=threads)
    return master, m, v, out


def test_shard_concatenation_equals_unpartitioned():
    """Elementwise independence ("ZeRO-1": a parameter's optimizer state
    depends only on its own gradient): updating N_d shards separately and
    concatenating equals updating the whole flat buffer, bit for bit."""
    w = S.by_name("tiny-zero1")
    n = 3 * 65536 + 1000
    whole = _whole_step(w, n, 3, quant_block=256)
    nd = 4
    per = -(-n // nd)
    per = -(-per // 256) * 256  # shard boundaries on block boundaries
    parts = []
    for r in range(nd):
        lo, hi = r * per, min(n, (r + 1) * per)
        master, m, v = S.host_state(w, lo, hi - lo)
        for s in range(1, 4):
            rows = S.host_contrib(w, s, lo, hi - lo)
            out = O.step(list(rows), master, m, v,
                         O.Hyper(lr=w.lr, t=s, quant_block=256))
        parts.append((master, m, v, out))
    assert np.array_equal(np.concatenate([p[0] for p in parts]), whole[0])
    assert np.array_equal(np.concatenate([p[1] for p in parts]), whole[1])
    assert np.array_equal(np.concatenate([p[2] for p in parts]), whole[2])
    assert np.array_equal(np.concatenate([p[3].p for p in parts]), whole[3].p)
    assert np.array_equal(np.concatenate([p[3].codes for p in parts]), whole[3].codes)
    assert np.array_equal(np.concatenate([p[3].scales for p in parts]), whole[3].scales)


def test_elastic_reslice_continues_bitwise():
    """Re-sharding is a re-slice of the fp32 state (elementwise independence,
    "ZeRO-1"): four shards stepped twice, concatenated, cut into two shards
    and stepped twice more equal four shards stepped four times, when the
    averaged gradient is the same (contributions in equal pairs: the mean
    over [a, a, b, b] is exactly the mean over [a, b])."""
    w = S.by_name("tiny-zero1")
    phi = 100_003

    def grads(s):
        return [S.host_bf16(phi, w.seed, S.GRAD, s, k, 0, w.grad_sigma) for k in (0, 1)]

    def run(state, nd, steps):
        master, m, v = state
        per = -(-phi // nd)
        for s in steps:
            a, b = grads(s)
            src = [a, a, b, b] if nd == 4 else [a, b]
            for r in range(nd):
                lo, hi = r * per, min(phi, (r + 1) * per)
                sl = slice(lo, hi)
                mm, mo, va = master[sl].copy(), m[sl].copy(), v[sl].copy()
                O.step([x[sl] for x in src], mm, mo, va,
                       O.Hyper(lr=w.lr, weight_decay=0.1, t=s))
                master[sl], m[sl], v[sl] = mm, mo, va
        return master, m, v

    ref = run(S.host_state(w, 0, phi), 4, range(1, 5))
    mid = run(S.host_state(w, 0, phi), 4, range(1, 3))
    got = run(mid, 2, range(3, 5))
    for x, y in zip(ref, got):
        assert np.array_equal(x.view(np.uint32), y.view(np.uint32))


def test_step_thread_invariance():
    w = S.by_name("13B-nd16-clip-int8")
    n = (1 << 20) * 2 + 777
    a = _whole_step(w, n, 2, threads=1, quant_block=256, max_norm=1.0)
    b = _whole_step(w, n, 2, threads=4, quant_block=256, max_norm=1.0)
    for x, y in zip(a[:3], b[:3]):
        assert np.array_equal(x, y)
    assert a[3].sumsq == b[3].sumsq
    assert np.array_equal(a[3].codes, b[3].codes)


def test_step_empty_shard_and_bad_args():
    h = O.Hyper()
    e = np.zeros(0, np.float32)
    out = O.step([np.zeros(0, np.uint16)] * 3, e, e.copy(), e.copy(), h)
    assert out.p.size == 0 and out.sumsq == 0.0
    with pytest.raises(ValueError):
        O.step([np.zeros(4, np.uint16)], np.zeros(4, np.float32), np.zeros(4, np.float32),
               np.zeros(4, np.float32), O.Hyper(t=0))


# ------------------------------------------- a1 with int8 contributions (qgZ)

def test_q8_reduce_exact_audit():
    """The rank-order binary64 sum of the products code * scale is the exact
    rational sum on the 64-rank workload's draws, and the average is that
    sum / N_d rounded once."""
    w = S.by_name("7.5B-nd64-zeropp")
    codes, scales = S.host_contrib_q8(w, 1, 256 * 10, 2048 + 100)
    s = O.reduce_sum_q8(list(codes), list(scales), 256)
    for i in range(0, codes.shape[1], 11):
        exact = sum(Fraction(int(codes[k, i])) * Fraction(float(scales[k, i // 256]))
                    for k in range(w.n_d))
        assert Fraction(float(s[i])) == exact
    g = O.reduce_average_q8(list(codes), list(scales), 256)
    assert np.array_equal(g, (s / w.n_d).astype(np.float32))


def test_q8_reduce_matches_bf16_reduce_on_exact_values():
    """With power-of-two scales every code * scale is an exact bf16 value
    (|code| <= 127 has at most 7 significant bits), so the int8 front end must
    agree bit for bit with the pinned bf16 reduce of those values."""
    rng = np.random.default_rng(3)
    nd, n, block = 8, 1000, 64
    codes = rng.integers(-127, 128, size=(nd, n)).astype(np.int8)
    nb = (n + block - 1) // block
    scales = np.ldexp(1.0, -rng.integers(5, 30, size=(nd, nb))).astype(np.float32)
    vals = codes.astype(np.float64) * np.repeat(scales, block, axis=1)[:, :n]
    rows = [_bf16_bits(vals[k].astype(np.float32)) for k in range(nd)]
    g8 = O.reduce_average_q8(list(codes), list(scales), block)
    assert np.array_equal(g8, O.reduce_average(rows))


def test_q8_roundtrip_through_the_block_quantizer():
    """Quantizing each rank's bf16 gradient with the a5 quantizer and reducing
    the codes lands within the ranks' half quantization steps (averaged) of
    the bf16 reduce: the two front ends describe the same gradient."""
    w = S.by_name("gpt2-small-flat")
    n, block = 5000, 256
    rows = S.host_contrib(w, 1, 0, n)
    qs = [O.quant_int8(rows[k], block) for k in range(w.n_d)]
    g8 = O.reduce_average_q8([c for c, _ in qs], [s for _, s in qs], block)
    g = O.reduce_average(list(rows))
    half = sum(np.repeat(s.astype(np.float64), block)[:n] for _, s in qs) / 2 / w.n_d
    err = np.abs(g8.astype(np.float64) - g.astype(np.float64))
    assert np.all(err <= half * (1 + 1e-6) + np.spacing(np.abs(g)))
    assert err.max() > 0  # quantization is not the identity here


def test_q8_block_indexing():
    """A scale in block b of rank k acts on block b's elements of rank k only."""
    nd, n, block = 4, 320, 32
    for k, b in [(0, 0), (3, 9), (2, 4)]:
        codes = [np.ones(n, np.int8) for _ in range(nd)]
        scales = [np.zeros((n + block - 1) // block, np.float32) for _ in range(nd)]
        scales[k][b] = 4.0
        g = O.reduce_average_q8(codes, scales, block)
        want = np.zeros(n, np.float32)
        want[b * block:(b + 1) * block] = 1.0
        assert np.array_equal(g, want)


def test_q8_step_equals_step_on_exact_values():
    """The whole q8 step equals the bf16 step when the values coincide."""
    rng = np.random.default_rng(5)
    nd, n, block = 16, 3000, 256
    codes = rng.integers(-127, 128, size=(nd, n)).astype(np.int8)
    nb = (n + block - 1) // block
    scales = np.ldexp(1.0, -rng.integers(14, 18, size=(nd, nb))).astype(np.float32)
    vals = codes.astype(np.float64) * np.repeat(scales, block, axis=1)[:, :n]
    rows = [_bf16_bits(vals[k].astype(np.float32)) for k in range(nd)]
    w = S.by_name("13B-nd16-clip-int8")
    outs = []
    for fn in ("q8", "bf16"):
        master, m, v = S.host_state(w, 0, n)
        h = O.Hyper(lr=1e-4, weight_decay=0.1, max_norm=0.01, quant_block=256, t=1)
        o = (O.step_q8(list(codes), list(scales), block, master, m, v, h) if fn == "q8"
             else O.step(rows, master, m, v, h))
        outs.append((master, m, v, o))
    for x, y in zip(outs[0][:3], outs[1][:3]):
        assert np.array_equal(x, y)
    assert np.array_equal(outs[0][3].codes, outs[1][3].codes)
    assert outs[0][3].sumsq == outs[1][3].sumsq


# ------------------------------------------------- qwZ receive side (dequant)

def test_dequant_hand_values_and_shard_geometry():
    """Values by hand: code * scale exact in bf16 come back exactly; each
    shard lands at r * ceil(phi / n_d) with its own block numbering."""
    phi, nd, block = 10, 4, 2                # shards of 3, 3, 3, 1
    codes = [np.array([1, -2, 3], np.int8), np.array([127, 0, -127], np.int8),
             np.array([5, 6, 7], np.int8), np.array([-1], np.int8)]
    scales = [np.array([0.5, 4.0], np.float32), np.array([1.0, 0.25], np.float32),
              np.array([-2.0, 1.0], np.float32), np.array([3.0], np.float32)]
    out = _bf16_to_float(O.dequant_bf16(codes, scales, phi, block))
    assert out.tolist() == [0.5, -1.0, 12.0, 127.0, 0.0, -31.75, -10.0, -12.0, 7.0, -3.0]


def test_dequant_roundtrips_the_quantizer():
    """qwZ end to end on one shard: quantize a bf16 shard with the a5 rule,
    dequantize: every element comes back within half a quantization step
    (plus the two roundings to binary32 and bf16), the block absmax element
    within a relative 2^-8, and zero blocks as zeros."""
    p = S.host_bf16(256 * 20 + 77, 21, S.AUX, 0, 0, 0, 0.02)
    p[256 * 3:256 * 4] = 0
    codes, scales = O.quant_int8(p, 256)
    back = _bf16_to_float(O.dequant_bf16([codes], [scales], p.size, 256)).astype(np.float64)
    x = _bf16_to_float(p).astype(np.float64)
    step = np.repeat(scales.astype(np.float64), 256)[:p.size]
    assert np.all(np.abs(back - x) <= 0.5 * step + np.abs(x) * 2.0 ** -8 + 1e-30)
    assert not back[256 * 3:256 * 4].any()
    for b in range(0, 20):
        blk = slice(b * 256, (b + 1) * 256)
        i = np.argmax(np.abs(x[blk]))
        if x[blk][i] != 0:
            assert abs(back[blk][i] - x[blk][i]) <= abs(x[blk][i]) * 2.0 ** -8


def test_dequant_is_two_roundings_of_the_exact_product():
    """Scales with 24 significant bits make code * scale inexact in binary32:
    the result is the bf16 of the binary32-rounded product (computed here
    with exact rationals and a by-hand nearest-even), not of the exact one."""
    rng = np.random.default_rng(9)
    n, block = 512, 64
    codes = rng.integers(-127, 128, size=n).astype(np.int8)
    scales = (rng.random(n // block) + 0.5).astype(np.float32)
    got = O.dequant_bf16([codes], [scales], n, block)

    def rne(fr: Fraction, bits: int) -> Fraction:
        if fr == 0:
            return fr
        sign = -1 if fr < 0 else 1
        a = abs(fr)
        e = 0
        while a >= 2:
            a /= 2
            e += 1
        while a < 1:
            a *= 2
            e -= 1
        q = a * 2 ** (bits - 1)
        fl = q.numerator // q.denominator
        rem = q - fl
        if rem > Fraction(1, 2) or (rem == Fraction(1, 2) and fl % 2):
            fl += 1
        return sign * Fraction(fl, 2 ** (bits - 1)) * Fraction(2) ** e

    for i in range(n):
        exact = Fraction(int(codes[i])) * Fraction(float(scales[i // block]))
        want = float(rne(rne(exact, 24), 8))
        assert _bf16_to_float(got[i:i + 1])[0] == want, i


# ------------------------------- global clip across shards (S = S_local + S_other)

def _dyadic_rows(nd: int, n: int, seed: int) -> list[np.ndarray]:
    """bf16 rows of small integers times 2^-12 (|k| <= 255): every average is
    exact in binary32, every square exact in binary64, and every partial sum
    of squares over these lengths stays below 2^53 units of 2^-30, so the sum
    of squares is exact in any order and any grouping."""
    rng = np.random.default_rng(seed)
    return [_bf16_bits(rng.integers(-255, 256, n).astype(np.float64) * 2.0**-12)
            for _ in range(nd)]


def _shard_bounds(n: int, nd: int, block: int) -> list[tuple[int, int]]:
    per = -(-n // nd)
    per = -(-per // block) * block
    return [(r * per, min(n, (r + 1) * per)) for r in range(nd) if r * per < n]


def _clipped_run(rows_of_step, n, h_of_step, nd_shards=None, s_other_scale=1.0, block=256):
    """Three clipped steps of the whole vector (nd_shards None), or of each
    shard separately with s_other = the other shards' summed S (times
    s_other_scale, to show the test's sensitivity); returns the concatenated
    master, m, v, bf16, codes and scales."""
    master0, m0, v0 = (S.host_f32(n, 9, S.MASTER, 0, 0, 0, 0.02), np.zeros(n, np.float32),
                       np.zeros(n, np.float32))
    if nd_shards is None:
        bounds = [(0, n)]
    else:
        bounds = _shard_bounds(n, nd_shards, block)
    state = [(master0[lo:hi].copy(), m0[lo:hi].copy(), v0[lo:hi].copy()) for lo, hi in bounds]
    outs = [None] * len(bounds)
    for s in (1, 2, 3):
        rows = rows_of_step(s)
        # each shard's own S (the norm pass), then the scalar exchange
        local = [O.gbar_sumsq([r[lo:hi] for r in rows])[1] for lo, hi in bounds]
        for j, (lo, hi) in enumerate(bounds):
            other = sum(x for i, x in enumerate(local) if i != j)
            h = h_of_step(s)
            h.s_other = other * s_other_scale
            mst, mo, va = state[j]
            outs[j] = O.step([r[lo:hi] for r in rows], mst, mo, va, h)
    cat = lambda xs: np.concatenate(xs)  # noqa: E731
    return (cat([x[0] for x in state]), cat([x[1] for x in state]), cat([x[2] for x in state]),
            cat([o.p for o in outs]), cat([o.codes for o in outs]), cat([o.scales for o in outs]))


def test_clipped_shard_concatenation_with_s_other_bitwise():
    """Global clipping ("ZeRO (딥 러닝)", "DeepSpeed에서 쓰기": gradient_clipping)
    scales every shard by the norm over ALL shards; elementwise independence
    ("ZeRO-1") then lets the shards update apart.  Each shard adds the other
    shards' sum of squares (s_other) to its own, and the concatenated shards
    must equal the unpartitioned clipped step.  On dyadic contributions every
    S is exact in any association, so the equality is bit for bit.  The clip
    threshold lies above every shard's own norm and below the global norm:
    dropping s_other leaves the shards unclipped, doubling it clips too hard,
    and both are shown to break the equality."""
    n, nd = 4 * 65536 + 3 * 256 + 40, 4
    rows = {s: _dyadic_rows(4, n, 100 + s) for s in (1, 2, 3)}
    g_norms = {s: np.sqrt(O.gbar_sumsq(rows[s])[1]) for s in rows}
    local_max = max(np.sqrt(O.gbar_sumsq([r[lo:hi] for r in rows[s]])[1])
                    for s in rows for lo, hi in _shard_bounds(n, nd, 256))
    max_norm = float(np.float32(0.5 * (local_max + min(g_norms.values()))))
    assert local_max < max_norm < min(g_norms.values())  # clip active only globally

    def hyper(s):
        return O.Hyper(lr=1e-3, beta1=0.9, beta2=0.999, eps=1e-8, weight_decay=0.1, t=s,
                       max_norm=max_norm, quant_block=256)

    whole = _clipped_run(rows.get, n, hyper)
    parts = _clipped_run(rows.get, n, hyper, nd_shards=nd)
    for name, a, b in zip(("master", "m", "v", "bf16", "codes", "scales"), whole, parts):
        assert np.array_equal(a.view(np.uint8), b.view(np.uint8)), name
    for scale in (0.0, 2.0):
        wrong = _clipped_run(rows.get, n, hyper, nd_shards=nd, s_other_scale=scale)
        assert not np.array_equal(wrong[1], whole[1]), scale  # m carries coef * gbar


def test_clipped_shard_concatenation_seeded_within_one_ulp():
    """The same on seeded N(0, 1e-3) contributions of the clipped 13B
    workload: the shards' S is associated differently from the whole
    vector's (the per-shard sums, then the exchange), so coef may differ in
    its last binary64 bits, and every stored value within one ulp."""
    w = S.by_name("13B-nd16-clip-int8")
    n, nd = 3 * 65536 + 5000, 3
    rows = {s: list(S.host_contrib(w, s, 0, n)) for s in (1, 2, 3)}
    norm = min(np.sqrt(O.gbar_sumsq(rows[s])[1]) for s in rows)

    def hyper(s):
        return O.Hyper(lr=w.lr, beta1=w.beta1, beta2=w.beta2, eps=w.eps,
                       weight_decay=w.weight_decay, t=s, max_norm=float(np.float32(norm / 3)),
                       quant_block=256)

    whole = _clipped_run(rows.get, n, hyper)
    parts = _clipped_run(rows.get, n, hyper, nd_shards=nd)
    for name, a, b in zip(("master", "m", "v"), whole[:3], parts[:3]):
        d = np.abs(a.view(np.int32).astype(np.int64) - b.view(np.int32).astype(np.int64))
        assert d.max() <= 1, name
    d = np.abs(whole[3].astype(np.int64) - parts[3].astype(np.int64))
    assert d.max() <= 1


def test_clip_sums_local_and_other_closed_form():
    """All-equal averaged gradient c over n = 4^k elements split into shards:
    S_local + S_other = n c^2 exactly, so every shard's coefficient is
    max_norm / (|c| 2^k + 1e-6), and with m = 0 at t = 1 the stored momentum
    is (1 - beta1) coef c.  A shard that ignored s_other would use its own
    n_r c^2 instead and store a momentum 2x (n_r = n/4) larger."""
    c, k, nd = 0.75, 8, 4
    n = 4**k
    rows = [np.full(n, _bf16_bits([c])[0], np.uint16) for _ in range(2)]
    max_norm = 1.0
    coef = max_norm / (abs(c) * 2**k + 1e-6)
    b1 = float(np.float32(0.9))
    per = n // nd
    for r in range(nd):
        lo, hi = r * per, (r + 1) * per
        master = np.zeros(per, np.float32)
        m = np.zeros(per, np.float32)
        v = np.zeros(per, np.float32)
        h = O.Hyper(lr=1e-3, t=1, max_norm=max_norm, s_other=(n - per) * c * c)
        out = O.step([x[lo:hi] for x in rows], master, m, v, h)
        assert out.sumsq == per * c * c
        want = np.float32((1.0 - b1) * coef * c)
        assert np.all(m == want), (r, m[0], want)


# --------------------------------------------- Adam without bias correction

def test_adam_no_bias_correction_closed_forms():
    """bias_correction = 0: the moments are used as they are.  With a constant
    gradient g from m = v = 0, m_T = (1 - b1^T) g and v_T = (1 - b2^T) g^2, so
    step T moves theta by -lr (1 - b1^T) g / (sqrt(1 - b2^T) |g| + eps): at
    t = 1 that is -lr (1 - b1) g / (sqrt(1 - b2) |g| + eps), about 3.2 lr for
    (0.9, 0.999), against -lr g / (|g| + eps) when the corrections are
    applied.  Checked per step for T = 1..6, and theta as the sum of the
    steps."""
    g = np.array([1e-3, -2e-4, 0.5, -7e-6, 3e-9, 0.0], np.float32)
    theta0 = np.array([0.01, -0.02, 0.3, 1.0, -1e-5, 0.02], np.float32)
    h = O.Hyper(lr=1e-3, beta1=0.9, beta2=0.999, eps=1e-8, bias_correction=0)
    T = 6
    hist, m, v = _adam_run([g] * T, theta0, h)
    lr, b1, b2, eps = (float(np.float32(x)) for x in (1e-3, 0.9, 0.999, 1e-8))
    g64 = g.astype(np.float64)
    want = theta0.astype(np.float64)
    for t, th in enumerate(hist, 1):
        mt = (1.0 - b1**t) * g64
        vt = (1.0 - b2**t) * g64 * g64
        want = want - lr * mt / (np.sqrt(vt) + eps)
        # theta carries one binary32 rounding per step
        assert np.allclose(th, want, rtol=4e-7 * t, atol=1e-12), t
    assert np.allclose(m, (1.0 - b1**T) * g64, rtol=1e-6, atol=0)
    assert np.allclose(v, (1.0 - b2**T) * g64 * g64, rtol=1e-6, atol=0)
    # the first step differs from the bias-corrected one by ~sqrt(1-b2)/(1-b1)
    (c1,), _, _ = _adam_run([g], theta0, O.Hyper(lr=1e-3, beta1=0.9, beta2=0.999, eps=1e-8))
    (u1,), _, _ = _adam_run([g], theta0, h)
    big = np.abs(g64) >= 1e-4  # eps negligible next to sqrt(1 - b2) |g|
    ratio = (u1 - theta0).astype(np.float64)[big] / (c1 - theta0).astype(np.float64)[big]
    assert np.allclose(ratio, (1 - b1) / np.sqrt(1 - b2), rtol=5e-3)


# ------------------------------------------------------ non-finite inputs

def test_nonfinite_propagate_per_ieee_through_reduce_and_adam():
    """Reading 16 (non-finite values propagate, no step is skipped), worked by
    hand: a NaN contribution makes that element's average, m, v and theta
    NaN; +inf gives m = v = +inf and theta = NaN (lr * inf / (inf + eps));
    +inf and -inf in one element give NaN; every other element is the
    finite step."""
    inf, nan = np.float32(np.inf), np.float32(np.nan)
    one = np.float32(1.0)
    r0 = np.array([nan, inf, inf, one, one], np.float32)
    r1 = np.array([one, one, -inf, one, one], np.float32)
    rows = [O.f32_to_bf16(r0), O.f32_to_bf16(r1)]
    g = O.reduce_average(rows)
    assert np.isnan(g[0]) and g[1] == inf and np.isnan(g[2])
    assert g[3] == 1.0 and g[4] == 1.0
    n = g.size
    master = np.full(n, 0.5, np.float32)
    m = np.zeros(n, np.float32)
    v = np.zeros(n, np.float32)
    h = O.Hyper(lr=1e-3, weight_decay=0.0, t=1)
    O.adam(master, m, v, g, 1.0, h)
    assert np.isnan(master[0]) and np.isnan(m[0]) and np.isnan(v[0])
    assert m[1] == inf and v[1] == inf and np.isnan(master[1])
    assert np.isnan(master[2]) and np.isnan(m[2])
    # the finite elements: first step from zero state, -lr g/(|g| + eps),
    # with lr and eps the binary32 values widened
    lr, eps = float(np.float32(1e-3)), float(np.float32(1e-8))
    want = np.float32(0.5 - lr * 1.0 / (1.0 + eps))
    assert np.all(master[3:] == want)


def test_quant_blocks_with_nonfinite_values():
    """Reading 7's rule for non-finite quotients: a block holding a NaN gets
    a NaN scale (the absmax propagates the NaN) and codes 0; a block holding
    +inf (and no NaN) gets scale +inf and codes 0 (finite / inf = 0, inf /
    inf is NaN -> 0); a finite block next to them is quantized as usual."""
    block = 4
    vals = np.array([1.0, np.nan, -2.0, 0.5,      # NaN block
                     np.inf, 3.0, -1.0, 0.25,     # inf block
                     127.0, -63.5, 2.5, 0.0],     # finite: scale 1, ties to even
                    np.float32)
    codes, scales = O.quant_int8(O.f32_to_bf16(vals), block)
    assert np.isnan(scales[0]) and np.all(codes[0:4] == 0)
    assert scales[1] == np.inf and np.all(codes[4:8] == 0)
    assert scales[2] == 1.0
    assert codes[8:12].tolist() == [127, -64, 2, 0]


def test_clip_coef_at_nonfinite_sums():
    """coef = min(1, max_norm / (sqrt(S) + 1e-6)): a NaN S gives NaN (no
    silent skip), S = +inf gives 0, S = 0 gives 1 (max_norm / 1e-6 >= 1)."""
    assert np.isnan(O.clip_coef(float("nan"), 1.0))
    assert O.clip_coef(float("inf"), 1.0) == 0.0
    assert O.clip_coef(0.0, 1.0) == 1.0
    assert O.clip_coef(4.0, 1.0) == 1.0 / (2.0 + 1e-6)
