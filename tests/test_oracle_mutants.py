"""The oracle's pins against planted mistakes.

Each mutant below is the oracle source (oracle/zs_oracle.cpp) with one
plausible slip: a dropped term, a wrong sign, index or constant, a swapped
operand, another rounding.  It is built into a library of its own and the
pin suite (tests/test_oracle_pins.py) is run against it; the pins must
fail.  A mutant the pins let through would be a part of the oracle that no
pin checks.  Mistakes that provably change no result (the int8 clamp, whose
bound a ratio of at most 127 * (1 + 2^-24) never reaches) are not listed.
The unmutated source, built the same way, must pass.  CPU only (g++).
"""

from __future__ import annotations

import concurrent.futures
import os
import shutil
import subprocess
import sys
import tempfile

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = os.path.join(ROOT, "oracle", "zs_oracle.cpp")
PINS = os.path.join(ROOT, "tests", "test_oracle_pins.py")

# (name, text in the oracle source, its replacement)
MUTANTS = [
    ("stage-1 memory keeps the whole optimizer state",
     "case 1: return 4.0 * psi + k * psi / nd;", "case 1: return 4.0 * psi + k * psi;"),
    ("stage-2 memory partitions only the optimizer state",
     "case 2: return 2.0 * psi + (2.0 + k) * psi / nd;",
     "case 2: return 2.0 * psi + 2.0 * psi + k * psi / nd;"),
    ("stage-3 memory keeps the weights whole",
     "case 3: return (2.0 + 2.0 + k) * psi / nd;", "case 3: return 2.0 * psi + (2.0 + k) * psi / nd;"),
    ("bf16 rounding ties away from zero",
     "if (lo > 0x8000u || (lo == 0x8000u && (hi & 1u))) hi += 1;", "if (lo >= 0x8000u) hi += 1;"),
    ("bf16 rounding truncates",
     "if (lo > 0x8000u || (lo == 0x8000u && (hi & 1u))) hi += 1;", "if (lo > 0xffffu) hi += 1;"),
    ("average drops the last rank",
     "for (int32_t k = 0; k < nd; ++k) s += double(orc_bf16_to_f32(rows[k][i]));\n"
     "    gbar[i] = float(s / double(nd));",
     "for (int32_t k = 0; k + 1 < nd; ++k) s += double(orc_bf16_to_f32(rows[k][i]));\n"
     "    gbar[i] = float(s / double(nd));"),
    ("average divides by n_d + 1",
     "for (int32_t k = 0; k < nd; ++k) s += double(orc_bf16_to_f32(rows[k][i]));\n"
     "    gbar[i] = float(s / double(nd));",
     "for (int32_t k = 0; k < nd; ++k) s += double(orc_bf16_to_f32(rows[k][i]));\n"
     "    gbar[i] = float(s / double(nd + 1));"),
    ("average rounds each addend to binary32",
     "for (int32_t k = 0; k < nd; ++k) s += double(orc_bf16_to_f32(rows[k][i]));\n"
     "    gbar[i] = float(s / double(nd));",
     "for (int32_t k = 0; k < nd; ++k) s = float(s + double(orc_bf16_to_f32(rows[k][i])));\n"
     "    gbar[i] = float(s / double(nd));"),
    ("int8 contributions take rank 0's scales",
     "s += double(codes[k][i]) * double(scales[k][i / block]);\n    gbar[i]",
     "s += double(codes[k][i]) * double(scales[0][i / block]);\n    gbar[i]"),
    ("sum of squares sums the gradient",
     "s += g * g;", "s += g;"),
    ("clip without the square root",
     "max_norm / (std::sqrt(sumsq) + 1e-6)", "max_norm / (sumsq + 1e-6)"),
    ("clip coefficient not capped at 1",
     "return c < 1.0 ? c : 1.0;", "return c;"),
    ("clip drops the other shards' sum",
     "orc_clip_coef(p + h->s_other, h->max_norm)", "orc_clip_coef(p, h->max_norm)"),
    ("clip counts the other shards' sum twice",
     "orc_clip_coef(p + h->s_other, h->max_norm)", "orc_clip_coef(p + 2.0 * h->s_other, h->max_norm)"),
    ("clip coefficient applied twice",
     "const double g = coef * double(gbar[i]);", "const double g = coef * coef * double(gbar[i]);"),
    ("momentum without bias correction",
     "const double mhat = m1 / bc1;", "const double mhat = m1;"),
    ("variance without bias correction",
     "const double vhat = v1 / bc2;", "const double vhat = v1;"),
    ("bias correction applied when it is off",
     "if (h->bias_correction) {", "if (h->t > 0) {"),
    ("eps inside the square root",
     "(std::sqrt(vhat) + h->eps)", "std::sqrt(vhat + h->eps)"),
    ("weight decay with the wrong sign",
     "th - h->lr * h->weight_decay * th", "th + h->lr * h->weight_decay * th"),
    ("weight decay without the learning rate",
     "th - h->lr * h->weight_decay * th", "th - h->weight_decay * th"),
    ("variance decays with beta1",
     "const double v1 = b2 * double(v[i]) + (1.0 - b2) * (g * g);",
     "const double v1 = b1 * double(v[i]) + (1.0 - b1) * (g * g);"),
    ("variance of the gradient, not its square",
     "(1.0 - b2) * (g * g);", "(1.0 - b2) * g;"),
    ("momentum update with beta2",
     "const double m1 = b1 * double(m[i]) + (1.0 - b1) * g;",
     "const double m1 = b2 * double(m[i]) + (1.0 - b2) * g;"),
    ("quantizer scale over 128",
     "float(double(a) / 127.0)", "float(double(a) / 128.0)"),
    ("quantizer rounds ties away from zero",
     "std::nearbyint(double(ratio))", "std::round(double(ratio))"),
    ("quantizer drops the partial last block",
     "const int64_t nb = (n + block - 1) / block;", "const int64_t nb = n / block;"),
    ("dequant shards placed one element short",
     "const int64_t base = int64_t(r) * per;", "const int64_t base = int64_t(r) * (per - 1);"),
    ("dequant truncates to bf16",
     "out[base + j] = orc_f32_to_bf16(x);", "out[base + j] = uint16_t(f32_to_bits(x) >> 16);"),
]


def _build(src_text: str, d: str) -> str:
    src = os.path.join(d, "zs_oracle.cpp")
    with open(src, "w") as f:
        f.write(src_text)
    shutil.copy(os.path.join(ROOT, "oracle", "zs_oracle.h"), d)
    so = os.path.join(d, "libzsoracle.so")
    subprocess.run(["g++", "-O2", "-std=c++17", "-fPIC", "-shared", "-ffp-contract=off",
                    "-fno-fast-math", "-pthread", src, "-o", so],
                   check=True, capture_output=True, text=True, timeout=300)
    return so


def _pins(so: str) -> subprocess.CompletedProcess:
    env = dict(os.environ)
    env["ZS_ORACLE_LIB"] = so
    env["OMP_NUM_THREADS"] = "2"
    return subprocess.run([sys.executable, "-m", "pytest", PINS, "-x", "-q",
                           "-p", "no:cacheprovider", "-m", "not gpu"],
                          cwd=ROOT, env=env, capture_output=True, text=True, timeout=900)


def _run_mutant(m) -> tuple[str, int, str]:
    name, old, new = m
    text = open(SRC).read()
    assert text.count(old) == 1, f"{name}: the text to mutate is not unique in the oracle"
    with tempfile.TemporaryDirectory() as d:
        so = _build(text.replace(old, new), d)
        r = _pins(so)
    return name, r.returncode, r.stdout[-400:]


@pytest.mark.skipif(shutil.which("g++") is None, reason="no g++")
def test_pins_pass_on_the_unmutated_source():
    with tempfile.TemporaryDirectory() as d:
        r = _pins(_build(open(SRC).read(), d))
    assert r.returncode == 0, r.stdout[-2000:] + r.stderr[-2000:]


@pytest.mark.skipif(shutil.which("g++") is None, reason="no g++")
def test_pins_catch_every_planted_mistake():
    with concurrent.futures.ThreadPoolExecutor(max_workers=4) as ex:
        results = list(ex.map(_run_mutant, MUTANTS))
    survivors = [(name, out) for name, rc, out in results if rc == 0]
    assert not survivors, "mutants no pin catches: " + "; ".join(n for n, _ in survivors)
