"""The host-only library code (zero_shard_host.cpp) and the oracle built
with AddressSanitizer + UndefinedBehaviorSanitizer, and with
ThreadSanitizer, running tests/native/host_sanitize.cpp: ragged shards,
every quantizer block, clipping, 1..5 threads; host update and oracle must
agree bit for bit and the sanitizers must stay silent.  CPU only (g++)."""

from __future__ import annotations

import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = [os.path.join(ROOT, "tests", "native", "host_sanitize.cpp"),
       os.path.join(ROOT, "sharded_mixed_precision_zero_amd", "csrc", "zero_shard_host.cpp"),
       os.path.join(ROOT, "oracle", "zs_oracle.cpp")]


@pytest.mark.skipif(shutil.which("g++") is None, reason="no g++")
@pytest.mark.parametrize("sanitize,isa", [
    ("address,undefined", None),
    ("address,undefined", "avx2"),
    ("thread", None),
])
def test_host_code_under_sanitizers(tmp_path, sanitize, isa):
    exe = str(tmp_path / "host_sanitize")
    cmd = ["g++", "-std=c++17", "-O1", "-g", f"-fsanitize={sanitize}",
           "-fno-sanitize-recover=all", "-fno-omit-frame-pointer", "-ffp-contract=off",
           "-fno-fast-math", "-march=x86-64-v3", "-pthread",
           "-I" + os.path.join(ROOT, "include"), "-I" + os.path.join(ROOT, "oracle"),
           "-I" + os.path.join(ROOT, "sharded_mixed_precision_zero_amd", "csrc"),
           *SRC, "-o", exe]
    subprocess.run(cmd, check=True, capture_output=True, text=True, timeout=300)
    env = dict(os.environ)
    env.pop("LD_PRELOAD", None)
    env["ASAN_OPTIONS"] = "detect_leaks=1:abort_on_error=0"
    env["UBSAN_OPTIONS"] = "print_stacktrace=1:halt_on_error=1"
    env["TSAN_OPTIONS"] = "halt_on_error=1"
    if isa == "avx2":
        env["ZS_HOST_NO_AVX512"] = "1"
    r = subprocess.run([exe], env=env, capture_output=True, text=True, timeout=600)
    assert r.returncode == 0, r.stdout[-2000:] + r.stderr[-4000:]
    assert "MISMATCH" not in r.stdout
    assert "runtime error" not in r.stderr
