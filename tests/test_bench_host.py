"""Host-side pieces of bench.py (no GPU): the stream probe's mix for each
launch, the parse of the probe's summary lines, each launch's fraction of its
mix's best, the launches one call of each timed kernel queues, and the
single-GPU refusal."""

import subprocess
import sys

import pytest

import bench
import seeded_inputs as S

SAMPLE = """device gfx950, 256 CUs, LDS 65536 B per workgroup / 163840 B per CU
norm16  Lnt-Snt U1 oneshot-cap3  s1280     6213 GB/s
BEST norm16  R16 W2    6213 GB/s (77.7% of 8 TB/s)  Lnt-Snt U1 oneshot-cap3 s1280
BEST upd     R8 W7    6240 GB/s (78.0% of 8 TB/s)  Lnt-Snt U1 oneshot-cap2 s1280
BEST nd64    R70 W7    6186 GB/s (77.3% of 8 TB/s)  Lnt-Snt U4 oneshot s0
"""


def test_probe_summary_parse():
    best = bench.parse_probe_best(SAMPLE)
    assert set(best) == {"norm16", "upd", "nd64"}
    assert best["norm16"] == {"reads": 16, "writes": 2, "best_GBps": 6213.0,
                              "shape": "Lnt-Snt U1 oneshot-cap3 s1280"}
    assert best["nd64"]["reads"] == 70 and best["nd64"]["writes"] == 7
    assert bench.parse_probe_best("no summary here\n") == {}


@pytest.mark.parametrize("name,spill,want", [
    ("13B-nd16-clip-int8", True, {"gnorm": "norm16", "step": "upd"}),
    ("13B-nd16-clip-int8", False, {"gnorm": None, "step": None}),
    ("7.5B-nd64", True, {"step": "nd64"}),
    ("7.5B-nd64-zeropp", True, {"step": "q8nd64"}),
    ("13B-nd1-stage0", True, {"step": "nd1"}),
    ("tiny-zero1", True, {"step": None}),
])
def test_probe_mix_per_launch(name, spill, want):
    w = S.by_name(name)
    assert {k: bench.probe_mix(w, k, spill) for k in bench.kernel_bytes(w, spill)} == want


@pytest.mark.parametrize("name,spill,want", [
    # the 812.5M-element norm pass: 12 launches of 2^26 and one of 7,193,632
    ("13B-nd16-clip-int8", True, {"gnorm": 13, "step": 1}),
    # clipping without the spill re-reads the 16 rows: below the wide form's
    # 32 rows for a quantizing update over bf16 rows, so one launch
    ("13B-nd16-clip-int8", False, {"gnorm": 13, "step": 1}),
    ("7.5B-nd64", True, {"step": 4}),
    ("7.5B-nd64-zeropp", True, {"step": 4}),
    ("13B-nd1-stage0", True, {"step": 1}),
    ("tiny-zero1", True, {"step": 1}),
])
def test_launches_per_call(name, spill, want):
    w = S.by_name(name)
    assert {k: bench.launches_per_call(w, k, spill) for k in bench.kernel_bytes(w, spill)} == want


def test_probe_mix_traffic_matches_launch_bytes():
    """A mix's reads and writes, in 16-byte vectors per 8 shard elements,
    are the launch's bytes per element (the int8 output, 1/8 of a vector
    plus scales, is left out of the update mixes)."""
    best = bench.parse_probe_best(SAMPLE)
    w = S.by_name("13B-nd16-clip-int8")
    kb = bench.kernel_bytes(w, True)
    n = best["norm16"]
    assert (n["reads"] + n["writes"]) * 16 / 8 == kb["gnorm"]
    u = best["upd"]
    assert (u["reads"] + u["writes"]) * 16 / 8 == pytest.approx(kb["step"], abs=1.1)
    w64 = S.by_name("7.5B-nd64")
    d = best["nd64"]
    assert (d["reads"] + d["writes"]) * 16 / 8 == bench.kernel_bytes(w64, True)["step"]


def test_fraction_of_probe():
    w = S.by_name("13B-nd16-clip-int8")
    r = {"per_kernel": {"gnorm": {"GBps": 5733.0}, "step": {"GBps": 5388.3}}}
    out = bench.against_probe(w, r, True, bench.parse_probe_best(SAMPLE))
    assert out["gnorm"]["mix"] == "norm16"
    assert out["gnorm"]["frac_of_probe"] == round(5733.0 / 6213.0, 4)
    assert out["step"]["frac_of_probe"] == round(5388.3 / 6240.0, 4)
    assert bench.against_probe(w, r, True, None) is None


def test_more_than_one_gpu_is_refused():
    p = subprocess.run([sys.executable, bench.__file__, "--gpus", "2"], capture_output=True,
                       text=True, timeout=120)
    assert p.returncode == 2
    assert "one GPU" in p.stderr


def test_measured_traffic_reads_the_committed_counters():
    """roofline.traffic: the HBM bytes per call of the dominant kernel from
    the committed counter summary, only while its source hash is the
    library's (then within 1% of the algorithmic bytes of a call)."""
    import hashlib
    import os
    import re

    w = S.by_name("13B-nd16-clip-int8")
    path = os.path.join(bench.ROOT, "profiles", "hbm_counters_13B-nd16-clip-int8.md")
    src = os.path.join(bench.ROOT, "sharded_mixed_precision_zero_amd", "csrc", "zero_shard.hip")
    rec = re.search(r"source_sha256 (\w+)", open(path).read()).group(1)
    got = bench.measured_traffic(w, "gnorm_partial_kernel")
    if rec != hashlib.sha256(open(src, "rb").read()).hexdigest():
        assert got is None
        return
    algo = bench.kernel_bytes(w, True)["gnorm"] * w.shard_len
    assert got is not None and abs(got / algo - 1.0) < 0.01


def test_spaced_layout_slots():
    """The benchmark's spaced layout: every state, spill and output array at
    the start of its own 16 GiB slot; arrays larger than a slot (the 13B
    stage-0 buffer) keep one allocation each; the arena and the contribution
    rows fit the 288 GB of one MI355X."""
    from tests._gpu import SLOT_BYTES, row_stride, spaced_slots

    w = S.by_name("13B-nd16-clip-int8")
    n = w.shard_len
    sizes = [4 * n, 4 * n, 4 * n, 2 * n, n, 4 * -(-n // w.quant_block), 4 * n]
    offs, total = spaced_slots(sizes)
    assert offs == [i * SLOT_BYTES for i in range(len(sizes))]
    assert all(b <= SLOT_BYTES for b in sizes)
    assert all(o % SLOT_BYTES == 0 for o in offs)
    rows = 2 * ((w.n_d - 1) * row_stride(n) + n)
    assert total + rows < 288e9
    big = S.by_name("13B-nd1-stage0")
    assert spaced_slots([4 * big.shard_len, 2 * big.shard_len]) is None
    assert spaced_slots([]) == ([], 0)
