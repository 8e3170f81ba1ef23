"""The C ABI on the CPU: the library loads, exports every declared symbol,
matches the header's struct layout, and rejects bad arguments before it
touches a device.  No kernel is launched here."""

from __future__ import annotations

import ctypes
import os
import re
import subprocess
import sys
import tempfile

import pytest

import seeded_inputs as S
import sharded_mixed_precision_zero_amd as Z

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "zero_shard.h")


def _declared_functions() -> list[str]:
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(zero_shard_\w+)\s*\(", text)))


def test_every_declared_symbol_is_exported():
    names = _declared_functions()
    assert set(names) == set(Z.EXPORTS)
    lib = ctypes.CDLL(Z.LIB_PATH)
    for nm in names:
        assert hasattr(lib, nm), nm
    # and the shared object's dynamic symbol table lists them
    out = subprocess.run(["nm", "-D", "--defined-only", Z.LIB_PATH], capture_output=True,
                         text=True, check=True).stdout
    for nm in names:
        assert re.search(rf"\bT {nm}$", out, flags=re.M), nm


def test_descriptor_layout_matches_header():
    fields = [f for f, _ in Z.zs_desc._fields_]
    prog = ["#include <stddef.h>", "#include <stdio.h>", '#include "zero_shard.h"',
            "int main(void) {", 'printf("size %zu\\n", sizeof(zs_desc));']
    prog += [f'printf("{f} %zu\\n", offsetof(zs_desc, {f}));' for f in fields]
    prog += ["return 0; }"]
    with tempfile.TemporaryDirectory() as d:
        src, exe = os.path.join(d, "l.c"), os.path.join(d, "l")
        open(src, "w").write("\n".join(prog))
        subprocess.run(["gcc", "-std=c99", "-I", os.path.dirname(HEADER), src, "-o", exe],
                       check=True)
        out = subprocess.run([exe], capture_output=True, text=True, check=True).stdout
    got = dict(line.split() for line in out.strip().splitlines())
    assert int(got.pop("size")) == ctypes.sizeof(Z.zs_desc)
    for f in fields:
        assert int(got[f]) == getattr(Z.zs_desc, f).offset, f


def test_constants_match_header():
    prog = ["#include <stdio.h>", '#include "zero_shard.h"', "int main(void) {",
            'printf("%d %lld %lld %d %d %d\\n", ZS_MAX_ND, (long long)ZS_NORM_LAUNCH_LEN,',
            "       (long long)ZS_WIDE_LAUNCH_LEN, ZS_WIDE_MIN_ROWS, ZS_WIDE_MIN_ROWS_QUANT,",
            "       ZS_WIDE_MIN_ROWS_Q8);", "return 0; }"]
    with tempfile.TemporaryDirectory() as d:
        src, exe = os.path.join(d, "c.c"), os.path.join(d, "c")
        open(src, "w").write("\n".join(prog))
        subprocess.run(["gcc", "-std=c99", "-I", os.path.dirname(HEADER), src, "-o", exe],
                       check=True)
        out = subprocess.run([exe], capture_output=True, text=True, check=True).stdout.split()
    assert [int(x) for x in out] == [Z.ZS_MAX_ND, Z.ZS_NORM_LAUNCH_LEN, Z.ZS_WIDE_LAUNCH_LEN,
                                     Z.ZS_WIDE_MIN_ROWS, Z.ZS_WIDE_MIN_ROWS_QUANT,
                                     Z.ZS_WIDE_MIN_ROWS_Q8]


def test_partition_geometry():
    for w in S.WORKLOADS:
        assert Z.zero_shard_len(w.phi, w.n_d, w.r) == w.shard_len
    # uneven: ceil(phi/n_d) per shard, the last one shorter, empty past phi
    assert [Z.zero_shard_len(10, 4, r) for r in range(4)] == [3, 3, 3, 1]
    assert [Z.zero_shard_len(3, 4, r) for r in range(4)] == [1, 1, 1, 0]
    assert sum(Z.zero_shard_len(1_000_003, 7, r) for r in range(7)) == 1_000_003
    assert Z.zero_shard_len(0, 1, 0) == 0
    for bad in [(-1, 4, 0), (10, 0, 0), (10, 4, 4), (10, 4, -1)]:
        assert Z.zero_shard_len(*bad) == -1


def test_strerror():
    for c in (0, -1, -2, -3, -4, -5, -6, -7):
        assert Z.zero_shard_strerror(c)
    assert "unknown" in Z.zero_shard_strerror(-99)


def _desc(**kw) -> Z.zs_desc:
    base = dict(phi=4096, n_d=4, r=1, shard_len=1024, beta1=0.9, beta2=0.999, eps=1e-8,
                weight_decay=0.0, bias_correction=1, max_norm=0.0, quant_block=0,
                master=0x10000, m=0x20000, v=0x30000, param_out=0x40000, q_codes=None,
                q_scales=None, gbar_ws=None, stream=None)
    base.update(kw)
    return Z.zs_desc(**base)


@pytest.mark.parametrize("kw,code", [
    (dict(n_d=0), Z.ZS_EINVAL),
    (dict(n_d=65, r=0, shard_len=64), Z.ZS_EINVAL),
    (dict(r=4), Z.ZS_EINVAL),
    (dict(r=-1), Z.ZS_EINVAL),
    (dict(shard_len=1000), Z.ZS_EINVAL),
    (dict(phi=-5), Z.ZS_EINVAL),
    (dict(beta1=1.0), Z.ZS_EINVAL),
    (dict(beta2=-0.1), Z.ZS_EINVAL),
    (dict(eps=0.0), Z.ZS_EINVAL),
    (dict(eps=float("inf")), Z.ZS_EINVAL),
    (dict(weight_decay=-1.0), Z.ZS_EINVAL),
    (dict(bias_correction=2), Z.ZS_EINVAL),
    (dict(max_norm=float("nan")), Z.ZS_EINVAL),
    (dict(quant_block=100), Z.ZS_EINVAL),
    (dict(quant_block=256), Z.ZS_EINVAL),            # codes/scales missing
    (dict(master=None), Z.ZS_EINVAL),
    (dict(param_out=None), Z.ZS_EINVAL),
    (dict(master=0x10004), Z.ZS_EALIGN),
    (dict(v=0x30008), Z.ZS_EALIGN),
    (dict(param_out=0x40002), Z.ZS_EALIGN),
    (dict(quant_block=256, q_codes=0x50004, q_scales=0x60000), Z.ZS_EALIGN),
    (dict(gbar_ws=0x70004), Z.ZS_EALIGN),
])
def test_init_rejects_bad_descriptors(kw, code):
    rc, h = Z.zero_shard_init(_desc(**kw))
    assert rc == code and not h.value


def test_calls_on_dead_handles_are_refused():
    assert Z.zero_shard_step(None, None, 1e-3, 1) == Z.ZS_ESTATE
    assert Z.zero_shard_gnorm(None, None, None) == Z.ZS_ESTATE
    assert Z.zero_shard_quant(None, 256) == Z.ZS_ESTATE
    assert Z.zero_shard_free(None) == Z.ZS_OK
    fake = ctypes.c_void_p(0x1234560)
    assert Z.zero_shard_step(fake, None, 1e-3, 1) == Z.ZS_ESTATE
    assert Z.zero_shard_free(fake) == Z.ZS_ESTATE


def test_valid_descriptor_needs_the_gpu():
    """With no GPU present a valid descriptor gets as far as the device check."""
    import torch

    if torch.cuda.is_available():
        pytest.skip("a GPU is present; covered by the GPU tests")
    rc, h = Z.zero_shard_init(_desc())
    assert rc == Z.ZS_EDEVICE and not h.value
    rc, h = Z.zero_shard_init(_desc(phi=3, n_d=4, r=3, shard_len=0, master=None, m=None,
                                    v=None, param_out=None))
    assert rc == Z.ZS_EDEVICE


def test_one_hip_runtime_in_process():
    """The library binds to the HIP runtime of the PyTorch that owns the
    memory: importing the binding must not map a second libamdhip64."""
    code = ("import sys; sys.path.insert(0, %r)\n"
            "import sharded_mixed_precision_zero_amd, seeded_inputs\n"
            "seeded_inputs.dev_lib()\n"
            "import torch\n"
            "maps = {l.split()[-1] for l in open('/proc/self/maps') if 'libamdhip64' in l}\n"
            "print(len(maps)); print(maps)\n") % ROOT
    out = subprocess.run([sys.executable, "-c", code], capture_output=True, text=True,
                         check=True).stdout
    assert out.splitlines()[0] == "1", out


@pytest.mark.parametrize("args,code", [
    (dict(n_d=0), Z.ZS_EINVAL),
    (dict(n_d=65), Z.ZS_EINVAL),
    (dict(phi=-1), Z.ZS_EINVAL),
    (dict(block=100), Z.ZS_EINVAL),
    (dict(out=None), Z.ZS_EINVAL),
    (dict(out=0x40002), Z.ZS_EALIGN),
    (dict(codes=[0x1000, 0x2004, 0x3000, 0x4000]), Z.ZS_EALIGN),
    (dict(scales=[0x1000, None, 0x3000, 0x4000]), Z.ZS_EINVAL),
])
def test_dequant_rejects_bad_arguments(args, code):
    a = dict(codes=[0x1000, 0x2000, 0x3000, 0x4000], scales=[0x5000, 0x6000, 0x7000, 0x8000],
             n_d=4, phi=1000, block=256, out=0x40000)
    a.update(args)
    ct = (ctypes.c_void_p * 4)(*a["codes"])
    st = (ctypes.c_void_p * 4)(*a["scales"])
    rc = Z._lib.zero_shard_dequant(ct, st, a["n_d"], a["phi"], a["block"], a["out"], None)
    assert rc == code


def test_offload_init_rejects_bad_hyperparameters_before_allocating():
    """zero_shard_offload_init checks everything the host update will check
    (partition geometry, beta in [0, 1), eps > 0, weight decay >= 0, all
    finite) before it allocates or touches a device, so a bad descriptor is
    ZS_EINVAL from this call and not an error of a later step.  (Device
    pointers here are never dereferenced.)"""
    import numpy as np

    n = 1000
    master, m, v = (np.zeros(n, np.float32) for _ in range(3))
    fake_dev = ctypes.c_void_p(1 << 20)  # 16-byte aligned, never used

    def init(**kw):
        hyper = dict(beta1=0.9, beta2=0.999, eps=1e-8, weight_decay=0.0)
        geo = dict(phi=n, n_d=1, r=0, shard_len=n)
        for k in list(kw):
            if k in hyper:
                hyper[k] = kw.pop(k)
            elif k in geo:
                geo[k] = kw.pop(k)
        d = Z.host_desc(master=master, m=m, v=v, param_out=None, **geo, **hyper)
        o = ctypes.c_void_p()
        return Z._lib.zero_shard_offload_init(ctypes.byref(d), fake_dev, fake_dev, None, 2,
                                              ctypes.byref(o)), o

    for bad in (dict(beta1=1.0), dict(beta1=-0.5), dict(beta2=1.0), dict(eps=0.0),
                dict(eps=-1e-8), dict(eps=float("inf")), dict(weight_decay=-0.1),
                dict(weight_decay=float("nan")), dict(shard_len=n - 1),
                dict(phi=n, n_d=2, r=2), dict(phi=n, n_d=2, r=1, shard_len=n)):
        rc, o = init(**bad)
        assert rc == Z.ZS_EINVAL and not o.value, bad


def test_noalloc_norm_rejects_bad_arguments_before_the_device():
    """zero_shard_gnorm_noalloc validates its descriptor, pointers and size
    before it touches a device (pointers here are never dereferenced)."""
    rows = (ctypes.c_void_p * 4)(*[0x100000 + 0x1000 * k for k in range(4)])
    s = ctypes.c_void_p(0x200000)
    lib = Z._lib

    def call(desc, contrib=rows, sumsq=s):
        return lib.zero_shard_gnorm_noalloc(ctypes.byref(desc) if desc is not None else None,
                                            contrib, sumsq)

    assert call(None) == Z.ZS_EINVAL
    assert call(_desc(), sumsq=None) == Z.ZS_EINVAL
    assert call(_desc(r=4)) == Z.ZS_EINVAL
    assert call(_desc(shard_len=1000)) == Z.ZS_EINVAL
    assert call(_desc(), sumsq=ctypes.c_void_p(0x200004)) == Z.ZS_EALIGN
    assert call(_desc(gbar_ws=0x70004)) == Z.ZS_EALIGN
    assert call(_desc(), contrib=None) == Z.ZS_EINVAL
    bad = (ctypes.c_void_p * 4)(0x100000, 0x100008, 0x102000, 0x103000)
    assert call(_desc(), contrib=bad) == Z.ZS_EALIGN
    big = (1 << 30) + 8
    assert call(_desc(phi=big, n_d=4, r=0, shard_len=big)) == Z.ZS_ETOOBIG


def test_step_constants():
    """zero_shard_step_consts: lr, lr * wd, 1 - beta1^t, 1 - beta2^t in
    binary64 from the binary32 hyper-parameters (1, 1 without bias
    correction); bad arguments are refused."""
    import math

    import numpy as np

    f = lambda x: float(np.float32(x))  # noqa: E731
    for t in (1, 2, 7, 1000, 1050):
        d = _desc(beta1=0.9, beta2=0.95, weight_decay=0.1)
        rc, out = Z.zero_shard_step_consts(d, 1e-4, t)
        assert rc == Z.ZS_OK
        assert out == [f(1e-4), f(1e-4) * f(0.1), 1.0 - math.pow(f(0.9), t),
                       1.0 - math.pow(f(0.95), t)]
    rc, out = Z.zero_shard_step_consts(_desc(bias_correction=0), 1e-3, 5)
    assert rc == Z.ZS_OK and out[2:] == [1.0, 1.0]
    for bad in ((_desc(), -1.0, 1), (_desc(), float("inf"), 1), (_desc(), 1e-3, 0),
                (_desc(beta1=1.0), 1e-3, 1)):
        assert Z.zero_shard_step_consts(*bad)[0] == Z.ZS_EINVAL
