"""The allocation-free norm pass (zero_shard_gnorm_noalloc, for callers that
cannot allocate) against zero_shard_gnorm on a handle: the same S_local and
the same averaged-gradient spill, bit for bit, on two calls in a row, the
second on a smaller shard (the static scratch keeps the first call's
partials; the second must not see them); a shard beyond the scratch is
refused with ZS_ETOOBIG and nothing is written.  Through the C ABI."""

from __future__ import annotations

import pytest

import seeded_inputs as S
import sharded_mixed_precision_zero_amd as Z
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


def _noalloc(g: GpuShard):
    import torch

    s_out = torch.full((1,), -1.0, dtype=torch.float64, device="cuda")
    spill = torch.full((max(1, g.n),), float("nan"), dtype=torch.float32, device="cuda")
    desc = Z.zs_desc.from_buffer_copy(g.shard.desc)
    desc.gbar_ws = spill.data_ptr()
    desc.stream = torch.cuda.current_stream().cuda_stream
    rc = Z.zero_shard_gnorm_noalloc(desc, g.tab, s_out)
    return rc, s_out, spill


def test_noalloc_norm_equals_handle_norm_on_two_calls():
    import torch

    w = S.by_name("13B-nd16-clip-int8")
    for n in (3_000_017, 70_001):  # the second call on a smaller shard
        log(f"case noalloc gnorm n={n} n_d={w.n_d}")
        g = GpuShard(w, n=n)
        g.fill_grads(1)
        g.norm()  # the handle's pass: S in g.sumsq, spill in g.gbar_ws
        rc, s_out, spill = _noalloc(g)
        assert rc == Z.ZS_OK, Z.zero_shard_strerror(rc)
        torch.cuda.synchronize()
        assert torch.equal(s_out.view(torch.int64), g.sumsq.view(torch.int64)), (
            float(s_out.item()), float(g.sumsq.item()))
        assert torch.equal(spill.view(torch.int32), g.gbar_ws.view(torch.int32))
        g.free()


def test_noalloc_norm_refuses_a_shard_beyond_its_scratch():
    import torch

    n = (1 << 30) + 8  # 65,538 partials > 65,536
    rows = torch.zeros(16 * 64, dtype=torch.int16, device="cuda")
    tab = [rows[64 * k:64 * (k + 1)] for k in range(16)]
    s_out = torch.full((1,), 7.0, dtype=torch.float64, device="cuda")
    desc = Z.zs_desc(phi=n, n_d=16, r=0, shard_len=n, beta1=0.9, beta2=0.999, eps=1e-8,
                     weight_decay=0.0, bias_correction=1, max_norm=1.0, quant_block=0,
                     master=None, m=None, v=None, param_out=None, q_codes=None, q_scales=None,
                     gbar_ws=None, stream=torch.cuda.current_stream().cuda_stream)
    assert Z.zero_shard_gnorm_noalloc(desc, tab, s_out) == Z.ZS_ETOOBIG
    desc.shard_len = desc.phi = 0  # an empty shard fits: S = 0
    assert Z.zero_shard_gnorm_noalloc(desc, tab, s_out) == Z.ZS_OK
    torch.cuda.synchronize()
    assert float(s_out.item()) == 0.0
