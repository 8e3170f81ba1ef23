"""One small shard step on cuda:0 through the C ABI, checked against the
oracle: 16 contributions, global-norm clipping, AdamW with decoupled weight
decay, bf16 output and the fused int8 block quantizer (every row of the
path), over a ragged 100,003-element shard, two steps."""

from __future__ import annotations

import dataclasses

import numpy as np

import oracle as O
import seeded_inputs as S
from tests import _parity as P
from tests._gpu import GpuShard, OracleWindow, log


def run_smoke() -> None:
    import torch

    assert torch.cuda.is_available(), "smoke() needs the GPU"
    w = dataclasses.replace(S.by_name("13B-nd16-clip-int8"), max_norm=0.05)
    n = 100_003
    g = GpuShard(w, n=n)
    g.init_state()
    ow = OracleWindow(w, 0, n)
    for s in (1, 2):
        g.fill_grads(s)
        g.step(s)
        torch.cuda.synchronize()
        _, ssq = O.gbar_sumsq(list(S.host_contrib(w, s, 0, n)))
        assert abs(g.sumsq.item() - ssq) <= P.sumsq_tolerance(n, ssq), (g.sumsq.item(), ssq)
        o = ow.step(s, sumsq_total=ssq)
        got = g.host()
        st = {k: P.f32_close(k, got[k], getattr(ow, k)) for k in ("master", "m", "v")}
        st["p"] = P.bf16_close("bf16", got["p"], o.p)
        P.int8_exact("int8", got["codes"], got["scales"], o.codes, o.scales, got["p"], o.p,
                     w.quant_block)
        log(f"smoke step {s}: coef={O.clip_coef(ssq, w.max_norm):.4f} {st}")
    g.free()
    log("smoke ok")
