"""The whole final shard after all 50 steps of the 7.5B workloads (bf16 and
int8 contributions), against the oracle chunk by chunk.  About 2.5 minutes
each on one MI355X machine with 16 host cores, so it runs only when asked for
(ZS_LONG_PARITY=1); the default GPU suite compares their whole shard after
two steps and 16 windows at every step, and the 13B clipped workload's
whole shard after all its 10 steps."""

from __future__ import annotations

import os

import pytest

import seeded_inputs as S
from tests.test_gpu_fullstate import run_and_compare

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(os.environ.get("ZS_LONG_PARITY") != "1",
                                 reason="long parity run; set ZS_LONG_PARITY=1")]


@pytest.fixture(autouse=True)
def _gpu_cleanup():
    import torch

    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    yield
    torch.cuda.synchronize()
    torch.cuda.empty_cache()


@pytest.mark.parametrize("name", ["7.5B-nd64", "7.5B-nd64-zeropp"])
def test_full_final_state_after_every_step(name):
    run_and_compare(name, S.by_name(name).steps)
