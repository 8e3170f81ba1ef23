"""The five shard-step workloads: sizes, value distributions, hyper-parameters.

Each is one rank's share of a ZeRO-1/2 optimizer step.  The model sizes come
from the pages' own examples: the 7.5B-parameter model on 64 GPUs of the
stage table in "ZeRO (딥 러닝)" ("ZeRO-DP의 세 단계"), the 13B parameters
trainable without model parallelism of the same page's ZeRO-R paragraph, and
GPT-2 of its memory section.  Every input is seeded and synthetic (the
generator in ``zs_gen.h``); no dataset or checkpoint is involved.
"""

from __future__ import annotations

from dataclasses import dataclass, field

SEED_BASE = 0x5A45524F00000000  # "ZERO" << 32


def _seg13b() -> list[tuple[str, int]]:
    """Flat buffer of a 13B-class decoder: an embedding 32000 x 5120, then 40
    layers of {Wq, Wk, Wv, Wo} 5120 x 5120 and {W_gate, W_up, W_down}
    5120 x 13824.  Each segment is padded to a multiple of 128 elements (all
    already are, so no padding is added)."""
    segs = [("embed", 32000 * 5120)]
    for layer in range(40):
        for nm in ("wq", "wk", "wv", "wo"):
            segs.append((f"l{layer}.{nm}", 5120 * 5120))
        for nm in ("w_gate", "w_up", "w_down"):
            segs.append((f"l{layer}.{nm}", 5120 * 13824))
    return [(nm, (sz + 127) // 128 * 128) for nm, sz in segs]


@dataclass(frozen=True)
class Workload:
    index: int
    name: str
    phi: int                 # parameters in the whole flat buffer
    n_d: int                 # data-parallel degree = contributions averaged
    r: int                   # this rank's partition index
    steps: int
    grad_sigma: float
    master_sigma: float = 0.02
    outliers: bool = False   # 1% of gradient elements x100
    warm: bool = False       # m ~ N(0, m_sigma), v = |N(0, v_sigma)|
    m_sigma: float = 0.0
    v_sigma: float = 0.0
    lr: float = 1e-3
    beta1: float = 0.9
    beta2: float = 0.999
    eps: float = 1e-8
    weight_decay: float = 0.0
    max_norm: float = 0.0    # > 0: global-norm clipping
    quant_block: int = 0     # > 0: int8 block quantization of the bf16 shard
    contrib_block: int = 0   # > 0: contributions arrive as int8 codes with one
                             # fp32 scale per contrib_block elements (qgZ)
    t0: int = 0              # step counter before the first step
    segments: tuple = field(default=(), compare=False)

    @property
    def seed(self) -> int:
        return SEED_BASE + self.index

    @property
    def scale_sigma(self) -> float:
        """sigma of the |N(0, sigma)| per-block scales of int8 contributions:
        codes have standard deviation 32, so code * scale has about the
        gradient's sigma."""
        return self.grad_sigma / 32.0

    @property
    def shard_len(self) -> int:
        """Elements in partition r: ceil(phi / n_d), the last one shorter."""
        per = -(-self.phi // self.n_d)
        return max(0, min(per, self.phi - self.r * per))

    def t_of(self, s: int) -> int:
        """Adam step counter at the s-th (1-based) step of the run."""
        return self.t0 + s

    def bytes_per_param(self, spill: bool = True) -> float:
        """Algorithmic HBM bytes per parameter of one whole step: N_d bf16
        contributions (or int8 codes plus a scale per block), fp32 master/m/v read and written, the bf16 output;
        with clipping the averaged gradient is spilled once as fp32 (written
        by the norm pass, read by the update), or the contributions are read
        twice; int8 codes plus one fp32 scale per block."""
        row = (1.0 + 4.0 / self.contrib_block) if self.contrib_block else 2.0
        b = row * self.n_d + 24.0 + 2.0
        if self.max_norm > 0:
            b += 8.0 if spill else row * self.n_d
        if self.quant_block:
            b += 1.0 + 4.0 / self.quant_block
        return b


# 0-4: the five shard-step workloads; 5: the 7.5B one with ZeRO++'s
# quantized gradients in (qgZ) and quantized weights out (qwZ).
WORKLOADS = [
    Workload(0, "tiny-zero1", phi=1_048_576, n_d=4, r=0, steps=10, grad_sigma=1e-3),
    Workload(1, "gpt2-small-flat", phi=124_439_808, n_d=8, r=0, steps=100,
             grad_sigma=1e-3, outliers=True),
    Workload(2, "7.5B-nd64", phi=7_500_000_000, n_d=64, r=0, steps=50, grad_sigma=5e-4,
             warm=True, m_sigma=1e-4, v_sigma=1e-6, lr=1e-4, beta2=0.95, t0=1000),
    Workload(3, "13B-nd16-clip-int8", phi=13_000_000_000, n_d=16, r=0, steps=10,
             grad_sigma=1e-3, lr=1e-4, weight_decay=0.1, max_norm=1.0, quant_block=256),
    Workload(4, "13B-nd1-stage0", phi=sum(s for _, s in _seg13b()), n_d=1, r=0, steps=20,
             grad_sigma=1e-3, segments=tuple(_seg13b())),
    Workload(5, "7.5B-nd64-zeropp", phi=7_500_000_000, n_d=64, r=0, steps=50,
             grad_sigma=5e-4, warm=True, m_sigma=1e-4, v_sigma=1e-6, lr=1e-4, beta2=0.95,
             t0=1000, quant_block=256, contrib_block=256),
]


def by_name(name_or_index) -> Workload:
    for w in WORKLOADS:
        if str(name_or_index) in (w.name, str(w.index)):
            return w
    raise KeyError(name_or_index)
