"""GPU-side and oracle-side drivers of a workload, shared by the GPU tests,
the smoke check and the benchmark's CPU baseline.

``GpuShard`` owns the device tensors of one shard (state, outputs, the
N_d contribution rows) and calls the library through its C ABI;
``OffloadShard`` drives the library's ZeRO-Offload pipeline.  The oracle
is imported only by the oracle-side helpers, so the benchmark can drive
``GpuShard`` without loading it.  ``OracleWindow`` evolves any window
[i0, i0+n) of the same shard on the CPU with the oracle; unclipped steps
are elementwise, so a window needs only its own inputs, and with clipping
the caller supplies the global sum of squares computed by
``oracle_global_sumsq``.  Inputs on both sides come from the seeded
generator (device and host builds of one definition).
"""

from __future__ import annotations

import sys

import numpy as np

import seeded_inputs as S
import sharded_mixed_precision_zero_amd as Z

DEV = "cuda:0"


def log(*a) -> None:
    print(*a, flush=True)
    sys.stdout.flush()


def row_stride(n: int) -> int:
    """Elements between contribution rows: 16-byte aligned, and offset by a
    non-power-of-two amount so rows do not start on the same HBM channel."""
    return (n + 127) // 128 * 128 + 640


SLOT_BYTES = 16 << 30  # the spaced layout's slot: arrays start at least this far apart


def spaced_slots(nbytes: list[int], slot: int = SLOT_BYTES) -> tuple[list[int], int] | None:
    """Offsets of arrays of the given byte sizes in one arena, each at the
    start of its own slot of `slot` bytes, and the arena's size; None when an
    array does not fit a slot (such arrays are allocated on their own, which
    places them at least their own size apart)."""
    if any(b > slot for b in nbytes):
        return None
    return [i * slot for i in range(len(nbytes))], len(nbytes) * slot


class GpuShard:
    """One shard's device buffers and its library handle.

    layout "separate" (default): one allocation per array.  layout
    "spaced": the state, spill and output arrays in one arena, each at the
    start of its own slot of slot_bytes (16 GiB; arrays larger than a slot
    keep one allocation each).  The kernels and results are the same either way; the
    layouts differ only in where the caller's arrays sit in HBM, which moves
    the update's streaming rate (the benchmark's --layout)."""

    def __init__(self, w: S.Workload, n: int | None = None, i0: int = 0, *, spill: bool = True,
                 quant_block: int | None = None, n_d: int | None = None, phi: int | None = None,
                 r: int | None = None, bias_correction: bool = True, stream=None,
                 layout: str = "separate", slot_bytes: int = SLOT_BYTES):
        import torch

        self.torch = torch
        self.w = w
        self.n = w.shard_len if n is None else int(n)
        self.i0 = i0
        self.nd = w.n_d if n_d is None else n_d
        self.qb = w.quant_block if quant_block is None else quant_block
        self.clip = w.max_norm > 0
        n_ = self.n
        f32 = dict(dtype=torch.float32, device=DEV)
        specs = [("master", n_, torch.float32), ("m", n_, torch.float32),
                 ("v", n_, torch.float32), ("p", n_, torch.int16)]
        if self.qb:
            specs += [("codes", n_, torch.int8),
                      ("scales", (n_ + self.qb - 1) // self.qb, torch.float32)]
        if self.clip and spill:
            specs.append(("gbar_ws", n_, torch.float32))
        if layout not in ("separate", "spaced"):
            raise ValueError(f"layout {layout!r}")
        self.layout = layout
        self.arena = None
        sizes = [k * torch.empty(0, dtype=dt).element_size() for _, k, dt in specs]
        plan = spaced_slots(sizes, slot_bytes) if layout == "spaced" else None
        if plan is not None:
            offs, total = plan
            self.arena = torch.empty(total, dtype=torch.uint8, device=DEV)
            for (nm, k, dt), off, nb in zip(specs, offs, sizes):
                setattr(self, nm, self.arena[off: off + nb].view(dt))
        else:
            for nm, k, dt in specs:
                setattr(self, nm, torch.empty(k, dtype=dt, device=DEV))
        if not self.qb:
            self.codes = self.scales = None
        if not (self.clip and spill):
            self.gbar_ws = None
        self.sumsq = torch.zeros(1, dtype=torch.float64, device=DEV)
        self.stride = row_stride(n_)
        self.cb = w.contrib_block
        if self.cb:  # int8 contributions: codes rows and per-block scale rows
            nb = (n_ + self.cb - 1) // self.cb
            self.sstride = (nb + 63) // 64 * 64 + 64
            self.codes_buf = torch.empty(max(1, (self.nd - 1) * self.stride + n_),
                                         dtype=torch.int8, device=DEV)
            self.scales_buf = torch.empty(max(1, (self.nd - 1) * self.sstride + nb), **f32)
            self.qrows = [self.codes_buf[k * self.stride: k * self.stride + n_]
                          for k in range(self.nd)]
            self.srows = [self.scales_buf[k * self.sstride: k * self.sstride + nb]
                          for k in range(self.nd)]
            self.rows_buf = self.rows = None
        else:
            self.rows_buf = torch.empty(max(1, (self.nd - 1) * self.stride + n_),
                                        dtype=torch.int16, device=DEV)
            self.rows = [self.rows_buf[k * self.stride: k * self.stride + n_]
                         for k in range(self.nd)]
        # the host pointer tables the library takes, built once
        if self.cb:
            self.qtab, self.stab = Z.contrib_table(self.qrows), Z.contrib_table(self.srows)
        else:
            self.tab = Z.contrib_table(self.rows)
        if phi is None:
            phi, r = (w.phi, w.r) if n is None else (n_, 0)
        self.shard = Z.ZeroShard(
            phi=phi, n_d=self.nd, r=w.r if r is None else r, shard_len=n_, master=self.master,
            m=self.m, v=self.v, param_out=self.p, beta1=w.beta1, beta2=w.beta2, eps=w.eps,
            weight_decay=w.weight_decay, bias_correction=bias_correction,
            max_norm=w.max_norm, quant_block=self.qb, q_codes=self.codes,
            q_scales=self.scales, gbar_ws=self.gbar_ws,
            stream=stream if stream is not None else torch.cuda.current_stream())

    def init_state(self) -> None:
        S.dev_state(self.w, self.master, self.m, self.v, i0=self.i0)

    def fill_grads(self, s: int) -> None:
        if self.cb:
            S.dev_contrib_q8(self.w, s, self.codes_buf, self.scales_buf, self.n, self.stride,
                             self.sstride, i0=self.i0)
        else:
            S.dev_contrib(self.w, s, self.rows_buf, self.n, self.stride, i0=self.i0)

    def norm(self) -> None:
        """The clipped step's first sweep: this shard's sum of squares into
        self.sumsq (and the gradient spill when there is one)."""
        if self.cb:
            self.shard.gnorm_q8(self.qtab, self.stab, self.cb, self.sumsq)
        else:
            self.shard.gnorm(self.tab, self.sumsq)

    def update(self, s: int, lr: float | None = None) -> None:
        """The update of step s (1-based) on the resident contributions."""
        lr = self.w.lr if lr is None else lr
        spill = self.clip and self.gbar_ws is not None
        ssq = self.sumsq if self.clip else None
        if self.cb:
            self.shard.step_q8(None if spill else self.qtab, None if spill else self.stab,
                               self.cb, lr, self.w.t_of(s), ssq)
        else:
            self.shard.step(None if spill else self.tab, lr, self.w.t_of(s), ssq)

    def step(self, s: int, lr: float | None = None) -> None:
        """Step s (1-based): the norm sweep when clipping, then the update."""
        if self.clip:
            self.norm()
        self.update(s, lr)

    def host(self, lo: int = 0, hi: int | None = None) -> dict:
        hi = self.n if hi is None else hi
        out = {
            "master": self.master[lo:hi].cpu().numpy(),
            "m": self.m[lo:hi].cpu().numpy(),
            "v": self.v[lo:hi].cpu().numpy(),
            "p": self.p[lo:hi].cpu().numpy().view(np.uint16),
        }
        if self.qb:
            out["codes"] = self.codes[lo:hi].cpu().numpy()
            assert lo % self.qb == 0
            out["scales"] = self.scales[lo // self.qb:(hi + self.qb - 1) // self.qb].cpu().numpy()
        return out

    def free(self) -> None:
        self.shard.free()


class OracleWindow:
    """Oracle state of shard elements [i0, i0+n) of workload w."""

    def __init__(self, w: S.Workload, i0: int, n: int, threads: int | None = None,
                 bias_correction: bool = True):
        import oracle

        self.O = oracle
        if threads is None:  # one host thread per 2^18 elements, at most 16
            threads = max(1, min(16, int(n) >> 18))
        self.w, self.i0, self.n, self.threads = w, int(i0), int(n), threads
        self.bias_correction = int(bool(bias_correction))
        self.master, self.m, self.v = S.host_state(w, i0, n)
        self.last = None

    def hyper(self, s: int):
        w = self.w
        return self.O.Hyper(lr=w.lr, beta1=w.beta1, beta2=w.beta2, eps=w.eps,
                       weight_decay=w.weight_decay, t=w.t_of(s),
                       bias_correction=self.bias_correction)

    def step(self, s: int, sumsq_total: float | None = None):
        O = self.O
        cb = self.w.contrib_block
        if cb:
            codes, scales = S.host_contrib_q8(self.w, s, self.i0, self.n)
        else:
            rows = list(S.host_contrib(self.w, s, self.i0, self.n))
        h = self.hyper(s)
        if self.w.max_norm > 0:
            assert sumsq_total is not None
            gbar = (O.reduce_average_q8(list(codes), list(scales), cb) if cb
                    else O.reduce_average(rows))
            coef = O.clip_coef(sumsq_total, float(np.float32(self.w.max_norm)))
            O.adam(self.master, self.m, self.v, gbar, coef, h)
            p = O.f32_to_bf16(self.master)
            codes = scales = None
            if self.w.quant_block:
                codes, scales = O.quant_int8(p, self.w.quant_block)
            self.last = O.StepOut(p, codes, scales, O.sumsq(gbar))
        else:
            h.quant_block = self.w.quant_block
            if cb:
                self.last = O.step_q8(list(codes), list(scales), cb, self.master, self.m,
                                      self.v, h, threads=self.threads)
            else:
                self.last = O.step(rows, self.master, self.m, self.v, h, threads=self.threads)
        return self.last


def oracle_global_sumsq(w: S.Workload, s: int, chunk: int = 1 << 23, threads: int = 16) -> float:
    """Sum of squares of the averaged gradient over the whole shard at step
    s, streamed through the host in chunks combined in chunk order."""
    import oracle as O

    total = 0.0
    for lo in range(0, w.shard_len, chunk):
        n = min(chunk, w.shard_len - lo)
        if w.contrib_block:
            codes, scales = S.host_contrib_q8(w, s, lo, n)
            _, part = O.gbar_sumsq_q8(list(codes), list(scales), w.contrib_block,
                                      threads=threads)
        else:
            rows = S.host_contrib(w, s, lo, n)
            _, part = O.gbar_sumsq(list(rows), threads=threads)
        total += part
    return total


def windows(n: int, count: int, size: int, seed: int, extra: tuple = ()) -> list[tuple[int, int]]:
    """Disjoint windows [lo, hi) of about `size` elements: the head, the tail
    (running to n), windows at the `extra` anchor points and at seeded
    offsets.  Every window starts on a multiple of 256 elements."""
    size = min(size, n)
    last = (n - size) // 256 * 256
    anchors = [0, last] + [int(a) for a in extra]
    rng = np.random.default_rng(seed)
    while len(anchors) < count:
        anchors.append(int(rng.integers(0, max(1, n - size))))
    out = []
    for a in anchors:
        lo = min(max(0, a), last) // 256 * 256
        hi = n if lo == last else min(n, lo + size)
        if all(hi <= l2 or lo >= h2 for l2, h2 in out):
            out.append((lo, hi))
    return sorted(out)


class OffloadShard:
    """ZeRO-Offload for one rank's shard through the library's native
    pipeline (zero_shard_offload_*): the contributions and the norm pass on
    the GPU, the fp32 optimizer state in host memory and its update on host
    threads, the bf16 parameters uploaded into two alternating device
    buffers, the host update of step s overlapping the caller's work after
    the call (the one-step delayed update)."""

    def __init__(self, w: S.Workload, n: int | None = None, threads: int = 16):
        import torch

        self.torch, self.w = torch, w
        self.n = w.shard_len if n is None else int(n)
        n_ = self.n
        self.nd = w.n_d
        self.stride = row_stride(n_)
        self.rows_buf = torch.empty(max(1, (self.nd - 1) * self.stride + n_), dtype=torch.int16,
                                    device=DEV)
        self.rows = [self.rows_buf[k * self.stride: k * self.stride + n_] for k in range(self.nd)]
        self.tab = Z.contrib_table(self.rows)
        phi, r = (w.phi, w.r) if n is None else (n_, 0)
        self.master, self.m, self.v = S.host_state(w, 0, n_)
        self.codes = np.empty(n_, np.int8) if w.quant_block else None
        self.scales = np.empty(-(-n_ // w.quant_block), np.float32) if w.quant_block else None
        self.desc = Z.host_desc(phi=phi, n_d=self.nd, r=r, shard_len=n_, master=self.master,
                                m=self.m, v=self.v, param_out=None, beta1=w.beta1,
                                beta2=w.beta2, eps=w.eps, weight_decay=w.weight_decay,
                                max_norm=w.max_norm, quant_block=w.quant_block,
                                q_codes=self.codes, q_scales=self.scales)
        self.p_dev = [torch.empty(max(1, n_), dtype=torch.int16, device=DEV) for _ in range(2)]
        rc, self.o = Z.zero_shard_offload_init(self.desc, self.p_dev[0], self.p_dev[1],
                                               threads=threads)
        if rc:
            raise Z.ZeroShardError(rc, "zero_shard_offload_init")

    def fill_grads(self, s: int) -> None:
        S.dev_contrib(self.w, s, self.rows_buf, self.n, self.stride)

    def step(self, s: int, delayed: bool = True, s_other: float = 0.0) -> None:
        """Step s (s_other: the other shards' sum of squares); without
        `delayed`, also wait for its host update."""
        rc = Z.zero_shard_offload_step(self.o, self.tab, self.w.lr, self.w.t_of(s), s_other)
        if rc:
            raise Z.ZeroShardError(rc, "zero_shard_offload_step")
        if not delayed:
            self.finish()

    def finish(self) -> None:
        rc = Z.zero_shard_offload_wait(self.o)
        if rc:
            raise Z.ZeroShardError(rc, "zero_shard_offload_wait")

    def params(self):
        """The device buffer holding the newest uploaded parameters."""
        ptr = Z.zero_shard_offload_params(self.o)
        for t in self.p_dev:
            if t.data_ptr() == ptr:
                return t
        return None

    def free(self) -> None:
        if self.o is not None and self.o.value:
            rc = Z.zero_shard_offload_free(self.o)
            self.o = None
            if rc:
                raise Z.ZeroShardError(rc, "zero_shard_offload_free")
        self.o = None

    def __del__(self):
        try:
            self.free()
        except Exception:  # noqa: BLE001  (interpreter shutdown)
            pass
