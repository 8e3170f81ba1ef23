"""Python binding of the MI355X ZeRO-1/2 shard optimizer step.

Argument marshalling only: every step of the path runs in the HIP kernels of
``libzeroshard.so`` behind the C ABI of ``include/zero_shard.h``.  The
functions below carry the C names; ``ZeroShard`` is a small owner object
over one handle.  PyTorch is used for device memory and streams only.

There is no fallback: importing this package without the built library
raises, and every call that returns a negative status raises ``ZeroShardError``.
"""

from __future__ import annotations

import ctypes
import os

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libzeroshard.so")

ZS_OK, ZS_EINVAL, ZS_EALIGN, ZS_ENOMEM, ZS_EHIP, ZS_EDEVICE, ZS_ESTATE, ZS_ETOOBIG = (
    0, -1, -2, -3, -4, -5, -6, -7)
ZS_MAX_ND = 64
# how a call's work is split into kernel launches (zero_shard.h)
ZS_NORM_LAUNCH_LEN = 1 << 26
ZS_WIDE_LAUNCH_LEN = 1 << 25
ZS_WIDE_MIN_ROWS = 18
ZS_WIDE_MIN_ROWS_QUANT = 32
ZS_WIDE_MIN_ROWS_Q8 = 16
QUANT_BLOCKS = (32, 64, 128, 256, 512)

if not os.path.exists(LIB_PATH):
    raise ImportError(f"{LIB_PATH} is not built; run __graft_entry__.build() (hipcc, gfx950)")

# The library must run on the same HIP runtime as the PyTorch that owns the
# device memory and streams.  Loading torch first makes the library's
# libamdhip64.so.7 dependency resolve to torch's already-loaded runtime;
# the other order would map a second runtime into the process.
import torch  # noqa: E402,F401

_lib = ctypes.CDLL(LIB_PATH)


class zs_desc(ctypes.Structure):  # noqa: N801  (the C name)
    _fields_ = [
        ("phi", ctypes.c_int64),
        ("n_d", ctypes.c_int32),
        ("r", ctypes.c_int32),
        ("shard_len", ctypes.c_int64),
        ("beta1", ctypes.c_float),
        ("beta2", ctypes.c_float),
        ("eps", ctypes.c_float),
        ("weight_decay", ctypes.c_float),
        ("bias_correction", ctypes.c_int32),
        ("max_norm", ctypes.c_float),
        ("quant_block", ctypes.c_int32),
        ("master", ctypes.c_void_p),
        ("m", ctypes.c_void_p),
        ("v", ctypes.c_void_p),
        ("param_out", ctypes.c_void_p),
        ("q_codes", ctypes.c_void_p),
        ("q_scales", ctypes.c_void_p),
        ("gbar_ws", ctypes.c_void_p),
        ("stream", ctypes.c_void_p),
    ]


_handle_p = ctypes.c_void_p
_lib.zero_shard_init.restype = ctypes.c_int
_lib.zero_shard_init.argtypes = [ctypes.POINTER(zs_desc), ctypes.POINTER(_handle_p)]
_lib.zero_shard_gnorm.restype = ctypes.c_int
_lib.zero_shard_gnorm.argtypes = [_handle_p, ctypes.c_void_p, ctypes.c_void_p]
_lib.zero_shard_step_consts.restype = ctypes.c_int
_lib.zero_shard_step_consts.argtypes = [ctypes.POINTER(zs_desc), ctypes.c_float, ctypes.c_int64,
                                        ctypes.c_void_p]
_lib.zero_shard_step_dev.restype = ctypes.c_int
_lib.zero_shard_step_dev.argtypes = [_handle_p, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p]
_lib.zero_shard_gnorm_noalloc.restype = ctypes.c_int
_lib.zero_shard_gnorm_noalloc.argtypes = [ctypes.POINTER(zs_desc), ctypes.c_void_p,
                                          ctypes.c_void_p]
_lib.zero_shard_step.restype = ctypes.c_int
_lib.zero_shard_step.argtypes = [_handle_p, ctypes.c_void_p, ctypes.c_float, ctypes.c_int64,
                                 ctypes.c_void_p]
_lib.zero_shard_gnorm_q8.restype = ctypes.c_int
_lib.zero_shard_gnorm_q8.argtypes = [_handle_p, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int32,
                                     ctypes.c_void_p]
_lib.zero_shard_step_q8.restype = ctypes.c_int
_lib.zero_shard_step_q8.argtypes = [_handle_p, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int32,
                                    ctypes.c_float, ctypes.c_int64, ctypes.c_void_p]
_lib.zero_shard_gnorm_bucketed.restype = ctypes.c_int
_lib.zero_shard_gnorm_bucketed.argtypes = [_handle_p, ctypes.c_void_p, ctypes.c_int64,
                                           ctypes.c_int32, ctypes.c_void_p, ctypes.c_void_p]
_lib.zero_shard_step_bucketed.restype = ctypes.c_int
_lib.zero_shard_step_bucketed.argtypes = [_handle_p, ctypes.c_void_p, ctypes.c_int64,
                                          ctypes.c_int32, ctypes.c_void_p, ctypes.c_float,
                                          ctypes.c_int64, ctypes.c_void_p]
_lib.zero_shard_gnorm_bucketed_q8.restype = ctypes.c_int
_lib.zero_shard_gnorm_bucketed_q8.argtypes = [_handle_p, ctypes.c_void_p, ctypes.c_void_p,
                                              ctypes.c_int32, ctypes.c_int64, ctypes.c_int32,
                                              ctypes.c_void_p, ctypes.c_void_p]
_lib.zero_shard_step_bucketed_q8.restype = ctypes.c_int
_lib.zero_shard_step_bucketed_q8.argtypes = [_handle_p, ctypes.c_void_p, ctypes.c_void_p,
                                             ctypes.c_int32, ctypes.c_int64, ctypes.c_int32,
                                             ctypes.c_void_p, ctypes.c_float, ctypes.c_int64,
                                             ctypes.c_void_p]
_lib.zero_shard_dequant.restype = ctypes.c_int
_lib.zero_shard_dequant.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int32,
                                    ctypes.c_int64, ctypes.c_int32, ctypes.c_void_p,
                                    ctypes.c_void_p]
_lib.zero_shard_host_step.restype = ctypes.c_int
_lib.zero_shard_host_step.argtypes = [ctypes.POINTER(zs_desc), ctypes.c_void_p, ctypes.c_float,
                                      ctypes.c_int64, ctypes.c_double, ctypes.c_int32]
_lib.zero_shard_offload_init.restype = ctypes.c_int
_lib.zero_shard_offload_init.argtypes = [ctypes.POINTER(zs_desc), ctypes.c_void_p,
                                         ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int32,
                                         ctypes.POINTER(_handle_p)]
_lib.zero_shard_offload_step.restype = ctypes.c_int
_lib.zero_shard_offload_step.argtypes = [_handle_p, ctypes.c_void_p, ctypes.c_float,
                                         ctypes.c_int64, ctypes.c_double]
_lib.zero_shard_offload_params.restype = ctypes.c_void_p
_lib.zero_shard_offload_params.argtypes = [_handle_p]
_lib.zero_shard_offload_wait.restype = ctypes.c_int
_lib.zero_shard_offload_wait.argtypes = [_handle_p]
_lib.zero_shard_offload_free.restype = ctypes.c_int
_lib.zero_shard_offload_free.argtypes = [_handle_p]
_lib.zero_shard_quant.restype = ctypes.c_int
_lib.zero_shard_quant.argtypes = [_handle_p, ctypes.c_int32]
_lib.zero_shard_free.restype = ctypes.c_int
_lib.zero_shard_free.argtypes = [_handle_p]
_lib.zero_shard_strerror.restype = ctypes.c_char_p
_lib.zero_shard_strerror.argtypes = [ctypes.c_int]
_lib.zero_shard_len.restype = ctypes.c_int64
_lib.zero_shard_len.argtypes = [ctypes.c_int64, ctypes.c_int32, ctypes.c_int32]

EXPORTS = ("zero_shard_init", "zero_shard_gnorm", "zero_shard_gnorm_noalloc", "zero_shard_step",
           "zero_shard_step_consts", "zero_shard_step_dev",
           "zero_shard_gnorm_q8",
           "zero_shard_step_q8", "zero_shard_gnorm_bucketed", "zero_shard_step_bucketed",
           "zero_shard_gnorm_bucketed_q8", "zero_shard_step_bucketed_q8",
           "zero_shard_quant", "zero_shard_dequant",
           "zero_shard_host_step", "zero_shard_offload_init", "zero_shard_offload_step",
           "zero_shard_offload_params", "zero_shard_offload_wait", "zero_shard_offload_free",
           "zero_shard_free", "zero_shard_strerror", "zero_shard_len")


class ZeroShardError(RuntimeError):
    def __init__(self, code: int, what: str):
        self.code = code
        super().__init__(f"{what}: {zero_shard_strerror(code)} ({code})")


def _check(rc: int, what: str) -> None:
    if rc != ZS_OK:
        raise ZeroShardError(rc, what)


def _ptr(t) -> int | None:
    if t is None:
        return None
    return int(t.data_ptr())


def contrib_table(contrib) -> ctypes.Array | None:
    """Host array of device pointers: a list of 1-D tensors (or None), or the
    rows of a 2-D tensor (row k = rank k's contribution, codes or scales)."""
    if contrib is None:
        return None
    if isinstance(contrib, ctypes.Array):  # already a table (kept by the caller)
        return contrib
    if hasattr(contrib, "dim") and contrib.dim() == 2:
        rows = [contrib[k] for k in range(contrib.shape[0])]
    else:
        rows = list(contrib)
    tab = (ctypes.c_void_p * max(1, len(rows)))(*[_ptr(r) for r in rows])
    tab._keep = rows
    return tab


# ------------------------------------------------------------ C-named calls

def zero_shard_strerror(code: int) -> str:
    return _lib.zero_shard_strerror(int(code)).decode()


def zero_shard_len(phi: int, n_d: int, r: int) -> int:
    return int(_lib.zero_shard_len(int(phi), int(n_d), int(r)))


def zero_shard_init(desc: zs_desc) -> tuple[int, ctypes.c_void_p]:
    h = _handle_p()
    rc = _lib.zero_shard_init(ctypes.byref(desc), ctypes.byref(h))
    return rc, h


def zero_shard_gnorm(h, contrib, sumsq_dev) -> int:
    return _lib.zero_shard_gnorm(h, contrib_table(contrib), _ptr(sumsq_dev))


def zero_shard_gnorm_noalloc(desc: zs_desc, contrib, sumsq_dev) -> int:
    """zero_shard_gnorm without a handle and without allocating (desc: a
    zs_desc; its n_d, shard_len, gbar_ws and stream are used)."""
    return _lib.zero_shard_gnorm_noalloc(ctypes.byref(desc), contrib_table(contrib),
                                         _ptr(sumsq_dev))


def zero_shard_step(h, contrib, lr: float, t: int, global_sumsq_dev=None) -> int:
    return _lib.zero_shard_step(h, contrib_table(contrib), float(lr), int(t),
                                _ptr(global_sumsq_dev))


def zero_shard_step_consts(desc: zs_desc, lr: float, t: int):
    """-> (status, [lr, lr*wd, bc1, bc2]) as the library computes them."""
    out = (ctypes.c_double * 4)()
    rc = _lib.zero_shard_step_consts(ctypes.byref(desc), float(lr), int(t), out)
    return rc, list(out)


def zero_shard_step_dev(h, contrib, consts_dev, global_sumsq_dev=None) -> int:
    """consts_dev: a float64 device tensor of 4 (see zero_shard_step_consts)."""
    return _lib.zero_shard_step_dev(h, contrib_table(contrib), _ptr(consts_dev),
                                    _ptr(global_sumsq_dev))


def zero_shard_gnorm_q8(h, codes, scales, block: int, sumsq_dev) -> int:
    return _lib.zero_shard_gnorm_q8(h, contrib_table(codes), contrib_table(scales), int(block),
                                    _ptr(sumsq_dev))


def zero_shard_step_q8(h, codes, scales, block: int, lr: float, t: int,
                       global_sumsq_dev=None) -> int:
    return _lib.zero_shard_step_q8(h, contrib_table(codes), contrib_table(scales), int(block),
                                   float(lr), int(t), _ptr(global_sumsq_dev))


def event_table(ready) -> ctypes.Array | None:
    """Host array of hipEvent_t from a list of torch.cuda.Event (or None
    entries); None stays None.  Each event must have been recorded."""
    if ready is None:
        return None
    tab = (ctypes.c_void_p * max(1, len(ready)))(
        *[None if e is None else int(e.cuda_event) for e in ready])
    tab._keep = list(ready)
    return tab


def zero_shard_gnorm_bucketed(h, contrib, bucket_len: int, streams: int, ready,
                              sumsq_dev) -> int:
    return _lib.zero_shard_gnorm_bucketed(h, contrib_table(contrib), int(bucket_len),
                                          int(streams), event_table(ready), _ptr(sumsq_dev))


def zero_shard_step_bucketed(h, contrib, bucket_len: int, streams: int, ready, lr: float,
                             t: int, global_sumsq_dev=None) -> int:
    return _lib.zero_shard_step_bucketed(h, contrib_table(contrib), int(bucket_len),
                                         int(streams), event_table(ready), float(lr), int(t),
                                         _ptr(global_sumsq_dev))


def zero_shard_gnorm_bucketed_q8(h, codes, scales, block: int, bucket_len: int, streams: int,
                                 ready, sumsq_dev) -> int:
    return _lib.zero_shard_gnorm_bucketed_q8(h, contrib_table(codes), contrib_table(scales),
                                             int(block), int(bucket_len), int(streams),
                                             event_table(ready), _ptr(sumsq_dev))


def zero_shard_step_bucketed_q8(h, codes, scales, block: int, bucket_len: int, streams: int,
                                ready, lr: float, t: int, global_sumsq_dev=None) -> int:
    return _lib.zero_shard_step_bucketed_q8(h, contrib_table(codes), contrib_table(scales),
                                            int(block), int(bucket_len), int(streams),
                                            event_table(ready), float(lr), int(t),
                                            _ptr(global_sumsq_dev))


def zero_shard_quant(h, block: int) -> int:
    return _lib.zero_shard_quant(h, int(block))


def zero_shard_dequant(codes, scales, n_d: int, phi: int, block: int, param_out,
                       stream=None) -> int:
    """param_out: 16-bit tensor of phi elements; stream: a torch stream
    (default: the current one)."""
    if stream is None:
        import torch

        stream = torch.cuda.current_stream()
    return _lib.zero_shard_dequant(contrib_table(codes), contrib_table(scales), int(n_d), int(phi),
                                   int(block), _ptr(param_out), int(stream.cuda_stream))


def zero_shard_host_step(desc: zs_desc, gbar_host_ptr: int, lr: float, t: int,
                         global_sumsq: float = 0.0, threads: int = 1) -> int:
    """desc carries HOST pointers; gbar_host_ptr: address of fp32[shard_len]
    in host memory."""
    return _lib.zero_shard_host_step(ctypes.byref(desc), gbar_host_ptr, float(lr), int(t),
                                     float(global_sumsq), int(threads))


def host_desc(*, phi: int, n_d: int, r: int, shard_len: int, master, m, v, param_out,
              beta1: float = 0.9, beta2: float = 0.999, eps: float = 1e-8,
              weight_decay: float = 0.0, bias_correction: bool = True, max_norm: float = 0.0,
              quant_block: int = 0, q_codes=None, q_scales=None) -> zs_desc:
    """A descriptor over host arrays (numpy arrays or CPU tensors) for
    zero_shard_host_step; keep the arrays alive while it is used."""
    def addr(a):
        if a is None:
            return None
        return int(a.ctypes.data) if hasattr(a, "ctypes") else int(a.data_ptr())

    return zs_desc(phi=int(phi), n_d=int(n_d), r=int(r), shard_len=int(shard_len),
                   beta1=beta1, beta2=beta2, eps=eps, weight_decay=weight_decay,
                   bias_correction=int(bool(bias_correction)), max_norm=max_norm,
                   quant_block=int(quant_block), master=addr(master), m=addr(m), v=addr(v),
                   param_out=addr(param_out), q_codes=addr(q_codes), q_scales=addr(q_scales),
                   gbar_ws=None, stream=None)


def zero_shard_offload_init(host: zs_desc, param_dev0, param_dev1, stream=None,
                            threads: int = 16):
    """-> (status, handle).  host: a host_desc(...); param_dev0/1: 16-bit
    device tensors of shard_len elements; stream: a torch stream (default:
    the current one)."""
    if stream is None:
        import torch

        stream = torch.cuda.current_stream()
    o = _handle_p()
    rc = _lib.zero_shard_offload_init(ctypes.byref(host), _ptr(param_dev0), _ptr(param_dev1),
                                      int(stream.cuda_stream), int(threads), ctypes.byref(o))
    return rc, o


def zero_shard_offload_step(o, contrib, lr: float, t: int, s_other: float = 0.0) -> int:
    return _lib.zero_shard_offload_step(o, contrib_table(contrib), float(lr), int(t),
                                        float(s_other))


def zero_shard_offload_params(o) -> int | None:
    return _lib.zero_shard_offload_params(o)


def zero_shard_offload_wait(o) -> int:
    return _lib.zero_shard_offload_wait(o)


def zero_shard_offload_free(o) -> int:
    return _lib.zero_shard_offload_free(o)


def zero_shard_free(h) -> int:
    return _lib.zero_shard_free(h)


# ------------------------------------------------------------- owner object

class ZeroShard:
    """One rank's shard step over caller-owned torch tensors.

    master, m, v: float32[shard_len]; param_out: 16-bit [shard_len] (bf16
    patterns); q_codes int8[shard_len] and q_scales float32[ceil(n/block)]
    when quantizing; gbar_ws float32[shard_len] optional (clipping spill).
    All on the current device.  ``stream`` is a torch stream (default: the
    current stream at construction)."""

    def __init__(self, *, phi: int, n_d: int, r: int, shard_len: int, master, m, v, param_out,
                 beta1: float = 0.9, beta2: float = 0.999, eps: float = 1e-8,
                 weight_decay: float = 0.0, bias_correction: bool = True,
                 max_norm: float = 0.0, quant_block: int = 0, q_codes=None, q_scales=None,
                 gbar_ws=None, stream=None):
        if stream is None:
            import torch

            stream = torch.cuda.current_stream()
        self._keep = (master, m, v, param_out, q_codes, q_scales, gbar_ws, stream)
        self.desc = zs_desc(
            phi=int(phi), n_d=int(n_d), r=int(r), shard_len=int(shard_len),
            beta1=beta1, beta2=beta2, eps=eps, weight_decay=weight_decay,
            bias_correction=int(bool(bias_correction)), max_norm=max_norm,
            quant_block=int(quant_block), master=_ptr(master), m=_ptr(m), v=_ptr(v),
            param_out=_ptr(param_out), q_codes=_ptr(q_codes), q_scales=_ptr(q_scales),
            gbar_ws=_ptr(gbar_ws), stream=int(stream.cuda_stream))
        rc, self.h = zero_shard_init(self.desc)
        _check(rc, "zero_shard_init")

    def gnorm(self, contrib, sumsq_dev) -> None:
        _check(zero_shard_gnorm(self.h, contrib, sumsq_dev), "zero_shard_gnorm")

    def step(self, contrib, lr: float, t: int, global_sumsq_dev=None) -> None:
        _check(zero_shard_step(self.h, contrib, lr, t, global_sumsq_dev), "zero_shard_step")

    def step_dev(self, contrib, consts_dev, global_sumsq_dev=None) -> None:
        _check(zero_shard_step_dev(self.h, contrib, consts_dev, global_sumsq_dev),
               "zero_shard_step_dev")

    def consts(self, lr: float, t: int) -> list[float]:
        rc, out = zero_shard_step_consts(self.desc, lr, t)
        _check(rc, "zero_shard_step_consts")
        return out

    def gnorm_q8(self, codes, scales, block: int, sumsq_dev) -> None:
        _check(zero_shard_gnorm_q8(self.h, codes, scales, block, sumsq_dev), "zero_shard_gnorm_q8")

    def step_q8(self, codes, scales, block: int, lr: float, t: int, global_sumsq_dev=None) -> None:
        _check(zero_shard_step_q8(self.h, codes, scales, block, lr, t, global_sumsq_dev),
               "zero_shard_step_q8")

    def gnorm_bucketed(self, contrib, bucket_len: int, sumsq_dev, streams: int = 2,
                       ready=None) -> None:
        _check(zero_shard_gnorm_bucketed(self.h, contrib, bucket_len, streams, ready, sumsq_dev),
               "zero_shard_gnorm_bucketed")

    def step_bucketed(self, contrib, bucket_len: int, lr: float, t: int, global_sumsq_dev=None,
                      streams: int = 2, ready=None) -> None:
        _check(zero_shard_step_bucketed(self.h, contrib, bucket_len, streams, ready, lr, t,
                                        global_sumsq_dev), "zero_shard_step_bucketed")

    def gnorm_bucketed_q8(self, codes, scales, block: int, bucket_len: int, sumsq_dev,
                          streams: int = 2, ready=None) -> None:
        _check(zero_shard_gnorm_bucketed_q8(self.h, codes, scales, block, bucket_len, streams,
                                            ready, sumsq_dev), "zero_shard_gnorm_bucketed_q8")

    def step_bucketed_q8(self, codes, scales, block: int, bucket_len: int, lr: float, t: int,
                         global_sumsq_dev=None, streams: int = 2, ready=None) -> None:
        _check(zero_shard_step_bucketed_q8(self.h, codes, scales, block, bucket_len, streams,
                                           ready, lr, t, global_sumsq_dev),
               "zero_shard_step_bucketed_q8")

    def quant(self, block: int) -> None:
        _check(zero_shard_quant(self.h, block), "zero_shard_quant")

    def free(self) -> None:
        if self.h is not None and self.h.value:
            _check(zero_shard_free(self.h), "zero_shard_free")
        self.h = None

    def __enter__(self):
        return self

    def __exit__(self, *exc):
        self.free()

    def __del__(self):
        try:
            if getattr(self, "h", None) is not None and self.h.value:
                zero_shard_free(self.h)
        except Exception:
            pass
