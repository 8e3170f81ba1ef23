"""Seeded synthetic inputs for the shard step: the generator and the workloads.

This package only makes numbers.  It holds none of the optimizer's
arithmetic, and both sides use it: the CPU checker regenerates windows of a
workload on the host (``libzsgen_host.so``) while the GPU path fills HBM
with the same values (``libzsgen_dev.so``); the definition is in ``zs_gen.h``
and the two builds agree bit for bit.
"""

from __future__ import annotations

import ctypes
import os

import numpy as np

from .workloads import WORKLOADS, Workload, by_name  # noqa: F401

_HERE = os.path.dirname(os.path.abspath(__file__))
HOST_LIB = os.path.join(_HERE, "libzsgen_host.so")
DEV_LIB = os.path.join(_HERE, "libzsgen_dev.so")

MASTER, MOM, VAR, GRAD, AUX, GRAD_SCALE = 0, 1, 2, 3, 4, 5
KIND_NORMAL, KIND_ABS = 0, 1

_u64, _u32, _i64, _i32, _f32, _vp = (ctypes.c_uint64, ctypes.c_uint32, ctypes.c_int64,
                                     ctypes.c_int32, ctypes.c_float, ctypes.c_void_p)

_host = None
_dev = None


def host_lib() -> ctypes.CDLL:
    global _host
    if _host is None:
        if not os.path.exists(HOST_LIB):
            raise RuntimeError(f"generator not built: {HOST_LIB} (run __graft_entry__.build())")
        L = ctypes.CDLL(HOST_LIB)
        L.zsg_host_key.restype = _u64
        L.zsg_host_key.argtypes = [_u64, _u32, _u32, _u32]
        L.zsg_host_fill_f32.argtypes = [_vp, _i64, _u64, _u32, _u32, _u32, _i64, _f32,
                                        ctypes.c_int, ctypes.c_int, ctypes.c_int]
        L.zsg_host_fill_bf16.argtypes = [_vp, _i64, _u64, _u32, _u32, _u32, _i64, _f32,
                                         ctypes.c_int, ctypes.c_int]
        L.zsg_host_fill_contrib.argtypes = [_vp, _i32, _i64, _i64, _u64, _u32, _i64, _f32,
                                            ctypes.c_int, ctypes.c_int]
        L.zsg_host_fill_contrib_q8.argtypes = [_vp, _vp, _i32, _i64, _i64, _i64, _u64, _u32,
                                               _i64, _i32, _f32, ctypes.c_int]
        _host = L
    return _host


def dev_lib() -> ctypes.CDLL:
    global _dev
    if _dev is None:
        import torch  # noqa: F401  (share torch's HIP runtime, see the binding)

        if not os.path.exists(DEV_LIB):
            raise RuntimeError(f"generator not built: {DEV_LIB} (run __graft_entry__.build())")
        L = ctypes.CDLL(DEV_LIB)
        L.zsg_dev_delay.restype = ctypes.c_int
        L.zsg_dev_delay.argtypes = [ctypes.c_double, ctypes.c_void_p]
        L.zsg_dev_fill_f32.restype = ctypes.c_int
        L.zsg_dev_fill_f32.argtypes = [_vp, _i64, _u64, _u32, _u32, _u32, _i64, _f32,
                                       ctypes.c_int, ctypes.c_int, _vp]
        L.zsg_dev_fill_bf16.restype = ctypes.c_int
        L.zsg_dev_fill_bf16.argtypes = [_vp, _i64, _u64, _u32, _u32, _u32, _i64, _f32,
                                        ctypes.c_int, _vp]
        L.zsg_dev_fill_contrib.restype = ctypes.c_int
        L.zsg_dev_fill_contrib.argtypes = [_vp, _i32, _i64, _i64, _u64, _u32, _i64, _f32,
                                           ctypes.c_int, _vp]
        L.zsg_dev_fill_contrib_q8.restype = ctypes.c_int
        L.zsg_dev_fill_contrib_q8.argtypes = [_vp, _vp, _i32, _i64, _i64, _i64, _u64, _u32,
                                              _i64, _i32, _f32, _vp]
        _dev = L
    return _dev


def _threads(values: int = 1 << 30) -> int:
    """Host threads for generating `values` numbers: at most 16 (the cores
    a GPU's share of the host has), at most one per 2^20 values (thread
    start-up costs more than small fills)."""
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:  # pragma: no cover
        n = os.cpu_count() or 1
    return max(1, min(16, n, int(values) >> 20))


# ----------------------------------------------------------------- host side

def key(seed: int, tid: int, step: int, rank: int) -> int:
    return host_lib().zsg_host_key(seed, tid, step, rank)


def host_f32(n: int, seed: int, tid: int, step: int, rank: int, i0: int, sigma: float,
             outliers: bool = False, kind: int = KIND_NORMAL) -> np.ndarray:
    out = np.empty(int(n), dtype=np.float32)
    host_lib().zsg_host_fill_f32(out.ctypes.data, int(n), seed, tid, step, rank, int(i0),
                                 float(sigma), int(outliers), int(kind), _threads(n))
    return out


def host_bf16(n: int, seed: int, tid: int, step: int, rank: int, i0: int, sigma: float,
              outliers: bool = False) -> np.ndarray:
    out = np.empty(int(n), dtype=np.uint16)
    host_lib().zsg_host_fill_bf16(out.ctypes.data, int(n), seed, tid, step, rank, int(i0),
                                  float(sigma), int(outliers), _threads(n))
    return out


def host_contrib(w: Workload, step: int, i0: int, n: int) -> np.ndarray:
    """[n_d, n] bf16 bit patterns: every rank's gradient for shard elements
    [i0, i0+n) at 1-based step `step`."""
    out = np.empty((w.n_d, int(n)), dtype=np.uint16)
    host_lib().zsg_host_fill_contrib(out.ctypes.data, w.n_d, int(n), int(n), w.seed, int(step),
                                     int(i0), float(w.grad_sigma), int(w.outliers),
                                     _threads(w.n_d * int(n)))
    return out


def host_contrib_q8(w: Workload, step: int, i0: int, n: int) -> tuple[np.ndarray, np.ndarray]:
    """Int8 contributions of every rank for shard elements [i0, i0+n) at
    step `step`: codes [n_d, n] and the scales [n_d, nb] of the blocks those
    elements fall in (i0 a multiple of the block)."""
    blk = w.contrib_block
    assert blk > 0 and i0 % blk == 0
    nb = (int(n) + blk - 1) // blk
    codes = np.empty((w.n_d, int(n)), dtype=np.int8)
    scales = np.empty((w.n_d, max(1, nb)), dtype=np.float32)
    host_lib().zsg_host_fill_contrib_q8(codes.ctypes.data, scales.ctypes.data, w.n_d, int(n),
                                        scales.shape[1], int(n), w.seed, int(step), int(i0),
                                        blk, float(w.scale_sigma), _threads(w.n_d * int(n)))
    return codes, scales[:, :nb]


def host_state(w: Workload, i0: int, n: int) -> tuple[np.ndarray, np.ndarray, np.ndarray]:
    """Initial fp32 master, m, v for shard elements [i0, i0+n)."""
    master = host_f32(n, w.seed, MASTER, 0, 0, i0, w.master_sigma)
    if w.warm:
        m = host_f32(n, w.seed, MOM, 0, 0, i0, w.m_sigma)
        v = host_f32(n, w.seed, VAR, 0, 0, i0, w.v_sigma, kind=KIND_ABS)
    else:
        m = np.zeros(int(n), dtype=np.float32)
        v = np.zeros(int(n), dtype=np.float32)
    return master, m, v


# --------------------------------------------------------------- device side

def _check(rc: int, what: str) -> None:
    if rc != 0:
        raise RuntimeError(f"{what} failed (rc={rc})")


def _stream(stream) -> int | None:
    if stream is None:
        import torch

        return torch.cuda.current_stream().cuda_stream
    if hasattr(stream, "cuda_stream"):  # a torch.cuda.Stream
        return int(stream.cuda_stream)
    return int(stream)


def dev_f32(t, seed: int, tid: int, step: int, rank: int, i0: int, sigma: float,
            outliers: bool = False, kind: int = KIND_NORMAL, stream=None) -> None:
    """Fill the contiguous float32 torch tensor `t` in place."""
    assert t.is_cuda and t.is_contiguous() and str(t.dtype) == "torch.float32"
    _check(dev_lib().zsg_dev_fill_f32(t.data_ptr(), t.numel(), seed, tid, step, rank, int(i0),
                                      float(sigma), int(outliers), int(kind), _stream(stream)),
           "zsg_dev_fill_f32")


def dev_bf16(t, seed: int, tid: int, step: int, rank: int, i0: int, sigma: float,
             outliers: bool = False, stream=None) -> None:
    """Fill the contiguous 16-bit torch tensor `t` (bf16 bit patterns)."""
    assert t.is_cuda and t.is_contiguous() and t.element_size() == 2
    _check(dev_lib().zsg_dev_fill_bf16(t.data_ptr(), t.numel(), seed, tid, step, rank, int(i0),
                                       float(sigma), int(outliers), _stream(stream)),
           "zsg_dev_fill_bf16")


def dev_delay(usec: float, stream=None) -> None:
    """Queue a wait of usec microseconds on `stream` (the arrival time of a
    bucket of inputs whose transfer is not modelled as memory traffic)."""
    _check(dev_lib().zsg_dev_delay(float(usec), _stream(stream)), "zsg_dev_delay")


def dev_contrib(w: Workload, step: int, buf, n: int, row_stride: int, i0: int = 0,
                stream=None) -> None:
    """Fill rows k = 0..n_d-1 of `buf` (16-bit, row k at k*row_stride
    elements) with every rank's gradient for shard elements [i0, i0+n)."""
    assert buf.is_cuda and buf.element_size() == 2
    assert buf.numel() >= (w.n_d - 1) * row_stride + n
    _check(dev_lib().zsg_dev_fill_contrib(buf.data_ptr(), w.n_d, int(row_stride), int(n),
                                          w.seed, int(step), int(i0), float(w.grad_sigma),
                                          int(w.outliers), _stream(stream)),
           "zsg_dev_fill_contrib")


def dev_contrib_q8(w: Workload, step: int, codes, scales, n: int, code_stride: int,
                   scale_stride: int, i0: int = 0, stream=None) -> None:
    """Fill rank k's int8 codes at codes[k*code_stride:] and its block scales
    at scales[k*scale_stride:] for shard elements [i0, i0+n)."""
    assert codes.is_cuda and codes.element_size() == 1 and scales.is_cuda
    _check(dev_lib().zsg_dev_fill_contrib_q8(codes.data_ptr(), scales.data_ptr(), w.n_d,
                                             int(code_stride), int(scale_stride), int(n),
                                             w.seed, int(step), int(i0), w.contrib_block,
                                             float(w.scale_sigma), _stream(stream)),
           "zsg_dev_fill_contrib_q8")


def dev_state(w: Workload, master, m, v, i0: int = 0, stream=None) -> None:
    dev_f32(master, w.seed, MASTER, 0, 0, i0, w.master_sigma, stream=stream)
    if w.warm:
        dev_f32(m, w.seed, MOM, 0, 0, i0, w.m_sigma, stream=stream)
        dev_f32(v, w.seed, VAR, 0, 0, i0, w.v_sigma, kind=KIND_ABS, stream=stream)
    else:
        m.zero_()
        v.zero_()
