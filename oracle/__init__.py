"""CPU oracle for one rank's ZeRO-1/2 shard optimizer step (Python binding).

TEST INFRASTRUCTURE ONLY.  Only the test suite, the smoke check and the
CPU-baseline leg of the benchmark may import this package.  The product path
(the HIP library and its binding) never loads it, and it shares no code with
it.  The arithmetic lives in ``zs_oracle.cpp`` (plain binary64 C++, built with
``-ffp-contract=off``); this module only marshals numpy arrays through ctypes.

Pins: every routine is checked against facts fixed by the pages or by the
mathematics in ``tests/test_oracle_pins.py``.  What no pin can fix (the
Adam epsilon placement, the 1e-6 in the clip coefficient, the quantizer's
scale convention) is a stated reading, documented at each routine.
"""

from __future__ import annotations

import ctypes
import os
from dataclasses import dataclass

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
# ZS_ORACLE_LIB names another build of zs_oracle.cpp (the mutation test
# runs the pins against builds with planted mistakes).
LIB_PATH = os.environ.get("ZS_ORACLE_LIB") or os.path.join(_HERE, "libzsoracle.so")

_c_f64 = ctypes.c_double
_c_i32 = ctypes.c_int32
_c_i64 = ctypes.c_int64
_vp = ctypes.c_void_p


class OrcHyper(ctypes.Structure):
    _fields_ = [
        ("lr", _c_f64),
        ("beta1", _c_f64),
        ("beta2", _c_f64),
        ("eps", _c_f64),
        ("weight_decay", _c_f64),
        ("bias_correction", _c_i32),
        ("quant_block", _c_i32),
        ("t", _c_i64),
        ("max_norm", _c_f64),
        ("s_other", _c_f64),
    ]


@dataclass
class Hyper:
    """Step hyper-parameters.  Float values are taken as the binary32 values
    the GPU library receives, widened to binary64."""

    lr: float = 1e-3
    beta1: float = 0.9
    beta2: float = 0.999
    eps: float = 1e-8
    weight_decay: float = 0.0
    bias_correction: int = 1
    quant_block: int = 0
    t: int = 1
    max_norm: float = 0.0
    s_other: float = 0.0

    def to_c(self) -> OrcHyper:
        f32 = lambda x: float(np.float32(x))  # noqa: E731
        return OrcHyper(
            f32(self.lr), f32(self.beta1), f32(self.beta2), f32(self.eps),
            f32(self.weight_decay), int(self.bias_correction),
            int(self.quant_block), int(self.t), f32(self.max_norm),
            float(self.s_other))


_lib = None


def lib() -> ctypes.CDLL:
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"oracle library not built: {LIB_PATH} (run __graft_entry__.build())")
        L = ctypes.CDLL(LIB_PATH)
        L.orc_model_state_bytes.restype = _c_f64
        L.orc_model_state_bytes.argtypes = [_c_f64, _c_f64, _c_i32, _c_f64]
        L.orc_bf16_to_f32.restype = ctypes.c_float
        L.orc_bf16_to_f32.argtypes = [ctypes.c_uint16]
        L.orc_f32_to_bf16.restype = ctypes.c_uint16
        L.orc_f32_to_bf16.argtypes = [ctypes.c_float]
        L.orc_cast_bf16.argtypes = [_vp, _c_i64, _vp]
        L.orc_reduce_sum.argtypes = [_vp, _c_i32, _c_i64, _vp]
        L.orc_reduce_average.argtypes = [_vp, _c_i32, _c_i64, _vp]
        L.orc_sumsq.restype = _c_f64
        L.orc_sumsq.argtypes = [_vp, _c_i64]
        L.orc_clip_coef.restype = _c_f64
        L.orc_clip_coef.argtypes = [_c_f64, _c_f64]
        L.orc_adam.argtypes = [_vp, _vp, _vp, _vp, _c_f64, _c_i64, ctypes.POINTER(OrcHyper)]
        L.orc_quant_int8.argtypes = [_vp, _c_i64, _c_i32, _vp, _vp]
        L.orc_step.restype = ctypes.c_int
        L.orc_step.argtypes = [_vp, _c_i32, _c_i64, _vp, _vp, _vp, _vp, _vp, _vp,
                               ctypes.POINTER(OrcHyper), ctypes.POINTER(_c_f64), _c_i32]
        L.orc_gbar_sumsq.restype = _c_f64
        L.orc_gbar_sumsq.argtypes = [_vp, _c_i32, _c_i64, _vp, _c_i32]
        L.orc_reduce_sum_q8.argtypes = [_vp, _vp, _c_i32, _c_i64, _c_i32, _vp]
        L.orc_reduce_average_q8.argtypes = [_vp, _vp, _c_i32, _c_i64, _c_i32, _vp]
        L.orc_gbar_sumsq_q8.restype = _c_f64
        L.orc_gbar_sumsq_q8.argtypes = [_vp, _vp, _c_i32, _c_i64, _c_i32, _vp, _c_i32]
        L.orc_dequant_bf16.argtypes = [_vp, _vp, _c_i32, _c_i64, _c_i32, _vp]
        L.orc_step_q8.restype = ctypes.c_int
        L.orc_step_q8.argtypes = [_vp, _vp, _c_i32, _c_i64, _c_i32, _vp, _vp, _vp, _vp, _vp,
                                  _vp, ctypes.POINTER(OrcHyper), ctypes.POINTER(_c_f64),
                                  _c_i32]
        _lib = L
    return _lib


def _ptr(a: np.ndarray) -> int:
    assert a.flags["C_CONTIGUOUS"]
    return a.ctypes.data


def _rows(rows) -> tuple[ctypes.Array, int, int]:
    rows = [np.ascontiguousarray(r, dtype=np.uint16) for r in rows]
    n = rows[0].size if rows else 0
    assert all(r.size == n for r in rows)
    arr = (ctypes.c_void_p * len(rows))(*[_ptr(r) for r in rows])
    arr._keep = rows  # keep the arrays alive with the pointer table
    return arr, len(rows), n


def _q8(codes, scales, block: int):
    codes = [np.ascontiguousarray(c, dtype=np.int8) for c in codes]
    n = codes[0].size if codes else 0
    nb = (n + block - 1) // block
    scales = [np.ascontiguousarray(x, dtype=np.float32) for x in scales]
    assert len(codes) == len(scales) and all(c.size == n for c in codes)
    assert all(x.size >= nb for x in scales)
    ct = (ctypes.c_void_p * len(codes))(*[_ptr(c) for c in codes])
    st = (ctypes.c_void_p * len(scales))(*[_ptr(x) for x in scales])
    ct._keep, st._keep = codes, scales
    return ct, st, len(codes), n


def model_state_bytes(n_params: float, n_gpus: float, stage: int, k: float = 12.0) -> float:
    return lib().orc_model_state_bytes(float(n_params), float(n_gpus), int(stage), float(k))


def f32_to_bf16(x: np.ndarray) -> np.ndarray:
    x = np.ascontiguousarray(x, dtype=np.float32)
    out = np.empty(x.shape, dtype=np.uint16)
    lib().orc_cast_bf16(_ptr(x), x.size, _ptr(out))
    return out


def bf16_to_f32(b) -> np.ndarray:
    b = np.ascontiguousarray(b, dtype=np.uint16)
    return np.array([lib().orc_bf16_to_f32(int(x)) for x in b.ravel()],
                    dtype=np.float32).reshape(b.shape)


def reduce_sum(rows) -> np.ndarray:
    arr, nd, n = _rows(rows)
    out = np.empty(n, dtype=np.float64)
    lib().orc_reduce_sum(arr, nd, n, _ptr(out))
    return out


def reduce_average(rows) -> np.ndarray:
    arr, nd, n = _rows(rows)
    out = np.empty(n, dtype=np.float32)
    lib().orc_reduce_average(arr, nd, n, _ptr(out))
    return out


def reduce_sum_q8(codes, scales, block: int) -> np.ndarray:
    ct, st, nd, n = _q8(codes, scales, block)
    out = np.empty(n, dtype=np.float64)
    lib().orc_reduce_sum_q8(ct, st, nd, n, int(block), _ptr(out))
    return out


def reduce_average_q8(codes, scales, block: int) -> np.ndarray:
    ct, st, nd, n = _q8(codes, scales, block)
    out = np.empty(n, dtype=np.float32)
    lib().orc_reduce_average_q8(ct, st, nd, n, int(block), _ptr(out))
    return out


def gbar_sumsq_q8(codes, scales, block: int, threads: int = 1) -> tuple[np.ndarray, float]:
    ct, st, nd, n = _q8(codes, scales, block)
    g = np.empty(n, dtype=np.float32)
    s = lib().orc_gbar_sumsq_q8(ct, st, nd, n, int(block), _ptr(g), int(threads))
    return g, s


def sumsq(gbar: np.ndarray) -> float:
    g = np.ascontiguousarray(gbar, dtype=np.float32)
    return lib().orc_sumsq(_ptr(g), g.size)


def clip_coef(s: float, max_norm: float) -> float:
    return lib().orc_clip_coef(float(s), float(max_norm))


def adam(master: np.ndarray, m: np.ndarray, v: np.ndarray, gbar: np.ndarray,
         coef: float, h: Hyper) -> None:
    """In-place update of the binary32 arrays master, m, v."""
    for a in (master, m, v):
        assert a.dtype == np.float32 and a.flags["C_CONTIGUOUS"]
    g = np.ascontiguousarray(gbar, dtype=np.float32)
    hc = h.to_c()
    lib().orc_adam(_ptr(master), _ptr(m), _ptr(v), _ptr(g), float(coef), g.size,
                   ctypes.byref(hc))


def quant_int8(p: np.ndarray, block: int) -> tuple[np.ndarray, np.ndarray]:
    p = np.ascontiguousarray(p, dtype=np.uint16)
    n = p.size
    codes = np.empty(n, dtype=np.int8)
    scales = np.empty((n + block - 1) // block, dtype=np.float32)
    lib().orc_quant_int8(_ptr(p), n, int(block), _ptr(codes), _ptr(scales))
    return codes, scales


def gbar_sumsq(rows, threads: int = 1) -> tuple[np.ndarray, float]:
    arr, nd, n = _rows(rows)
    g = np.empty(n, dtype=np.float32)
    s = lib().orc_gbar_sumsq(arr, nd, n, _ptr(g), int(threads))
    return g, s


@dataclass
class StepOut:
    p: np.ndarray
    codes: np.ndarray | None
    scales: np.ndarray | None
    sumsq: float


def step(rows, master: np.ndarray, m: np.ndarray, v: np.ndarray, h: Hyper,
         threads: int = 1) -> StepOut:
    """One shard step (a1..a5).  master, m, v are updated in place."""
    arr, nd, n = _rows(rows)
    for a in (master, m, v):
        assert a.dtype == np.float32 and a.flags["C_CONTIGUOUS"] and a.size == n
    p = np.empty(n, dtype=np.uint16)
    codes = scales = None
    cp = sp = None
    if h.quant_block > 0:
        codes = np.empty(n, dtype=np.int8)
        scales = np.empty((n + h.quant_block - 1) // h.quant_block, dtype=np.float32)
        cp, sp = _ptr(codes), _ptr(scales)
    s = _c_f64(0.0)
    hc = h.to_c()
    rc = lib().orc_step(arr, nd, n, _ptr(master), _ptr(m), _ptr(v), _ptr(p), cp, sp,
                        ctypes.byref(hc), ctypes.byref(s), int(threads))
    if rc != 0:
        raise ValueError(f"orc_step rejected its arguments (rc={rc})")
    return StepOut(p, codes, scales, s.value)


def step_q8(codes, scales, block: int, master: np.ndarray, m: np.ndarray, v: np.ndarray,
            h: Hyper, threads: int = 1) -> StepOut:
    """One shard step with int8 contributions (value = code * scale of its
    block).  master, m, v are updated in place."""
    ct, st, nd, n = _q8(codes, scales, block)
    for a in (master, m, v):
        assert a.dtype == np.float32 and a.flags["C_CONTIGUOUS"] and a.size == n
    p = np.empty(n, dtype=np.uint16)
    qc = qs = None
    cp = sp = None
    if h.quant_block > 0:
        qc = np.empty(n, dtype=np.int8)
        qs = np.empty((n + h.quant_block - 1) // h.quant_block, dtype=np.float32)
        cp, sp = _ptr(qc), _ptr(qs)
    s = _c_f64(0.0)
    hc = h.to_c()
    rc = lib().orc_step_q8(ct, st, nd, n, int(block), _ptr(master), _ptr(m), _ptr(v), _ptr(p),
                           cp, sp, ctypes.byref(hc), ctypes.byref(s), int(threads))
    if rc != 0:
        raise ValueError(f"orc_step_q8 rejected its arguments (rc={rc})")
    return StepOut(p, qc, qs, s.value)


def dequant_bf16(codes, scales, phi: int, block: int) -> np.ndarray:
    """Full bf16 vector of phi elements from the n_d shards' int8 codes and
    block scales (shard r = elements [r*ceil(phi/n_d), ...))."""
    codes = [np.ascontiguousarray(c, dtype=np.int8) for c in codes]
    scales = [np.ascontiguousarray(x, dtype=np.float32) for x in scales]
    nd = len(codes)
    per = -(-phi // nd)
    for r, (c, x) in enumerate(zip(codes, scales)):
        ln = max(0, min(per, phi - r * per))
        assert c.size >= ln and x.size >= -(-ln // block)
    ct = (ctypes.c_void_p * nd)(*[_ptr(c) if c.size else None for c in codes])
    st = (ctypes.c_void_p * nd)(*[_ptr(x) if x.size else None for x in scales])
    out = np.empty(phi, dtype=np.uint16)
    lib().orc_dequant_bf16(ct, st, nd, int(phi), int(block), _ptr(out))
    return out
