"""Comparison rules of the parity tests (GPU result vs oracle).

* fp32 master, m, v: |gpu - oracle| <= 1e-9 + 2e-6 |oracle| element by
  element (NaN matches NaN);
* bf16 parameters: at most 1 apart in the ordered sequence of bf16 patterns
  (+0 and -0 count as equal);
* int8 codes and fp32 scales: equal bit for bit, on every block whose bf16
  input is bit-identical on both sides.  A block whose input differs (by the
  allowed 1 ulp) has another correct quantization; there the GPU's codes
  must be those of the GPU's own bf16 block, which the caller checks with
  the stand-alone quantizer.
"""

from __future__ import annotations

import numpy as np

RTOL = 2e-6
ATOL = 1e-9


def f32_close(name: str, gpu: np.ndarray, orc: np.ndarray, rtol: float = RTOL,
              atol: float = ATOL) -> dict:
    assert gpu.shape == orc.shape and gpu.dtype == np.float32 and orc.dtype == np.float32
    gpu, orc = gpu.ravel(), orc.ravel()
    # elements with equal bits pass; the rules apply to the others
    idx = np.flatnonzero(gpu.view(np.uint32) != orc.view(np.uint32))
    gs, os_ = gpu[idx], orc[idx]
    g, o = gs.astype(np.float64), os_.astype(np.float64)
    both_nan = np.isnan(g) & np.isnan(o)
    with np.errstate(invalid="ignore"):
        ok = (np.abs(g - o) <= atol + rtol * np.abs(o)) | both_nan
    if not ok.all():
        i = int(idx[np.flatnonzero(~ok)[0]])
        raise AssertionError(f"{name}: {int((~ok).sum())} of {gpu.size} out of tolerance; "
                             f"first at {i}: gpu={gpu[i]!r} oracle={orc[i]!r}")
    with np.errstate(divide="ignore", invalid="ignore"):
        rel = np.where(o != 0, np.abs(g - o) / np.abs(o), 0.0)
        rtol_only = int(((np.abs(g - o) > rtol * np.abs(o)) & ~both_nan).sum())
    ulps = np.abs(_f32_order(gs) - _f32_order(os_))
    ulps[both_nan] = 0
    return {"bitwise": 1.0 - idx.size / max(1, gpu.size),
            "max_rel": float(np.nanmax(rel)) if (~np.isnan(rel)).any() else 0.0,
            # diagnostics, not gates: binary32 ulps apart, and the elements
            # the relative bound alone (without the 1e-9 floor) would reject
            "ulp_hist": {"0": int(gpu.size - idx.size + (ulps == 0).sum()),
                         "1": int((ulps == 1).sum()), "2+": int((ulps >= 2).sum())},
            "rtol_only_out": rtol_only}


def _f32_order(x: np.ndarray) -> np.ndarray:
    """binary32 patterns mapped to integers in the order of their values
    (+0 and -0 both to 0), so that a difference counts ulps."""
    b = x.view(np.uint32).astype(np.int64)
    return np.where(b & 0x80000000, -(b & 0x7FFFFFFF), b)


def _bf16_order(b: np.ndarray) -> np.ndarray:
    b = b.astype(np.int32)
    return np.where(b & 0x8000, -(b & 0x7FFF), b)


def bf16_close(name: str, gpu: np.ndarray, orc: np.ndarray, max_ulp: int = 1) -> dict:
    gpu, orc = gpu.view(np.uint16), orc.view(np.uint16)
    assert gpu.shape == orc.shape
    nan_g = ((gpu & 0x7F80) == 0x7F80) & ((gpu & 0x7F) != 0)
    nan_o = ((orc & 0x7F80) == 0x7F80) & ((orc & 0x7F) != 0)
    d = np.abs(_bf16_order(gpu) - _bf16_order(orc))
    ok = ((d <= max_ulp) & ~nan_g & ~nan_o) | (nan_g & nan_o)
    if not ok.all():
        i = int(np.flatnonzero(~ok)[0])
        raise AssertionError(f"{name}: {int((~ok).sum())} of {ok.size} more than {max_ulp} ulp "
                             f"apart; first at {i}: gpu=0x{gpu[i]:04x} oracle=0x{orc[i]:04x}")
    return {"bitwise": float((gpu == orc).mean())}


def int8_exact(name: str, gpu_codes: np.ndarray, gpu_scales: np.ndarray, orc_codes: np.ndarray,
               orc_scales: np.ndarray, gpu_p: np.ndarray, orc_p: np.ndarray, block: int) -> np.ndarray:
    """Exact equality on blocks with identical bf16 input; returns the mask
    of blocks whose input differs (to be checked against the stand-alone
    quantizer)."""
    n = gpu_p.size
    nb = (n + block - 1) // block
    pad = nb * block - n
    diff = np.concatenate([gpu_p.view(np.uint16) != orc_p.view(np.uint16),
                           np.zeros(pad, bool)]).reshape(nb, block).any(axis=1)
    same_blk = ~diff
    cg = np.concatenate([gpu_codes, np.zeros(pad, np.int8)]).reshape(nb, block)
    co = np.concatenate([orc_codes, np.zeros(pad, np.int8)]).reshape(nb, block)
    bad_codes = (cg != co).any(axis=1) & same_blk
    both_nan = np.isnan(gpu_scales) & np.isnan(orc_scales)
    bad_scales = (gpu_scales.view(np.uint32) != orc_scales.view(np.uint32)) & same_blk & ~both_nan
    if bad_codes.any() or bad_scales.any():
        b = int(np.flatnonzero(bad_codes | bad_scales)[0])
        raise AssertionError(f"{name}: block {b} differs with identical input "
                             f"({int(bad_codes.sum())} code blocks, {int(bad_scales.sum())} scales)")
    return diff


def sumsq_tolerance(n: int, s: float, buckets: int = 1) -> float:
    """Bound on |S_gpu - S_oracle| for two binary64 sums of the same n
    non-negative (exact) squares in different orders.  A summation tree of
    height h (the most additions any term passes through) errs by at most
    h u S (u = 2^-53).  The oracle sums 2^20-element chunks, then the chunk
    partials.  The GPU sums per lane at most 64 squares (8 lane-vectors of
    8 elements), then a 64-lane butterfly (6 levels) and the 4 wave sums;
    the final kernel gives each of 1024 threads a strided run of the block
    partials (one per 16384 elements, or per 4096 with int8 contributions)
    and reduces them in a 10-level tree; the bucketed norm adds the bucket
    sums in order."""
    u = 2.0 ** -53
    chunk = 1 << 20
    orc = min(n, chunk) + n // chunk + 1
    partials = n // 4096 + 2
    gpu = 64 + 6 + 4 + partials // 1024 + 1 + 10 + buckets
    return (orc + gpu) * u * s
