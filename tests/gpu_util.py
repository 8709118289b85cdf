"""Helpers for the GPU parity tests: device upload, comparison metric."""
from __future__ import annotations

import numpy as np
import torch

import quantized_grouped_gemm_amd as qgg

DEV = "cuda:0"
TOL = 2e-2   # max relative error (row-RMS floor), BF16 operands, fp32 accumulate


def dev_bf16(a_u16: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(a_u16).view(np.int16)).to(DEV).view(torch.bfloat16)


def host_u16(t: torch.Tensor) -> np.ndarray:
    return t.contiguous().view(torch.int16).cpu().numpy().view(np.uint16)


def dev_weights(fmt: int, packed: np.ndarray, scales: np.ndarray,
                layout: int = qgg.LAYOUT_ROWS) -> qgg.QWeight:
    """Row-layout weights on the device, repacked by the library when the
    MFMA-tiled layout is asked for."""
    p = torch.from_numpy(np.ascontiguousarray(packed)).to(DEV)
    if scales.dtype == np.uint16:
        s = torch.from_numpy(np.ascontiguousarray(scales).view(np.int16)).to(DEV)
    else:
        s = torch.from_numpy(np.ascontiguousarray(scales)).to(DEV)
    w = qgg.QWeight(fmt, p, s)
    return qgg.repack(w) if layout == qgg.LAYOUT_MFMA else w


LAYOUTS = (qgg.LAYOUT_ROWS, qgg.LAYOUT_MFMA)


def bf16_to_f64(u16: np.ndarray) -> np.ndarray:
    return (u16.astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def rel_err(out: np.ndarray, ref: np.ndarray) -> float:
    """max over elements of |out - ref| / max(|ref|, rms of the reference row)."""
    out = np.asarray(out, np.float64).reshape(ref.shape[0], -1)
    ref = np.asarray(ref, np.float64).reshape(ref.shape[0], -1)
    rms = np.sqrt(np.mean(ref * ref, axis=1, keepdims=True))
    den = np.maximum(np.abs(ref), np.maximum(rms, 1e-30))
    return float(np.max(np.abs(out - ref) / den))


def assert_close(out, ref, tol=TOL, what=""):
    assert np.all(np.isfinite(out)), f"{what}: non-finite output"
    e = rel_err(out, ref)
    assert e <= tol, f"{what}: max rel err {e:.3e} > {tol}"
    return e


def sync():
    torch.cuda.synchronize()
