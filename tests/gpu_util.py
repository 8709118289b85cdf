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


def check_router_grads(dg, dl, dg_ref, dl_ref, ids, gates, tol=TOL, what=""):
    """dgates and dlogits against the oracle.

    dgates: dg_j is a dot product over the intermediate width whose terms take
    their size from dY, W_down and h, which do not depend on the token; the
    BF16 rounding of h (relative 2^-9 per term) gives an error that scales
    with that common term size, not with the particular dg_j, which can be
    small by cancellation.  So the floor of the relative error is the RMS of
    dg over the whole tensor (not over one token's k values).

    dlogits: dl_j = g_j (dg_j - sum_i g_i dg_i) cancels when the dg_j are
    close, so its relative error is not bounded by that of dg.  With
    |err dg_i| <= tol * m (m = max of the token's |dg_i| and the floor above),
    |err dl_j| <= g_j (1 + sum_i g_i) tol m = 2 g_j tol m, up to the fp32
    rounding of the final product.  Entries outside the kept experts must be
    exactly 0."""
    dg = np.asarray(dg, np.float64)
    dl = np.asarray(dl, np.float64)
    assert np.all(np.isfinite(dg)) and np.all(np.isfinite(dl)), f"{what}: non-finite output"
    floor = max(float(np.sqrt(np.mean(dg_ref * dg_ref))), 1e-30)
    e = float(np.max(np.abs(dg - dg_ref) / np.maximum(np.abs(dg_ref), floor)))
    assert e <= tol, f"{what} dgates: max rel err {e:.3e} > {tol}"
    T, k = ids.shape
    rows = np.arange(T)[:, None]
    kept = np.zeros(dl.shape, bool)
    kept[rows, ids] = True
    assert np.all(dl[~kept] == 0.0), f"{what}: nonzero dlogits outside the kept experts"
    m = np.maximum(np.max(np.abs(dg_ref), axis=1, keepdims=True), floor)
    bound = 2.0 * np.asarray(gates, np.float64) * tol * m + 1e-6 * np.abs(dl_ref[rows, ids])
    err = np.abs(dl[rows, ids] - dl_ref[rows, ids])
    assert np.all(err <= bound), f"{what}: dlogits error {np.max(err / bound):.3f} x bound"
    return e
