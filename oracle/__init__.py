"""CPU oracle for the quantized MoE grouped-GEMM path (``oracle.c``).

TEST INFRASTRUCTURE ONLY: the tests, ``__graft_entry__.smoke()`` and the bench's
``cpu_baseline`` leg may use it; the product library never does.  It shares no
code with the HIP library.  Every function computes a plain definition in
double precision; the citations are in ``oracle.c``.

Parity pins (what checks the oracle against something other than itself) live
in ``tests/test_oracle_*.py``.  Parity unpinned: the last fp32 ulps of the gate
values (compared under a tolerance only).
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SO = os.path.join(_HERE, "liboracle.so")
_lib = None

FMT_MXFP4 = 1
FMT_INT4 = 2


def build(force: bool = True, extra_cflags=()) -> str:
    """Compile ``oracle.c`` into ``liboracle.so`` with gcc and OpenMP."""
    global _lib
    if force or not os.path.exists(_SO):
        src = os.path.join(_HERE, "oracle.c")
        tmp = _SO + ".tmp"
        subprocess.check_call(["gcc", "-O2", "-fopenmp", "-fPIC", "-shared", "-std=c11",
                               "-Wall", *extra_cflags, src, "-o", tmp, "-lm"])
        os.replace(tmp, _SO)
        _lib = None
    return _SO


def _L():
    global _lib
    if _lib is None:
        if not os.path.exists(_SO):
            build()
        lib = ctypes.CDLL(_SO)
        P, i32, i64 = ctypes.c_void_p, ctypes.c_int, ctypes.c_int64
        lib.oracle_route.argtypes = [P, i32, i32, i32, P, P]
        lib.oracle_permute.argtypes = [P, i32, i32, i32, P, P, P, P, P, P]
        lib.oracle_decode.argtypes = [i32, P, P, i64, i64, P]
        lib.oracle_bf16_view.argtypes = [P, i64, P]
        lib.oracle_bf16_to_f64.argtypes = [P, i64, P]
        lib.oracle_project.argtypes = [i32, P, P, i32, i64, i64, P, i64, P, P, P]
        lib.oracle_project_t.argtypes = [i32, P, P, i32, i64, i64, P, i64, P, P]
        lib.oracle_ffn.argtypes = [i32, P, P, P, P, i32, i64, i64, P, i32, P, P, i64, P, P, P]
        lib.oracle_dx.argtypes = [i32, P, P, P, P, i32, i64, i64, P, P, i32, P, P, i64, P, P, P]
        lib.oracle_router_bwd.argtypes = [i32, P, P, P, P, i32, i64, i64, P, P, P, i32, P, i64,
                                          P, P, P]
        lib.oracle_lora_project.argtypes = [i32, P, P, i32, i64, i64, P, i64, P, P, i32,
                                            ctypes.c_double, P, P, P, P]
        lib.oracle_lora_bwd.argtypes = [i32, i64, i64, P, P, i64, P, P, i32, ctypes.c_double,
                                        P, P, P, P, P]
        lib.oracle_ffn_lora.argtypes = [i32, P, P, P, P, i32, i64, i64, P, i32, P, P, i64, P,
                                        i32, ctypes.c_double, ctypes.c_double, P, P, P, P, P]
        lib.oracle_ffn_lora_bwd.argtypes = [i32, P, P, P, P, i32, i64, i64, P, P, i32, P, P, i64,
                                            P, i32, i32, ctypes.c_double, ctypes.c_double, P, P,
                                            P, P, P, P, P, P, P]
        lib.oracle_silu.argtypes = [ctypes.c_double]
        lib.oracle_silu.restype = ctypes.c_double
        lib.oracle_silu_grad.argtypes = [ctypes.c_double]
        lib.oracle_silu_grad.restype = ctypes.c_double
        lib.oracle_num_threads.restype = i32
        _lib = lib
    return _lib


def _p(a):
    if a is None:
        return None
    assert isinstance(a, np.ndarray) and a.flags["C_CONTIGUOUS"], "arrays must be C-contiguous"
    return a.ctypes.data_as(ctypes.c_void_p)


def _check(rc, what):
    if rc != 0:
        raise ValueError(f"oracle {what} failed with code {rc}")


def num_threads() -> int:
    return int(_L().oracle_num_threads())


def route(logits: np.ndarray, k: int):
    """(ids int32 [T,k], gates float64 [T,k]) for fp32 logits [T,E]."""
    logits = np.ascontiguousarray(logits, np.float32)
    T, E = logits.shape
    ids = np.zeros((T, k), np.int32)
    gates = np.zeros((T, k), np.float64)
    _check(_L().oracle_route(_p(logits), T, E, k, _p(ids), _p(gates)), "route")
    return ids, gates


def permute(ids: np.ndarray, E: int) -> dict:
    ids = np.ascontiguousarray(ids, np.int32)
    T, k = ids.shape
    P = T * k
    out = dict(counts=np.zeros(E, np.int32), offsets=np.zeros(E + 1, np.int32),
               perm=np.zeros(P, np.int32), inv_perm=np.zeros(P, np.int32),
               active=np.zeros(E, np.int32), n_active=np.zeros(1, np.int32))
    _check(_L().oracle_permute(_p(ids), T, k, E, _p(out["counts"]), _p(out["offsets"]),
                               _p(out["perm"]), _p(out["inv_perm"]), _p(out["active"]),
                               _p(out["n_active"])), "permute")
    out["n_active"] = int(out["n_active"][0])
    return out


def decode(fmt: int, packed: np.ndarray, scales: np.ndarray) -> np.ndarray:
    """fp32 weights [N][K] of one expert (packed [N][K/2], scales [N][K/32])."""
    packed = np.ascontiguousarray(packed, np.uint8)
    scales = np.ascontiguousarray(scales)
    N, K2 = packed.shape
    w = np.zeros((N, 2 * K2), np.float32)
    _check(_L().oracle_decode(fmt, _p(packed), _p(scales), N, 2 * K2, _p(w)), "decode")
    return w


def bf16_view(w: np.ndarray) -> np.ndarray:
    w = np.ascontiguousarray(w, np.float32)
    out = np.zeros(w.shape, np.uint16)
    _L().oracle_bf16_view(_p(w), w.size, _p(out))
    return out


def bf16_to_f64(h: np.ndarray) -> np.ndarray:
    h = np.ascontiguousarray(h, np.uint16)
    out = np.zeros(h.shape, np.float64)
    _L().oracle_bf16_to_f64(_p(h), h.size, _p(out))
    return out


def project(fmt, packed, scales, x, tok, expert) -> np.ndarray:
    """double y [npairs][N] = x[tok[i]] . W_{expert[i]}^T."""
    E, N, K2 = packed.shape
    tok = np.ascontiguousarray(tok, np.int32)
    expert = np.ascontiguousarray(expert, np.int32)
    y = np.zeros((tok.size, N), np.float64)
    _check(_L().oracle_project(fmt, _p(packed), _p(scales), E, N, 2 * K2, _p(x), tok.size,
                               _p(tok), _p(expert), _p(y)), "project")
    return y


def project_t(fmt, packed, scales, a, expert) -> np.ndarray:
    """double y [npairs][K] = a[i] . W_{expert[i]} (a is BF16 [npairs][N])."""
    E, N, K2 = packed.shape
    a = np.ascontiguousarray(a, np.uint16)
    expert = np.ascontiguousarray(expert, np.int32)
    y = np.zeros((expert.size, 2 * K2), np.float64)
    _check(_L().oracle_project_t(fmt, _p(packed), _p(scales), E, N, 2 * K2, _p(a), expert.size,
                                 _p(expert), _p(y)), "project_t")
    return y


def ffn(fmt, gu, dn, x, ids, gates, toks, want_h=False):
    """(y [ntok][d], h [ntok*k][2I] or None) for the selected tokens."""
    gu_p, gu_s = gu
    dn_p, dn_s = dn
    E, N2, d2 = gu_p.shape
    d, I = 2 * d2, N2 // 2
    k = ids.shape[1]
    toks = np.ascontiguousarray(toks, np.int32)
    y = np.zeros((toks.size, d), np.float64)
    h = np.zeros((toks.size * k, N2), np.float64) if want_h else None
    gates = np.ascontiguousarray(gates, np.float64)
    _check(_L().oracle_ffn(fmt, _p(gu_p), _p(gu_s), _p(dn_p), _p(dn_s), E, d, I, _p(x), k,
                           _p(np.ascontiguousarray(ids, np.int32)), _p(gates), toks.size,
                           _p(toks), _p(y), _p(h)), "ffn")
    return y, h


def dx(fmt, gu, dn, x, dy, ids, gates, toks, want_da=False):
    """(dX [ntok][d], dA [ntok*k][I] or None) for the selected tokens."""
    gu_p, gu_s = gu
    dn_p, dn_s = dn
    E, N2, d2 = gu_p.shape
    d, I = 2 * d2, N2 // 2
    k = ids.shape[1]
    toks = np.ascontiguousarray(toks, np.int32)
    out = np.zeros((toks.size, d), np.float64)
    da = np.zeros((toks.size * k, I), np.float64) if want_da else None
    gates = np.ascontiguousarray(gates, np.float64)
    _check(_L().oracle_dx(fmt, _p(gu_p), _p(gu_s), _p(dn_p), _p(dn_s), E, d, I, _p(x), _p(dy),
                          k, _p(np.ascontiguousarray(ids, np.int32)), _p(gates), toks.size,
                          _p(toks), _p(out), _p(da)), "dx")
    return out, da


def lora_project(fmt, packed, scales, x, tok, expert, A, B, alpha, want_u=False):
    """double y [npairs][N] = x W^T + alpha (x A^T) B^T per pair (A BF16 [E][r][K],
    B BF16 [E][N][r]); with want_u also alpha * (x A^T) [npairs][r]."""
    E, N, K2 = packed.shape
    rank = A.shape[1]
    assert A.shape == (E, rank, 2 * K2) and B.shape == (E, N, rank)
    tok = np.ascontiguousarray(tok, np.int32)
    expert = np.ascontiguousarray(expert, np.int32)
    y = np.zeros((tok.size, N), np.float64)
    u = np.zeros((tok.size, rank), np.float64) if want_u else None
    _check(_L().oracle_lora_project(fmt, _p(packed), _p(scales), E, N, 2 * K2, _p(x), tok.size,
                                    _p(tok), _p(expert), rank, float(alpha),
                                    _p(np.ascontiguousarray(A, np.uint16)),
                                    _p(np.ascontiguousarray(B, np.uint16)), _p(y), _p(u)),
           "lora_project")
    return (y, u) if want_u else y


def lora_bwd(x, dy, tok, expert, A, B, alpha):
    """(dx [npairs][K], dA [E][r][K], dB [E][N][r]) in double: the adapter term's
    gradients for L = <dY, y> (dy BF16 [npairs][N])."""
    E, rank, K = A.shape
    N = B.shape[1]
    tok = np.ascontiguousarray(tok, np.int32)
    expert = np.ascontiguousarray(expert, np.int32)
    dx = np.zeros((tok.size, K), np.float64)
    dA = np.zeros((E, rank, K), np.float64)
    dB = np.zeros((E, N, rank), np.float64)
    _check(_L().oracle_lora_bwd(E, N, K, _p(np.ascontiguousarray(x, np.uint16)),
                                _p(np.ascontiguousarray(dy, np.uint16)), tok.size, _p(tok),
                                _p(expert), rank, float(alpha),
                                _p(np.ascontiguousarray(A, np.uint16)),
                                _p(np.ascontiguousarray(B, np.uint16)), _p(dx), _p(dA), _p(dB)),
           "lora_bwd")
    return dx, dA, dB


def ffn_lora(fmt, gu, dn, x, ids, gates, toks, lora_gu, lora_dn, alpha_gu, alpha_dn=None):
    """y [ntok][d] of the SwiGLU FFN with LoRA adapters: lora_gu = (A [E][r][d],
    B [E][2I][r]) and lora_dn = (A [E][r][I], B [E][d][r]) BF16 bits, or None;
    alpha_dn defaults to alpha_gu."""
    alpha_dn = alpha_gu if alpha_dn is None else alpha_dn
    gu_p, gu_s = gu
    dn_p, dn_s = dn
    E, N2, d2 = gu_p.shape
    d, I = 2 * d2, N2 // 2
    k = ids.shape[1]
    rank = (lora_gu or lora_dn)[0].shape[1]
    toks = np.ascontiguousarray(toks, np.int32)
    y = np.zeros((toks.size, d), np.float64)
    c = lambda a: None if a is None else np.ascontiguousarray(a, np.uint16)
    Agu, Bgu = (c(lora_gu[0]), c(lora_gu[1])) if lora_gu else (None, None)
    Adn, Bdn = (c(lora_dn[0]), c(lora_dn[1])) if lora_dn else (None, None)
    _check(_L().oracle_ffn_lora(fmt, _p(gu_p), _p(gu_s), _p(dn_p), _p(dn_s), E, d, I, _p(x), k,
                                _p(np.ascontiguousarray(ids, np.int32)),
                                _p(np.ascontiguousarray(gates, np.float64)), toks.size, _p(toks),
                                rank, float(alpha_gu), float(alpha_dn), _p(Agu), _p(Bgu), _p(Adn),
                                _p(Bdn), _p(y)),
           "ffn_lora")
    return y


def ffn_lora_bwd(fmt, gu, dn, x, dy, ids, gates, toks, lora_gu=None, lora_dn=None):
    """Backward of the SwiGLU FFN with LoRA adapters for L = <dY, y>, base and
    gates fixed.  lora_gu = (A [E][r][d], B [E][2I][r], alpha) and lora_dn =
    (A [E][r][I], B [E][d][r], alpha) BF16 bits, or None.  Returns a dict of
    double arrays: dx [ntok][d] for the selected tokens, dA_gu, dB_gu, dA_dn,
    dB_dn (None for an absent adapter; sums over the selected tokens' pairs)."""
    gu_p, gu_s = gu
    dn_p, dn_s = dn
    E, N2, d2 = gu_p.shape
    d, I = 2 * d2, N2 // 2
    k = ids.shape[1]
    toks = np.ascontiguousarray(toks, np.int32)
    c = lambda a: np.ascontiguousarray(a, np.uint16)  # noqa: E731
    out = {"dx": np.zeros((toks.size, d), np.float64)}
    args = []
    for name, l, K, N in (("gu", lora_gu, d, N2), ("dn", lora_dn, I, d)):
        if l is None:
            args.append((0, 0.0, None, None))
            out["dA_" + name] = out["dB_" + name] = None
            continue
        A, B, alpha = l
        r = A.shape[1]
        assert A.shape == (E, r, K) and B.shape == (E, N, r)
        out["dA_" + name] = np.zeros((E, r, K), np.float64)
        out["dB_" + name] = np.zeros((E, N, r), np.float64)
        args.append((r, float(alpha), c(A), c(B)))
    (rg, ag, Ag, Bg), (rd, ad, Ad, Bd) = args
    _check(_L().oracle_ffn_lora_bwd(fmt, _p(gu_p), _p(gu_s), _p(dn_p), _p(dn_s), E, d, I,
                                    _p(c(x)), _p(c(dy)), k,
                                    _p(np.ascontiguousarray(ids, np.int32)),
                                    _p(np.ascontiguousarray(gates, np.float64)), toks.size,
                                    _p(toks), rg, rd, ag, ad, _p(Ag), _p(Bg), _p(Ad), _p(Bd),
                                    _p(out["dx"]), _p(out["dA_gu"]), _p(out["dB_gu"]),
                                    _p(out["dA_dn"]), _p(out["dB_dn"])), "ffn_lora_bwd")
    return out


def router_bwd(fmt, gu, dn, x, dy, logits, ids, toks):
    """(dgates [ntok][k], dlogits [ntok][E]) of L = <dY, y> for the selected
    tokens, routing choice held fixed; gates re-derived from the logits."""
    gu_p, gu_s = gu
    dn_p, dn_s = dn
    E, N2, d2 = gu_p.shape
    d, I = 2 * d2, N2 // 2
    k = ids.shape[1]
    toks = np.ascontiguousarray(toks, np.int32)
    logits = np.ascontiguousarray(logits, np.float32)
    assert logits.shape[1] == E
    dg = np.zeros((toks.size, k), np.float64)
    dl = np.zeros((toks.size, E), np.float64)
    _check(_L().oracle_router_bwd(fmt, _p(gu_p), _p(gu_s), _p(dn_p), _p(dn_s), E, d, I, _p(x),
                                  _p(dy), _p(logits), k, _p(np.ascontiguousarray(ids, np.int32)),
                                  toks.size, _p(toks), _p(dg), _p(dl)), "router_bwd")
    return dg, dl


def silu(z: float) -> float:
    return float(_L().oracle_silu(z))


def silu_grad(z: float) -> float:
    return float(_L().oracle_silu_grad(z))
