"""Seeded synthetic inputs shared by the CPU oracle and the GPU library.

The C source (``synth.c``) draws every tensor from Philox4x32-10 streams and
encodes expert weights into the frozen-base formats (MXFP4: E2M1 codes with
one E8M0 exponent per 32 elements along K; INT4: two's-complement nibbles with
one BF16 scale per 32 elements).  Nothing here routes, permutes, decodes or
multiplies: the method's arithmetic lives only in ``oracle/`` (CPU reference)
and in the HIP library.

Microscaling groups of 32 sharing one scale follow the MXFP4 description on the
page "超大规模开放权重模型技术解析" (section 三, 微缩放量化的原理); the INT4 base
is the one named for Kimi-K2.6 on the Orbit page (单节点 Kimi-K2.6 驱散).
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

from .configs import CONFIGS, Config, STREAM  # noqa: F401

_HERE = os.path.dirname(os.path.abspath(__file__))
_SO = os.path.join(_HERE, "libsynth.so")
_lib = None

FMT_MXFP4 = 1
FMT_INT4 = 2


def build(force: bool = True) -> str:
    """Compile ``synth.c`` into ``libsynth.so`` (gcc, OpenMP)."""
    global _lib
    if force or not os.path.exists(_SO):
        src = os.path.join(_HERE, "synth.c")
        tmp = _SO + ".tmp"
        subprocess.check_call(
            ["gcc", "-O3", "-march=x86-64-v2", "-fopenmp", "-fPIC", "-shared",
             "-std=c11", "-Wall", src, "-o", tmp, "-lm"])
        os.replace(tmp, _SO)
        _lib = None
    return _SO


def _L():
    global _lib
    if _lib is None:
        if not os.path.exists(_SO):
            build()
        lib = ctypes.CDLL(_SO)
        P = ctypes.c_void_p
        i64, u64, u32, f32 = ctypes.c_int64, ctypes.c_uint64, ctypes.c_uint32, ctypes.c_float
        lib.synth_philox4x32_10.argtypes = [P, P, P]
        lib.synth_normal_bf16.argtypes = [u64, u32, i64, i64, f32, f32, P]
        lib.synth_normal_f32.argtypes = [u64, u32, i64, i64, f32, P, i64, P]
        lib.synth_zipf_bias.argtypes = [u64, u32, ctypes.c_int, ctypes.c_double, P, P]
        lib.synth_qweights.argtypes = [u64, u32, ctypes.c_int, i64, i64, i64, i64, i64, f32, P, P]
        lib.synth_qweights.restype = ctypes.c_int
        lib.synth_weights_f32.argtypes = [u64, u32, i64, i64, i64, f32, P]
        lib.synth_encode_mxfp4_group.argtypes = [P, P]
        lib.synth_encode_mxfp4_group.restype = ctypes.c_uint8
        lib.synth_encode_int4_group.argtypes = [P, P]
        lib.synth_encode_int4_group.restype = ctypes.c_uint16
        lib.synth_quantile_table.restype = ctypes.POINTER(ctypes.c_float)
        lib.synth_num_threads.restype = ctypes.c_int
        _lib = lib
    return _lib


def _p(a: np.ndarray):
    assert a.flags["C_CONTIGUOUS"]
    return a.ctypes.data_as(ctypes.c_void_p)


def philox4x32_10(ctr, key) -> np.ndarray:
    c = np.asarray(ctr, dtype=np.uint32).copy()
    k = np.asarray(key, dtype=np.uint32).copy()
    out = np.zeros(4, np.uint32)
    _L().synth_philox4x32_10(_p(c), _p(k), _p(out))
    return out


def quantile_table() -> np.ndarray:
    ptr = _L().synth_quantile_table()
    return np.ctypeslib.as_array(ptr, shape=(65536,)).copy()


def normal_bf16(seed: int, sid: int, shape, mean: float = 0.0, std: float = 1.0) -> np.ndarray:
    """BF16 bit patterns (uint16) of mean + std * N(0,1)."""
    n = int(np.prod(shape))
    out = np.empty(n, np.uint16)
    _L().synth_normal_bf16(seed, sid, 0, n, mean, std, _p(out))
    return out.reshape(shape)


def normal_f32(seed: int, sid: int, shape, std: float = 1.0, bias: np.ndarray | None = None) -> np.ndarray:
    n = int(np.prod(shape))
    out = np.empty(n, np.float32)
    if bias is not None:
        bias = np.ascontiguousarray(bias, np.float32)
        _L().synth_normal_f32(seed, sid, 0, n, std, _p(bias), bias.size, _p(out))
    else:
        _L().synth_normal_f32(seed, sid, 0, n, std, None, 1, _p(out))
    return out.reshape(shape)


def zipf_bias(seed: int, sid: int, E: int, s: float):
    """(rank[E], bias[E]) with bias = -s * ln(rank) for a seeded expert ranking."""
    rank = np.zeros(E, np.int32)
    bias = np.zeros(E, np.float32)
    _L().synth_zipf_bias(seed, sid, E, s, _p(rank), _p(bias))
    return rank, bias


def qweights(seed: int, sid: int, fmt: int, E: int, N: int, K: int,
             e0: int = 0, e1: int | None = None, std: float = 0.02):
    """Encoded expert weights for experts [e0, e1): (packed u8 [n,N,K/2], scales)."""
    e1 = E if e1 is None else e1
    ne = e1 - e0
    packed = np.empty((ne, N, K // 2), np.uint8)
    scales = np.empty((ne, N, K // 32), np.uint8 if fmt == FMT_MXFP4 else np.uint16)
    rc = _L().synth_qweights(seed, sid, fmt, E, N, K, e0, e1, std, _p(packed), _p(scales))
    if rc:
        raise ValueError(f"synth_qweights failed ({rc})")
    return packed, scales


def weights_f32(seed: int, sid: int, K: int, row0: int, nrows: int, std: float = 0.02) -> np.ndarray:
    """fp32 weights of rows [row0, row0+nrows) of the flattened [E*N][K] tensor."""
    out = np.empty((nrows, K), np.float32)
    _L().synth_weights_f32(seed, sid, K, row0, nrows, std, _p(out))
    return out


def encode_mxfp4_group(w32: np.ndarray):
    w = np.ascontiguousarray(w32, np.float32)
    assert w.size == 32
    nib = np.zeros(16, np.uint8)
    sc = _L().synth_encode_mxfp4_group(_p(w), _p(nib))
    return nib, int(sc)


def encode_int4_group(w32: np.ndarray):
    w = np.ascontiguousarray(w32, np.float32)
    assert w.size == 32
    nib = np.zeros(16, np.uint8)
    sc = _L().synth_encode_int4_group(_p(w), _p(nib))
    return nib, int(sc)


def num_threads() -> int:
    return int(_L().synth_num_threads())
