"""Python binding of ``libqgg.so``, the gfx950 quantized MoE grouped-GEMM library.

Argument marshalling only: every step of the path runs in the library's HIP
kernels, which this module reaches through ctypes with raw device pointers and
the current HIP stream.  PyTorch supplies device memory and streams.  If the
library is not built, every call raises; there is no fallback.

Names follow the C-ABI in ``include/qgg.h``: ``moe_route``, ``expert_permute``,
``dequant_grouped_gemm``, ``lora_grouped_gemm``, ``moe_ffn_fwd``, ``moe_dx_bwd``,
``moe_router_bwd``.
"""
from __future__ import annotations

import ctypes
import os
from dataclasses import dataclass

from . import accounting  # noqa: F401  (host-side byte/FLOP accounting)

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libqgg.so")

FMT_MXFP4 = 1
FMT_INT4 = 2
LAYOUT_ROWS = 0
LAYOUT_MFMA = 1
CHUNKED = 0
FUSED = 1
A_SORTED = 0
A_TOKENS = 1
TRANSPOSE_W = 2
DEQUANT_ONLY = 4
CALL_PERMUTE = 1
CALL_GEMM = 2
CALL_FFN_FWD = 3
CALL_DX_BWD = 4
CALL_LORA_BWD = 5
CALL_FFN_LORA_BWD = 6

STATUS = {0: "ok", 1: "invalid argument", 2: "unsupported", 3: "workspace too small", 4: "HIP error"}

# Every symbol include/qgg.h declares.
EXPORTS = ("moe_route", "expert_permute", "dequant_grouped_gemm", "lora_grouped_gemm",
           "lora_grouped_gemm_bwd", "moe_ffn_fwd", "moe_ffn_fwd_noalloc", "moe_ffn_fwd_lora",
           "moe_dx_bwd", "moe_ffn_bwd_lora",
           "moe_router_bwd", "qgg_repack_weights", "qgg_check_weights", "qgg_workspace_bytes",
           "qgg_set_timing_events", "qgg_timing_count", "qgg_timing_kind", "qgg_status_string",
           "qgg_version")

_lib = None


class QggError(RuntimeError):
    pass


class _QWeight(ctypes.Structure):
    _fields_ = [("fmt", ctypes.c_int32), ("E", ctypes.c_int32), ("N", ctypes.c_int32),
                ("K", ctypes.c_int32), ("packed", ctypes.c_void_p), ("scales", ctypes.c_void_p),
                ("layout", ctypes.c_int32)]


class _Lora(ctypes.Structure):
    _fields_ = [("rank", ctypes.c_int32), ("alpha", ctypes.c_float), ("A", ctypes.c_void_p),
                ("B", ctypes.c_void_p)]


class _Perm(ctypes.Structure):
    _fields_ = [(n, ctypes.c_void_p) for n in
                ("counts", "offsets", "perm", "inv_perm", "active", "n_active")]


def lib():
    """The loaded library; raises if it has not been built."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise QggError(f"{LIB_PATH} is missing: build it with "
                           "`python -m quantized_grouped_gemm_amd.build`")
        L = ctypes.CDLL(LIB_PATH)
        P, i32, sz = ctypes.c_void_p, ctypes.c_int, ctypes.c_size_t
        L.moe_route.argtypes = [P, i32, i32, i32, P, P, P, P]
        L.expert_permute.argtypes = [P, i32, i32, i32, ctypes.POINTER(_Perm), P, i32, P, P, P, sz, P]
        L.dequant_grouped_gemm.argtypes = [ctypes.POINTER(_QWeight), P, i32, ctypes.POINTER(_Perm),
                                           i32, i32, i32, i32, P, sz, P, P]
        L.lora_grouped_gemm.argtypes = [ctypes.POINTER(_QWeight), ctypes.POINTER(_Lora), P, i32,
                                        ctypes.POINTER(_Perm), i32, i32, i32, i32, P, sz, P, P, P]
        L.lora_grouped_gemm_bwd.argtypes = [ctypes.POINTER(_Lora), i32, i32, i32, P, i32, P, P,
                                            ctypes.POINTER(_Perm), i32, i32, P, sz, P, P, P, P]
        L.moe_ffn_fwd.argtypes = [ctypes.POINTER(_QWeight), ctypes.POINTER(_QWeight), P, P, i32,
                                  i32, i32, i32, i32, i32, i32, P, P, ctypes.POINTER(_Perm), P, P,
                                  P, sz, P, P]
        L.moe_ffn_fwd_noalloc.argtypes = [ctypes.POINTER(_QWeight), ctypes.POINTER(_QWeight), P,
                                          P, i32, i32, i32, i32, i32, i32, i32, P, P,
                                          ctypes.POINTER(_Perm), P, P, P, P]
        L.moe_ffn_fwd_lora.argtypes = [ctypes.POINTER(_QWeight), ctypes.POINTER(_QWeight),
                                       ctypes.POINTER(_Lora), ctypes.POINTER(_Lora), P, P, i32,
                                       i32, i32, i32, i32, i32, i32, P, P, ctypes.POINTER(_Perm),
                                       P, P, P, P, P, sz, P, P]
        L.moe_dx_bwd.argtypes = [ctypes.POINTER(_QWeight), ctypes.POINTER(_QWeight), P, P,
                                 ctypes.POINTER(_Perm), P, i32, i32, i32, i32, i32, i32, i32, P,
                                 sz, P, P]
        L.moe_ffn_bwd_lora.argtypes = [ctypes.POINTER(_QWeight), ctypes.POINTER(_QWeight),
                                       ctypes.POINTER(_Lora), ctypes.POINTER(_Lora), P, P, P,
                                       ctypes.POINTER(_Perm), P, P, P, i32, i32, i32, i32, i32,
                                       i32, i32, P, sz, P, P, P, P, P, P]
        L.moe_router_bwd.argtypes = [ctypes.POINTER(_QWeight), ctypes.POINTER(_QWeight), P, P, P,
                                     ctypes.POINTER(_Perm), P, i32, i32, i32, i32, i32, i32, i32,
                                     P, sz, P, P, P, P]
        L.qgg_repack_weights.argtypes = [ctypes.POINTER(_QWeight), P, P, P]
        L.qgg_repack_weights.restype = ctypes.c_int
        L.qgg_check_weights.argtypes = [ctypes.POINTER(_QWeight), P, P]
        L.qgg_check_weights.restype = ctypes.c_int
        L.qgg_workspace_bytes.argtypes = [i32, i32, i32, i32, i32, i32, i32, i32,
                                          ctypes.POINTER(ctypes.c_size_t)]
        L.qgg_workspace_bytes.restype = ctypes.c_size_t
        L.qgg_set_timing_events.argtypes = [P, i32]
        L.qgg_set_timing_events.restype = ctypes.c_int
        L.qgg_timing_count.restype = ctypes.c_int
        L.qgg_timing_kind.argtypes = [i32]
        L.qgg_timing_kind.restype = ctypes.c_int
        L.qgg_status_string.argtypes = [i32]
        L.qgg_status_string.restype = ctypes.c_char_p
        L.qgg_version.restype = ctypes.c_char_p
        for f in ("moe_route", "expert_permute", "dequant_grouped_gemm", "lora_grouped_gemm",
                  "lora_grouped_gemm_bwd", "moe_ffn_fwd", "moe_ffn_fwd_noalloc",
                  "moe_ffn_fwd_lora", "moe_dx_bwd", "moe_ffn_bwd_lora", "moe_router_bwd"):
            getattr(L, f).restype = ctypes.c_int
        _lib = L
    return _lib


def _check(rc: int, what: str):
    if rc != 0:
        raise QggError(f"{what}: {lib().qgg_status_string(rc).decode()} ({rc})")


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream():
    import torch
    return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)


@dataclass
class QWeight:
    """Frozen 4-bit expert weights on the device: packed bytes and scales
    (uint8 E8M0 for MXFP4, BF16 bits for INT4) of E experts of [N][K], in
    LAYOUT_ROWS ([E][N][K/2], [E][N][K/32]) or LAYOUT_MFMA order (same sizes,
    see include/qgg.h).  Shapes are given by E, N, K."""
    fmt: int
    packed: "object"
    scales: "object"
    layout: int = LAYOUT_ROWS
    shape: tuple = None

    def __post_init__(self):
        if self.shape is None:
            self.shape = (self.packed.shape[0], self.packed.shape[1], self.packed.shape[2] * 2)

    @property
    def E(self):
        return self.shape[0]

    @property
    def N(self):
        return self.shape[1]

    @property
    def K(self):
        return self.shape[2]

    def c(self):
        return _QWeight(self.fmt, self.E, self.N, self.K, self.packed.data_ptr(),
                        self.scales.data_ptr(), self.layout)


def repack(w: "QWeight") -> "QWeight":
    """The MFMA-tiled copy of row-layout weights (qgg_repack_weights)."""
    import torch
    assert w.layout == LAYOUT_ROWS
    p = torch.empty_like(w.packed)
    s = torch.empty_like(w.scales)
    wc = w.c()
    _check(lib().qgg_repack_weights(ctypes.byref(wc), _ptr(p), _ptr(s), _stream()),
           "qgg_repack_weights")
    return QWeight(w.fmt, p, s, LAYOUT_MFMA, w.shape)


def check_weights(w: "QWeight", err_flag=None):
    """qgg_check_weights: bit 4 of the returned device int32 flag is set when a
    scale of ``w`` lies outside the fused decoder's exact domain (``err_flag``,
    if given, is that device tensor, zeroed by the caller)."""
    import torch
    if err_flag is None:
        err_flag = torch.zeros(1, dtype=torch.int32, device=w.packed.device)
    wc = w.c()
    _check(lib().qgg_check_weights(ctypes.byref(wc), _ptr(err_flag), _stream()),
           "qgg_check_weights")
    return err_flag


_timing_keep = None


def set_timing_events(events, capacity: int):
    """qgg_set_timing_events with a list of 2*capacity recorded-once
    torch.cuda.Event(enable_timing=True) objects (None stops)."""
    global _timing_keep
    if events is None:
        _timing_keep = None
        _check(lib().qgg_set_timing_events(None, 0), "qgg_set_timing_events")
        return
    arr = (ctypes.c_void_p * len(events))(*[e.cuda_event for e in events])
    _timing_keep = arr
    _check(lib().qgg_set_timing_events(ctypes.cast(arr, ctypes.c_void_p), capacity),
           "qgg_set_timing_events")


def timing_count() -> int:
    return int(lib().qgg_timing_count())


def timing_kinds(n: int):
    return [int(lib().qgg_timing_kind(i)) for i in range(n)]


@dataclass
class Perm:
    """Routing permutation (device int32 tensors), see ``qgg_perm``."""
    counts: "object"
    offsets: "object"
    perm: "object"
    inv_perm: "object"
    active: "object"
    n_active: "object"

    @staticmethod
    def empty(P: int, E: int, device):
        import torch
        z = lambda n: torch.empty(max(n, 1), dtype=torch.int32, device=device)  # noqa: E731
        return Perm(z(E), z(E + 1), z(P), z(P), z(E), z(1))

    def c(self):
        return _Perm(*(t.data_ptr() for t in (self.counts, self.offsets, self.perm,
                                               self.inv_perm, self.active, self.n_active)))


def workspace_bytes(call: int, T: int, d: int, E: int, k: int, n_or_inter: int, variant: int,
                    chunk: int):
    """(total workspace bytes, dequant scratch bytes) for a call."""
    s = ctypes.c_size_t(0)
    total = lib().qgg_workspace_bytes(call, T, d, E, k, n_or_inter, variant, chunk,
                                      ctypes.byref(s))
    return int(total), int(s.value)


class Workspace:
    """A reusable device byte buffer that grows on demand.

    Calls run in stream order on the current stream, so one workspace serves any
    number of calls issued on that stream; calls that may run concurrently on
    different streams each need their own (the module default is shared)."""

    def __init__(self):
        self.buf = None

    def get(self, nbytes: int, device):
        import torch
        if self.buf is None or self.buf.numel() < nbytes or self.buf.device != device:
            self.buf = None
            self.buf = torch.empty(max(nbytes, 256), dtype=torch.uint8, device=device)
        return self.buf


_default_ws = Workspace()


def moe_route(logits, k: int, err_flag=None):
    """(topk_ids int32 [T,k], topk_gates fp32 [T,k]) for fp32 logits [T,E]."""
    import torch
    T, E = logits.shape
    ids = torch.empty((T, k), dtype=torch.int32, device=logits.device)
    gates = torch.empty((T, k), dtype=torch.float32, device=logits.device)
    _check(lib().moe_route(_ptr(logits), T, E, k, _ptr(ids), _ptr(gates), _ptr(err_flag),
                           _stream()), "moe_route")
    return ids, gates


def expert_permute(topk_ids, E: int, x=None, err_flag=None, ws: Workspace | None = None):
    """Perm for int32 ids [T,k]; with x [T,d] BF16 also returns x_perm [P,d]."""
    import torch
    T, k = topk_ids.shape
    dev = topk_ids.device
    p = Perm.empty(T * k, E, dev)
    x_perm = None
    d = 0
    if x is not None:
        d = x.shape[1]
        x_perm = torch.empty((T * k, d), dtype=x.dtype, device=dev)
    nb, _ = workspace_bytes(CALL_PERMUTE, T, 128, E, k, 64, FUSED, 0)
    buf = (ws or _default_ws).get(nb, dev)
    pc = p.c()
    _check(lib().expert_permute(_ptr(topk_ids), T, k, E, ctypes.byref(pc), _ptr(x), d,
                                _ptr(x_perm), _ptr(err_flag), _ptr(buf), buf.numel(), _stream()),
           "expert_permute")
    return p, x_perm


def dequant_grouped_gemm(w: QWeight, a, perm: Perm, T: int, k: int, variant: int = FUSED,
                         chunk: int = 0, flags: int = A_TOKENS, ws: Workspace | None = None,
                         out=None):
    """y [P, N] (or [P, K] with TRANSPOSE_W) in sorted order, BF16."""
    import torch
    dev = w.packed.device
    P = T * k
    trans = bool(flags & TRANSPOSE_W)
    ncols = w.K if trans else w.N
    if flags & DEQUANT_ONLY:
        y = None
    else:
        y = out if out is not None else torch.empty((P, ncols), dtype=torch.bfloat16, device=dev)
    nb, _ = workspace_bytes(CALL_GEMM, T, w.K, w.E, k, w.N, variant, chunk)
    buf = (ws or _default_ws).get(nb, dev)
    wc, pc = w.c(), perm.c()
    _check(lib().dequant_grouped_gemm(ctypes.byref(wc), _ptr(a), flags, ctypes.byref(pc), T, k,
                                      variant, chunk, _ptr(buf), buf.numel(), _ptr(y), _stream()),
           "dequant_grouped_gemm")
    return y if y is not None else buf


def lora_grouped_gemm(w: QWeight, A, B, alpha: float, a, perm: Perm, T: int, k: int,
                      variant: int = FUSED, chunk: int = 0, flags: int = A_TOKENS,
                      ws: Workspace | None = None):
    """(y [P, N], u [P, rank]) BF16 in sorted order: the projection with a LoRA adapter,
    A [E, rank, K] and B [E, N, rank] BF16 device tensors."""
    import torch
    dev = w.packed.device
    P = T * k
    rank = A.shape[1]
    y = torch.empty((P, w.N), dtype=torch.bfloat16, device=dev)
    u = torch.empty((P, rank), dtype=torch.bfloat16, device=dev)
    nb, _ = workspace_bytes(CALL_GEMM, T, w.K, w.E, k, w.N, variant, chunk)
    buf = (ws or _default_ws).get(nb, dev)
    wc, pc = w.c(), perm.c()
    lc = _Lora(rank, float(alpha), A.data_ptr(), B.data_ptr())
    _check(lib().lora_grouped_gemm(ctypes.byref(wc), ctypes.byref(lc), _ptr(a), flags,
                                   ctypes.byref(pc), T, k, variant, chunk, _ptr(buf), buf.numel(),
                                   _ptr(u), _ptr(y), _stream()), "lora_grouped_gemm")
    return y, u


def lora_grouped_gemm_bwd(A, B, alpha: float, a, dy, u, perm: Perm, T: int, k: int,
                          flags: int = A_TOKENS, want=("dx", "dA", "dB"),
                          ws: Workspace | None = None):
    """{"dx": [P, K] BF16, "dA": [E, rank, K] fp32, "dB": [E, N, rank] fp32} (those in
    `want`): the adapter's backward for the upstream gradient dy [P, N] (sorted)."""
    import torch
    E, rank, K = A.shape
    N = B.shape[1]
    dev = dy.device
    P = T * k
    dx = torch.empty((P, K), dtype=torch.bfloat16, device=dev) if "dx" in want else None
    dA = torch.empty((E, rank, K), dtype=torch.float32, device=dev) if "dA" in want else None
    dB = torch.empty((E, N, rank), dtype=torch.float32, device=dev) if "dB" in want else None
    nb, _ = workspace_bytes(CALL_LORA_BWD, T, N, E, k, rank, FUSED, 0)
    buf = (ws or _default_ws).get(nb, dev)
    pc = perm.c()
    lc = _Lora(rank, float(alpha), A.data_ptr(), B.data_ptr())
    _check(lib().lora_grouped_gemm_bwd(ctypes.byref(lc), E, N, K, _ptr(a), flags, _ptr(dy),
                                       _ptr(u), ctypes.byref(pc), T, k, _ptr(buf), buf.numel(),
                                       _ptr(dx), _ptr(dA), _ptr(dB), _stream()),
           "lora_grouped_gemm_bwd")
    return {"dx": dx, "dA": dA, "dB": dB}


def moe_ffn_fwd(w_gate_up: QWeight, w_down: QWeight, x, logits, k: int, variant: int = FUSED,
                chunk: int = 0, save_h: bool = False, err_flag=None, ws: Workspace | None = None):
    """dict(y [T,d], topk_ids, topk_gates, perm, h [P,2I] or None)."""
    import torch
    T, d = x.shape
    E = w_gate_up.E
    inter = w_gate_up.N // 2
    dev = x.device
    P = T * k
    ids = torch.empty((T, k), dtype=torch.int32, device=dev)
    gates = torch.empty((T, k), dtype=torch.float32, device=dev)
    p = Perm.empty(P, E, dev)
    h = torch.empty((P, 2 * inter), dtype=torch.bfloat16, device=dev) if save_h else None
    y = torch.empty((T, d), dtype=torch.bfloat16, device=dev)
    nb, _ = workspace_bytes(CALL_FFN_FWD, T, d, E, k, inter, variant, chunk)
    buf = (ws or _default_ws).get(nb, dev)
    g, dn, pc = w_gate_up.c(), w_down.c(), p.c()
    _check(lib().moe_ffn_fwd(ctypes.byref(g), ctypes.byref(dn), _ptr(x), _ptr(logits), T, d, E, k,
                             inter, variant, chunk, _ptr(ids), _ptr(gates), ctypes.byref(pc),
                             _ptr(h), _ptr(err_flag), _ptr(buf), buf.numel(), _ptr(y), _stream()),
           "moe_ffn_fwd")
    return dict(y=y, topk_ids=ids, topk_gates=gates, perm=p, h=h)


STATIC_SCRATCH_BYTES = 32 << 20


def moe_ffn_fwd_noalloc(w_gate_up: QWeight, w_down: QWeight, x, logits, k: int,
                        variant: int = FUSED, chunk: int = 0, save_h: bool = False,
                        err_flag=None):
    """moe_ffn_fwd on the library's static scratch (no workspace); same result dict."""
    import torch
    T, d = x.shape
    E = w_gate_up.E
    inter = w_gate_up.N // 2
    dev = x.device
    P = T * k
    ids = torch.empty((T, k), dtype=torch.int32, device=dev)
    gates = torch.empty((T, k), dtype=torch.float32, device=dev)
    p = Perm.empty(P, E, dev)
    h = torch.empty((P, 2 * inter), dtype=torch.bfloat16, device=dev) if save_h else None
    y = torch.empty((T, d), dtype=torch.bfloat16, device=dev)
    g, dn, pc = w_gate_up.c(), w_down.c(), p.c()
    _check(lib().moe_ffn_fwd_noalloc(ctypes.byref(g), ctypes.byref(dn), _ptr(x), _ptr(logits), T,
                                     d, E, k, inter, variant, chunk, _ptr(ids), _ptr(gates),
                                     ctypes.byref(pc), _ptr(h), _ptr(err_flag), _ptr(y),
                                     _stream()), "moe_ffn_fwd_noalloc")
    return dict(y=y, topk_ids=ids, topk_gates=gates, perm=p, h=h)


def moe_ffn_fwd_lora(w_gate_up: QWeight, w_down: QWeight, lora_gate_up, lora_down, x, logits,
                     k: int, variant: int = FUSED, chunk: int = 0, save_h: bool = False,
                     err_flag=None, ws: Workspace | None = None):
    """moe_ffn_fwd with BF16 LoRA adapters: lora_gate_up / lora_down are (A, B, alpha)
    tuples of device tensors (A [E, r, K], B [E, N, r]) or None.  Adds u_gate_up /
    u_down [P, r] (sorted order) to the result."""
    import torch
    T, d = x.shape
    E = w_gate_up.E
    inter = w_gate_up.N // 2
    dev = x.device
    P = T * k
    ids = torch.empty((T, k), dtype=torch.int32, device=dev)
    gates = torch.empty((T, k), dtype=torch.float32, device=dev)
    p = Perm.empty(P, E, dev)
    h = torch.empty((P, 2 * inter), dtype=torch.bfloat16, device=dev) if save_h else None
    y = torch.empty((T, d), dtype=torch.bfloat16, device=dev)

    def adapter(l):
        if l is None:
            return None, None
        A, B, alpha = l
        u = torch.empty((P, A.shape[1]), dtype=torch.bfloat16, device=dev)
        return _Lora(A.shape[1], float(alpha), A.data_ptr(), B.data_ptr()), u

    lgu, ugu = adapter(lora_gate_up)
    ldn, udn = adapter(lora_down)
    nb, _ = workspace_bytes(CALL_FFN_FWD, T, d, E, k, inter, variant, chunk)
    buf = (ws or _default_ws).get(nb, dev)
    g, dn, pc = w_gate_up.c(), w_down.c(), p.c()
    _check(lib().moe_ffn_fwd_lora(ctypes.byref(g), ctypes.byref(dn),
                                  ctypes.byref(lgu) if lgu else None,
                                  ctypes.byref(ldn) if ldn else None, _ptr(x), _ptr(logits), T, d,
                                  E, k, inter, variant, chunk, _ptr(ids), _ptr(gates),
                                  ctypes.byref(pc), _ptr(h), _ptr(ugu), _ptr(udn),
                                  _ptr(err_flag), _ptr(buf), buf.numel(), _ptr(y), _stream()),
           "moe_ffn_fwd_lora")
    return dict(y=y, topk_ids=ids, topk_gates=gates, perm=p, h=h, u_gate_up=ugu, u_down=udn)


def moe_dx_bwd(w_gate_up: QWeight, w_down: QWeight, dy, topk_gates, perm: Perm, h_saved, k: int,
               variant: int = FUSED, chunk: int = 0, ws: Workspace | None = None):
    """dx [T,d] BF16: the input gradient through the frozen base."""
    import torch
    T, d = dy.shape
    E = w_gate_up.E
    inter = w_gate_up.N // 2
    dev = dy.device
    dx = torch.empty((T, d), dtype=torch.bfloat16, device=dev)
    nb, _ = workspace_bytes(CALL_DX_BWD, T, d, E, k, inter, variant, chunk)
    buf = (ws or _default_ws).get(nb, dev)
    g, dn, pc = w_gate_up.c(), w_down.c(), perm.c()
    _check(lib().moe_dx_bwd(ctypes.byref(g), ctypes.byref(dn), _ptr(dy), _ptr(topk_gates),
                            ctypes.byref(pc), _ptr(h_saved), T, d, E, k, inter, variant, chunk,
                            _ptr(buf), buf.numel(), _ptr(dx), _stream()), "moe_dx_bwd")
    return dx


def moe_ffn_bwd_lora(w_gate_up: QWeight, w_down: QWeight, lora_gate_up, lora_down, x, dy,
                     topk_gates, perm: Perm, h_saved, u_gate_up, u_down, k: int,
                     variant: int = FUSED, chunk: int = 0,
                     want=("dx", "dA_gate_up", "dB_gate_up", "dA_down", "dB_down"),
                     ws: Workspace | None = None):
    """Backward of moe_ffn_fwd_lora: {"dx": [T, d] BF16, "dA_gate_up": [E, r, d],
    "dB_gate_up": [E, 2I, r], "dA_down": [E, r, I], "dB_down": [E, d, r]} (fp32;
    those in `want` whose adapter is given, else None).  lora_gate_up /
    lora_down are (A, B, alpha) tuples as for moe_ffn_fwd_lora, or None."""
    import torch
    T, d = dy.shape
    E = w_gate_up.E
    inter = w_gate_up.N // 2
    dev = dy.device

    def grad(name, l, shape_of):
        if l is None or name not in want:
            return None
        return torch.empty(shape_of(l), dtype=torch.float32, device=dev)

    dx = torch.empty((T, d), dtype=torch.bfloat16, device=dev) if "dx" in want else None
    dAg = grad("dA_gate_up", lora_gate_up, lambda l: tuple(l[0].shape))
    dBg = grad("dB_gate_up", lora_gate_up, lambda l: tuple(l[1].shape))
    dAd = grad("dA_down", lora_down, lambda l: tuple(l[0].shape))
    dBd = grad("dB_down", lora_down, lambda l: tuple(l[1].shape))

    def adapter(l):
        if l is None:
            return None
        A, B, alpha = l
        return _Lora(A.shape[1], float(alpha), A.data_ptr(), B.data_ptr())

    lg, ld = adapter(lora_gate_up), adapter(lora_down)
    nb, _ = workspace_bytes(CALL_FFN_LORA_BWD, T, d, E, k, inter, variant, chunk)
    buf = (ws or _default_ws).get(nb, dev)
    g, dn, pc = w_gate_up.c(), w_down.c(), perm.c()
    _check(lib().moe_ffn_bwd_lora(ctypes.byref(g), ctypes.byref(dn),
                                  ctypes.byref(lg) if lg else None,
                                  ctypes.byref(ld) if ld else None, _ptr(x), _ptr(dy),
                                  _ptr(topk_gates), ctypes.byref(pc), _ptr(h_saved),
                                  _ptr(u_gate_up), _ptr(u_down), T, d, E, k, inter, variant,
                                  chunk, _ptr(buf), buf.numel(), _ptr(dx), _ptr(dAg), _ptr(dBg),
                                  _ptr(dAd), _ptr(dBd), _stream()), "moe_ffn_bwd_lora")
    return {"dx": dx, "dA_gate_up": dAg, "dB_gate_up": dBg, "dA_down": dAd, "dB_down": dBd}


def moe_router_bwd(w_gate_up: QWeight, w_down: QWeight, dy, topk_ids, topk_gates, perm: Perm,
                   h_saved, k: int, variant: int = FUSED, chunk: int = 0, want_dx: bool = True,
                   ws: Workspace | None = None):
    """{"dx": [T,d] BF16 or None, "dgates": [T,k] fp32, "dlogits": [T,E] fp32}: the
    router gradient through the frozen base (and the input gradient if want_dx)."""
    import torch
    T, d = dy.shape
    E = w_gate_up.E
    inter = w_gate_up.N // 2
    dev = dy.device
    dx = torch.empty((T, d), dtype=torch.bfloat16, device=dev) if want_dx else None
    dg = torch.empty((T, k), dtype=torch.float32, device=dev)
    dl = torch.empty((T, E), dtype=torch.float32, device=dev)
    nb, _ = workspace_bytes(CALL_DX_BWD, T, d, E, k, inter, variant, chunk)
    buf = (ws or _default_ws).get(nb, dev)
    g, dn, pc = w_gate_up.c(), w_down.c(), perm.c()
    _check(lib().moe_router_bwd(ctypes.byref(g), ctypes.byref(dn), _ptr(dy), _ptr(topk_ids),
                                _ptr(topk_gates), ctypes.byref(pc), _ptr(h_saved), T, d, E, k,
                                inter, variant, chunk, _ptr(buf), buf.numel(), _ptr(dx), _ptr(dg),
                                _ptr(dl), _stream()), "moe_router_bwd")
    return {"dx": dx, "dgates": dg, "dlogits": dl}
