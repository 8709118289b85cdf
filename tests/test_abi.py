"""Host-side checks of the C-ABI library (no GPU needed).

The library loads, exports every function ``include/qgg.h`` declares, sizes
workspaces by the documented formulas, and rejects bad arguments on the host
before any HIP call.
"""
import ctypes
import os
import re

import pytest

import quantized_grouped_gemm_amd as qgg

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _lib_or_skip():
    if not os.path.exists(qgg.LIB_PATH):
        pytest.skip("libqgg.so not built")
    return qgg.lib()


def _header_functions():
    src = open(os.path.join(ROOT, "include", "qgg.h")).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:qgg_status|size_t|int|const char\*)\s+(\w+)\s*\(", src,
                                 flags=re.M)))


def test_header_declares_the_five_calls():
    fns = _header_functions()
    for f in ("moe_route", "expert_permute", "dequant_grouped_gemm", "moe_ffn_fwd", "moe_dx_bwd"):
        assert f in fns
    assert sorted(qgg.EXPORTS) == fns


def test_library_exports_every_declared_symbol():
    L = _lib_or_skip()
    for f in _header_functions():
        assert hasattr(L, f), f
    assert L.qgg_version().decode().startswith("qgg")
    assert L.qgg_status_string(3).decode() == "workspace too small"


def test_workspace_formulas():
    _lib_or_skip()
    T, d, E, k, N = 4096, 7168, 384, 8, 4096
    tot_f, scr_f = qgg.workspace_bytes(qgg.CALL_GEMM, T, d, E, k, N, qgg.FUSED, 32)
    tot_c, scr_c = qgg.workspace_bytes(qgg.CALL_GEMM, T, d, E, k, N, qgg.CHUNKED, 32)
    assert scr_f == 0
    assert scr_c == 32 * N * d * 2 == 1879048192
    assert tot_c >= scr_c and tot_f < 1 << 20
    # FFN: scratch holds one chunk of the larger projection (gate_up, 2I x d)
    _, s8 = qgg.workspace_bytes(qgg.CALL_FFN_FWD, 64, 7168, 384, 8, 2048, qgg.CHUNKED, 8)
    assert s8 == 8 * 4096 * 7168 * 2 == 448 * 2 ** 20
    # all-active chunk: bounded by min(E, T*k) experts
    _, sa = qgg.workspace_bytes(qgg.CALL_FFN_FWD, 64, 7168, 384, 8, 2048, qgg.CHUNKED, 0)
    assert sa == 384 * 4096 * 7168 * 2
    _, sa = qgg.workspace_bytes(qgg.CALL_FFN_FWD, 2, 7168, 384, 2, 2048, qgg.CHUNKED, 0)
    assert sa == 4 * 4096 * 7168 * 2
    # bad dims -> 0
    assert qgg.workspace_bytes(qgg.CALL_GEMM, 4, 256, 8, 9, 512, qgg.FUSED, 0)[0] == 0
    assert qgg.workspace_bytes(99, 4, 256, 8, 2, 512, qgg.FUSED, 0)[0] == 0


def test_host_side_argument_errors():
    L = _lib_or_skip()
    fake = ctypes.c_void_p(0x1000)  # never dereferenced: validation fails first
    # k > E, k = 0, E > 1024
    assert L.moe_route(fake, 4, 8, 9, fake, fake, None, None) == 1
    assert L.moe_route(fake, 4, 8, 0, fake, fake, None, None) == 1
    assert L.moe_route(fake, 4, 2048, 2, fake, fake, None, None) == 1
    assert L.moe_route(None, 4, 8, 2, fake, fake, None, None) == 1
    # permute: missing arrays, then too-small workspace
    p = qgg._Perm(0x1000, 0x1000, 0x1000, 0x1000, 0x1000, 0)
    assert L.expert_permute(fake, 4, 2, 8, ctypes.byref(p), None, 0, None, None, fake, 1 << 20,
                            None) == 1
    p = qgg._Perm(*([0x1000] * 6))
    assert L.expert_permute(fake, 4, 2, 8, ctypes.byref(p), None, 0, None, None, fake, 4,
                            None) == 3
    # gemm: K not a multiple of 128 -> unsupported; bad format; bad flags
    w = qgg._QWeight(1, 8, 512, 96, 0x1000, 0x1000)
    assert L.dequant_grouped_gemm(ctypes.byref(w), fake, 1, ctypes.byref(p), 4, 2, 1, 0, fake,
                                  1 << 20, fake, None) == 2
    w = qgg._QWeight(7, 8, 512, 256, 0x1000, 0x1000)
    assert L.dequant_grouped_gemm(ctypes.byref(w), fake, 1, ctypes.byref(p), 4, 2, 1, 0, fake,
                                  1 << 20, fake, None) == 1
    w = qgg._QWeight(1, 8, 512, 256, 0x1000, 0x1000)
    assert L.dequant_grouped_gemm(ctypes.byref(w), fake, 64, ctypes.byref(p), 4, 2, 1, 0, fake,
                                  1 << 20, fake, None) == 1
    # dequant-only is a chunked-variant hook
    assert L.dequant_grouped_gemm(ctypes.byref(w), fake, 4, ctypes.byref(p), 4, 2, 1, 0, fake,
                                  1 << 20, fake, None) == 1
    assert L.dequant_grouped_gemm(ctypes.byref(w), fake, 1, ctypes.byref(p), 4, 2, 1, 0, fake,
                                  16, fake, None) == 3
    # ffn: gate_up / down shapes must agree with d, inter, E
    gu = qgg._QWeight(1, 8, 512, 256, 0x1000, 0x1000)
    dn = qgg._QWeight(1, 8, 256, 128, 0x1000, 0x1000)   # inter would be 256 -> K mismatch
    assert L.moe_ffn_fwd(ctypes.byref(gu), ctypes.byref(dn), fake, fake, 4, 256, 8, 2, 256, 1, 0,
                         fake, fake, ctypes.byref(p), None, None, fake, 1 << 30, fake, None) == 1
    dn = qgg._QWeight(2, 8, 256, 256, 0x1000, 0x1000)   # format mismatch
    assert L.moe_ffn_fwd(ctypes.byref(gu), ctypes.byref(dn), fake, fake, 4, 256, 8, 2, 256, 1, 0,
                         fake, fake, ctypes.byref(p), None, None, fake, 1 << 30, fake, None) == 1
    dn = qgg._QWeight(1, 8, 256, 256, 0x1000, 0x1000)
    assert L.moe_dx_bwd(ctypes.byref(gu), ctypes.byref(dn), fake, fake, ctypes.byref(p), None, 4,
                        256, 8, 2, 256, 1, 0, fake, 1 << 30, fake, None) == 1
    assert L.moe_dx_bwd(ctypes.byref(gu), ctypes.byref(dn), fake, fake, ctypes.byref(p), fake, 4,
                        256, 8, 2, 256, 1, 0, fake, 16, fake, None) == 3


def test_host_side_errors_router_and_adapter():
    L = _lib_or_skip()
    fake = ctypes.c_void_p(0x1000)
    p = qgg._Perm(*([0x1000] * 6))
    gu = qgg._QWeight(1, 8, 512, 256, 0x1000, 0x1000)
    dn = qgg._QWeight(1, 8, 256, 256, 0x1000, 0x1000)
    # router backward: needs an output, ids for dlogits, and a big enough workspace
    assert L.moe_router_bwd(ctypes.byref(gu), ctypes.byref(dn), fake, fake, fake, ctypes.byref(p),
                            fake, 4, 256, 8, 2, 256, 1, 0, fake, 1 << 30, fake, None, None,
                            None) == 1
    assert L.moe_router_bwd(ctypes.byref(gu), ctypes.byref(dn), fake, None, fake, ctypes.byref(p),
                            fake, 4, 256, 8, 2, 256, 1, 0, fake, 1 << 30, None, None, fake,
                            None) == 1
    assert L.moe_router_bwd(ctypes.byref(gu), ctypes.byref(dn), fake, fake, fake, ctypes.byref(p),
                            fake, 4, 256, 8, 2, 256, 1, 0, fake, 16, None, fake, fake, None) == 3
    # adapter forward: rank limits, alpha, flags, workspace
    w = qgg._QWeight(2, 8, 512, 256, 0x1000, 0x1000)
    for rank, alpha, flags, want in ((8, 1.0, 1, 2), (24, 1.0, 1, 2), (160, 1.0, 1, 2),
                                     (32, float("nan"), 1, 1), (32, 1.0, 3, 1), (32, 1.0, 5, 1)):
        lo = qgg._Lora(rank, alpha, 0x1000, 0x1000)
        assert L.lora_grouped_gemm(ctypes.byref(w), ctypes.byref(lo), fake, flags,
                                   ctypes.byref(p), 4, 2, 1, 0, fake, 1 << 20, fake, fake,
                                   None) == want, (rank, alpha, flags)
    lo = qgg._Lora(32, 1.0, 0x1000, 0x1000)
    assert L.lora_grouped_gemm(ctypes.byref(w), ctypes.byref(lo), fake, 1, ctypes.byref(p), 4, 2,
                               1, 0, fake, 1 << 20, None, fake, None) == 1
    assert L.lora_grouped_gemm(ctypes.byref(w), ctypes.byref(lo), fake, 1, ctypes.byref(p), 4, 2,
                               1, 0, fake, 16, fake, fake, None) == 3
    # adapter backward: rank, at least one output, u for dB, workspace
    assert L.lora_grouped_gemm_bwd(ctypes.byref(qgg._Lora(40, 1.0, 0x1000, 0x1000)), 8, 512, 256,
                                   fake, 1, fake, fake, ctypes.byref(p), 4, 2, fake, 1 << 30,
                                   fake, None, None, None) == 2
    assert L.lora_grouped_gemm_bwd(ctypes.byref(lo), 8, 512, 256, fake, 1, fake, fake,
                                   ctypes.byref(p), 4, 2, fake, 1 << 30, None, None, None,
                                   None) == 1
    assert L.lora_grouped_gemm_bwd(ctypes.byref(lo), 8, 512, 256, fake, 1, fake, None,
                                   ctypes.byref(p), 4, 2, fake, 1 << 30, None, None, fake,
                                   None) == 1
    assert L.lora_grouped_gemm_bwd(ctypes.byref(lo), 8, 512, 256, fake, 1, fake, fake,
                                   ctypes.byref(p), 4, 2, fake, 16, fake, fake, fake, None) == 3


def test_workspace_formulas_backward():
    _lib_or_skip()
    T, d, E, k, I = 8192, 7168, 256, 8, 2048
    P = T * k
    # the router partials (P x I/256 fp32) sit after the backward's other buffers
    fused, _ = qgg.workspace_bytes(qgg.CALL_DX_BWD, T, d, E, k, I, qgg.FUSED, 0)
    assert fused >= P * 2 * I * 2 + P * d * 2 + P * (I // 256) * 4
    # adapter backward: du (P x rank fp32) and B transposed (E x rank x N BF16)
    N, rank = 4096, 32
    lb, _ = qgg.workspace_bytes(qgg.CALL_LORA_BWD, 4096, N, 384, 8, rank, qgg.FUSED, 0)
    assert lb >= 4096 * 8 * rank * 4 + 384 * rank * N * 2


def test_workspace_formula_ffn_adapter_backward():
    _lib_or_skip()
    T, d, E, k, I = 64, 7168, 384, 8, 2048
    P = T * k
    base, _ = qgg.workspace_bytes(qgg.CALL_DX_BWD, T, d, E, k, I, qgg.FUSED, 0)
    lb, _ = qgg.workspace_bytes(qgg.CALL_FFN_LORA_BWD, T, d, E, k, I, qgg.FUSED, 0)
    # + a and the down share [P][I], the gate_up share [P][d], du and us
    # [P][128] fp32, B transposed [E][128][max(d, 2I)] BF16
    assert lb >= base + 2 * P * I * 2 + P * d * 2 + 2 * P * 128 * 4 + E * 128 * max(d, 2 * I) * 2
    _, s8 = qgg.workspace_bytes(qgg.CALL_FFN_LORA_BWD, T, d, E, k, I, qgg.CHUNKED, 8)
    assert s8 == 8 * 2 * I * d * 2


def test_missing_library_raises(monkeypatch, tmp_path):
    monkeypatch.setattr(qgg, "LIB_PATH", str(tmp_path / "nope.so"))
    monkeypatch.setattr(qgg, "_lib", None)
    with pytest.raises(qgg.QggError):
        qgg.lib()
