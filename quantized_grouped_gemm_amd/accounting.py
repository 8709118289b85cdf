"""Byte and FLOP accounting for the quantized MoE grouped-GEMM path.

Bytes per stored weight follow the grouped low-bit storage arithmetic on the
page "超大规模开放权重模型技术解析" (section 三, 先算清存储账 and the
estimate_storage helper in 实践提醒): a b-bit body plus one s-bit scale per group
of g elements costs b + s/g bits per weight.  MXFP4 (4-bit E2M1, 8-bit E8M0
scale, g = 32) is 4.25 bits; INT4 with a BF16 scale per 32 is 4.5 bits.
"""
from __future__ import annotations

FMT_MXFP4 = 1
FMT_INT4 = 2

GROUP = 32
SCALE_BITS = {FMT_MXFP4: 8, FMT_INT4: 16}

# MI355X published peaks used for roofline fractions.
HBM_PEAK_GBPS = 8000.0
BF16_DENSE_PEAK_TFLOPS = 2516.6   # 256 CU x 4096 FLOP/clk x 2.4 GHz


def storage_bytes(total_params: float, bits: int = 4, group_size: int = 32, scale_bits: int = 8,
                  sensitive_ratio: float = 0.0, sensitive_bytes: float = 2.0) -> float:
    """Grouped low-bit storage: body + one scale per group (+ a high-precision share)."""
    quantized = total_params * (1.0 - sensitive_ratio)
    body = quantized * bits / 8.0
    scales = quantized / group_size * scale_bits / 8.0
    sensitive = total_params * sensitive_ratio * sensitive_bytes
    return body + scales + sensitive


def bits_per_weight(fmt: int) -> float:
    return 4.0 + SCALE_BITS[fmt] / GROUP


def packed_bytes(fmt: int, N: int, K: int) -> int:
    """Bytes of one expert's packed [N][K] weights plus its scales."""
    return N * K // 2 + N * (K // GROUP) * SCALE_BITS[fmt] // 8


def proj_flops(P: int, N: int, K: int) -> float:
    """2 * P * N * K for P routed rows through an N x K projection."""
    return 2.0 * P * N * K


def proj_alg_bytes(fmt: int, n_active: int, N: int, K: int, T: int, P: int) -> float:
    """Algorithmic HBM bytes of one grouped projection: the active experts'
    packed weights and scales, each token's input row once, each routed output
    row once (BF16)."""
    return n_active * packed_bytes(fmt, N, K) + T * K * 2.0 + P * N * 2.0


def ffn_alg_bytes(fmt: int, n_active: int, d: int, inter: int, T: int, P: int) -> float:
    """Algorithmic bytes of the SwiGLU expert FFN: both projections' active
    weights, x once and y once (intermediates are the method's own traffic)."""
    w = n_active * (packed_bytes(fmt, 2 * inter, d) + packed_bytes(fmt, d, inter))
    return w + T * d * 2.0 + T * d * 2.0


def ffn_flops(P: int, d: int, inter: int) -> float:
    return 2.0 * P * (2 * inter) * d + 2.0 * P * d * inter


def dequant_scratch_bytes(chunk: int, N: int, K: int) -> int:
    """BF16 scratch that holds one chunk of dequantized experts."""
    return chunk * N * K * 2
