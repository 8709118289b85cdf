"""Byte and FLOP accounting for the quantized MoE grouped-GEMM path.

Bits per stored weight follow from the microscaling format itself (page
"超大规模开放权重模型技术解析", section 三, 微缩放量化的原理: a group of g
elements stored with b bits each shares one s-bit scale), so a grouped 4-bit
weight costs b + s/g bits: MXFP4 (E2M1 body, 8-bit E8M0 scale, g = 32) is
4.25 bits, INT4 with a BF16 scale per 32 is 4.5 bits.  The same section's
storage arithmetic (先算清存储账) then keeps a small share of the parameters
in 16-bit precision.
"""
from __future__ import annotations

FMT_MXFP4 = 1
FMT_INT4 = 2

GROUP = 32
SCALE_BITS = {FMT_MXFP4: 8, FMT_INT4: 16}

# MI355X published peaks used for roofline fractions.
HBM_PEAK_GBPS = 8000.0
BF16_DENSE_PEAK_TFLOPS = 2516.6   # 256 CU x 4096 FLOP/clk x 2.4 GHz


def grouped_bits(body_bits: float, group: int, scale_bits: float) -> float:
    """Bits per weight of a group-scaled format: the body plus the group's
    shared scale spread over its elements."""
    return body_bits + scale_bits / group


def storage_bytes(total_params: float, bits_per_weight: float, high_share: float = 0.0,
                  high_bytes: float = 2.0) -> float:
    """Bytes of a checkpoint whose parameters are stored at bits_per_weight,
    except a fraction high_share kept at high_bytes each (FP16: 2)."""
    return total_params * ((1.0 - high_share) * bits_per_weight / 8.0 + high_share * high_bytes)


def bits_per_weight(fmt: int) -> float:
    return grouped_bits(4, GROUP, SCALE_BITS[fmt])


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
