"""The five synthetic workloads of the quantized MoE grouped-GEMM path.

Each entry states shapes, the weight format, the chunk sizes to run and the
routing recipe.  ``generate`` turns an entry into seeded host arrays through the
generator in ``synth.c``; every consumer (oracle, GPU library, bench) reads the
same bytes.
"""
from __future__ import annotations

from dataclasses import dataclass, field

import numpy as np

# Philox stream ids, one per tensor role.
STREAM = {"logits": 1, "x": 2, "w_gate_up": 3, "w_down": 4, "dy": 5, "zipf": 6, "lora_a": 7,
          "lora_b": 8}


@dataclass(frozen=True)
class Config:
    name: str
    kind: str                 # "proj" | "ffn" | "bwd"
    T: int
    d: int
    E: int
    k: int
    N: int                    # output width of the first projection (2*inter for FFN)
    inter: int                # FFN intermediate size (0 for a single projection)
    fmt: int                  # 1 = MXFP4, 2 = INT4 (BF16 scale)
    chunks: tuple = (32,)     # chunk sizes (experts per chunk); 0 means "all active"
    zipf_s: float = 0.0       # > 0: router logits biased so popularity ~ rank^-s
    seed: int = 0
    w_std: float = 0.02
    note: str = field(default="", compare=False)

    @property
    def P(self) -> int:
        return self.T * self.k

    @property
    def fmt_name(self) -> str:
        return "mxfp4" if self.fmt == 1 else "int4"


CONFIGS = {
    "tiny_mxfp4_proj": Config(
        "tiny_mxfp4_proj", "proj", T=64, d=256, E=8, k=2, N=512, inter=0, fmt=1,
        chunks=(4,), note="single MXFP4 projection, T=64 d=256 E=8 top-2 N=512 chunk=4"),
    "kimi_int4_gate_up": Config(
        "kimi_int4_gate_up", "proj", T=4096, d=7168, E=384, k=8, N=4096, inter=2048, fmt=2,
        chunks=(32,), note="INT4 gate_up grouped GEMM, T=4096 d=7168 E=384 top-8 N=4096 chunk=32"),
    "mxfp4_ffn_prefill": Config(
        "mxfp4_ffn_prefill", "ffn", T=8192, d=7168, E=256, k=8, N=4096, inter=2048, fmt=1,
        chunks=(32,), note="MXFP4 SwiGLU expert FFN, T=8192 d=7168 E=256 top-8 inter=2048 chunk=32"),
    "int4_ffn_decode_zipf": Config(
        "int4_ffn_decode_zipf", "ffn", T=64, d=7168, E=384, k=8, N=4096, inter=2048, fmt=2,
        chunks=(8, 32, 0), zipf_s=1.2,
        note="INT4 FFN decode, T=64 d=7168 E=384 top-8 inter=2048, Zipf s=1.2 routing"),
    "mxfp4_dx_bwd": Config(
        "mxfp4_dx_bwd", "bwd", T=8192, d=7168, E=256, k=8, N=4096, inter=2048, fmt=1,
        chunks=(8, 32, 0),
        note="MXFP4 input-gradient backward, T=8192 d=7168 E=256 top-8 inter=2048"),
}

ORDER = ["tiny_mxfp4_proj", "kimi_int4_gate_up", "mxfp4_ffn_prefill",
         "int4_ffn_decode_zipf", "mxfp4_dx_bwd"]


def scaled(cfg: Config, **kw) -> Config:
    """A copy of ``cfg`` with some fields replaced (smaller parity cases)."""
    d = dict(cfg.__dict__)
    d.update(kw)
    return Config(**d)


def router_logits(cfg: Config) -> np.ndarray:
    from . import normal_f32, zipf_bias
    bias = None
    if cfg.zipf_s > 0:
        _, bias = zipf_bias(cfg.seed, STREAM["zipf"], cfg.E, cfg.zipf_s)
    return normal_f32(cfg.seed, STREAM["logits"], (cfg.T, cfg.E), 1.0, bias)


def activations(cfg: Config) -> np.ndarray:
    from . import normal_bf16
    return normal_bf16(cfg.seed, STREAM["x"], (cfg.T, cfg.d))


def grad_output(cfg: Config) -> np.ndarray:
    from . import normal_bf16
    return normal_bf16(cfg.seed, STREAM["dy"], (cfg.T, cfg.d))


def first_weights(cfg: Config, e0: int = 0, e1: int | None = None):
    """Single projection / gate_up weights [E][N][K=d] (gate rows first, then up)."""
    from . import qweights
    return qweights(cfg.seed, STREAM["w_gate_up"], cfg.fmt, cfg.E, cfg.N, cfg.d, e0, e1, cfg.w_std)


def down_weights(cfg: Config, e0: int = 0, e1: int | None = None):
    """Down projection weights [E][N=d][K=inter]."""
    from . import qweights
    assert cfg.inter > 0
    return qweights(cfg.seed, STREAM["w_down"], cfg.fmt, cfg.E, cfg.d, cfg.inter, e0, e1, cfg.w_std)
