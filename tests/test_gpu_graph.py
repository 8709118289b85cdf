"""HIP-graph capture of whole calls.  The entry points never synchronize with
the host (the chunked variant runs a fixed-length chunk loop whose bounds are
read on the device), so moe_ffn_fwd, moe_dx_bwd, moe_router_bwd and the adapter
calls can be captured once and replayed.  Each replay, with unrelated eager work and host synchronizations
between replays, must reproduce the eager result bit for bit."""
import numpy as np
import pytest
import torch

import quantized_grouped_gemm_amd as qgg
import synth
from synth.configs import CONFIGS, scaled

from .gpu_util import DEV, dev_bf16, dev_weights, host_u16, sync

pytestmark = pytest.mark.gpu

CASES = [
    # Zipf routing: most chunks of 4 experts are empty, the loop still runs
    # ceil(min(E, T*k) / 4) iterations
    (scaled(CONFIGS["int4_ffn_decode_zipf"], T=48, d=256, E=40, k=4, N=512, inter=256,
            chunks=(4,), name="int4_zipf_graph"), qgg.CHUNKED, 4),
    (scaled(CONFIGS["int4_ffn_decode_zipf"], T=48, d=256, E=40, k=4, N=512, inter=256,
            chunks=(4,), name="int4_zipf_graph"), qgg.FUSED, 0),
    (scaled(CONFIGS["mxfp4_ffn_prefill"], T=96, d=256, E=16, k=4, N=512, inter=256, chunks=(3,),
            name="mxfp4_ffn_graph"), qgg.CHUNKED, 3),
]


@pytest.mark.parametrize("cfg,variant,chunk", CASES,
                         ids=lambda v: v.name if hasattr(v, "name") else str(v))
def test_ffn_and_dx_graph_replays_match_eager(cfg, variant, chunk):
    print(f"case {cfg.name} variant {variant} chunk {chunk}", flush=True)
    logits = torch.from_numpy(synth.configs.router_logits(cfg)).to(DEV)
    x = dev_bf16(synth.configs.activations(cfg))
    dy = dev_bf16(synth.configs.grad_output(cfg))
    wg = dev_weights(cfg.fmt, *synth.configs.first_weights(cfg), layout=qgg.LAYOUT_MFMA)
    wd = dev_weights(cfg.fmt, *synth.configs.down_weights(cfg), layout=qgg.LAYOUT_MFMA)

    def step():
        r = qgg.moe_ffn_fwd(wg, wd, x, logits, cfg.k, variant, chunk, save_h=True)
        dx = qgg.moe_dx_bwd(wg, wd, dy, r["topk_gates"], r["perm"], r["h"], cfg.k, variant,
                            chunk)
        g = qgg.moe_router_bwd(wg, wd, dy, r["topk_ids"], r["topk_gates"], r["perm"], r["h"],
                               cfg.k, variant, chunk, want_dx=False)
        return r["y"], r["h"], dx, g["dgates"], g["dlogits"]

    def host(outs):
        return [host_u16(t) for t in outs[:3]] + [t.cpu().numpy() for t in outs[3:]]

    ref = host(step())                                     # eager reference
    sync()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):                          # warm up on the side stream
        step()
    torch.cuda.current_stream().wait_stream(side)
    sync()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        outs = step()
    for rep in range(3):
        graph.replay()
        sync()
        got = host(outs)
        for name, a, b in zip(("y", "h", "dx", "dgates", "dlogits"), got, ref):
            np.testing.assert_array_equal(a, b, err_msg=f"{name} replay {rep}")
        for t in outs:                                     # eager work between replays
            t.zero_()
        step()
        sync()


def test_adapter_calls_graph_replays_match_eager():
    cfg = scaled(CONFIGS["kimi_int4_gate_up"], T=96, d=256, E=12, k=4, N=320, chunks=(5,),
                 name="int4_lora_graph")
    rank = 32
    print(f"case {cfg.name} rank {rank}", flush=True)
    logits = torch.from_numpy(synth.configs.router_logits(cfg)).to(DEV)
    x = dev_bf16(synth.configs.activations(cfg))
    w = dev_weights(cfg.fmt, *synth.configs.first_weights(cfg), layout=qgg.LAYOUT_MFMA)
    A = dev_bf16(synth.normal_bf16(cfg.seed, 7, (cfg.E, rank, cfg.d), std=0.05))
    B = dev_bf16(synth.normal_bf16(cfg.seed, 8, (cfg.E, cfg.N, rank), std=0.05))
    dy = dev_bf16(synth.normal_bf16(cfg.seed, 5, (cfg.T * cfg.k, cfg.N)))

    def step():
        ids, _ = qgg.moe_route(logits, cfg.k)
        p, _ = qgg.expert_permute(ids, cfg.E)
        y, u = qgg.lora_grouped_gemm(w, A, B, 0.5, x, p, cfg.T, cfg.k, qgg.CHUNKED, 5)
        g = qgg.lora_grouped_gemm_bwd(A, B, 0.5, x, dy, u, p, cfg.T, cfg.k)
        return y, u, g["dx"], g["dA"], g["dB"]

    def host(outs):
        return [host_u16(t) for t in outs[:3]] + [t.cpu().numpy() for t in outs[3:]]

    ref = host(step())
    sync()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step()
    torch.cuda.current_stream().wait_stream(side)
    sync()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        outs = step()
    for rep in range(3):
        graph.replay()
        sync()
        for name, a, b in zip(("y", "u", "dx", "dA", "dB"), host(outs), ref):
            np.testing.assert_array_equal(a, b, err_msg=f"{name} replay {rep}")
        for t in outs:
            t.zero_()
        step()
        sync()


def test_ffn_adapter_forward_and_backward_graph_replays_match_eager():
    cfg = scaled(CONFIGS["int4_ffn_decode_zipf"], T=48, d=256, E=40, k=4, N=512, inter=256,
                 chunks=(4,), name="int4_zipf_lora_graph")
    rank = 16
    print(f"case {cfg.name} rank {rank}", flush=True)
    logits = torch.from_numpy(synth.configs.router_logits(cfg)).to(DEV)
    x = dev_bf16(synth.configs.activations(cfg))
    dy = dev_bf16(synth.configs.grad_output(cfg))
    wg = dev_weights(cfg.fmt, *synth.configs.first_weights(cfg), layout=qgg.LAYOUT_MFMA)
    wd = dev_weights(cfg.fmt, *synth.configs.down_weights(cfg), layout=qgg.LAYOUT_MFMA)
    I = cfg.inter
    lg = (dev_bf16(synth.normal_bf16(cfg.seed, 7, (cfg.E, rank, cfg.d), std=0.05)),
          dev_bf16(synth.normal_bf16(cfg.seed, 8, (cfg.E, 2 * I, rank), std=0.05)), 0.5)
    ld = (dev_bf16(synth.normal_bf16(cfg.seed, 9, (cfg.E, rank, I), std=0.05)),
          dev_bf16(synth.normal_bf16(cfg.seed, 10, (cfg.E, cfg.d, rank), std=0.05)), 0.75)

    def step():
        r = qgg.moe_ffn_fwd_lora(wg, wd, lg, ld, x, logits, cfg.k, qgg.CHUNKED, 4, save_h=True)
        g = qgg.moe_ffn_bwd_lora(wg, wd, lg, ld, x, dy, r["topk_gates"], r["perm"], r["h"],
                                 r["u_gate_up"], r["u_down"], cfg.k, qgg.CHUNKED, 4)
        f = qgg.moe_ffn_bwd_lora(wg, wd, lg, ld, x, dy, r["topk_gates"], r["perm"], r["h"],
                                 r["u_gate_up"], r["u_down"], cfg.k, qgg.FUSED, 0)
        return (r["y"], g["dx"], f["dx"], g["dA_gate_up"], g["dB_gate_up"], g["dA_down"],
                g["dB_down"], f["dA_down"])

    def host(outs):
        return [host_u16(t) for t in outs[:3]] + [t.cpu().numpy() for t in outs[3:]]

    ref = host(step())
    sync()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step()
    torch.cuda.current_stream().wait_stream(side)
    sync()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        outs = step()
    names = ("y", "dx", "dx_fused", "dA_gate_up", "dB_gate_up", "dA_down", "dB_down",
             "dA_down_fused")
    for rep in range(3):
        graph.replay()
        sync()
        for name, a, b in zip(names, host(outs), ref):
            np.testing.assert_array_equal(a, b, err_msg=f"{name} replay {rep}")
        for t in outs:
            t.zero_()
        step()
        sync()
