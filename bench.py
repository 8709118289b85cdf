"""Benchmark of the quantized MoE grouped-GEMM hot path on one MI355X.

Workload (default): the Kimi-class INT4 gate_up grouped GEMM -- T=4096 tokens,
d=7168, E=384 experts, top-8, N=4096 (gate|up of inter=2048), group-32 INT4
weights with BF16 scales, chunk=32.  One step is the whole path over one batch:
moe_route -> expert_permute -> dequant_grouped_gemm (token rows gathered in the
GEMM's A loader), fused variant.  Inputs are generated once, uploaded to HBM,
and stay resident; the timed region holds only the kernels.

Prints ONE JSON line: TFLOP/s of the step, plus weight GB/s, roofline fraction
of the dominant kernel (the grouped GEMM, timed with HIP events on its stream),
peak dequant scratch per variant, and the CPU oracle's throughput on a bounded
sample of the same workload.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "MoE dequant grouped-GEMM TFLOP/s + weight GB/s (% roofline), peak scratch MB"
DOMINANT_KERNEL = "k_gemm_nt"
KERNEL_SOURCES = ["quantized_grouped_gemm_amd/csrc/gemm_nt.hip",
                  "quantized_grouped_gemm_amd/csrc/qgg_device.hpp"]
COUNTERS_FILE = os.path.join(ROOT, "profiles", "k_gemm_nt_kimi_int4_gate_up_counters.json")


def kernel_hash() -> str:
    h = hashlib.sha256()
    for f in KERNEL_SOURCES:
        with open(os.path.join(ROOT, f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def measured_traffic():
    """HBM bytes per launch of the dominant kernel from the committed counter
    summary, if it was taken on the current kernel source; else None."""
    try:
        with open(COUNTERS_FILE) as f:
            c = json.load(f)
    except (OSError, ValueError):
        return None
    if c.get("kernel_hash") != kernel_hash():
        return None
    return c.get("hbm_bytes_per_launch")


def cpu_baseline(cfg, logits, x, budget_s: float = 15.0):
    """The CPU oracle on a bounded sample: every routed row of the first active
    experts, one expert at a time until the time budget is spent."""
    import oracle
    import synth.configs as sc
    ids, _ = oracle.route(logits, cfg.k)
    perm = oracle.permute(ids, cfg.E)
    flat = ids.reshape(-1)
    flops = 0.0
    n_exp = 0
    rows = 0
    busy = 0.0
    for a in range(perm["n_active"]):
        e = int(perm["active"][a])
        sel = perm["perm"][perm["offsets"][e]:perm["offsets"][e + 1]]
        assert np.all(flat[sel] == e)
        p, s = sc.first_weights(cfg, e, e + 1)          # this expert's bytes (not timed)
        t1 = time.perf_counter()
        oracle.project(cfg.fmt, p, s, x, (sel // cfg.k).astype(np.int32),
                       np.zeros(sel.size, np.int32))
        busy += time.perf_counter() - t1
        flops += 2.0 * sel.size * cfg.N * cfg.d
        rows += sel.size
        n_exp += 1
        if busy > budget_s and n_exp >= 2:
            break
    return flops, rows, n_exp, busy


def run(args):
    import torch
    import quantized_grouped_gemm_amd as qgg
    from quantized_grouped_gemm_amd import accounting as acc
    import synth
    import synth.configs as sc

    cfg = sc.CONFIGS[args.config]
    if cfg.kind != "proj":
        return run_ffn(args, cfg)
    dev = torch.device("cuda:0")
    t_gen = time.perf_counter()
    logits = sc.router_logits(cfg)
    x = sc.activations(cfg)
    packed, scales = sc.first_weights(cfg)
    t_gen = time.perf_counter() - t_gen

    lt = torch.from_numpy(logits).to(dev)
    xd = torch.from_numpy(x.view(np.int16)).to(dev).view(torch.bfloat16)
    pd = torch.from_numpy(packed).to(dev)
    sd = torch.from_numpy(scales.view(np.int16) if scales.dtype == np.uint16 else scales).to(dev)
    del packed, scales
    # the frozen base is stored in the MFMA-tiled order (one repack at load)
    w = qgg.repack(qgg.QWeight(cfg.fmt, pd, sd))
    del pd, sd
    torch.cuda.synchronize()
    P = cfg.P
    ws = qgg.Workspace()
    y = torch.empty((P, cfg.N), dtype=torch.bfloat16, device=dev)
    stream = torch.cuda.current_stream()

    def step(variant, chunk, ev=None):
        ids, _ = qgg.moe_route(lt, cfg.k)
        p, _ = qgg.expert_permute(ids, cfg.E, ws=ws)
        if ev is not None:
            ev[0].record(stream)
        qgg.dequant_grouped_gemm(w, xd, p, cfg.T, cfg.k, variant, chunk, flags=qgg.A_TOKENS,
                                 ws=ws, out=y)
        if ev is not None:
            ev[1].record(stream)
        return p

    if args.calib_copy_mib > 0:
        # a plain device copy of known size, so that a counter run over this
        # command can scale FETCH_SIZE / WRITE_SIZE to bytes
        # (an elementwise add: reads n bytes, writes n bytes, one kernel)
        n = args.calib_copy_mib << 20
        src = torch.empty(n // 4, dtype=torch.float32, device=dev).fill_(1.0)
        dst = torch.empty_like(src)
        for _ in range(3):
            torch.add(src, 1.0, out=dst)
        torch.cuda.synchronize()
        del src, dst

    results = {}
    variants = [("fused", qgg.FUSED, 0), ("chunked", qgg.CHUNKED, cfg.chunks[0])]
    if args.fused_only:
        variants = variants[:1]
    for vname, variant, chunk in variants:
        for _ in range(args.warmup):
            p = step(variant, chunk)
        torch.cuda.synchronize()
        evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
               for _ in range(args.steps)]
        t0 = time.perf_counter()
        for i in range(args.steps):
            p = step(variant, chunk, evs[i])
        torch.cuda.synchronize()
        wall = (time.perf_counter() - t0) / args.steps
        gemm_ms = float(np.mean([a.elapsed_time(b) for a, b in evs]))
        n_active = int(p.n_active.item())
        _, scratch = qgg.workspace_bytes(qgg.CALL_GEMM, cfg.T, cfg.d, cfg.E, cfg.k, cfg.N,
                                         variant, chunk)
        results[vname] = dict(ms_per_step=wall * 1e3, gemm_ms=gemm_ms, n_active=n_active,
                              chunk=chunk, peak_scratch_MB=scratch / 2 ** 20)

    F = acc.proj_flops(P, cfg.N, cfg.d)
    n_active = results["fused"]["n_active"]
    wbytes = n_active * acc.packed_bytes(cfg.fmt, cfg.N, cfg.d)
    alg_bytes = acc.proj_alg_bytes(cfg.fmt, n_active, cfg.N, cfg.d, cfg.T, P)
    t_mfma = F / (acc.BF16_DENSE_PEAK_TFLOPS * 1e12)
    t_hbm = alg_bytes / (acc.HBM_PEAK_GBPS * 1e9)
    bound = "hbm" if t_hbm >= t_mfma else "mfma"
    fused = results["fused"]
    gemm_s = fused["gemm_ms"] / 1e3
    if bound == "hbm":
        achieved, peak, unit = alg_bytes / gemm_s / 1e9, acc.HBM_PEAK_GBPS, "GB/s"
    else:
        achieved, peak, unit = F / gemm_s / 1e12, acc.BF16_DENSE_PEAK_TFLOPS, "TFLOP/s"
    for r in results.values():
        r["step_TFLOPs"] = F / (r["ms_per_step"] / 1e3) / 1e12
        r["gemm_TFLOPs"] = F / (r["gemm_ms"] / 1e3) / 1e12
        r["weight_GBps"] = wbytes / (r["gemm_ms"] / 1e3) / 1e9
        r["pct_roofline"] = 100.0 * max(t_mfma, t_hbm) / (r["gemm_ms"] / 1e3)

    out = {
        "metric": METRIC,
        "value": round(F / (fused["ms_per_step"] / 1e3) / 1e12, 3),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(fused["ms_per_step"], 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": cfg.name, "T": cfg.T, "d": cfg.d, "E": cfg.E, "top_k": cfg.k,
                   "N": cfg.N, "weights": cfg.fmt_name + " group-32", "chunk": cfg.chunks[0],
                   "variant": "fused", "weight_layout": "mfma-tiled", "seed": cfg.seed},
        "roofline": {"bound": bound, "achieved": round(achieved, 2), "peak": peak, "unit": unit,
                     "frac": round(achieved / peak, 4), "traffic": measured_traffic(),
                     "kernel": DOMINANT_KERNEL, "kernel_ms": round(fused["gemm_ms"], 4),
                     "alg_bytes": alg_bytes, "alg_flops": F,
                     "mfma_frac": round(F / gemm_s / 1e12 / acc.BF16_DENSE_PEAK_TFLOPS, 4)},
        "weight_GBps": round(fused["weight_GBps"], 1),
        "peak_scratch_MB": {k: round(v["peak_scratch_MB"], 1) for k, v in results.items()},
        "variants": {k: {kk: (round(vv, 4) if isinstance(vv, float) else vv)
                         for kk, vv in v.items()} for k, v in results.items()},
        "n_active": n_active,
        "input_gen_s": round(t_gen, 2),
    }
    if not args.no_cpu_baseline:
        import oracle
        flops, rows, n_exp, dt = cpu_baseline(cfg, logits, x, args.cpu_budget)
        out["cpu_baseline"] = {
            "value": round(flops / dt / 1e12, 6), "unit": "TFLOP/s", "cores": oracle.num_threads(),
            "kind": "oracle",
            "sample": f"all {rows} routed rows of the first {n_exp} active experts "
                      f"(oracle: decode + fp64 dot products), {dt:.1f} s"}
    print(json.dumps(out), flush=True)


def run_ffn(args, cfg):
    """The expert-FFN workloads (not the default line): moe_ffn_fwd for an "ffn"
    configuration, moe_dx_bwd (after one forward that saves h) for a "bwd" one,
    FUSED, whole-call time.  The roofline is the call's flops against the dense
    BF16 MFMA peak; per-kernel figures come from a rocprofv3 trace of this
    command."""
    import torch
    import quantized_grouped_gemm_amd as qgg
    import synth.configs as sc

    dev = torch.device("cuda:0")

    def up_w(pk_sc):
        pk, scl = pk_sc
        scl = scl.view(np.int16) if scl.dtype == np.uint16 else scl
        return qgg.repack(qgg.QWeight(cfg.fmt, torch.from_numpy(pk).to(dev),
                                      torch.from_numpy(scl).to(dev)))

    def up_bf16(a):
        return torch.from_numpy(a.view(np.int16)).to(dev).view(torch.bfloat16)

    lt = torch.from_numpy(sc.router_logits(cfg)).to(dev)
    x = up_bf16(sc.activations(cfg))
    wg, wd = up_w(sc.first_weights(cfg)), up_w(sc.down_weights(cfg))
    ws = qgg.Workspace()
    if cfg.kind == "ffn":
        def call():
            return qgg.moe_ffn_fwd(wg, wd, x, lt, cfg.k, qgg.FUSED, 0, ws=ws)
    else:
        fwd = qgg.moe_ffn_fwd(wg, wd, x, lt, cfg.k, qgg.FUSED, 0, save_h=True)
        dy = up_bf16(sc.grad_output(cfg))

        def call():
            return qgg.moe_dx_bwd(wg, wd, dy, fwd["topk_gates"], fwd["perm"], fwd["h"], cfg.k,
                                  qgg.FUSED, 0, ws=ws)
    for _ in range(args.warmup):
        call()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        call()
    torch.cuda.synchronize()
    ms = (time.perf_counter() - t0) / args.steps * 1e3
    P = cfg.T * cfg.k
    flops = 2.0 * P * (2 * cfg.inter * cfg.d + cfg.d * cfg.inter)
    tf = flops / (ms / 1e3) / 1e12
    from quantized_grouped_gemm_amd import accounting as acc
    out = {
        "metric": "MoE expert FFN TFLOP/s (whole call)", "value": round(tf, 3),
        "unit": "TFLOP/s", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": round(ms, 4), "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
        "config": {"workload": cfg.name, "T": cfg.T, "d": cfg.d, "E": cfg.E, "top_k": cfg.k,
                   "inter": cfg.inter, "weights": cfg.fmt_name + " group-32",
                   "variant": "fused", "call": "moe_ffn_fwd" if cfg.kind == "ffn" else "moe_dx_bwd"},
        "roofline": {"bound": "mfma", "achieved": round(tf, 2),
                     "peak": acc.BF16_DENSE_PEAK_TFLOPS, "unit": "TFLOP/s",
                     "frac": round(tf / acc.BF16_DENSE_PEAK_TFLOPS, 4), "traffic": None,
                     "kernel": "whole call"},
    }
    print(json.dumps(out), flush=True)


def main():
    ap = argparse.ArgumentParser(description=__doc__.splitlines()[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--config", default="kimi_int4_gate_up")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-budget", type=float, default=15.0)
    ap.add_argument("--calib-copy-mib", type=int, default=0,
                    help="run a plain device copy of this size first (counter calibration)")
    ap.add_argument("--fused-only", action="store_true")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: this path runs on a single MI355X "
              "(run with --gpus 1)", file=sys.stderr)
        sys.exit(2)
    run(args)


if __name__ == "__main__":
    main()
