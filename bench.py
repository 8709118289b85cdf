"""Benchmark of the quantized MoE grouped-GEMM hot path on one MI355X.

Headline workload (the N=1 line): the MXFP4 SwiGLU expert FFN, prefill-shaped --
T=8192 tokens, d=7168, E=256 experts, top-8, inter=2048, E2M1 weights with one
E8M0 scale per 32 elements along K.  One step is the whole path over one batch:
moe_ffn_fwd = route -> permute -> gate_up grouped GEMM (token rows gathered in
the A loader, SwiGLU in the epilogue) -> down grouped GEMM -> gate-weighted
combine, fused variant.  Inputs are generated once, uploaded to HBM and stay
resident; the timed region holds only the library's kernels.

Beside it, as sub-objects of the same JSON line, the other workloads of the
path, each with its own roofline for its dominant kernel: the Kimi-class INT4
gate_up projection, the INT4 decode FFN with Zipf routing (HBM-bound) and the
MXFP4 input-gradient backward, plus the chunk-size sweeps (weight GB/s and
peak dequant scratch, the scratch checked against the caching allocator).

Per-kernel durations come from HIP events the library records around each of
its kernel launches on the call's stream (qgg_set_timing_events), over the
same number of steps as the timed region; each roofline takes the mean launch
duration and also reports the median and the minimum.  No cache flush runs
between steps: every workload's per-step stream of packed weights (1.1-6.7 GB)
exceeds the 256 MB MALL four times over or more.

Prints ONE JSON line.
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
HEADLINE = "mxfp4_ffn_prefill"
KERNEL_SOURCES = {"k_gemm_nt": ["quantized_grouped_gemm_amd/csrc/gemm_nt.hip",
                                "quantized_grouped_gemm_amd/csrc/qgg_device.hpp"],
                  "k_gemm_tn": ["quantized_grouped_gemm_amd/csrc/gemm_tn.hip",
                                "quantized_grouped_gemm_amd/csrc/qgg_device.hpp"]}
KIND = {1: "route", 2: "permute", 3: "gemm", 4: "gemm_t", 5: "dequant", 6: "combine",
        7: "lora", 8: "router_bwd"}


def kernel_hash(kernel: str) -> str:
    h = hashlib.sha256()
    for f in KERNEL_SOURCES[kernel]:
        with open(os.path.join(ROOT, f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def measured_traffic(kernel: str, workload: str):
    """(HBM bytes per launch, where the figure comes from) for `kernel` on
    `workload`: the committed counter summary (FETCH_SIZE and WRITE_SIZE of a
    separate rocprofv3 run, scaled by a copy kernel of known size) if it was
    taken on the current kernel source; else (None, why not)."""
    rel = os.path.join("profiles", f"{kernel}_{workload}_counters.json")
    try:
        with open(os.path.join(ROOT, rel)) as f:
            c = json.load(f)
    except (OSError, ValueError):
        return None, f"no counter summary {rel}"
    h = kernel_hash(kernel)
    if c.get("kernel_hash") != h:
        return None, f"{rel} was taken on another kernel source (hash {c.get('kernel_hash')})"
    return c.get("hbm_bytes_per_launch"), (
        f"{rel}: rocprofv3 FETCH_SIZE x {c.get('fetch_scale', 0):.3f} + WRITE_SIZE x "
        f"{c.get('write_scale', 0):.3f} per launch, counters of a separate profiled run on "
        f"this kernel source (hash {h})")


# ------------------------------------------------------------------ timing

class KernelTimer:
    """Caller-owned HIP events handed to the library, which records a pair
    around each kernel launch it makes (on the launch's stream)."""

    def __init__(self, capacity: int):
        import torch
        self.cap = capacity
        self.events = [torch.cuda.Event(enable_timing=True) for _ in range(2 * capacity)]
        for e in self.events:            # creates the underlying hipEvent
            e.record()
        torch.cuda.synchronize()

    def run(self, fn, steps: int):
        """Run fn() `steps` times with launch timing on; returns a list per
        step of (kind, ms) in launch order."""
        import torch
        import quantized_grouped_gemm_amd as qgg
        per_step = []
        for _ in range(steps):
            qgg.set_timing_events(self.events, self.cap)
            fn()
            n = qgg.timing_count()
            kinds = qgg.timing_kinds(n)
            qgg.set_timing_events(None, 0)
            torch.cuda.synchronize()
            per_step.append([(KIND.get(kinds[i], str(kinds[i])),
                              self.events[2 * i].elapsed_time(self.events[2 * i + 1]))
                             for i in range(n)])
        return per_step


def time_steps(fn, steps: int, warmup: int):
    """ms per step of fn() over exactly `steps` calls, synchronised on both
    sides (warm-up calls first)."""
    import torch
    for _ in range(warmup):
        fn()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(steps):
        fn()
    torch.cuda.synchronize()
    return (time.perf_counter() - t0) / steps * 1e3


def launch_means(per_step, pick):
    """Mean duration (ms) of the launches `pick` selects from each step's
    launch list (pick(list) -> index)."""
    return float(np.mean([s[pick(s)][1] for s in per_step]))


def launch_spread(per_step, pick):
    """(median, min) duration (ms) of the same launches."""
    v = [s[pick(s)][1] for s in per_step]
    return float(np.median(v)), float(np.min(v))


def nth(kind, n):
    def pick(s):
        idx = [i for i, (k, _) in enumerate(s) if k == kind]
        return idx[n]
    return pick


def roofline(alg_flops, alg_bytes, kernel_ms, traffic, kernel_name, spread=None):
    """Roofline object of a kernel: bound by whichever of the MFMA and HBM
    times at the published peaks is larger (achieved from the mean launch
    duration `kernel_ms`; `spread` adds the median and minimum).  `traffic`
    is None or (bytes or None, source) from measured_traffic."""
    traffic, traffic_src = traffic if isinstance(traffic, tuple) else (traffic, None)
    from quantized_grouped_gemm_amd import accounting as acc
    t_mfma = alg_flops / (acc.BF16_DENSE_PEAK_TFLOPS * 1e12)
    t_hbm = alg_bytes / (acc.HBM_PEAK_GBPS * 1e9)
    s = kernel_ms / 1e3
    if t_hbm >= t_mfma:
        bound, achieved, peak, unit = "hbm", alg_bytes / s / 1e9, acc.HBM_PEAK_GBPS, "GB/s"
    else:
        bound, achieved, peak, unit = ("mfma", alg_flops / s / 1e12, acc.BF16_DENSE_PEAK_TFLOPS,
                                       "TFLOP/s")
    return {"bound": bound, "achieved": round(achieved, 2), "peak": peak, "unit": unit,
            "frac": round(achieved / peak, 4), "traffic": traffic,
            **({"traffic_source": traffic_src} if traffic_src else {}), "kernel": kernel_name,
            "kernel_ms": round(kernel_ms, 4),
            **({"kernel_ms_median": round(spread[0], 4), "kernel_ms_min": round(spread[1], 4)}
               if spread else {}),
            "alg_flops": alg_flops, "alg_bytes": alg_bytes,
            "mfma_frac": round(alg_flops / s / 1e12 / acc.BF16_DENSE_PEAK_TFLOPS, 4),
            "hbm_frac": round(alg_bytes / s / 1e9 / acc.HBM_PEAK_GBPS, 4)}


def scratch_check(call, variant, chunk, ws_query):
    """(formula scratch MiB, allocator-measured workspace MiB): one call with
    a fresh workspace, peak allocated bytes above the level before it."""
    import torch
    import quantized_grouped_gemm_amd as qgg
    torch.cuda.synchronize()
    torch.cuda.empty_cache()
    base = torch.cuda.memory_allocated()
    torch.cuda.reset_peak_memory_stats()
    ws = qgg.Workspace()
    out = call(variant, chunk, ws)
    torch.cuda.synchronize()
    peak = torch.cuda.max_memory_allocated() - base
    total, scratch = ws_query(variant, chunk)
    del out, ws
    torch.cuda.synchronize()
    return scratch / 2 ** 20, total / 2 ** 20, peak / 2 ** 20


# ------------------------------------------------------------------ inputs

def _dev():
    import torch
    return torch.device("cuda:0")


def up_bf16(a):
    import torch
    return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).to(_dev()).view(torch.bfloat16)


def up_weights(cfg, pk_sc):
    """The frozen base in the MFMA-tiled order (one repack at load)."""
    import torch
    import quantized_grouped_gemm_amd as qgg
    pk, scl = pk_sc
    scl = scl.view(np.int16) if scl.dtype == np.uint16 else scl
    w = qgg.QWeight(cfg.fmt, torch.from_numpy(pk).to(_dev()), torch.from_numpy(scl).to(_dev()))
    t = qgg.repack(w)
    del w
    return t


# ------------------------------------------------------------------ workloads

def run_ffn_fwd(cfg, args, cpu_budget=None):
    """moe_ffn_fwd, fused; dominant kernel = the gate_up GEMM (first forward
    GEMM launch).  For the decode workload also the chunk sweep."""
    import torch
    import quantized_grouped_gemm_amd as qgg
    from quantized_grouped_gemm_amd import accounting as acc
    import synth.configs as sc

    t_gen = time.perf_counter()
    logits, x_h = sc.router_logits(cfg), sc.activations(cfg)
    gu_h, dn_h = sc.first_weights(cfg), sc.down_weights(cfg)
    t_gen = time.perf_counter() - t_gen
    lt, x = torch.from_numpy(logits).to(_dev()), up_bf16(x_h)
    wg, wd = up_weights(cfg, gu_h), up_weights(cfg, dn_h)
    if cpu_budget is None:
        del gu_h, dn_h
    ws = qgg.Workspace()
    P, I, d = cfg.P, cfg.inter, cfg.d

    def call(variant=qgg.FUSED, chunk=0, w=ws):
        return qgg.moe_ffn_fwd(wg, wd, x, lt, cfg.k, variant, chunk, ws=w)

    ms = time_steps(call, args.steps, args.warmup)
    r = call()
    torch.cuda.synchronize()
    A = int(r["perm"].n_active.item())
    per = KernelTimer(16).run(call, args.steps)
    gu_ms = launch_means(per, nth("gemm", 0))
    dn_ms = launch_means(per, nth("gemm", 1))
    kern = {}
    for kind in ("route", "permute", "combine"):
        # decode-sized batches route and permute in one launch (kind "route")
        if any(k == kind for k, _ in per[0]):
            kern[kind + "_ms"] = round(launch_means(per, nth(kind, 0)), 4)
    kern.update(gate_up_ms=round(gu_ms, 4), down_ms=round(dn_ms, 4))

    F = acc.ffn_flops(P, d, I)
    w_gu = A * acc.packed_bytes(cfg.fmt, 2 * I, d)
    w_dn = A * acc.packed_bytes(cfg.fmt, d, I)
    # gate_up kernel: its experts' weights, each token row once, the SwiGLU
    # output a [P][I] written once
    gu_flops = 2.0 * P * 2 * I * d
    gu_bytes = w_gu + cfg.T * d * 2.0 + P * I * 2.0
    dom = "k_gemm_nt"
    rl = roofline(gu_flops, gu_bytes, gu_ms, measured_traffic(dom, cfg.name),
                  "k_gemm_nt (gate_up, SwiGLU epilogue)", launch_spread(per, nth("gemm", 0)))
    out = {
        "ms_per_step": round(ms, 4),
        "step_TFLOPs": round(F / (ms / 1e3) / 1e12, 3),
        "weight_GBps": round((w_gu + w_dn) / (ms / 1e3) / 1e9, 1),
        "gemm_weight_GBps": round((w_gu + w_dn) / ((gu_ms + dn_ms) / 1e3) / 1e9, 1),
        "n_active": A,
        "kernels": kern,
        "roofline": rl,
        "input_gen_s": round(t_gen, 2),
    }
    # down kernel roofline too (the step's second GEMM)
    dn_bytes = w_dn + P * I * 2.0 + P * d * 2.0
    out["roofline_down"] = roofline(2.0 * P * d * I, dn_bytes, dn_ms, None,
                                    "k_gemm_nt (down)", launch_spread(per, nth("gemm", 1)))

    def ws_query(variant, chunk):
        return qgg.workspace_bytes(qgg.CALL_FFN_FWD, cfg.T, d, cfg.E, cfg.k, I, variant, chunk)

    sweep = {}
    chunks = list(cfg.chunks) if args.sweep else []
    if args.sweep and 0 in chunks:
        chunks = [c for c in chunks if c != 0] + ["A", 0]
    for c in chunks:
        chunk = A if c == "A" else c
        label = "all_active_A" if c == "A" else ("all_0" if c == 0 else str(c))
        cms = time_steps(lambda: call(qgg.CHUNKED, chunk), max(2, args.steps // 4), 1)
        s_mib, tot_mib, peak_mib = scratch_check(
            lambda v, ch, w: call(v, ch, w), qgg.CHUNKED, chunk, ws_query)
        sweep[label] = {"chunk": chunk, "ms": round(cms, 4),
                        "weight_GBps": round((w_gu + w_dn) / (cms / 1e3) / 1e9, 1),
                        "scratch_MiB": round(s_mib, 1), "workspace_MiB": round(tot_mib, 1),
                        "allocator_peak_MiB": round(peak_mib, 1)}
    if chunks:
        s_mib, tot_mib, peak_mib = scratch_check(lambda v, ch, w: call(v, ch, w), qgg.FUSED, 0,
                                                 ws_query)
        sweep["fused"] = {"chunk": 0, "ms": round(ms, 4),
                          "weight_GBps": out["weight_GBps"], "scratch_MiB": round(s_mib, 1),
                          "workspace_MiB": round(tot_mib, 1),
                          "allocator_peak_MiB": round(peak_mib, 1)}
        out["sweep"] = sweep
    if cpu_budget is not None:
        out["cpu_baseline"] = cpu_baseline_ffn(cfg, logits, x_h, gu_h, dn_h, cpu_budget)
    del wg, wd, x, lt, ws, r
    torch.cuda.empty_cache()
    return out


def cpu_baseline_ffn(cfg, logits, x, gu, dn, budget_s):
    """The CPU oracle (oracle.ffn: decode, double dot products, SwiGLU,
    combine) on a bounded sample of the same workload: the first n tokens,
    n doubled from 16 until one run takes at least budget_s / 2 (the runs
    before it are probes, not counted)."""
    import oracle
    ids, gates = oracle.route(logits, cfg.k)
    n = 16
    while True:
        toks = np.arange(n, dtype=np.int32)
        t0 = time.perf_counter()
        oracle.ffn(cfg.fmt, gu, dn, x, ids, gates, toks)
        dt = time.perf_counter() - t0
        if dt >= budget_s / 2 or n >= cfg.T:
            break
        n = min(cfg.T, 2 * n if dt >= budget_s / 8 else 4 * n)
    from quantized_grouped_gemm_amd import accounting as acc
    flops = acc.ffn_flops(n * cfg.k, cfg.d, cfg.inter)
    return {"value": round(flops / dt / 1e12, 6), "unit": "TFLOP/s",
            "cores": oracle.num_threads(), "kind": "oracle",
            "sample": f"moe_ffn_fwd of the first {n} tokens ({n * cfg.k} routed rows; "
                      f"oracle: decode + fp64 dot products + SwiGLU + combine), {dt:.1f} s"}


def run_proj(cfg, args):
    """route -> permute -> dequant_grouped_gemm (fused, then chunked at the
    workload's chunk size); dominant kernel = the grouped GEMM."""
    import torch
    import quantized_grouped_gemm_amd as qgg
    from quantized_grouped_gemm_amd import accounting as acc
    import synth.configs as sc

    logits, x_h = sc.router_logits(cfg), sc.activations(cfg)
    lt, x = torch.from_numpy(logits).to(_dev()), up_bf16(x_h)
    w = up_weights(cfg, sc.first_weights(cfg))
    ws = qgg.Workspace()
    y = torch.empty((cfg.P, cfg.N), dtype=torch.bfloat16, device=_dev())

    def call(variant=qgg.FUSED, chunk=0):
        ids, _ = qgg.moe_route(lt, cfg.k)
        p, _ = qgg.expert_permute(ids, cfg.E, ws=ws)
        qgg.dequant_grouped_gemm(w, x, p, cfg.T, cfg.k, variant, chunk, flags=qgg.A_TOKENS,
                                 ws=ws, out=y)
        return p

    ms = time_steps(call, args.steps, args.warmup)
    p = call()
    torch.cuda.synchronize()
    A = int(p.n_active.item())
    per = KernelTimer(16).run(call, args.steps)
    g_ms = launch_means(per, nth("gemm", 0))
    F = acc.proj_flops(cfg.P, cfg.N, cfg.d)
    wbytes = A * acc.packed_bytes(cfg.fmt, cfg.N, cfg.d)
    alg = acc.proj_alg_bytes(cfg.fmt, A, cfg.N, cfg.d, cfg.T, cfg.P)
    out = {"ms_per_step": round(ms, 4), "step_TFLOPs": round(F / (ms / 1e3) / 1e12, 3),
           "gemm_ms": round(g_ms, 4), "weight_GBps": round(wbytes / (g_ms / 1e3) / 1e9, 1),
           "n_active": A,
           "roofline": roofline(F, alg, g_ms, measured_traffic("k_gemm_nt", cfg.name),
                                "k_gemm_nt (INT4 gate_up projection)",
                                launch_spread(per, nth("gemm", 0)))}
    C = cfg.chunks[0]
    if args.sweep:
        cms = time_steps(lambda: call(qgg.CHUNKED, C), max(2, args.steps // 4), 1)
        _, scratch = qgg.workspace_bytes(qgg.CALL_GEMM, cfg.T, cfg.d, cfg.E, cfg.k, cfg.N,
                                         qgg.CHUNKED, C)
        out["chunked"] = {"chunk": C, "ms_per_step": round(cms, 4),
                          "weight_GBps": round(wbytes / (cms / 1e3) / 1e9, 1),
                          "scratch_MiB": round(scratch / 2 ** 20, 1)}
    del w, x, lt, ws, y
    torch.cuda.empty_cache()
    return out


def run_bwd(cfg, args):
    """moe_dx_bwd after one forward that saves h; dominant kernel = the
    transposed gate_up GEMM (dXp = dH . W_gu, the second transposed launch)."""
    import torch
    import quantized_grouped_gemm_amd as qgg
    from quantized_grouped_gemm_amd import accounting as acc
    import synth.configs as sc

    logits, x_h = sc.router_logits(cfg), sc.activations(cfg)
    lt, x = torch.from_numpy(logits).to(_dev()), up_bf16(x_h)
    wg, wd = up_weights(cfg, sc.first_weights(cfg)), up_weights(cfg, sc.down_weights(cfg))
    dy = up_bf16(sc.grad_output(cfg))
    fwd = qgg.moe_ffn_fwd(wg, wd, x, lt, cfg.k, qgg.FUSED, 0, save_h=True)
    ws = qgg.Workspace()
    P, I, d = cfg.P, cfg.inter, cfg.d

    def call(variant=qgg.FUSED, chunk=0, w=ws):
        return qgg.moe_dx_bwd(wg, wd, dy, fwd["topk_gates"], fwd["perm"], fwd["h"], cfg.k,
                              variant, chunk, ws=w)

    ms = time_steps(call, args.steps, args.warmup)
    A = int(fwd["perm"].n_active.item())
    per = KernelTimer(16).run(call, args.steps)
    dn_ms = launch_means(per, nth("gemm_t", 0))
    gu_ms = launch_means(per, nth("gemm_t", 1))
    F = acc.ffn_flops(P, d, I)
    w_gu = A * acc.packed_bytes(cfg.fmt, 2 * I, d)
    w_dn = A * acc.packed_bytes(cfg.fmt, d, I)
    # transposed gate_up: weights, dH [P][2I] read once, dXp [P][d] written once
    gu_bytes = w_gu + P * 2 * I * 2.0 + P * d * 2.0
    out = {"ms_per_step": round(ms, 4), "step_TFLOPs": round(F / (ms / 1e3) / 1e12, 3),
           "n_active": A,
           "kernels": {"down_t_ms": round(dn_ms, 4), "gate_up_t_ms": round(gu_ms, 4),
                       "combine_ms": round(launch_means(per, nth("combine", 0)), 4)},
           "roofline": roofline(2.0 * P * 2 * I * d, gu_bytes, gu_ms,
                                measured_traffic("k_gemm_tn", cfg.name),
                                "k_gemm_tn (dXp = dH . W_gate_up)",
                                launch_spread(per, nth("gemm_t", 1))),
           "roofline_down": roofline(2.0 * P * d * I, w_dn + cfg.T * d * 2.0 + P * I * 2 * 2.0
                                     + P * 2 * I * 2.0, dn_ms, None,
                                     "k_gemm_tn (dA = g dY . W_down, SwiGLU backward)",
                                     launch_spread(per, nth("gemm_t", 0)))}

    def ws_query(variant, chunk):
        return qgg.workspace_bytes(qgg.CALL_DX_BWD, cfg.T, d, cfg.E, cfg.k, I, variant, chunk)

    if args.sweep:
        sweep = {}
        for c in cfg.chunks:
            label = "all_0" if c == 0 else str(c)
            cms = time_steps(lambda: call(qgg.CHUNKED, c), 2, 1)
            s_mib, tot_mib, peak_mib = scratch_check(lambda v, ch, w: call(v, ch, w),
                                                     qgg.CHUNKED, c, ws_query)
            sweep[label] = {"chunk": c, "ms": round(cms, 4),
                            "weight_GBps": round((w_gu + w_dn) / (cms / 1e3) / 1e9, 1),
                            "scratch_MiB": round(s_mib, 1), "workspace_MiB": round(tot_mib, 1),
                            "allocator_peak_MiB": round(peak_mib, 1)}
        s_mib, tot_mib, peak_mib = scratch_check(lambda v, ch, w: call(v, ch, w), qgg.FUSED, 0,
                                                 ws_query)
        sweep["fused"] = {"chunk": 0, "ms": round(ms, 4),
                          "weight_GBps": round((w_gu + w_dn) / (ms / 1e3) / 1e9, 1),
                          "scratch_MiB": round(s_mib, 1), "workspace_MiB": round(tot_mib, 1),
                          "allocator_peak_MiB": round(peak_mib, 1)}
        out["sweep"] = sweep
    del wg, wd, dy, fwd, ws, x, lt
    torch.cuda.empty_cache()
    return out


def run(args):
    import torch
    import synth.configs as sc
    import quantized_grouped_gemm_amd as qgg

    qgg.lib()
    if args.calib_copy_mib > 0:
        # a plain device copy of known size, so that a counter run over this
        # command can scale FETCH_SIZE / WRITE_SIZE to bytes
        # (an elementwise add: reads n bytes, writes n bytes, one kernel)
        n = args.calib_copy_mib << 20
        src = torch.empty(n // 4, dtype=torch.float32, device=_dev()).fill_(1.0)
        dst = torch.empty_like(src)
        for _ in range(3):
            torch.add(src, 1.0, out=dst)
        torch.cuda.synchronize()
        del src, dst

    cfg = sc.CONFIGS[args.config]
    budget = None if args.no_cpu_baseline else args.cpu_budget
    runner = {"proj": run_proj, "ffn": run_ffn_fwd, "bwd": run_bwd}[cfg.kind]
    head = runner(cfg, args, budget) if cfg.kind == "ffn" else runner(cfg, args)
    print(f"[bench] {cfg.name}: {head['ms_per_step']} ms/step", file=sys.stderr, flush=True)
    F = {"proj": lambda c: 2.0 * c.P * c.N * c.d,
         "ffn": lambda c: 2.0 * c.P * 3 * c.inter * c.d,
         "bwd": lambda c: 2.0 * c.P * 3 * c.inter * c.d}[cfg.kind](cfg)
    out = {
        "metric": METRIC,
        "value": round(F / (head["ms_per_step"] / 1e3) / 1e12, 3),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": head["ms_per_step"],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": cfg.name, "T": cfg.T, "d": cfg.d, "E": cfg.E, "top_k": cfg.k,
                   "inter": cfg.inter, "N": cfg.N, "weights": cfg.fmt_name + " group-32",
                   "variant": "fused", "weight_layout": "mfma-tiled", "seed": cfg.seed,
                   "call": {"proj": "dequant_grouped_gemm", "ffn": "moe_ffn_fwd",
                            "bwd": "moe_dx_bwd"}[cfg.kind]},
        "roofline": head.pop("roofline"),
    }
    if "cpu_baseline" in head:
        out["cpu_baseline"] = head.pop("cpu_baseline")
    out["detail"] = head
    if not args.no_sub:
        subs = {}
        for name in sc.ORDER:
            c = sc.CONFIGS[name]
            if name == cfg.name or name == "tiny_mxfp4_proj":
                continue
            r = {"proj": run_proj, "ffn": run_ffn_fwd, "bwd": run_bwd}[c.kind](c, args)
            print(f"[bench] {name}: {r['ms_per_step']} ms/step", file=sys.stderr, flush=True)
            subs[name] = r
        out["workloads"] = subs
    print(json.dumps(out), flush=True)


def main():
    ap = argparse.ArgumentParser(description=__doc__.splitlines()[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--config", default=HEADLINE)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-budget", type=float, default=15.0)
    ap.add_argument("--no-sub", action="store_true",
                    help="only the --config workload (no other workloads, no sweeps)")
    ap.add_argument("--no-sweep", action="store_true", help="skip the chunk-size sweeps")
    ap.add_argument("--calib-copy-mib", type=int, default=0,
                    help="run a plain device copy of this size first (counter calibration)")
    args = ap.parse_args()
    args.sweep = not (args.no_sweep or args.no_sub)
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: this path runs on a single MI355X "
              "(run with --gpus 1)", file=sys.stderr)
        sys.exit(2)
    run(args)


if __name__ == "__main__":
    main()
