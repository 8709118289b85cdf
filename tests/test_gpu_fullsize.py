"""GPU parity at the full workload sizes, in the launch configuration the bench
times.  Routing and permutation are compared in full (bit-exact); GEMM outputs
are compared on rows the oracle computes one by one (a seeded sample with at
least 8 routed rows of every active expert and at least 2048 rows; with
QGG_FULL_ORACLE=1 every row), and every chunk size must reproduce the fused
variant bit for bit over the whole output."""
import gc
import os

import numpy as np
import pytest
import torch

import oracle
import quantized_grouped_gemm_amd as qgg
import synth
import synth.configs as sc

from .gpu_util import (DEV, assert_close, bf16_to_f64, check_router_grads, dev_bf16,
                       dev_weights, host_u16, sync)

pytestmark = [pytest.mark.gpu, pytest.mark.timeout(900)]


def _free():
    gc.collect()
    torch.cuda.empty_cache()


def _check_routing(cfg, logits, ids, perm):
    ids_ref, gates_ref = oracle.route(logits, cfg.k)
    np.testing.assert_array_equal(ids.cpu().numpy(), ids_ref)
    ref = oracle.permute(ids_ref, cfg.E)
    for name in ("counts", "offsets", "perm", "inv_perm", "active"):
        np.testing.assert_array_equal(getattr(perm, name).cpu().numpy(), ref[name], err_msg=name)
    assert int(perm.n_active.item()) == ref["n_active"]
    return ids_ref, gates_ref, ref


# QGG_FULL_ORACLE=1 adds comparisons of every output element with the oracle
# (minutes of CPU time on the GPU host); the routine runs compare samples
FULL = os.environ.get("QGG_FULL_ORACLE", "") == "1"


def _covering_tokens(pref, T, k, seed, per_expert=8, min_rows=2048):
    """Seeded tokens whose routed pairs include at least `per_expert` rows of
    every active expert (all of them when it has fewer) and at least
    `min_rows` pairs in all; sorted, int32."""
    rng = np.random.default_rng(seed)
    chosen = np.zeros(T, bool)
    for e in pref["active"][:pref["n_active"]]:
        pairs = pref["perm"][pref["offsets"][e]:pref["offsets"][e + 1]]
        have = int(np.sum(chosen[pairs // k]))
        want = min(per_expert, pairs.size)
        if have >= want:
            continue
        free = pairs[~chosen[pairs // k]]
        pick = rng.choice(free, want - have, replace=False)
        chosen[pick // k] = True
    while chosen.sum() * k < min(min_rows, T * k):
        chosen[rng.choice(np.nonzero(~chosen)[0], 1)] = True
    return np.nonzero(chosen)[0].astype(np.int32)


def _in_slices(fn, toks, what, per=1024):
    """fn(toks) for slices of `per` tokens, concatenated along axis 0; a line
    per slice, so that minutes of oracle time still show progress."""
    outs = []
    for i in range(0, toks.size, per):
        outs.append(fn(toks[i:i + per]))
        if toks.size > per:
            print(f"  {what}: oracle tokens {i + min(per, toks.size - i)}/{toks.size}", flush=True)
    if isinstance(outs[0], tuple):
        return tuple(np.concatenate(parts, axis=0) for parts in zip(*outs))
    return np.concatenate(outs, axis=0)


def _rows_per_expert(pref, toks, k):
    slots = (toks[:, None] * k + np.arange(k)[None, :]).reshape(-1)
    rows = pref["inv_perm"][slots]
    counts = np.diff(pref["offsets"])
    per = np.bincount(np.searchsorted(pref["offsets"], rows, side="right") - 1,
                      minlength=counts.size)
    act = pref["active"][:pref["n_active"]]
    return int(np.min(np.minimum(per[act], 8) - np.minimum(counts[act], 8))), rows.size


def test_kimi_int4_gate_up_full():
    cfg = sc.CONFIGS["kimi_int4_gate_up"]
    print(f"case {cfg.name}: generating inputs", flush=True)
    logits, x = sc.router_logits(cfg), sc.activations(cfg)
    packed, scales = sc.first_weights(cfg)
    w_rows = dev_weights(cfg.fmt, packed, scales)
    w = qgg.repack(w_rows)
    xd = dev_bf16(x)
    ids, _ = qgg.moe_route(torch.from_numpy(logits).to(DEV), cfg.k)
    p, _ = qgg.expert_permute(ids, cfg.E)
    y_f = qgg.dequant_grouped_gemm(w, xd, p, cfg.T, cfg.k, qgg.FUSED, 0)
    y_c = qgg.dequant_grouped_gemm(w, xd, p, cfg.T, cfg.k, qgg.CHUNKED, cfg.chunks[0])
    y_r = qgg.dequant_grouped_gemm(w_rows, xd, p, cfg.T, cfg.k, qgg.FUSED, 0)
    sync()
    assert torch.equal(y_f.view(torch.int16), y_r.view(torch.int16))
    del w_rows, y_r
    print("case kimi: GPU done, checking", flush=True)
    ids_ref, _, pref = _check_routing(cfg, logits, ids, p)
    assert torch.equal(y_f.view(torch.int16), y_c.view(torch.int16))
    # 8 seeded rows from every active expert (every row with QGG_FULL_ORACLE=1)
    rng = np.random.default_rng(0)
    rows = []
    for e in pref["active"][:pref["n_active"]]:
        seg = np.arange(pref["offsets"][e], pref["offsets"][e + 1])
        rows.append(seg if FULL else rng.choice(seg, min(8, seg.size), replace=False))
    rows = np.sort(np.concatenate(rows))
    pairs = pref["perm"][rows]
    ref = oracle.project(cfg.fmt, packed, scales, x, (pairs // cfg.k).astype(np.int32),
                         ids_ref.reshape(-1)[pairs])
    got = host_u16(y_f[torch.from_numpy(rows).to(DEV)])
    e = assert_close(bf16_to_f64(got), ref, what="kimi int4 gate_up")
    print(f"case kimi: {rows.size} rows checked, max rel err {e:.2e}", flush=True)
    del w, xd, y_f, y_c, packed, scales
    _free()


def test_kimi_int4_gate_up_lora_full():
    """The bench workload with a rank-32 BF16 LoRA adapter on every expert."""
    cfg = sc.CONFIGS["kimi_int4_gate_up"]
    rank, alpha = 32, 0.5
    print(f"case {cfg.name} + LoRA rank {rank}: generating inputs", flush=True)
    logits, x = sc.router_logits(cfg), sc.activations(cfg)
    packed, scales = sc.first_weights(cfg)
    A = synth.normal_bf16(cfg.seed, sc.STREAM["lora_a"], (cfg.E, rank, cfg.d), std=0.02)
    B = synth.normal_bf16(cfg.seed, sc.STREAM["lora_b"], (cfg.E, cfg.N, rank), std=0.02)
    w = qgg.repack(dev_weights(cfg.fmt, packed, scales))
    xd, Ad, Bd = dev_bf16(x), dev_bf16(A), dev_bf16(B)
    ids, _ = qgg.moe_route(torch.from_numpy(logits).to(DEV), cfg.k)
    p, _ = qgg.expert_permute(ids, cfg.E)
    y_f, u_f = qgg.lora_grouped_gemm(w, Ad, Bd, alpha, xd, p, cfg.T, cfg.k, qgg.FUSED, 0)
    y_c, u_c = qgg.lora_grouped_gemm(w, Ad, Bd, alpha, xd, p, cfg.T, cfg.k, qgg.CHUNKED,
                                     cfg.chunks[0])
    sync()
    assert torch.equal(y_f.view(torch.int16), y_c.view(torch.int16))
    assert torch.equal(u_f.view(torch.int16), u_c.view(torch.int16))
    del y_c, u_c
    print("case kimi lora: GPU done, checking", flush=True)
    ids_ref, _, pref = _check_routing(cfg, logits, ids, p)
    rng = np.random.default_rng(3)
    rows = []
    for e in pref["active"][:pref["n_active"]]:
        seg = np.arange(pref["offsets"][e], pref["offsets"][e + 1])
        rows.append(rng.choice(seg, min(2, seg.size), replace=False))
    rows = np.sort(np.concatenate(rows))
    pairs = pref["perm"][rows]
    y_ref, u_ref = oracle.lora_project(cfg.fmt, packed, scales, x,
                                       (pairs // cfg.k).astype(np.int32),
                                       ids_ref.reshape(-1)[pairs], A, B, alpha, want_u=True)
    sel = torch.from_numpy(rows).to(DEV)
    assert_close(bf16_to_f64(host_u16(u_f[sel])), u_ref, what="kimi lora u")
    e = assert_close(bf16_to_f64(host_u16(y_f[sel])), y_ref, what="kimi lora y")
    print(f"case kimi lora: {rows.size} rows checked, max rel err {e:.2e}", flush=True)
    # adapter backward at the same size: two active experts' gradients and
    # their rows' dx against the oracle
    P = cfg.T * cfg.k
    dy_pairs = synth.normal_bf16(cfg.seed, sc.STREAM["dy"], (P, cfg.N))
    dyd = dev_bf16(dy_pairs[pref["perm"]])
    g = qgg.lora_grouped_gemm_bwd(Ad, Bd, alpha, xd, dyd, u_f, p, cfg.T, cfg.k)
    sync()
    sel_e = pref["active"][[0, pref["n_active"] // 2]]
    srows = np.concatenate([np.arange(pref["offsets"][e], pref["offsets"][e + 1]) for e in sel_e])
    spairs = pref["perm"][srows]
    remap = np.full(cfg.E, -1, np.int32)
    remap[sel_e] = np.arange(sel_e.size)
    dx_ref, dA_ref, dB_ref = oracle.lora_bwd(
        x, dy_pairs[spairs], (spairs // cfg.k).astype(np.int32),
        remap[ids_ref.reshape(-1)[spairs]], A[sel_e], B[sel_e], alpha)
    assert_close(bf16_to_f64(host_u16(g["dx"][torch.from_numpy(srows).to(DEV)])), dx_ref,
                 what="kimi lora dx")
    esel = torch.from_numpy(sel_e.astype(np.int64)).to(DEV)
    assert_close(g["dA"][esel].cpu().numpy().reshape(-1, cfg.d), dA_ref.reshape(-1, cfg.d),
                 what="kimi lora dA")
    assert_close(g["dB"][esel].cpu().numpy().reshape(-1, rank), dB_ref.reshape(-1, rank),
                 what="kimi lora dB")
    print(f"case kimi lora bwd: experts {sel_e.tolist()}, {srows.size} rows checked", flush=True)
    del w, xd, Ad, Bd, y_f, u_f, packed, scales, g, dyd
    _free()


_FFN_CACHE = {}


def _ffn_inputs(cfg):
    key = (cfg.T, cfg.d, cfg.E, cfg.k, cfg.inter, cfg.fmt, cfg.seed, cfg.zipf_s)
    if key not in _FFN_CACHE:
        _FFN_CACHE.clear()
        _FFN_CACHE[key] = (sc.router_logits(cfg), sc.activations(cfg), sc.first_weights(cfg),
                           sc.down_weights(cfg))
    return _FFN_CACHE[key]


@pytest.mark.parametrize("name", ["mxfp4_ffn_prefill", "int4_ffn_decode_zipf"])
def test_moe_ffn_fwd_full(name):
    cfg = sc.CONFIGS[name]
    print(f"case {cfg.name}: generating inputs", flush=True)
    logits, x, gu, dn = _ffn_inputs(cfg)
    wg = dev_weights(cfg.fmt, *gu, layout=qgg.LAYOUT_MFMA)
    wd = dev_weights(cfg.fmt, *dn, layout=qgg.LAYOUT_MFMA)
    xd, lt = dev_bf16(x), torch.from_numpy(logits).to(DEV)
    r = qgg.moe_ffn_fwd(wg, wd, xd, lt, cfg.k, qgg.FUSED, 0, save_h=True)
    sync()
    y0, h0 = host_u16(r["y"]), host_u16(r["h"])
    for chunk in cfg.chunks:
        rc = qgg.moe_ffn_fwd(wg, wd, xd, lt, cfg.k, qgg.CHUNKED, chunk, save_h=True)
        sync()
        np.testing.assert_array_equal(host_u16(rc["y"]), y0, err_msg=f"chunk {chunk}")
        np.testing.assert_array_equal(host_u16(rc["h"]), h0, err_msg=f"chunk {chunk}")
        del rc
    print(f"case {cfg.name}: GPU done, checking", flush=True)
    ids_ref, gates_ref, pref = _check_routing(cfg, logits, r["topk_ids"], r["perm"])
    if FULL or cfg.T <= 64:
        toks = np.arange(cfg.T, dtype=np.int32)
    else:
        toks = _covering_tokens(pref, cfg.T, cfg.k, seed=1)
    short, nrows = _rows_per_expert(pref, toks, cfg.k)
    assert short == 0, "the sample misses rows of an active expert"
    n_tok = toks.size
    y_ref, h_ref = _in_slices(lambda t: oracle.ffn(cfg.fmt, gu, dn, x, ids_ref, gates_ref, t,
                                                   want_h=True), toks, cfg.name)
    e = assert_close(bf16_to_f64(y0[toks]), y_ref, what=f"{cfg.name} y")
    slots = (toks[:, None] * cfg.k + np.arange(cfg.k)[None, :]).reshape(-1)
    assert_close(bf16_to_f64(h0[pref["inv_perm"][slots]]), h_ref, what=f"{cfg.name} h")
    print(f"case {cfg.name}: {n_tok} tokens ({nrows} routed rows, >= 8 per active expert) "
          f"checked, n_active {pref['n_active']}, max rel err y {e:.2e}", flush=True)
    del wg, wd, xd, lt, r
    _free()


def test_moe_dx_bwd_full():
    cfg = sc.CONFIGS["mxfp4_dx_bwd"]
    print(f"case {cfg.name}: generating inputs", flush=True)
    logits, x, gu, dn = _ffn_inputs(cfg)
    dy = sc.grad_output(cfg)
    wg = dev_weights(cfg.fmt, *gu, layout=qgg.LAYOUT_MFMA)
    wd = dev_weights(cfg.fmt, *dn, layout=qgg.LAYOUT_MFMA)
    fwd = qgg.moe_ffn_fwd(wg, wd, dev_bf16(x), torch.from_numpy(logits).to(DEV), cfg.k,
                          qgg.FUSED, 0, save_h=True)
    dyd = dev_bf16(dy)
    dx0 = host_u16(qgg.moe_dx_bwd(wg, wd, dyd, fwd["topk_gates"], fwd["perm"], fwd["h"], cfg.k,
                                  qgg.FUSED, 0))
    for chunk in cfg.chunks:
        dxc = qgg.moe_dx_bwd(wg, wd, dyd, fwd["topk_gates"], fwd["perm"], fwd["h"], cfg.k,
                             qgg.CHUNKED, chunk)
        sync()
        np.testing.assert_array_equal(host_u16(dxc), dx0, err_msg=f"chunk {chunk}")
        del dxc
        _free()
    print("case dx: GPU done, checking", flush=True)
    ids_ref, gates_ref, pref = _check_routing(cfg, logits, fwd["topk_ids"], fwd["perm"])
    toks = (np.arange(cfg.T, dtype=np.int32) if FULL
            else _covering_tokens(pref, cfg.T, cfg.k, seed=2))
    short, nrows = _rows_per_expert(pref, toks, cfg.k)
    assert short == 0, "the sample misses rows of an active expert"
    dx_ref = _in_slices(lambda t: oracle.dx(cfg.fmt, gu, dn, x, dy, ids_ref, gates_ref, t)[0],
                        toks, "dx")
    e = assert_close(bf16_to_f64(dx0[toks]), dx_ref, what="dx")
    print(f"case dx: {toks.size} tokens ({nrows} routed rows, >= 8 per active expert) checked, "
          f"max rel err {e:.2e}", flush=True)
    # router gradient, same launch configuration: dx bit-identical to the
    # plain backward, dgates / dlogits identical across variants, sampled
    # tokens against the oracle
    r = qgg.moe_router_bwd(wg, wd, dyd, fwd["topk_ids"], fwd["topk_gates"], fwd["perm"],
                           fwd["h"], cfg.k, qgg.FUSED, 0)
    sync()
    np.testing.assert_array_equal(host_u16(r["dx"]), dx0, err_msg="router_bwd dx")
    dg0, dl0 = r["dgates"].cpu().numpy(), r["dlogits"].cpu().numpy()
    del r
    rc = qgg.moe_router_bwd(wg, wd, dyd, fwd["topk_ids"], fwd["topk_gates"], fwd["perm"],
                            fwd["h"], cfg.k, qgg.CHUNKED, cfg.chunks[0], want_dx=False)
    sync()
    np.testing.assert_array_equal(rc["dgates"].cpu().numpy(), dg0)
    np.testing.assert_array_equal(rc["dlogits"].cpu().numpy(), dl0)
    del rc
    rt = toks[:8]
    dg_ref, dl_ref = oracle.router_bwd(cfg.fmt, gu, dn, x, dy, logits, ids_ref, rt)
    gates = fwd["topk_gates"].cpu().numpy()
    e = check_router_grads(dg0[rt], dl0[rt], dg_ref, dl_ref, ids_ref[rt], gates[rt], what="router")
    print(f"case router: {rt.size} tokens checked, dgates max rel err {e:.2e}", flush=True)
    del wg, wd, fwd, dyd
    _FFN_CACHE.clear()
    _free()
