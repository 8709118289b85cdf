"""The allocation-free FFN forward (library-owned static scratch) against the
workspace entry point it shares its kernels with: identical outputs, bit for
bit, over two calls in a row (the second smaller, so it runs on what the
first left in the scratch), both variants; a call larger than the scratch is
refused before any launch."""
import numpy as np
import pytest
import torch

import quantized_grouped_gemm_amd as qgg
import synth.configs as sc

from .gpu_util import DEV, dev_bf16, dev_weights, host_u16, sync

pytestmark = pytest.mark.gpu


def _decode_case(T):
    # decode-shaped, Zipf-skewed routing, INT4 weights
    return sc.scaled(sc.CONFIGS["int4_ffn_decode_zipf"], T=T, d=1024, E=48, k=8, N=1024,
                     inter=512, name=f"noalloc_T{T}")


def _outputs(r):
    return [host_u16(r["y"]), host_u16(r["h"]), r["topk_ids"].cpu().numpy(),
            r["topk_gates"].cpu().numpy()] + [getattr(r["perm"], f).cpu().numpy() for f in
                                              ("counts", "offsets", "perm", "inv_perm",
                                               "active", "n_active")]


def test_noalloc_ffn_matches_workspace_entry_point():
    base = _decode_case(64)
    gu, dn = sc.first_weights(base), sc.down_weights(base)
    wg = dev_weights(base.fmt, *gu, layout=qgg.LAYOUT_MFMA)
    wd = dev_weights(base.fmt, *dn, layout=qgg.LAYOUT_MFMA)
    for T in (64, 16):
        cfg = _decode_case(T)
        x, lt = dev_bf16(sc.activations(cfg)), torch.from_numpy(sc.router_logits(cfg)).to(DEV)
        for variant, chunk in ((qgg.FUSED, 0), (qgg.CHUNKED, 4)):
            print(f"case T={T} variant={variant} chunk={chunk}", flush=True)
            ref = qgg.moe_ffn_fwd(wg, wd, x, lt, cfg.k, variant, chunk, save_h=True)
            got = qgg.moe_ffn_fwd_noalloc(wg, wd, x, lt, cfg.k, variant, chunk, save_h=True)
            sync()
            for a, b in zip(_outputs(got), _outputs(ref)):
                np.testing.assert_array_equal(a, b)


def test_noalloc_refuses_calls_larger_than_its_scratch():
    cfg = sc.scaled(_decode_case(64), T=4096)
    total, _ = qgg.workspace_bytes(qgg.CALL_FFN_FWD, cfg.T, cfg.d, cfg.E, cfg.k, cfg.inter,
                                   qgg.FUSED, 0)
    assert total > qgg.STATIC_SCRATCH_BYTES
    gu, dn = sc.first_weights(_decode_case(64)), sc.down_weights(_decode_case(64))
    wg, wd = dev_weights(cfg.fmt, *gu), dev_weights(cfg.fmt, *dn)
    x = torch.zeros((cfg.T, cfg.d), dtype=torch.bfloat16, device=DEV)
    lt = torch.zeros((cfg.T, cfg.E), dtype=torch.float32, device=DEV)
    with pytest.raises(qgg.QggError, match="workspace too small"):
        qgg.moe_ffn_fwd_noalloc(wg, wd, x, lt, cfg.k, qgg.FUSED, 0)
