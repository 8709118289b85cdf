"""GPU parity of the HIP path against the CPU oracle, at sizes the oracle
finishes in seconds (several tiles, ragged tails).  Integer and byte outputs
(routing ids, permutation, dequantized weights) must match bit for bit; GEMM
outputs must be within max relative error 2e-2 (row-RMS floor)."""
import numpy as np
import pytest
import torch

import oracle
import quantized_grouped_gemm_amd as qgg
import synth
from synth.configs import CONFIGS, STREAM, Config, scaled

from .gpu_util import (DEV, LAYOUTS, assert_close, bf16_to_f64, check_router_grads, dev_bf16,
                       dev_weights, host_u16, sync)

pytestmark = pytest.mark.gpu


def _inputs(cfg: Config):
    logits = synth.configs.router_logits(cfg)
    x = synth.configs.activations(cfg)
    w = synth.configs.first_weights(cfg)
    return logits, x, w


# ---------------------------------------------------------------- routing

ROUTE_CASES = [CONFIGS["tiny_mxfp4_proj"], CONFIGS["kimi_int4_gate_up"],
               CONFIGS["mxfp4_ffn_prefill"], CONFIGS["int4_ffn_decode_zipf"],
               scaled(CONFIGS["tiny_mxfp4_proj"], T=37, E=1000, k=32, name="wide"),
               # <= 1024 pairs: the one-workgroup ballot permutation, wide E
               scaled(CONFIGS["tiny_mxfp4_proj"], T=31, E=1000, k=32, name="wide_small")]


@pytest.mark.parametrize("cfg", ROUTE_CASES, ids=lambda c: c.name)
def test_route_and_permute_bit_exact(cfg):
    print(f"case {cfg.name} T={cfg.T} E={cfg.E} k={cfg.k}", flush=True)
    logits = synth.configs.router_logits(cfg)
    if cfg.name.startswith("wide"):
        logits[:, 3] = logits[:, 5]          # exact ties
        logits[::2, 7] = -0.0                # signed zeros tie with +0
        logits[::2, 9] = 0.0
    ids_ref, gates_ref = oracle.route(logits, cfg.k)
    lt = torch.from_numpy(logits).to(DEV)
    err = torch.zeros(1, dtype=torch.int32, device=DEV)
    ids, gates = qgg.moe_route(lt, cfg.k, err_flag=err)
    sync()
    assert int(err.item()) == 0
    np.testing.assert_array_equal(ids.cpu().numpy(), ids_ref)
    g = gates.cpu().numpy().astype(np.float64)
    assert np.max(np.abs(g - gates_ref)) <= 1e-6
    assert np.max(np.abs(g.sum(1) - 1.0)) <= 1e-6

    ref = oracle.permute(ids_ref, cfg.E)
    x = synth.normal_bf16(cfg.seed, STREAM["x"], (cfg.T, 256))
    p, x_perm = qgg.expert_permute(ids, cfg.E, x=dev_bf16(x), err_flag=err)
    sync()
    assert int(err.item()) == 0
    for name in ("counts", "offsets", "perm", "inv_perm", "active"):
        np.testing.assert_array_equal(getattr(p, name).cpu().numpy(), ref[name], err_msg=name)
    assert int(p.n_active.item()) == ref["n_active"]
    np.testing.assert_array_equal(host_u16(x_perm), x[ref["perm"] // cfg.k])


def test_permute_skewed_and_ragged():
    # every token picks the same experts; P = 4099 * 3 spans 4 segments raggedly
    T, k, E = 4099, 3, 700
    ids = np.tile(np.array([[699, 3, 0]], np.int32), (T, 1))
    ids[::7] = np.array([5, 699, 1], np.int32)
    ref = oracle.permute(ids, E)
    p, _ = qgg.expert_permute(torch.from_numpy(ids).to(DEV), E)
    sync()
    for name in ("counts", "offsets", "perm", "inv_perm", "active"):
        np.testing.assert_array_equal(getattr(p, name).cpu().numpy(), ref[name], err_msg=name)
    assert int(p.n_active.item()) == ref["n_active"] == 5


def test_route_flags_non_finite_and_permute_flags_bad_ids():
    logits = np.zeros((4, 16), np.float32)
    logits[2, 7] = np.nan
    err = torch.zeros(1, dtype=torch.int32, device=DEV)
    qgg.moe_route(torch.from_numpy(logits).to(DEV), 2, err_flag=err)
    sync()
    assert int(err.item()) & 1
    err.zero_()
    ids = torch.tensor([[0, 1], [2, 16]], dtype=torch.int32, device=DEV)
    qgg.expert_permute(ids, 16, err_flag=err)
    sync()
    assert int(err.item()) & 2


# ------------------------------------------------------------- dequantize

def _single_expert_perm():
    ids = torch.zeros((1, 1), dtype=torch.int32, device=DEV)
    p, _ = qgg.expert_permute(ids, 1)
    return p


def test_dequant_only_mxfp4_exhaustive():
    # 256 rows (one per E8M0 code) x 128 columns holding every E2M1 code
    N, K = 256, 128
    codes = np.arange(16, dtype=np.uint8)
    row = (codes[0::2] | (codes[1::2] << 4)).astype(np.uint8)
    packed = np.tile(row, (N, K // 16))[None]
    scales = np.tile(np.arange(256, dtype=np.uint8)[:, None], (1, K // 32))[None]
    w = dev_weights(1, packed, scales)
    buf = qgg.dequant_grouped_gemm(w, None, _single_expert_perm(), 1, 1, qgg.CHUNKED, 1,
                                   flags=qgg.DEQUANT_ONLY)
    sync()
    got = host_u16(buf[: N * K * 2].view(torch.bfloat16)).reshape(N, K)
    ref32 = oracle.decode(1, packed[0], scales[0])
    ref = oracle.bf16_view(ref32)
    nan = np.isnan(ref32)
    np.testing.assert_array_equal(got[~nan], ref[~nan])
    assert np.all(got[nan] == 0x7FC0)


def test_dequant_only_int4_all_bf16_scales():
    N, K = 16384, 128                      # 65536 groups = every BF16 scale pattern
    codes = np.arange(16, dtype=np.uint8)
    row = (codes[0::2] | (codes[1::2] << 4)).astype(np.uint8)
    packed = np.tile(row, (N, K // 16))[None]
    scales = np.arange(65536, dtype=np.uint32).astype(np.uint16).reshape(1, N, K // 32)
    w = dev_weights(2, packed, scales)
    buf = qgg.dequant_grouped_gemm(w, None, _single_expert_perm(), 1, 1, qgg.CHUNKED, 1,
                                   flags=qgg.DEQUANT_ONLY)
    sync()
    got = host_u16(buf[: N * K * 2].view(torch.bfloat16)).reshape(N, K)
    ref32 = oracle.decode(2, packed[0], scales[0])
    ref = oracle.bf16_view(ref32)
    nan = np.isnan(ref32)
    np.testing.assert_array_equal(got[~nan], ref[~nan])
    assert np.all((got[nan] & 0x7F80) == 0x7F80) and np.all((got[nan] & 0x7F) != 0)


@pytest.mark.parametrize("fmt", [1, 2])
def test_repack_is_the_documented_permutation(fmt):
    E, N, K = 3, 128, 256
    packed, scales = synth.qweights(4, 3, fmt, E, N, K)
    w = dev_weights(fmt, packed, scales, layout=qgg.LAYOUT_MFMA)
    sync()
    got_p = w.packed.cpu().numpy().reshape(E, N // 32, K // 64, 64, 16)
    got_s = w.scales.cpu().numpy().reshape(E, N // 32, K // 64, 64)
    if fmt == 2:
        got_s = got_s.view(np.uint16)
    for L in range(64):
        h, c = divmod(L, 32)
        rows = np.arange(N // 32) * 32 + c
        for j in range(K // 64):
            g = 2 * j + h
            np.testing.assert_array_equal(got_p[:, :, j, L, :],
                                          packed[:, rows, g * 16:(g + 1) * 16])
            np.testing.assert_array_equal(got_s[:, :, j, L], scales[:, rows, g])
    # the chunked hook decodes the tiled tensor to the same row-major BF16
    ids = torch.zeros((1, 1), dtype=torch.int32, device=DEV)
    perm1, _ = qgg.expert_permute(ids, E)
    a = qgg.dequant_grouped_gemm(dev_weights(fmt, packed, scales), None, perm1, 1, 1,
                                 qgg.CHUNKED, 1, flags=qgg.DEQUANT_ONLY)[: N * K * 2].clone()
    b = qgg.dequant_grouped_gemm(w, None, perm1, 1, 1, qgg.CHUNKED, 1,
                                 flags=qgg.DEQUANT_ONLY)[: N * K * 2].clone()
    sync()
    assert torch.equal(a, b)


# ------------------------------------------------------------ projections

PROJ_CASES = [
    CONFIGS["tiny_mxfp4_proj"],
    scaled(CONFIGS["kimi_int4_gate_up"], T=160, d=384, E=24, k=4, N=320, chunks=(5,),
           name="int4_ragged_n"),
    scaled(CONFIGS["tiny_mxfp4_proj"], T=200, d=256, E=8, k=2, N=256, name="mxfp4_mb2"),
    scaled(CONFIGS["kimi_int4_gate_up"], T=512, d=256, E=8, k=2, N=256, chunks=(3,),
           name="int4_mb4"),
    # >200 rows per expert: several 128-row tiles per expert, ragged
    scaled(CONFIGS["kimi_int4_gate_up"], T=700, d=256, E=6, k=2, N=320, chunks=(4,),
           name="int4_tall"),
    # 128-row tiles take 512-column items: one full item and a 64-column item
    # on which only the first wavefront stores
    scaled(CONFIGS["kimi_int4_gate_up"], T=600, d=256, E=3, k=1, N=576, chunks=(2,),
           name="int4_512col_ragged"),
    scaled(CONFIGS["tiny_mxfp4_proj"], T=600, d=128, E=2, k=1, N=64, chunks=(1,),
           name="mxfp4_n64_tall"),
    # decode-sized batches (33..64 tokens): one 64-row tile per expert, with
    # one and two live 32-row blocks, on four-wave workgroups
    scaled(CONFIGS["tiny_mxfp4_proj"], T=64, d=256, E=3, k=2, N=320, chunks=(2,),
           name="mxfp4_decode_tile64"),
    scaled(CONFIGS["kimi_int4_gate_up"], T=48, d=256, E=5, k=3, N=256, chunks=(2,),
           name="int4_decode_tile64"),
]


def _proj_ref(cfg, w, x, ids):
    P = cfg.T * cfg.k
    tok = np.arange(P, dtype=np.int32) // cfg.k
    return oracle.project(cfg.fmt, w[0], w[1], x, tok, ids.reshape(-1))


@pytest.mark.parametrize("cfg", PROJ_CASES, ids=lambda c: c.name)
def test_grouped_gemm_parity_and_chunk_invariance(cfg):
    print(f"case {cfg.name}", flush=True)
    logits, x, w = _inputs(cfg)
    ids_ref, _ = oracle.route(logits, cfg.k)
    ref = _proj_ref(cfg, w, x, ids_ref)
    ids, _ = qgg.moe_route(torch.from_numpy(logits).to(DEV), cfg.k)
    p, _ = qgg.expert_permute(ids, cfg.E)
    xd = dev_bf16(x)
    inv = p.inv_perm.cpu().numpy()
    outs = {}
    for layout in LAYOUTS:
        wd = dev_weights(cfg.fmt, *w, layout=layout)
        for variant, chunk in [(qgg.FUSED, 0), (qgg.CHUNKED, cfg.chunks[0]), (qgg.CHUNKED, 1),
                               (qgg.CHUNKED, 0)]:
            y = qgg.dequant_grouped_gemm(wd, xd, p, cfg.T, cfg.k, variant, chunk,
                                         flags=qgg.A_TOKENS)
            sync()
            yh = host_u16(y)
            assert_close(bf16_to_f64(yh[inv]), ref,
                         what=f"{cfg.name} layout{layout} v{variant} c{chunk}")
            outs[(layout, variant, chunk)] = yh
    base = outs[(qgg.LAYOUT_ROWS, qgg.CHUNKED, 0)]
    for key, v in outs.items():
        np.testing.assert_array_equal(v, base, err_msg=f"layout/variant/chunk {key} differs")


LORA_CASES = [(PROJ_CASES[0], 16), (PROJ_CASES[1], 48), (PROJ_CASES[3], 32),
              (PROJ_CASES[4], 128),
              # most experts get no rows: their adapter gradients must be zero
              (scaled(CONFIGS["kimi_int4_gate_up"], T=8, d=256, E=40, k=2, N=256, chunks=(4,),
                      name="int4_sparse"), 32)]


@pytest.mark.parametrize("cfg,rank", LORA_CASES, ids=lambda v: v.name if hasattr(v, "name") else str(v))
def test_lora_grouped_gemm_parity(cfg, rank):
    print(f"case {cfg.name} rank {rank}", flush=True)
    logits, x, w = _inputs(cfg)
    A = synth.normal_bf16(cfg.seed, STREAM["lora_a"], (cfg.E, rank, cfg.d), std=0.05)
    B = synth.normal_bf16(cfg.seed, STREAM["lora_b"], (cfg.E, cfg.N, rank), std=0.05)
    alpha = 0.5
    ids_ref, _ = oracle.route(logits, cfg.k)
    tok = np.arange(cfg.T * cfg.k, dtype=np.int32) // cfg.k
    y_ref, u_ref = oracle.lora_project(cfg.fmt, w[0], w[1], x, tok, ids_ref.reshape(-1), A, B,
                                       alpha, want_u=True)
    ids, _ = qgg.moe_route(torch.from_numpy(logits).to(DEV), cfg.k)
    p, _ = qgg.expert_permute(ids, cfg.E)
    xd, Ad, Bd = dev_bf16(x), dev_bf16(A), dev_bf16(B)
    inv = p.inv_perm.cpu().numpy()
    outs = {}
    for layout in LAYOUTS:
        wd = dev_weights(cfg.fmt, *w, layout=layout)
        for variant, chunk in [(qgg.FUSED, 0), (qgg.CHUNKED, cfg.chunks[0])]:
            y, u = qgg.lora_grouped_gemm(wd, Ad, Bd, alpha, xd, p, cfg.T, cfg.k, variant, chunk)
            sync()
            what = f"{cfg.name} r{rank} layout{layout} v{variant} c{chunk}"
            yh, uh = host_u16(y), host_u16(u)
            assert_close(bf16_to_f64(uh[inv]), u_ref, what=what + " u")
            assert_close(bf16_to_f64(yh[inv]), y_ref, what=what + " y")
            outs[(layout, variant, chunk)] = (yh, uh)
        if layout == qgg.LAYOUT_MFMA:
            # alpha = 0: the adapter steps add exact zeros to the base product
            y0, _ = qgg.lora_grouped_gemm(wd, Ad, Bd, 0.0, xd, p, cfg.T, cfg.k, qgg.FUSED, 0)
            yb = qgg.dequant_grouped_gemm(wd, xd, p, cfg.T, cfg.k, qgg.FUSED, 0)
            sync()
            np.testing.assert_array_equal(host_u16(y0), host_u16(yb))
    first = next(iter(outs.values()))
    for key, (yh, uh) in outs.items():
        np.testing.assert_array_equal(yh, first[0], err_msg=f"y {key} differs")
        np.testing.assert_array_equal(uh, first[1], err_msg=f"u {key} differs")


@pytest.mark.parametrize("cfg,rank", LORA_CASES, ids=lambda v: v.name if hasattr(v, "name") else str(v))
def test_lora_grouped_gemm_bwd_parity(cfg, rank):
    print(f"case {cfg.name} rank {rank} backward", flush=True)
    logits, x, w = _inputs(cfg)
    A = synth.normal_bf16(cfg.seed, STREAM["lora_a"], (cfg.E, rank, cfg.d), std=0.05)
    B = synth.normal_bf16(cfg.seed, STREAM["lora_b"], (cfg.E, cfg.N, rank), std=0.05)
    P = cfg.T * cfg.k
    dy_pairs = synth.normal_bf16(cfg.seed, STREAM["dy"], (P, cfg.N))
    alpha = 0.5
    ids_ref, _ = oracle.route(logits, cfg.k)
    tok = np.arange(P, dtype=np.int32) // cfg.k
    dx_ref, dA_ref, dB_ref = oracle.lora_bwd(x, dy_pairs, tok, ids_ref.reshape(-1), A, B, alpha)
    ids, _ = qgg.moe_route(torch.from_numpy(logits).to(DEV), cfg.k)
    p, _ = qgg.expert_permute(ids, cfg.E)
    perm, inv = p.perm.cpu().numpy(), p.inv_perm.cpu().numpy()
    xd, Ad, Bd = dev_bf16(x), dev_bf16(A), dev_bf16(B)
    wd = dev_weights(cfg.fmt, *w, layout=qgg.LAYOUT_MFMA)
    _, u = qgg.lora_grouped_gemm(wd, Ad, Bd, alpha, xd, p, cfg.T, cfg.k, qgg.FUSED, 0)
    dyd = dev_bf16(dy_pairs[perm])                      # sorted order
    g1 = qgg.lora_grouped_gemm_bwd(Ad, Bd, alpha, xd, dyd, u, p, cfg.T, cfg.k)
    g2 = qgg.lora_grouped_gemm_bwd(Ad, Bd, alpha, xd, dyd, u, p, cfg.T, cfg.k, want=("dB",))
    sync()
    what = f"{cfg.name} r{rank}"
    dx = bf16_to_f64(host_u16(g1["dx"]))[inv]
    dA, dB = g1["dA"].cpu().numpy(), g1["dB"].cpu().numpy()
    assert_close(dx, dx_ref, what=what + " dx")
    assert_close(dA.reshape(-1, cfg.d), dA_ref.reshape(-1, cfg.d), what=what + " dA")
    assert_close(dB.reshape(-1, rank), dB_ref.reshape(-1, rank), what=what + " dB")
    used = np.zeros(cfg.E, bool)
    used[ids_ref.reshape(-1)] = True
    assert np.all(dA[~used] == 0) and np.all(dB[~used] == 0)
    np.testing.assert_array_equal(g2["dB"].cpu().numpy(), dB)


def test_grouped_gemm_one_hot_rows_return_weight_columns():
    # Rows of x that are one-hot pick single weight columns, so the output is
    # the dequantized weights themselves (exactly representable in BF16).
    for fmt in (1, 2):
        E, N, K, k = 4, 256, 256, 1
        T = K
        packed, scales = synth.qweights(3, 3, fmt, E, N, K)
        x = np.zeros((T, K), np.uint16)
        x[np.arange(T), np.arange(K)] = 0x3F80
        logits = np.full((T, E), -5.0, np.float32)
        logits[:, 2] = 5.0                                   # all rows to expert 2
        ids, _ = qgg.moe_route(torch.from_numpy(logits).to(DEV), k)
        p, _ = qgg.expert_permute(ids, E)
        for layout, variant in [(lo, v) for lo in LAYOUTS for v in (qgg.FUSED, qgg.CHUNKED)]:
            wd = dev_weights(fmt, packed, scales, layout=layout)
            y = qgg.dequant_grouped_gemm(wd, dev_bf16(x), p, T, k, variant, 0)
            sync()
            got = host_u16(y)                               # row t = W[:, t]
            ref = oracle.bf16_view(oracle.decode(fmt, packed[2], scales[2]))
            # a -0 weight comes back as +0: the fp32 sum of a -0 product with +0
            # products is +0, and the two are the same value
            ref = np.where(ref == 0x8000, 0, ref).astype(np.uint16)
            assert np.count_nonzero(ref) > ref.size // 2
            np.testing.assert_array_equal(got, ref.T,
                                          err_msg=f"fmt {fmt} layout {layout} variant {variant}")


def test_grouped_gemm_exact_integer_inputs_bit_exact():
    # Integer x and MXFP4 weights with unit scale keep every partial sum exact
    # in fp32, so the GPU result equals the oracle's exact value rounded to
    # BF16, bit for bit, whatever the summation order.
    E, N, K, T, k = 6, 256, 512, 96, 2
    rng = np.random.default_rng(5)
    codes = rng.integers(0, 16, (E, N, K), dtype=np.uint8)
    packed = (codes[..., 0::2] | (codes[..., 1::2] << 4)).astype(np.uint8)
    scales = np.full((E, N, K // 32), 127, np.uint8)
    xi = rng.integers(-3, 4, (T, K)).astype(np.float32)
    x = (xi.view(np.uint32) >> 16).astype(np.uint16)
    logits = rng.standard_normal((T, E)).astype(np.float32)
    ids_ref, _ = oracle.route(logits, k)
    ref = oracle.project(1, packed, scales, x, np.arange(T * k, dtype=np.int32) // k,
                         ids_ref.reshape(-1))
    ref_bits = oracle.bf16_view(ref.astype(np.float32))
    assert np.all(ref.astype(np.float32) == ref)            # exact in fp32
    ids, _ = qgg.moe_route(torch.from_numpy(logits).to(DEV), k)
    p, _ = qgg.expert_permute(ids, E)
    inv = p.inv_perm.cpu().numpy()
    for layout, variant in [(lo, v) for lo in LAYOUTS for v in (qgg.FUSED, qgg.CHUNKED)]:
        wd = dev_weights(1, packed, scales, layout=layout)
        y = qgg.dequant_grouped_gemm(wd, dev_bf16(x), p, T, k, variant, 2)
        sync()
        np.testing.assert_array_equal(host_u16(y)[inv], ref_bits)


@pytest.mark.parametrize("fmt", [1, 2])
def test_transposed_grouped_gemm_parity(fmt):
    E, N, K, T, k = 10, 384, 512, 120, 3
    packed, scales = synth.qweights(8, 4, fmt, E, N, K)
    logits = synth.normal_f32(8, 1, (T, E))
    ids_ref, _ = oracle.route(logits, k)
    pref = oracle.permute(ids_ref, E)
    a = synth.normal_bf16(8, 5, (T * k, N))                 # sorted rows, [P][N]
    ref = oracle.project_t(fmt, packed, scales, a, ids_ref.reshape(-1)[pref["perm"]])
    ids, _ = qgg.moe_route(torch.from_numpy(logits).to(DEV), k)
    p, _ = qgg.expert_permute(ids, E)
    outs = []
    for layout, variant, chunk in [(lo, v, c) for lo in LAYOUTS
                                   for v, c in [(qgg.FUSED, 0), (qgg.CHUNKED, 4), (qgg.CHUNKED, 0)]]:
        wd = dev_weights(fmt, packed, scales, layout=layout)
        y = qgg.dequant_grouped_gemm(wd, dev_bf16(a), p, T, k, variant, chunk,
                                     flags=qgg.A_SORTED | qgg.TRANSPOSE_W)
        sync()
        outs.append(host_u16(y))
        assert_close(bf16_to_f64(outs[-1]), ref, what=f"transposed v{variant} c{chunk}")
    for o in outs[1:]:
        np.testing.assert_array_equal(o, outs[0])


# ------------------------------------------------------------------- FFN

FFN_CASES = [
    scaled(CONFIGS["mxfp4_ffn_prefill"], T=96, d=256, E=16, k=4, N=256, inter=128, chunks=(3,),
           name="mxfp4_ffn_small"),
    scaled(CONFIGS["int4_ffn_decode_zipf"], T=64, d=512, E=48, k=8, N=512, inter=256,
           chunks=(8,), name="int4_zipf_decode_small"),
    scaled(CONFIGS["mxfp4_ffn_prefill"], T=320, d=256, E=4, k=3, N=512, inter=256, chunks=(3,),
           name="mxfp4_ffn_tall"),
    scaled(CONFIGS["mxfp4_ffn_prefill"], T=300, d=256, E=8, k=2, N=256, inter=128, chunks=(4,),
           name="mxfp4_ffn_mb4"),
    # SwiGLU items of 256 intermediate columns (384 = one full + one half item)
    # and a down projection of 640 = 512 + 128 columns
    scaled(CONFIGS["mxfp4_ffn_prefill"], T=400, d=640, E=3, k=1, N=768, inter=384, chunks=(2,),
           name="mxfp4_ffn_ragged_items"),
]


def _ffn_weights(cfg):
    return synth.configs.first_weights(cfg), synth.configs.down_weights(cfg)


@pytest.mark.parametrize("cfg", FFN_CASES, ids=lambda c: c.name)
def test_moe_ffn_fwd_parity(cfg):
    print(f"case {cfg.name}", flush=True)
    logits = synth.configs.router_logits(cfg)
    x = synth.configs.activations(cfg)
    gu, dn = _ffn_weights(cfg)
    ids_ref, gates_ref = oracle.route(logits, cfg.k)
    toks = np.arange(cfg.T, dtype=np.int32)
    y_ref, h_ref = oracle.ffn(cfg.fmt, gu, dn, x, ids_ref, gates_ref, toks, want_h=True)
    lt, xd = torch.from_numpy(logits).to(DEV), dev_bf16(x)
    outs = []
    runs = [(lo, v, c) for lo in LAYOUTS for v, c in
            [(qgg.FUSED, 0), (qgg.CHUNKED, cfg.chunks[0]), (qgg.CHUNKED, 1), (qgg.CHUNKED, 0)]]
    for layout, variant, chunk in runs:
        wg = dev_weights(cfg.fmt, *gu, layout=layout)
        wd = dev_weights(cfg.fmt, *dn, layout=layout)
        r = qgg.moe_ffn_fwd(wg, wd, xd, lt, cfg.k, variant, chunk, save_h=True)
        sync()
        np.testing.assert_array_equal(r["topk_ids"].cpu().numpy(), ids_ref)
        inv = r["perm"].inv_perm.cpu().numpy()
        y = host_u16(r["y"])
        h = host_u16(r["h"])
        assert_close(bf16_to_f64(h[inv]), h_ref, what=f"{cfg.name} h v{variant} c{chunk}")
        assert_close(bf16_to_f64(y), y_ref, what=f"{cfg.name} y v{variant} c{chunk}")
        outs.append((y, h))
    for y, h in outs[1:]:
        np.testing.assert_array_equal(y, outs[0][0])
        np.testing.assert_array_equal(h, outs[0][1])


DX_CASES = [
    scaled(CONFIGS["mxfp4_dx_bwd"], T=80, d=512, E=12, k=3, N=512, inter=256, chunks=(5,),
           name="mxfp4_dx_small"),
    scaled(CONFIGS["mxfp4_dx_bwd"], T=256, d=256, E=4, k=2, N=512, inter=256, chunks=(3,),
           name="mxfp4_dx_mb4"),
    scaled(CONFIGS["int4_ffn_decode_zipf"], T=40, d=256, E=20, k=4, N=512, inter=256,
           chunks=(6,), kind="bwd", name="int4_dx_zipf"),
]


@pytest.mark.parametrize("cfg", DX_CASES, ids=lambda c: c.name)
def test_moe_dx_bwd_parity(cfg):
    print(f"case {cfg.name}", flush=True)
    logits = synth.configs.router_logits(cfg)
    x = synth.configs.activations(cfg)
    dy = synth.configs.grad_output(cfg)
    gu, dn = _ffn_weights(cfg)
    ids_ref, gates_ref = oracle.route(logits, cfg.k)
    toks = np.arange(cfg.T, dtype=np.int32)
    dx_ref, _ = oracle.dx(cfg.fmt, gu, dn, x, dy, ids_ref, gates_ref, toks)
    wg, wd = dev_weights(cfg.fmt, *gu), dev_weights(cfg.fmt, *dn)
    fwd = qgg.moe_ffn_fwd(wg, wd, dev_bf16(x), torch.from_numpy(logits).to(DEV), cfg.k,
                          qgg.FUSED, 0, save_h=True)
    outs = []
    runs = [(lo, v, c) for lo in LAYOUTS for v, c in
            [(qgg.FUSED, 0), (qgg.CHUNKED, cfg.chunks[0]), (qgg.CHUNKED, 0)]]
    for layout, variant, chunk in runs:
        wg = dev_weights(cfg.fmt, *gu, layout=layout)
        wd = dev_weights(cfg.fmt, *dn, layout=layout)
        dx = qgg.moe_dx_bwd(wg, wd, dev_bf16(dy), fwd["topk_gates"], fwd["perm"], fwd["h"],
                            cfg.k, variant, chunk)
        sync()
        outs.append(host_u16(dx))
        assert_close(bf16_to_f64(outs[-1]), dx_ref, what=f"{cfg.name} dx v{variant} c{chunk}")
    for o in outs[1:]:
        np.testing.assert_array_equal(o, outs[0])


ROUTER_CASES = DX_CASES + [
    scaled(CONFIGS["mxfp4_dx_bwd"], T=64, d=256, E=6, k=1, N=512, inter=256, chunks=(4,),
           name="mxfp4_router_k1"),
]


@pytest.mark.parametrize("cfg", ROUTER_CASES, ids=lambda c: c.name)
def test_moe_router_bwd_parity(cfg):
    print(f"case {cfg.name}", flush=True)
    logits = synth.configs.router_logits(cfg)
    x = synth.configs.activations(cfg)
    dy = synth.configs.grad_output(cfg)
    gu, dn = _ffn_weights(cfg)
    ids_ref, gates_ref = oracle.route(logits, cfg.k)
    toks = np.arange(cfg.T, dtype=np.int32)
    dg_ref, dl_ref = oracle.router_bwd(cfg.fmt, gu, dn, x, dy, logits, ids_ref, toks)
    wg, wd = dev_weights(cfg.fmt, *gu), dev_weights(cfg.fmt, *dn)
    fwd = qgg.moe_ffn_fwd(wg, wd, dev_bf16(x), torch.from_numpy(logits).to(DEV), cfg.k,
                          qgg.FUSED, 0, save_h=True)
    dyd = dev_bf16(dy)
    dx_plain = host_u16(qgg.moe_dx_bwd(wg, wd, dyd, fwd["topk_gates"], fwd["perm"], fwd["h"],
                                       cfg.k, qgg.FUSED, 0))
    gates = fwd["topk_gates"].cpu().numpy()
    outs = []
    runs = [(lo, v, c, want_dx) for lo in LAYOUTS for v, c in
            [(qgg.FUSED, 0), (qgg.CHUNKED, cfg.chunks[0])] for want_dx in (True, False)]
    for layout, variant, chunk, want_dx in runs:
        wg = dev_weights(cfg.fmt, *gu, layout=layout)
        wd = dev_weights(cfg.fmt, *dn, layout=layout)
        r = qgg.moe_router_bwd(wg, wd, dyd, fwd["topk_ids"], fwd["topk_gates"], fwd["perm"],
                               fwd["h"], cfg.k, variant, chunk, want_dx=want_dx)
        sync()
        what = f"{cfg.name} v{variant} c{chunk} dx{int(want_dx)}"
        dg, dl = r["dgates"].cpu().numpy(), r["dlogits"].cpu().numpy()
        check_router_grads(dg, dl, dg_ref, dl_ref, ids_ref, gates, what=what)
        if cfg.k == 1:
            assert np.all(dl == 0.0), f"{what}: k = 1 leaves the gate constant"
        if want_dx:
            np.testing.assert_array_equal(host_u16(r["dx"]), dx_plain, err_msg=what)
        outs.append((dg, dl))
    for dg, dl in outs[1:]:
        np.testing.assert_array_equal(dg, outs[0][0])
        np.testing.assert_array_equal(dl, outs[0][1])


def test_router_bwd_ignores_pairs_the_permutation_dropped():
    """An expert id outside [0, E) is flagged by expert_permute and its pair is
    dropped from the sort (inv_perm -1).  The router backward must then read
    no partial sums for that pair: its dgate is 0, every other token's
    gradients are those of the same call without the bad id, bit for bit, and
    the token's other experts get the kept-softmax backward with the dropped
    pair's dg = 0."""
    cfg = scaled(CONFIGS["mxfp4_dx_bwd"], T=64, d=256, E=6, k=2, N=512, inter=256,
                 chunks=(4,), name="router_dropped_pair")
    logits = synth.configs.router_logits(cfg)
    x = synth.configs.activations(cfg)
    dy = synth.configs.grad_output(cfg)
    gu, dn = _ffn_weights(cfg)
    wg, wd = dev_weights(cfg.fmt, *gu), dev_weights(cfg.fmt, *dn)
    xd, dyd = dev_bf16(x), dev_bf16(dy)
    ids, gates = qgg.moe_route(torch.from_numpy(logits).to(DEV), cfg.k)
    t0, j0 = 17, 1
    bad_ids = ids.clone()
    bad_ids[t0, j0] = cfg.E + 5
    flag = torch.zeros(1, dtype=torch.int32, device=DEV)
    runs = {}
    for name, rid, fl in (("good", ids, None), ("bad", bad_ids, flag)):
        p, _ = qgg.expert_permute(rid, cfg.E, err_flag=fl)
        # h in this permutation's sorted order (the gate_up projection)
        h = qgg.dequant_grouped_gemm(wg, xd, p, cfg.T, cfg.k, qgg.FUSED, 0)
        for variant, chunk in ((qgg.FUSED, 0), (qgg.CHUNKED, cfg.chunks[0])):
            r = qgg.moe_router_bwd(wg, wd, dyd, rid, gates, p, h, cfg.k, variant, chunk)
            sync()
            runs[(name, variant)] = (r["dgates"].cpu().numpy(), r["dlogits"].cpu().numpy())
    assert int(flag.item()) & 2, "expert_permute did not flag the bad id"
    g = gates.cpu().numpy().astype(np.float64)
    idn = ids.cpu().numpy()
    dg_good, dl_good = runs[("good", qgg.FUSED)]
    for variant in (qgg.FUSED, qgg.CHUNKED):
        dg, dl = runs[("bad", variant)]
        assert np.all(np.isfinite(dg)) and np.all(np.isfinite(dl))
        assert dg[t0, j0] == 0.0
        other = np.arange(cfg.T) != t0
        np.testing.assert_array_equal(dg[other], dg_good[other])
        np.testing.assert_array_equal(dl[other], dl_good[other])
        np.testing.assert_array_equal(dg[t0, :j0], dg_good[t0, :j0])
        np.testing.assert_array_equal(dg[t0, j0 + 1:], dg_good[t0, j0 + 1:])
        d = dg_good[t0].astype(np.float64)
        d[j0] = 0.0
        want = g[t0] * (d - np.sum(g[t0] * d))
        kept = [j for j in range(cfg.k) if j != j0]
        got = dl[t0, idn[t0, kept]]
        np.testing.assert_allclose(got, want[kept], rtol=1e-5,
                                   atol=1e-6 * np.max(np.abs(want)))
        mask = np.ones(cfg.E, bool)
        mask[idn[t0, kept]] = False
        assert np.all(dl[t0, mask] == 0.0)


def _random_shapes(seed, n):
    """Seeded shapes within the documented limits: ragged expert groups, k up
    to 8, K a multiple of 128, N of 64, and both weight formats."""
    rng = np.random.default_rng(seed)
    out = []
    for i in range(n):
        fmt = int(rng.integers(1, 3))
        E = int(rng.integers(1, 40))
        k = int(rng.integers(1, min(E, 8) + 1))
        T = int(rng.integers(1, 300))
        d = 128 * int(rng.integers(1, 5))
        N = 64 * int(rng.integers(1, 9))
        out.append(scaled(CONFIGS["tiny_mxfp4_proj"], T=T, d=d, E=E, k=k, N=N, fmt=fmt,
                          seed=100 + i, chunks=(int(rng.integers(1, E + 1)),),
                          name=f"rand{i}_f{fmt}_T{T}_E{E}_k{k}_d{d}_N{N}"))
    return out


@pytest.mark.parametrize("cfg", _random_shapes(7, 8), ids=lambda c: c.name)
def test_grouped_gemm_random_shapes(cfg):
    print(f"case {cfg.name}", flush=True)
    logits, x, w = _inputs(cfg)
    ids_ref, _ = oracle.route(logits, cfg.k)
    ref = _proj_ref(cfg, w, x, ids_ref)
    ids, _ = qgg.moe_route(torch.from_numpy(logits).to(DEV), cfg.k)
    p, _ = qgg.expert_permute(ids, cfg.E)
    np.testing.assert_array_equal(ids.cpu().numpy(), ids_ref)
    xd = dev_bf16(x)
    inv = p.inv_perm.cpu().numpy()
    wd = dev_weights(cfg.fmt, *w, layout=qgg.LAYOUT_MFMA)
    yf = host_u16(qgg.dequant_grouped_gemm(wd, xd, p, cfg.T, cfg.k, qgg.FUSED, 0))
    yc = host_u16(qgg.dequant_grouped_gemm(wd, xd, p, cfg.T, cfg.k, qgg.CHUNKED, cfg.chunks[0]))
    sync()
    assert_close(bf16_to_f64(yf[inv]), ref, what=cfg.name)
    np.testing.assert_array_equal(yc, yf)


def _random_ffn_shapes(seed, n):
    rng = np.random.default_rng(seed)
    out = []
    for i in range(n):
        fmt = int(rng.integers(1, 3))
        E = int(rng.integers(2, 24))
        k = int(rng.integers(1, min(E, 6) + 1))
        T = int(rng.integers(1, 160))
        d = 256 * int(rng.integers(1, 3))
        inter = 256 * int(rng.integers(1, 3))
        out.append(scaled(CONFIGS["mxfp4_ffn_prefill"], T=T, d=d, E=E, k=k, N=2 * inter,
                          inter=inter, fmt=fmt, seed=200 + i,
                          chunks=(int(rng.integers(1, E + 1)),),
                          name=f"rffn{i}_f{fmt}_T{T}_E{E}_k{k}_d{d}_I{inter}"))
    return out


@pytest.mark.parametrize("cfg", _random_ffn_shapes(11, 4), ids=lambda c: c.name)
def test_ffn_and_dx_random_shapes(cfg):
    print(f"case {cfg.name}", flush=True)
    logits = synth.configs.router_logits(cfg)
    x = synth.configs.activations(cfg)
    dy = synth.configs.grad_output(cfg)
    gu, dn = _ffn_weights(cfg)
    ids_ref, gates_ref = oracle.route(logits, cfg.k)
    toks = np.arange(cfg.T, dtype=np.int32)
    y_ref, _ = oracle.ffn(cfg.fmt, gu, dn, x, ids_ref, gates_ref, toks)
    dx_ref, _ = oracle.dx(cfg.fmt, gu, dn, x, dy, ids_ref, gates_ref, toks)
    wg = dev_weights(cfg.fmt, *gu, layout=qgg.LAYOUT_MFMA)
    wd = dev_weights(cfg.fmt, *dn, layout=qgg.LAYOUT_MFMA)
    lt, xd, dyd = torch.from_numpy(logits).to(DEV), dev_bf16(x), dev_bf16(dy)
    outs = []
    for variant, chunk in [(qgg.FUSED, 0), (qgg.CHUNKED, cfg.chunks[0])]:
        r = qgg.moe_ffn_fwd(wg, wd, xd, lt, cfg.k, variant, chunk, save_h=True)
        dx = qgg.moe_dx_bwd(wg, wd, dyd, r["topk_gates"], r["perm"], r["h"], cfg.k, variant, chunk)
        sync()
        y, dxh = host_u16(r["y"]), host_u16(dx)
        assert_close(bf16_to_f64(y), y_ref, what=f"{cfg.name} y v{variant}")
        assert_close(bf16_to_f64(dxh), dx_ref, what=f"{cfg.name} dx v{variant}")
        outs.append((y, dxh))
    np.testing.assert_array_equal(outs[0][0], outs[1][0])
    np.testing.assert_array_equal(outs[0][1], outs[1][1])


FFN_LORA_CASES = [(FFN_CASES[0], 16), (FFN_CASES[2], 32),
                  (scaled(CONFIGS["int4_ffn_decode_zipf"], T=40, d=256, E=20, k=4, N=512,
                          inter=256, chunks=(6,), name="int4_ffn_zipf_lora"), 48)]


@pytest.mark.parametrize("cfg,rank", FFN_LORA_CASES,
                         ids=lambda v: v.name if hasattr(v, "name") else str(v))
def test_moe_ffn_fwd_lora_parity(cfg, rank):
    print(f"case {cfg.name} rank {rank}", flush=True)
    logits = synth.configs.router_logits(cfg)
    x = synth.configs.activations(cfg)
    gu, dn = _ffn_weights(cfg)
    I = cfg.inter
    Agu = synth.normal_bf16(cfg.seed, STREAM["lora_a"], (cfg.E, rank, cfg.d), std=0.05)
    Bgu = synth.normal_bf16(cfg.seed, STREAM["lora_b"], (cfg.E, 2 * I, rank), std=0.05)
    Adn = synth.normal_bf16(cfg.seed + 1, STREAM["lora_a"], (cfg.E, rank, I), std=0.05)
    Bdn = synth.normal_bf16(cfg.seed + 1, STREAM["lora_b"], (cfg.E, cfg.d, rank), std=0.05)
    ids_ref, gates_ref = oracle.route(logits, cfg.k)
    toks = np.arange(cfg.T, dtype=np.int32)
    wg = dev_weights(cfg.fmt, *gu, layout=qgg.LAYOUT_MFMA)
    wd = dev_weights(cfg.fmt, *dn, layout=qgg.LAYOUT_MFMA)
    lt, xd = torch.from_numpy(logits).to(DEV), dev_bf16(x)
    agu = (dev_bf16(Agu), dev_bf16(Bgu), 0.5)
    adn = (dev_bf16(Adn), dev_bf16(Bdn), 0.75)
    for which, (lg, ld) in {"both": (agu, adn), "gate_up": (agu, None),
                            "down": (None, adn)}.items():
        ref = oracle.ffn_lora(cfg.fmt, gu, dn, x, ids_ref, gates_ref, toks,
                              (Agu, Bgu) if lg else None, (Adn, Bdn) if ld else None, 0.5, 0.75)
        outs = []
        for variant, chunk in [(qgg.FUSED, 0), (qgg.CHUNKED, cfg.chunks[0])]:
            r = qgg.moe_ffn_fwd_lora(wg, wd, lg, ld, xd, lt, cfg.k, variant, chunk)
            sync()
            y = host_u16(r["y"])
            assert_close(bf16_to_f64(y), ref, what=f"{cfg.name} r{rank} {which} v{variant}")
            outs.append(y)
        np.testing.assert_array_equal(outs[0], outs[1])
    # zero scales: the adapters add exact zeros to the base FFN
    r0 = qgg.moe_ffn_fwd_lora(wg, wd, (agu[0], agu[1], 0.0), (adn[0], adn[1], 0.0), xd, lt,
                              cfg.k, qgg.FUSED, 0)
    rb = qgg.moe_ffn_fwd(wg, wd, xd, lt, cfg.k, qgg.FUSED, 0)
    sync()
    np.testing.assert_array_equal(host_u16(r0["y"]), host_u16(rb["y"]))


FFN_LORA_BWD_CASES = [
    (DX_CASES[0], 16), (DX_CASES[1], 32), (DX_CASES[2], 48),
    # 32 routed pairs over 40 experts: most experts have no rows
    (scaled(CONFIGS["int4_ffn_decode_zipf"], T=16, d=256, E=40, k=2, N=512, inter=256,
            chunks=(4,), kind="bwd", name="int4_lora_bwd_sparse"), 16),
]


GRAD_NORM_TOL = 1e-2   # per expert, ||got - ref||_F / ||ref||_F
GRAD_MAX_TOL = 5e-2    # per element, floor = RMS of the expert's gradient matrix


def _grad_close(got, ref, what):
    """Adapter weight gradients [E][rows][cols] against the oracle.  Each
    entry is a sum over the expert's routed rows of products whose factors
    carry the BF16 rounding of the base weights (an INT4 q*s is rounded once)
    and of the stored h, dH and du; its error therefore scales with the
    expert's typical gradient entry, not with that entry (which can be small
    by cancellation).  A CPU model of exactly those rounding points reproduces
    the kernels' error to three digits and puts the worst test case at 0.47 %
    normwise and 3.2 % elementwise under the expert-wide floor (1.6-2.0 % of it
    from the weights' BF16 rounding alone), while a dropped term, a missing
    gate or a wrong scale moves the normwise error to 23-980 %.  Experts
    without rows must be exact zeros."""
    got = np.asarray(got, np.float64)
    assert np.all(np.isfinite(got)), f"{what}: non-finite"
    zero = np.all(ref.reshape(ref.shape[0], -1) == 0, axis=1)
    assert np.all(got[zero] == 0), f"{what}: nonzero gradient for an expert with no rows"
    worst_n = worst_m = 0.0
    for e in np.nonzero(~zero)[0]:
        nrm = float(np.linalg.norm(got[e] - ref[e]) / np.linalg.norm(ref[e]))
        floor = float(np.sqrt(np.mean(ref[e] ** 2)))
        mx = float(np.max(np.abs(got[e] - ref[e]) / np.maximum(np.abs(ref[e]), floor)))
        worst_n, worst_m = max(worst_n, nrm), max(worst_m, mx)
    assert worst_n <= GRAD_NORM_TOL, f"{what}: normwise err {worst_n:.3e} > {GRAD_NORM_TOL}"
    assert worst_m <= GRAD_MAX_TOL, f"{what}: max rel err {worst_m:.3e} > {GRAD_MAX_TOL}"
    return worst_n, worst_m


@pytest.mark.parametrize("cfg,rank", FFN_LORA_BWD_CASES,
                         ids=lambda v: v.name if hasattr(v, "name") else str(v))
def test_moe_ffn_bwd_lora_parity(cfg, rank):
    """The FFN adapter backward against the oracle: dX through the frozen base
    and both adapters, and both adapters' weight gradients; both adapters, each
    alone, both variants (bit-identical), both weight layouts."""
    print(f"case {cfg.name} rank {rank}", flush=True)
    logits = synth.configs.router_logits(cfg)
    x = synth.configs.activations(cfg)
    dy = synth.configs.grad_output(cfg)
    gu, dn = _ffn_weights(cfg)
    I = cfg.inter
    Agu = synth.normal_bf16(cfg.seed, STREAM["lora_a"], (cfg.E, rank, cfg.d), std=0.05)
    Bgu = synth.normal_bf16(cfg.seed, STREAM["lora_b"], (cfg.E, 2 * I, rank), std=0.05)
    Adn = synth.normal_bf16(cfg.seed + 1, STREAM["lora_a"], (cfg.E, rank, I), std=0.05)
    Bdn = synth.normal_bf16(cfg.seed + 1, STREAM["lora_b"], (cfg.E, cfg.d, rank), std=0.05)
    ids_ref, gates_ref = oracle.route(logits, cfg.k)
    toks = np.arange(cfg.T, dtype=np.int32)
    lt, xd, dyd = torch.from_numpy(logits).to(DEV), dev_bf16(x), dev_bf16(dy)
    agu = (dev_bf16(Agu), dev_bf16(Bgu), 0.5)
    adn = (dev_bf16(Adn), dev_bf16(Bdn), 0.75)
    for which, (lg, ld) in {"both": (agu, adn), "gate_up": (agu, None),
                            "down": (None, adn)}.items():
        ref = oracle.ffn_lora_bwd(cfg.fmt, gu, dn, x, dy, ids_ref, gates_ref, toks,
                                  (Agu, Bgu, 0.5) if lg else None,
                                  (Adn, Bdn, 0.75) if ld else None)
        outs = []
        for layout in LAYOUTS:
            wg = dev_weights(cfg.fmt, *gu, layout=layout)
            wd = dev_weights(cfg.fmt, *dn, layout=layout)
            fwd = qgg.moe_ffn_fwd_lora(wg, wd, lg, ld, xd, lt, cfg.k, qgg.FUSED, 0, save_h=True)
            for variant, chunk in [(qgg.FUSED, 0), (qgg.CHUNKED, cfg.chunks[0])]:
                g = qgg.moe_ffn_bwd_lora(wg, wd, lg, ld, xd, dyd, fwd["topk_gates"], fwd["perm"],
                                         fwd["h"], fwd["u_gate_up"], fwd["u_down"], cfg.k,
                                         variant, chunk)
                sync()
                what = f"{cfg.name} r{rank} {which} L{layout} v{variant}"
                dxg = host_u16(g["dx"])
                assert_close(bf16_to_f64(dxg), ref["dx"], what=what + " dx")
                got = {"dx": dxg}
                for name, rname in (("dA_gate_up", "dA_gu"), ("dB_gate_up", "dB_gu"),
                                    ("dA_down", "dA_dn"), ("dB_down", "dB_dn")):
                    if ref[rname] is None:
                        assert g[name] is None
                        continue
                    got[name] = g[name].cpu().numpy()
                    _grad_close(got[name], ref[rname], f"{what} {name}")
                outs.append(got)
        for o in outs[1:]:
            for name in o:
                np.testing.assert_array_equal(o[name], outs[0][name], err_msg=name)
    # zero scales: dx is the frozen-base backward, bit for bit
    wg = dev_weights(cfg.fmt, *gu, layout=qgg.LAYOUT_MFMA)
    wd = dev_weights(cfg.fmt, *dn, layout=qgg.LAYOUT_MFMA)
    z = ((agu[0], agu[1], 0.0), (adn[0], adn[1], 0.0))
    fwd = qgg.moe_ffn_fwd_lora(wg, wd, z[0], z[1], xd, lt, cfg.k, qgg.FUSED, 0, save_h=True)
    g = qgg.moe_ffn_bwd_lora(wg, wd, z[0], z[1], xd, dyd, fwd["topk_gates"], fwd["perm"],
                             fwd["h"], fwd["u_gate_up"], fwd["u_down"], cfg.k, qgg.FUSED, 0)
    base = qgg.moe_dx_bwd(wg, wd, dyd, fwd["topk_gates"], fwd["perm"], fwd["h"], cfg.k,
                          qgg.FUSED, 0)
    sync()
    np.testing.assert_array_equal(host_u16(g["dx"]), host_u16(base))
    for name in ("dA_gate_up", "dA_down", "dB_gate_up", "dB_down"):
        assert torch.all(g[name] == 0), name


def test_empty_batch_every_entry_point():
    """T = 0: every call succeeds; the adapter gradients come back as exact zeros."""
    print("case empty batch", flush=True)
    E, d, inter, k, rank = 6, 256, 256, 2, 16
    logits = torch.zeros((0, E), dtype=torch.float32, device=DEV)
    x = torch.zeros((0, d), dtype=torch.bfloat16, device=DEV)
    ids, gates = qgg.moe_route(logits, k)
    p, _ = qgg.expert_permute(ids, E)
    sync()
    assert p.counts.cpu().numpy().tolist() == [0] * E and int(p.n_active.item()) == 0
    gu = dev_weights(2, *synth.qweights(0, 3, 2, E, 2 * inter, d), layout=qgg.LAYOUT_MFMA)
    dn = dev_weights(2, *synth.qweights(0, 4, 2, E, d, inter), layout=qgg.LAYOUT_MFMA)
    y = qgg.dequant_grouped_gemm(gu, x, p, 0, k)
    assert y.shape == (0, 2 * inter)
    for variant, chunk in [(qgg.FUSED, 0), (qgg.CHUNKED, 2)]:
        r = qgg.moe_ffn_fwd(gu, dn, x, logits, k, variant, chunk, save_h=True)
        assert r["y"].shape == (0, d)
        dx = qgg.moe_dx_bwd(gu, dn, x, r["topk_gates"], r["perm"], r["h"], k, variant, chunk)
        g = qgg.moe_router_bwd(gu, dn, x, r["topk_ids"], r["topk_gates"], r["perm"], r["h"], k,
                               variant, chunk)
        assert dx.shape == (0, d) and g["dlogits"].shape == (0, E)
    A = dev_bf16(synth.normal_bf16(0, STREAM["lora_a"], (E, rank, d)))
    B = dev_bf16(synth.normal_bf16(0, STREAM["lora_b"], (E, 2 * inter, rank)))
    yl, u = qgg.lora_grouped_gemm(gu, A, B, 0.5, x, p, 0, k)
    dy = torch.zeros((0, 2 * inter), dtype=torch.bfloat16, device=DEV)
    gl = qgg.lora_grouped_gemm_bwd(A, B, 0.5, x, dy, u, p, 0, k)
    sync()
    assert yl.shape == (0, 2 * inter) and gl["dx"].shape == (0, d)
    assert torch.count_nonzero(gl["dA"]).item() == 0
    assert torch.count_nonzero(gl["dB"]).item() == 0


def test_repeat_runs_bit_identical_and_outputs_fully_written():
    cfg = FFN_CASES[0]
    logits = synth.configs.router_logits(cfg)
    x = synth.configs.activations(cfg)
    gu, dn = _ffn_weights(cfg)
    wg, wd = dev_weights(cfg.fmt, *gu), dev_weights(cfg.fmt, *dn)
    lt, xd = torch.from_numpy(logits).to(DEV), dev_bf16(x)
    ws = qgg.Workspace()
    nb, _ = qgg.workspace_bytes(qgg.CALL_FFN_FWD, cfg.T, cfg.d, cfg.E, cfg.k, cfg.inter,
                                qgg.FUSED, 0)
    ws.get(nb, torch.device(DEV)).fill_(0xFF)               # NaN-poison the workspace
    r1 = qgg.moe_ffn_fwd(wg, wd, xd, lt, cfg.k, qgg.FUSED, 0, save_h=True, ws=ws)
    r2 = qgg.moe_ffn_fwd(wg, wd, xd, lt, cfg.k, qgg.FUSED, 0, save_h=True, ws=ws)
    sync()
    assert torch.isfinite(r1["y"].float()).all() and torch.isfinite(r1["h"].float()).all()
    assert torch.equal(r1["y"].view(torch.int16), r2["y"].view(torch.int16))
    assert torch.equal(r1["h"].view(torch.int16), r2["h"].view(torch.int16))
