"""Pins for the CPU oracle and the input generator (CPU only).

Each test checks the oracle against something other than itself: published
known-answer vectors, the bit-level definitions of the number formats, library
routines (numpy float64 matmul, Python's stable sort, torch's BF16 cast,
scipy's softmax and normal quantile), brute force on tiny inputs, closed forms
and finite differences.
"""
import math
import os

import numpy as np
import pytest
import torch
from scipy import special

import oracle
import synth
from quantized_grouped_gemm_amd import accounting

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _f32_bits(a):
    return np.ascontiguousarray(a, np.float32).view(np.uint32)


# ----------------------------------------------------------------- generator

def test_philox_known_answers():
    with open(os.path.join(GOLDEN, "philox4x32_10_kat.txt")) as f:
        rows = [ln.split() for ln in f if ln.strip() and not ln.startswith("#")]
    assert len(rows) == 3
    for r in rows:
        v = [int(t, 16) for t in r]
        out = synth.philox4x32_10(v[0:4], v[4:6])
        assert out.tolist() == v[6:10]


def test_normal_quantile_table_matches_library():
    q = synth.quantile_table().astype(np.float64)
    ref = special.ndtri((np.arange(65536) + 0.5) / 65536.0)
    np.testing.assert_allclose(q, ref, rtol=2e-7, atol=1e-7)
    assert np.all(np.diff(q) > 0)
    np.testing.assert_array_equal(q, -q[::-1])


def test_generator_subrange_reproduces():
    p_all, s_all = synth.qweights(7, 3, 1, 4, 64, 128)
    p_sub, s_sub = synth.qweights(7, 3, 1, 4, 64, 128, e0=2, e1=3)
    np.testing.assert_array_equal(p_all[2:3], p_sub)
    np.testing.assert_array_equal(s_all[2:3], s_sub)
    x1 = synth.normal_bf16(1, 2, (16, 64))
    x2 = synth.normal_bf16(1, 2, (16, 64))
    np.testing.assert_array_equal(x1, x2)
    assert not np.array_equal(x1, synth.normal_bf16(2, 2, (16, 64)))


def _e2m1_bits_value(code):
    """E2M1 by its bit fields: sign b3, exponent b2..b1 (bias 1), mantissa b0."""
    s = -1.0 if code & 8 else 1.0
    e = (code >> 1) & 3
    m = code & 1
    if e == 0:
        return s * m * 0.5
    return s * 2.0 ** (e - 1) * (1.0 + m / 2.0)


def test_mxfp4_encoder_grid_ties_and_exponent():
    # Grid values of a group whose amax is 6 (floor(log2 6) - 2 = 0, scale 1)
    # round-trip to their own codes.
    grid = [0, .5, 1, 1.5, 2, 3, 4, 6]
    w = np.array(grid + [-g for g in grid] + [0.0] * 16, np.float32)
    w[16:] = 0.0
    w[16] = 6.0
    nib, sc = synth.encode_mxfp4_group(w)
    codes = np.stack([nib & 15, nib >> 4], 1).reshape(-1)
    assert sc == 127
    for i, v in enumerate(w[:16]):
        assert _e2m1_bits_value(int(codes[i])) == v
    # Ties go to the even code: .25->0, .75->1, 1.25->1, 1.75->2, 2.5->2, 3.5->4, 5->4.
    ties = [(0.25, 0.0), (0.75, 1.0), (1.25, 1.0), (1.75, 2.0), (2.5, 2.0), (3.5, 4.0), (5.0, 4.0)]
    w = np.zeros(32, np.float32)
    w[0] = 6.0
    for i, (v, _) in enumerate(ties):
        w[1 + i] = v
        w[9 + i] = -v
    w[20] = 7.9  # saturates to 6 (amax stays 7.9 -> floor(log2) = 2 -> scale 1)
    w[0] = 7.9
    nib, sc = synth.encode_mxfp4_group(w)
    codes = np.stack([nib & 15, nib >> 4], 1).reshape(-1)
    assert sc == 127
    for i, (_, r) in enumerate(ties):
        assert _e2m1_bits_value(int(codes[1 + i])) == r
        assert _e2m1_bits_value(int(codes[9 + i])) == -r
        assert codes[9 + i] & 8
    assert _e2m1_bits_value(int(codes[20])) == 6.0
    # Negative values that round to zero keep their sign (code 8).
    w = np.zeros(32, np.float32)
    w[0], w[1] = 1.0, -0.01
    nib, sc = synth.encode_mxfp4_group(w)
    assert (nib[0] >> 4) == 8
    # Shared exponent = floor(log2(amax)) - 2 on values where log2 is unambiguous.
    for amax in [1.0, 1.999, 2.0, 0.0625, 0.05, 3e-3, 100.0, 2.0 ** -120]:
        w = np.zeros(32, np.float32)
        w[5] = amax
        _, sc = synth.encode_mxfp4_group(w)
        e = math.floor(math.log2(float(np.float32(amax)))) - 2
        assert sc == max(0, min(254, e + 127))


def test_int4_encoder_scale_and_rounding():
    w = np.zeros(32, np.float32)
    w[0] = 0.07
    w[1] = -0.035
    w[2] = 0.015
    nib, sc = synth.encode_int4_group(w)
    s_ref = torch.tensor(np.float32(0.07) / np.float32(7.0)).to(torch.bfloat16).float().item()
    s = np.array([sc], np.uint16).astype(np.uint32) << 16
    assert s.view(np.float32)[0] == np.float32(s_ref)
    codes = np.stack([nib & 15, nib >> 4], 1).reshape(-1).astype(np.int32)
    q = np.where(codes >= 8, codes - 16, codes)
    for i in range(3):
        assert q[i] == int(np.clip(np.rint(float(w[i]) / s_ref), -8, 7))
    assert np.all(q[3:] == 0)
    nib, sc = synth.encode_int4_group(np.zeros(32, np.float32))
    assert sc == 0 and np.all(nib == 0)


# -------------------------------------------------------------------- decode

def test_decode_mxfp4_exhaustive():
    codes = np.arange(16, dtype=np.uint8)
    packed = np.zeros((256, 16), np.uint8)
    # each row n uses scale code n; the 32 elements are codes 0..15 twice
    row = (codes[0::2] | (codes[1::2] << 4)).astype(np.uint8)
    packed[:, 0:8] = row
    packed[:, 8:16] = row
    scales = np.arange(256, dtype=np.uint8).reshape(256, 1)
    w = oracle.decode(oracle.FMT_MXFP4, packed, scales)
    for sc in range(256):
        for c in range(16):
            scale = float("nan") if sc == 255 else 2.0 ** (sc - 127)
            ref = np.float32(_e2m1_bits_value(c) * scale)
            got = w[sc, c]
            if math.isnan(ref):
                assert math.isnan(got)
            else:
                assert _f32_bits(got) == _f32_bits(ref), (sc, c, got, ref)
                assert got == w[sc, 16 + c]
    # BF16 view of MXFP4 values is exact (low 16 bits are zero, except where
    # the value is NaN).
    finite = w[:255]
    assert np.all((_f32_bits(finite) & 0xFFFF) == 0)
    np.testing.assert_array_equal(oracle.bf16_view(finite), (_f32_bits(finite) >> 16).astype(np.uint16))


def test_decode_int4_exhaustive():
    # 65536 BF16 scale patterns x 16 codes.
    scales = np.arange(65536, dtype=np.uint32).astype(np.uint16).reshape(65536, 1)
    codes = np.arange(16, dtype=np.uint8)
    row = (codes[0::2] | (codes[1::2] << 4)).astype(np.uint8)
    packed = np.tile(np.concatenate([row, row]), (65536, 1))
    w = oracle.decode(oracle.FMT_INT4, packed, scales)
    q = np.where(codes >= 8, codes.astype(np.int32) - 16, codes.astype(np.int32)).astype(np.float32)
    s = (scales.astype(np.uint32) << 16).view(np.float32)
    ref = (q[None, :] * s).astype(np.float32)   # numpy fp32 products
    got = w[:, :16]
    nan = np.isnan(ref)
    np.testing.assert_array_equal(np.isnan(got), nan)
    np.testing.assert_array_equal(_f32_bits(got)[~nan], _f32_bits(ref)[~nan])
    # BF16 view = round-to-nearest-even, checked against torch's BF16 cast.
    fin = ~nan
    tb = torch.from_numpy(got[fin].copy()).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    np.testing.assert_array_equal(oracle.bf16_view(got[fin]), tb)


# --------------------------------------------------------------------- route

def _brute_route(l, k):
    E = l.size
    order = sorted(range(E), key=lambda e: (-float(l[e]), e))[:k]
    p = special.softmax(l.astype(np.float64))
    g = np.array([p[e] for e in order])
    return order, g / g.sum()


@pytest.mark.parametrize("T,E,k", [(16, 8, 2), (9, 37, 5), (4, 384, 8), (3, 5, 5)])
def test_route_brute_force(T, E, k):
    rng = np.random.default_rng(T * 1000 + E)
    l = rng.standard_normal((T, E)).astype(np.float32)
    # force exact ties, including a tie at the selection boundary
    l[0, 1] = l[0, 0]
    l[1, :] = np.float32(0.5)
    ids, gates = oracle.route(l, k)
    for t in range(T):
        order, g = _brute_route(l[t], k)
        assert ids[t].tolist() == order
        np.testing.assert_allclose(gates[t], g, rtol=1e-12, atol=1e-15)
        assert abs(gates[t].sum() - 1.0) < 1e-12
        assert np.all(np.diff(gates[t]) <= 1e-15)
        assert len(set(ids[t].tolist())) == k


def test_route_special_cases():
    rng = np.random.default_rng(3)
    l = rng.standard_normal((8, 16)).astype(np.float32)
    ids, gates = oracle.route(l, 1)
    assert np.all(gates == 1.0)
    np.testing.assert_array_equal(ids[:, 0], np.argmax(l, 1))
    ids, gates = oracle.route(l, 16)
    for t in range(8):
        p = special.softmax(l[t].astype(np.float64))
        np.testing.assert_allclose(gates[t], p[ids[t]], rtol=1e-12)
        np.testing.assert_array_equal(np.sort(ids[t]), np.arange(16))
    with pytest.raises(ValueError):
        oracle.route(np.full((2, 4), np.nan, np.float32), 2)


# ------------------------------------------------------------------- permute

@pytest.mark.parametrize("T,k,E", [(64, 2, 8), (33, 8, 384), (5, 3, 40), (1, 1, 1)])
def test_permute_stable_sort(T, k, E):
    rng = np.random.default_rng(T + E)
    ids = np.stack([rng.choice(E, k, replace=False) for _ in range(T)]).astype(np.int32)
    out = oracle.permute(ids, E)
    flat = ids.reshape(-1)
    ref = sorted(range(T * k), key=lambda p: flat[p])   # Python's sort is stable
    assert out["perm"].tolist() == ref
    np.testing.assert_array_equal(out["counts"], np.bincount(flat, minlength=E))
    np.testing.assert_array_equal(out["offsets"], np.concatenate([[0], np.cumsum(out["counts"])]))
    np.testing.assert_array_equal(out["inv_perm"][out["perm"]], np.arange(T * k))
    act = np.nonzero(out["counts"])[0]
    assert out["n_active"] == act.size
    np.testing.assert_array_equal(out["active"][:act.size], act)
    for e in range(E):
        seg = out["perm"][out["offsets"][e]:out["offsets"][e + 1]]
        assert np.all(flat[seg] == e) and np.all(np.diff(seg) > 0)


def test_permute_rejects_bad_ids():
    with pytest.raises(ValueError):
        oracle.permute(np.array([[0, 9]], np.int32), 4)


# ---------------------------------------------------------------- projection

def _decode_bits(fmt, packed, scales):
    """Independent decoder written from the format definitions (numpy)."""
    N, K2 = packed.shape
    K = 2 * K2
    codes = np.empty((N, K), np.int32)
    codes[:, 0::2] = packed & 15
    codes[:, 1::2] = packed >> 4
    if fmt == 1:
        vals = np.array([_e2m1_bits_value(c) for c in range(16)])
        sc = np.where(scales == 255, np.nan, np.ldexp(1.0, scales.astype(np.int32) - 127))
        return (vals[codes] * np.repeat(sc, 32, axis=1)).astype(np.float32)
    q = np.where(codes >= 8, codes - 16, codes).astype(np.float64)
    s = (scales.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    return (q * np.repeat(s, 32, axis=1)).astype(np.float32)


@pytest.mark.parametrize("fmt", [1, 2])
def test_project_matches_numpy_matmul(fmt):
    E, N, K, T, k = 4, 48, 96, 10, 2
    p, s = synth.qweights(11, 3, fmt, E, N, K)
    x = synth.normal_bf16(11, 2, (T, K))
    rng = np.random.default_rng(0)
    tok = rng.integers(0, T, 12).astype(np.int32)
    ex = rng.integers(0, E, 12).astype(np.int32)
    y = oracle.project(fmt, p, s, x, tok, ex)
    xf = oracle.bf16_to_f64(x)
    for i in range(12):
        W = _decode_bits(fmt, p[ex[i]], s[ex[i]]).astype(np.float64)
        ref = W @ xf[tok[i]]
        np.testing.assert_allclose(y[i], ref, rtol=1e-12, atol=1e-12)
    # decode agrees with the independent decoder bit for bit
    for e in range(E):
        np.testing.assert_array_equal(_f32_bits(oracle.decode(fmt, p[e], s[e])),
                                      _f32_bits(_decode_bits(fmt, p[e], s[e])))


@pytest.mark.parametrize("fmt", [1, 2])
def test_project_t_matches_numpy_matmul(fmt):
    E, N, K = 3, 64, 96
    p, s = synth.qweights(12, 4, fmt, E, N, K)
    a = synth.normal_bf16(12, 5, (7, N))
    ex = np.array([0, 2, 2, 1, 0, 1, 2], np.int32)
    y = oracle.project_t(fmt, p, s, a, ex)
    af = oracle.bf16_to_f64(a)
    for i in range(7):
        W = _decode_bits(fmt, p[ex[i]], s[ex[i]]).astype(np.float64)
        np.testing.assert_allclose(y[i], af[i] @ W, rtol=1e-12, atol=1e-12)
    # adjoint of the forward projection: <a, W x> = <a W, x>
    x = synth.normal_bf16(12, 6, (1, K))
    fwd = oracle.project(fmt, p, s, x, np.zeros(1, np.int32), np.array([2], np.int32))[0]
    assert abs(np.dot(af[1], fwd) - np.dot(y[1], oracle.bf16_to_f64(x)[0])) < 1e-10


def test_project_one_hot_returns_weight_column():
    E, N, K = 2, 32, 64
    p, s = synth.qweights(5, 3, 1, E, N, K)
    x = np.zeros((K, K), np.uint16)
    x[np.arange(K), np.arange(K)] = 0x3F80  # BF16 1.0
    y = oracle.project(1, p, s, x, np.arange(K, dtype=np.int32), np.ones(K, np.int32))
    W = _decode_bits(1, p[1], s[1])
    np.testing.assert_array_equal(y.astype(np.float32), W.T)


# ----------------------------------------------------------------------- FFN

def _twin_ffn(fmt, gu, dn, xf, ids, gates, toks):
    """Per-token brute force: for each token, loop over its k experts, decode
    with the independent decoder, evaluate the expert FFN, sum gate-weighted."""
    I = gu[0].shape[1] // 2
    ys = []
    for t in toks:
        y = np.zeros(xf.shape[1])
        for j in range(ids.shape[1]):
            e = ids[t, j]
            Wg = _decode_bits(fmt, gu[0][e], gu[1][e]).astype(np.float64)
            Wd = _decode_bits(fmt, dn[0][e], dn[1][e]).astype(np.float64)
            h = Wg @ xf[t]
            a = h[:I] / (1.0 + np.exp(-h[:I])) * h[I:]
            y += gates[t, j] * (Wd @ a)
        ys.append(y)
    return np.array(ys)


def _tiny_ffn_inputs(fmt, T=6, d=64, I=32, E=5, k=2, seed=1):
    gu = synth.qweights(seed, 3, fmt, E, 2 * I, d, std=0.2)
    dn = synth.qweights(seed, 4, fmt, E, d, I, std=0.2)
    x = synth.normal_bf16(seed, 2, (T, d))
    logits = synth.normal_f32(seed, 1, (T, E))
    ids, gates = oracle.route(logits, k)
    return gu, dn, x, ids, gates


@pytest.mark.parametrize("fmt", [1, 2])
def test_ffn_matches_brute_force_twin(fmt):
    gu, dn, x, ids, gates = _tiny_ffn_inputs(fmt)
    toks = np.arange(x.shape[0], dtype=np.int32)
    y, h = oracle.ffn(fmt, gu, dn, x, ids, gates, toks, want_h=True)
    xf = oracle.bf16_to_f64(x)
    ref = _twin_ffn(fmt, gu, dn, xf, ids, gates, toks)
    np.testing.assert_allclose(y, ref, rtol=1e-12, atol=1e-12)
    # h per (token, slot) equals the numpy product with the slot's expert
    for s in range(toks.size * ids.shape[1]):
        t, j = divmod(s, ids.shape[1])
        W = _decode_bits(fmt, gu[0][ids[t, j]], gu[1][ids[t, j]]).astype(np.float64)
        np.testing.assert_allclose(h[s], W @ xf[t], rtol=1e-12, atol=1e-12)


def test_ffn_power_of_two_gates_count_each_pair_once():
    gu, dn, x, ids, _ = _tiny_ffn_inputs(1, k=3)
    T, k = ids.shape
    toks = np.arange(T, dtype=np.int32)
    base, _ = oracle.ffn(1, gu, dn, x, ids, np.zeros((T, k)), toks)
    assert np.all(base == 0)
    per_slot = []
    for j in range(k):
        g = np.zeros((T, k))
        g[:, j] = 1.0
        per_slot.append(oracle.ffn(1, gu, dn, x, ids, g, toks)[0])
    g = np.tile(2.0 ** -np.arange(k), (T, 1))
    y, _ = oracle.ffn(1, gu, dn, x, ids, g, toks)
    ref = sum(2.0 ** -j * per_slot[j] for j in range(k))
    np.testing.assert_allclose(y, ref, rtol=1e-13, atol=1e-14)


def test_silu_closed_forms():
    assert oracle.silu(0.0) == 0.0
    assert oracle.silu_grad(0.0) == 0.5
    assert abs(oracle.silu(30.0) - 30.0) < 1e-9
    assert abs(oracle.silu(-30.0)) < 1e-9
    for z in [-3.0, -0.7, 0.2, 1.5, 4.0]:
        fd = (oracle.silu(z + 1e-6) - oracle.silu(z - 1e-6)) / 2e-6
        assert abs(fd - oracle.silu_grad(z)) < 1e-8
        assert abs(oracle.silu(z) - z / (1 + math.exp(-z))) < 1e-15


# ------------------------------------------------------------------ backward

@pytest.mark.parametrize("fmt", [1, 2])
def test_dx_matches_finite_differences_of_forward(fmt):
    T, d, I, E, k = 4, 64, 32, 4, 2
    gu, dn, x, ids, gates = _tiny_ffn_inputs(fmt, T=T, d=d, I=I, E=E, k=k, seed=2)
    dy = synth.normal_bf16(2, 5, (T, d))
    toks = np.arange(T, dtype=np.int32)
    dx, _ = oracle.dx(fmt, gu, dn, x, dy, ids, gates, toks)
    xf = oracle.bf16_to_f64(x)
    dyf = oracle.bf16_to_f64(dy)
    # The twin forward is pinned to the oracle forward above; here its central
    # differences pin the oracle backward (a different code path).
    rng = np.random.default_rng(9)
    eps = 1e-4
    for _ in range(6):
        v = rng.standard_normal(xf.shape)
        fp = _twin_ffn(fmt, gu, dn, xf + eps * v, ids, gates, toks)
        fm = _twin_ffn(fmt, gu, dn, xf - eps * v, ids, gates, toks)
        fd = np.sum(dyf * (fp - fm)) / (2 * eps)
        an = np.sum(dx * v)
        assert abs(fd - an) <= 1e-6 * max(1.0, abs(an)), (fd, an)
    # per-token directional check as well
    for t in range(T):
        v = np.zeros_like(xf)
        v[t] = rng.standard_normal(d)
        fp = _twin_ffn(fmt, gu, dn, xf + eps * v, ids, gates, toks)
        fm = _twin_ffn(fmt, gu, dn, xf - eps * v, ids, gates, toks)
        fd = np.sum(dyf * (fp - fm)) / (2 * eps)
        assert abs(fd - np.dot(dx[t], v[t])) <= 1e-6 * max(1.0, abs(fd))


def test_dx_adjoint_of_down_projection():
    # dA returned by the oracle equals W_down^T (g * dY) computed by numpy.
    T, d, I, E, k = 3, 64, 32, 4, 2
    gu, dn, x, ids, gates = _tiny_ffn_inputs(2, T=T, d=d, I=I, E=E, k=k, seed=4)
    dy = synth.normal_bf16(4, 5, (T, d))
    toks = np.arange(T, dtype=np.int32)
    _, da = oracle.dx(2, gu, dn, x, dy, ids, gates, toks, want_da=True)
    dyf = oracle.bf16_to_f64(dy)
    xf = oracle.bf16_to_f64(x)
    for s in range(T * k):
        t, j = divmod(s, k)
        e = ids[t, j]
        Wd = _decode_bits(2, dn[0][e], dn[1][e]).astype(np.float64)
        np.testing.assert_allclose(da[s], Wd.T @ (gates[t, j] * dyf[t]), rtol=1e-12, atol=1e-13)
        # adjoint identity <dO, W a> = <W^T dO, a> for a random a
        a = np.random.default_rng(s).standard_normal(I)
        assert abs(np.dot(gates[t, j] * dyf[t], Wd @ a) - np.dot(da[s], a)) < 1e-10


# ------------------------------------------------------------- LoRA adapter

def _bf16_bits_to_f64(u16):
    return (np.asarray(u16, np.uint32) << 16).view(np.float32).astype(np.float64)


def _lora_inputs(fmt, P=7, T=5, K=128, N=64, E=3, rank=16, seed=7):
    packed, scales = synth.qweights(seed, 3, fmt, E, N, K, std=0.2)
    x = synth.normal_bf16(seed, 2, (T, K))
    A = synth.normal_bf16(seed, 7, (E, rank, K), std=0.05)
    B = synth.normal_bf16(seed, 8, (E, N, rank), std=0.05)
    rng = np.random.default_rng(seed)
    tok = rng.integers(0, T, P).astype(np.int32)
    expert = rng.integers(0, E, P).astype(np.int32)
    return packed, scales, x, A, B, tok, expert


@pytest.mark.parametrize("fmt", [1, 2])
def test_lora_project_matches_numpy_twin(fmt):
    packed, scales, x, A, B, tok, expert = _lora_inputs(fmt)
    alpha = 0.75
    y, u = oracle.lora_project(fmt, packed, scales, x, tok, expert, A, B, alpha, want_u=True)
    xf = _bf16_bits_to_f64(x)
    for i in range(tok.size):
        e = expert[i]
        W = _decode_bits(fmt, packed[e], scales[e]).astype(np.float64)
        Ae, Be = _bf16_bits_to_f64(A[e]), _bf16_bits_to_f64(B[e])
        ui = Ae @ xf[tok[i]]
        np.testing.assert_allclose(u[i], alpha * ui, rtol=1e-12, atol=1e-14)
        np.testing.assert_allclose(y[i], W @ xf[tok[i]] + alpha * (Be @ ui), rtol=1e-12, atol=1e-13)


def test_lora_project_special_cases():
    fmt = 2
    packed, scales, x, A, B, tok, expert = _lora_inputs(fmt)
    base = oracle.project(fmt, packed, scales, x, tok, expert)
    # no adapter contribution: alpha = 0, or B = 0
    assert np.array_equal(oracle.lora_project(fmt, packed, scales, x, tok, expert, A, B, 0.0), base)
    assert np.array_equal(
        oracle.lora_project(fmt, packed, scales, x, tok, expert, A, np.zeros_like(B), 2.0), base)
    # rank-one adapter A = e_k0, B = e_n0 (per expert): column n0 gains alpha x[k0]
    E, rank, K = A.shape
    N = B.shape[1]
    A1 = np.zeros_like(A)
    B1 = np.zeros_like(B)
    k0, n0 = 37, 11
    A1[:, 0, k0] = 0x3F80          # BF16 1.0
    B1[:, n0, 0] = 0x3F80
    y = oracle.lora_project(fmt, packed, scales, x, tok, expert, A1, B1, 0.5)
    d = y - base
    xf = _bf16_bits_to_f64(x)
    np.testing.assert_array_equal(d[:, n0], 0.5 * xf[tok, k0])
    d[:, n0] = 0
    assert np.all(d == 0)


def _lora_term_loss(xp, dyf, expert, Af, Bf, alpha):
    """<dY, alpha (x A^T) B^T> summed over pairs, in float64 (xp: per-pair rows)."""
    return sum(dyf[i] @ (alpha * (Bf[e] @ (Af[e] @ xp[i]))) for i, e in enumerate(expert))


def test_lora_bwd_matches_finite_differences():
    packed, scales, x, A, B, tok, expert = _lora_inputs(1, P=9, E=12, rank=16)
    N = B.shape[1]
    dy = synth.normal_bf16(7, 5, (tok.size, N))
    alpha = 0.75
    dx, dA, dB = oracle.lora_bwd(x, dy, tok, expert, A, B, alpha)
    xp = _bf16_bits_to_f64(x)[tok]
    dyf, Af, Bf = _bf16_bits_to_f64(dy), _bf16_bits_to_f64(A), _bf16_bits_to_f64(B)
    rng = np.random.default_rng(11)
    eps = 1e-3
    for name, grad in (("x", dx), ("A", dA), ("B", dB)):
        for _ in range(3):
            V = rng.standard_normal(grad.shape)
            args = {"x": xp, "A": Af, "B": Bf}
            lp = dict(args)
            lm = dict(args)
            lp[name] = args[name] + eps * V
            lm[name] = args[name] - eps * V
            fd = (_lora_term_loss(lp["x"], dyf, expert, lp["A"], lp["B"], alpha)
                  - _lora_term_loss(lm["x"], dyf, expert, lm["A"], lm["B"], alpha)) / (2 * eps)
            an = float(np.sum(grad * V))
            assert abs(fd - an) <= 1e-9 * max(1.0, abs(an)), (name, fd, an)
    # experts no pair uses get zero adapter gradients
    unused = sorted(set(range(A.shape[0])) - set(expert.tolist()))
    assert unused
    for e in unused:
        assert np.all(dA[e] == 0) and np.all(dB[e] == 0)


@pytest.mark.parametrize("fmt", [1, 2])
def test_ffn_lora_matches_twin_and_reduces_to_ffn(fmt):
    T, d, I, E, k, rank = 5, 64, 32, 4, 2, 16
    gu, dn, x, ids, gates = _tiny_ffn_inputs(fmt, T=T, d=d, I=I, E=E, k=k, seed=8)
    Agu = synth.normal_bf16(8, 7, (E, rank, d), std=0.1)
    Bgu = synth.normal_bf16(8, 8, (E, 2 * I, rank), std=0.1)
    Adn = synth.normal_bf16(8, 9, (E, rank, I), std=0.1)
    Bdn = synth.normal_bf16(8, 10, (E, d, rank), std=0.1)
    toks = np.arange(T, dtype=np.int32)
    alpha = 0.5
    y = oracle.ffn_lora(fmt, gu, dn, x, ids, gates, toks, (Agu, Bgu), (Adn, Bdn), alpha)
    # without adapters (alpha = 0) it is the plain FFN, exactly
    y0 = oracle.ffn_lora(fmt, gu, dn, x, ids, gates, toks, (Agu, Bgu), (Adn, Bdn), 0.0)
    yf, _ = oracle.ffn(fmt, gu, dn, x, ids, gates, toks)
    np.testing.assert_array_equal(y0, yf)
    # numpy twin
    xf = _bf16_bits_to_f64(x)
    for t in range(T):
        ref = np.zeros(d)
        for j in range(k):
            e = ids[t, j]
            Wg = _decode_bits(fmt, gu[0][e], gu[1][e]).astype(np.float64)
            Wd = _decode_bits(fmt, dn[0][e], dn[1][e]).astype(np.float64)
            h = Wg @ xf[t] + alpha * (_bf16_bits_to_f64(Bgu[e]) @ (_bf16_bits_to_f64(Agu[e]) @ xf[t]))
            a = h[:I] / (1.0 + np.exp(-h[:I])) * h[I:]
            o = Wd @ a + alpha * (_bf16_bits_to_f64(Bdn[e]) @ (_bf16_bits_to_f64(Adn[e]) @ a))
            ref += gates[t, j] * o
        np.testing.assert_allclose(y[t], ref, rtol=1e-12, atol=1e-12)
    # an adapter on one projection only
    yg = oracle.ffn_lora(fmt, gu, dn, x, ids, gates, toks, (Agu, Bgu), None, alpha)
    assert not np.array_equal(yg, yf) and not np.array_equal(yg, y)


def _twin_ffn_lora_loss(fmt, gu, dn, xf, dyf, ids, gates, ad_gu, ad_dn):
    """<dY, y> of the SwiGLU FFN with LoRA adapters, numpy float64 (adapters
    as (A, B, alpha) float arrays, or None)."""
    T, d = xf.shape
    I = gu[0].shape[1] // 2
    total = 0.0
    for t in range(T):
        y = np.zeros(d)
        for j in range(ids.shape[1]):
            e = ids[t, j]
            Wg = _decode_bits(fmt, gu[0][e], gu[1][e]).astype(np.float64)
            Wd = _decode_bits(fmt, dn[0][e], dn[1][e]).astype(np.float64)
            h = Wg @ xf[t]
            if ad_gu is not None:
                A, B, al = ad_gu
                h = h + B[e] @ (al * (A[e] @ xf[t]))
            a = h[:I] / (1.0 + np.exp(-h[:I])) * h[I:]
            o = Wd @ a
            if ad_dn is not None:
                A, B, al = ad_dn
                o = o + B[e] @ (al * (A[e] @ a))
            y += gates[t, j] * o
        total += float(dyf[t] @ y)
    return total


@pytest.mark.parametrize("which", ["both", "gate_up", "down"])
def test_ffn_lora_bwd_matches_finite_differences(which):
    fmt = 1 if which == "both" else 2
    T, d, I, E, k = 5, 64, 32, 5, 2
    gu, dn, x, ids, gates = _tiny_ffn_inputs(fmt, T=T, d=d, I=I, E=E, k=k, seed=12)
    dy = synth.normal_bf16(12, 5, (T, d))
    toks = np.arange(T, dtype=np.int32)
    lgu = (synth.normal_bf16(12, 7, (E, 16, d), std=0.1),
           synth.normal_bf16(12, 8, (E, 2 * I, 16), std=0.1), 0.5)
    ldn = (synth.normal_bf16(12, 9, (E, 32, I), std=0.1),
           synth.normal_bf16(12, 10, (E, d, 32), std=0.1), 0.75)
    lgu = lgu if which in ("both", "gate_up") else None
    ldn = ldn if which in ("both", "down") else None
    g = oracle.ffn_lora_bwd(fmt, gu, dn, x, dy, ids, gates, toks, lgu, ldn)
    xf, dyf = _bf16_bits_to_f64(x), _bf16_bits_to_f64(dy)
    f64 = lambda l: None if l is None else (_bf16_bits_to_f64(l[0]), _bf16_bits_to_f64(l[1]), l[2])  # noqa: E731
    point = {"x": xf, "gu": f64(lgu), "dn": f64(ldn)}

    def loss(pt):
        return _twin_ffn_lora_loss(fmt, gu, dn, pt["x"], dyf, ids, gates, pt["gu"], pt["dn"])

    def moved(name, V, eps):
        pt = dict(point)
        if name == "x":
            pt["x"] = xf + eps * V
        else:
            side, part = name[-2:], name[1]            # dA_gu -> ("gu", "A")
            A, B, al = pt[side]
            pt[side] = (A + eps * V, B, al) if part == "A" else (A, B + eps * V, al)
        return pt

    rng = np.random.default_rng(13)
    eps = 1e-4
    names = ["dx"] + [f"d{p}_{s}" for s in ("gu", "dn") for p in "AB"
                      if point[s] is not None]
    for name in names:
        grad = g[name]
        for _ in range(3):
            V = rng.standard_normal(grad.shape)
            key = "x" if name == "dx" else name
            fd = (loss(moved(key, V, eps)) - loss(moved(key, V, -eps))) / (2 * eps)
            an = float(np.sum(grad * V))
            assert abs(fd - an) <= 1e-6 * max(1.0, abs(an)), (which, name, fd, an)
    # experts no pair uses get zero adapter gradients
    unused = sorted(set(range(E)) - set(ids.reshape(-1).tolist()))
    for name in names[1:]:
        for e in unused:
            assert np.all(g[name][e] == 0)


def test_ffn_lora_bwd_special_cases():
    T, d, I, E, k = 4, 64, 32, 4, 2
    gu, dn, x, ids, gates = _tiny_ffn_inputs(1, T=T, d=d, I=I, E=E, k=k, seed=14)
    dy = synth.normal_bf16(14, 5, (T, d))
    toks = np.arange(T, dtype=np.int32)
    A1 = synth.normal_bf16(14, 7, (E, 16, d), std=0.1)
    B1 = synth.normal_bf16(14, 8, (E, 2 * I, 16), std=0.1)
    A2 = synth.normal_bf16(14, 9, (E, 16, I), std=0.1)
    B2 = synth.normal_bf16(14, 10, (E, d, 16), std=0.1)
    # alpha = 0: the adapters are inert, dx is the frozen-base backward and
    # every adapter gradient is exactly zero
    g = oracle.ffn_lora_bwd(1, gu, dn, x, dy, ids, gates, toks, (A1, B1, 0.0), (A2, B2, 0.0))
    dx0, _ = oracle.dx(1, gu, dn, x, dy, ids, gates, toks)
    np.testing.assert_allclose(g["dx"], dx0, rtol=1e-12, atol=1e-12)
    for name in ("dA_gu", "dB_gu", "dA_dn", "dB_dn"):
        assert np.all(g[name] == 0), name
    # B = 0: the adapters add nothing to the forward, so dx is again the base
    # one and dA (which goes through B) is zero; dB is not
    z1, z2 = np.zeros_like(B1), np.zeros_like(B2)
    g = oracle.ffn_lora_bwd(1, gu, dn, x, dy, ids, gates, toks, (A1, z1, 0.5), (A2, z2, 0.5))
    np.testing.assert_allclose(g["dx"], dx0, rtol=1e-12, atol=1e-12)
    assert np.all(g["dA_gu"] == 0) and np.all(g["dA_dn"] == 0)
    assert np.any(g["dB_gu"] != 0) and np.any(g["dB_dn"] != 0)


# ------------------------------------------------------------ router backward

def _twin_pair_outputs(fmt, gu, dn, xf, ids, t):
    """o[t, j] for each slot j of token t, by the numpy twin of the forward."""
    I = gu[0].shape[1] // 2
    outs = []
    for e in ids[t]:
        Wg = _decode_bits(fmt, gu[0][e], gu[1][e]).astype(np.float64)
        Wd = _decode_bits(fmt, dn[0][e], dn[1][e]).astype(np.float64)
        h = Wg @ xf[t]
        outs.append(Wd @ (h[:I] / (1.0 + np.exp(-h[:I])) * h[I:]))
    return np.array(outs)


def _kept_gates(l64, ids_t):
    p = special.softmax(l64)
    g = p[ids_t]
    return g / g.sum()


@pytest.mark.parametrize("fmt", [1, 2])
def test_router_bwd_matches_twin_and_finite_differences(fmt):
    T, d, I, E, k = 4, 64, 32, 6, 3
    gu, dn, x, ids, _ = _tiny_ffn_inputs(fmt, T=T, d=d, I=I, E=E, k=k, seed=5)
    logits = synth.normal_f32(5, 1, (T, E))
    ids, _ = oracle.route(logits, k)
    dy = synth.normal_bf16(5, 5, (T, d))
    toks = np.arange(T, dtype=np.int32)
    dg, dl = oracle.router_bwd(fmt, gu, dn, x, dy, logits, ids, toks)
    xf, dyf = oracle.bf16_to_f64(x), oracle.bf16_to_f64(dy)
    eps = 1e-6
    for t in range(T):
        o = _twin_pair_outputs(fmt, gu, dn, xf, ids, t)
        dg_twin = o @ dyf[t]
        np.testing.assert_allclose(dg[t], dg_twin, rtol=1e-12, atol=1e-12)
        l64 = logits[t].astype(np.float64)
        for e in range(E):
            lp, lm = l64.copy(), l64.copy()
            lp[e] += eps
            lm[e] -= eps
            # the perturbation is far smaller than any gap at the top-k boundary
            fd = (_kept_gates(lp, ids[t]) @ dg_twin - _kept_gates(lm, ids[t]) @ dg_twin) / (2 * eps)
            assert abs(fd - dl[t, e]) <= 1e-7 * max(1.0, abs(fd)), (t, e, fd, dl[t, e])
        kept = np.zeros(E, bool)
        kept[ids[t]] = True
        assert np.all(np.abs(dl[t, ~kept]) <= 1e-14 * np.abs(dl[t]).max())
        assert abs(dl[t].sum()) <= 1e-13 * np.abs(dl[t]).max()   # shift invariance


def test_router_bwd_special_cases():
    T, d, I, E = 3, 64, 32, 5
    gu, dn, x, _, _ = _tiny_ffn_inputs(1, T=T, d=d, I=I, E=E, k=1, seed=6)
    logits = synth.normal_f32(6, 1, (T, E))
    dy = synth.normal_bf16(6, 5, (T, d))
    toks = np.arange(T, dtype=np.int32)
    # k = 1: the gate is identically 1, so no gradient reaches the logits
    ids, _ = oracle.route(logits, 1)
    dg, dl = oracle.router_bwd(1, gu, dn, x, dy, logits, ids, toks)
    assert np.all(np.abs(dl) <= 1e-15 * np.abs(dg).max())
    # k = E: the gates are the plain softmax; torch's autograd of softmax
    ids, _ = oracle.route(logits, E)
    dg, dl = oracle.router_bwd(1, gu, dn, x, dy, logits, ids, toks)
    for t in range(T):
        l = torch.tensor(logits[t].astype(np.float64), requires_grad=True)
        up = torch.zeros(E, dtype=torch.float64)
        up[torch.from_numpy(ids[t].astype(np.int64))] = torch.from_numpy(dg[t])
        torch.softmax(l, 0).backward(up)
        np.testing.assert_allclose(dl[t], l.grad.numpy(), rtol=1e-12, atol=1e-14)


# ------------------------------------------------------- storage accounting

def test_storage_accounting_worked_example():
    kv = {}
    with open(os.path.join(GOLDEN, "mxfp4_storage_example.txt")) as f:
        for ln in f:
            if ln.strip() and not ln.startswith("#"):
                a, b = ln.split()
                kv[a] = float(b)
    P = kv["total_params"]
    bpw = accounting.grouped_bits(kv["bits"], int(kv["group_size"]), kv["scale_bits"])
    assert bpw == 4.25
    total = accounting.storage_bytes(P, bpw, kv["sensitive_ratio"])
    assert abs(total - 1.56975e12) < 1e3
    assert round(total / 1e12, 2) in (1.56, 1.57)     # page prints ~1.56 TB
    assert abs(P * 2 - kv["fp16_bytes_printed"]) < 1
    assert abs(P * kv["bits"] / 8 - kv["pure_4bit_bytes_printed"]) < 1
    assert round(P * 2 / total, 1) == kv["ratio_printed"]
    # bits per weight used for weight GB/s
    assert accounting.bits_per_weight(accounting.FMT_MXFP4) == 4.25
    assert accounting.bits_per_weight(accounting.FMT_INT4) == 4.5
    assert accounting.packed_bytes(1, 4096, 7168) * 8 == 4096 * 7168 * 4.25
