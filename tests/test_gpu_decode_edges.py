"""The fused decoder against the oracle over the whole scale range.

The fused variant decodes nibbles and scales in registers with other
instructions than the chunked variant's dequant kernel (MXFP4 through the
hardware's scaled E2M1 conversion, INT4 through an FP8 conversion and a fused
multiply-add), so its exactness is checked on its own here: identity probes
read every decoded weight back through the grouped GEMM.  A one-hot A row
e_k gives y[n] = W[n][k] (one exact product; every other term is 0 * a finite
weight), in both orientations: y = x W^T (one-hot over K) and the transposed
y = a W (one-hot over N).  The reference is the oracle's decode in its BF16
view (the value rounded once to BF16, as both variants feed it to the
matrix cores), element by element.  A weight that is NaN or Inf turns the
zero terms of its own dot products into NaN, so each probe row holds one
group of interest, every group that can decode to a non-finite value sits in
W positions no other such group shares, and the reference marks as NaN every
output whose dot product holds such a term.

Formats ("超大规模开放权重模型技术解析", 三 微缩放量化的原理: 32 elements share
one scale): all 256 E8M0 codes x 16 E2M1 codes, and all 65536 BF16 INT4 scale
patterns x 16 codes, in both storage layouts and on the 32-row and the
128-row tile kernels.  Every output is also compared bit for bit with the
chunked variant, whose decoded weights are pinned to the oracle bit for bit
by the dequant-only tests.  INT4 scales outside the fused decoder's exact
domain (+-Inf, or magnitude >= 2^119) are the only allowed differences, and
qgg_check_weights must flag exactly those weights."""
import numpy as np
import pytest
import torch

import oracle
import quantized_grouped_gemm_amd as qgg

from .gpu_util import DEV, bf16_to_f64, dev_bf16, dev_weights, host_u16, sync

pytestmark = pytest.mark.gpu

ONE = np.uint16(0x3F80)   # BF16 1.0


def _same(a, b):
    """Elementwise equality with NaN equal to NaN (+0 == -0)."""
    return (a == b) | (np.isnan(a) & np.isnan(b))


def _pack_rows(codes):
    """[..., K] nibble codes -> [..., K/2] bytes (element k in byte k>>1, low
    nibble for even k)."""
    codes = codes.astype(np.uint8)
    return (codes[..., 0::2] | (codes[..., 1::2] << 4)).astype(np.uint8)


def _int4_out_of_domain(sbits):
    m = sbits.astype(np.uint32) & 0x7FFF
    return (m >= 0x7B00) & (m <= 0x7F80)


# ------------------------------------------------------------ probe builders

def _mxfp4_forward_probe():
    """N = 8192 rows, K = 128: row n holds E8M0 code c = n >> 5 on group g and
    one nonzero nibble v = (n >> 1) & 15 at position p of that group (both
    parities for every (c, v)); every other element is 0 under code 127."""
    N, K = 8192, 128
    n = np.arange(N)
    c, v, r = n >> 5, (n >> 1) & 15, n & 1
    g = (c + v + r) & 3
    p = (2 * v + r + 3 * c) & 31
    codes = np.zeros((N, K), np.uint8)
    codes[n, 32 * g + p] = v
    scales = np.full((N, K // 32), 127, np.uint8)
    scales[n, g] = c
    return _pack_rows(codes), scales


def _mxfp4_transposed_probes():
    """Two matrices for y = a W (rows dealt to experts by the caller).  Finite
    codes (0..252): 253 x 32 rows as in the forward probe, then zero rows up
    to 8192.  Codes that can decode to Inf or NaN (253, 254, 255): 96 rows
    (then zero rows up to 128), row i's group at K block i, so that no two of
    them share a column."""
    out = []
    n = np.arange(253 * 32)
    c, v, r = n >> 5, (n >> 1) & 15, n & 1
    N, K = 8192, 128
    g = (c + v + r) & 3
    p = (2 * v + r + 3 * c) & 31
    codes = np.zeros((N, K), np.uint8)
    codes[n, 32 * g + p] = v
    scales = np.full((N, K // 32), 127, np.uint8)
    scales[n, g] = c
    out.append((_pack_rows(codes), scales))
    i = np.arange(96)
    c, v, r = 253 + (i >> 5), (i >> 1) & 15, i & 1
    N, K = 128, 96 * 32
    p = (2 * v + r) & 31
    codes = np.zeros((N, K), np.uint8)
    codes[i, 32 * i + p] = v
    scales = np.full((N, K // 32), 127, np.uint8)
    scales[i, i] = c
    out.append((_pack_rows(codes), scales))
    return out


def _int4_group_codes(n):
    """The 32 codes of row n's group: every code twice, at positions of both
    parities."""
    i = np.arange(32)
    return ((i[None, :] + n[:, None] + (i[None, :] >= 16)) % 16).astype(np.uint8)


def _int4_forward_probe():
    """N = 65536 rows, K = 128: row n's group g = n & 3 has BF16 scale bits n
    and all 16 codes; the other groups are zeros under scale +0."""
    N, K = 65536, 128
    n = np.arange(N)
    g = n & 3
    codes = np.zeros((N, K), np.uint8)
    codes[n[:, None], 32 * g[:, None] + np.arange(32)[None, :]] = _int4_group_codes(n)
    scales = np.zeros((N, K // 32), np.uint16)
    scales[n, g] = n.astype(np.uint16)
    return _pack_rows(codes), scales


def _int4_transposed_probes():
    """For y = a W: every finite in-domain scale (rows whose scale is NaN, Inf
    or of magnitude >= 2^119 hold scale +0 instead, so no column is
    poisoned), and a second small matrix with NaN scales, each in its own K
    block."""
    pk, sc = _int4_forward_probe()
    n = np.arange(65536)
    bits = n.astype(np.uint16)
    nonfinite = (bits & 0x7F80) == 0x7F80
    drop = nonfinite | _int4_out_of_domain(bits)
    sc[n[drop], n[drop] & 3] = 0
    out = [(pk, sc)]
    nan_bits = np.array([0x7FC0, 0xFFC0, 0x7F81, 0xFFFF], np.uint16)
    N, K = 64, 128
    rows = np.arange(4)
    codes = np.zeros((N, K), np.uint8)
    codes[rows[:, None], 32 * rows[:, None] + np.arange(32)[None, :]] = _int4_group_codes(rows)
    scales = np.zeros((N, K // 32), np.uint16)
    scales[rows, rows] = nan_bits
    out.append((_pack_rows(codes), scales))
    return out, drop


# ------------------------------------------------------------ runners

def _perm_for(ids, E):
    p, _ = qgg.expert_permute(torch.from_numpy(ids).to(DEV), E)
    return p


def _forward(fmt, packed, scales, layout, E):
    """y [T=K][N] for one-hot rows e_t (t < K), tokens t routed to expert
    t // (K / E) of E identical copies of the probe.  Returns (fused, chunked)
    BF16 bits, both in token order."""
    N, K = packed.shape[0], packed.shape[1] * 2
    pk = np.ascontiguousarray(np.broadcast_to(packed, (E,) + packed.shape))
    sc = np.ascontiguousarray(np.broadcast_to(scales, (E,) + scales.shape))
    w = dev_weights(fmt, pk, sc, layout=layout)
    x = np.zeros((K, K), np.uint16)
    x[np.arange(K), np.arange(K)] = ONE
    ids = (np.arange(K) // (K // E)).astype(np.int32)[:, None]
    p = _perm_for(ids, E)
    xd = dev_bf16(x)
    yf = qgg.dequant_grouped_gemm(w, xd, p, K, 1, qgg.FUSED, 0)
    yc = qgg.dequant_grouped_gemm(w, xd, p, K, 1, qgg.CHUNKED, 1)
    sync()
    inv = p.inv_perm.cpu().numpy()
    return host_u16(yf)[inv], host_u16(yc)[inv]


def _split(packed, scales, rows_per_expert):
    """The probe's rows dealt to experts of rows_per_expert rows each."""
    N = packed.shape[0]
    E = max(N // rows_per_expert, 1)
    Ne = N // E
    return packed.reshape(E, Ne, -1), scales.reshape(E, Ne, -1)


def _one_hot_over_rows(E, Ne):
    """Token t = e * Ne + n is routed to expert e with a = e_n over that
    expert's Ne rows."""
    T = E * Ne
    a = np.zeros((T, Ne), np.uint16)
    a[np.arange(T), np.arange(T) % Ne] = ONE
    ids = (np.arange(T) // Ne).astype(np.int32)[:, None]
    return a, ids


def _transposed(fmt, packed, scales, layout):
    """y [T][K] = a W_e for one-hot rows a_t over the rows of t's expert
    (packed [E][Ne][K/2]): row t of y is row t % Ne of expert t // Ne."""
    E, Ne = packed.shape[0], packed.shape[1]
    w = dev_weights(fmt, packed, scales, layout=layout)
    a, ids = _one_hot_over_rows(E, Ne)
    T = a.shape[0]
    p = _perm_for(ids, E)
    ad = dev_bf16(a)
    yf = qgg.dequant_grouped_gemm(w, ad, p, T, 1, qgg.FUSED, 0,
                                  flags=qgg.A_TOKENS | qgg.TRANSPOSE_W)
    yc = qgg.dequant_grouped_gemm(w, ad, p, T, 1, qgg.CHUNKED, 1,
                                  flags=qgg.A_TOKENS | qgg.TRANSPOSE_W)
    sync()
    inv = p.inv_perm.cpu().numpy()
    return host_u16(yf)[inv], host_u16(yc)[inv]


def _decoded(fmt, packed, scales):
    """The oracle's decoded weights of one expert in their BF16 view, as
    float64 (the GEMMs' B operand values)."""
    return oracle.bf16_to_f64(oracle.bf16_view(oracle.decode(fmt, packed, scales)))


def _poisoned(w):
    """For each element, whether another element of the same dot product is
    non-finite: along the row (axis 1) for the one-hot probes over K."""
    bad = ~np.isfinite(w)
    return (bad.sum(axis=1, keepdims=True) - bad) > 0


def _oracle_forward(fmt, packed, scales):
    """y[t][n] = sum_k e_t[k] W[n][k] = W[n][t], plus NaN when another weight
    of row n is non-finite (0 * Inf or 0 * NaN)."""
    w = _decoded(fmt, packed, scales)
    ref = w.copy()
    ref[_poisoned(w)] = np.nan
    return np.ascontiguousarray(ref.T)


def _oracle_transposed(fmt, packed, scales):
    """Token t = e * Ne + n: y[t][c] = sum_m e_n[m] W_e[m][c] = W_e[n][c], plus
    NaN when another weight of column c of W_e is non-finite."""
    out = []
    for e in range(packed.shape[0]):
        w = _decoded(fmt, packed[e], scales[e])
        ref = w.copy()
        ref[_poisoned(w.T).T] = np.nan
        out.append(ref)
    return np.concatenate(out, axis=0)


def _check(what, fused, chunked, ref, allowed_cols=None):
    """fused == chunked bit for bit and == oracle (NaN-equal), except in the
    allowed output columns.  Returns the columns where the fused output
    differs from the oracle."""
    got = bf16_to_f64(fused)
    ok = _same(got, ref)
    bad_cols = np.unique(np.nonzero(~ok)[1])
    if allowed_cols is not None:
        unexpected = np.setdiff1d(bad_cols, allowed_cols)
    else:
        unexpected = bad_cols
    if unexpected.size:
        r, c = np.nonzero(~ok)
        sel = np.isin(c, unexpected)
        ex = [(int(a), int(b), float(got[a, b]), float(ref[a, b]))
              for a, b in zip(r[sel][:8], c[sel][:8])]
        pytest.fail(f"{what}: fused decode differs from the oracle in {unexpected.size} "
                    f"columns, e.g. (row, col, fused, oracle) {ex}")
    keep = np.ones(fused.shape[1], bool)
    if allowed_cols is not None:
        keep[allowed_cols] = False
    cmp_f, cmp_c = fused[:, keep], chunked[:, keep]
    same = (cmp_f == cmp_c) | (np.isnan(bf16_to_f64(cmp_f)) & np.isnan(bf16_to_f64(cmp_c)))
    assert np.all(same), f"{what}: fused and chunked outputs differ ({np.sum(~same)} values)"
    return bad_cols


@pytest.mark.parametrize("layout", [qgg.LAYOUT_ROWS, qgg.LAYOUT_MFMA], ids=["rows", "mfma"])
@pytest.mark.parametrize("E", [1, 4], ids=["tile128", "tile32"])
def test_fused_mxfp4_decode_every_scale_code(layout, E):
    packed, scales = _mxfp4_forward_probe()
    ref = _oracle_forward(1, packed, scales)
    yf, yc = _forward(1, packed, scales, layout, E)
    _check(f"mxfp4 forward layout {layout} E {E}", yf, yc, ref)


@pytest.mark.parametrize("layout", [qgg.LAYOUT_ROWS, qgg.LAYOUT_MFMA], ids=["rows", "mfma"])
def test_fused_mxfp4_transposed_decode_every_scale_code(layout):
    for i, (packed, scales) in enumerate(_mxfp4_transposed_probes()):
        packed, scales = _split(packed, scales, 1024)
        ref = _oracle_transposed(1, packed, scales)
        yf, yc = _transposed(1, packed, scales, layout)
        _check(f"mxfp4 transposed probe {i} layout {layout}", yf, yc, ref)


@pytest.mark.parametrize("layout", [qgg.LAYOUT_ROWS, qgg.LAYOUT_MFMA], ids=["rows", "mfma"])
@pytest.mark.parametrize("E", [1, 4], ids=["tile128", "tile32"])
def test_fused_int4_decode_every_bf16_scale(layout, E):
    packed, scales = _int4_forward_probe()
    ref = _oracle_forward(2, packed, scales)
    yf, yc = _forward(2, packed, scales, layout, E)
    n = np.arange(65536)
    allowed = n[_int4_out_of_domain(n.astype(np.uint16))]
    bad = _check(f"int4 forward layout {layout} E {E}", yf, yc, ref, allowed_cols=allowed)
    print(f"int4 forward layout {layout} E {E}: {bad.size} out-of-domain scales differ",
          flush=True)


@pytest.mark.parametrize("layout", [qgg.LAYOUT_ROWS, qgg.LAYOUT_MFMA], ids=["rows", "mfma"])
def test_fused_int4_transposed_decode_every_bf16_scale(layout):
    probes, _ = _int4_transposed_probes()
    for i, (packed, scales) in enumerate(probes):
        packed, scales = _split(packed, scales, 1024)
        ref = _oracle_transposed(2, packed, scales)
        yf, yc = _transposed(2, packed, scales, layout)
        _check(f"int4 transposed probe {i} layout {layout}", yf, yc, ref)


def test_check_weights_flags_exactly_the_out_of_domain_scales():
    # INT4: every scale pattern in one tensor is flagged; the same tensor
    # without the out-of-domain scales is not; a single out-of-domain scale
    # anywhere (either layout) is
    packed, scales = _int4_forward_probe()
    for layout in (qgg.LAYOUT_ROWS, qgg.LAYOUT_MFMA):
        w = dev_weights(2, packed[None], scales[None], layout=layout)
        assert int(qgg.check_weights(w).item()) == 4
    bits = scales.copy()
    bad = _int4_out_of_domain(bits)
    bits[bad] = 0x3F80
    assert not np.any(_int4_out_of_domain(bits))
    for layout in (qgg.LAYOUT_ROWS, qgg.LAYOUT_MFMA):
        w = dev_weights(2, packed[None], bits[None], layout=layout)
        assert int(qgg.check_weights(w).item()) == 0
    for one in (0x7B00, 0xFB00, 0x7F80, 0xFF80, 0x7F7F):
        b2 = bits.copy()
        b2[12345 % b2.shape[0], 1] = one
        w = dev_weights(2, packed[None], b2[None])
        assert int(qgg.check_weights(w).item()) == 4, hex(one)
    for fine in (0x7AFF, 0xFAFF, 0x7FC0, 0xFFC1, 0x0001):
        b2 = bits.copy()
        b2[7, 2] = fine
        w = dev_weights(2, packed[None], b2[None])
        assert int(qgg.check_weights(w).item()) == 0, hex(fine)
    # MXFP4: every code decodes exactly on both variants, nothing is flagged
    pk, sc = _mxfp4_forward_probe()
    w = dev_weights(1, pk[None], sc[None])
    assert int(qgg.check_weights(w).item()) == 0
