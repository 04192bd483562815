"""Pins of the CPU oracle against what the pages and the mathematics fix.

Each test checks the oracle against something other than itself: values the
pages print, closed forms, an independent library routine, high-precision
evaluation, exhaustive or brute-force checks, or identities of the linear
algebra.  A plausible slip anywhere in the oracle (a dropped term, a wrong
sign, index or transposition, a wrong scale) fails at least one of them.
"""
import json
import math
import os
from fractions import Fraction

import numpy as np
import pytest

import synthetic_inputs as si

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def f32_bits(x):
    return int(np.float32(x).view(np.uint32))


# --------------------------------------------------------------------------
# O1: the NF4 table (Ultralytics "QLoRA", "How QLoRA works", the snippet)
# --------------------------------------------------------------------------
def _levels_from_quantile(q):
    """16 NF4 levels from a given quantile function, rounded once to fp32."""
    off = 0.9677083
    pos = [q(off + (0.5 - off) * i / 8) for i in range(8)]
    neg = [-q(off + (0.5 - off) * i / 7) for i in range(7)]
    v = sorted(pos + neg + [0.0])
    return np.array([float(x / v[-1]) for x in v], np.float32)


def test_table_matches_mpmath_50_digits(orc):
    mpmath = pytest.importorskip("mpmath")
    mpmath.mp.dps = 50

    def q(p):
        return mpmath.sqrt(2) * mpmath.erfinv(2 * mpmath.mpf(p) - 1)

    off = mpmath.mpf("0.9677083")
    pos = [q(off + (mpmath.mpf("0.5") - off) * i / 8) for i in range(8)]
    neg = [-q(off + (mpmath.mpf("0.5") - off) * i / 7) for i in range(7)]
    v = sorted(pos + neg + [mpmath.mpf(0)])
    ref = np.array([float(x / v[-1]) for x in v], np.float32)
    got = orc.nf4_levels()
    assert [f32_bits(x) for x in got] == [f32_bits(x) for x in ref]


def test_table_matches_statistics_normaldist(orc):
    from statistics import NormalDist
    ref = _levels_from_quantile(NormalDist().inv_cdf)
    got = orc.nf4_levels()
    assert [f32_bits(x) for x in got] == [f32_bits(x) for x in ref]


def test_table_invariants(orc):
    L = orc.nf4_levels()
    assert L.dtype == np.float32 and L.shape == (16,)
    assert np.all(np.diff(L.astype(np.float64)) > 0), "strictly increasing"
    assert L[0] == -1.0 and L[15] == 1.0
    assert L[7] == 0.0 and f32_bits(L[7]) == 0, "an exact +0 level at code 7"
    assert int(np.sum(L < 0)) == 7 and int(np.sum(L > 0)) == 8
    # normaliser: the largest quantile is Phi^-1(0.9677083)
    assert orc.normal_quantile(0.9677083) == pytest.approx(1.8481309597573738, rel=1e-14)
    # minimum gap (codes 7->8, 0.0796) and maximum gap (codes 0->1, 0.3038)
    gaps = np.diff(L.astype(np.float64))
    assert int(np.argmin(gaps)) == 7 and int(np.argmax(gaps)) == 0


# --------------------------------------------------------------------------
# O2-O5: encode
# --------------------------------------------------------------------------
def snippet_sample():
    """The sample the Ultralytics "QLoRA" snippet measures its MSE on ("How
    QLoRA works"): 4096 blocks of 64 standard-normal fp32 values scaled by
    0.02, drawn from torch's CPU generator seeded with 0."""
    torch = pytest.importorskip("torch")
    g = torch.Generator().manual_seed(0)
    return (torch.randn(4096 * 64, generator=g) * 0.02).reshape(4096, 64).numpy()


def snippet_mse(orc, w, codebook):
    """Mean squared error of the oracle's codes with one exact fp32 absmax per
    block (no double quantization): level times absmax in fp32."""
    codes, qs, ds, am = orc.quantize(w, codebook, double_quant=False)
    assert qs is None and np.array_equal(ds, np.abs(w).max(axis=1)) and np.array_equal(am, ds)
    c = np.empty(w.size, np.int64)
    c[0::2], c[1::2] = codes & 15, codes >> 4
    restored = orc.codebook_levels(codebook)[c].reshape(w.shape) * ds[:, None]   # fp32 products
    return float(np.mean((restored - w).astype(np.float64) ** 2))


def test_snippet_printed_mse(orc):
    """The page prints NF4 MSE 3.395e-06 and 4.053e-06 for 16 evenly spaced
    levels on its seeded sample (tests/golden/snippet_mse.json); the oracle's
    own NF4 and INT4 tables reproduce both printed values."""
    gold = json.load(open(os.path.join(GOLDEN, "snippet_mse.json")))
    w = snippet_sample()
    nf4, int4 = snippet_mse(orc, w, "nf4"), snippet_mse(orc, w, "int4")
    assert f"{nf4:.3e}" == gold["nf4_mse_printed"], nf4
    assert f"{int4:.3e}" == gold["int4_mse_printed"], int4
    assert 0.15 < 1.0 - nf4 / int4 < 0.17, "the page's 'about 16%' lower error"


def test_self_codes(orc):
    """Encoding each level (times the block absmax) returns its own code."""
    L = orc.nf4_levels()
    for e in (-20, -7, -3, 0, 5, 30):
        block = np.tile(L, 4).astype(np.float32) * np.float32(2.0 ** e)   # absmax = 2^e
        codes, am = orc.encode_blocks(block.reshape(1, 64), L)
        assert am[0] == np.float32(2.0 ** e)
        c = np.empty(64, np.int64)
        c[0::2], c[1::2] = codes & 15, codes >> 4
        assert list(c) == list(range(16)) * 4


def test_exact_ties_take_lower_code(orc):
    """The listed values are exact fp32 ties (checked with numpy float32) and
    encode to the lower code, as argmin does."""
    L = orc.nf4_levels()
    rows = [ln.split() for ln in open(os.path.join(GOLDEN, "nf4_ties.txt"))
            if ln.strip() and not ln.startswith("#")]
    assert len(rows) == 5
    for j, h, _ in rows:
        j = int(j)
        v = np.array([int(h, 16)], np.uint32).view(np.float32)[0]
        assert np.abs(v - L[j]) == np.abs(L[j + 1] - v)
        assert orc.nearest_level(float(v), L) == j
        # one ulp either side decides for the nearer level
        up = np.nextafter(v, np.float32(2)); dn = np.nextafter(v, np.float32(-2))
        assert {orc.nearest_level(float(up), L), orc.nearest_level(float(dn), L)} == {j, j + 1}


def test_nearest_level_matches_exact_rational_rule(orc):
    """Away from the five exact fp32 ties, the fp32-distance argmin equals the
    nearest level in exact rational arithmetic."""
    L = orc.nf4_levels()
    Lq = [Fraction(float(x)) for x in L]
    ties = {int(ln.split()[1], 16) for ln in open(os.path.join(GOLDEN, "nf4_ties.txt"))
            if ln.strip() and not ln.startswith("#")}
    rng = np.random.default_rng(123)
    v = np.concatenate([rng.uniform(-1, 1, 4000).astype(np.float32),
                        # values within a few ulps of each midpoint
                        np.concatenate([np.float32((float(L[j]) + float(L[j + 1])) / 2) +
                                        np.arange(-6, 7, dtype=np.float32) *
                                        np.spacing(np.float32(abs(L[j]) + abs(L[j + 1])))
                                        for j in range(15)]).astype(np.float32)])
    for x in v:
        if int(np.float32(x).view(np.uint32)) in ties:
            continue
        xq = Fraction(float(x))
        ref = min(range(16), key=lambda i: (abs(xq - Lq[i]), i))
        assert orc.nearest_level(float(x), L) == ref, x


def test_pack_nibble_order_and_all_zero_block(orc):
    """Two codes per byte, element e of the flattened row in byte e/2, even e in
    the low nibble; an all-zero block gets the exact-zero code 7."""
    L = orc.nf4_levels()
    want = [(3 * e + 5) % 16 for e in range(64)]
    row = np.array([L[c] for c in want], np.float32) * np.float32(0.75)
    row[want.index(0)] = np.float32(-0.75)     # a code-0 element: absmax 0.75
    W = np.stack([row, np.zeros(64, np.float32)])
    codes, am = orc.encode_blocks(W.reshape(1, 128), L)
    assert am[0] == np.float32(0.75) and am[1] == 0
    expect = bytes((want[2 * i] | (want[2 * i + 1] << 4)) for i in range(32))
    assert bytes(codes[:32]) == expect
    assert bytes(codes[32:]) == bytes([0x77] * 32)
    qc, qs, ds, _ = orc.nf4_quantize(np.zeros((1, 64), np.float32))
    assert bytes(qc) == bytes([0x77] * 32) and qs[0] == 0 and ds[0] == 0
    deq = orc.nf4_dequantize(qc, qs, ds, 1, 64)
    assert np.all(deq == 0)


# --------------------------------------------------------------------------
# O6: double quantization (E4M3 in groups of 256)
# --------------------------------------------------------------------------
def test_e4m3_values_match_torch(orc):
    torch = pytest.importorskip("torch")
    codes = torch.arange(256, dtype=torch.int32).to(torch.uint8).view(torch.float8_e4m3fn)
    ref = codes.to(torch.float64).numpy()
    for c in range(256):
        if (c & 0x7F) == 0x7F:
            assert math.isnan(ref[c])
            continue
        assert orc.e4m3_value(c) == ref[c], c


def test_e4m3_encode_matches_torch(orc):
    torch = pytest.importorskip("torch")
    vals = [orc.e4m3_value(c) for c in range(0x7F)]
    mids = [(a + b) / 2 for a, b in zip(vals[:-1], vals[1:])]
    rng = np.random.default_rng(7)
    xs = np.concatenate([np.array(vals, np.float32), np.array(mids, np.float32),
                         np.nextafter(np.array(mids, np.float32), np.float32(0)),
                         np.nextafter(np.array(mids, np.float32), np.float32(1e9)),
                         rng.uniform(0, 448, 20000).astype(np.float32),
                         np.exp2(rng.uniform(-14, 8.8, 20000)).astype(np.float32),
                         np.array([0.0, 448.0, np.float32(448.0) * np.float32(1 + 2**-23)],
                                  np.float32)])
    xs = xs[xs <= np.float32(448.0) * np.float32(1 + 2**-22)]
    ref = torch.from_numpy(xs).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    got = np.array([orc.e4m3_encode(float(x)) for x in xs], np.uint8)
    bad = np.nonzero(got != ref)[0]
    assert bad.size == 0, [(xs[i], got[i], ref[i]) for i in bad[:5]]


def test_bf16_rne_matches_torch(orc):
    torch = pytest.importorskip("torch")
    rng = np.random.default_rng(11)
    u = rng.integers(0, 2**32, 50000, dtype=np.uint64).astype(np.uint32)
    u = u[((u >> 23) & 0xFF) != 0xFF]                     # finite only
    ties = (rng.integers(0, 2**16, 2000, dtype=np.uint32) << 16) | 0x8000
    ties = ties[((ties >> 23) & 0xFF) != 0xFF]
    xs = np.concatenate([u, ties.astype(np.uint32)]).view(np.float32)
    ref = torch.from_numpy(xs.copy()).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    got = np.array([orc.bf16_rne(float(x)) for x in xs], np.uint16)
    assert np.array_equal(got, ref)


def test_double_quant_structure(orc):
    """Per group of 256 blocks the largest scale maps to E4M3 max (code 0x7E,
    value 448); every restored scale is within E4M3's half-ulp (2^-4 relative)
    of the exact absmax; the last group may be short."""
    cfg = si.custom(N=64 * 3, K=192, M=1, r=8, outlier_frac=0.01, seed=3)   # 576 blocks
    W = si.weight(cfg, 0)
    codes, qs, ds, am = orc.nf4_quantize(W)
    nb = W.size // 64
    assert qs.size == nb and ds.size == (nb + 255) // 256 == 3
    for g in range(ds.size):
        b0, b1 = 256 * g, min(256 * g + 256, nb)
        c = am[b0:b1].max()
        assert ds[g] == np.float32(c / np.float32(448.0))
        assert qs[b0 + int(np.argmax(am[b0:b1]))] == 0x7E
        restored = np.array([orc.e4m3_value(int(q)) for q in qs[b0:b1]]) * float(ds[g])
        rel = np.abs(restored - am[b0:b1].astype(np.float64)) / am[b0:b1]
        assert rel.max() <= 2.0 ** -4 + 1e-7


def _uint8_restored(qs, ds):
    """q_b * d_g in float64 (exact: 8-bit integer times an fp32)."""
    return qs.astype(np.float64) * np.repeat(ds.astype(np.float64), 256)[:qs.size]


def test_uint8_double_quant_is_a_uniform_8bit_grid(orc):
    """The uint8-linear reading of "8 bits in blocks of 256" (Ultralytics "QLoRA",
    double-quantization bullet): per group the 256 values 0, d, ..., 255 d with
    255 d = the group's largest scale.  Every restored scale is within d / 2 of
    the exact absmax (plus the fp32 roundings of d and of the quotient), the
    largest block of each group gets 255, and the error is far below E4M3's
    (8 even steps against 3 mantissa bits)."""
    cfg = si.custom(N=64 * 3, K=192, M=1, r=8, outlier_frac=0.01, seed=3)   # 576 blocks
    W = si.weight(cfg, 0)
    codes, qs, ds, am = orc.quantize(W, "nf4", dq_format="uint8")
    codes_e, qs_e, ds_e, _ = orc.quantize(W, "nf4", dq_format="e4m3")
    assert np.array_equal(codes, codes_e)           # the codes use the exact absmax either way
    nb = W.size // 64
    assert qs.size == nb and ds.size == 3
    rest = _uint8_restored(qs, ds)
    a = am.astype(np.float64)
    d = np.repeat(ds.astype(np.float64), 256)[:nb]
    assert np.all(np.abs(rest - a) <= d * (0.5 + 2.0 ** -16))
    for g in range(3):
        b0, b1 = 256 * g, min(256 * g + 256, nb)
        top = b0 + int(np.argmax(am[b0:b1]))
        assert qs[top] == 255
        assert abs(rest[top] - a[top]) <= a[top] * 2.0 ** -22
    # on Gaussian weights without outliers the block scales sit near the group
    # maximum, where the even grid's step (max / 255) beats E4M3's 2^-4
    Wg = si.weight(si.custom(N=64 * 3, K=192, M=1, r=8, seed=4), 0)
    _, qg, dg, ag = orc.quantize(Wg, "nf4", dq_format="uint8")
    _, qe, de, _ = orc.quantize(Wg, "nf4", dq_format="e4m3")
    ag = ag.astype(np.float64)
    rest_e = np.array([orc.e4m3_value(int(q)) for q in qe]) * np.repeat(de.astype(np.float64), 256)[:nb]
    rel_u8 = np.sqrt(np.mean(((_uint8_restored(qg, dg) - ag) / ag) ** 2))
    rel_e4 = np.sqrt(np.mean(((rest_e - ag) / ag) ** 2))
    assert rel_u8 < 0.25 * rel_e4


def test_uint8_double_quant_exact_on_a_grid_and_ties_to_even(orc):
    """Scales on the grid k 2^-10 with the group maximum 255 * 2^-10 make
    d = 2^-10 exactly, so each code is k itself and the restored scale is
    exact; scales halfway between grid points, (k + 1/2) 2^-10, go to the even
    neighbour (round half to even)."""
    ks = [255, 0, 1, 2, 3, 17, 128, 254, 77, 200]
    halves = [0.5, 1.5, 2.5, 100.5, 253.5]
    targets = [k * 2.0 ** -10 for k in ks] + [h * 2.0 ** -10 for h in halves]
    W = np.zeros((len(targets), 64), np.float32)
    for i, t in enumerate(targets):
        W[i, 5] = np.float32(-t if i % 2 else t)     # the block absmax is |W[i, 5]|
    codes, qs, ds, am = orc.quantize(W, "nf4", dq_format="uint8")
    assert ds[0] == np.float32(2.0 ** -10)
    assert list(qs[:len(ks)]) == ks
    assert list(qs[len(ks):]) == [0, 2, 2, 100, 254]
    rest = _uint8_restored(qs, ds)
    assert np.array_equal(rest[:len(ks)], np.array(ks, np.float64) * 2.0 ** -10)
    # an all-zero group: d = 0 and every code 0
    c0, q0, d0, _ = orc.quantize(np.zeros((4, 64), np.float32), "nf4", dq_format="uint8")
    assert d0[0] == 0.0 and not q0.any()


def test_uint8_dequantize_uses_q_times_d(orc):
    """Dequantized weights of the uint8 format equal those of the fp32-scale
    format whose block scales are q_b * d_g rounded once to fp32 (numpy's
    double -> float rounding): the two scale decodes agree."""
    cfg = si.custom(N=32, K=256, M=1, r=8, seed=8)
    W = si.weight(cfg, 0)
    codes, qs, ds, am = orc.quantize(W, "nf4", dq_format="uint8")
    sc = _uint8_restored(qs, ds).astype(np.float32)
    got = orc.dequantize(codes, qs, ds, *W.shape, dq_format="uint8")
    want = orc.dequantize(codes, None, sc, *W.shape)
    assert np.array_equal(got, want)


def test_storage_footprint_closed_forms(orc):
    """Ultralytics "QLoRA" and vnread "Grokking QLoRA": 0.5 -> ~0.127 bits/param,
    ~0.37 saved, ~3 GB at 65B, ~130 GB at 16 bit, NF4 ~33 GB, NF4+DQ ~34 GB."""
    g = json.load(open(os.path.join(GOLDEN, "storage_footprint.json")))
    W = np.zeros((256, 4096), np.float32)   # 16384 blocks, 64 groups
    codes, qs, ds, _ = orc.nf4_quantize(W)
    n = W.size
    bits_dq = 8 * (qs.nbytes + ds.nbytes) / n
    bits_nodq = 32 * (n // 64) / n
    assert bits_nodq == g["no_dq_overhead_bits_per_param"]
    assert bits_dq == pytest.approx(8 / 64 + 32 / (64 * 256))
    assert round(bits_dq, 3) == g["dq_overhead_bits_per_param"]
    assert round(bits_nodq - bits_dq, 2) == g["dq_saving_bits_per_param"]
    P = g["params_65b"]
    assert round((bits_nodq - bits_dq) * P / 8 / 1e9) == g["dq_saving_gb_65b"]
    assert round(16 * P / 8 / 1e9) == g["fp16_gb_65b"]
    nf4_total_gb = (8 * codes.nbytes / n + bits_dq) * P / 8 / 1e9
    assert math.floor(4 * P / 8 / 1e9) >= g["nf4_gb_65b_low"] - 1
    assert round(nf4_total_gb) == g["nf4_dq_gb_65b"]


# --------------------------------------------------------------------------
# O7: dequantize
# --------------------------------------------------------------------------
def test_dequant_error_bound(orc):
    """|w' - w| <= (largest half-gap between levels) * restored scale + scale error
    + bf16 half-ulp; and the dequantized value has the sign of its level."""
    cfg = si.custom(N=128, K=256, M=1, r=8, seed=5)
    W = si.weight(cfg, 0)
    codes, qs, ds, am = orc.nf4_quantize(W)
    deq = si.bf16_bits_to_f32(orc.nf4_dequantize(codes, qs, ds, *W.shape)).astype(np.float64)
    L = orc.nf4_levels().astype(np.float64)
    half_gap = np.max(np.diff(L)) / 2
    a = np.repeat(am.astype(np.float64), 64).reshape(W.shape)
    sc = np.repeat(np.array([orc.e4m3_value(int(q)) for q in qs]) *
                   np.repeat(ds.astype(np.float64), 256)[:qs.size], 64).reshape(W.shape)
    bound = half_gap * a + np.abs(sc - a) + np.abs(deq) * 2.0 ** -8
    assert np.all(np.abs(deq - W) <= bound + 1e-12)
    c = np.empty(W.size, np.int64)
    c[0::2], c[1::2] = codes & 15, codes >> 4
    lv = L[c].reshape(W.shape)
    assert np.all(np.sign(deq) == np.sign(lv))


# --------------------------------------------------------------------------
# O8-O9: forward and backward, pinned by identities of the linear algebra
# --------------------------------------------------------------------------
def _small_problem(orc, N=48, K=128, M=5, r=4, alpha=8.0, seed=2):
    cfg = si.custom(N=N, K=K, M=M, r=r, alpha=alpha, seed=seed)
    W = si.weight(cfg, 0)
    codes, qs, ds, _ = orc.nf4_quantize(W)
    Wdq = orc.nf4_dequantize(codes, qs, ds, N, K)
    X = si.activations(cfg, 0)
    A, B = si.adapters(cfg, 0)
    dY = si.upstream(cfg, 0)
    return cfg, Wdq, X, A, B, dY


def _f(h):
    return si.bf16_bits_to_f32(h).astype(np.float64)


def test_forward_equals_merged_weight_matmul(orc):
    """Y = X (W' + (alpha/r) B A)^T, evaluated with numpy's float64 matmul."""
    cfg, Wdq, X, A, B, dY = _small_problem(orc)
    Y, T = orc.qlora_fwd(Wdq, X, A, B, cfg.alpha)
    s = cfg.alpha / cfg.r
    ref = _f(X) @ (_f(Wdq) + s * _f(B) @ _f(A)).T
    np.testing.assert_allclose(Y, ref, rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(T, _f(X) @ _f(A).T, rtol=1e-12, atol=1e-12)


def test_forward_rows_subset_and_alpha_linearity(orc):
    cfg, Wdq, X, A, B, dY = _small_problem(orc)
    Y, _ = orc.qlora_fwd(Wdq, X, A, B, cfg.alpha)
    Ys, _ = orc.qlora_fwd(Wdq, X, A, B, cfg.alpha, rows=[4, 0, 2])
    assert np.array_equal(Ys, Y[[4, 0, 2]])
    Y0, _ = orc.qlora_fwd(Wdq, X, A, B, 0.0)
    Y2, _ = orc.qlora_fwd(Wdq, X, A, B, 2 * cfg.alpha)
    np.testing.assert_allclose(Y2 - Y, Y - Y0, rtol=1e-10, atol=1e-12)
    np.testing.assert_allclose(Y0, _f(X) @ _f(Wdq).T, rtol=1e-12, atol=1e-12)


def test_zero_B_gives_base_output_and_zero_dA(orc):
    cfg, Wdq, X, A, B, dY = _small_problem(orc)
    Bz = np.zeros_like(B)
    Y, _ = orc.qlora_fwd(Wdq, X, A, Bz, cfg.alpha)
    Y0, _ = orc.qlora_fwd(Wdq, X, A, B, 0.0)
    assert np.array_equal(Y, Y0)
    dA, dB = orc.qlora_bwd_adapters(X, dY, A, Bz, cfg.alpha)
    assert np.all(dA == 0)
    np.testing.assert_allclose(dB, cfg.alpha / cfg.r * _f(dY).T @ (_f(X) @ _f(A).T),
                               rtol=1e-12, atol=1e-12)


def test_zero_A_gives_zero_dB(orc):
    cfg, Wdq, X, A, B, dY = _small_problem(orc)
    dA, dB = orc.qlora_bwd_adapters(X, dY, np.zeros_like(A), B, cfg.alpha)
    assert np.all(dB == 0)
    np.testing.assert_allclose(dA, cfg.alpha / cfg.r * (_f(dY) @ _f(B)).T @ _f(X),
                               rtol=1e-12, atol=1e-12)


def test_backward_adjoint_identities(orc):
    """Y is linear in X, in A and in B: <dY, Y(X)> = <dX, X>, and
    <dA, A> = <dB, B> = <dY, Y - Y_base>."""
    cfg, Wdq, X, A, B, dY = _small_problem(orc)
    Y, _ = orc.qlora_fwd(Wdq, X, A, B, cfg.alpha)
    Yb, _ = orc.qlora_fwd(Wdq, X, A, B, 0.0)
    dX = orc.qlora_bwd_dx(Wdq, dY, A, B, cfg.alpha)
    dA, dB = orc.qlora_bwd_adapters(X, dY, A, B, cfg.alpha)
    g = _f(dY)
    lhs = float(np.sum(g * Y))
    assert lhs == pytest.approx(float(np.sum(dX * _f(X))), rel=1e-10)
    lora = float(np.sum(g * (Y - Yb)))
    assert float(np.sum(dA * _f(A))) == pytest.approx(lora, rel=1e-9)
    assert float(np.sum(dB * _f(B))) == pytest.approx(lora, rel=1e-9)


def test_backward_secants(orc):
    """L = <dY, Y> is linear in each input element, so a secant through two exact
    bf16 values of one element equals that element's gradient."""
    cfg, Wdq, X, A, B, dY = _small_problem(orc, N=24, K=64, M=3, r=3)
    g = _f(dY)
    dX = orc.qlora_bwd_dx(Wdq, dY, A, B, cfg.alpha)
    dA, dB = orc.qlora_bwd_adapters(X, dY, A, B, cfg.alpha)
    one, half = np.uint16(0x3F80), np.uint16(0xBF00)     # +1.0 and -0.5 in bf16

    def L(Xm, Am, Bm):
        Y, _ = orc.qlora_fwd(Wdq, Xm, Am, Bm, cfg.alpha)
        return float(np.sum(g * Y))

    for (name, arr, grad, idx) in (("X", X, dX, (1, 17)), ("A", A, dA, (2, 40)),
                                   ("B", B, dB, (13, 1)), ("X", X, dX, (2, 63))):
        a1, a2 = arr.copy(), arr.copy()
        a1[idx], a2[idx] = one, half
        args1 = {"X": X, "A": A, "B": B}; args1[name] = a1
        args2 = {"X": X, "A": A, "B": B}; args2[name] = a2
        sec = (L(args1["X"], args1["A"], args1["B"]) - L(args2["X"], args2["A"], args2["B"])) / 1.5
        assert sec == pytest.approx(float(grad[idx]), rel=1e-9, abs=1e-9), name


def test_dx_rows_subset(orc):
    cfg, Wdq, X, A, B, dY = _small_problem(orc)
    dX = orc.qlora_bwd_dx(Wdq, dY, A, B, cfg.alpha)
    dXs = orc.qlora_bwd_dx(Wdq, dY, A, B, cfg.alpha, rows=[3, 1])
    assert np.array_equal(dXs, dX[[3, 1]])
    s = cfg.alpha / cfg.r
    ref = _f(dY) @ (_f(Wdq) + s * _f(B) @ _f(A))
    np.testing.assert_allclose(dX, ref, rtol=1e-12, atol=1e-12)


def test_results_do_not_depend_on_thread_count(orc):
    cfg, Wdq, X, A, B, dY = _small_problem(orc, N=40, K=192, M=7, r=5)
    W = si.weight(cfg, 0)
    q1 = orc.nf4_quantize(W, threads=1)
    q7 = orc.nf4_quantize(W, threads=7)
    for a, b in zip(q1, q7):
        assert np.array_equal(a, b)
    y1, _ = orc.qlora_fwd(Wdq, X, A, B, cfg.alpha, threads=1)
    y3, _ = orc.qlora_fwd(Wdq, X, A, B, cfg.alpha, threads=3)
    assert np.array_equal(y1, y3)


def test_adapter_entries_match_full_adapters(orc):
    cfg, Wdq, X, A, B, dY = _small_problem(orc, N=40, K=128, M=9, r=5)
    dA, dB = orc.qlora_bwd_adapters(X, dY, A, B, cfg.alpha)
    ia = [(0, 3), (4, 127), (2, 64), (4, 0)]
    ib = [(39, 4), (0, 0), (17, 2)]
    ea, eb = orc.qlora_adapter_entries(X, dY, A, B, cfg.alpha, ia, ib)
    assert np.array_equal(ea, np.array([dA[j, k] for j, k in ia]))
    assert np.array_equal(eb, np.array([dB[n, j] for n, j in ib]))


# --------------------------------------------------------------------------
# f1: the adapter merged into the weight (IBM "What is LoRA?"; Ultralytics
# "QLoRA", "Trade-offs"), and the double -> bf16 rounding it uses
# --------------------------------------------------------------------------
def test_bf16_rne_double_rounds_once(orc):
    """Doubles that are floats round as the float rounding (pinned against
    torch above); values a hair off a tie, closer than a float can express,
    round by the exact rule, which a float intermediate would get wrong."""
    rng = np.random.default_rng(21)
    u = rng.integers(0, 2**32, 20000, dtype=np.uint64).astype(np.uint32)
    u = u[((u >> 23) & 0xFF) != 0xFF]
    for x in u.view(np.float32)[:5000]:
        assert orc.bf16_rne_double(float(x)) == orc.bf16_rne(float(x))
    one = 0x3F80
    assert orc.bf16_rne_double(1.0 + 2.0**-8) == one                 # tie -> even (1.0)
    assert orc.bf16_rne_double(1.0 + 2.0**-8 + 2.0**-40) == one + 1  # just above the tie
    assert orc.bf16_rne_double(1.0 + 3 * 2.0**-8) == one + 2          # tie -> even (1 + 2^-6)
    assert orc.bf16_rne_double(1.0 + 3 * 2.0**-8 - 2.0**-40) == one + 1
    assert orc.bf16_rne_double(-(1.0 + 2.0**-8 + 2.0**-40)) == 0x8000 | (one + 1)
    assert orc.bf16_rne_double(0.0) == 0x0000 and orc.bf16_rne_double(-0.0) == 0x8000
    big = float(np.float32(3.3895314e38))                              # largest finite bf16
    assert orc.bf16_rne_double(big) == 0x7F7F
    assert orc.bf16_rne_double(2.0**128) == 0x7F80                    # overflow -> inf


def _merge_problem(orc, N=40, K=192, M=6, r=5, alpha=10.0, seed=4):
    cfg, Wdq, X, A, B, dY = _small_problem(orc, N=N, K=K, M=M, r=r, alpha=alpha, seed=seed)
    return cfg, Wdq, X, A, B


def _ulp_bf16(v):
    """Spacing of bf16 at |v| (normal range)."""
    e = np.floor(np.log2(np.maximum(np.abs(v), 2.0**-126)))
    return 2.0 ** (e - 7)


def test_merge_with_zero_B_is_the_dequantized_weight(orc):
    cfg, Wdq, X, A, B = _merge_problem(orc)
    Bz = np.zeros_like(B)
    assert np.array_equal(orc.lora_merge(Wdq, A, Bz, cfg.alpha), Wdq)
    assert np.array_equal(orc.lora_merge(Wdq, A, B, 0.0), Wdq)


def test_merged_weight_reproduces_the_forward(orc):
    """X bf16(W' + s B A)^T equals the forward oracle's Y up to the one bf16
    rounding per weight; the adapter's share is far above that rounding, so a
    wrong sign, scale or operand order fails."""
    cfg, Wdq, X, A, B = _merge_problem(orc)
    Wm = orc.lora_merge(Wdq, A, B, cfg.alpha)
    Y, _ = orc.qlora_fwd(Wdq, X, A, B, cfg.alpha)
    Ym = _f(X) @ _f(Wm).T
    bound = np.abs(_f(X)) @ (np.abs(_f(Wm)) * 2.0**-8).T
    assert np.all(np.abs(Ym - Y) <= bound + 1e-300)
    Y0, _ = orc.qlora_fwd(Wdq, X, A, B, 0.0)
    assert np.max(np.abs(Y - Y0)) > 20 * np.max(bound)                # the adapter matters here


def test_unmerge_inverts_merge(orc):
    cfg, Wdq, X, A, B = _merge_problem(orc)
    Wm = orc.lora_merge(Wdq, A, B, cfg.alpha)
    Wu = orc.lora_merge(Wm, A, B, cfg.alpha, sign=-1)
    d = np.abs(_f(Wu) - _f(Wdq))
    assert np.all(d <= 0.5 * (_ulp_bf16(_f(Wm)) + _ulp_bf16(_f(Wu))) + 1e-300)
    assert np.mean(Wu == Wdq) > 0.5
    assert not np.array_equal(Wm, Wdq)


def test_merge_does_not_depend_on_thread_count(orc):
    cfg, Wdq, X, A, B = _merge_problem(orc, N=33, K=128, r=3)
    assert np.array_equal(orc.lora_merge(Wdq, A, B, cfg.alpha, threads=1),
                          orc.lora_merge(Wdq, A, B, cfg.alpha, threads=7))


def test_merge_is_exact_on_small_integers(orc):
    """With integer base, adapters and s = alpha/r = 2, W + s B A is an integer
    below 2^8, so bf16 holds it exactly: the merge must equal the integer
    product (numpy) bit for bit.  This fixes the scale, sign and operand order
    exactly, beyond what a rounding bound can."""
    rng = np.random.default_rng(8)
    N, K, r, alpha = 24, 64, 5, 10.0
    Wi = rng.integers(-40, 41, (N, K))
    Ai = rng.integers(-2, 3, (r, K))
    Bi = rng.integers(-2, 3, (N, r))
    exact = Wi + 2 * (Bi @ Ai)
    assert np.max(np.abs(exact)) < 256
    bits = lambda a: si.to_bf16_bits(a.astype(np.float32))
    got = orc.lora_merge(bits(Wi), bits(Ai), bits(Bi), alpha)
    assert np.array_equal(got, bits(exact))
    back = orc.lora_merge(got, bits(Ai), bits(Bi), alpha, sign=-1)
    assert np.array_equal(back, bits(Wi))


def test_swiglu_closed_forms(orc):
    """silu(x) = x sigmoid(x) against forms the oracle does not use: the tanh
    form (x/2)(1 + tanh(x/2)) for x >= 0, x e^x / (1 + e^x) for x < 0 (each
    free of cancellation on its side), the odd part silu(x) - silu(-x) = x,
    zero at zero, the identity for large x, and linearity in the up input."""
    rng = np.random.default_rng(8)
    g = np.concatenate([rng.normal(0.0, 3.0, 2000), [0.0, 1e-300, -1e-300, 2.0, -2.0, -30.0]])
    one = np.ones_like(g)
    h = orc.swiglu(g, one)
    pos = g >= 0
    tanh_form = 0.5 * g[pos] * (1.0 + np.tanh(0.5 * g[pos]))
    assert np.allclose(h[pos], tanh_form, rtol=1e-14, atol=1e-300)
    e = np.exp(g[~pos])
    assert np.allclose(h[~pos], g[~pos] * e / (1.0 + e), rtol=1e-14, atol=1e-300)
    assert np.allclose(h - orc.swiglu(-g, one), g, rtol=1e-13, atol=1e-15)
    assert orc.swiglu(np.array([0.0]), np.array([5.0]))[0] == 0.0
    assert orc.swiglu(np.array([2.0]), np.array([1.0]))[0] == pytest.approx(1.0 + math.tanh(1.0), rel=1e-15)
    assert orc.swiglu(np.array([50.0]), np.array([1.0]))[0] == pytest.approx(50.0, rel=1e-15)
    u = rng.normal(size=g.shape)
    assert np.allclose(orc.swiglu(g, 3.0 * u), 3.0 * orc.swiglu(g, u), rtol=1e-14, atol=1e-300)


# --------------------------------------------------------------------------
# Codebook and scale-format variants: the INT4 comparison codebook of the
# Ultralytics snippet, and block scales kept in fp32 (no double quantization)
# --------------------------------------------------------------------------
def _f32_nearest(fr: Fraction) -> np.float32:
    """The fp32 value nearest to an exact rational (ties to even), by search."""
    f = np.float32(float(fr))
    cands = [np.nextafter(f, np.float32(-2)), f, np.nextafter(f, np.float32(2))]
    best = min(cands, key=lambda c: (abs(Fraction(float(c)) - fr), int(c.view(np.uint32)) & 1))
    return np.float32(best)


def test_int4_table_is_evenly_spaced_rounded_once(orc):
    """Sixteen levels from -1 to 1 in equal steps of 2/15, each the exact value
    rounded once to fp32; symmetric, with no zero level."""
    L = orc.int4_levels()
    for i in range(16):
        assert L[i] == _f32_nearest(Fraction(2 * i - 15, 15)), i
    assert L[0] == -1.0 and L[15] == 1.0
    assert np.array_equal(L[::-1], -L)
    assert not np.any(L == 0)
    assert np.all(np.diff(L.astype(np.float64)) > 0)


def test_int4_nearest_level_matches_exact_rational_rule(orc):
    """With the INT4 table the fp32-distance argmin equals the exact rational
    nearest level, lower code on an exact tie; all-zero blocks take code 7, the
    lower of the two levels nearest zero."""
    L = orc.int4_levels()
    Lq = [Fraction(float(x)) for x in L]
    rng = np.random.default_rng(77)
    mids = [np.float32((float(L[j]) + float(L[j + 1])) / 2) + np.arange(-4, 5, dtype=np.float32) *
            np.spacing(np.float32(1.0)) for j in range(15)]
    v = np.concatenate([rng.uniform(-1, 1, 3000).astype(np.float32), *mids]).astype(np.float32)
    for x in v:
        xq = Fraction(float(x))
        d = [abs(xq - q) for q in Lq]
        # fp32 distances decide: skip values whose two nearest fp32 distances round equal
        df = sorted(abs(np.float32(x) - L))
        if df[0] == df[1] and min(d) != sorted(d)[1]:
            continue
        ref = min(range(16), key=lambda i: (d[i], i))
        assert orc.nearest_level(float(x), L) == ref, x
    W = np.zeros((2, 128), np.float32)
    W[1, 64:] = 0.5
    for dq in (True, False):
        codes, _, _, _ = orc.quantize(W, "int4", double_quant=dq)
        assert np.all(codes[:64] == 0x77)


@pytest.mark.parametrize("codebook", ["nf4", "int4"])
@pytest.mark.parametrize("dq,fmt", [(True, "e4m3"), (True, "uint8"), (False, "e4m3")],
                         ids=["e4m3", "uint8", "fp32"])
def test_variant_dequant_error_bound_and_self_codes(orc, codebook, dq, fmt):
    """For every codebook and scale format: |w' - w| <= half the largest level gap
    times the block absmax, plus the scale's own error, plus half a bf16 ulp; a
    block holding the levels times 2^e comes back as bf16 of the levels times 2^e
    (rounded by torch), code for code."""
    torch = pytest.importorskip("torch")
    L = orc.codebook_levels(codebook).astype(np.float64)
    cfg = si.custom(N=96, K=256, M=1, r=8, seed=9, outlier_frac=0.01)
    W = si.weight(cfg, 0)
    codes, qs, ds, am = orc.quantize(W, codebook, double_quant=dq, dq_format=fmt)
    deq = si.bf16_bits_to_f32(orc.dequantize(codes, qs, ds, *W.shape, codebook=codebook,
                                             dq_format=fmt)).astype(np.float64)
    a = np.repeat(am.astype(np.float64), 64).reshape(W.shape)
    if dq and fmt == "uint8":
        sc = np.repeat(_uint8_restored(qs, ds), 64).reshape(W.shape)
    elif dq:
        sc = np.repeat(np.array([orc.e4m3_value(int(q)) for q in qs]) *
                       np.repeat(ds.astype(np.float64), 256)[:qs.size], 64).reshape(W.shape)
    else:
        assert np.array_equal(ds, am)
        sc = a
    bound = np.max(np.diff(L)) / 2 * a + np.abs(sc - a) + np.abs(deq) * 2.0 ** -8
    assert np.all(np.abs(deq - W) <= bound + 1e-12)
    Lf = orc.codebook_levels(codebook)
    for e in (-9, 0, 4):
        blk = (np.tile(Lf, 4) * np.float32(2.0 ** e)).astype(np.float32).reshape(1, 64)
        c2, q2, d2, _ = orc.quantize(blk, codebook, double_quant=dq, dq_format=fmt)
        got = orc.dequantize(c2, q2, d2, 1, 64, codebook=codebook, dq_format=fmt)
        want = torch.from_numpy(blk).bfloat16().view(torch.int16).numpy().view(np.uint16)
        assert np.array_equal(got, want), (codebook, dq, e)


# --------------------------------------------------------------------------
# Adapter optimizer step (AdamW)
# --------------------------------------------------------------------------
def test_adamw_closed_forms(orc):
    """First step from zero state moves by lr g / (|g| + eps) after the decay;
    a constant gradient keeps the bias-corrected moments at g and g^2, so t
    steps move by t lr g / (|g| + eps); with g = 0 only the decay acts,
    theta (1 - lr wd)^t."""
    rng = np.random.default_rng(31)
    n = 257
    th0 = rng.normal(size=n)
    g = rng.normal(size=n) * 10.0 ** rng.integers(-4, 2, n)
    lr, wd, eps = 1e-3, 0.05, 1e-8
    th, m, v = orc.adamw_step(th0, np.zeros(n), np.zeros(n), g, lr, weight_decay=wd, eps=eps)
    assert np.allclose(th, th0 * (1 - lr * wd) - lr * g / (np.abs(g) + eps), rtol=0, atol=1e-15)
    assert np.allclose(m, 0.1 * g, rtol=1e-15) and np.allclose(v, 0.001 * g * g, rtol=1e-12)
    th, m, v = th0.copy(), np.zeros(n), np.zeros(n)
    for t in range(1, 8):
        th, m, v = orc.adamw_step(th, m, v, g, lr, step=t, eps=eps)
    assert np.allclose(th, th0 - 7 * lr * g / (np.abs(g) + eps), rtol=0, atol=1e-13)
    th, m, v = th0.copy(), np.zeros(n), np.zeros(n)
    for t in range(1, 6):
        th, m, v = orc.adamw_step(th, m, v, np.zeros(n), lr, weight_decay=wd, step=t)
    assert np.allclose(th, th0 * (1 - lr * wd) ** 5, rtol=1e-14, atol=0)


def test_adamw_matches_torch_in_float64(orc):
    """Five steps against torch.optim.AdamW (an independent implementation) in
    float64, with weight decay and non-default betas."""
    torch = pytest.importorskip("torch")
    rng = np.random.default_rng(32)
    n = 300
    th0 = rng.normal(size=n)
    grads = [rng.normal(size=n) for _ in range(5)]
    p = torch.nn.Parameter(torch.tensor(th0, dtype=torch.float64))
    opt = torch.optim.AdamW([p], lr=2e-3, betas=(0.8, 0.95), eps=1e-6, weight_decay=0.1)
    th, m, v = th0.copy(), np.zeros(n), np.zeros(n)
    for t, gr in enumerate(grads, start=1):
        p.grad = torch.tensor(gr, dtype=torch.float64)
        opt.step()
        th, m, v = orc.adamw_step(th, m, v, gr, 2e-3, beta1=0.8, beta2=0.95, eps=1e-6,
                                  weight_decay=0.1, step=t)
        assert np.allclose(th, p.detach().numpy(), rtol=1e-13, atol=1e-15), t
    st = opt.state[p]
    assert np.allclose(m, st["exp_avg"].numpy(), rtol=1e-13)
    assert np.allclose(v, st["exp_avg_sq"].numpy(), rtol=1e-13)
