"""GPU parity of the adapter merge and unmerge against the CPU oracle, through
the C ABI.  IBM "What is LoRA?" (the update B A merged into the pretrained
weight; adapters swapped per task); Ultralytics glossary "QLoRA",
"Trade-offs" (the merge needs the base dequantized to 16 bit first).

The oracle evaluates W +/- (alpha/r) B A in double and rounds once to bf16;
the kernel sums the rank-r product in fp32, adds it with one fused
multiply-add (s = fl32(alpha/r)) and rounds that to bf16.  The bar, from that
arithmetic: every value the kernel writes is the bf16 rounding of some number
within the fp32 error of the exact result, that is
    |got - exact| <= ulp_bf16(got) / 2 + 2^-22 (|W| + |s| sum_j |B A|),
which allows the two roundings to part only on values within that error of a
rounding boundary (ties, and results that cancel to about zero).  The share
of elements that differ from the oracle's rounding is reported and must stay
small."""
import numpy as np
import pytest

import synthetic_inputs as si
from helpers import GpuLayer, bf16_tensor, log, tensor_bits

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
if not torch.cuda.is_available():  # pragma: no cover
    pytest.skip("needs a GPU", allow_module_level=True)

import bit_nf4_quantized_17_amd as q  # noqa: E402


def _f64(bits):
    return si.bf16_bits_to_f32(bits).astype(np.float64)


def _ulp_bf16(x):
    e = np.floor(np.log2(np.maximum(np.abs(x), 2.0**-126)))
    return 2.0 ** (e - 7)


def check_rounded(got_bits, ref_bits, exact, mag, label, max_frac=1e-2):
    """mag: |W| + |s| sum_j |B[n][j] A[j][k]|, the scale of the fp32 error."""
    got = _f64(got_bits)
    far = np.abs(got - exact) > 0.5 * _ulp_bf16(got) + 2.0**-22 * mag
    if far.any():
        i = tuple(np.argwhere(far)[0])
        raise AssertionError(f"{label}: {int(far.sum())} elements out of bound, first {i}: "
                             f"got {got[i]!r} exact {exact[i]!r} scale {mag[i]!r}")
    frac = float(np.mean(got_bits != ref_bits))
    log(f"  {label}: {frac:.2e} of elements round differently from the oracle")
    assert frac <= max_frac, f"{label}: {frac:.2e} of elements differ from the oracle's rounding"
    return frac


def _merge_case(orc, N, K, r, alpha, seed):
    cfg = si.custom(N=N, K=K, M=1, r=r, alpha=alpha, seed=seed)
    lay = GpuLayer(cfg)
    codes, qs, ds = (lay.w.codes.cpu().numpy(), lay.w.qscale.cpu().numpy(), lay.w.dscale.cpu().numpy())
    Wdq = orc.nf4_dequantize(codes, qs, ds, N, K)
    return lay, Wdq


MERGE = [
    # N, K, r, alpha
    (256, 256, 8, 16.0),        # one tile
    (300, 320, 3, 16.0),        # ragged rows and columns, rank below one MFMA step
    (1, 64, 1, 2.0),            # a single row and block
    (513, 1088, 64, 16.0),      # several tiles both ways, partial last ones
    (128, 8192, 128, 32.0),     # the largest rank
    (4100, 2304, 16, 32.0),     # many row tiles
]


@pytest.mark.parametrize("N,K,r,alpha", MERGE)
def test_merge_and_unmerge(orc, N, K, r, alpha):
    lay, Wdq = _merge_case(orc, N, K, r, alpha, seed=7 * N + K)
    label = f"merge {N}x{K} r={r}"
    log(f"[{label}]")
    Wm = q.qlora_merge(lay.w, lay.dA_in, lay.dB_in, alpha)
    Wm2 = q.qlora_merge(lay.w, lay.dA_in, lay.dB_in, alpha)
    torch.cuda.synchronize()
    got = tensor_bits(Wm)
    assert np.array_equal(got, tensor_bits(Wm2)), "run-to-run"
    s = alpha / r
    prod = _f64(lay.B) @ _f64(lay.A)
    absprod = np.abs(s) * (np.abs(_f64(lay.B)) @ np.abs(_f64(lay.A)))
    exact = _f64(Wdq) + s * prod
    check_rounded(got, orc.lora_merge(Wdq, lay.A, lay.B, alpha), exact, np.abs(_f64(Wdq)) + absprod, label)

    log(f"[un{label}]")
    Wu = q.qlora_unmerge(Wm, lay.dA_in, lay.dB_in, alpha)
    torch.cuda.synchronize()
    gu = tensor_bits(Wu)
    exact_u = _f64(got) - s * prod
    check_rounded(gu, orc.lora_merge(got, lay.A, lay.B, alpha, sign=-1), exact_u,
                  np.abs(_f64(got)) + absprod, "un" + label)
    # back to the dequantized weight within the two roundings and the fp32 errors
    assert np.all(np.abs(_f64(gu) - _f64(Wdq)) <=
                  _ulp_bf16(_f64(got)) + _ulp_bf16(_f64(gu)) + 2.0**-21 * (np.abs(_f64(got)) + absprod))
    # in place gives the same bits
    Wi = Wm.clone()
    q.qlora_unmerge(Wi, lay.dA_in, lay.dB_in, alpha, out=Wi)
    torch.cuda.synchronize()
    assert np.array_equal(tensor_bits(Wi), gu), "in place"


def test_merge_with_zero_adapter_is_dequantize(orc):
    lay, Wdq = _merge_case(orc, 320, 512, 16, 32.0, seed=3)
    Wm = q.qlora_merge(lay.w, lay.dA_in, torch.zeros_like(lay.dB_in), 32.0)
    torch.cuda.synchronize()
    assert np.array_equal(tensor_bits(Wm), Wdq)


def test_merge_full_size_sampled_rows(orc):
    """The 70B-class up projection (28672x8192, r = 64): the whole merge on the
    GPU, sampled rows against the oracle."""
    cfg = si.CONFIGS["mlp70b_28672"]
    lay = GpuLayer(cfg, 0, M=1)
    N, K, alpha = lay.N, lay.K, lay.alpha
    log(f"[merge full size] {N}x{K} r={lay.r}")
    Wm = q.qlora_merge(lay.w, lay.dA_in, lay.dB_in, alpha)
    torch.cuda.synchronize()
    codes, qs, ds = (lay.w.codes.cpu().numpy(), lay.w.qscale.cpu().numpy(), lay.w.dscale.cpu().numpy())
    rng = np.random.default_rng(5)
    rows = sorted({0, N - 1, *(int(x) for x in rng.integers(0, N, 6))})
    # dequantize only the sampled rows, block by block: block b of row n
    # belongs to group (n * K/64 + b) // 256 of the full weight
    Wdq_rows = np.zeros((len(rows), K), np.uint16)
    nbk = K // 64
    for i, n in enumerate(rows):
        c = codes.reshape(N, K // 2)[n]
        qrow = qs.reshape(N, nbk)[n]
        for b in range(nbk):
            g = (n * nbk + b) // 256
            Wdq_rows[i, 64 * b:64 * b + 64] = orc.nf4_dequantize(
                c[32 * b:32 * b + 32], qrow[b:b + 1], ds[g:g + 1], 1, 64)[0]
    got = tensor_bits(Wm[rows])
    ref = orc.lora_merge(Wdq_rows, lay.A, lay.B[rows], alpha)
    s = alpha / lay.r
    exact = _f64(Wdq_rows) + s * (_f64(lay.B[rows]) @ _f64(lay.A))
    mag = np.abs(_f64(Wdq_rows)) + abs(s) * (np.abs(_f64(lay.B[rows])) @ np.abs(_f64(lay.A)))
    check_rounded(got, ref, exact, mag, "merge full size")
