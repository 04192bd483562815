"""GPU parity of the codebook and scale-format variants through the C ABI.

Variants (the NF4 + E4M3 double-quantized default is covered by
test_gpu_parity): the INT4 comparison codebook of the Ultralytics "QLoRA"
snippet; block scales kept as fp32 (the Transformers "Bitsandbytes" 4-bit
configuration without nested quantization); and the uint8-linear reading of
the double quantization's "8 bits in blocks of 256" (Ultralytics "QLoRA");
alone and combined.  Codes, scales and the
dequantized weight must match the oracle bit for bit; forward, backward,
decode-size forward, merge and the dual projection are held to the same bars
as the default format."""
import numpy as np
import pytest

import synthetic_inputs as si
from helpers import assert_close, bf16_tensor, log, tensor_bits, tensor_f64

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
if not torch.cuda.is_available():  # pragma: no cover
    pytest.skip("needs a GPU", allow_module_level=True)

import bit_nf4_quantized_17_amd as q  # noqa: E402

FORMATS = [("nf4", False, "e4m3"), ("int4", True, "e4m3"), ("int4", False, "e4m3"),
           ("nf4", True, "uint8"), ("int4", True, "uint8")]
FMT_IDS = ["nf4-fp32scale", "int4-dq", "int4-fp32scale", "nf4-u8dq", "int4-u8dq"]


def _quantize(orc, W, codebook, dq, label, fmt="e4m3"):
    """GPU quantize + dequantize against the oracle, bit for bit; returns the
    GPU weight and the oracle's dequantized bf16 weight."""
    dW = torch.from_numpy(np.ascontiguousarray(W)).cuda()
    absmax = torch.empty(W.size // 64, dtype=torch.float32, device="cuda")
    w = q.nf4_quantize(dW, absmax=absmax, codebook=codebook, double_quant=dq, dq_format=fmt)
    rc, rq, rd, ra = orc.quantize(W, codebook, double_quant=dq, dq_format=fmt)
    assert np.array_equal(w.codes.cpu().numpy(), rc), f"{label}: codes differ"
    assert np.array_equal(absmax.cpu().numpy().view(np.uint32), ra.view(np.uint32)), f"{label}: absmax"
    assert np.array_equal(w.dscale.cpu().numpy().view(np.uint32), rd.view(np.uint32)), f"{label}: dscale"
    if dq:
        assert np.array_equal(w.qscale.cpu().numpy(), rq), f"{label}: qscale differs"
    else:
        assert w.qscale is None
    ref = orc.dequantize(rc, rq, rd, *W.shape, codebook=codebook, dq_format=fmt)
    assert np.array_equal(tensor_bits(q.nf4_dequantize(w)), ref), f"{label}: dequantized bf16 differs"
    return w, ref


@pytest.mark.parametrize("codebook,dq,fmt", FORMATS, ids=FMT_IDS)
@pytest.mark.parametrize("N,K,outliers", [(300, 256, 0.01), (513, 1088, 0.01), (7, 320, 0.0)])
def test_quantize_formats_bitwise(orc, codebook, dq, fmt, N, K, outliers):
    cfg = si.custom(N=N, K=K, M=1, r=8, outlier_frac=outliers, seed=N + 2 * K)
    log(f"[quantize {codebook} dq={dq} {fmt}] {N}x{K}")
    _quantize(orc, si.weight(cfg, 0), codebook, dq, f"{codebook} dq={dq} {fmt} {N}x{K}", fmt)


@pytest.mark.parametrize("codebook,dq,fmt", FORMATS, ids=FMT_IDS)
def test_quantize_formats_zero_blocks_and_ties(orc, codebook, dq, fmt):
    """All-zero blocks (two whole groups) take the code of v = 0; values on the
    codebook's decision points and its levels times powers of two."""
    L = orc.codebook_levels(codebook)
    W = np.zeros((64, 512), np.float32)
    W[40, 100] = 1e-3
    rng = np.random.default_rng(4)
    for row in range(48, 64):
        e = float(rng.integers(-30, 30))
        mids = (L[:-1].astype(np.float64) + L[1:]) / 2
        vals = np.concatenate([L, mids.astype(np.float32), -L[::-1]]).astype(np.float32)
        W[row, :vals.size] = vals * np.float32(2.0 ** e)
        W[row, 64:128] = np.tile(L, 4) * np.float32(2.0 ** (e / 2))
    _quantize(orc, W, codebook, dq, f"{codebook} dq={dq} {fmt} edge", fmt)


SHAPES = [
    # N, K, M, r, alpha
    (130, 320, 129, 17, 34.0),    # ragged tiles in every dimension
    (384, 512, 257, 64, 16.0),
    (1000, 512, 3, 8, 16.0),      # decode size (the streaming kernel, factored form)
    (4100, 2304, 7, 64, 16.0),    # decode size, T precomputed
    (600, 8448, 5, 24, 16.0),     # decode size, K > 8192: the streaming kernel's exact form
]


@pytest.mark.parametrize("codebook,dq,fmt", FORMATS, ids=FMT_IDS)
@pytest.mark.parametrize("N,K,M,r,alpha", SHAPES)
def test_fwd_bwd_formats(orc, codebook, dq, fmt, N, K, M, r, alpha):
    cfg = si.custom(N=N, K=K, M=M, r=r, alpha=alpha, seed=5 * N + K)
    label = f"{codebook} dq={dq} {fmt} N={N} K={K} M={M} r={r}"
    log(f"[fwd/bwd] {label}")
    w, Wdq = _quantize(orc, si.weight(cfg, 0), codebook, dq, label, fmt)
    X, A, B, dY = si.activations(cfg, 0), *si.adapters(cfg, 0), si.upstream(cfg, 0)
    dXin, dA_in, dB_in, ddY = bf16_tensor(X), bf16_tensor(A), bf16_tensor(B), bf16_tensor(dY)
    Y, T = q.qlora_linear_fwd(w, dXin, dA_in, dB_in, alpha)
    torch.cuda.synchronize()
    Yr, Tr = orc.qlora_fwd(Wdq, X, A, B, alpha)
    assert_close(tensor_f64(T), Tr, "T")
    assert_close(tensor_f64(Y), Yr, "Y")
    dX, dA, dB = q.qlora_linear_bwd(w, dXin, ddY, dA_in, dB_in, alpha, T=T)
    torch.cuda.synchronize()
    assert_close(tensor_f64(dX), orc.qlora_bwd_dx(Wdq, dY, A, B, alpha), "dX")
    dAr, dBr = orc.qlora_bwd_adapters(X, dY, A, B, alpha)
    assert_close(tensor_f64(dA), dAr, "dA")
    assert_close(tensor_f64(dB), dBr, "dB")


@pytest.mark.parametrize("codebook,dq,fmt", FORMATS, ids=FMT_IDS)
def test_merge_formats(orc, codebook, dq, fmt):
    """Merge with a zero B gives the dequantized weight bit for bit; with the
    adapter, every element is within the merge's rounding bound of the exact
    W' + s B A (the bar of test_gpu_merge)."""
    from test_gpu_merge import check_rounded
    N, K, r, alpha = 300, 320, 16, 32.0
    cfg = si.custom(N=N, K=K, M=1, r=r, alpha=alpha, seed=12)
    w, Wdq = _quantize(orc, si.weight(cfg, 0), codebook, dq, f"merge {codebook} dq={dq} {fmt}", fmt)
    A, B = si.adapters(cfg, 0)
    dA_in, dB_in = bf16_tensor(A), bf16_tensor(B)
    Wz = q.qlora_merge(w, dA_in, torch.zeros_like(dB_in), alpha)
    Wm = q.qlora_merge(w, dA_in, dB_in, alpha)
    torch.cuda.synchronize()
    assert np.array_equal(tensor_bits(Wz), Wdq)
    f64 = lambda h: si.bf16_bits_to_f32(h).astype(np.float64)  # noqa: E731
    s = alpha / r
    exact = f64(Wdq) + s * (f64(B) @ f64(A))
    mag = np.abs(f64(Wdq)) + abs(s) * (np.abs(f64(B)) @ np.abs(f64(A)))
    check_rounded(tensor_bits(Wm), orc.lora_merge(Wdq, A, B, alpha), exact, mag, f"merge {codebook} dq={dq}")


@pytest.mark.parametrize("gate,up", [(("int4", True, "e4m3"), ("nf4", False, "e4m3")),
                                     (("nf4", True, "uint8"), ("int4", True, "e4m3"))],
                         ids=["int4e4m3-nf4fp32", "nf4u8-int4e4m3"])
def test_dual_mixed_formats_match_single_calls(orc, gate, up):
    """A dual projection whose gate and up weights have different codebooks
    and scale formats: each wave decodes its own weight's format, and the
    outputs equal two single forwards bit for bit."""
    N, K, M, r, alpha = 320, 512, 96, 16, 32.0
    cg = si.custom(N=N, K=K, M=M, r=r, alpha=alpha, seed=21)
    cu = si.custom(N=N, K=K, M=M, r=r, alpha=alpha, seed=22)
    wg, Wg = _quantize(orc, si.weight(cg, 0), gate[0], gate[1], "dual gate", gate[2])
    wu, Wu = _quantize(orc, si.weight(cu, 0), up[0], up[1], "dual up", up[2])
    X = si.activations(cg, 0)
    Ag, Bg = si.adapters(cg, 0)
    Au, Bu = si.adapters(cu, 0)
    t = [bf16_tensor(a) for a in (X, Ag, Bg, Au, Bu)]
    Yg, Yu, _, _ = q.qlora_dual_fwd(wg, wu, *t, alpha)
    Ys, _ = q.qlora_linear_fwd(wg, t[0], t[1], t[2], alpha)
    Yus, _ = q.qlora_linear_fwd(wu, t[0], t[3], t[4], alpha)
    torch.cuda.synchronize()
    assert np.array_equal(tensor_bits(Yg), tensor_bits(Ys))
    assert np.array_equal(tensor_bits(Yu), tensor_bits(Yus))
    Gr, _ = orc.qlora_fwd(Wg, X, Ag, Bg, alpha)
    assert_close(tensor_f64(Yg), Gr, "Y_gate")
    Ur, _ = orc.qlora_fwd(Wu, X, Au, Bu, alpha)
    assert_close(tensor_f64(Yu), Ur, "Y_up")


@pytest.mark.parametrize("fmt", ["uint8", "e4m3"])
def test_quantize_dq_formats_at_a_workload_size(orc, fmt):
    """The 7B attention projection's weight (4096 x 4096, N(0, 0.02)) in both
    8-bit scale formats, bit for bit, with a decode-size forward (M = 4)."""
    cfg = si.CONFIGS["attn_4096"]
    W = si.weight(cfg, 0)
    log(f"[quantize {fmt}] 4096x4096")
    w, Wdq = _quantize(orc, W, "nf4", True, f"attn7b {fmt}", fmt)
    X = si.activations(cfg, 0, 4)
    A, B = si.adapters(cfg, 0)
    Y, T = q.qlora_linear_fwd(w, bf16_tensor(X), bf16_tensor(A), bf16_tensor(B), cfg.alpha)
    torch.cuda.synchronize()
    Yr, Tr = orc.qlora_fwd(Wdq, X, A, B, cfg.alpha)
    assert_close(tensor_f64(Y), Yr, f"Y {fmt}")
