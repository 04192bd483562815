"""GPU parity of the fused fallback kernels, through the C ABI.

The buffer-load GEMMs take operands whose byte offsets fit in 32 bits; larger
activations go to the tile-128 fused kernels (guarded 64-bit loads), with the
same arithmetic.  These tests reach those kernels with a 2 GiB activation:
X (forward) or dY (backward) of 2^30 bf16 elements.  The big operand repeats a
seeded 512-row block, so the oracle computes the sampled rows from that block;
everything else is at its real shape."""
import numpy as np
import pytest

import synthetic_inputs as si
from helpers import assert_close, bf16_tensor, log, tensor_f64

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
if not torch.cuda.is_available():  # pragma: no cover
    pytest.skip("needs a GPU", allow_module_level=True)

import bit_nf4_quantized_17_amd as q  # noqa: E402

BLOCK = 512


def _rows(M, seed):
    rng = np.random.default_rng(seed)
    return sorted({0, M - 1, BLOCK - 1, BLOCK, *(int(x) for x in rng.integers(0, M, 6))})


def _layer(orc, N, K, r, alpha, seed):
    cfg = si.custom(N=N, K=K, M=BLOCK, r=r, alpha=alpha, seed=seed)
    W = si.weight(cfg, 0)
    w = q.nf4_quantize(torch.from_numpy(W).cuda())
    Wdq = orc.nf4_dequantize(w.codes.cpu().numpy(), w.qscale.cpu().numpy(), w.dscale.cpu().numpy(), N, K)
    A, B = si.adapters(cfg, 0)
    return cfg, w, Wdq, A, B


def test_forward_with_a_2gib_activation(orc):
    """M = 262144, K = 4096: X is 2 GiB, so the forward runs the tile-128
    fused kernel (NF4 producer, T B^T prologue)."""
    M, N, K, r, alpha = 262144, 320, 4096, 16, 32.0
    cfg, w, Wdq, A, B = _layer(orc, N, K, r, alpha, seed=41)
    Xs = si.activations(cfg, 0)                                    # [512][K], repeated
    X = bf16_tensor(Xs).repeat(M // BLOCK, 1)
    assert X.numel() * 2 >= 2**31
    log(f"[large fwd] M={M} N={N} K={K} r={r}")
    Y, T = q.qlora_linear_fwd(w, X, bf16_tensor(A), bf16_tensor(B), alpha)
    torch.cuda.synchronize()
    rows = _rows(M, 1)
    Yr, Tr = orc.qlora_fwd(Wdq, Xs[[m % BLOCK for m in rows]], A, B, alpha)
    sel = torch.tensor(rows, device="cuda")
    assert_close(tensor_f64(Y.index_select(0, sel)), Yr, "Y rows")
    assert_close(T.index_select(0, sel).cpu().numpy(), Tr, "T rows")


def test_backward_dx_with_a_2gib_gradient(orc):
    """M = 131072, N = 8192: dY is 2 GiB, so dX runs the tile-128 fused kernel
    (transposed NF4 producer, U A prologue)."""
    M, N, K, r, alpha = 131072, 8192, 64, 8, 16.0
    cfg, w, Wdq, A, B = _layer(orc, N, K, r, alpha, seed=43)
    Xs, dYs = si.activations(cfg, 0), si.upstream(cfg, 0)          # [512][K], [512][N], repeated
    X = bf16_tensor(Xs).repeat(M // BLOCK, 1)
    dY = bf16_tensor(dYs).repeat(M // BLOCK, 1)
    assert dY.numel() * 2 >= 2**31
    log(f"[large bwd] M={M} N={N} K={K} r={r}")
    dA_in, dB_in = bf16_tensor(A), bf16_tensor(B)
    _, T = q.qlora_linear_fwd(w, X, dA_in, dB_in, alpha)
    dX, dA, dB = q.qlora_linear_bwd(w, X, dY, dA_in, dB_in, alpha, T=T)
    torch.cuda.synchronize()
    rows = _rows(M, 2)
    dXr = orc.qlora_bwd_dx(Wdq, dYs[[m % BLOCK for m in rows]], A, B, alpha)
    sel = torch.tensor(rows, device="cuda")
    assert_close(tensor_f64(dX.index_select(0, sel)), dXr, "dX rows")
    # The adapters' gradients sum M / 512 copies of the block's sums.  Each
    # entry is a sum of 131072 products, and an entry that cancels to a small
    # value keeps the fp32 summation error of the large terms, which the
    # elementwise bar (relative to the entry itself) does not allow for; they
    # are held to the relative Frobenius bar.
    dAr, dBr = orc.qlora_bwd_adapters(Xs, dYs, A, B, alpha)
    for got, ref, name in ((tensor_f64(dA), dAr * (M // BLOCK), "dA"), (tensor_f64(dB), dBr * (M // BLOCK), "dB")):
        rel = float(np.linalg.norm(got - ref) / np.linalg.norm(ref))
        assert rel <= 5e-3, f"{name}: relative Frobenius error {rel:.3e}"


def test_dual_projection_slices_a_2gib_activation(orc):
    """The dual forward cuts M into slices whose X fits the 32-bit offsets
    (here two: 261632 rows and 512); rows on both sides of the cut against the
    oracle, per projection and for silu(G) U."""
    M, N, K, r, alpha = 262144, 320, 4096, 16, 32.0
    cfg, wg, Wg, Ag, Bg = _layer(orc, N, K, r, alpha, seed=45)
    _, wu, Wu, Au, Bu = _layer(orc, N, K, r, alpha, seed=46)
    Xs = si.activations(cfg, 0)
    X = bf16_tensor(Xs).repeat(M // BLOCK, 1)
    t = [bf16_tensor(a) for a in (Ag, Bg, Au, Bu)]
    log(f"[large dual] M={M} N={N} K={K} r={r}")
    Yg, Yu, Tg, Tu = q.qlora_dual_fwd(wg, wu, X, *t, alpha)
    H, _, _ = q.qlora_dual_fwd(wg, wu, X, *t, alpha, swiglu=True)
    torch.cuda.synchronize()
    rows = sorted(set(_rows(M, 3)) | {261631, 261632, 261633})
    xr = Xs[[m % BLOCK for m in rows]]
    Gr, Tgr = orc.qlora_fwd(Wg, xr, Ag, Bg, alpha)
    Ur, Tur = orc.qlora_fwd(Wu, xr, Au, Bu, alpha)
    sel = torch.tensor(rows, device="cuda")
    assert_close(tensor_f64(Yg.index_select(0, sel)), Gr, "Y_gate rows")
    assert_close(tensor_f64(Yu.index_select(0, sel)), Ur, "Y_up rows")
    assert_close(Tg.index_select(0, sel).cpu().numpy(), Tgr, "T_gate rows")
    assert_close(tensor_f64(H.index_select(0, sel)), orc.swiglu(Gr, Ur), "H rows")
