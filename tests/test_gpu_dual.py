"""GPU parity of the gate/up dual projection (qlora_dual_fwd) through the C ABI.

Each of the two outputs is the QLoRA forward of its own weight and adapter,
so the oracle is the single-layer forward applied per projection, and the
SwiGLU output is the oracle's silu(G) * U of those two exact results.  The
dual kernel sums the same products in the same order as qlora_linear_fwd's
tiled kernel (the other projection's half of the shared LoRA prologue adds
exact zeros), so for M > 16 its two outputs must equal the single calls bit
for bit."""
import numpy as np
import pytest

import synthetic_inputs as si
from helpers import GpuLayer, assert_close, log, tensor_bits, tensor_f64

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
if not torch.cuda.is_available():  # pragma: no cover
    pytest.skip("needs a GPU", allow_module_level=True)

import bit_nf4_quantized_17_amd as q  # noqa: E402


def _pair(N, K, M, r, alpha, seed):
    """Gate and up layers of one shape with independent weights and adapters,
    both reading the gate layer's X."""
    gate = GpuLayer(si.custom(N=N, K=K, M=M, r=r, alpha=alpha, seed=seed))
    up = GpuLayer(si.custom(N=N, K=K, M=M, r=r, alpha=alpha, seed=seed + 7919))
    return gate, up


def _dequant_host(orc, lay):
    w = lay.w
    return orc.nf4_dequantize(w.codes.cpu().numpy(), w.qscale.cpu().numpy(), w.dscale.cpu().numpy(),
                              lay.N, lay.K)


DUAL = [
    # M, N, K, r
    (257, 256, 256, 8),      # one column tile of each weight, ragged M
    (300, 200, 320, 3),      # ragged N inside a 32-row slice, odd rank
    (129, 520, 384, 16),     # several column tiles, a partial last one
    (64, 128, 512, 64),      # two prologue steps of 64
    (33, 96, 1024, 128),     # the largest rank: four prologue steps
    (5, 160, 256, 12),       # decode-size M still runs the tiled kernel
]


@pytest.mark.parametrize("M,N,K,r", DUAL)
def test_dual_matches_single_and_oracle(orc, M, N, K, r):
    alpha = 2.0 * r
    gate, up = _pair(N, K, M, r, alpha, seed=M + N + K + r)
    X = gate.dX_in
    log(f"[dual] M={M} N={N} K={K} r={r}")
    Yg, Yu, Tg, Tu = q.qlora_dual_fwd(gate.w, up.w, X, gate.dA_in, gate.dB_in, up.dA_in, up.dB_in, alpha)
    H, Tg2, Tu2 = q.qlora_dual_fwd(gate.w, up.w, X, gate.dA_in, gate.dB_in, up.dA_in, up.dB_in, alpha,
                                   swiglu=True)
    torch.cuda.synchronize()
    assert torch.equal(Tg, Tg2) and torch.equal(Tu, Tu2)

    # each output against the single-projection oracle
    rows = np.arange(M, dtype=np.int64)
    Gref, Tgref = orc.qlora_fwd(_dequant_host(orc, gate), gate.X, gate.A, gate.B, alpha, rows=rows)
    Uref, Turef = orc.qlora_fwd(_dequant_host(orc, up), gate.X, up.A, up.B, alpha, rows=rows)
    assert_close(tensor_f64(Yg), Gref, "Y_gate")
    assert_close(tensor_f64(Yu), Uref, "Y_up")
    assert_close(Tg.cpu().numpy(), Tgref, "T_gate")
    assert_close(Tu.cpu().numpy(), Turef, "T_up")
    assert_close(tensor_f64(H), orc.swiglu(Gref, Uref), "H = silu(G) U")

    # the tiled single-projection forward gives the same bits (decode sizes
    # take another kernel there)
    if M > 16:
        Ys, Ts = q.qlora_linear_fwd(gate.w, X, gate.dA_in, gate.dB_in, alpha)
        Yus, Tus = q.qlora_linear_fwd(up.w, X, up.dA_in, up.dB_in, alpha)
        torch.cuda.synchronize()
        assert np.array_equal(tensor_bits(Yg), tensor_bits(Ys)), "Y_gate differs from qlora_linear_fwd"
        assert np.array_equal(tensor_bits(Yu), tensor_bits(Yus)), "Y_up differs from qlora_linear_fwd"
        assert torch.equal(Tg, Ts) and torch.equal(Tu, Tus)


def test_dual_swapped_weights_swap_outputs(orc):
    """Passing up as gate and gate as up exchanges the two outputs exactly."""
    gate, up = _pair(192, 256, 96, 16, 32.0, seed=11)
    X = gate.dX_in
    Yg, Yu, _, _ = q.qlora_dual_fwd(gate.w, up.w, X, gate.dA_in, gate.dB_in, up.dA_in, up.dB_in, 32.0)
    Zg, Zu, _, _ = q.qlora_dual_fwd(up.w, gate.w, X, up.dA_in, up.dB_in, gate.dA_in, gate.dB_in, 32.0)
    torch.cuda.synchronize()
    assert torch.equal(Yg, Zu) and torch.equal(Yu, Zg)


def test_dual_full_size_sampled_rows(orc):
    """Gate and up projections of the 70B-class MLP (two 28672x8192 weights,
    4096 tokens, r = 64): the whole dual forward on the GPU, sampled rows of
    G, U and H against the oracle."""
    cfg = si.CONFIGS["mlp70b_28672"]
    gate = GpuLayer(cfg, 0)
    up_cfg = si.custom(N=gate.N, K=gate.K, M=gate.M, r=gate.r, alpha=gate.alpha, seed=cfg.seed + 101,
                       outlier_frac=cfg.outlier_frac)
    up = GpuLayer(up_cfg)
    X = gate.dX_in
    log(f"[dual full size] M={gate.M} N={gate.N} K={gate.K} r={gate.r}")
    Yg, Yu, Tg, Tu = q.qlora_dual_fwd(gate.w, up.w, X, gate.dA_in, gate.dB_in, up.dA_in, up.dB_in,
                                      gate.alpha)
    H, _, _ = q.qlora_dual_fwd(gate.w, up.w, X, gate.dA_in, gate.dB_in, up.dA_in, up.dB_in, gate.alpha,
                               swiglu=True)
    torch.cuda.synchronize()
    rng = np.random.default_rng(3)
    rows = np.array(sorted({0, gate.M - 1, *(int(x) for x in rng.integers(0, gate.M, 4))}), np.int64)
    Gref, _ = orc.qlora_fwd(_dequant_host(orc, gate), gate.X, gate.A, gate.B, gate.alpha, rows=rows)
    Uref, _ = orc.qlora_fwd(_dequant_host(orc, up), gate.X, up.A, up.B, gate.alpha, rows=rows)
    sel = torch.from_numpy(rows).cuda()
    assert_close(tensor_f64(Yg.index_select(0, sel)), Gref, "Y_gate rows")
    assert_close(tensor_f64(Yu.index_select(0, sel)), Uref, "Y_up rows")
    assert_close(tensor_f64(H.index_select(0, sel)), orc.swiglu(Gref, Uref), "H rows")
