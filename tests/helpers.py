"""Shared helpers of the tests: moving seeded inputs to the GPU, and the
floating-point parity bar.

Parity bar for fwd/bwd outputs (Y, dX, dA, dB), from the layer's accuracy
target: relative Frobenius error <= 5e-3 AND elementwise
|got - ref| <= 2e-2 * (1 + |ref|), where ref is the oracle's double result
and got the library's bf16 output.  Codes, scale bytes, group constants and
dequantized weights must match bit for bit."""
from __future__ import annotations

import sys

import numpy as np

REL_FRO = 5e-3
ELEM_ABS = 2e-2


def log(msg: str):
    print(msg, flush=True)
    sys.stdout.flush()


from synthetic_inputs import bf16_tensor, tensor_bits  # noqa: E402,F401  (re-exported for the tests)


def tensor_f64(t) -> np.ndarray:
    return t.detach().float().cpu().numpy().astype(np.float64)


def assert_close(got: np.ndarray, ref: np.ndarray, what: str):
    got = np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    assert got.shape == ref.shape, (what, got.shape, ref.shape)
    assert np.all(np.isfinite(got)), f"{what}: non-finite output"
    err = got - ref
    nref = float(np.linalg.norm(ref))
    rel = float(np.linalg.norm(err)) / nref if nref > 0 else float(np.linalg.norm(err))
    bound = ELEM_ABS * (1.0 + np.abs(ref))
    worst = float(np.max(np.abs(err) / bound)) if err.size else 0.0
    assert rel <= REL_FRO, f"{what}: relative Frobenius error {rel:.3e} > {REL_FRO}"
    assert worst <= 1.0, f"{what}: elementwise error reaches {worst:.3f} of the bound"
    return rel, worst


class GpuLayer:
    """One layer's seeded inputs on the GPU plus the host copies the oracle uses."""

    def __init__(self, cfg, li: int = 0, M: int | None = None, quantize: bool = True):
        import torch
        import synthetic_inputs as si
        import bit_nf4_quantized_17_amd as q
        self.cfg = cfg
        L = cfg.layers[li]
        self.N, self.K = L.N, L.K
        self.M = cfg.M if M is None else M
        self.r, self.alpha = cfg.r, cfg.alpha
        self.W = si.weight(cfg, li)
        self.X = si.activations(cfg, li, self.M)
        self.A, self.B = si.adapters(cfg, li)
        self.dY = si.upstream(cfg, li, self.M)
        self.dW = torch.from_numpy(self.W).cuda()
        self.dX_in = bf16_tensor(self.X)
        self.dA_in = bf16_tensor(self.A)
        self.dB_in = bf16_tensor(self.B)
        self.ddY = bf16_tensor(self.dY)
        self.w = q.nf4_quantize(self.dW) if quantize else None
