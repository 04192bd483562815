"""The allocation-free backward (qlora_linear_bwd_noalloc) against the
backward with a caller workspace (qlora_linear_bwd), through the C ABI.

Both run the same kernels in the same order, so dX, dA and dB must agree bit
for bit.  Two calls in a row share the GPU's scratch array: the second, with
a smaller input, must not see anything the first left there.  The forward's
saved T is passed on one call and recomputed in the scratch on the other."""
import ctypes

import numpy as np
import pytest

import synthetic_inputs as si
from helpers import GpuLayer, log, tensor_bits

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
if not torch.cuda.is_available():  # pragma: no cover
    pytest.skip("needs a GPU", allow_module_level=True)

import bit_nf4_quantized_17_amd as q  # noqa: E402


def _compare(layer: GpuLayer, use_T: bool, label: str):
    M, N, K, r = layer.M, layer.N, layer.K, layer.r
    T = None
    if use_T:
        _, T = q.qlora_linear_fwd(layer.w, layer.dX_in, layer.dA_in, layer.dB_in, layer.alpha)
    ref = q.qlora_linear_bwd(layer.w, layer.dX_in, layer.ddY, layer.dA_in, layer.dB_in, layer.alpha, T=T)
    dX = torch.empty(M, K, dtype=torch.bfloat16, device="cuda")
    dA = torch.empty(r, K, dtype=torch.bfloat16, device="cuda")
    dB = torch.empty(N, r, dtype=torch.bfloat16, device="cuda")
    log(f"[noalloc] {label}: M={M} N={N} K={K} r={r} T_saved={use_T} "
        f"scratch need={q.qlora_bwd_workspace_bytes(M, N, K, r)} B")
    q.qlora_linear_bwd_noalloc(layer.w, layer.dX_in, layer.ddY, layer.dA_in, layer.dB_in, layer.alpha,
                               dX, dA, dB, T=T)
    torch.cuda.synchronize()
    for name, got, want in (("dX", dX, ref[0]), ("dA", dA, ref[1]), ("dB", dB, ref[2])):
        g, w = tensor_bits(got), tensor_bits(want)
        bad = np.count_nonzero(g != w)
        assert bad == 0, f"{label} {name}: {bad} of {g.size} elements differ from qlora_linear_bwd"


def test_noalloc_matches_workspace_backward_twice():
    big = GpuLayer(si.custom(N=3000, K=2304, M=1100, r=64, alpha=16.0, seed=7))
    small = GpuLayer(si.custom(N=256, K=256, M=16, r=8, alpha=16.0, seed=0))
    assert q.qlora_bwd_workspace_bytes(big.M, big.N, big.K, big.r) > \
        q.qlora_bwd_workspace_bytes(small.M, small.N, small.K, small.r)
    _compare(big, use_T=False, label="first call (larger)")
    _compare(small, use_T=True, label="second call (smaller)")
    _compare(big, use_T=True, label="third call (larger again)")


def test_noalloc_rejects_oversize_before_launching():
    M, N, K, r = 65536, 28672, 8192, 128
    assert q.qlora_bwd_workspace_bytes(M, N, K, r) > q.QLORA_BWD_NOALLOC_MAX_BYTES
    w = q.NF4Weight.empty(N, K)
    fake = torch.empty(16, dtype=torch.uint8, device="cuda").data_ptr()
    d = w.descriptor()
    rc = q.lib().qlora_linear_bwd_noalloc(ctypes.byref(d), fake, fake, M, fake, fake, r, 16.0, q.QL_DTYPE_BF16, None,
                                          fake, fake, fake, None)
    assert rc == -5, q.lib().qlora_last_error()
    assert b"scratch" in q.lib().qlora_last_error()
