"""MI355X (gfx950) QLoRA NF4 linear layer -- Python binding of libqlora_nf4.

Argument marshalling only: every step of the layer runs in the HIP kernels of
``libqlora_nf4.so`` behind the C ABI of ``include/qlora_nf4.h``.  PyTorch is
used for device memory and the current HIP stream.  There is no fallback: if
the library is missing or fails to load, every call raises.

Functions keep the C ABI's names:
  nf4_levels, nf4_storage_bytes, nf4_quantize, nf4_dequantize,
  qlora_fwd_workspace_bytes, qlora_linear_fwd,
  qlora_bwd_workspace_bytes, qlora_linear_bwd, qlora_linear_bwd_noalloc,
  qlora_abi_version
"""
from __future__ import annotations

import ctypes
import dataclasses
import os
from typing import Optional, Tuple

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libqlora_nf4.so")

QL_DTYPE_BF16 = 1
QL_CODEBOOK_NF4 = 0
QL_CODEBOOK_INT4 = 1
CODEBOOKS = {"nf4": QL_CODEBOOK_NF4, "int4": QL_CODEBOOK_INT4}
QL_DQ_E4M3 = 0
QL_DQ_UINT8 = 1
DQ_FORMATS = {"e4m3": QL_DQ_E4M3, "uint8": QL_DQ_UINT8}
QL_DUAL_SEPARATE = 1
QL_DUAL_SWIGLU = 2
QLORA_MAX_RANK = 128
QLORA_BWD_NOALLOC_MAX_BYTES = 32 << 20
_STATUS = {0: "QL_OK", -1: "QL_ERR_NULL", -2: "QL_ERR_SHAPE", -3: "QL_ERR_UNSUPPORTED",
           -4: "QL_ERR_ALIGN", -5: "QL_ERR_WORKSPACE", -6: "QL_ERR_HIP"}

_lib = None


class QLoRAError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(f"{_STATUS.get(status, status)}: {message}")
        self.status = status


class _AdamwTensor(ctypes.Structure):
    _fields_ = [("param", ctypes.c_void_p), ("grad", ctypes.c_void_p), ("exp_avg", ctypes.c_void_p),
                ("exp_avg_sq", ctypes.c_void_p), ("master", ctypes.c_void_p), ("numel", ctypes.c_int64)]


class _Weight(ctypes.Structure):
    _fields_ = [("codes", ctypes.c_void_p), ("qscale", ctypes.c_void_p),
                ("dscale", ctypes.c_void_p), ("rows", ctypes.c_int64), ("cols", ctypes.c_int64),
                ("block", ctypes.c_int32), ("dq_block", ctypes.c_int32), ("codebook", ctypes.c_int32),
                ("dq_format", ctypes.c_int32)]


def lib() -> ctypes.CDLL:
    """Load libqlora_nf4.so (built by build.py); raises if it is not there."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"{LIB_PATH} is not built; run python -m bit_nf4_quantized_17_amd.build")
    L = ctypes.CDLL(LIB_PATH)
    P, I64, I, F, SZ = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int, ctypes.c_float, ctypes.c_size_t
    WP = ctypes.POINTER(_Weight)
    L.qlora_abi_version.argtypes, L.qlora_abi_version.restype = [], I
    L.qlora_last_error.argtypes, L.qlora_last_error.restype = [], ctypes.c_char_p
    L.nf4_levels.argtypes, L.nf4_levels.restype = [P], None
    L.nf4_storage_bytes.argtypes = [I64, I64, I, I, P, P, P]
    L.nf4_storage_bytes.restype = I
    L.nf4_quantize.argtypes = [P, I64, I64, I, I, P, P, P, P, P]
    L.nf4_quantize.restype = I
    L.qlora_quantize.argtypes = [P, I64, I64, I, I, I, P, P, P, P, P]
    L.qlora_quantize.restype = I
    L.qlora_codebook_levels.argtypes = [I, P]
    L.qlora_codebook_levels.restype = I
    L.nf4_dequantize.argtypes = [WP, P, P]
    L.nf4_dequantize.restype = I
    L.qlora_fwd_workspace_bytes.argtypes = [I64, I64, I64, I]
    L.qlora_fwd_workspace_bytes.restype = SZ
    L.qlora_linear_fwd.argtypes = [WP, P, I64, P, P, I, F, I, P, P, P, SZ, P]
    L.qlora_linear_fwd.restype = I
    L.qlora_dual_fwd.argtypes = [WP, WP, P, I64, P, P, P, P, I, F, I, I, P, P, P, P, P, P, SZ, P]
    L.qlora_dual_fwd.restype = I
    L.qlora_adamw_step.argtypes = [P, I, F, F, F, F, F, I, P]
    L.qlora_adamw_step.restype = I
    L.qlora_bwd_workspace_bytes.argtypes = [I64, I64, I64, I]
    L.qlora_bwd_workspace_bytes.restype = SZ
    L.qlora_linear_bwd.argtypes = [WP, P, P, I64, P, P, I, F, I, P, P, P, P, P, SZ, P]
    L.qlora_linear_bwd.restype = I
    L.qlora_linear_bwd_noalloc.argtypes = [WP, P, P, I64, P, P, I, F, I, P, P, P, P, P]
    L.qlora_linear_bwd_noalloc.restype = I
    L.qlora_merge.argtypes = [WP, P, P, I, F, P, P]
    L.qlora_merge.restype = I
    L.qlora_unmerge.argtypes = [P, I64, I64, P, P, I, F, P, P]
    L.qlora_unmerge.restype = I
    L.qlora_set_timing_events.argtypes = [P, P, P, P]
    L.qlora_set_timing_events.restype = I
    _lib = L
    return L


def _check(rc: int):
    if rc != 0:
        raise QLoRAError(rc, lib().qlora_last_error().decode())


def _stream(stream):
    import torch
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream)


def _ptr(t) -> Optional[int]:
    return None if t is None else t.data_ptr()


def _need(t, dtype, shape, name):
    if tuple(t.shape) != tuple(shape) or t.dtype != dtype or not t.is_contiguous() or not t.is_cuda:
        raise ValueError(f"{name}: expected contiguous cuda {dtype} {tuple(shape)}, "
                         f"got {t.dtype} {tuple(t.shape)} on {t.device}")


def qlora_set_timing_events(fwd_begin=None, fwd_end=None, dx_begin=None, dx_end=None) -> None:
    """Raw hipEvent_t handles (ints) recorded around the main GEMM kernels of
    later calls on this thread; all None clears the hook."""
    _check(lib().qlora_set_timing_events(fwd_begin, fwd_end, dx_begin, dx_end))


def qlora_abi_version() -> int:
    return lib().qlora_abi_version()


def nf4_levels():
    """The 16 fp32 NF4 levels in code order (a list of floats)."""
    buf = (ctypes.c_float * 16)()
    lib().nf4_levels(ctypes.cast(buf, ctypes.c_void_p))
    return list(buf)


def codebook_levels(codebook: str = "nf4"):
    """The 16 fp32 levels of a codebook ("nf4" or "int4") in code order."""
    buf = (ctypes.c_float * 16)()
    _check(lib().qlora_codebook_levels(CODEBOOKS[codebook], ctypes.cast(buf, ctypes.c_void_p)))
    return list(buf)


def nf4_storage_bytes(rows: int, cols: int, block: int = 64, dq_block: int = 256):
    c, q, d = ctypes.c_size_t(), ctypes.c_size_t(), ctypes.c_size_t()
    _check(lib().nf4_storage_bytes(rows, cols, block, dq_block, ctypes.byref(c), ctypes.byref(q),
                                   ctypes.byref(d)))
    return c.value, q.value, d.value


@dataclasses.dataclass
class NF4Weight:
    """A quantized frozen weight [rows][cols] held in device tensors.  With
    double_quant the block scales are 8-bit codes in qscale (dq_format "e4m3" or
    "uint8") and group constants in dscale; without, qscale is None and dscale
    holds the fp32 block scales."""
    codes: "torch.Tensor"              # uint8 [rows*cols/2]
    qscale: Optional["torch.Tensor"]   # uint8 [rows*cols/64], or None
    dscale: "torch.Tensor"             # float32 [ceil(nb/256)], or [nb]
    rows: int
    cols: int
    codebook: str = "nf4"
    dq_format: str = "e4m3"

    @property
    def double_quant(self) -> bool:
        return self.qscale is not None

    def validate(self) -> None:
        """Raise ValueError unless every buffer is a contiguous cuda tensor of the
        dtype and element count nf4_storage_bytes gives for [rows][cols], all on
        one device: the kernels index these buffers by the descriptor's shape."""
        import torch
        if self.codebook not in CODEBOOKS:
            raise ValueError(f"unknown codebook {self.codebook!r}")
        if self.dq_format not in DQ_FORMATS:
            raise ValueError(f"unknown dq_format {self.dq_format!r}")
        c, q, d = nf4_storage_bytes(self.rows, self.cols, 64, 256 if self.double_quant else 0)
        _need(self.codes, torch.uint8, (c,), "codes")
        if self.qscale is not None:
            _need(self.qscale, torch.uint8, (q,), "qscale")
        _need(self.dscale, torch.float32, (d // 4,), "dscale")
        devs = {t.device for t in (self.codes, self.qscale, self.dscale) if t is not None}
        if len(devs) != 1:
            raise ValueError(f"weight buffers are on different devices: {sorted(map(str, devs))}")

    def descriptor(self) -> _Weight:
        self.validate()
        return _Weight(self.codes.data_ptr(), _ptr(self.qscale), self.dscale.data_ptr(),
                       self.rows, self.cols, 64, 256 if self.double_quant else 0,
                       CODEBOOKS[self.codebook], DQ_FORMATS[self.dq_format])

    @staticmethod
    def empty(rows: int, cols: int, device="cuda", codebook: str = "nf4",
              double_quant: bool = True, dq_format: str = "e4m3") -> "NF4Weight":
        import torch
        c, q, d = nf4_storage_bytes(rows, cols, 64, 256 if double_quant else 0)
        return NF4Weight(torch.empty(c, dtype=torch.uint8, device=device),
                         torch.empty(q, dtype=torch.uint8, device=device) if double_quant else None,
                         torch.empty(d // 4, dtype=torch.float32, device=device), rows, cols, codebook,
                         dq_format)


def nf4_quantize(W, out: Optional[NF4Weight] = None, absmax=None, stream=None,
                 codebook: str = "nf4", double_quant: bool = True,
                 dq_format: str = "e4m3") -> NF4Weight:
    """Quantize a cuda fp32 [rows, cols] weight with a codebook ("nf4" or "int4"),
    with double-quantized scales (default; dq_format "e4m3" or "uint8") or fp32
    block scales.  ``absmax`` (optional cuda fp32 [rows*cols/64]) receives the
    exact block scales."""
    import torch
    rows, cols = W.shape
    _need(W, torch.float32, (rows, cols), "W")
    if dq_format not in DQ_FORMATS:
        raise ValueError(f"unknown dq_format {dq_format!r}")
    if out is None:
        out = NF4Weight.empty(rows, cols, W.device, codebook, double_quant, dq_format)
    w = out
    if w.codebook != codebook or w.double_quant != double_quant or \
            (double_quant and w.dq_format != dq_format):
        raise ValueError("out has another codebook or scale format")
    if (w.rows, w.cols) != (rows, cols):
        raise ValueError(f"out holds a {w.rows}x{w.cols} weight, W is {rows}x{cols}")
    w.validate()
    if absmax is not None:
        _need(absmax, torch.float32, (rows * cols // 64,), "absmax")
    _check(lib().qlora_quantize(W.data_ptr(), rows, cols, CODEBOOKS[codebook],
                                256 if double_quant else 0, DQ_FORMATS[dq_format],
                                w.codes.data_ptr(), _ptr(w.qscale),
                                w.dscale.data_ptr(), _ptr(absmax), _stream(stream)))
    return w


def nf4_dequantize(w: NF4Weight, out=None, stream=None):
    """bf16 [rows, cols] dequantized weight."""
    import torch
    if out is None:
        out = torch.empty(w.rows, w.cols, dtype=torch.bfloat16, device=w.codes.device)
    _need(out, torch.bfloat16, (w.rows, w.cols), "out")
    d = w.descriptor()
    _check(lib().nf4_dequantize(ctypes.byref(d), out.data_ptr(), _stream(stream)))
    return out


def qlora_merge(w: NF4Weight, A, B, alpha: float, out=None, stream=None):
    """bf16 [rows, cols] = bf16(W' + (alpha/r) B A): the adapter merged into the weight."""
    import torch
    r = A.shape[0]
    _need(A, torch.bfloat16, (r, w.cols), "A")
    _need(B, torch.bfloat16, (w.rows, r), "B")
    if out is None:
        out = torch.empty(w.rows, w.cols, dtype=torch.bfloat16, device=w.codes.device)
    _need(out, torch.bfloat16, (w.rows, w.cols), "out")
    d = w.descriptor()
    _check(lib().qlora_merge(ctypes.byref(d), A.data_ptr(), B.data_ptr(), r, float(alpha),
                             out.data_ptr(), _stream(stream)))
    return out


def qlora_unmerge(W_merged, A, B, alpha: float, out=None, stream=None):
    """bf16 [rows, cols] = bf16(W_merged - (alpha/r) B A); out may be W_merged (in place)."""
    import torch
    rows, cols = W_merged.shape
    r = A.shape[0]
    _need(W_merged, torch.bfloat16, (rows, cols), "W_merged")
    _need(A, torch.bfloat16, (r, cols), "A")
    _need(B, torch.bfloat16, (rows, r), "B")
    if out is None:
        out = torch.empty_like(W_merged)
    _need(out, torch.bfloat16, (rows, cols), "out")
    _check(lib().qlora_unmerge(W_merged.data_ptr(), rows, cols, A.data_ptr(), B.data_ptr(), r, float(alpha),
                               out.data_ptr(), _stream(stream)))
    return out


def qlora_fwd_workspace_bytes(M: int, N: int, K: int, r: int) -> int:
    return lib().qlora_fwd_workspace_bytes(M, N, K, r)


def qlora_bwd_workspace_bytes(M: int, N: int, K: int, r: int) -> int:
    return lib().qlora_bwd_workspace_bytes(M, N, K, r)


def _workspace(nbytes: int, device, given):
    import torch
    if given is not None:
        return given
    if nbytes == 0:
        return None
    return torch.empty(nbytes, dtype=torch.uint8, device=device)


def qlora_linear_fwd(w: NF4Weight, X, A, B, alpha: float, Y=None, T=None, workspace=None,
                     stream=None) -> Tuple["torch.Tensor", "torch.Tensor"]:
    """Y = X W'^T + (alpha/r) (X A^T) B^T ; returns (Y [M, N] bf16, T [M, r] fp32)."""
    import torch
    M, K = X.shape
    r = A.shape[0]
    N = w.rows
    _need(X, torch.bfloat16, (M, w.cols), "X")
    _need(A, torch.bfloat16, (r, K), "A")
    _need(B, torch.bfloat16, (N, r), "B")
    Y = Y if Y is not None else torch.empty(M, N, dtype=torch.bfloat16, device=X.device)
    T = T if T is not None else torch.empty(M, r, dtype=torch.float32, device=X.device)
    _need(Y, torch.bfloat16, (M, N), "Y")
    _need(T, torch.float32, (M, r), "T")
    nbytes = qlora_fwd_workspace_bytes(M, N, K, r)
    ws = _workspace(nbytes, X.device, workspace)
    d = w.descriptor()
    _check(lib().qlora_linear_fwd(ctypes.byref(d), X.data_ptr(), M, A.data_ptr(), B.data_ptr(), r,
                                  float(alpha), QL_DTYPE_BF16, Y.data_ptr(), T.data_ptr(), _ptr(ws),
                                  0 if ws is None else ws.numel(), _stream(stream)))
    return Y, T


def qlora_dual_fwd(w_gate: NF4Weight, w_up: NF4Weight, X, A_gate, B_gate, A_up, B_up,
                   alpha: float, swiglu: bool = False, workspace=None, stream=None):
    """Gate and up projections of one X in one kernel.  Returns
    (Y_gate, Y_up, T_gate, T_up), or with swiglu=True (H, T_gate, T_up) where
    H = bf16(silu(G) * U) from the fp32 sums."""
    import torch
    M, K = X.shape
    r = A_gate.shape[0]
    N = w_gate.rows
    _need(X, torch.bfloat16, (M, w_gate.cols), "X")
    for t, nm in ((A_gate, "A_gate"), (A_up, "A_up")):
        _need(t, torch.bfloat16, (r, K), nm)
    for t, nm in ((B_gate, "B_gate"), (B_up, "B_up")):
        _need(t, torch.bfloat16, (N, r), nm)
    dev = X.device
    Tg = torch.empty(M, r, dtype=torch.float32, device=dev)
    Tu = torch.empty(M, r, dtype=torch.float32, device=dev)
    if swiglu:
        H = torch.empty(M, N, dtype=torch.bfloat16, device=dev)
        Yg = Yu = None
    else:
        Yg = torch.empty(M, N, dtype=torch.bfloat16, device=dev)
        Yu = torch.empty(M, N, dtype=torch.bfloat16, device=dev)
        H = None
    ws = _workspace(qlora_fwd_workspace_bytes(M, N, K, r), dev, workspace)
    dg, du = w_gate.descriptor(), w_up.descriptor()
    _check(lib().qlora_dual_fwd(ctypes.byref(dg), ctypes.byref(du), X.data_ptr(), M,
                                A_gate.data_ptr(), B_gate.data_ptr(), A_up.data_ptr(), B_up.data_ptr(),
                                r, float(alpha), QL_DTYPE_BF16,
                                QL_DUAL_SWIGLU if swiglu else QL_DUAL_SEPARATE,
                                _ptr(Yg), _ptr(Yu), _ptr(H), Tg.data_ptr(), Tu.data_ptr(), _ptr(ws),
                                0 if ws is None else ws.numel(), _stream(stream)))
    return (H, Tg, Tu) if swiglu else (Yg, Yu, Tg, Tu)


def qlora_adamw_step(params, grads, exp_avgs, exp_avg_sqs, lr: float, betas=(0.9, 0.999),
                     eps: float = 1e-8, weight_decay: float = 0.0, step: int = 1, masters=None,
                     stream=None) -> None:
    """One AdamW step over lists of tensors, in place: bf16 params (cuda),
    bf16 grads, fp32 moments, optional fp32 master copies (a list with None
    entries allowed)."""
    import torch
    n = len(params)
    masters = masters if masters is not None else [None] * n
    if not (len(grads) == len(exp_avgs) == len(exp_avg_sqs) == len(masters) == n):
        raise ValueError("tensor lists differ in length")
    arr = (_AdamwTensor * max(1, n))()
    for i, (p, g, m, v, w) in enumerate(zip(params, grads, exp_avgs, exp_avg_sqs, masters)):
        shape = tuple(p.shape)
        _need(p, torch.bfloat16, shape, f"params[{i}]")
        _need(g, torch.bfloat16, shape, f"grads[{i}]")
        _need(m, torch.float32, shape, f"exp_avgs[{i}]")
        _need(v, torch.float32, shape, f"exp_avg_sqs[{i}]")
        if w is not None:
            _need(w, torch.float32, shape, f"masters[{i}]")
        arr[i] = _AdamwTensor(p.data_ptr(), g.data_ptr(), m.data_ptr(), v.data_ptr(), _ptr(w), p.numel())
    _check(lib().qlora_adamw_step(ctypes.cast(arr, ctypes.c_void_p), n, float(lr), float(betas[0]),
                                  float(betas[1]), float(eps), float(weight_decay), int(step),
                                  _stream(stream)))


def qlora_linear_bwd(w: NF4Weight, X, dY, A, B, alpha: float, T=None, want_dX: bool = True,
                     dX=None, dA=None, dB=None, workspace=None, stream=None):
    """Returns (dX [M, K] or None, dA [r, K], dB [N, r]) in bf16."""
    import torch
    M, K = X.shape
    r = A.shape[0]
    N = w.rows
    _need(X, torch.bfloat16, (M, w.cols), "X")
    _need(dY, torch.bfloat16, (M, N), "dY")
    _need(A, torch.bfloat16, (r, K), "A")
    _need(B, torch.bfloat16, (N, r), "B")
    if T is not None:
        _need(T, torch.float32, (M, r), "T")
    if want_dX and dX is None:
        dX = torch.empty(M, K, dtype=torch.bfloat16, device=X.device)
    if dX is not None:
        _need(dX, torch.bfloat16, (M, K), "dX")
    dA = dA if dA is not None else torch.empty(r, K, dtype=torch.bfloat16, device=X.device)
    dB = dB if dB is not None else torch.empty(N, r, dtype=torch.bfloat16, device=X.device)
    _need(dA, torch.bfloat16, (r, K), "dA")
    _need(dB, torch.bfloat16, (N, r), "dB")
    ws = _workspace(qlora_bwd_workspace_bytes(M, N, K, r), X.device, workspace)
    d = w.descriptor()
    _check(lib().qlora_linear_bwd(ctypes.byref(d), X.data_ptr(), dY.data_ptr(), M, A.data_ptr(),
                                  B.data_ptr(), r, float(alpha), QL_DTYPE_BF16, _ptr(T), _ptr(dX),
                                  dA.data_ptr(), dB.data_ptr(), _ptr(ws),
                                  0 if ws is None else ws.numel(), _stream(stream)))
    return dX, dA, dB


def qlora_linear_bwd_noalloc(w: NF4Weight, X, dY, A, B, alpha: float, dX, dA, dB, T=None,
                             stream=None):
    """The backward over the library's fixed per-GPU scratch (no workspace,
    nothing allocated here either: dX (or None), dA [r, K] and dB [N, r] are
    the caller's bf16 outputs).  Calls that can overlap on one GPU race."""
    import torch
    M, K = X.shape
    r = A.shape[0]
    N = w.rows
    _need(X, torch.bfloat16, (M, w.cols), "X")
    _need(dY, torch.bfloat16, (M, N), "dY")
    _need(A, torch.bfloat16, (r, K), "A")
    _need(B, torch.bfloat16, (N, r), "B")
    if T is not None:
        _need(T, torch.float32, (M, r), "T")
    if dX is not None:
        _need(dX, torch.bfloat16, (M, K), "dX")
    _need(dA, torch.bfloat16, (r, K), "dA")
    _need(dB, torch.bfloat16, (N, r), "dB")
    d = w.descriptor()
    _check(lib().qlora_linear_bwd_noalloc(ctypes.byref(d), X.data_ptr(), dY.data_ptr(), M,
                                          A.data_ptr(), B.data_ptr(), r, float(alpha),
                                          QL_DTYPE_BF16, _ptr(T), _ptr(dX), dA.data_ptr(),
                                          dB.data_ptr(), _stream(stream)))
    return dX, dA, dB
