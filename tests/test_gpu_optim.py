"""GPU parity of the adapters' AdamW step (qlora_adamw_step) through the C
ABI, against the oracle's double-precision step on the same inputs.

The kernel computes each element's update in fp32 (a handful of roundings),
so the bar is: moments within 2^-20 relative; the fp32 master within 2^-21 of
|theta| plus 2^-18 of the update; the bf16 parameter is the bf16 rounding of a
value within that bound of the exact result."""
import numpy as np
import pytest

from helpers import log, tensor_bits

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
if not torch.cuda.is_available():  # pragma: no cover
    pytest.skip("needs a GPU", allow_module_level=True)

import bit_nf4_quantized_17_amd as q  # noqa: E402
import synthetic_inputs as si  # noqa: E402


def _ulp_bf16(x):
    e = np.floor(np.log2(np.maximum(np.abs(x), 2.0**-126)))
    return 2.0 ** (e - 7)


def _bf16(x):
    return torch.from_numpy(np.ascontiguousarray(si.to_bf16_bits(x.astype(np.float32))).view(np.int16)) \
        .view(torch.bfloat16).cuda()


def _f64_bits(bits):
    return si.bf16_bits_to_f32(bits).astype(np.float64)


class Case:
    def __init__(self, n, master, rng):
        self.n = n
        self.theta = rng.normal(0.0, 0.05, n).astype(np.float32)
        self.g = rng.normal(0.0, 1e-3, n) * 10.0 ** rng.integers(-2, 2, n)
        self.m = (rng.normal(0.0, 1e-3, n)).astype(np.float32)
        self.v = (rng.normal(0.0, 1e-3, n) ** 2).astype(np.float32)
        self.p = _bf16(self.theta)
        self.gd = _bf16(self.g)
        self.g = _f64_bits(tensor_bits(self.gd))                 # the bf16 gradient the kernel sees
        self.md = torch.from_numpy(self.m.copy()).cuda()
        self.vd = torch.from_numpy(self.v.copy()).cuda()
        self.w = torch.from_numpy(self.theta.copy()).cuda() if master else None
        self.theta0 = self.theta.astype(np.float64) if master else _f64_bits(tensor_bits(self.p))


def _check(orc, cases, lr, b1, b2, eps, wd, step):
    """fp32 error bounds from the magnitudes of the terms each result sums (the
    first moment can cancel, so its bound is relative to |b1 m| + |(1-b1) g|,
    and the update inherits that through m / denom)."""
    # the hyperparameters cross the C ABI as fp32: the oracle takes those values
    lr, b1, b2, eps, wd = (float(np.float32(x)) for x in (lr, b1, b2, eps, wd))
    for c in cases:
        th, m, v = orc.adamw_step(c.theta0, c.m, c.v, c.g, lr, beta1=b1, beta2=b2, eps=eps,
                                  weight_decay=wd, step=step)
        m_mag = b1 * np.abs(c.m.astype(np.float64)) + (1 - b1) * np.abs(c.g)
        bc1, bc2 = 1 - b1 ** step, 1 - b2 ** step
        upd_mag = lr / bc1 * m_mag / (np.sqrt(v) / np.sqrt(bc2) + eps)
        gm = c.md.cpu().numpy().astype(np.float64)
        gv = c.vd.cpu().numpy().astype(np.float64)
        assert np.all(np.abs(gm - m) <= 2.0**-21 * m_mag + 1e-30), f"n={c.n}: exp_avg"
        assert np.all(np.abs(gv - v) <= 2.0**-20 * np.abs(v) + 1e-30), f"n={c.n}: exp_avg_sq"
        tol = 2.0**-21 * np.abs(c.theta0) + 2.0**-18 * upd_mag + 1e-30
        if c.w is not None:
            gw = c.w.cpu().numpy().astype(np.float64)
            assert np.all(np.abs(gw - th) <= tol), f"n={c.n}: master"
        gp = _f64_bits(tensor_bits(c.p))
        assert np.all(np.abs(gp - th) <= 0.5 * _ulp_bf16(gp) + tol), f"n={c.n}: param"


SIZES = [1, 7, 8, 9, 2047, 2048, 2049, 4095, 4096, 4097, 6151, 64 * 8192, 1000 * 64 + 3]


@pytest.mark.parametrize("step", [1, 3, 1000])
def test_adamw_step_mixed_tensor_list(orc, step):
    """One call over ragged tensors, half with a master copy (two launches)."""
    rng = np.random.default_rng(step)
    cases = [Case(n, i % 2 == 1, rng) for i, n in enumerate(SIZES)]
    lr, b1, b2, eps, wd = 1e-3, 0.9, 0.999, 1e-8, 0.01
    log(f"[adamw] {len(cases)} tensors, step {step}")
    q.qlora_adamw_step([c.p for c in cases], [c.gd for c in cases], [c.md for c in cases],
                       [c.vd for c in cases], lr, betas=(b1, b2), eps=eps, weight_decay=wd, step=step,
                       masters=[c.w for c in cases])
    torch.cuda.synchronize()
    _check(orc, cases, lr, b1, b2, eps, wd, step)


def test_adamw_many_tensors_split_launches(orc):
    """More tensors than one launch holds, with empty ones in between."""
    rng = np.random.default_rng(9)
    cases = [Case(int(n), False, rng) for n in rng.integers(0, 5000, 60)]
    q.qlora_adamw_step([c.p for c in cases], [c.gd for c in cases], [c.md for c in cases],
                       [c.vd for c in cases], 3e-4, betas=(0.8, 0.95), eps=1e-6, weight_decay=0.1, step=2)
    torch.cuda.synchronize()
    _check(orc, cases, 3e-4, 0.8, 0.95, 1e-6, 0.1, 2)


def test_adamw_five_steps_with_master(orc):
    """Five steps on the GPU against five in double: the fp32 state drifts from
    the double one by a few roundings per step."""
    rng = np.random.default_rng(4)
    c = Case(50000, True, rng)
    th, m, v = c.theta0, c.m.astype(np.float64), c.v.astype(np.float64)
    grads = [rng.normal(0.0, 1e-3, c.n) for _ in range(5)]
    for t, g in enumerate(grads, start=1):
        gd = _bf16(g)
        gb = _f64_bits(tensor_bits(gd))
        q.qlora_adamw_step([c.p], [gd], [c.md], [c.vd], 1e-3, weight_decay=0.01, step=t, masters=[c.w])
        th, m, v = orc.adamw_step(th, m, v, gb, *(float(np.float32(x)) for x in (1e-3, 0.9, 0.999, 1e-8)),
                                  weight_decay=float(np.float32(0.01)), step=t)
    torch.cuda.synchronize()
    # absolute floors: five steps of fp32 roundings on terms of size (1 - b1) |g| ~ 1e-4
    # (the first moment can cancel to far below that) and (1 - b2) g^2 ~ 1e-9
    assert np.allclose(c.w.cpu().numpy(), th, rtol=1e-5, atol=1e-9)
    assert np.allclose(c.md.cpu().numpy(), m, rtol=1e-5, atol=1e-10)
    assert np.allclose(c.vd.cpu().numpy(), v, rtol=1e-5, atol=1e-15)


# ---------------------------------------------------------------------------
# optimizer state in managed (unified) memory
# ---------------------------------------------------------------------------
HIP_ATTR_MANAGED_MEMORY = 24      # hipDeviceAttributeManagedMemory
HIP_MEM_ATTACH_GLOBAL = 1         # hipMemAttachGlobal
HIP_MEMCPY_DEFAULT = 4          # hipMemcpyDefault: the runtime tells the directions apart


class _Managed:
    """fp32 arrays in hipMallocManaged memory (attached globally, no prefetch
    or advice), filled and read back with hipMemcpy.  The HIP runtime's
    symbols resolve through the library's handle: the runtime torch and the
    library already share."""

    def __init__(self):
        import ctypes
        self.ct = ctypes
        L = q.lib()
        vp, sz = ctypes.c_void_p, ctypes.c_size_t
        L.hipMallocManaged.argtypes = [ctypes.POINTER(vp), sz, ctypes.c_uint]
        L.hipFree.argtypes = [vp]
        L.hipMemcpy.argtypes = [vp, vp, sz, ctypes.c_int]
        L.hipDeviceGetAttribute.argtypes = [ctypes.POINTER(ctypes.c_int), ctypes.c_int, ctypes.c_int]
        L.hipDeviceSynchronize.argtypes = []
        self.L = L
        self.ptrs = []

    def attribute(self) -> int:
        v = self.ct.c_int(-1)
        self.L.hipDeviceGetAttribute(self.ct.byref(v), HIP_ATTR_MANAGED_MEMORY, torch.cuda.current_device())
        return v.value

    def array(self, host: np.ndarray) -> int:
        host = np.ascontiguousarray(host, np.float32)
        p = self.ct.c_void_p()
        rc = self.L.hipMallocManaged(self.ct.byref(p), max(16, host.nbytes), HIP_MEM_ATTACH_GLOBAL)
        if rc != 0:
            pytest.skip(f"hipMallocManaged refused the allocation (status {rc})")
        self.ptrs.append(p.value)
        assert self.L.hipMemcpy(p.value, host.ctypes.data, host.nbytes, HIP_MEMCPY_DEFAULT) == 0
        return p.value

    def read(self, ptr: int, n: int) -> np.ndarray:
        out = np.empty(n, np.float32)
        assert self.L.hipMemcpy(out.ctypes.data, ptr, out.nbytes, HIP_MEMCPY_DEFAULT) == 0
        return out

    def free(self):
        assert self.L.hipDeviceSynchronize() == 0
        for p in self.ptrs:
            self.L.hipFree(p)
        self.ptrs = []


def test_adamw_state_in_managed_memory(orc):
    """Ultralytics "QLoRA" (paged-optimizer bullet) and vnread "Grokking QLoRA"
    ("Paged Optimizers"): the optimizer state lives in unified memory that the
    runtime may page.  The moments and fp32 masters here are hipMallocManaged
    allocations handed to the C ABI as raw pointers; three steps must match the
    oracle to the same bar as device memory."""
    mm = _Managed()
    log(f"[adamw managed] hipDeviceAttributeManagedMemory = {mm.attribute()}")
    import ctypes
    rng = np.random.default_rng(21)
    sizes = [9, 2049, 64 * 1000 + 5]
    lr, b1, b2, eps, wd = 1e-3, 0.9, 0.999, 1e-8, 0.01
    try:
        cases = []
        for n in sizes:
            c = Case(n, True, rng)
            c.mp = mm.array(c.m)
            c.vp = mm.array(c.v)
            c.wp = mm.array(c.theta)
            cases.append(c)
        T = q._AdamwTensor
        for step in (1, 2, 3):
            arr = (T * len(cases))(*[T(c.p.data_ptr(), c.gd.data_ptr(), c.mp, c.vp, c.wp, c.n) for c in cases])
            log(f"[adamw managed] step {step}")
            q._check(q.lib().qlora_adamw_step(ctypes.cast(arr, ctypes.c_void_p), len(cases), lr, b1, b2, eps,
                                             wd, step, ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)))
            torch.cuda.synchronize()
            for c in cases:
                # the device-memory checker reads c.md, c.vd, c.w: point them at the managed state
                c.md = torch.from_numpy(mm.read(c.mp, c.n))
                c.vd = torch.from_numpy(mm.read(c.vp, c.n))
                c.w = torch.from_numpy(mm.read(c.wp, c.n))
            _check(orc, cases, lr, b1, b2, eps, wd, step)
            for c in cases:   # the next step starts from the state the GPU wrote
                c.m, c.v = c.md.numpy().copy(), c.vd.numpy().copy()
                c.theta0 = c.w.numpy().astype(np.float64)
    finally:
        mm.free()
