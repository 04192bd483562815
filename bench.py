"""Benchmark of the QLoRA NF4 linear layer on one MI355X.

A step is one pass of the whole hot path over one batch of synthetic input,
on the 70B-class MLP slice (W 28672x8192 "up" and 8192x28672 "down", 4096
tokens, LoRA rank 64, alpha 16; weights N(0, 0.02) with 1% x20 outliers):
    nf4_quantize(up), nf4_quantize(down)          absmax, encode, pack, double quant
    qlora_linear_fwd(up), qlora_linear_fwd(down)  T = X A^T, fused dequant GEMM + LoRA
    qlora_linear_bwd(down), qlora_linear_bwd(up)  U, dB, fused dequant dX GEMM, dA
    qlora_linear_fwd(up|down) at M = 16           the decode-sized forward
Inputs are resident in HBM before timing starts.  value = algorithmic flops
of the step (4MNK + 6Mr(N+K) per trained linear, plus the decode forwards;
dequantization and quantization count no flops) / wall time of the step.

Also reported: the roofline of the dominant kernel (HIP events recorded by
the library's timing hook around that kernel's launches); the decode-shape
and quantize bandwidths against HBM; the smaller training shapes C1-C3
(tiny-layer latency, TFLOP/s of the 7B attention projection and of the 7B
MLP); the dequantize, merge, dual-projection, format-variant and AdamW
figures; context from the chip itself (a pure MFMA loop with zero and random
operands, a streaming HBM read, a device copy, the empty-kernel launch
floor, and the vendor's dense bf16 GEMM on the fused GEMMs' shapes); and the
CPU oracle timed on a bounded sample of the same workload.

    python bench.py [--steps K] [--warmup W] [--gpus 1] [--no-cpu-baseline]
"""
from __future__ import annotations

import argparse
import ctypes
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "QLoRA linear fwd+bwd TFLOP/s (bf16 MFMA) and NF4 decode GB/s vs roofline"
PEAK_BF16_TFLOPS = 2516.6      # MI355X dense bf16 MFMA: 256 CU x 4096 flop/clk x 2.4 GHz
PEAK_HBM_GBS = 8000.0          # MI355X HBM3E


def log(msg):
    print(msg, file=sys.stderr, flush=True)


# ---------------------------------------------------------------------------
# HIP events straight from the runtime (the library records them on the
# stream its kernels are launched on)
# ---------------------------------------------------------------------------
class Hip:
    def __init__(self):
        # resolve through libqlora_nf4's handle: the HIP runtime already loaded
        # in this process (the one torch and the library use), never a second copy
        import bit_nf4_quantized_17_amd as q
        self.L = q.lib()
        self.L.hipEventCreate.argtypes = [ctypes.POINTER(ctypes.c_void_p)]
        self.L.hipEventRecord.argtypes = [ctypes.c_void_p, ctypes.c_void_p]
        self.L.hipEventSynchronize.argtypes = [ctypes.c_void_p]
        self.L.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.c_void_p,
                                               ctypes.c_void_p]
        self.L.hipEventDestroy.argtypes = [ctypes.c_void_p]

    def event(self) -> int:
        e = ctypes.c_void_p()
        assert self.L.hipEventCreate(ctypes.byref(e)) == 0
        return e.value

    def record(self, ev, stream):
        assert self.L.hipEventRecord(ev, stream) == 0

    def elapsed_ms(self, a, b) -> float:
        assert self.L.hipEventSynchronize(b) == 0
        ms = ctypes.c_float()
        assert self.L.hipEventElapsedTime(ctypes.byref(ms), a, b) == 0
        return ms.value


# ---------------------------------------------------------------------------
# workload
# ---------------------------------------------------------------------------
def linear_flops(M, N, K, r):
    """fwd 2MNK + 2Mr(K+N); bwd 2MNK + 4Mr(K+N) (dX base, U, U A, dA, dB)."""
    fwd = 2 * M * N * K + 2 * M * r * (K + N)
    bwd = 2 * M * N * K + 4 * M * r * (K + N)
    return fwd, bwd


def decode_bytes(M, N, K, r):
    """Algorithmic bytes of one decode-sized forward: the NF4 weight (codes,
    E4M3 scales, group constants), X, Y, A, B and the fp32 T."""
    nb = N * K // 64
    w = N * K // 2 + nb + 4 * ((nb + 255) // 256)
    return w + 2 * M * K + 2 * M * N + 2 * r * K + 2 * N * r + 4 * M * r


def quantize_bytes(N, K):
    """fp32 read + packed codes + E4M3 scales + group constants written."""
    nb = N * K // 64
    return 4 * N * K + N * K // 2 + nb + 4 * ((nb + 255) // 256)


class Layer:
    def __init__(self, cfg, li, M_decode=16):
        import torch
        import bit_nf4_quantized_17_amd as q
        import synthetic_inputs as si
        from synthetic_inputs import bf16_tensor
        L = cfg.layers[li]
        self.name, self.N, self.K, self.M, self.r, self.alpha = L.name, L.N, L.K, cfg.M, cfg.r, cfg.alpha
        self.W = torch.from_numpy(si.weight(cfg, li)).cuda()
        self.X = bf16_tensor(si.activations(cfg, li))
        A, B = si.adapters(cfg, li)
        self.A, self.B = bf16_tensor(A), bf16_tensor(B)
        self.dY = bf16_tensor(si.upstream(cfg, li))
        self.w = q.NF4Weight.empty(self.N, self.K)
        dev = "cuda"
        self.Y = torch.empty(self.M, self.N, dtype=torch.bfloat16, device=dev)
        self.T = torch.empty(self.M, self.r, dtype=torch.float32, device=dev)
        self.dXo = torch.empty(self.M, self.K, dtype=torch.bfloat16, device=dev)
        self.dA = torch.empty(self.r, self.K, dtype=torch.bfloat16, device=dev)
        self.dB = torch.empty(self.N, self.r, dtype=torch.bfloat16, device=dev)
        self.wsf = torch.empty(max(256, q.qlora_fwd_workspace_bytes(self.M, self.N, self.K, self.r)),
                               dtype=torch.uint8, device=dev)
        self.wsb = torch.empty(q.qlora_bwd_workspace_bytes(self.M, self.N, self.K, self.r),
                               dtype=torch.uint8, device=dev)
        self.Md = M_decode
        self.Xd = self.X[:M_decode].contiguous()
        self.Yd = torch.empty(M_decode, self.N, dtype=torch.bfloat16, device=dev)
        self.Td = torch.empty(M_decode, self.r, dtype=torch.float32, device=dev)
        self.wsd = torch.empty(max(256, q.qlora_fwd_workspace_bytes(M_decode, self.N, self.K, self.r)),
                               dtype=torch.uint8, device=dev)

    def quantize(self):
        import bit_nf4_quantized_17_amd as q
        q.nf4_quantize(self.W, out=self.w)

    def fwd(self):
        import bit_nf4_quantized_17_amd as q
        q.qlora_linear_fwd(self.w, self.X, self.A, self.B, self.alpha, Y=self.Y, T=self.T,
                           workspace=self.wsf)

    def bwd(self):
        import bit_nf4_quantized_17_amd as q
        q.qlora_linear_bwd(self.w, self.X, self.dY, self.A, self.B, self.alpha, T=self.T,
                           dX=self.dXo, dA=self.dA, dB=self.dB, workspace=self.wsb)

    def decode(self):
        import bit_nf4_quantized_17_amd as q
        q.qlora_linear_fwd(self.w, self.Xd, self.A, self.B, self.alpha, Y=self.Yd, T=self.Td,
                           workspace=self.wsd)

    def flops(self):
        f, b = linear_flops(self.M, self.N, self.K, self.r)
        d, _ = linear_flops(self.Md, self.N, self.K, self.r)
        return f, b, d


def source_hash(*names):
    h = hashlib.sha256()
    for n in names:
        with open(os.path.join(ROOT, "bit_nf4_quantized_17_amd", "csrc", n), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def load_traffic(kernel_key: str, src_hash: str):
    """Per-launch HBM bytes measured with rocprofv3 counters (profiles/), or
    None when absent or taken on a different kernel source."""
    path = os.path.join(ROOT, "profiles", "traffic.json")
    if not os.path.exists(path):
        return None
    try:
        d = json.load(open(path)).get(kernel_key)
    except (ValueError, OSError):
        return None
    if not d or d.get("source_hash") != src_hash:
        return None
    return d.get("bytes_per_launch")


# ---------------------------------------------------------------------------
# decode and quantize bandwidth (cache-defeating rotation over >= 512 MB)
# ---------------------------------------------------------------------------
def bench_decode(hip, reps=200):
    """The decode shapes (W 8192x8192 and 28672x8192, M = 1, 4, 16, r = 16), each
    forward's weight taken in turn from copies that together exceed 512 MB, so
    the 256 MB Infinity Cache cannot serve it.  kernel_us: HIP events recorded
    by the library around the forward's launches (the T-partials launch and
    the weight stream), averaged over `reps` eager calls; graph_us: the same
    calls captured in one HIP graph and replayed back to back (GPU time per
    call with no host gaps).  GB/s counts the algorithmic bytes of one call
    against graph_us."""
    import torch
    import bit_nf4_quantized_17_amd as q
    import synthetic_inputs as si
    from synthetic_inputs import bf16_tensor
    cfg = si.CONFIGS["decode_8192_28672"]
    out = []
    st = torch.cuda.current_stream().cuda_stream
    for li, L in enumerate(cfg.layers):
        w0 = q.nf4_quantize(torch.from_numpy(si.weight(cfg, li)).cuda())
        wbytes = sum(t.numel() * t.element_size() for t in (w0.codes, w0.qscale, w0.dscale))
        ncopy = max(2, -(-512 * 2**20 // wbytes))
        copies = [w0] + [q.NF4Weight(w0.codes.clone(), w0.qscale.clone(), w0.dscale.clone(),
                                     w0.rows, w0.cols) for _ in range(ncopy - 1)]
        A, B = si.adapters(cfg, li)
        A, B = bf16_tensor(A), bf16_tensor(B)
        for M in cfg.decode_M:
            X = bf16_tensor(si.activations(cfg, li, M))
            Y = torch.empty(M, L.N, dtype=torch.bfloat16, device="cuda")
            T = torch.empty(M, cfg.r, dtype=torch.float32, device="cuda")
            ws = torch.empty(max(256, q.qlora_fwd_workspace_bytes(M, L.N, L.K, cfg.r)),
                             dtype=torch.uint8, device="cuda")

            def call(i):
                q.qlora_linear_fwd(copies[i % ncopy], X, A, B, cfg.alpha, Y=Y, T=T, workspace=ws)
            for i in range(5):
                call(i)
            kev = [(hip.event(), hip.event()) for _ in range(reps)]
            torch.cuda.synchronize()
            for i in range(reps):
                q.qlora_set_timing_events(kev[i][0], kev[i][1])
                call(i)
            q.qlora_set_timing_events()
            kms = sum(hip.elapsed_ms(a, b) for a, b in kev) / reps
            # back to back: the same calls in one graph (side stream for capture)
            side = torch.cuda.Stream()
            side.wait_stream(torch.cuda.current_stream())
            with torch.cuda.stream(side):
                call(0)
            torch.cuda.current_stream().wait_stream(side)
            torch.cuda.synchronize()
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g):
                for i in range(reps):
                    call(i)
            g.replay()
            torch.cuda.synchronize()
            best = None
            for _ in range(3):
                e0, e1 = hip.event(), hip.event()
                hip.record(e0, st)
                g.replay()
                hip.record(e1, st)
                ms = hip.elapsed_ms(e0, e1) / reps
                best = ms if best is None else min(best, ms)
            del g
            nbytes = decode_bytes(M, L.N, L.K, cfg.r)
            gbs = nbytes / (best * 1e-3) / 1e9
            out.append({"W": f"{L.N}x{L.K}", "M": M, "reps": reps, "graph_us": round(best * 1e3, 2),
                        "GB/s": round(gbs, 1), "frac_hbm": round(gbs / PEAK_HBM_GBS, 4),
                        "kernel_us": round(kms * 1e3, 2), "bytes": nbytes})
        del copies, w0
        torch.cuda.empty_cache()
    return out


def bench_bf16_weight(hip, lay, reps=10):
    """The calls that write a bf16 weight, on the up projection (28672x8192,
    r=64): nf4_dequantize, the adapter merge and its inverse.  Algorithmic
    bytes: dequantize reads the NF4 weight (0.516 B/weight) and writes bf16
    (2 B/weight); merge also reads the adapters; unmerge reads and writes
    bf16.  The NF4 input rotates over copies of >= 512 MB in total and the
    two 470 MB bf16 buffers alternate, so the 256 MB Infinity Cache serves
    neither side."""
    import torch
    import bit_nf4_quantized_17_amd as q
    st = torch.cuda.current_stream().cuda_stream
    out = torch.empty(lay.N, lay.K, dtype=torch.bfloat16, device="cuda")
    out2 = torch.empty_like(out)
    nk = lay.N * lay.K
    adapters = 2 * lay.r * (lay.N + lay.K)
    # the NF4 input is taken in turn from copies that together exceed 512 MB
    w0 = lay.w
    wbytes = sum(t.numel() * t.element_size() for t in (w0.codes, w0.qscale, w0.dscale))
    ncopy = max(2, -(-512 * 2**20 // wbytes))
    ws = [w0] + [q.NF4Weight(w0.codes.clone(), w0.qscale.clone(), w0.dscale.clone(), w0.rows, w0.cols)
                 for _ in range(ncopy - 1)]
    outs = (out, out2)
    res = {}
    for name, fn, nbytes in (
            ("dequantize", lambda i: q.nf4_dequantize(ws[i % ncopy], out=outs[i % 2]),
             nk * (0.5 + 1 / 64 + 4 / 16384 + 2)),
            ("merge", lambda i: q.qlora_merge(ws[i % ncopy], lay.A, lay.B, lay.alpha, out=outs[i % 2]),
             nk * (0.5 + 1 / 64 + 4 / 16384 + 2) + adapters),
            ("unmerge", lambda i: q.qlora_unmerge(outs[i % 2], lay.A, lay.B, lay.alpha, out=outs[(i + 1) % 2]),
             nk * 4 + adapters)):
        for i in range(3):
            fn(i)
        e0, e1 = hip.event(), hip.event()
        torch.cuda.synchronize()
        hip.record(e0, st)
        for i in range(reps):
            fn(i)
        hip.record(e1, st)
        ms = hip.elapsed_ms(e0, e1) / reps
        gbs = nbytes / (ms * 1e-3) / 1e9
        res[name] = {"W": f"{lay.N}x{lay.K}", "us_per_call": round(ms * 1e3, 1),
                     "GB/s": round(gbs, 1), "frac_hbm": round(gbs / PEAK_HBM_GBS, 4)}
        if name != "dequantize":
            res[name]["r"] = lay.r
        res[name]["input_copies"] = ncopy if name != "unmerge" else 2
    del out, out2, ws
    torch.cuda.empty_cache()
    return res


def bench_dual(hip, lay, reps=10):
    """Gate and up projections of one X (qlora_dual_fwd, both epilogues)
    against two qlora_linear_fwd calls: two 28672x8192 NF4 weights, 4096
    tokens, r=64.  The up layer is the step's up projection; the gate weight
    and adapters are seeded synthetic tensors of the same shapes."""
    import math
    import torch
    import bit_nf4_quantized_17_amd as q
    st = torch.cuda.current_stream().cuda_stream
    gen = torch.Generator(device="cuda")
    gen.manual_seed(20240)
    Wg = torch.randn(lay.N, lay.K, generator=gen, device="cuda") * 0.02
    wg = q.nf4_quantize(Wg)
    del Wg
    Ag = (torch.randn(lay.r, lay.K, generator=gen, device="cuda") / math.sqrt(lay.r)).to(torch.bfloat16)
    Bg = (torch.randn(lay.N, lay.r, generator=gen, device="cuda") * 0.01).to(torch.bfloat16)
    Yg = torch.empty_like(lay.Y)
    Tg = torch.empty_like(lay.T)
    fwd, _ = linear_flops(lay.M, lay.N, lay.K, lay.r)
    res = {"W": f"2x {lay.N}x{lay.K}", "M": lay.M, "r": lay.r}
    for name, fn in (
            ("two_single_fwd", lambda: (q.qlora_linear_fwd(wg, lay.X, Ag, Bg, lay.alpha, Y=Yg, T=Tg,
                                                           workspace=lay.wsf), lay.fwd())),
            ("dual_separate", lambda: q.qlora_dual_fwd(wg, lay.w, lay.X, Ag, Bg, lay.A, lay.B, lay.alpha,
                                                       workspace=lay.wsf)),
            ("dual_swiglu", lambda: q.qlora_dual_fwd(wg, lay.w, lay.X, Ag, Bg, lay.A, lay.B, lay.alpha,
                                                     swiglu=True, workspace=lay.wsf))):
        for _ in range(2):
            fn()
        e0, e1 = hip.event(), hip.event()
        torch.cuda.synchronize()
        hip.record(e0, st)
        for _ in range(reps):
            fn()
        hip.record(e1, st)
        ms = hip.elapsed_ms(e0, e1) / reps
        res[name] = {"ms": round(ms, 4), "TFLOP/s": round(2 * fwd / (ms * 1e-3) / 1e12, 1)}
    del wg, Ag, Bg, Yg, Tg
    torch.cuda.empty_cache()
    return res


def bench_formats(hip, lay, reps=10):
    """Codebook and scale-format variants on the up projection (28672x8192,
    4096 tokens, r=64): quantize and dequantize bandwidth and the fused
    forward, for INT4 with E4M3 scales, NF4 with fp32 block scales and NF4
    with uint8-linear double-quantized scales.
    Algorithmic bytes per weight: quantize 4 read + 0.5 + scale bytes written
    (1/64 + 4/16384 with double quantization, 4/64 without); dequantize the
    reverse plus 2 written."""
    import torch
    import bit_nf4_quantized_17_amd as q
    st = torch.cuda.current_stream().cuda_stream
    nk = lay.N * lay.K
    fwd, _ = linear_flops(lay.M, lay.N, lay.K, lay.r)
    out = torch.empty(lay.N, lay.K, dtype=torch.bfloat16, device="cuda")

    def timed(fn):
        for _ in range(2):
            fn()
        e0, e1 = hip.event(), hip.event()
        torch.cuda.synchronize()
        hip.record(e0, st)
        for _ in range(reps):
            fn()
        hip.record(e1, st)
        return hip.elapsed_ms(e0, e1) / reps

    res = []
    for codebook, dq, fmt in (("int4", True, "e4m3"), ("nf4", False, "e4m3"), ("nf4", True, "uint8")):
        w = q.NF4Weight.empty(lay.N, lay.K, codebook=codebook, double_quant=dq, dq_format=fmt)
        scale_b = (1 / 64 + 4 / 16384) if dq else 4 / 64
        qms = timed(lambda: q.nf4_quantize(lay.W, out=w, codebook=codebook, double_quant=dq, dq_format=fmt))
        dms = timed(lambda: q.nf4_dequantize(w, out=out))
        fms = timed(lambda: q.qlora_linear_fwd(w, lay.X, lay.A, lay.B, lay.alpha, Y=lay.Y, T=lay.T,
                                               workspace=lay.wsf))
        qb, db = nk * (4 + 0.5 + scale_b), nk * (0.5 + scale_b + 2)
        res.append({"format": f"{codebook}, {(fmt.upper() + ' double-quantized') if dq else 'fp32'} scales",
                    "quantize_us": round(qms * 1e3, 1),
                    "quantize_frac_hbm": round(qb / (qms * 1e-3) / 1e9 / PEAK_HBM_GBS, 4),
                    "dequantize_us": round(dms * 1e3, 1),
                    "dequantize_frac_hbm": round(db / (dms * 1e-3) / 1e9 / PEAK_HBM_GBS, 4),
                    "fwd_ms": round(fms, 4), "fwd_TFLOP/s": round(fwd / (fms * 1e-3) / 1e12, 1)})
        del w
    del out
    torch.cuda.empty_cache()
    return res


def bench_adamw(hip, layers, reps=20):
    """AdamW step over the step's four adapter tensors (A and B of the up and
    down projections, r=64: 4.72M parameters), without and with fp32 master
    copies.  Algorithmic bytes per parameter: 22 (bf16 param and grad read,
    fp32 moments read and written, bf16 param written), 30 with a master.
    Copies of the state are rotated so that the 256 MB Infinity Cache cannot
    hold what one step reads.  us_per_step: `reps` steps captured in a graph
    (median of five replays); eager_us_per_step: the same steps host-launched."""
    import torch
    import bit_nf4_quantized_17_amd as q
    st = torch.cuda.current_stream().cuda_stream
    shapes = [tuple(t.shape) for lay in layers for t in (lay.A, lay.B)]
    nparam = sum(a * b for a, b in shapes)
    res = {"params": nparam}
    for master in (False, True):
        per = 30 if master else 22
        ncopy = max(2, -(-512 * 2**20 // (per * nparam)))
        sets = []
        for c in range(ncopy):
            g = torch.Generator(device="cuda")
            g.manual_seed(100 + c)
            ps = [(torch.randn(sh, generator=g, device="cuda") * 0.02).to(torch.bfloat16) for sh in shapes]
            gs = [(torch.randn(sh, generator=g, device="cuda") * 1e-3).to(torch.bfloat16) for sh in shapes]
            ms = [torch.zeros(sh, device="cuda") for sh in shapes]
            vs = [torch.zeros(sh, device="cuda") for sh in shapes]
            ws = [p.float() for p in ps] if master else None
            sets.append((ps, gs, ms, vs, ws))

        def one(i):
            ps, gs, ms, vs, ws = sets[i % ncopy]
            q.qlora_adamw_step(ps, gs, ms, vs, 1e-4, weight_decay=0.01, step=i + 1, masters=ws)
        for i in range(3):
            one(i)
        e0, e1 = hip.event(), hip.event()
        torch.cuda.synchronize()
        hip.record(e0, st)
        for i in range(reps):
            one(i)
        hip.record(e1, st)
        eager_ms = hip.elapsed_ms(e0, e1) / reps
        # the same steps captured in a graph: a step takes about as long on the
        # host as on the GPU, so back-to-back host calls leave gaps between kernels
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph):
            for i in range(reps):
                one(i)
        torch.cuda.synchronize()
        ts = []
        for _ in range(5):
            hip.record(e0, st)
            graph.replay()
            hip.record(e1, st)
            ts.append(hip.elapsed_ms(e0, e1) / reps)
        ms_step = sorted(ts)[2]
        del graph
        gbs = per * nparam / (ms_step * 1e-3) / 1e9
        res["master" if master else "no_master"] = {"us_per_step": round(ms_step * 1e3, 1), "GB/s": round(gbs, 1),
                                                    "frac_hbm": round(gbs / PEAK_HBM_GBS, 4),
                                                    "eager_us_per_step": round(eager_ms * 1e3, 1)}
        del sets
        torch.cuda.empty_cache()
    return res


def bench_library_reference(hip, layers, reps=10):
    """Context only, not part of the path: a dense bf16 matmul from the vendor
    library (torch -> hipBLASLt) on the same shapes as the two fused forward
    GEMMs, with random operands.  It bounds what a dense GEMM reaches on this
    chip without any NF4 work; the fused kernels are compared with it."""
    import torch
    st = torch.cuda.current_stream().cuda_stream
    out = []
    g = torch.Generator(device="cuda").manual_seed(1)
    for lay in layers:
        X = torch.randn(lay.M, lay.K, device="cuda", dtype=torch.bfloat16, generator=g)
        Wt = torch.randn(lay.K, lay.N, device="cuda", dtype=torch.bfloat16, generator=g) * 0.02
        Wt = Wt.contiguous()
        for _ in range(3):
            X @ Wt
        e0, e1 = hip.event(), hip.event()
        torch.cuda.synchronize()
        hip.record(e0, st)
        for _ in range(reps):
            X @ Wt
        hip.record(e1, st)
        ms = hip.elapsed_ms(e0, e1) / reps
        fl = 2 * lay.M * lay.N * lay.K
        out.append({"MxNxK": f"{lay.M}x{lay.N}x{lay.K}", "ms": round(ms, 4),
                    "TFLOP/s": round(fl / (ms * 1e-3) / 1e12, 1)})
        del X, Wt
    torch.cuda.empty_cache()
    return out


def bench_training_configs(hip, reps=10):
    """The three smaller training shapes, fwd + bwd of every linear (inputs
    resident, weights quantized beforehand):
      C1 tiny 256x256, 16 tokens, r=8 (latency-bound: us per fwd + bwd);
      C2 7B attention projection 4096x4096, 4096 tokens, r=16;
      C3 7B MLP gate/up 4096->11008 and down 11008->4096, 8192 tokens, r=64
         (three forwards, then three backwards).
    graph_us: the steps captured in one HIP graph and replayed back to back;
    eager_us: host-launched steps (python + ctypes launch cost included)."""
    import torch
    import synthetic_inputs as si
    st = torch.cuda.current_stream().cuda_stream
    res = {}
    for tag, key, nrep in (("C1", "tiny_256", 200), ("C2", "attn_4096", reps), ("C3", "mlp7b_11008", reps)):
        cfg = si.CONFIGS[key]
        lays = [Layer(cfg, i) for i in range(len(cfg.layers))]
        for lay in lays:
            lay.quantize()

        def step():
            for lay in lays:
                lay.fwd()
            for lay in reversed(lays):
                lay.bwd()
        for _ in range(3):
            step()
        torch.cuda.synchronize()
        e0, e1 = hip.event(), hip.event()
        hip.record(e0, st)
        for _ in range(nrep):
            step()
        hip.record(e1, st)
        eager_ms = hip.elapsed_ms(e0, e1) / nrep
        side = torch.cuda.Stream()
        side.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(side):
            step()
        torch.cuda.current_stream().wait_stream(side)
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            for _ in range(nrep):
                step()
        g.replay()
        torch.cuda.synchronize()
        graph_ms = None
        for _ in range(3):
            e0, e1 = hip.event(), hip.event()
            hip.record(e0, st)
            g.replay()
            hip.record(e1, st)
            ms = hip.elapsed_ms(e0, e1) / nrep
            graph_ms = ms if graph_ms is None else min(graph_ms, ms)
        del g
        flops = sum(sum(lay.flops()[:2]) for lay in lays)
        tf = flops / (graph_ms * 1e-3) / 1e12
        res[tag] = {"workload": cfg.title, "flops_per_step": flops, "reps": nrep,
                    "graph_us": round(graph_ms * 1e3, 2), "eager_us": round(eager_ms * 1e3, 2),
                    "TFLOP/s": round(tf, 2), "frac_bf16_peak": round(tf / PEAK_BF16_TFLOPS, 4)}
        del lays
        torch.cuda.empty_cache()
    return res


def bench_context(hip):
    """What the chip itself delivers, from the benchmark's probe kernels
    (libqlora_probes.so, not part of the path) and torch's device copy:
      mfma_loop: v_mfma_f32_32x32x16_bf16 on register operands, 8 waves a
        compute unit, four accumulators a wave, zero and random operands;
      mfma_lds: the same MFMAs fed from LDS at the fused GEMMs' 128 x 64
        wave tile (six 16-byte fragment reads per eight MFMAs), random operands;
      hbm_read: 16-byte streaming loads over a 2 GiB buffer;
      hbm_copy: torch copy_ of 1 GiB (read + write counted);
      lds_read: 16-byte conflict-free LDS reads, one 512-thread workgroup a
        compute unit; bytes per clock per compute unit from the shader clock;
      empty_kernel: back-to-back launches of an empty kernel in a HIP graph."""
    import torch
    import bit_nf4_quantized_17_amd as q
    st = torch.cuda.current_stream().cuda_stream
    P = ctypes.CDLL(os.path.join(ROOT, "bit_nf4_quantized_17_amd", "libqlora_probes.so"))
    P.qlora_probe_mfma.argtypes = [ctypes.c_void_p, ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_void_p]
    P.qlora_probe_read.argtypes = [ctypes.c_void_p, ctypes.c_uint64, ctypes.c_void_p, ctypes.c_int,
                                   ctypes.c_void_p]
    P.qlora_probe_mfma_lds.argtypes = [ctypes.c_void_p, ctypes.c_int, ctypes.c_int, ctypes.c_int,
                                       ctypes.c_void_p]
    P.qlora_probe_lds.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int, ctypes.c_int,
                                  ctypes.c_void_p]
    P.qlora_probe_empty.argtypes = [ctypes.c_void_p]
    res = {}

    def timed(fn, reps):
        fn()
        torch.cuda.synchronize()
        e0, e1 = hip.event(), hip.event()
        hip.record(e0, st)
        for _ in range(reps):
            fn()
        hip.record(e1, st)
        return hip.elapsed_ms(e0, e1) / reps

    grid, iters = 512, 20000
    out = torch.empty(grid * 256, dtype=torch.float32, device="cuda")
    flops = grid * 4 * iters * 4 * 32768
    for zero in (1, 0):
        ms = timed(lambda: P.qlora_probe_mfma(out.data_ptr(), iters, zero, grid, st), 3)
        tf = flops / (ms * 1e-3) / 1e12
        res["mfma_loop_" + ("zero" if zero else "random")] = {
            "TFLOP/s": round(tf, 1), "frac_bf16_peak": round(tf / PEAK_BF16_TFLOPS, 4)}
    grid, iters = 256, 4000
    out = torch.empty(grid * 512, dtype=torch.float32, device="cuda")
    flops = grid * 8 * iters * 32 * 32768
    ms = timed(lambda: P.qlora_probe_mfma_lds(out.data_ptr(), iters, 0, grid, st), 3)
    tf = flops / (ms * 1e-3) / 1e12
    res["mfma_lds_random"] = {"TFLOP/s": round(tf, 1), "frac_bf16_peak": round(tf / PEAK_BF16_TFLOPS, 4)}
    del out
    buf = torch.empty(1 << 31, dtype=torch.uint8, device="cuda")
    sink = torch.empty(2048 * 256, dtype=torch.int32, device="cuda")
    ms = timed(lambda: P.qlora_probe_read(buf.data_ptr(), buf.numel(), sink.data_ptr(), 2048, st), 5)
    gbs = buf.numel() / (ms * 1e-3) / 1e9
    res["hbm_read"] = {"bytes": buf.numel(), "GB/s": round(gbs, 1), "frac_hbm": round(gbs / PEAK_HBM_GBS, 4)}
    del buf
    a = torch.empty(1 << 30, dtype=torch.uint8, device="cuda")
    b = torch.empty_like(a)
    ms = timed(lambda: b.copy_(a), 5)
    gbs = 2 * a.numel() / (ms * 1e-3) / 1e9
    res["hbm_copy"] = {"bytes_each_way": a.numel(), "GB/s": round(gbs, 1), "frac_hbm": round(gbs / PEAK_HBM_GBS, 4)}
    del a, b
    grid, iters = 256, 20000
    lsink = torch.empty(grid * 512, dtype=torch.int32, device="cuda")
    cyc = torch.zeros(grid, dtype=torch.int64, device="cuda")
    ms = timed(lambda: P.qlora_probe_lds(lsink.data_ptr(), cyc.data_ptr(), iters, grid, st), 3)
    per_wg = 512 * iters * 8 * 16
    cycles = cyc.double().median().item()
    res["lds_read"] = {"TB/s": round(grid * per_wg / (ms * 1e-3) / 1e12, 2),
                       "bytes_per_clk_cu": round(per_wg / cycles, 1),
                       "clock_GHz": round(cycles / (ms * 1e-3) / 1e9, 3)}
    del lsink, cyc
    n = 1000
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        P.qlora_probe_empty(torch.cuda.current_stream().cuda_stream)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        cap = torch.cuda.current_stream().cuda_stream
        for _ in range(n):
            P.qlora_probe_empty(cap)
    g.replay()
    torch.cuda.synchronize()
    e0, e1 = hip.event(), hip.event()
    hip.record(e0, st)
    g.replay()
    hip.record(e1, st)
    res["empty_kernel_us"] = round(hip.elapsed_ms(e0, e1) / n * 1e3, 3)
    del g
    torch.cuda.empty_cache()
    return res


def bench_quantize(hip, layers, reps=20):
    import torch
    st = torch.cuda.current_stream().cuda_stream
    res = []
    for lay in layers:
        e0, e1 = hip.event(), hip.event()
        lay.quantize()
        torch.cuda.synchronize()
        hip.record(e0, st)
        for _ in range(reps):
            lay.quantize()
        hip.record(e1, st)
        ms = hip.elapsed_ms(e0, e1) / reps
        gbs = quantize_bytes(lay.N, lay.K) / (ms * 1e-3) / 1e9
        res.append({"W": f"{lay.N}x{lay.K}", "us_per_call": round(ms * 1e3, 1),
                    "GB/s": round(gbs, 1), "frac_hbm": round(gbs / PEAK_HBM_GBS, 4)})
    return res


# ---------------------------------------------------------------------------
# CPU baseline: the oracle, as it stands, on a bounded sample
# ---------------------------------------------------------------------------
def cpu_baseline(lay, target_s=15.0):
    import numpy as np
    import oracle
    from synthetic_inputs import tensor_bits
    threads = oracle.default_threads()
    codes = lay.w.codes.cpu().numpy()
    qs = lay.w.qscale.cpu().numpy()
    ds = lay.w.dscale.cpu().numpy()
    Wdq = oracle.nf4_dequantize(codes, qs, ds, lay.N, lay.K)
    X, A, B, dY = (tensor_bits(t) for t in (lay.X, lay.A, lay.B, lay.dY))
    row_flops = (2 * lay.N * lay.K + 2 * lay.r * (lay.K + lay.N)) + \
        (2 * lay.N * lay.K + 2 * lay.r * (lay.K + lay.N))

    def run(nrows):
        rows = np.arange(nrows, dtype=np.int64)
        t0 = time.perf_counter()
        oracle.qlora_fwd(Wdq, X, A, B, lay.alpha, rows=rows, threads=threads)
        oracle.qlora_bwd_dx(Wdq, dY, A, B, lay.alpha, rows=rows, threads=threads)
        return time.perf_counter() - t0

    t1 = run(threads)                      # calibration: one row per thread
    n = int(max(threads, min(lay.M, threads * max(1, round(target_s / max(t1, 1e-3))))))
    n = (n // threads) * threads
    t = run(n)
    tf = n * row_flops / t / 1e12
    return {"value": round(tf, 6), "unit": "TFLOP/s", "cores": threads, "kind": "oracle",
            "seconds": round(t, 2),
            "sample": f"{n} token rows of the {lay.name} projection ({lay.N}x{lay.K}, r={lay.r}): "
                      f"forward rows of Y (with T) and backward rows of dX (with U), double sums"}


# ---------------------------------------------------------------------------
def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=10)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-extras", action="store_true", help="skip decode/quantize bandwidth runs")
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="only copy 1 GiB device-to-device 3 times (for scaling HBM byte counters)")
    ap.add_argument("--profile-decode", action="store_true",
                    help="only run each decode shape three times (for profiler counter passes)")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU: the library has no multi-GPU path "
              "(run with --gpus 1)", file=sys.stderr)
        sys.exit(2)

    import torch
    import bit_nf4_quantized_17_amd as q
    import synthetic_inputs as si

    torch.cuda.set_device(0)
    if args.calibrate_copy:
        a = torch.zeros(1 << 28, dtype=torch.float32, device="cuda")   # 1 GiB
        b = torch.empty_like(a)
        for _ in range(3):
            b.copy_(a)
        torch.cuda.synchronize()
        print(json.dumps({"calibrate_copy_bytes": a.numel() * 4, "copies": 3}))
        return
    if args.profile_decode:
        from synthetic_inputs import bf16_tensor
        dc = si.CONFIGS["decode_8192_28672"]
        for li, L in enumerate(dc.layers):
            w = q.nf4_quantize(torch.from_numpy(si.weight(dc, li)).cuda())
            A, B = (bf16_tensor(t) for t in si.adapters(dc, li))
            for M in dc.decode_M:
                X = bf16_tensor(si.activations(dc, li, M))
                for _ in range(3):
                    q.qlora_linear_fwd(w, X, A, B, dc.alpha)
        torch.cuda.synchronize()
        print(json.dumps({"profile_decode": [f"{L.N}x{L.K}" for L in dc.layers], "M": list(dc.decode_M),
                          "calls_each": 3}))
        return
    hip = Hip()
    cfg = si.CONFIGS["mlp70b_28672"]
    log("[bench] generating the 70B-class MLP slice inputs")
    layers = [Layer(cfg, 0), Layer(cfg, 1)]
    up, down = layers

    def step():
        up.quantize()
        down.quantize()
        up.fwd()
        down.fwd()
        down.bwd()
        up.bwd()
        up.decode()
        down.decode()

    log(f"[bench] warmup {args.warmup}")
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()

    # per-kernel events through the library's hook
    st = torch.cuda.current_stream().cuda_stream
    K = args.steps
    ev = {k: [[hip.event(), hip.event()] for _ in range(K)] for k in ("fwd_up", "fwd_down",
                                                                     "dx_up", "dx_down")}
    log(f"[bench] timing {K} steps")
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for s in range(K):
        up.quantize()
        down.quantize()
        q.qlora_set_timing_events(ev["fwd_up"][s][0], ev["fwd_up"][s][1])
        up.fwd()
        q.qlora_set_timing_events(ev["fwd_down"][s][0], ev["fwd_down"][s][1])
        down.fwd()
        q.qlora_set_timing_events(None, None, ev["dx_down"][s][0], ev["dx_down"][s][1])
        down.bwd()
        q.qlora_set_timing_events(None, None, ev["dx_up"][s][0], ev["dx_up"][s][1])
        up.bwd()
        q.qlora_set_timing_events()
        up.decode()
        down.decode()
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    ms_step = (t1 - t0) * 1e3 / K

    kern = {k: sum(hip.elapsed_ms(a, b) for a, b in v) / K for k, v in ev.items()}
    step_flops = sum(sum(l.flops()) for l in layers)
    value = step_flops / (ms_step * 1e-3) / 1e12

    # the dominant kernel: the larger of the fused fwd GEMM and the fused dX GEMM
    fwd_ms = (kern["fwd_up"] + kern["fwd_down"]) / 2
    dx_ms = (kern["dx_up"] + kern["dx_down"]) / 2
    main_flops = 2 * cfg.M * up.N * up.K + 2 * cfg.M * up.N * cfg.r   # base + LoRA prologue
    if dx_ms >= fwd_ms:
        dom, dom_ms = "k_gemm_big<1, 0> dX (NF4 transposed producer, U A prologue)", dx_ms
        dom_key = "gemm_dx"
    else:
        dom, dom_ms = "k_gemm_big<0, 0> fwd (NF4 producer, T B^T prologue)", fwd_ms
        dom_key = "gemm_fwd"
    achieved = main_flops / (dom_ms * 1e-3) / 1e12
    src = source_hash("gemm_big.hip")
    roofline = {"bound": "mfma", "achieved": round(achieved, 1), "peak": PEAK_BF16_TFLOPS,
                "unit": "TFLOP/s", "frac": round(achieved / PEAK_BF16_TFLOPS, 4),
                "traffic": load_traffic(dom_key, src), "kernel": dom,
                "launch_ms": round(dom_ms, 4), "flops_per_launch": main_flops,
                "other_gemm_ms": round(min(dx_ms, fwd_ms), 4)}

    # per-call breakdown (one extra step with events around every call)
    calls = [("quantize_up", up.quantize), ("quantize_down", down.quantize), ("fwd_up", up.fwd),
             ("fwd_down", down.fwd), ("bwd_down", down.bwd), ("bwd_up", up.bwd),
             ("decode_up_M16", up.decode), ("decode_down_M16", down.decode)]
    ce = [(n, f, hip.event(), hip.event()) for n, f in calls]
    torch.cuda.synchronize()
    for n, f, a, b in ce:
        hip.record(a, st)
        f()
        hip.record(b, st)
    breakdown = {n: round(hip.elapsed_ms(a, b), 4) for n, f, a, b in ce}
    fb_ms = sum(breakdown[k] for k in ("fwd_up", "fwd_down", "bwd_down", "bwd_up"))
    fb_flops = sum(l.flops()[0] + l.flops()[1] for l in layers)

    extras = {}
    if not args.no_extras:
        log("[bench] quantize bandwidth")
        extras["quantize"] = bench_quantize(hip, layers)
        log("[bench] decode shapes")
        extras["decode"] = bench_decode(hip)

    if not args.no_extras:
        log("[bench] dequantize, adapter merge")
        bw = bench_bf16_weight(hip, up)
        extras["dequantize"] = bw.pop("dequantize")
        extras["merge"] = bw
        log("[bench] gate/up dual projection")
        extras["dual"] = bench_dual(hip, up)
        log("[bench] codebook and scale-format variants")
        extras["formats"] = bench_formats(hip, up)
        log("[bench] adapter AdamW step")
        extras["adamw"] = bench_adamw(hip, layers)
        log("[bench] library reference")
        extras["context"] = {"hipblaslt_bf16_dense": bench_library_reference(hip, layers)}
        log("[bench] chip context probes")
        extras["context"].update(bench_context(hip))
        log("[bench] training shapes C1-C3")
        extras["training_configs"] = bench_training_configs(hip)

    cpu = None
    if not args.no_cpu_baseline:
        log("[bench] CPU oracle baseline")
        cpu = cpu_baseline(up)

    line = {
        "metric": METRIC, "value": round(value, 2), "unit": "TFLOP/s", "n_gpus": 1,
        "steps": K, "warmup": args.warmup, "ms_per_step": round(ms_step, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": "70B-class MLP slice: up W 28672x8192 and down W 8192x28672 "
                               "(NF4, double quant), 4096 tokens, LoRA r=64 alpha=16",
                   "M": cfg.M, "r": cfg.r, "alpha": cfg.alpha,
                   "step": "2x nf4_quantize + 2x fwd + 2x bwd + 2x decode fwd (M=16)",
                   "parallelism": "single GPU"},
        "roofline": roofline,
        "cpu_baseline": cpu,
        "fwd_bwd_tflops": round(fb_flops / (fb_ms * 1e-3) / 1e12, 2),
        "breakdown_ms": breakdown,
    }
    line.update(extras)
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
