"""Seeded synthetic inputs for the QLoRA NF4 linear layer.

This module only draws random numbers and lays them out; it holds none of the
method's arithmetic.  The tests, the smoke check and the benchmark take every
input from here, so the oracle and the HIP library always see identical bytes.

Workload shapes follow the layer sizes of 7B- and 70B-class transformer
projections (the pages' subject is fine-tuning such models on one GPU); the
value distributions follow the Ultralytics "QLoRA" snippet, which draws
pretrained-like weights as N(0, 0.02) in blocks of 64.  N(mu, x) means
standard deviation x.

Streams: numpy's PCG64 seeded with (seed, tensor id, layer index), one stream
per tensor, so that changing one tensor's size never shifts another's values.
bf16 tensors are drawn in fp32 and rounded to bf16 by torch (a library
conversion, not our code).
"""
from __future__ import annotations

import dataclasses
from typing import Dict, List

import numpy as np

_TENSOR_IDS = {"W": 1, "X": 2, "A": 3, "B": 4, "dY": 5, "outlier": 6}


@dataclasses.dataclass(frozen=True)
class Layer:
    name: str
    N: int          # out_features (rows of W)
    K: int          # in_features (cols of W)


@dataclasses.dataclass(frozen=True)
class Config:
    key: str
    title: str
    layers: List[Layer]
    M: int
    r: int
    alpha: float
    w_std: float = 0.02
    outlier_frac: float = 0.0
    outlier_scale: float = 20.0
    decode_M: tuple = ()
    seed: int = 0

    @property
    def a_std(self) -> float:
        return 1.0 / self.r


CONFIGS: Dict[str, Config] = {
    "tiny_256": Config("tiny_256", "tiny QLoRA linear 256x256, 16 tokens, r=8",
                 [Layer("proj", 256, 256)], M=16, r=8, alpha=16.0),
    "attn_4096": Config("attn_4096", "7B-class attention projection 4096x4096, 4096 tokens, r=16",
                 [Layer("attn", 4096, 4096)], M=4096, r=16, alpha=32.0),
    "mlp7b_11008": Config("mlp7b_11008", "7B-class MLP gate/up 4096->11008, down 11008->4096, 8192 tokens, r=64",
                 [Layer("gate", 11008, 4096), Layer("up", 11008, 4096), Layer("down", 4096, 11008)],
                 M=8192, r=64, alpha=16.0),
    "mlp70b_28672": Config("mlp70b_28672", "70B-class MLP slice up 8192->28672, down 28672->8192, 4096 tokens, r=64",
                 [Layer("up", 28672, 8192), Layer("down", 8192, 28672)],
                 M=4096, r=64, alpha=16.0, outlier_frac=0.01),
    "decode_8192_28672": Config("decode_8192_28672", "decode: W 8192x8192 and 28672x8192, M in {1,4,16}, r=16",
                 [Layer("sq", 8192, 8192), Layer("up", 28672, 8192)],
                 M=16, r=16, alpha=32.0, decode_M=(1, 4, 16)),
}


def _rng(seed: int, tensor: str, layer: int = 0) -> np.random.Generator:
    return np.random.default_rng([seed, _TENSOR_IDS[tensor], layer])


def normal_f32(shape, std: float, seed: int, tensor: str, layer: int = 0) -> np.ndarray:
    g = _rng(seed, tensor, layer)
    x = g.standard_normal(size=shape, dtype=np.float32)
    if std != 1.0:
        x *= np.float32(std)
    return x


def to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """fp32 -> bf16 (torch's round-to-nearest-even), returned as uint16 bit patterns."""
    import torch
    t = torch.from_numpy(np.ascontiguousarray(x, np.float32)).to(torch.bfloat16)
    return t.view(torch.int16).numpy().view(np.uint16).copy()


def bf16_bits_to_f32(h: np.ndarray) -> np.ndarray:
    return (np.asarray(h, np.uint16).astype(np.uint32) << 16).view(np.float32)


def bf16_tensor(bits: np.ndarray, device="cuda"):
    """bf16 bit patterns (uint16) -> a torch bfloat16 tensor on `device` (a copy)."""
    import torch
    t = torch.from_numpy(np.ascontiguousarray(bits, np.uint16).view(np.int16).copy())
    return t.view(torch.bfloat16).to(device)


def tensor_bits(t) -> np.ndarray:
    """A torch bf16 tensor's bit patterns as a host uint16 array."""
    import torch
    return t.detach().contiguous().view(torch.int16).cpu().numpy().view(np.uint16)


def weight(cfg: Config, li: int) -> np.ndarray:
    """fp32 frozen weight [N, K] ~ N(0, w_std); with outlier_frac > 0 a Bernoulli
    mask of that rate multiplies entries by outlier_scale."""
    L = cfg.layers[li]
    w = normal_f32((L.N, L.K), cfg.w_std, cfg.seed, "W", li)
    if cfg.outlier_frac > 0:
        g = _rng(cfg.seed, "outlier", li)
        mask = g.random(size=(L.N, L.K), dtype=np.float32) < np.float32(cfg.outlier_frac)
        w[mask] *= np.float32(cfg.outlier_scale)
    return w


def activations(cfg: Config, li: int, M: int | None = None) -> np.ndarray:
    """X [M, K] bf16 bits ~ N(0, 1); each projection gets its own input."""
    L = cfg.layers[li]
    M = cfg.M if M is None else M
    return to_bf16_bits(normal_f32((M, L.K), 1.0, cfg.seed, "X", li))


def adapters(cfg: Config, li: int):
    """(A [r, K], B [N, r]) bf16 bits; A ~ N(0, 1/r), B ~ N(0, 0.01)."""
    L = cfg.layers[li]
    A = to_bf16_bits(normal_f32((cfg.r, L.K), cfg.a_std, cfg.seed, "A", li))
    B = to_bf16_bits(normal_f32((L.N, cfg.r), 0.01, cfg.seed, "B", li))
    return A, B


def upstream(cfg: Config, li: int, M: int | None = None) -> np.ndarray:
    """dY [M, N] bf16 bits ~ N(0, 1)."""
    L = cfg.layers[li]
    M = cfg.M if M is None else M
    return to_bf16_bits(normal_f32((M, L.N), 1.0, cfg.seed, "dY", li))


def custom(N: int, K: int, M: int, r: int, alpha: float = 16.0, seed: int = 0,
           w_std: float = 0.02, outlier_frac: float = 0.0) -> Config:
    """A one-layer config of any shape (edge cases, ragged sizes)."""
    return Config(f"custom_{N}x{K}_m{M}_r{r}_s{seed}", f"custom {N}x{K} M={M} r={r}",
                  [Layer("proj", N, K)], M=M, r=r, alpha=alpha, w_std=w_std,
                  outlier_frac=outlier_frac, seed=seed)
