"""Seeded synthetic inputs shared by the tests, the smoke check and the bench.

This module draws random numbers and stores them in the element types the
library takes.  It holds none of the normalisation's arithmetic: the same
tensors are handed to the CPU oracle and to the GPU library.

Recipe (every tensor): a NumPy PCG64 stream keyed by (seed, tag) draws
binary64 standard normals; they are scaled and shifted, rounded to binary32 by
NumPy, and, for bfloat16, rounded again by torch's float32 -> bfloat16
conversion (round-to-nearest-even).  Tags keep tensors independent: "x", "r",
"w", "dy", "outlier-cols", "pos", "wq", "wk".

The pages run RMSNorm and fused Add + RMSNorm on bfloat16 LLM activations (the
KernelAgent digest's SM100 benchmark suite of Quack and DeepSeek norm
workloads, whose shape lists are not printed); the named workloads below are
synthetic stand-ins of the same kind: zero-mean unit-scale activations, a
residual stream, and weights near one.
"""
from __future__ import annotations

import zlib

import numpy as np
import torch


def _rng(seed: int, tag: str) -> np.random.Generator:
    return np.random.default_rng(np.random.SeedSequence(entropy=seed,
                                                        spawn_key=(zlib.crc32(tag.encode()),)))


def normal(seed: int, tag: str, shape, mean: float = 0.0, std: float = 1.0) -> np.ndarray:
    """binary64 draws of N(mean, std^2)."""
    return mean + std * _rng(seed, tag).standard_normal(size=shape, dtype=np.float64)


def store(a: np.ndarray, dtype: torch.dtype) -> torch.Tensor:
    """Store binary64 draws in a torch CPU tensor of the given element type."""
    if dtype == torch.float64:
        return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float64))
    t = torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32))
    return t if dtype == torch.float32 else t.to(dtype)


def weight(seed: int, n: int, dtype: torch.dtype, tag: str = "w") -> torch.Tensor:
    """w = 1 + 0.1 * N(0, 1), the per-channel scale."""
    return store(normal(seed, tag, (n,), mean=1.0, std=0.1), dtype)


def positions(seed: int, T: int, P: int, seq_len: int | None = None) -> torch.Tensor:
    """int64 positions of T tokens in [0, P): with seq_len, a batch of
    sequences that each count 0, 1, ..., seq_len - 1 (a prefill batch);
    otherwise independent uniform draws (tag "pos")."""
    if seq_len is not None:
        return torch.arange(T, dtype=torch.int64) % min(seq_len, P)
    return torch.from_numpy(_rng(seed, "pos").integers(0, P, size=T, dtype=np.int64))


def rope_table(P: int, D: int, base: float = 10000.0):
    """cos and sin tables [P, D/2] float32 of the angles p * base^(-2i/D),
    formed in binary64 and rounded once.  They are inputs of the RMSNorm +
    RoPE op, which reads them and never forms an angle itself."""
    i = np.arange(D // 2, dtype=np.float64)
    ang = np.arange(P, dtype=np.float64)[:, None] * base ** (-2.0 * i / D)[None, :]
    return (torch.from_numpy(np.cos(ang).astype(np.float32)),
            torch.from_numpy(np.sin(ang).astype(np.float32)))


def rmsnorm_rope_inputs(T: int, Hq: int, Hk: int, D: int, dtype=torch.bfloat16, w_dtype=None,
                        seed: int = 0, P: int = 32768, seq_len: int | None = None):
    """A packed query/key/value projection output qkv [T, (Hq + 2 Hk) * D] ~ N(0, 1),
    per-dimension query and key norm weights wq, wk [D] (tags "wq", "wk"),
    rotary tables cos, sin [P, D/2] and positions pos [T]."""
    cos, sin = rope_table(P, D)
    return {"qkv": store(normal(seed, "x", (T, (Hq + 2 * Hk) * D)), dtype),
            "wq": weight(seed, D, w_dtype or dtype, "wq"),
            "wk": weight(seed, D, w_dtype or dtype, "wk"),
            "cos": cos, "sin": sin, "pos": positions(seed, T, P, seq_len)}


def outlier_columns(seed: int, n: int, frac: float = 0.01) -> np.ndarray:
    """round(frac * n) distinct column indices, sorted, fixed by the seed."""
    k = int(round(frac * n))
    return np.sort(_rng(seed, "outlier-cols").choice(n, size=k, replace=False))


def rmsnorm_fwd_inputs(M: int, N: int, dtype=torch.float32, w_dtype=None, seed: int = 0,
                       x_std: float = 1.0):
    """Plain RMSNorm forward: x ~ N(0, x_std^2), w = 1 + 0.1 N(0,1)."""
    return {"x": store(normal(seed, "x", (M, N), std=x_std), dtype),
            "w": weight(seed, N, w_dtype or dtype)}


def add_rmsnorm_fwd_inputs(M: int, N: int, dtype=torch.bfloat16, w_dtype=None, seed: int = 0,
                           x_std: float = 1.0, r_std: float = 1.0, outlier_frac: float = 0.0,
                           outlier_scale: float = 300.0):
    """Fused Add+RMSNorm forward inputs.  With outlier_frac > 0, the columns
    chosen by outlier_columns() carry x drawn with outlier_scale times the
    std (scaled before the single rounding)."""
    xa = normal(seed, "x", (M, N), std=x_std)
    if outlier_frac > 0.0:
        cols = outlier_columns(seed, N, outlier_frac)
        xa[:, cols] *= outlier_scale
    return {"x": store(xa, dtype),
            "r": store(normal(seed, "r", (M, N), std=r_std), dtype),
            "w": weight(seed, N, w_dtype or dtype)}


def rmsnorm_bwd_inputs(M: int, N: int, dtype=torch.bfloat16, w_dtype=None, seed: int = 0):
    """Backward inputs x, dy ~ N(0,1), w = 1 + 0.1 N(0,1).  The saved rstd is
    produced by a forward over x (by the side under test's own reference)."""
    return {"x": store(normal(seed, "x", (M, N)), dtype),
            "dy": store(normal(seed, "dy", (M, N)), dtype),
            "w": weight(seed, N, w_dtype or dtype)}


# The named workloads: shapes, element types and distributions.
WORKLOADS = {
    "rmsnorm_fwd_f32_256x4096": dict(
        op="rmsnorm_fwd", M=256, N=4096, dtype=torch.float32, w_dtype=torch.float32, eps=1e-6),
    "add_rmsnorm_fwd_bf16_4096x4096": dict(
        op="add_rmsnorm_fwd", M=4096, N=4096, dtype=torch.bfloat16, w_dtype=torch.bfloat16,
        eps=1e-6),
    "add_rmsnorm_fwd_bf16_16384x7168": dict(
        op="add_rmsnorm_fwd", M=16384, N=7168, dtype=torch.bfloat16, w_dtype=torch.bfloat16,
        eps=1e-6, r_std=0.5),
    "add_rmsnorm_fwd_bf16_decode_n8192": dict(
        op="add_rmsnorm_fwd", M_list=(1, 8, 32, 128, 512), N=8192, dtype=torch.bfloat16,
        w_dtype=torch.float32, eps=1e-5, outlier_frac=0.01, outlier_scale=300.0),
    "rmsnorm_bwd_bf16_32768x4096": dict(
        op="rmsnorm_bwd", M=32768, N=4096, dtype=torch.bfloat16, w_dtype=torch.bfloat16,
        eps=1e-6),
    # per-head RMSNorm + RoPE of the query and key heads: 4 sequences of 4096
    # tokens, 32 query and 8 key heads of 128
    "rmsnorm_rope_bf16_t16384_q32_k8_d128": dict(
        op="rmsnorm_rope", T=16384, Hq=32, Hk=8, D=128, dtype=torch.bfloat16,
        w_dtype=torch.bfloat16, eps=1e-6, P=32768, seq_len=4096),
}


def workload_inputs(name: str, M: int | None = None, seed: int = 0):
    """Inputs of a named workload (M overrides the row count)."""
    cfg = WORKLOADS[name]
    M = M if M is not None else cfg.get("M")
    if cfg["op"] == "rmsnorm_fwd":
        return rmsnorm_fwd_inputs(M, cfg["N"], cfg["dtype"], cfg["w_dtype"], seed)
    if cfg["op"] == "add_rmsnorm_fwd":
        return add_rmsnorm_fwd_inputs(M, cfg["N"], cfg["dtype"], cfg["w_dtype"], seed,
                                      r_std=cfg.get("r_std", 1.0),
                                      outlier_frac=cfg.get("outlier_frac", 0.0),
                                      outlier_scale=cfg.get("outlier_scale", 300.0))
    if cfg["op"] == "rmsnorm_rope":
        return rmsnorm_rope_inputs(M if M is not None else cfg["T"], cfg["Hq"], cfg["Hk"], cfg["D"],
                                   cfg["dtype"], cfg["w_dtype"], seed, cfg["P"], cfg["seq_len"])
    return rmsnorm_bwd_inputs(M, cfg["N"], cfg["dtype"], cfg["w_dtype"], seed)
