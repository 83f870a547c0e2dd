"""Seeded synthetic inputs for the per-block mixed-precision linear.

This module only draws random numbers; it holds none of the method's
arithmetic (no scales, codes, rounding rules or error measures).  The GPU path,
the CPU oracle, the tests and the benchmark all take their inputs from here, so
both sides of every comparison see the same bytes.

Every weight set is a stand-in with the shape and value distribution of the
workloads on the HyperTensor page ("Usage Example": a 4096-wide MLP of depth 4
with ReLU; "TinyLLaMA Benchmark": a TinyLlama model).  No trained weights are
used; values are drawn from the distributions stated next to each generator.

Conventions
  * "x% of entries / blocks / columns" means exactly round(x * count) distinct
    positions, drawn without replacement.
  * "times c" multiplies the chosen entries by c.
  * Each tensor gets its own numpy PCG64 stream, seeded from
    (config id, layer index, tensor name) through ``seed_for``.
  * Activations are drawn in float32 and handed to the library as bfloat16 bit
    patterns (uint16); the float32 -> bfloat16 cast is torch's (round to
    nearest even).
"""
from __future__ import annotations

import hashlib
from dataclasses import dataclass

import numpy as np

BLOCK_K = 64


def seed_for(*parts) -> int:
    """A stable 63-bit seed derived from a tuple of names / integers."""
    h = hashlib.sha256("/".join(str(p) for p in parts).encode()).digest()
    return int.from_bytes(h[:8], "little") & ((1 << 63) - 1)


def rng_for(*parts) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(seed_for(*parts)))


def _choose(rng: np.random.Generator, count: int, frac: float) -> np.ndarray:
    k = int(round(frac * count))
    return rng.choice(count, size=k, replace=False)


def to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """float32 array -> bfloat16 bit patterns (uint16), via torch's cast."""
    import torch

    t = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32))
    return t.to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16).copy()


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    """bfloat16 bit patterns -> float32 values (exact widening)."""
    return (b.astype(np.uint32) << 16).view(np.float32)


# ---------------------------------------------------------------------------
# Small correctness case: one 256 x 256 fp32 weight.
# ---------------------------------------------------------------------------
def small_weight(seed: int = 0, n: int = 256, k: int = 256) -> np.ndarray:
    """W ~ N(0, 0.02); 2% of the 64-wide K-blocks scaled x20; then 1% of the
    entries replaced by N(0, 1) outliers.  Seed 0 by default."""
    rng = np.random.Generator(np.random.PCG64(seed))
    w = rng.normal(0.0, 0.02, size=(n, k)).astype(np.float32)
    kb = k // BLOCK_K
    blocks = _choose(rng, n * kb, 0.02)
    for b in blocks:
        r, j = divmod(int(b), kb)
        w[r, j * BLOCK_K:(j + 1) * BLOCK_K] *= np.float32(20.0)
    ent = _choose(rng, n * k, 0.01)
    w.reshape(-1)[ent] = rng.normal(0.0, 1.0, size=ent.size).astype(np.float32)
    return w


def small_activation(seed: int = 0, m: int = 1, k: int = 256) -> np.ndarray:
    """x ~ N(0, 1) as float32 (the caller rounds it to bfloat16 once)."""
    rng = np.random.Generator(np.random.PCG64(seed + 1_000_003))
    return rng.normal(0.0, 1.0, size=(m, k)).astype(np.float32)


# ---------------------------------------------------------------------------
# 4-layer MLP, dim 4096: Linear(4096, 4096) + ReLU, four times, no bias.
# ---------------------------------------------------------------------------
MLP_DIM = 4096
MLP_DEPTH = 4


def mlp_weight(layer: int, dim: int = MLP_DIM, seed: int = 0) -> np.ndarray:
    """Student-t (nu = 4) scaled to std 1/64 (a t4 variable has variance 2);
    0.5% of the input columns multiplied by 8."""
    rng = rng_for("mlp4096", seed, layer, "W")
    w = rng.standard_t(4.0, size=(dim, dim)) * (1.0 / 64.0) / np.sqrt(2.0)
    w = w.astype(np.float32)
    cols = _choose(rng, dim, 0.005)
    w[:, cols] *= np.float32(8.0)
    return w


def mlp_activation(m: int, dim: int = MLP_DIM, seed: int = 0) -> np.ndarray:
    rng = rng_for("mlp4096", seed, m, "x")
    return rng.normal(0.0, 1.0, size=(m, dim)).astype(np.float32)


# ---------------------------------------------------------------------------
# Transformer-shaped linear stacks (random init, shapes only).
# ---------------------------------------------------------------------------
@dataclass(frozen=True)
class LinearShape:
    name: str
    n: int  # output features (rows of W)
    k: int  # input features


def tinyllama_shapes() -> list[LinearShape]:
    """One TinyLlama-1.1B decoder layer: hidden 2048, intermediate 5632,
    4 KV heads x 64."""
    h, i, kv = 2048, 5632, 256
    return [LinearShape("q", h, h), LinearShape("k", kv, h), LinearShape("v", kv, h),
            LinearShape("o", h, h), LinearShape("gate", i, h), LinearShape("up", i, h),
            LinearShape("down", h, i)]


TINYLLAMA_LAYERS = 22


def llama8b_shapes() -> list[LinearShape]:
    """One Llama-3.1-8B decoder layer: hidden 4096, intermediate 14336,
    KV dim 1024."""
    h, i, kv = 4096, 14336, 1024
    return [LinearShape("q", h, h), LinearShape("k", kv, h), LinearShape("v", kv, h),
            LinearShape("o", h, h), LinearShape("gate", i, h), LinearShape("up", i, h),
            LinearShape("down", h, i)]


LLAMA8B_LAYERS = 32


def tinyllama_weight(layer: int, shape: LinearShape, seed: int = 0) -> np.ndarray:
    """N(0, 0.02) plus 0.1% of the entries multiplied by 30."""
    rng = rng_for("tinyllama", seed, layer, shape.name)
    w = rng.normal(0.0, 0.02, size=(shape.n, shape.k)).astype(np.float32)
    ent = _choose(rng, w.size, 0.001)
    w.reshape(-1)[ent] *= np.float32(30.0)
    return w


def llama8b_weight(layer: int, shape: LinearShape, seed: int = 0) -> np.ndarray:
    """N(0, 0.02) times a per-row log-normal(0, 0.5) factor, plus 0.1% of the
    entries multiplied by 30."""
    rng = rng_for("llama8b", seed, layer, shape.name)
    w = rng.normal(0.0, 0.02, size=(shape.n, shape.k))
    w *= np.exp(rng.normal(0.0, 0.5, size=(shape.n, 1)))
    w = w.astype(np.float32)
    ent = _choose(rng, w.size, 0.001)
    w.reshape(-1)[ent] *= np.float32(30.0)
    return w


def activation(tag: str, m: int, k: int, seed: int = 0) -> np.ndarray:
    rng = rng_for(tag, seed, m, k, "x")
    return rng.normal(0.0, 1.0, size=(m, k)).astype(np.float32)


# ---------------------------------------------------------------------------
# Adversarial tiny blocks for edge cases (each row of the result is one
# 64-wide block; the caller lays them out as it needs).
# ---------------------------------------------------------------------------
def edge_blocks(seed: int = 0) -> np.ndarray:
    """A fixed catalogue of hard 64-element blocks: zeros, signed zeros,
    subnormals, huge values, exact integer grids, ties at half-integers, single
    outliers, bfloat16- and float16-valued blocks, and NaN / Inf."""
    rng = np.random.Generator(np.random.PCG64(seed + 77))
    rows = []
    rows.append(np.zeros(64, np.float32))
    z = np.zeros(64, np.float32); z[::2] = -0.0; rows.append(z)
    rows.append((rng.normal(size=64) * 1e-39).astype(np.float32))      # subnormal
    rows.append((rng.normal(size=64) * 1e-44).astype(np.float32))      # deep subnormal
    rows.append((rng.normal(size=64) * 1e37).astype(np.float32))       # huge
    rows.append(np.full(64, 3.4e38, np.float32))                      # near FLT_MAX
    g = rng.integers(-127, 128, size=64).astype(np.float32); g[5] = 127.0
    rows.append(g * np.float32(2.0 ** -10))                           # INT8 grid
    rows.append(g * np.float32(3.0))                                  # INT8 grid, non-pow2 scale
    g4 = rng.integers(-7, 8, size=64).astype(np.float32); g4[9] = -7.0
    rows.append(g4 * np.float32(2.0 ** -3))                           # INT4 grid
    h = (rng.integers(-7, 7, size=64) + 0.5).astype(np.float32); h[0] = 7.0
    rows.append(h)                                                    # half-integer ties, s = 1
    o = (rng.normal(size=64) * 0.01).astype(np.float32); o[17] = 5.0
    rows.append(o)                                                    # single outlier
    b = rng.normal(size=64).astype(np.float32)
    b = (b.view(np.uint32) & np.uint32(0xFFFF0000)).view(np.float32); b[3] = 40.0
    rows.append(b)                                                    # bfloat16-valued
    f = rng.normal(size=64).astype(np.float16).astype(np.float32); f[7] = 9.0
    rows.append(f)                                                    # float16-valued
    f2 = (rng.normal(size=64) * 1e-6).astype(np.float16).astype(np.float32)
    rows.append(f2)                                                   # fp16 subnormals
    big16 = np.full(64, 65520.0, np.float32); big16[1::2] = 1.0
    rows.append(big16)                                                # fp16 overflow tie
    n1 = rng.normal(size=64).astype(np.float32); n1[11] = np.nan
    rows.append(n1)
    n2 = rng.normal(size=64).astype(np.float32); n2[40] = np.inf
    rows.append(n2)
    n3 = rng.normal(size=64).astype(np.float32); n3[0] = -np.inf
    rows.append(n3)
    rows.append(np.full(64, 1.0, np.float32))
    rows.append(np.full(64, -2.5, np.float32))
    one = np.zeros(64, np.float32); one[63] = 1e-30
    rows.append(one)
    return np.stack(rows).astype(np.float32)


# ---------------------------------------------------------------------------
# Device-side generators for the full-size stacks (billions of entries, too
# many to draw on the host).  Same distributions as the numpy generators
# above, drawn with torch's device generator seeded through ``seed_for``; the
# outlier positions are Bernoulli(frac) per entry rather than an exact count.
# ---------------------------------------------------------------------------
def torch_generator(device, *parts):
    import torch

    g = torch.Generator(device=device)
    g.manual_seed(seed_for(*parts))
    return g


def tinyllama_weight_gpu(layer: int, shape: LinearShape, device, seed: int = 0):
    """fp32 [n, k] on `device`: N(0, 0.02), 0.1% of the entries times 30."""
    import torch

    g = torch_generator(device, "tinyllama-gpu", seed, layer, shape.name)
    w = torch.randn(shape.n, shape.k, generator=g, device=device) * 0.02
    hit = torch.rand(shape.n, shape.k, generator=g, device=device) < 0.001
    return torch.where(hit, w * 30.0, w)


def llama8b_weight_gpu(layer: int, shape: LinearShape, device, seed: int = 0):
    """fp32 [n, k] on `device`: N(0, 0.02) times a per-row log-normal(0, 0.5)
    factor, 0.1% of the entries times 30."""
    import torch

    g = torch_generator(device, "llama8b-gpu", seed, layer, shape.name)
    w = torch.randn(shape.n, shape.k, generator=g, device=device) * 0.02
    w *= torch.exp(torch.randn(shape.n, 1, generator=g, device=device) * 0.5)
    hit = torch.rand(shape.n, shape.k, generator=g, device=device) < 0.001
    return torch.where(hit, w * 30.0, w)
