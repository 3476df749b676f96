"""Seeded synthetic inputs shared by the tests, the benchmark and the oracle checks.

This module only draws random numbers and lays them out in the canonical GGUF
Q4_0 byte format; it holds none of the GEMV's arithmetic.  Both the GPU path
and the CPU oracle receive exactly the bytes produced here.

Distributions (Qwen2.5-shaped decode workloads, "minfer" README, "Other
sizes" table and reproducibility notes of the nano-inference page):
  * Q4_0 block scale d_w = binary16(|N(0, 0.02)| / 8), drawn in fp64 then
    rounded to nearest even by NumPy (subnormal scales occur and are kept).
  * Nibble bytes uniform in 0..255, i.e. 32 uniform nibbles in 0..15 per block.
  * Activations x ~ N(0, 1) in fp32; optionally 8 distinct feature channels
    (shared by all N rows of one matrix) multiplied by 20.
Every stream is ``Generator(PCG64(SeedSequence([2026, cfg, m, copy, kind])))``.
"""
from __future__ import annotations

from dataclasses import dataclass

import numpy as np

Q4_BLOCK_BYTES = 18


def generator(cfg: int, m: int, copy: int = 0, kind: int = 0) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence([2026, cfg, m, copy, kind])))


def q4_0_weights(rows: int, cols: int, rng: np.random.Generator) -> np.ndarray:
    """uint8 [rows][cols/32][18]: fp16 scale (little-endian) then 16 uniform nibble bytes."""
    assert cols % 32 == 0
    nb = cols // 32
    nblk = rows * nb
    d = (np.abs(rng.normal(0.0, 0.02, size=nblk)) / 8.0).astype("<f2")
    qs = rng.integers(0, 256, size=(nblk, 16), dtype=np.uint8)
    out = np.empty((nblk, Q4_BLOCK_BYTES), np.uint8)
    out[:, 0:2] = d.view(np.uint8).reshape(nblk, 2)
    out[:, 2:] = qs
    return out.reshape(rows, nb, Q4_BLOCK_BYTES)


def q8_0_weights(rows: int, cols: int, rng: np.random.Generator) -> np.ndarray:
    """uint8 [rows][cols/32][34]: fp16 scale (little-endian) then 32 int8 values uniform in
    -127..127 (the range a Q8_0 quantizer produces); the scale as for Q4_0 weights."""
    assert cols % 32 == 0
    nb = cols // 32
    nblk = rows * nb
    d = (np.abs(rng.normal(0.0, 0.02, size=nblk)) / 8.0).astype("<f2")
    qs = rng.integers(-127, 128, size=(nblk, 32), dtype=np.int8)
    out = np.empty((nblk, 34), np.uint8)
    out[:, 0:2] = d.view(np.uint8).reshape(nblk, 2)
    out[:, 2:] = qs.view(np.uint8)
    return out.reshape(rows, nb, 34)


def activation(n: int, cols: int, rng: np.random.Generator, outliers: int = 8,
               factor: float = 20.0) -> np.ndarray:
    """fp32 [n][cols] ~ N(0,1), with `outliers` shared channels scaled by `factor`."""
    x = rng.standard_normal(size=(n, cols), dtype=np.float32)
    if outliers:
        ch = rng.choice(cols, size=min(outliers, cols), replace=False)
        x[:, ch] *= np.float32(factor)
    return x


@dataclass(frozen=True)
class MatShape:
    name: str
    rows: int
    cols: int

    @property
    def q4_bytes(self) -> int:
        return self.rows * (self.cols // 32) * Q4_BLOCK_BYTES


def qwen_stack(hidden: int, kv: int, ff: int, vocab: int, layers: int = 28) -> list[MatShape]:
    """Every projection of one decode token in layer order, then the output head."""
    mats: list[MatShape] = []
    for layer in range(layers):
        mats += [MatShape(f"l{layer}.q", hidden, hidden), MatShape(f"l{layer}.k", kv, hidden),
                 MatShape(f"l{layer}.v", kv, hidden), MatShape(f"l{layer}.o", hidden, hidden),
                 MatShape(f"l{layer}.gate", ff, hidden), MatShape(f"l{layer}.up", ff, hidden),
                 MatShape(f"l{layer}.down", hidden, ff)]
    mats.append(MatShape("lm_head", vocab, hidden))
    return mats


def qwen25_1p5b() -> list[MatShape]:
    """Qwen2.5-1.5B: 28 layers, d=1536, ff=8960, 2 KV heads x 128, vocab 151936."""
    return qwen_stack(1536, 256, 8960, 151936)


def qwen25_7b() -> list[MatShape]:
    """Qwen2.5-7B-shaped stream: d=3584, ff=18944, 4 KV heads x 128, vocab 152064."""
    return qwen_stack(3584, 512, 18944, 152064)


def stack_inputs(cfg: int, shapes: list[MatShape], n: int, copy: int = 0,
                 act_cfg: int | None = None, outliers: int = 8):
    """Weights and fresh activations for every matrix of a stack (generator)."""
    for m, s in enumerate(shapes):
        w = q4_0_weights(s.rows, s.cols, generator(cfg, m, copy, 0))
        x = activation(n, s.cols, generator(cfg if act_cfg is None else act_cfg, m, copy, 1),
                       outliers=outliers)
        yield s, w, x
