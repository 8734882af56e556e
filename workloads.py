"""Synthetic FSDP units and seeded inputs shared by the tests and the benchmark.

This module holds no arithmetic of the data path: it only names unit shapes and
draws random numbers.  Both the HIP library and the CPU oracle are fed from it.

Unit shapes stand in for the pages' workloads (T5, GPT-175B, GPT-2 Large
blocks; no dataset, checkpoint or trained weight is needed or used).  Parameter
order inside a unit is the order the shapes are listed in: for GPT blocks the
two LayerNorms first (weight, bias each), then every Linear weight followed by
its bias.
"""
from __future__ import annotations

from dataclasses import dataclass, field
from typing import List, Sequence, Tuple

import numpy as np

FLAT = 1
ROWS = 2

Shape = Tuple[int, ...]


@dataclass
class Unit:
    name: str
    layout: int                 # FLAT (FSDP1 FlatParameter) or ROWS (FSDP2 dim-0)
    N: int                      # simulated shard count
    names: List[str]
    shapes: List[Shape]
    std: float = 0.02           # parameter init ~ N(0, std)
    grad_std: float = 1e-3      # gradient contributions ~ N(0, grad_std), rounded to bf16
    adam: dict = field(default_factory=lambda: dict(lr=1e-3, betas=(0.9, 0.999), eps=1e-8,
                                                     weight_decay=0.01))

    @property
    def numels(self) -> List[int]:
        out = []
        for s in self.shapes:
            n = 1
            for d in s:
                n *= int(d)
            out.append(n)
        return out

    @property
    def total(self) -> int:
        return sum(self.numels)


def gpt_block(d: int) -> Tuple[List[str], List[Shape]]:
    """One GPT-2 style transformer block of width d (4d MLP)."""
    names = ["ln1.w", "ln1.b", "ln2.w", "ln2.b",
             "attn.qkv.w", "attn.qkv.b", "attn.proj.w", "attn.proj.b",
             "mlp.fc.w", "mlp.fc.b", "mlp.fc2.w", "mlp.fc2.b"]
    shapes = [(d,), (d,), (d,), (d,),
              (3 * d, d), (3 * d,), (d, d), (d,),
              (4 * d, d), (4 * d,), (d, 4 * d), (d,)]
    return names, shapes


def tiny_mlp(N: int = 4) -> Unit:
    """Two-layer MLP: W1[64,32], b1[64], W2[16,64], b2[16] (3,152 elements)."""
    return Unit("tiny-mlp", FLAT, N, ["W1", "b1", "W2", "b2"],
                [(64, 32), (64,), (16, 64), (16,)])


def gpt2_large_block(N: int = 8) -> Unit:
    names, shapes = gpt_block(1280)
    return Unit("gpt2-large-block", FLAT, N, names, shapes)


def gpt2_large_emb_rows(N: int = 8) -> Unit:
    """FSDP2 unit: token embedding [50257,1280] plus one GPT-2 Large block, dim-0 sharded."""
    names, shapes = gpt_block(1280)
    return Unit("gpt2-large-emb+block-rows", ROWS, N, ["wte"] + names, [(50257, 1280)] + shapes)


def t5_11b_block(N: int = 8) -> Unit:
    """T5-11B style block: d_model 1024, 128 heads x 128, FFN 65536, one RMSNorm."""
    names = ["q", "k", "v", "o", "wi", "wo", "rmsnorm.w"]
    shapes = [(16384, 1024), (16384, 1024), (16384, 1024), (1024, 16384),
              (65536, 1024), (1024, 65536), (1024,)]
    return Unit("t5-11b-block", FLAT, N, names, shapes)


def gpt175b_block(N: int = 128) -> Unit:
    names, shapes = gpt_block(12288)
    return Unit("gpt-175b-block", FLAT, N, names, shapes, std=0.006)


# ---------------------------------------------------------------------------
# seeded generators
# ---------------------------------------------------------------------------

def host_params(unit: Unit, seed: int = 0) -> List[np.ndarray]:
    """fp32 ~ N(0, std) in the unit's shapes, drawn in parameter order (numpy PCG64)."""
    rng = np.random.Generator(np.random.PCG64(seed))
    out = []
    for s in unit.shapes:
        a = rng.standard_normal(size=s, dtype=np.float32)
        a *= np.float32(unit.std)
        out.append(a)
    return out


def host_normal(n: int, std: float, seed: int) -> np.ndarray:
    rng = np.random.Generator(np.random.PCG64(seed))
    a = rng.standard_normal(size=n, dtype=np.float32)
    a *= np.float32(std)
    return a


def contrib_seed(step: int, r: int) -> int:
    """Seed of rank r's gradient contribution at optimizer step t."""
    return 1000 * step + r


def host_contribs(N: int, length: int, std: float = 1e-3, step: int = 1) -> np.ndarray:
    """N bf16 gradient contributions of `length` elements, as a uint16 [N, length] array.

    Each is fp32 ~ N(0, std) rounded to bf16 by torch's CPU cast (a library
    routine, so that neither side under test produces its own inputs)."""
    import torch
    out = np.empty((N, length), dtype=np.uint16)
    for r in range(N):
        x = torch.from_numpy(host_normal(length, std, contrib_seed(step, r)))
        out[r] = x.to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    return out


def random_bits_f32(n: int, seed: int) -> np.ndarray:
    """Arbitrary binary32 bit patterns (every class: zeros, subnormals, normals, inf, NaN)."""
    rng = np.random.Generator(np.random.PCG64(seed))
    return rng.integers(0, 2 ** 32, size=n, dtype=np.uint64).astype(np.uint32).view(np.float32)


def special_f32() -> np.ndarray:
    """Hand-picked binary32 values around every rounding boundary of bf16."""
    bits = [
        0x00000000, 0x80000000,                  # +-0
        0x00000001, 0x00007FFF, 0x00008000, 0x00008001, 0x00018000, 0x007FFFFF,  # subnormals
        0x00800000, 0x3F800000, 0x3F808000, 0x3F818000, 0x3F808001, 0x3F80FFFF,  # ties / near
        0xBF808000, 0xBF818000, 0x7F7F7FFF, 0x7F7F8000, 0x7F7FFFFF, 0xFF7FFFFF,  # overflow
        0x7F800000, 0xFF800000, 0x7FC00000, 0xFFC00001, 0x7F800001, 0x7FBFFFFF,  # inf / NaN
        0x3EFFFFFF, 0x33800000, 0x4B800000, 0x4B800001,
    ]
    return np.asarray(bits, dtype=np.uint32).view(np.float32)


# ---------------------------------------------------------------------------
# device generators (large units; the same bytes are copied to the host for the oracle)
# ---------------------------------------------------------------------------

def device_params(unit: Unit, seed: int = 0, device: str = "cuda"):
    import torch
    g = torch.Generator(device=device)
    g.manual_seed(seed)
    out = []
    for s in unit.shapes:
        t = torch.randn(s, generator=g, device=device, dtype=torch.float32)
        t.mul_(unit.std)
        out.append(t)
    return out


def device_contribs(N: int, length: int, std: float = 1e-3, step: int = 1, device: str = "cuda",
                    pitch: int = None):
    """[N, length] bf16 contributions drawn on the device (one row per rank).  With `pitch`
    the rows sit `pitch` elements apart in one buffer and the [N, length] view is returned."""
    import torch
    pitch = length if pitch is None else pitch
    if pitch < length:
        raise ValueError("pitch must be at least the row length")
    buf = torch.empty((N, pitch), dtype=torch.bfloat16, device=device)
    out = buf[:, :length]
    g = torch.Generator(device=device)
    for r in range(N):
        g.manual_seed(contrib_seed(step, r))
        x = torch.randn(length, generator=g, device=device, dtype=torch.float32)
        x.mul_(std)
        out[r].copy_(x)
    return out


def random_unit_shapes(rng: np.random.Generator, max_params: int = 5, max_dim: int = 6) -> List[Shape]:
    """Small random shapes for brute force: 0-d, 1-d, 2-d and 3-d, zero-size included."""
    shapes: List[Shape] = []
    for _ in range(int(rng.integers(1, max_params + 1))):
        nd = int(rng.integers(0, 4))
        shapes.append(tuple(int(rng.integers(0, max_dim + 1)) for _ in range(nd)))
    return shapes


def all_units() -> Sequence[Unit]:
    return [tiny_mlp(), gpt2_large_block(), gpt2_large_emb_rows(), t5_11b_block(), gpt175b_block()]
