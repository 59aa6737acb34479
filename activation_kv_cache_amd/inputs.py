"""Seeded synthetic inputs for the decode step.

This module holds only random-number generation and bf16 packing of the
draws; none of the decode step's arithmetic lives here.  Both the HIP path's
tests and the CPU oracle's tests draw their inputs from it.

Recipe: numpy PCG64 seeded by one base seed; every tensor gets its own child
SeedSequence, spawned by name in a fixed order, so a tensor's values do not
depend on which other tensors were drawn.  Values are drawn in float32 and
rounded to bf16 (round to nearest even, via torch's CPU conversion).
"""
from __future__ import annotations

import hashlib

import numpy as np
import torch


def _child_seed(base_seed: int, name: str) -> np.random.SeedSequence:
    tag = int.from_bytes(hashlib.sha256(name.encode()).digest()[:8], "little")
    return np.random.SeedSequence([int(base_seed), tag])


def rng(base_seed: int, name: str) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(_child_seed(base_seed, name)))


def to_bf16_bits(a: np.ndarray) -> np.ndarray:
    t = torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32))
    return t.to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16).copy()


def normal_bf16(base_seed: int, name: str, shape, std: float = 1.0, mean: float = 0.0) -> np.ndarray:
    g = rng(base_seed, name)
    return to_bf16_bits(g.standard_normal(size=shape, dtype=np.float32) * np.float32(std)
                        + np.float32(mean))


def outlier_positions(base_seed: int, name: str, n: int, frac: float = 0.01) -> np.ndarray:
    """Fixed seeded channel positions for the outlier channels:
    floor(frac * n + 1/2) distinct positions, ascending."""
    cnt = int(np.floor(frac * n + 0.5))
    g = rng(base_seed, name + "/outliers")
    return np.sort(g.choice(n, size=cnt, replace=False)).astype(np.int64)


def activation_bf16(base_seed: int, name: str, n: int, outlier_frac: float = 0.01,
                    outlier_scale: float = 10.0) -> np.ndarray:
    """x ~ N(0, 1) with a fixed 1% of channels scaled by 10 (the activation
    branch's input distribution)."""
    g = rng(base_seed, name)
    x = g.standard_normal(size=n, dtype=np.float32)
    if outlier_frac > 0:
        pos = outlier_positions(base_seed, name, n, outlier_frac)
        x[pos] *= np.float32(outlier_scale)
    return to_bf16_bits(x)


def tie_ladder_bf16(n: int, levels: int, base_seed: int = 0, name: str = "ladder") -> np.ndarray:
    """Values drawn from only `levels` distinct magnitudes with random signs,
    so that many channels tie on |x|."""
    g = rng(base_seed, name)
    mags = (np.arange(1, levels + 1, dtype=np.float32) / levels)
    x = mags[g.integers(0, levels, size=n)] * np.where(g.integers(0, 2, size=n) == 1, 1.0, -1.0)
    return to_bf16_bits(x.astype(np.float32))


def layer_weights(base_seed: int, dims: dict, std: float = 0.02, layer: int = 0) -> dict:
    """W^T matrices of one decoder layer ([d_in][d_out] bf16) and unit norm
    gains.  qkv columns are q (H*D) then k (Hkv*D) then v (Hkv*D)."""
    d, H, Hkv, D, dff = dims["d"], dims["n_heads"], dims["n_kv_heads"], dims["head_dim"], dims["d_ff"]
    p = f"layer{layer}/"
    one = to_bf16_bits(np.ones(d, np.float32))
    return {
        "qkv": normal_bf16(base_seed, p + "wqkv", (d, H * D + 2 * Hkv * D), std),
        "o": normal_bf16(base_seed, p + "wo", (H * D, d), std),
        "gate": normal_bf16(base_seed, p + "wgate", (d, dff), std),
        "up": normal_bf16(base_seed, p + "wup", (d, dff), std),
        "down": normal_bf16(base_seed, p + "wdown", (dff, d), std),
        "g1": one.copy(),
        "g2": one.copy(),
    }


def kv_cache(base_seed: int, dims: dict, n_cap: int, std: float, layer: int = 0):
    """K and V [Hkv][n_cap][D] bf16."""
    Hkv, D = dims["n_kv_heads"], dims["head_dim"]
    p = f"layer{layer}/"
    return (normal_bf16(base_seed, p + "kcache", (Hkv, n_cap, D), std),
            normal_bf16(base_seed, p + "vcache", (Hkv, n_cap, D), std))


TINY = dict(d=512, n_heads=8, n_kv_heads=2, head_dim=64, d_ff=1408, vocab=1024, n_layers=1)
LLAMA8B = dict(d=4096, n_heads=32, n_kv_heads=8, head_dim=128, d_ff=14336, vocab=128256,
               n_layers=32)


def device_normal_bf16(base_seed: int, name: str, shape, std: float = 1.0, device="cuda"):
    """Large seeded tensors drawn on the device (torch Philox generator seeded
    from the same per-name child seed); returned as int16-viewed bf16."""
    seed = int(_child_seed(base_seed, name).generate_state(1, dtype=np.uint64)[0] & 0x7FFFFFFFFFFFFFFF)
    g = torch.Generator(device=device)
    g.manual_seed(seed)
    t = torch.empty(shape, dtype=torch.bfloat16, device=device)
    t.normal_(0.0, std, generator=g)
    return t.view(torch.int16)
