"""Byte account of one decode step -- test infrastructure (oracle).

TEST INFRASTRUCTURE ONLY: the product path never imports this module.

Source: "Where Activation Sparsity and KV-Cache Sparsity Cross in LLM
Decoding" (ByteCross), GitHub README page, sections "Overview", "Quick start",
"Usage / The byte account", "The quality-matched crossover" and "Byte
crossover lengths (paper Table 1)".  The pages cite the paper's Equations 1
to 5 without printing them; the forms below are the reading that reproduces
every value the README prints (the pins live in tests/golden/).

Per decode step of one sequence, with e bytes per element (bf16: 2):
  W_proj  = e * L * P_layer,  P_layer = 2 d^2 + 2 d kvd + 3 d d_ff
            (q and o: d x d each; k and v: d x kvd each; gate, up, down:
            d x d_ff each), kvd = n_kv_heads * d / n_heads
  W_head  = e * vocab * d                       (the LM head)
  KV(n)   = e * 2 * L * kvd * n                 (keys and values)
  n*      = (1 - r_p) W_proj / ((1 - r_kv) KV(1))   -- the byte crossover
  bound   = B / (B - dB),  B = W_proj + W_head + KV(n),
            dB = (1 - r_p) W_proj + (1 - r_kv) KV(n)
With ff_only the projection term counts only the three feed-forward matrices.
Nothing here imports numpy or torch.
"""
from __future__ import annotations

from dataclasses import dataclass

BF16_BYTES = 2


@dataclass(frozen=True)
class Model:
    """Decoder dimensions read from a Hugging Face style config
    (README "Quick start": the fields the byte account reads).
    The head dimension is d / n_heads (README FAQ: n_heads * head_dim = d)."""

    n_layers: int
    d: int
    d_ff: int
    vocab: int
    n_heads: int
    n_kv_heads: int
    max_position: int = 131072

    @staticmethod
    def from_config(cfg: dict) -> "Model":
        return Model(
            n_layers=int(cfg["num_hidden_layers"]),
            d=int(cfg["hidden_size"]),
            d_ff=int(cfg["intermediate_size"]),
            vocab=int(cfg["vocab_size"]),
            n_heads=int(cfg["num_attention_heads"]),
            n_kv_heads=int(cfg.get("num_key_value_heads", cfg["num_attention_heads"])),
            max_position=int(cfg.get("max_position_embeddings", 131072)),
        )

    @property
    def head_dim(self) -> int:
        return self.d // self.n_heads

    @property
    def kv_dim(self) -> int:
        return self.n_kv_heads * self.head_dim


LLAMA_31_8B = Model(n_layers=32, d=4096, d_ff=14336, vocab=128256, n_heads=32,
                    n_kv_heads=8, max_position=131072)


def layer_projection_params(m: Model, ff_only: bool = False) -> int:
    """Weights in the seven projections of one layer (or the three FF ones)."""
    ff = 3 * m.d * m.d_ff
    if ff_only:
        return ff
    return 2 * m.d * m.d + 2 * m.d * m.kv_dim + ff


def projection_bytes(m: Model, ff_only: bool = False, e: int = BF16_BYTES) -> int:
    return e * m.n_layers * layer_projection_params(m, ff_only)


def head_bytes(m: Model, e: int = BF16_BYTES) -> int:
    return e * m.vocab * m.d


def kv_bytes(m: Model, n: float, e: int = BF16_BYTES) -> float:
    return e * 2 * m.n_layers * m.kv_dim * n


def crossover(m: Model, rp: float, rkv: float, ff_only: bool = False) -> float:
    """Byte crossover n* in tokens: the context where the projection saving
    (1 - r_p) W_proj equals the KV saving (1 - r_kv) KV(n)."""
    return (1.0 - rp) * projection_bytes(m, ff_only) / ((1.0 - rkv) * kv_bytes(m, 1))


def step_bytes(m: Model, n: float, rp: float = 1.0, rkv: float = 1.0) -> float:
    """Bytes one step reads under the account: r_p W_proj + W_head + r_kv KV(n)."""
    return rp * projection_bytes(m) + head_bytes(m) + rkv * kv_bytes(m, n)


def bound(m: Model, n: float, rp: float = 1.0, rkv: float = 1.0) -> float:
    """Ideal speedup of a purely bandwidth-bound step: B / (B - dB)."""
    b_total = projection_bytes(m) + head_bytes(m) + kv_bytes(m, n)
    saved = (1.0 - rp) * projection_bytes(m) + (1.0 - rkv) * kv_bytes(m, n)
    return b_total / (b_total - saved)


def crossover_batch(m: Model, union_keep: float, rkv: float, batch: int) -> float:
    """Crossover for a batch: projection weights are read once for the union
    keep of the batch, KV bytes are paid per sequence."""
    return (1.0 - union_keep) * projection_bytes(m) / ((1.0 - rkv) * batch * kv_bytes(m, 1))


def _lowest_keep_within(curve: dict, budget: float) -> float:
    """Lowest keep whose linearly interpolated quality loss stays within the
    budget, scanning from keep 1.0 (loss 0) downwards; never below the lowest
    tabulated keep (README "The quality-matched crossover")."""
    pts = [(1.0, 0.0)] + sorted(((float(k), float(v)) for k, v in curve.items() if k < 1.0),
                                reverse=True)
    best = pts[0][0]
    for (k0, v0), (k1, v1) in zip(pts, pts[1:]):
        if v1 <= budget:
            best = k1
            continue
        if v0 <= budget:
            # the loss crosses the budget between k0 (within) and k1 (beyond)
            best = k0 + (k1 - k0) * (budget - v0) / (v1 - v0)
        break
    return best


def matched_crossover(m: Model, proj: dict, sel: dict, budget: float) -> float:
    """n* at the lowest keeps of both branches that meet one quality budget."""
    rp = _lowest_keep_within(proj, budget)
    rkv = _lowest_keep_within(sel, budget)
    return crossover(m, rp, rkv)
