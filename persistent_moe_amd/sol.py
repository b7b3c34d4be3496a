"""Speed-of-light byte accounting of one decode step.

The bound the persistent decode megakernel pages use ("Why decode leaves the
GPU idle" on page 1; "Where the bandwidth actually goes" on page 3): one step
must read every active weight once plus the KV cache of every visible key, so
its time is at least those bytes over the HBM bandwidth.  Here the bytes are
counted from the actual shapes, the routed experts and the live lengths:

* weights: the embedding rows of the fed tokens, every norm gain, QKV and O
  projections, the router, each *distinct* routed expert of the step (gate,
  up and down: one byte per weight plus a float32 scale per row when they
  are stored as FP8), or the dense FFN, and the LM head;
* KV: for every sequence and layer, K and V of every key it attends to,
  including the token being decoded.
"""
from __future__ import annotations

from typing import Iterable, Sequence

HBM_BYTES_PER_S_MI355X = 8.0e12
BF16 = 2
FP8 = 1
F32 = 4


def layer_weight_bytes(cfg, distinct_experts: int) -> int:
    d = cfg.d_model
    b = d * BF16                                   # attention (or shared) norm gain
    b += cfg.qkv_rows * d * BF16
    b += d * cfg.attn_dim * BF16
    if cfg.is_moe:
        b += cfg.n_experts * d * BF16              # router
        if getattr(cfg, "expert_fp8", False):
            # codes, then one scale per row: 2I gate/up rows and d down rows
            b += distinct_experts * (3 * cfg.expert_inter * d * FP8 + (2 * cfg.expert_inter + d) * F32)
        else:
            b += distinct_experts * 3 * cfg.expert_inter * d * BF16
    else:
        b += d * BF16                              # second norm gain
        b += 3 * cfg.ffn_inter * d * BF16
    return b


def weight_bytes(cfg, batch: int, distinct_experts_per_layer: Sequence[int]) -> int:
    """Active weight bytes of one step; ``distinct_experts_per_layer`` has one
    entry per layer (ignored for dense models)."""
    b = batch * cfg.d_model * BF16                 # embedding rows
    for l in range(cfg.n_layers):
        ne = distinct_experts_per_layer[l] if cfg.is_moe else 0
        b += layer_weight_bytes(cfg, ne)
    b += cfg.d_model * BF16                        # final norm gain
    b += cfg.vocab * cfg.d_model * BF16            # LM head (tied or not, it is read)
    return b


def visible_keys(cfg, layer: int, pos: int) -> int:
    """Keys a token at position ``pos`` attends to at ``layer`` (incl. itself)."""
    w = cfg.layer_window(layer)
    return min(pos + 1, w) if w > 0 else pos + 1


def kv_bytes(cfg, positions: Iterable[int]) -> int:
    """KV bytes read in one step by tokens at ``positions`` (one per sequence)."""
    per_key = 2 * cfg.n_kv_heads * cfg.head_dim * BF16
    return sum(visible_keys(cfg, l, p) * per_key for p in positions for l in range(cfg.n_layers))


def step_bytes(cfg, positions: Sequence[int], distinct_experts_per_layer: Sequence[int]) -> int:
    return weight_bytes(cfg, len(positions), distinct_experts_per_layer) + kv_bytes(cfg, positions)


def sol_step_seconds(nbytes: float, bw: float = HBM_BYTES_PER_S_MI355X) -> float:
    return nbytes / bw


def sol_tok_s(nbytes: float, batch: int, bw: float = HBM_BYTES_PER_S_MI355X) -> float:
    return batch / sol_step_seconds(nbytes, bw)
