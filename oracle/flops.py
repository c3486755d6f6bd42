"""FLOP counts and MFU arithmetic (fp64 host arithmetic).

Test infrastructure only (see the package docstring).

Source: MegaScale study guide, ch.2 §2.1 (paper §2): MFU is observed
throughput over theoretical peak, and a training step costs about 6N FLOPs per
token for N parameters (2N forward, 4N backward), ignoring the attention term.
The page's worked check on Table 2's last row is reproduced by ``mfu``.
"""
from __future__ import annotations


def model_flops(n_params: float, tokens: float) -> float:
    """6 * N * tokens: forward (2N) plus backward (4N) per token."""
    return 6.0 * n_params * tokens


def mfu(tokens_per_s: float, n_params: float, n_gpus: int, peak_per_gpu: float) -> float:
    """Model FLOPs utilisation: 6N FLOP/token times tokens/s over the summed peak."""
    return model_flops(n_params, tokens_per_s) / (n_gpus * peak_per_gpu)


def dense_params(hidden: int, n_layers: int) -> float:
    """12 h^2 per GPT layer (4h^2 attention + 8h^2 MLP), no embeddings or biases."""
    return 12.0 * hidden * hidden * n_layers


def shard_matrix_params(hidden: int, attn_width: int, ffn: int) -> int:
    """Matrix parameters in one shard of the fused block:
    w_in [3A + F, h] plus w_out [h, A + F]."""
    return (3 * attn_width + ffn) * hidden + hidden * (attn_width + ffn)


def band_pairs(seq: int, window: int) -> int:
    """Number of (query, key) pairs with 0 <= i - j < window in one sequence."""
    w = min(window, seq)
    # rows i < w see i + 1 keys; the other rows see w keys
    return w * (w + 1) // 2 + (seq - w) * w


def attention_flops_fwd(batch: int, seq: int, n_heads: int, head_dim: int, window: int) -> float:
    """Band FLOPs of QK^T and PV: 2 products of 2*d FLOPs per visible pair."""
    return 4.0 * head_dim * band_pairs(seq, window) * batch * n_heads


def attention_flops_bwd(batch: int, seq: int, n_heads: int, head_dim: int, window: int) -> float:
    """Band FLOPs of the four backward products dV, dP, dQ, dK (no recompute)."""
    return 2.0 * attention_flops_fwd(batch, seq, n_heads, head_dim, window)
