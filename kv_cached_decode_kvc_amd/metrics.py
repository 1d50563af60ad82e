"""Algorithmic byte and FLOP counts of the decode-attention step.

KV size per token ("Inference-1", brunomaga.github.io, section "KV cache";
"Inference o quy mo lon", truongducdung.dev, section 03 "KV cache: toan bo
nho"): 2 (keys and values) x layers x KV heads x head size x bytes per value.
A decode step reads every attended key and value row of every KV head once,
whatever the number of query heads sharing it ("Efficient Inference",
learn.obvix.io, GQA passage: the grouped heads are never materialised).
"""
from __future__ import annotations

import numpy as np


def kv_bytes_per_token(n_layers: int, n_kv_heads: int, head_dim: int, bytes_per_value: int) -> int:
    return 2 * n_layers * n_kv_heads * head_dim * bytes_per_value


def kv_cache_bytes(n_layers, n_kv_heads, head_dim, bytes_per_value, seq_len, batch=1) -> int:
    return kv_bytes_per_token(n_layers, n_kv_heads, head_dim, bytes_per_value) * seq_len * batch


def attended_kv_bytes(seq_lens, n_kv_heads: int, head_dim: int, bytes_per_value: int) -> int:
    """K and V bytes one attention call reads: every attended row of every KV head once."""
    return int(np.asarray(seq_lens, dtype=np.int64).sum()) * kv_bytes_per_token(
        1, n_kv_heads, head_dim, bytes_per_value)


def attended_cache_bytes(seq_lens, n_kv_heads: int, row_bytes: int, tensors: int = 2) -> int:
    """Cache bytes one attention call reads, for any cache format: every
    attended row (token, KV head) of each cache tensor once, `row_bytes` each
    (FP8: codes plus the row's scale).  tensors = 2 for K and V, 1 for an MLA
    latent cache whose rows serve as both."""
    return int(np.asarray(seq_lens, dtype=np.int64).sum()) * n_kv_heads * tensors * row_bytes


def attention_flops(seq_lens, n_q: int, n_q_heads: int, head_dim: int) -> int:
    """2*D for q.k plus 2*D for p*v per visible (query row, key) pair; row r of n_q sees
    L - n_q + r + 1 keys."""
    L = np.asarray(seq_lens, dtype=np.int64)
    visible = (L[:, None] - n_q + np.arange(n_q)[None, :] + 1).sum()
    return int(visible) * n_q_heads * 4 * head_dim
