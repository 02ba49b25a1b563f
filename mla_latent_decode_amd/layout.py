"""Cache layout sizes of the QK-Normed MLA decode library (host-side arithmetic).

Per token and sequence the library keeps three rows: the latent c_t (r
elements), the normalised, rotated RoPE key (d_r elements), both in the storage
dtype, and -- only with QK norm -- one float32 inverse-RMS scalar per KV group
(the scalar cache of the technical summary's Cache Layout paragraph)."""
from __future__ import annotations


def elem_bytes(dtype: str) -> int:
    return {"f32": 4, "bf16": 2}[dtype]


def cache_bytes_per_token(shape, qk_norm: bool = True) -> int:
    """Bytes of latent + RoPE (+ alpha) cache per cached token."""
    e = elem_bytes(shape.dtype)
    b = e * (shape.latent_rank + shape.rope_dim)
    if qk_norm:
        b += 4 * shape.n_groups
    return b


def decode_flops_per_token(shape) -> int:
    """Algorithmic MFMA work per cached token in one decode step: the logit
    contraction over latent + RoPE dims and the P.C accumulation, all heads."""
    H, r, dr = shape.n_heads, shape.latent_rank, shape.rope_dim
    return 2 * H * (r + dr) + 2 * H * r


def train_attention_flops(shape, batch: int, seq_len: int) -> tuple:
    """Algorithmic attention FLOPs of one causal training step (forward,
    backward): every head scores T(T+1)/2 (query, key) pairs.  Forward per
    pair: the logit over d_c + d_r and the value sum over d_v.  Backward per
    pair: the recomputed logit, d_o . V, dV, dK^ and dQ^."""
    pairs = batch * shape.n_heads * seq_len * (seq_len + 1) // 2
    dqk, dv = shape.head_dim + shape.rope_dim, shape.v_head_dim
    return 2 * pairs * (dqk + dv), 2 * pairs * (3 * dqk + 2 * dv)


def append_bytes_per_token(shape, qk_norm: bool = True) -> int:
    """Bytes one appended token moves: new latent and raw RoPE key read, the
    three cache rows written."""
    e = elem_bytes(shape.dtype)
    return e * (shape.latent_rank + shape.rope_dim) + cache_bytes_per_token(shape, qk_norm)
