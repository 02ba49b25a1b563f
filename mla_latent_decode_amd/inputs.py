"""Seeded synthetic inputs for QK-Normed MLA latent decode.

This module only draws random numbers and rounds them to the storage dtype.
It holds none of the method's arithmetic (no norm, no RoPE, no attention), so
both the fp64 oracle and the GPU path can be fed from it.

Shapes and distributions follow the five workloads the decode is measured on:

  0  tiny fp32 check: H=4 query heads in G=2 KV groups, latent rank r=32,
     content head dim d_c=16, RoPE dim d_r=8, V head dim d_v=16, batch 1,
     context 64.
  1  DeepSeek-V3-like layer (H=128, G=8, r=512, d_c=128, d_r=64, d_v=128),
     bf16 caches with an fp32 alpha cache, batch 16, context 4096.
  2  same layer, batch 4, context 32768 (the last token of each sequence is
     appended in the decode step itself).
  3  same layer, batch 1, context 262144.
  4  same layer, batch 64, ragged lengths uniform in [1024, 16384], each latent
     row scaled by 10**clip(N(0,1), -3, 3) to stress the key-RMS range.

Distributions: latents, raw RoPE keys and queries ~ N(0, 1); W^UK and W^UV ~
N(0, 1/r) (fan-in r); all four RMSNorm weights ~ U(0.5, 1.5).  Draw order from
``numpy.random.default_rng(1000 + config_id)``: W^UK, W^UV, gamma_q, gamma_k,
gamma_q_rope, gamma_k_rope, lengths (ragged workloads only), then per sequence
latents, (row scales), raw RoPE keys, then q_c and q_rope.

Values meant for bf16 storage are rounded to bf16 (round to nearest even) here,
on the host, so that the oracle sees exactly the numbers the GPU stores.
"""
from __future__ import annotations

import dataclasses
from typing import Optional, Sequence

import numpy as np


@dataclasses.dataclass(frozen=True)
class Shape:
    n_heads: int      # H, query heads
    n_groups: int     # G, KV groups
    latent_rank: int  # r
    head_dim: int     # d_c, content head dim
    rope_dim: int     # d_r
    v_head_dim: int   # d_v
    dtype: str        # "f32" or "bf16": latent/rope caches, queries, W~, W^UV

    @property
    def heads_per_group(self) -> int:
        return self.n_heads // self.n_groups


TINY = Shape(4, 2, 32, 16, 8, 16, "f32")
DSV3 = Shape(128, 8, 512, 128, 64, 128, "bf16")


@dataclasses.dataclass(frozen=True)
class Workload:
    config_id: int
    name: str
    shape: Shape
    batch: int
    lengths: Optional[tuple]       # fixed lengths, or None when drawn (ragged)
    ragged: Optional[tuple] = None  # (lo, hi) inclusive for drawn lengths
    row_scale_log10_clip: Optional[float] = None
    append_last: bool = False       # last token of each sequence arrives in the step


WORKLOADS = {
    0: Workload(0, "tiny fp32 H4 G2 r32 dc16 dr8 dv16 B1 L64", TINY, 1, (64,)),
    1: Workload(1, "dsv3 layer bf16 B16 L4096", DSV3, 16, (4096,) * 16),
    2: Workload(2, "dsv3 layer bf16 B4 L32768 (+1 appended)", DSV3, 4, (32768,) * 4, append_last=True),
    3: Workload(3, "dsv3 layer bf16 B1 L262144", DSV3, 1, (262144,)),
    4: Workload(4, "dsv3 layer bf16 B64 ragged L~U[1024,16384] log-normal row scales", DSV3, 64, None,
                ragged=(1024, 16384), row_scale_log10_clip=3.0),
}


def round_bf16(x: np.ndarray) -> np.ndarray:
    """Round float32 values to the nearest bf16 (ties to even); returns float32."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    bias = ((u >> np.uint32(16)) & np.uint32(1)) + np.uint32(0x7FFF)
    return ((u + bias) & np.uint32(0xFFFF0000)).view(np.float32)


def _store(x: np.ndarray, dtype: str) -> np.ndarray:
    x = np.asarray(x, dtype=np.float32)
    return round_bf16(x) if dtype == "bf16" else x


@dataclasses.dataclass
class Inputs:
    shape: Shape
    lengths: list            # L_b per sequence
    w_uk: np.ndarray         # [G][r][d_c] float32
    w_uv: np.ndarray         # [G][r][d_v] float32 (bf16-representable for bf16 shapes)
    gamma_q: np.ndarray      # [d_c]
    gamma_k: np.ndarray      # [d_c]
    gamma_q_rope: np.ndarray  # [d_r]
    gamma_k_rope: np.ndarray  # [d_r]
    latents: list            # per sequence [L_b][r] float32 (storage-rounded)
    k_rope_raw: list         # per sequence [L_b][d_r] float32 (storage-rounded), pre-norm pre-RoPE
    q_c: np.ndarray          # [B][H][d_c] (storage-rounded)
    q_rope: np.ndarray       # [B][H][d_r] (storage-rounded), pre-norm pre-RoPE


def make_inputs(shape: Shape, lengths: Sequence[int], seed: int,
                row_scale_log10_clip: Optional[float] = None,
                ragged: Optional[tuple] = None, batch: Optional[int] = None) -> Inputs:
    """Draw one batch of inputs.  With ``ragged=(lo, hi)`` the lengths are drawn
    (``batch`` of them, uniform on [lo, hi]) after the weights."""
    rng = np.random.default_rng(seed)
    s = shape
    G, r, dc, dr, dv, H = s.n_groups, s.latent_rank, s.head_dim, s.rope_dim, s.v_head_dim, s.n_heads
    w_uk = rng.standard_normal((G, r, dc), dtype=np.float32) * np.float32(1.0 / np.sqrt(r))
    w_uv = _store(rng.standard_normal((G, r, dv), dtype=np.float32) * np.float32(1.0 / np.sqrt(r)), s.dtype)
    gamma_q = rng.uniform(0.5, 1.5, dc).astype(np.float32)
    gamma_k = rng.uniform(0.5, 1.5, dc).astype(np.float32)
    gamma_q_rope = rng.uniform(0.5, 1.5, dr).astype(np.float32)
    gamma_k_rope = rng.uniform(0.5, 1.5, dr).astype(np.float32)
    if ragged is not None:
        lengths = [int(x) for x in rng.integers(ragged[0], ragged[1], size=batch, endpoint=True)]
    lengths = [int(x) for x in lengths]
    latents, k_rope_raw = [], []
    for L in lengths:
        c = rng.standard_normal((L, r), dtype=np.float32)
        if row_scale_log10_clip is not None:
            z = np.clip(rng.standard_normal(L), -row_scale_log10_clip, row_scale_log10_clip)
            c = c * (10.0 ** z).astype(np.float32)[:, None]
        latents.append(_store(c, s.dtype))
        k_rope_raw.append(_store(rng.standard_normal((L, dr), dtype=np.float32), s.dtype))
    B = len(lengths)
    q_c = _store(rng.standard_normal((B, H, dc), dtype=np.float32), s.dtype)
    q_rope = _store(rng.standard_normal((B, H, dr), dtype=np.float32), s.dtype)
    return Inputs(s, lengths, w_uk, w_uv, gamma_q, gamma_k, gamma_q_rope, gamma_k_rope,
                  latents, k_rope_raw, q_c, q_rope)


def multi_query_rows(shape: Shape, batch: int, s_q: int, seed: int):
    """s_q query rows per sequence for a multi-query decode step: q_c
    [B][s_q][H][d_c] and q_rope [B][s_q][H][d_r] ~ N(0, 1), storage-rounded,
    drawn from their own seeded generator."""
    rng = np.random.default_rng(seed)
    H, dc, dr = shape.n_heads, shape.head_dim, shape.rope_dim
    q_c = _store(rng.standard_normal((batch, s_q, H, dc), dtype=np.float32), shape.dtype)
    q_rope = _store(rng.standard_normal((batch, s_q, H, dr), dtype=np.float32), shape.dtype)
    return q_c, q_rope


def workload_inputs(config_id: int, seed: Optional[int] = None) -> Inputs:
    w = WORKLOADS[config_id]
    return make_inputs(w.shape, w.lengths or (), 1000 + config_id if seed is None else seed,
                       row_scale_log10_clip=w.row_scale_log10_clip, ragged=w.ragged, batch=w.batch)


def device_cache_fill_source(shape: Shape, lengths, seed: int, device, row_scale_log10_clip=None,
                             chunk: int = 65536):
    """Yield (b or None, start, c_new, k_rope_raw) chunks of N(0,1) latents and raw
    RoPE keys drawn on the GPU (same distributions as make_inputs; not the same
    numbers).  Used by the benchmark, which never compares against the oracle.
    With equal lengths the chunks cover the whole batch (b is None)."""
    import torch
    g = torch.Generator(device=device)
    g.manual_seed(seed)
    dt = torch.bfloat16 if shape.dtype == "bf16" else torch.float32
    r, dr = shape.latent_rank, shape.rope_dim

    def draw(n_seq, n):
        c = torch.randn((n_seq, n, r), generator=g, device=device, dtype=torch.float32)
        if row_scale_log10_clip is not None:
            z = torch.randn((n_seq, n, 1), generator=g, device=device).clamp_(
                -row_scale_log10_clip, row_scale_log10_clip)
            c = c * torch.pow(10.0, z)
        k = torch.randn((n_seq, n, dr), generator=g, device=device, dtype=torch.float32)
        return c.to(dt).contiguous(), k.to(dt).contiguous()

    lengths = list(lengths)
    if len(set(lengths)) == 1:
        for s in range(0, lengths[0], chunk):
            e = min(lengths[0], s + chunk)
            c, k = draw(len(lengths), e - s)
            yield None, s, c, k
    else:
        for b, L in enumerate(lengths):
            for s in range(0, L, chunk):
                e = min(L, s + chunk)
                c, k = draw(1, e - s)
                yield b, s, c, k


def train_inputs(shape: Shape, batch: int, seq_len: int, seed: int) -> dict:
    """Inputs of one training / prefill step over ``batch`` sequences of
    ``seq_len`` tokens, as a dict of float32 arrays (storage-rounded where the
    layer stores them in its dtype): c [B][T][r], q_c [B][T][H][d_c],
    q_rope [B][T][H][d_r], k_rope [B][T][d_r] (raw), w_uk [G][r][d_c] (fp32),
    w_uv [G][r][d_v], the four RMSNorm weights, and the upstream gradient
    d_o [B][T][H][d_v] (fp32).  Same distributions as make_inputs (d_o ~ N(0,1)),
    drawn in that order from default_rng(seed)."""
    rng = np.random.default_rng(seed)
    s = shape
    G, r, dc, dr, dv, H = s.n_groups, s.latent_rank, s.head_dim, s.rope_dim, s.v_head_dim, s.n_heads
    B, T = batch, seq_len
    out = {}
    out["w_uk"] = rng.standard_normal((G, r, dc), dtype=np.float32) * np.float32(1.0 / np.sqrt(r))
    out["w_uv"] = _store(rng.standard_normal((G, r, dv), dtype=np.float32) *
                         np.float32(1.0 / np.sqrt(r)), s.dtype)
    for n, d in (("gamma_q", dc), ("gamma_k", dc), ("gamma_q_rope", dr), ("gamma_k_rope", dr)):
        out[n] = rng.uniform(0.5, 1.5, d).astype(np.float32)
    out["c"] = _store(rng.standard_normal((B, T, r), dtype=np.float32), s.dtype)
    out["k_rope"] = _store(rng.standard_normal((B, T, dr), dtype=np.float32), s.dtype)
    out["q_c"] = _store(rng.standard_normal((B, T, H, dc), dtype=np.float32), s.dtype)
    out["q_rope"] = _store(rng.standard_normal((B, T, H, dr), dtype=np.float32), s.dtype)
    out["d_o"] = rng.standard_normal((B, T, H, dv), dtype=np.float32)
    return out


def train_inputs_varlen(shape: Shape, lengths: Sequence[int], seed: int) -> dict:
    """train_inputs for packed sequences of the given lengths: the per-token
    arrays become [sum(lengths)][...] (sequence s on the rows after those of
    sequences 0..s-1), drawn as one batch of sum(lengths) tokens."""
    total = int(sum(int(L) for L in lengths))
    d = train_inputs(shape, 1, max(total, 1), seed)
    for n in ("c", "q_c", "q_rope", "k_rope", "d_o"):
        d[n] = np.ascontiguousarray(d[n][0, :total])
    return d
