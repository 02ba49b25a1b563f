"""fp64 CPU oracle for training and prefill of QK-Normed MLA: the explicit
form, forward and backward.

TEST INFRASTRUCTURE ONLY.  Only the tests, the smoke check and the benchmark's
CPU-baseline leg may import this module.  It shares no code with the HIP path
and imports nothing from it (nor from the decode oracle).

Sources (both pages carry the title "QK-Normed MLA: QK normalization without
full key caching"):
  [TS]  the technical summary, sections Problem Statement, Methodology
        (RMSNorm decomposition, Blockwise Normalization) and Results (the
        400M-parameter models are trained with QK-normed MLA);
  [ABS] the authors' abstract: post-projection QK RMSNorm in MLA.

What is computed: every token of a sequence attends the keys at or before its
own position (causal self-attention, the training and prefill form).  Keys are
materialised, k_{t,g} = c_t W^UK_g, and normalised after the up-projection;
the query content part is normalised with its own gamma; the RoPE parts of
query and key are normalised separately and then rotated ([TS] Methodology,
Blockwise Normalization).  Values are v_{t,g} = c_t W^UV_g.

Readings (the same as the decode oracle's, restated): S(z) = sqrt(mean z^2 +
eps); gamma_q, gamma_k over d_c shared by all heads and groups; gamma_q_rope,
gamma_k_rope over d_r; one RoPE key per token shared by all heads; RoPE turns
interleaved pairs (2i, 2i+1) by p * base**(-2i/d_r) with p the token's
position in its sequence (query and key alike); logit = tau * (content +
rope); head h belongs to group floor(h*G/H).  Plain MLA drops both norms.

The backward is torch autograd of ``train_forward`` (the gradient of the
forward by definition); the tests pin it with central finite differences.

Array conventions: c [B][T][r], q_c [B][T][H][d_c], q_rope [B][T][H][d_r],
k_rope [B][T][d_r] (raw, before norm and rotation), w_uk [G][r][d_c],
w_uv [G][r][d_v].  Outputs o [B][T][H][d_v], lse [B][T][H] (natural log of the
sum of exp of the tau-scaled logits).
"""
from __future__ import annotations

import math
from typing import Dict, Optional

import numpy as np
import torch

D = torch.float64
INPUT_NAMES = ("c", "q_c", "q_rope", "k_rope", "w_uk", "w_uv", "gamma_q", "gamma_k",
               "gamma_q_rope", "gamma_k_rope")


def _t(x) -> torch.Tensor:
    return torch.as_tensor(np.asarray(x, dtype=np.float64), dtype=D)


def _rms(z: torch.Tensor, eps: float) -> torch.Tensor:
    """S(z) over the last axis ([TS] Methodology: RMSNorm decomposition)."""
    return torch.sqrt((z * z).mean(dim=-1, keepdim=True) + eps)


def _rmsnorm(z: torch.Tensor, gamma: torch.Tensor, eps: float) -> torch.Tensor:
    """z * gamma / S(z)."""
    return z * gamma / _rms(z, eps)


def _rope(x: torch.Tensor, pos: torch.Tensor, base: float) -> torch.Tensor:
    """Turn pairs (x_2i, x_2i+1) by pos * base**(-2i/d_r); pos broadcasts
    against x[..., 0]."""
    d = x.shape[-1]
    theta = torch.pow(torch.tensor(base, dtype=D), -2.0 * torch.arange(d // 2, dtype=D) / d)
    ang = pos.to(D).unsqueeze(-1) * theta
    cos, sin = torch.cos(ang), torch.sin(ang)
    x0, x1 = x[..., 0::2], x[..., 1::2]
    return torch.stack((x0 * cos - x1 * sin, x0 * sin + x1 * cos), dim=-1).flatten(-2)


def train_forward(c, q_c, q_rope, k_rope, w_uk, w_uv, gamma_q, gamma_k, gamma_q_rope,
                  gamma_k_rope, *, eps: float = 1e-6, tau: Optional[float] = None,
                  base: float = 10000.0, qk_norm: bool = True):
    """Causal explicit-form attention over whole sequences (torch fp64 tensors
    in, (o, lse) out).  For sequence b, query token i, head h in group g:
      k^_{j,g} = RMSNorm_{gamma_k}(c_j W^UK_g),   q^_{i,h} = RMSNorm_{gamma_q}(q^C_{i,h})
      k^R_j    = RoPE_j(RMSNorm_{gamma_k_rope}(k^R_j)),
      q^R_{i,h} = RoPE_i(RMSNorm_{gamma_q_rope}(q^R_{i,h}))
      l_{i,j}  = tau (q^_{i,h} . k^_{j,g} + q^R_{i,h} . k^R_j)  for j <= i
      o_{i,h}  = sum_{j<=i} softmax_j(l_{i,.}) c_j W^UV_g."""
    B, T, H, dc = q_c.shape
    G = w_uk.shape[0]
    dr = q_rope.shape[-1]
    if tau is None:
        tau = 1.0 / math.sqrt(dc + dr)
    k = torch.einsum("btr,grd->btgd", c, w_uk)          # materialised keys [B][T][G][d_c]
    v = torch.einsum("btr,grd->btgd", c, w_uv)          # values [B][T][G][d_v]
    if qk_norm:
        qh, kh = _rmsnorm(q_c, gamma_q, eps), _rmsnorm(k, gamma_k, eps)
        qr, kr = _rmsnorm(q_rope, gamma_q_rope, eps), _rmsnorm(k_rope, gamma_k_rope, eps)
    else:
        qh, kh, qr, kr = q_c, k, q_rope, k_rope
    pos = torch.arange(T, dtype=D)
    qr = _rope(qr, pos[:, None], base)                 # query token i at position i
    kr = _rope(kr, pos, base)                          # key token j at position j
    gmap = [(h * G) // H for h in range(H)]
    kh_h, v_h = kh[:, :, gmap], v[:, :, gmap]          # per head [B][T][H][.]
    logits = tau * (torch.einsum("bihd,bjhd->bhij", qh, kh_h) +
                    torch.einsum("bihd,bjd->bhij", qr, kr))
    future = torch.triu(torch.ones(T, T, dtype=torch.bool), diagonal=1)  # j > i
    logits = logits.masked_fill(future, float("-inf"))
    lse = torch.logsumexp(logits, dim=-1)              # [B][H][T]
    p = torch.exp(logits - lse.unsqueeze(-1))
    o = torch.einsum("bhij,bjhd->bihd", p, v_h)
    return o, lse.permute(0, 2, 1)


def train_reference(inputs: Dict[str, np.ndarray], d_o: Optional[np.ndarray] = None, **kw):
    """Forward (and, given d_o [B][T][H][d_v], the backward of the loss
    sum(o * d_o)) as float64 numpy arrays.  Returns {"o", "lse"} plus
    {"d_" + name} for every input in INPUT_NAMES."""
    ts = {n: _t(inputs[n]).requires_grad_(d_o is not None) for n in INPUT_NAMES}
    o, lse = train_forward(*(ts[n] for n in INPUT_NAMES), **kw)
    out = {"o": o.detach().numpy(), "lse": lse.detach().numpy()}
    if d_o is not None:
        grads = torch.autograd.grad((o * _t(d_o)).sum(), [ts[n] for n in INPUT_NAMES],
                                    allow_unused=True)
        for n, g in zip(INPUT_NAMES, grads):
            out["d_" + n] = (np.zeros(ts[n].shape) if g is None else g.numpy())
    return out


def train_reference_varlen(inputs: Dict[str, np.ndarray], lengths, d_o: Optional[np.ndarray] = None,
                           **kw):
    """Packed sequences: the per-token arrays are [total][...] with sequence s
    on rows sum(lengths[:s]) .. + lengths[s] - 1, each token at its position
    in its own sequence.  Each sequence is ``train_reference`` on its rows
    (batch 1); the loss is the sum over sequences, so the per-token gradients
    are those of each sequence and the weight gradients their sums.
    Returns the same keys as ``train_reference``, per-token arrays packed."""
    per_tok = ("c", "q_c", "q_rope", "k_rope")
    weights = [n for n in INPUT_NAMES if n not in per_tok]
    total = sum(int(L) for L in lengths)
    first = inputs["q_c"]
    H, dv = first.shape[1], inputs["w_uv"].shape[-1]
    out = {"o": np.zeros((total, H, dv)), "lse": np.zeros((total, H))}
    if d_o is not None:
        for n in INPUT_NAMES:
            out["d_" + n] = np.zeros(np.shape(inputs[n]))
    row = 0
    for L in lengths:
        L = int(L)
        if L == 0:
            continue
        seq = {n: inputs[n][row:row + L][None] for n in per_tok}
        seq.update({n: inputs[n] for n in weights})
        r = train_reference(seq, None if d_o is None else d_o[row:row + L][None], **kw)
        out["o"][row:row + L] = r["o"][0]
        out["lse"][row:row + L] = r["lse"][0]
        if d_o is not None:
            for n in per_tok:
                out["d_" + n][row:row + L] = r["d_" + n][0]
            for n in weights:
                out["d_" + n] += r["d_" + n]
        row += L
    return out
