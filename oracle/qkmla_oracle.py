"""fp64 CPU oracle for QK-Normed MLA latent decode.

TEST INFRASTRUCTURE ONLY.  Only the tests, the smoke check and the benchmark's
CPU-baseline leg may import this module.  It shares no code with the HIP path
and imports nothing from it.

Sources (both pages carry the title "QK-Normed MLA: QK normalization without
full key caching"):
  [TS]  the technical summary on gist.science/paper/2606.16310, sections
        Problem Statement, Methodology, Key Contributions, Results;
  [ABS] the authors' abstract (thelatestinai.com/papers/2606.16310 and
        searcharxiv.com/abs/2606.16310).

What is computed, in the pages' notation:
  * RMSNorm(z) = z * gamma / S(z), with gamma a static weight and S(z) the
    dynamic RMS of z ([TS] Methodology, RMSNorm decomposition).
  * MLA caches a latent c_t per token; a KV group g recovers its key by the
    up-projection k_{t,g} = c_t W^K_g ([TS] Problem Statement).
  * Post-projection QK RMSNorm normalises the projected query and key before
    the dot product ([TS] Problem Statement; [ABS]).
  * Content and RoPE parts are normalised separately; the RoPE part uses
    materialised vectors ([TS] Methodology, Blockwise Normalization).
  * Absorbed form: gamma_k (and gamma_q) fold into the query-side projection,
    the key statistic becomes alpha_{t,g} = 1/S_{t,g}, and the logit is
    (q~ . c_t) alpha^q alpha^k ([TS] Methodology, Static Weight Absorption,
    Dynamic Scalar Caching and the decode-logit formula).  [ABS] states that
    this form equals the explicit one in exact arithmetic; ``absorbed_decode``
    is the independent check of that claim.

Readings where the pages are silent (shared with the GPU path by specification
only, never by code):
  * S(z) = sqrt(mean(z^2) + eps): eps inside the square root.
  * gamma_q, gamma_k are vectors over d_c shared by all heads/groups; the RoPE
    part has its own gamma_q_rope, gamma_k_rope over d_r.
  * One RoPE key per token, shared by all heads; normalised, then rotated.
  * RoPE rotates interleaved pairs (2i, 2i+1) by angle p * base**(-2i/d_r);
    the key at cache row t has position t, the query position L_b - 1.
  * Logit = tau * (content + rope), tau = 1/sqrt(d_c + d_r) by default; the
    alpha factors scale only the content term.
  * Head h belongs to group g(h) = floor(h * G / H); W^UV is per group.
  * Plain MLA (the overhead baseline) is the same computation with both
    normalisations removed.

Array conventions: w_uk [G][r][d_c], w_uv [G][r][d_v], latents / raw RoPE keys
are per-sequence arrays [L_b][r] / [L_b][d_r], q_c [B][H][d_c],
q_rope [B][H][d_r].  All arithmetic is float64.
"""
from __future__ import annotations

import math
from typing import Iterable, Optional, Sequence

import numpy as np

F64 = np.float64


def default_tau(head_dim: int, rope_dim: int) -> float:
    """Softmax scale used when none is given: 1/sqrt(d_c + d_r)."""
    return 1.0 / math.sqrt(head_dim + rope_dim)


def rms(z: np.ndarray, eps: float) -> np.ndarray:
    """S(z) over the last axis ([TS] Methodology: the dynamic scalar statistic)."""
    z = np.asarray(z, dtype=F64)
    return np.sqrt(np.mean(z * z, axis=-1, keepdims=True) + eps)


def rmsnorm(z: np.ndarray, gamma: np.ndarray, eps: float) -> np.ndarray:
    """z * gamma / S(z) ([TS] Methodology: RMSNorm decomposition)."""
    z = np.asarray(z, dtype=F64)
    return z * np.asarray(gamma, dtype=F64) / rms(z, eps)


def rope_inv_freq(rope_dim: int, base: float) -> np.ndarray:
    """theta_i = base**(-2i/d_r) for i < d_r/2."""
    i = np.arange(rope_dim // 2, dtype=F64)
    return np.power(F64(base), -2.0 * i / rope_dim)


def rope(x: np.ndarray, pos, base: float) -> np.ndarray:
    """Rotate interleaved pairs (x_2i, x_2i+1) by pos * theta_i.

    ``x`` is [..., d_r]; ``pos`` broadcasts against x[..., 0]."""
    x = np.asarray(x, dtype=F64)
    d = x.shape[-1]
    ang = np.asarray(pos, dtype=F64)[..., None] * rope_inv_freq(d, base)
    cos, sin = np.cos(ang), np.sin(ang)
    x0, x1 = x[..., 0::2], x[..., 1::2]
    out = np.empty_like(x)
    out[..., 0::2] = x0 * cos - x1 * sin
    out[..., 1::2] = x0 * sin + x1 * cos
    return out


def group_of_head(h: int, n_heads: int, n_groups: int) -> int:
    return (h * n_groups) // n_heads


def _softmax(logits: np.ndarray):
    """Exact two-pass softmax over the last axis; also returns log-sum-exp."""
    m = np.max(logits, axis=-1, keepdims=True)
    e = np.exp(logits - m)
    s = np.sum(e, axis=-1, keepdims=True)
    return e / s, (m + np.log(s))[..., 0]


# ---------------------------------------------------------------------------
# Append: the per-token state written next to the latent cache.
# ---------------------------------------------------------------------------

def append_ref(latent: np.ndarray, k_rope_raw: np.ndarray, positions: np.ndarray,
               w_uk: np.ndarray, gamma_k_rope: np.ndarray, eps: float, base: float,
               qk_norm: bool = True):
    """alpha^k and the stored RoPE key for new tokens.

    latent [n][r], k_rope_raw [n][d_r], positions [n] (cache rows).
    Returns (alpha [n][G] or None, k_rope_hat [n][d_r]).

    alpha_{t,g} = 1/S(c_t W^K_g) is the one inverse-RMS scalar per token and
    KV group that the method caches ([TS] Methodology, Dynamic Scalar Caching
    and Cache Layout).  The RoPE key is normalised on its own and then rotated
    ([TS] Methodology, Blockwise Normalization)."""
    c = np.asarray(latent, dtype=F64)
    kr = np.asarray(k_rope_raw, dtype=F64)
    pos = np.asarray(positions, dtype=F64)
    if qk_norm:
        alpha = np.empty((c.shape[0], w_uk.shape[0]), dtype=F64)
        for g in range(w_uk.shape[0]):
            k = c @ np.asarray(w_uk[g], dtype=F64)          # [n][d_c]
            alpha[:, g] = 1.0 / rms(k, eps)[:, 0]
        return alpha, rope(rmsnorm(kr, gamma_k_rope, eps), pos, base)
    return None, rope(kr, pos, base)


# ---------------------------------------------------------------------------
# Explicit form: the oracle's answer.
# ---------------------------------------------------------------------------

def _group_logits(q_hat, qr_hat, c, k_rope_hat, w_uk_g, gamma_k, eps, tau, qk_norm, chunk):
    """tau (q^_h . k^_{t,g} + q^R_h . k^R_t) for the heads of one group over
    every token t of one sequence, the keys materialised chunk by chunk
    ([TS] Problem Statement: k_{t,g} = c_t W^K_g, normalised after the
    up-projection).  Returns [heads][L]."""
    L = c.shape[0]
    logits = np.empty((q_hat.shape[0], L))
    wk = np.asarray(w_uk_g, dtype=F64)
    for t0 in range(0, L, chunk):
        t1 = min(L, t0 + chunk)
        k = c[t0:t1] @ wk                                 # materialised keys [n][d_c]
        k_hat = rmsnorm(k, gamma_k, eps) if qk_norm else k
        logits[:, t0:t1] = tau * (q_hat @ k_hat.T + qr_hat @ k_rope_hat[t0:t1].T)
    return logits


def _rope_keys(k_rope_raw_b, gamma_k_rope, eps, base, qk_norm):
    """Stored RoPE keys of one sequence: RMS-normalised with gamma_k_rope (QK
    norm only), then rotated by their cache row ([TS] Methodology, Blockwise
    Normalization)."""
    kr = np.asarray(k_rope_raw_b, dtype=F64)
    pos = np.arange(kr.shape[0], dtype=F64)
    if qk_norm:
        return rope(rmsnorm(kr, gamma_k_rope, eps), pos, base)
    return rope(kr, pos, base)


def _queries(qc, qr, L, gamma_q, gamma_q_rope, eps, base, qk_norm):
    """Content and RoPE queries of some heads of one sequence of length L:
    RMS-normalised (QK norm only); the RoPE query is rotated to position L-1."""
    if qk_norm:
        q_hat = rmsnorm(qc, gamma_q, eps)
        qr_hat = rope(rmsnorm(qr, gamma_q_rope, eps), L - 1, base)
    else:
        q_hat = qc
        qr_hat = rope(qr, L - 1, base)
    return q_hat, qr_hat


def explicit_logits(q_c, q_rope, latent, k_rope_raw, w_uk, gamma_q, gamma_k, gamma_q_rope,
                    gamma_k_rope, b: int, g: int, *, eps: float = 1e-6,
                    tau: Optional[float] = None, base: float = 10000.0, qk_norm: bool = True,
                    chunk: int = 65536):
    """The natural-log logits l_{h,t} that ``explicit_decode`` feeds its
    softmax, for the heads of group g of sequence b: [H/G][L_b].  latent and
    k_rope_raw are that sequence's [L_b][r] and [L_b][d_r] arrays."""
    q_c = np.asarray(q_c, dtype=F64)
    q_rope = np.asarray(q_rope, dtype=F64)
    _, H, dc = q_c.shape
    G = w_uk.shape[0]
    dr = q_rope.shape[-1]
    if tau is None:
        tau = default_tau(dc, dr)
    c = np.asarray(latent, dtype=F64)
    heads = [h for h in range(H) if group_of_head(h, H, G) == g]
    k_rope_hat = _rope_keys(k_rope_raw, gamma_k_rope, eps, base, qk_norm)
    q_hat, qr_hat = _queries(q_c[b, heads], q_rope[b, heads], c.shape[0], gamma_q, gamma_q_rope,
                             eps, base, qk_norm)
    return _group_logits(q_hat, qr_hat, c, k_rope_hat, w_uk[g], gamma_k, eps, tau, qk_norm, chunk)


def explicit_decode(q_c, q_rope, latents: Sequence[np.ndarray], k_rope_raw: Sequence[np.ndarray],
                    w_uk, w_uv, gamma_q, gamma_k, gamma_q_rope, gamma_k_rope, *,
                    eps: float = 1e-6, tau: Optional[float] = None, base: float = 10000.0,
                    qk_norm: bool = True, batch_ids: Optional[Iterable[int]] = None,
                    groups: Optional[Iterable[int]] = None, chunk: int = 65536):
    """Decode step computed the explicit way: materialise every key, RMSNorm it.

    For each sequence b, group g and head h in g:
      k_{t,g}   = c_t W^UK_g                      (materialised, fp64)
      k^_{t,g}  = RMSNorm_{gamma_k}(k_{t,g});  q^_h = RMSNorm_{gamma_q}(q^C_h)
      k^R_t     = RoPE_t(RMSNorm_{gamma_k_rope}(raw k^R_t))
      q^R_h     = RoPE_{L_b-1}(RMSNorm_{gamma_q_rope}(q^R_h))
      l_{h,t}   = tau (q^_h . k^_{t,g} + q^R_h . k^R_t)
      p         = softmax_t(l)
      o_h       = sum_t p_{h,t} c_t W^UV_g,   o_lat_h = sum_t p_{h,t} c_t
    With qk_norm=False both normalisations are dropped (plain MLA).

    Only the sequences in ``batch_ids`` and the groups in ``groups`` are
    computed (default: all); other rows of the outputs are NaN.
    Returns dict with o [B][H][d_v], o_lat [B][H][r], lse [B][H] (natural log,
    of the tau-scaled logits)."""
    q_c = np.asarray(q_c, dtype=F64)
    q_rope = np.asarray(q_rope, dtype=F64)
    B, H, dc = q_c.shape
    G, r, dv = w_uv.shape
    dr = q_rope.shape[-1]
    if tau is None:
        tau = default_tau(dc, dr)
    hpg = H // G
    o = np.full((B, H, dv), np.nan)
    o_lat = np.full((B, H, r), np.nan)
    lse = np.full((B, H), np.nan)
    bs = range(B) if batch_ids is None else list(batch_ids)
    gs = range(G) if groups is None else list(groups)
    for b in bs:
        c = np.asarray(latents[b], dtype=F64)
        L = c.shape[0]
        if L == 0:
            continue
        k_rope_hat = _rope_keys(k_rope_raw[b], gamma_k_rope, eps, base, qk_norm)
        for g in gs:
            heads = [h for h in range(H) if group_of_head(h, H, G) == g]
            q_hat, qr_hat = _queries(q_c[b, heads], q_rope[b, heads], L, gamma_q, gamma_q_rope,
                                     eps, base, qk_norm)
            logits = _group_logits(q_hat, qr_hat, c, k_rope_hat, w_uk[g], gamma_k, eps, tau,
                                   qk_norm, chunk)
            p, lse_g = _softmax(logits)
            v_lat = p @ c                                     # [hpg][r]
            o_lat[b, heads] = v_lat
            # value side: v_{t,g} = c_t W^UV_g, o_h = sum_t p v_t (linear in c)
            o[b, heads] = v_lat @ np.asarray(w_uv[g], dtype=F64)
            lse[b, heads] = lse_g
        del c
    assert hpg * G == H
    return {"o": o, "o_lat": o_lat, "lse": lse}


def explicit_decode_multi(q_c, q_rope, latents: Sequence[np.ndarray],
                          k_rope_raw: Sequence[np.ndarray], w_uk, w_uv, gamma_q, gamma_k,
                          gamma_q_rope, gamma_k_rope, **kw):
    """Decode of s_q query rows per sequence (multi-token prediction or
    speculative verification), each causal over the cache.

    q_c [B][s_q][H][d_c], q_rope [B][s_q][H][d_r]; latents[b] holds L_b rows,
    the last s_q of them belonging to the s_q new tokens.  Query row i is the
    token at position P_i = L_b - s_q + i: it attends cache rows 0..P_i and
    its RoPE query is rotated by P_i.  That is an ordinary decode step over
    the causal prefix, so each row is ``explicit_decode`` on rows [0, P_i]
    ([TS] Methodology: the decode logit carries a query index i).
    Returns o [B][s_q][H][d_v], o_lat [B][s_q][H][r], lse [B][s_q][H]."""
    q_c = np.asarray(q_c, dtype=F64)
    q_rope = np.asarray(q_rope, dtype=F64)
    B, s_q = q_c.shape[:2]
    out = None
    bs = kw.pop("batch_ids", None)
    bs = range(B) if bs is None else list(bs)
    for i in range(s_q):
        prefix_lat, prefix_kr = [], []
        for b in range(B):
            P_i = len(latents[b]) - s_q + i
            keep = max(P_i + 1, 0)
            prefix_lat.append(np.asarray(latents[b])[:keep])
            prefix_kr.append(np.asarray(k_rope_raw[b])[:keep])
        res = explicit_decode(q_c[:, i], q_rope[:, i], prefix_lat, prefix_kr, w_uk, w_uv,
                              gamma_q, gamma_k, gamma_q_rope, gamma_k_rope, batch_ids=bs, **kw)
        if out is None:
            out = {k: np.full((B, s_q) + v.shape[1:], np.nan) for k, v in res.items()}
        for k, v in res.items():
            out[k][:, i] = v
    return out


def plain_mla_decode(*args, **kwargs):
    """Plain MLA decode (no QK normalisation): the overhead baseline."""
    kwargs["qk_norm"] = False
    return explicit_decode(*args, **kwargs)


# ---------------------------------------------------------------------------
# Absorbed form: brute-force self-check of the exact-equivalence claim.
# ---------------------------------------------------------------------------

def absorb_weights_ref(w_uk, gamma_q, gamma_k):
    """W~_g = diag(gamma_q * gamma_k) (W^UK_g)^T, shape [G][d_c][r]
    ([TS] Methodology, Static Weight Absorption)."""
    w = np.asarray(w_uk, dtype=F64)
    gg = np.asarray(gamma_q, dtype=F64) * np.asarray(gamma_k, dtype=F64)
    return np.stack([np.diag(gg) @ w[g].T for g in range(w.shape[0])])


def absorbed_decode(q_c, q_rope, latents, k_rope_raw, w_uk, w_uv, gamma_q, gamma_k,
                    gamma_q_rope, gamma_k_rope, *, eps: float = 1e-6,
                    tau: Optional[float] = None, base: float = 10000.0):
    """Decode step in the absorbed form, looping over sequences and heads.

      q~_h    = q^C_h W~_g,  alpha^q_h = 1/S(q^C_h)
      alpha^k = 1/S(c_t W^UK_g)
      l_{h,t} = tau (alpha^q_h alpha^k_{t,g} (q~_h . c_t) + q^R_h . k^R_t)
      o^lat_h = sum_t p_{h,t} c_t,   o_h = o^lat_h W^UV_g
    ([TS] Methodology: decode-logit formula and row-column scaling.)"""
    q_c = np.asarray(q_c, dtype=F64)
    q_rope = np.asarray(q_rope, dtype=F64)
    B, H, dc = q_c.shape
    G = w_uk.shape[0]
    dr = q_rope.shape[-1]
    if tau is None:
        tau = default_tau(dc, dr)
    w_abs = absorb_weights_ref(w_uk, gamma_q, gamma_k)
    out_o = np.zeros((B, H, w_uv.shape[2]))
    out_lat = np.zeros((B, H, w_uk.shape[1]))
    for b in range(B):
        c = np.asarray(latents[b], dtype=F64)
        L = c.shape[0]
        alpha_k, kr_hat = append_ref(c, k_rope_raw[b], np.arange(L), w_uk, gamma_k_rope, eps, base)
        for h in range(H):
            g = group_of_head(h, H, G)
            q_tilde = q_c[b, h] @ w_abs[g]                    # [r]
            alpha_q = 1.0 / math.sqrt(float(np.mean(q_c[b, h] ** 2)) + eps)
            qr_hat = rope(rmsnorm(q_rope[b, h], gamma_q_rope, eps), L - 1, base)
            logit = tau * (alpha_q * alpha_k[:, g] * (c @ q_tilde) + kr_hat @ qr_hat)
            p = np.exp(logit - logit.max())
            p /= p.sum()
            out_lat[b, h] = p @ c
            out_o[b, h] = out_lat[b, h] @ np.asarray(w_uv[g], dtype=F64)
    return {"o": out_o, "o_lat": out_lat}


# ---------------------------------------------------------------------------
# Output comparison helpers used by the parity tests.
# ---------------------------------------------------------------------------

def rowwise_rel_err(x, ref) -> np.ndarray:
    """Per-row infinity-norm relative error over the last axis."""
    x = np.asarray(x, dtype=F64)
    ref = np.asarray(ref, dtype=F64)
    num = np.max(np.abs(x - ref), axis=-1)
    den = np.max(np.abs(ref), axis=-1)
    return num / np.where(den == 0, 1.0, den)
