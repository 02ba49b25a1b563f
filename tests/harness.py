"""Test helpers: run the GPU path through the C ABI and compare with the fp64
oracle on the same seeded inputs."""
from __future__ import annotations

import numpy as np

import oracle
from mla_latent_decode_amd.inputs import Inputs

# Tolerances (per (b,h) infinity-norm relative for o and o_lat; elementwise
# relative for alpha; per-row infinity-norm relative for the RoPE cache).
TOL = {
    "f32": {"o": 1e-5, "o_lat": 1e-5, "alpha": 1e-5, "rope": 1e-5, "lse": 1e-5},
    "bf16": {"o": 2e-2, "o_lat": 2e-2, "alpha": 1e-3, "rope": 1e-2, "lse": 5e-2},
}


def oracle_decode(inp: Inputs, cfg, batch_ids=None, groups=None, qk_norm=None):
    return oracle.explicit_decode(
        inp.q_c, inp.q_rope, inp.latents, inp.k_rope_raw, inp.w_uk, inp.w_uv, inp.gamma_q,
        inp.gamma_k, inp.gamma_q_rope, inp.gamma_k_rope, eps=cfg.eps, tau=cfg.tau,
        base=cfg.rope_base, qk_norm=cfg.qk_norm if qk_norm is None else qk_norm,
        batch_ids=batch_ids, groups=groups)


def heads_of(groups, H, G):
    return [h for h in range(H) if (h * G) // H in groups]


def worst_of(x) -> float:
    """Largest value of an error array; NaN (an output the kernel never wrote or
    a non-finite result) counts as infinitely wrong instead of being skipped."""
    x = np.asarray(x, dtype=np.float64)
    return float("inf") if np.isnan(x).any() else float(x.max())


def check_outputs(got_o, got_lat, got_lse, ref, dtype, bs, hs, label="", lse_rel=0.0):
    """lse_rel: for unnormalised logits (plain MLA on scaled latents) the
    log-sum-exp carries the bf16 rounding of q~ (2^-9 relative) of logits as
    large as |lse|, so its bound grows by lse_rel * |lse|."""
    tol = TOL[dtype]
    worst = {}
    for b in bs:
        eo = oracle.rowwise_rel_err(got_o[b, hs], ref["o"][b, hs])
        el = oracle.rowwise_rel_err(got_lat[b, hs], ref["o_lat"][b, hs])
        bound = 1.0 + lse_rel * np.abs(ref["lse"][b, hs]) / tol["lse"]
        else_ = np.abs(got_lse[b, hs] - ref["lse"][b, hs]) / bound
        worst["o"] = max(worst.get("o", 0), worst_of(eo))
        worst["o_lat"] = max(worst.get("o_lat", 0), worst_of(el))
        worst["lse"] = max(worst.get("lse", 0), worst_of(else_))
    print(f"[{label}] worst errors: {worst}", flush=True)
    assert worst["o"] <= tol["o"], (label, worst)
    assert worst["o_lat"] <= tol["o_lat"], (label, worst)
    assert worst["lse"] <= tol["lse"], (label, worst)
    return worst


def check_caches(sess, inp: Inputs, cfg, bs, max_rows=None):
    """alpha and RoPE caches written by qkmla_append vs oracle.append_ref."""
    tol = TOL[cfg.dtype]
    worst_a, worst_r = 0.0, 0.0
    alpha = sess.alpha.float().cpu().numpy() if cfg.qk_norm else None
    rope = sess.rope.float().cpu().numpy()
    for b in bs:
        L = inp.lengths[b]
        rows = np.arange(L) if max_rows is None or L <= max_rows else np.unique(
            np.linspace(0, L - 1, max_rows).astype(np.int64))
        a_ref, r_ref = oracle.append_ref(inp.latents[b][rows], inp.k_rope_raw[b][rows], rows,
                                         inp.w_uk, inp.gamma_k_rope, cfg.eps, cfg.rope_base,
                                         qk_norm=cfg.qk_norm)
        if cfg.qk_norm:
            ea = np.abs(alpha[b, rows] - a_ref) / np.abs(a_ref)
            worst_a = max(worst_a, worst_of(ea))
        er = oracle.rowwise_rel_err(rope[b, rows], r_ref)
        worst_r = max(worst_r, worst_of(er))
    print(f"cache errors: alpha {worst_a:.3e} rope {worst_r:.3e}", flush=True)
    assert worst_a <= tol["alpha"] and worst_r <= tol["rope"], (worst_a, worst_r)
