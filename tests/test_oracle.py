"""Pins for the fp64 oracle: each test ties it to something other than itself
(the pages' exact-equivalence claim and printed cache figures, library
routines, closed forms and invariants)."""
import json
import math
import os

import numpy as np
import pytest
import scipy.special
import torch
import torch.nn.functional as F

from oracle import (absorb_weights_ref, absorbed_decode, append_ref, default_tau,
                    explicit_decode, explicit_decode_multi, explicit_logits, group_of_head,
                    plain_mla_decode, rms, rmsnorm, rope, rope_inv_freq)
from oracle.qkmla_oracle import _softmax
from mla_latent_decode_amd.inputs import (DSV3, TINY, Shape, make_inputs, multi_query_rows,
                                          workload_inputs)

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _decode_args(inp):
    return (inp.q_c, inp.q_rope, inp.latents, inp.k_rope_raw, inp.w_uk, inp.w_uv,
            inp.gamma_q, inp.gamma_k, inp.gamma_q_rope, inp.gamma_k_rope)


def _rel(a, b):
    return float(np.max(np.abs(a - b)) / max(np.max(np.abs(b)), 1e-300))


# --- the pages' claim: absorbed == explicit in exact arithmetic --------------

TINY_SHAPES = [
    # (H, G, r, d_c, d_r, d_v, lengths)
    (4, 2, 32, 16, 8, 16, (64,)),
    (4, 4, 32, 16, 8, 16, (7, 1)),       # G = H
    (4, 1, 32, 16, 8, 16, (5, 13)),      # G = 1
    (6, 3, 20, 12, 4, 10, (9,)),
    (8, 2, 24, 8, 6, 12, (1, 2, 3)),
    (2, 1, 16, 32, 2, 8, (17,)),         # d_c > r
    (16, 8, 64, 16, 8, 16, (33, 31)),
    (3, 3, 10, 6, 4, 5, (11,)),
]


@pytest.mark.parametrize("case", range(len(TINY_SHAPES) + 12))
def test_absorbed_equals_explicit(case):
    rng = np.random.default_rng(case)
    if case < len(TINY_SHAPES):
        H, G, r, dc, dr, dv, lens = TINY_SHAPES[case]
    else:
        G = int(rng.integers(1, 4))
        H = G * int(rng.integers(1, 4))
        r = int(rng.integers(4, 40))
        dc = int(rng.integers(2, 20))
        dr = 2 * int(rng.integers(1, 5))
        dv = int(rng.integers(1, 12))
        lens = tuple(int(x) for x in rng.integers(1, 40, size=int(rng.integers(1, 3))))
    inp = make_inputs(Shape(H, G, r, dc, dr, dv, "f32"), lens, seed=100 + case)
    for eps in (1e-6, 0.0, 0.3):
        ex = explicit_decode(*_decode_args(inp), eps=eps)
        ab = absorbed_decode(*_decode_args(inp), eps=eps)
        assert _rel(ab["o"], ex["o"]) < 1e-12
        assert _rel(ab["o_lat"], ex["o_lat"]) < 1e-12


def test_absorbed_equals_explicit_config0():
    inp = workload_inputs(0)
    ex = explicit_decode(*_decode_args(inp))
    ab = absorbed_decode(*_decode_args(inp))
    assert _rel(ab["o"], ex["o"]) < 1e-12


# --- library special cases ---------------------------------------------------

def test_rmsnorm_matches_torch_rms_norm():
    rng = np.random.default_rng(1)
    for d, eps in ((16, 1e-6), (128, 1e-6), (64, 0.5), (7, 0.0)):
        z = rng.standard_normal((5, d)) * rng.uniform(0.01, 100, (5, 1))
        g = rng.uniform(0.5, 1.5, d)
        ref = F.rms_norm(torch.from_numpy(z), (d,), weight=torch.from_numpy(g), eps=eps).numpy()
        assert _rel(rmsnorm(z, g, eps), ref) < 1e-14


def test_softmax_matches_scipy():
    rng = np.random.default_rng(2)
    x = rng.standard_normal((3, 1000)) * 30
    p, lse = _softmax(x)
    assert _rel(p, scipy.special.softmax(x, axis=-1)) < 1e-13
    assert _rel(lse, scipy.special.logsumexp(x, axis=-1)) < 1e-14


def test_attention_matches_torch_sdpa():
    """Build normalised q/k and values with torch ops (rms_norm, matmul), rotate
    with the pinned RoPE, run torch's fp64 SDPA and compare to the oracle."""
    inp = make_inputs(Shape(8, 2, 24, 12, 6, 10, "f32"), (19, 5), seed=7)
    eps, tau, base = 1e-6, 0.37, 10000.0
    ref = explicit_decode(*_decode_args(inp), eps=eps, tau=tau, base=base)
    H, G = 8, 2
    for b, L in enumerate(inp.lengths):
        c = torch.from_numpy(inp.latents[b].astype(np.float64))
        kr = F.rms_norm(torch.from_numpy(inp.k_rope_raw[b].astype(np.float64)), (6,),
                        weight=torch.from_numpy(inp.gamma_k_rope.astype(np.float64)), eps=eps)
        kr = torch.from_numpy(rope(kr.numpy(), np.arange(L), base))
        for h in range(H):
            g = h * G // H
            k = c @ torch.from_numpy(inp.w_uk[g].astype(np.float64))
            k = F.rms_norm(k, (12,), weight=torch.from_numpy(inp.gamma_k.astype(np.float64)), eps=eps)
            q = F.rms_norm(torch.from_numpy(inp.q_c[b, h].astype(np.float64)), (12,),
                           weight=torch.from_numpy(inp.gamma_q.astype(np.float64)), eps=eps)
            qr = F.rms_norm(torch.from_numpy(inp.q_rope[b, h].astype(np.float64)), (6,),
                            weight=torch.from_numpy(inp.gamma_q_rope.astype(np.float64)), eps=eps)
            qr = torch.from_numpy(rope(qr.numpy(), L - 1, base))
            v = c @ torch.from_numpy(inp.w_uv[g].astype(np.float64))
            o = F.scaled_dot_product_attention(torch.cat([q, qr])[None, None, None],
                                               torch.cat([k, kr], -1)[None, None],
                                               v[None, None], scale=tau)[0, 0, 0].numpy()
            assert _rel(ref["o"][b, h], o) < 1e-12


def test_token_chunk_loop_matches_one_chunk():
    """The keys are materialised chunk by chunk (the loop only runs more than
    once past 65536 tokens).  Chunks of 7 over 50 and 23 tokens (several full
    chunks and a ragged tail) must give the one-chunk result; in QK-norm mode
    both must also equal the absorbed form, which has no chunk loop."""
    inp = make_inputs(Shape(8, 2, 24, 12, 6, 10, "f32"), (50, 23), seed=71)
    for qk_norm in (True, False):
        one = explicit_decode(*_decode_args(inp), qk_norm=qk_norm)
        for chunk in (7, 16, 49, 50):
            many = explicit_decode(*_decode_args(inp), qk_norm=qk_norm, chunk=chunk)
            for k in ("o", "o_lat", "lse"):
                assert _rel(many[k], one[k]) < 1e-13, (qk_norm, chunk, k)
    ab = absorbed_decode(*_decode_args(inp))
    many = explicit_decode(*_decode_args(inp), chunk=7)
    assert _rel(many["o"], ab["o"]) < 1e-12 and _rel(many["o_lat"], ab["o_lat"]) < 1e-12


def test_explicit_logits_are_the_softmax_inputs():
    """explicit_logits (what the GPU tests use to state conditions on the
    inputs) gives logits whose log-sum-exp is the oracle's lse and whose
    softmax-weighted latents are its o_lat; with chunk=5 the same."""
    inp = make_inputs(Shape(8, 4, 24, 12, 6, 10, "f32"), (19, 30), seed=72)
    H, G = 8, 4
    for qk_norm, b in ((True, 0), (True, 1), (False, 0), (False, 1)):
        ref = explicit_decode(*_decode_args(inp), qk_norm=qk_norm)
        for g in range(G):
            heads = [h for h in range(H) if group_of_head(h, H, G) == g]
            for chunk in (65536, 5):
                lg = explicit_logits(inp.q_c, inp.q_rope, inp.latents[b], inp.k_rope_raw[b],
                                     inp.w_uk, inp.gamma_q, inp.gamma_k, inp.gamma_q_rope,
                                     inp.gamma_k_rope, b, g, qk_norm=qk_norm, chunk=chunk)
                assert lg.shape == (len(heads), inp.lengths[b])
                lse = scipy.special.logsumexp(lg, axis=-1)
                assert np.max(np.abs(lse - ref["lse"][b, heads])) < 1e-12
                p = scipy.special.softmax(lg, axis=-1)
                assert _rel(p @ inp.latents[b].astype(np.float64), ref["o_lat"][b, heads]) < 1e-12


# --- several query rows per sequence (causal) --------------------------------

def test_multi_query_matches_causal_sdpa():
    """s_q query rows per sequence: torch's fp64 SDPA with an explicit causal
    mask (row i sees cache rows 0..L-s_q+i) and each RoPE query rotated by its
    own position, against the multi-query oracle."""
    shape = Shape(6, 3, 20, 12, 4, 10, "f32")
    inp = make_inputs(shape, (9, 5, 3), seed=71)
    s_q = 3
    q_c, q_rope = multi_query_rows(shape, 3, s_q, seed=72)
    eps, tau, base = 1e-6, 0.41, 10000.0
    ref = explicit_decode_multi(q_c, q_rope, inp.latents, inp.k_rope_raw, inp.w_uk, inp.w_uv,
                                inp.gamma_q, inp.gamma_k, inp.gamma_q_rope, inp.gamma_k_rope,
                                eps=eps, tau=tau, base=base)
    H, G, dc, dr = 6, 3, 12, 4
    t64 = lambda x: torch.from_numpy(np.asarray(x, dtype=np.float64))  # noqa: E731
    for b, L in enumerate(inp.lengths):
        c = t64(inp.latents[b])
        kr = F.rms_norm(t64(inp.k_rope_raw[b]), (dr,), weight=t64(inp.gamma_k_rope), eps=eps)
        kr = t64(rope(kr.numpy(), np.arange(L), base))
        pos = np.arange(L - s_q, L)                              # query positions
        mask = torch.from_numpy(np.arange(L)[None, :] <= pos[:, None])   # [s_q][L]
        for h in range(H):
            g = h * G // H
            k = F.rms_norm(c @ t64(inp.w_uk[g]), (dc,), weight=t64(inp.gamma_k), eps=eps)
            q = F.rms_norm(t64(q_c[b, :, h]), (dc,), weight=t64(inp.gamma_q), eps=eps)
            qr = F.rms_norm(t64(q_rope[b, :, h]), (dr,), weight=t64(inp.gamma_q_rope), eps=eps)
            qr = t64(rope(qr.numpy(), pos, base))
            v = c @ t64(inp.w_uv[g])
            o = F.scaled_dot_product_attention(torch.cat([q, qr], -1)[None, None],
                                               torch.cat([k, kr], -1)[None, None], v[None, None],
                                               attn_mask=mask, scale=tau)[0, 0].numpy()
            assert _rel(ref["o"][b, :, h], o) < 1e-12, (b, h)


def test_multi_query_rows_are_causal():
    """Changing the cache rows after query row i's position leaves row i (and
    every earlier row) unchanged and changes the later rows."""
    shape = Shape(4, 2, 16, 8, 4, 8, "f32")
    inp = make_inputs(shape, (12,), seed=73)
    s_q = 4
    q_c, q_rope = multi_query_rows(shape, 1, s_q, seed=74)
    args = (inp.w_uk, inp.w_uv, inp.gamma_q, inp.gamma_k, inp.gamma_q_rope, inp.gamma_k_rope)
    a = explicit_decode_multi(q_c, q_rope, inp.latents, inp.k_rope_raw, *args)
    lat = [inp.latents[0].copy()]
    lat[0][10:] *= 3.0                    # rows 10, 11 = positions of query rows 2, 3
    b = explicit_decode_multi(q_c, q_rope, lat, inp.k_rope_raw, *args)
    assert np.array_equal(a["o"][0, :2], b["o"][0, :2])
    assert np.all(np.abs(a["o"][0, 2:] - b["o"][0, 2:]).max(axis=-1) > 1e-6)


# --- RoPE closed forms -------------------------------------------------------

def test_rope_closed_form_golden():
    gold = json.load(open(os.path.join(GOLDEN, "rope_closed_form.json")))
    d, base = gold["d_r"], gold["base"]
    assert np.allclose(rope_inv_freq(d, base), gold["theta"], rtol=1e-14, atol=0)
    for case in gold["cases"]:
        i, p = case["pair"], case["pos"]
        e = np.zeros(d)
        e[2 * i] = 1.0
        out = rope(e, p, base)
        assert abs(out[2 * i] - case["cos"]) < 1e-12 and abs(out[2 * i + 1] - case["sin"]) < 1e-12
        e = np.zeros(d)
        e[2 * i + 1] = 1.0
        out = rope(e, p, base)
        assert abs(out[2 * i] + case["sin"]) < 1e-12 and abs(out[2 * i + 1] - case["cos"]) < 1e-12
        others = [j for j in range(d) if j not in (2 * i, 2 * i + 1)]
        assert np.all(out[others] == 0)


def test_rope_invariants():
    rng = np.random.default_rng(3)
    x, y = rng.standard_normal(64), rng.standard_normal(64)
    assert np.allclose(rope(x, 0, 10000.0), x, rtol=0, atol=0)
    for p, pp in ((5, 9), (1000, 77), (262143, 3)):
        a = rope(x, p, 10000.0) @ rope(y, pp, 10000.0)
        b = x @ rope(y, pp - p, 10000.0)
        assert abs(a - b) < 1e-9 * (np.abs(x).sum() * np.abs(y).sum())
        assert abs(np.linalg.norm(rope(x, p, 10000.0)) - np.linalg.norm(x)) < 1e-12


# --- closed forms of the decode -------------------------------------------------

def test_single_token_value_path():
    """L_b = 1: softmax is 1 whatever the logits, so o = c_0 W^UV_g."""
    inp = make_inputs(Shape(4, 2, 32, 16, 8, 16, "f32"), (1, 1), seed=4)
    for qk in (True, False):
        out = explicit_decode(*_decode_args(inp), qk_norm=qk)
        for b in range(2):
            for h in range(4):
                g = h * 2 // 4
                c0 = inp.latents[b][0].astype(np.float64)
                assert np.allclose(out["o_lat"][b, h], c0, rtol=1e-15, atol=0)
                assert _rel(out["o"][b, h], c0 @ inp.w_uv[g].astype(np.float64)) < 1e-14


def test_zero_query_gives_uniform_softmax():
    inp = make_inputs(Shape(4, 2, 32, 16, 8, 16, "f32"), (23,), seed=5)
    inp.q_c[:] = 0
    inp.q_rope[:] = 0
    out = explicit_decode(*_decode_args(inp), eps=1e-6)
    mean_c = inp.latents[0].astype(np.float64).mean(0)
    for h in range(4):
        assert _rel(out["o_lat"][0, h], mean_c) < 1e-14
        assert abs(out["lse"][0, h] - math.log(23)) < 1e-14


def test_scale_invariance_eps0():
    """With eps = 0, c_t -> lambda c_t leaves every logit (hence lse) unchanged
    and divides alpha^k by lambda; o_lat is linear in c."""
    inp = make_inputs(Shape(4, 2, 32, 16, 8, 16, "f32"), (40,), seed=6)
    base = explicit_decode(*_decode_args(inp), eps=0.0)
    a0, _ = append_ref(inp.latents[0], inp.k_rope_raw[0], np.arange(40), inp.w_uk,
                       inp.gamma_k_rope, 0.0, 10000.0)
    rng = np.random.default_rng(0)
    lam = rng.uniform(1e-3, 1e3, 40)
    inp.latents[0] = inp.latents[0].astype(np.float64) * lam[:, None]
    sc = explicit_decode(*_decode_args(inp), eps=0.0)
    a1, _ = append_ref(inp.latents[0], inp.k_rope_raw[0], np.arange(40), inp.w_uk,
                       inp.gamma_k_rope, 0.0, 10000.0)
    assert np.allclose(sc["lse"], base["lse"], rtol=1e-13, atol=0)
    assert np.allclose(a1 * lam[:, None], a0, rtol=1e-13, atol=0)


def test_reduces_to_plain_mla():
    """gamma = 1, eps = 0, unit-RMS keys in every group and unit-RMS queries and
    RoPE inputs: the normalisations are identities, so QK-normed == plain."""
    rng = np.random.default_rng(8)
    H, G, r, dc, dr, dv, L = 8, 4, 32, 16, 8, 12, 29
    w0 = rng.standard_normal((r, dc)) / math.sqrt(r)
    rots = [np.linalg.qr(rng.standard_normal((dc, dc)))[0] for _ in range(G)]
    w_uk = np.stack([w0 @ R for R in rots])
    c = rng.standard_normal((L, r))
    c /= rms(c @ w0, 0.0)                                   # RMS(c_t W^UK_g) = 1 for every g
    kr = rng.standard_normal((L, dr))
    kr /= rms(kr, 0.0)
    q_c = rng.standard_normal((1, H, dc))
    q_c /= rms(q_c, 0.0)
    q_r = rng.standard_normal((1, H, dr))
    q_r /= rms(q_r, 0.0)
    w_uv = rng.standard_normal((G, r, dv))
    ones_c, ones_r = np.ones(dc), np.ones(dr)
    args = (q_c, q_r, [c], [kr], w_uk, w_uv, ones_c, ones_c, ones_r, ones_r)
    a = explicit_decode(*args, eps=0.0, qk_norm=True)
    b = plain_mla_decode(*args, eps=0.0)
    assert _rel(a["o"], b["o"]) < 1e-12
    assert np.allclose(a["lse"], b["lse"], rtol=1e-12, atol=1e-12)
    # and a non-unit-RMS key breaks it (the normalisation is really there)
    c2 = c.copy()
    c2[3] *= 5.0
    args2 = (q_c, q_r, [c2], [kr], w_uk, w_uv, ones_c, ones_c, ones_r, ones_r)
    assert _rel(explicit_decode(*args2, eps=0.0)["o"], plain_mla_decode(*args2, eps=0.0)["o"]) > 1e-3


def test_constant_gamma_scales_content_logit():
    """gamma_q = a, gamma_k = b (constants) multiply the content logit by a*b:
    with a zero RoPE query that equals running gamma = 1 with tau * a * b."""
    inp = make_inputs(Shape(4, 2, 32, 16, 8, 16, "f32"), (31,), seed=9)
    inp.q_rope[:] = 0
    a, b = 1.7, 0.6
    ga, gb = np.full(16, a), np.full(16, b)
    tau = 0.21
    x = explicit_decode(inp.q_c, inp.q_rope, inp.latents, inp.k_rope_raw, inp.w_uk, inp.w_uv,
                        ga, gb, inp.gamma_q_rope, inp.gamma_k_rope, tau=tau)
    y = explicit_decode(inp.q_c, inp.q_rope, inp.latents, inp.k_rope_raw, inp.w_uk, inp.w_uv,
                        np.ones(16), np.ones(16), inp.gamma_q_rope, inp.gamma_k_rope, tau=tau * a * b)
    assert _rel(x["o"], y["o"]) < 1e-13


def test_head_to_group_map_is_contiguous():
    """Head h uses group floor(h G / H): its output equals a one-group model
    holding that group's weights."""
    inp = make_inputs(Shape(6, 3, 20, 8, 4, 6, "f32"), (15,), seed=10)
    full = explicit_decode(*_decode_args(inp))
    for h in range(6):
        g = group_of_head(h, 6, 3)
        assert g == h // 2
        one = explicit_decode(inp.q_c[:, h:h + 1], inp.q_rope[:, h:h + 1], inp.latents,
                              inp.k_rope_raw, inp.w_uk[g:g + 1], inp.w_uv[g:g + 1], inp.gamma_q,
                              inp.gamma_k, inp.gamma_q_rope, inp.gamma_k_rope)
        assert _rel(full["o"][:, h], one["o"][:, 0]) < 1e-14


def test_alpha_matches_definition_elementwise():
    """alpha_{t,g} = 1/sqrt(mean_j (sum_i c_ti W_gij)^2 + eps), written with loops."""
    inp = make_inputs(Shape(4, 2, 6, 5, 4, 3, "f32"), (3,), seed=11)
    eps = 1e-3
    alpha, kr_hat = append_ref(inp.latents[0], inp.k_rope_raw[0], np.arange(3), inp.w_uk,
                               inp.gamma_k_rope, eps, 10000.0)
    for t in range(3):
        for g in range(2):
            s = 0.0
            for j in range(5):
                kj = sum(float(inp.latents[0][t, i]) * float(inp.w_uk[g, i, j]) for i in range(6))
                s += kj * kj
            assert abs(alpha[t, g] - 1.0 / math.sqrt(s / 5 + eps)) < 1e-13 * alpha[t, g]
    # stored RoPE key at row 0 is the normalised raw key (no rotation at position 0)
    x = inp.k_rope_raw[0][0].astype(np.float64)
    want = x * inp.gamma_k_rope / math.sqrt(float(np.mean(x * x)) + eps)
    assert np.allclose(kr_hat[0], want, rtol=1e-14, atol=0)


def test_absorbed_weight_layout():
    rng = np.random.default_rng(12)
    w = rng.standard_normal((2, 5, 3))
    gq, gk = rng.uniform(0.5, 1.5, 3), rng.uniform(0.5, 1.5, 3)
    wt = absorb_weights_ref(w, gq, gk)
    assert wt.shape == (2, 3, 5)
    for g in range(2):
        for j in range(3):
            for i in range(5):
                assert wt[g, j, i] == pytest.approx(gq[j] * gk[j] * w[g, i, j], rel=1e-15)


def test_default_tau():
    assert default_tau(128, 64) == pytest.approx(1 / math.sqrt(192))


# --- the pages' printed cache figures -------------------------------------------

def test_cache_size_fractions_match_pages():
    gold = json.load(open(os.path.join(GOLDEN, "cache_size.json")))
    s = gold["shape"]
    G, r, dr = s["n_groups"], s["latent_rank"], s["rope_dim"]
    assert (G, r, dr) == (DSV3.n_groups, DSV3.latent_rank, DSV3.rope_dim)
    from mla_latent_decode_amd.layout import cache_bytes_per_token
    per_tok = cache_bytes_per_token(DSV3, qk_norm=True)
    plain = cache_bytes_per_token(DSV3, qk_norm=False)
    assert per_tok == 1184 and plain == 1152
    elem_pct = 100.0 * G / r
    byte_pct = 100.0 * (per_tok - plain) / plain
    assert round(elem_pct, 2) == gold["printed"]["element_fraction_pct"]
    assert round(byte_pct, 1) == gold["printed"]["byte_fraction_pct"]


# --- inputs -----------------------------------------------------------------------

def test_bf16_rounding_is_rne_and_exact_in_torch():
    from mla_latent_decode_amd.inputs import round_bf16
    rng = np.random.default_rng(13)
    x = (rng.standard_normal(100000) * 10 ** rng.uniform(-5, 5, 100000)).astype(np.float32)
    ours = round_bf16(x)
    ref = torch.from_numpy(x).to(torch.bfloat16).float().numpy()
    assert np.array_equal(ours, ref)


def test_workload_generation_is_seeded():
    a = workload_inputs(0)
    b = workload_inputs(0)
    assert np.array_equal(a.latents[0], b.latents[0]) and np.array_equal(a.q_c, b.q_c)
    assert a.shape == TINY and a.lengths == [64]


def test_harness_counts_nan_as_a_failure():
    """The GPU tests' comparison must not skip NaN (Python's max drops it)."""
    from harness import worst_of
    assert worst_of([0.1, float("nan"), 0.2]) == float("inf")
    assert worst_of([float("nan")]) == float("inf")
    assert worst_of([0.1, 0.3]) == 0.3
