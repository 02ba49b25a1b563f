"""Pins of the training / prefill oracle (oracle/qkmla_train_oracle.py), all on
the CPU.

Forward: every query row of the causal forward is a decode step over its
prefix, so it must equal the decode oracle (itself pinned in test_oracle.py)
on that prefix.  Backward: the autograd gradient is checked element by element
against central finite differences of the forward, plus closed forms for one
token and the zero directional derivatives that the RMSNorm scale invariance
forces ("QK-Normed MLA: QK normalization without full key caching", technical
summary, Methodology: RMSNorm decomposition).
"""
import numpy as np
import pytest
import torch

import oracle
from oracle.qkmla_train_oracle import INPUT_NAMES, train_forward, train_reference
from mla_latent_decode_amd.inputs import Shape, train_inputs

SMALL = Shape(4, 2, 12, 6, 4, 5, "f32")


@pytest.mark.parametrize("qk_norm", [True, False])
@pytest.mark.parametrize("shape", [SMALL, Shape(6, 3, 10, 4, 6, 3, "f32"), Shape(2, 2, 8, 4, 2, 4, "f32")])
def test_each_row_is_a_decode_over_its_prefix(shape, qk_norm):
    B, T = 2, 9
    inp = train_inputs(shape, B, T, seed=11)
    ref = train_reference(inp, qk_norm=qk_norm, eps=1e-6, base=10000.0)
    for i in range(T):
        lat = [inp["c"][b, :i + 1] for b in range(B)]
        kr = [inp["k_rope"][b, :i + 1] for b in range(B)]
        dec = oracle.explicit_decode(inp["q_c"][:, i], inp["q_rope"][:, i], lat, kr, inp["w_uk"],
                                     inp["w_uv"], inp["gamma_q"], inp["gamma_k"],
                                     inp["gamma_q_rope"], inp["gamma_k_rope"], eps=1e-6,
                                     base=10000.0, qk_norm=qk_norm)
        np.testing.assert_allclose(ref["o"][:, i], dec["o"], rtol=1e-11, atol=1e-12)
        np.testing.assert_allclose(ref["lse"][:, i], dec["lse"], rtol=1e-11, atol=1e-12)


def _loss(inp, d_o, qk_norm, eps):
    ts = {n: torch.as_tensor(inp[n], dtype=torch.float64) for n in INPUT_NAMES}
    o, _ = train_forward(*(ts[n] for n in INPUT_NAMES), qk_norm=qk_norm, eps=eps)
    return float((o * torch.as_tensor(d_o, dtype=torch.float64)).sum())


@pytest.mark.parametrize("qk_norm", [True, False])
def test_backward_matches_central_differences(qk_norm):
    """Every element of every gradient against (f(x+h) - f(x-h)) / 2h, h=1e-6."""
    shape = Shape(4, 2, 6, 4, 4, 3, "f32")
    inp = {k: v.astype(np.float64) for k, v in train_inputs(shape, 2, 4, seed=21).items()}
    d_o = inp.pop("d_o")
    ref = train_reference(inp, d_o, qk_norm=qk_norm, eps=1e-6)
    h = 1e-6
    for n in INPUT_NAMES:
        x = inp[n]
        fd = np.zeros_like(x)
        for idx in np.ndindex(x.shape):
            keep = x[idx]
            x[idx] = keep + h
            up = _loss(inp, d_o, qk_norm, 1e-6)
            x[idx] = keep - h
            dn = _loss(inp, d_o, qk_norm, 1e-6)
            x[idx] = keep
            fd[idx] = (up - dn) / (2 * h)
        scale = max(1.0, float(np.abs(fd).max()))
        np.testing.assert_allclose(ref["d_" + n], fd, rtol=0, atol=1e-6 * scale, err_msg=n)
        if not qk_norm and n.startswith("gamma"):
            assert not np.any(ref["d_" + n])


def test_one_token_closed_forms():
    """T = 1: the softmax has one entry, so o = c W^UV_g; nothing upstream of
    the logits gets a gradient, and the value path's gradients are plain
    products with the summed per-group d_o."""
    shape = SMALL
    inp = train_inputs(shape, 3, 1, seed=31)
    d_o = inp.pop("d_o").astype(np.float64)
    ref = train_reference(inp, d_o)
    G, H = shape.n_groups, shape.n_heads
    c = inp["c"][:, 0].astype(np.float64)                        # [B][r]
    wuv = inp["w_uv"].astype(np.float64)
    for h in range(H):
        g = h * G // H
        np.testing.assert_allclose(ref["o"][:, 0, h], c @ wuv[g], rtol=1e-12, atol=1e-12)
    for n in ("q_c", "q_rope", "k_rope", "w_uk", "gamma_q", "gamma_k", "gamma_q_rope",
              "gamma_k_rope"):
        assert np.abs(ref["d_" + n]).max() < 1e-12, n
    dsum = np.stack([d_o[:, 0, [h for h in range(H) if h * G // H == g]].sum(1)
                     for g in range(G)], 1)                      # [B][G][d_v]
    d_c = np.einsum("bgv,grv->br", dsum, wuv)
    np.testing.assert_allclose(ref["d_c"][:, 0], d_c, rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(ref["d_w_uv"], np.einsum("br,bgv->grv", c, dsum), rtol=1e-12,
                               atol=1e-12)


def test_scale_invariance_gives_zero_directional_derivatives():
    """With eps = 0 the output does not change when a query row, a RoPE query
    row, a raw RoPE key row or a group's W^UK is scaled, so the gradient is
    orthogonal to each of them."""
    inp = train_inputs(SMALL, 2, 6, seed=41)
    d_o = inp.pop("d_o")
    ref = train_reference(inp, d_o, eps=0.0)
    def dot(a, b, axes):
        return np.abs(np.sum(a.astype(np.float64) * b, axis=axes)).max()
    assert dot(inp["q_c"], ref["d_q_c"], -1) < 1e-12
    assert dot(inp["q_rope"], ref["d_q_rope"], -1) < 1e-12
    assert dot(inp["k_rope"], ref["d_k_rope"], -1) < 1e-12
    assert dot(inp["w_uk"], ref["d_w_uk"], (1, 2)) < 1e-12
    # and they are not zero vectors themselves
    assert np.abs(ref["d_q_c"]).max() > 1e-3 and np.abs(ref["d_w_uk"]).max() > 1e-3


def test_future_tokens_do_not_change_earlier_rows():
    """Causality: changing the last token's inputs leaves rows 0..T-2 unchanged."""
    inp = train_inputs(SMALL, 1, 6, seed=51)
    a = train_reference(inp)
    for n in ("c", "k_rope", "q_c", "q_rope"):
        inp[n][:, -1] += 1.0
    b = train_reference(inp)
    assert np.array_equal(a["o"][:, :-1], b["o"][:, :-1])
    assert not np.allclose(a["o"][:, -1], b["o"][:, -1])


def test_packed_sequences_equal_the_batched_form():
    """Equal lengths packed end to end give the batched forward and gradients
    (the per-sequence sum is the batch's loss)."""
    from oracle.qkmla_train_oracle import train_reference_varlen
    B, T = 3, 5
    inp = train_inputs(SMALL, B, T, seed=61)
    d_o = inp.pop("d_o")
    ref = train_reference(inp, d_o)
    packed = {n: (v.reshape((B * T,) + v.shape[2:]) if n in ("c", "q_c", "q_rope", "k_rope")
                  else v) for n, v in inp.items()}
    var = train_reference_varlen(packed, [T] * B, d_o.reshape((B * T,) + d_o.shape[2:]))
    np.testing.assert_allclose(var["o"], ref["o"].reshape(var["o"].shape), rtol=1e-13, atol=1e-13)
    for n in INPUT_NAMES:
        np.testing.assert_allclose(var["d_" + n], ref["d_" + n].reshape(var["d_" + n].shape),
                                   rtol=1e-12, atol=1e-12, err_msg=n)


def test_packed_rows_do_not_see_other_sequences():
    """A row of sequence 1 is unchanged when sequence 0's tokens change."""
    from oracle.qkmla_train_oracle import train_reference_varlen
    from mla_latent_decode_amd.inputs import train_inputs_varlen
    lens = [4, 0, 3]
    inp = train_inputs_varlen(SMALL, lens, seed=62)
    a = train_reference_varlen(inp, lens)
    for n in ("c", "q_c", "q_rope", "k_rope"):
        inp[n][:4] += 1.0
    b = train_reference_varlen(inp, lens)
    assert np.array_equal(a["o"][4:], b["o"][4:])
    assert not np.allclose(a["o"][:4], b["o"][:4])
