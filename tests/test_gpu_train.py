"""GPU parity of the training / prefill path (qkmla_train_forward and
qkmla_train_backward through the C ABI) against the fp64 oracle's forward and
autograd backward.

Row-parallel path (any shape): all device arithmetic is fp32; bf16 storage
only rounds the inputs, and the oracle is given the same rounded values.
Bounds: o per (token, head) row 2e-5 relative to its largest element, lse
2e-5 relative (at least 1), every gradient tensor 1e-4 of its largest element
(fp32 sums of up to a few thousand terms against fp64).
MFMA path (the bf16 layer with 16 heads per group, d_c + d_r = 192,
d_v = 128): normalised queries and keys, values, softmax weights, dS and d_o
are rounded to bf16 (2^-9 relative), so o is held to 2e-2, lse to 5e-2
(absolute) and every gradient to 2e-2 of its largest element."""
import numpy as np
import pytest
import torch

from harness import worst_of

pytestmark = pytest.mark.gpu

if torch.cuda.is_available():
    from mla_latent_decode_amd import ops
    from mla_latent_decode_amd.inputs import DSV3, Shape, train_inputs

NAMES = ("c", "q_c", "q_rope", "k_rope", "w_uk", "w_uv", "gamma_q", "gamma_k", "gamma_q_rope",
         "gamma_k_rope")


FP32_TOL = dict(o=2e-5, lse=2e-5, grad=1e-4)
BF16_TOL = dict(o=2e-2, lse=5e-2, grad=2e-2)


def _run(shape, B, T, seed, qk_norm=True, tol=FP32_TOL):
    import oracle
    from oracle.qkmla_train_oracle import train_reference
    print(f"\n[train {shape} B={B} T={T} qk_norm={qk_norm}]", flush=True)
    cfg = ops.Config.from_shape(shape, qk_norm=qk_norm)
    inp = train_inputs(shape, B, T, seed)
    d_o = inp.pop("d_o")
    dt = cfg.torch_dtype
    dev = {n: torch.from_numpy(np.ascontiguousarray(inp[n])).to(
        "cuda", torch.float32 if (n == "w_uk" or n.startswith("gamma")) else dt) for n in NAMES}
    ws = torch.empty((ops.train_workspace_size(cfg, B, T),), dtype=torch.uint8, device="cuda")
    o, lse = ops.train_forward(cfg, dev, ws)
    g_o = torch.from_numpy(d_o).cuda()
    grads = ops.train_backward(cfg, dev, o, lse, g_o, ws)
    torch.cuda.synchronize()
    ref = train_reference(inp, d_o, qk_norm=qk_norm, eps=cfg.eps, base=cfg.rope_base)
    dv = shape.v_head_dim
    err_o = worst_of(oracle.rowwise_rel_err(o.cpu().numpy().reshape(-1, dv),
                                            ref["o"].reshape(-1, dv)))
    lse_np = lse.cpu().numpy()
    err_l = worst_of(np.abs(lse_np - ref["lse"]) / np.maximum(1.0, np.abs(ref["lse"])))
    if tol is BF16_TOL:
        err_l = worst_of(np.abs(lse_np - ref["lse"]))
    errs = {}
    for n in NAMES:
        r_ = ref["d_" + n]
        scale = float(np.max(np.abs(r_))) if np.any(r_) else 1.0
        errs[n] = worst_of(np.abs(grads["d_" + n].cpu().numpy() - r_)) / scale
    print(f"  o {err_o:.2e} lse {err_l:.2e} " + " ".join(f"{k} {v:.1e}" for k, v in errs.items()),
          flush=True)
    assert err_o <= tol["o"] and err_l <= tol["lse"], (err_o, err_l)
    for n, e in errs.items():
        assert e <= tol["grad"], (n, e)


@pytest.mark.parametrize("qk_norm", [True, False])
def test_train_small_fp32(qk_norm):
    _run(Shape(4, 2, 12, 6, 4, 5, "f32"), 2, 7, 700, qk_norm=qk_norm)


def test_train_bf16_storage_odd_groups():
    _run(Shape(6, 3, 40, 16, 8, 12, "bf16"), 2, 45, 701)


def test_train_sequences_longer_than_a_chunk():
    _run(Shape(4, 2, 32, 16, 8, 16, "f32"), 2, 600, 702)


@pytest.mark.parametrize("B,T,qk_norm", [(2, 96, True), (1, 300, True), (2, 77, False)])
def test_train_deepseek_like_layer_mfma(B, T, qk_norm):
    """The DeepSeek-V3-like layer (H=128, G=8, r=512, d_c=128, d_r=64,
    d_v=128) in bf16 storage, on the MFMA attention: whole and partial key
    tiles and query blocks."""
    _run(DSV3, B, T, 703 + T, qk_norm=qk_norm, tol=BF16_TOL)


@pytest.mark.parametrize("T", [2048, 8192])
def test_train_full_length_sampled_and_invariants(T):
    """2048 and 8192 tokens of the bf16 layer (at 8192 the projection GEMMs
    take their 128 x 128 tiles, below it 64 x 64): sampled forward rows
    against the decode oracle over their prefix (a training row is a decode
    step), and the backward against properties that hold at any size: the
    RMSNorm scale invariance makes each gradient row of q_c, q_rope and
    k_rope, and each group's W^UK gradient, orthogonal to its input (up to
    eps = 1e-6)."""
    import oracle
    B = 1
    cfg = ops.Config.from_shape(DSV3)
    inp = train_inputs(DSV3, B, T, {2048: 720, 8192: 721}[T])
    d_o = inp.pop("d_o")
    dt = cfg.torch_dtype
    dev = {n: torch.from_numpy(np.ascontiguousarray(inp[n])).to(
        "cuda", torch.float32 if (n == "w_uk" or n.startswith("gamma")) else dt) for n in NAMES}
    ws = torch.empty((ops.train_workspace_size(cfg, B, T),), dtype=torch.uint8, device="cuda")
    print(f"\n[train full length T={T}]", flush=True)
    o, lse = ops.train_forward(cfg, dev, ws)
    grads = ops.train_backward(cfg, dev, o, lse, torch.from_numpy(d_o).cuda(), ws)
    torch.cuda.synchronize()
    o_np, lse_np = o.cpu().numpy(), lse.cpu().numpy()
    G, hpg = DSV3.n_groups, DSV3.n_heads // DSV3.n_groups
    for i, g in ((0, 0), (777, 3), (T - 1, 7)):
        ref = oracle.explicit_decode(inp["q_c"][:, i], inp["q_rope"][:, i],
                                     [inp["c"][0, :i + 1]], [inp["k_rope"][0, :i + 1]],
                                     inp["w_uk"], inp["w_uv"], inp["gamma_q"], inp["gamma_k"],
                                     inp["gamma_q_rope"], inp["gamma_k_rope"], groups=[g])
        hs = list(range(g * hpg, (g + 1) * hpg))
        e = worst_of(oracle.rowwise_rel_err(o_np[0, i, hs], ref["o"][0, hs]))
        el = worst_of(np.abs(lse_np[0, i, hs] - ref["lse"][0, hs]))
        print(f"  row {i} group {g}: o {e:.2e} lse {el:.2e}", flush=True)
        assert e <= BF16_TOL["o"] and el <= BF16_TOL["lse"]
    def cos(a, b, axes):
        num = np.abs(np.sum(a * b, axis=axes))
        den = np.sqrt(np.sum(a * a, axis=axes) * np.sum(b * b, axis=axes)) + 1e-30
        return float(np.max(num / den))
    g_np = {k: v.cpu().numpy().astype(np.float64) for k, v in grads.items()}
    worst = {"q_c": cos(g_np["d_q_c"], inp["q_c"].astype(np.float64), -1),
             "q_rope": cos(g_np["d_q_rope"], inp["q_rope"].astype(np.float64), -1),
             "k_rope": cos(g_np["d_k_rope"], inp["k_rope"].astype(np.float64), -1),
             "w_uk": cos(g_np["d_w_uk"], inp["w_uk"].astype(np.float64), (1, 2))}
    print("  |cos(grad, input)| " + " ".join(f"{k} {v:.1e}" for k, v in worst.items()), flush=True)
    # the RMSNorm backward makes these exact up to fp32 rounding, whatever
    # the accuracy of the attention gradient that enters it
    for k, v in worst.items():
        assert v <= 1e-3, (k, v)
    assert all(np.isfinite(v).all() for v in g_np.values())


@pytest.mark.parametrize("shape_name,lengths,tol", [
    ("small", (5, 0, 130, 1, 33), "fp32"), ("dsv3", (70, 0, 1, 257, 8), "bf16")])
def test_train_packed_sequences(shape_name, lengths, tol):
    """Packed sequences of different lengths (one empty, one of a single
    token) through qkmla_train_forward_varlen / _backward_varlen against the
    oracle's per-sequence sum."""
    from oracle.qkmla_train_oracle import train_reference_varlen
    import oracle
    from mla_latent_decode_amd.inputs import train_inputs_varlen
    shape = Shape(4, 2, 32, 16, 8, 16, "f32") if shape_name == "small" else DSV3
    tl = FP32_TOL if tol == "fp32" else BF16_TOL
    print(f"\n[train varlen {shape_name} {lengths}]", flush=True)
    cfg = ops.Config.from_shape(shape)
    inp = train_inputs_varlen(shape, lengths, 730)
    d_o = inp.pop("d_o")
    dt = cfg.torch_dtype
    dev = {n: torch.from_numpy(np.ascontiguousarray(inp[n])).to(
        "cuda", torch.float32 if (n == "w_uk" or n.startswith("gamma")) else dt) for n in NAMES}
    cu = torch.tensor(np.concatenate([[0], np.cumsum(lengths)]), dtype=torch.int32, device="cuda")
    total, mx = int(sum(lengths)), max(lengths)
    ws = torch.empty((ops.train_workspace_size_varlen(cfg, len(lengths), total, mx),),
                     dtype=torch.uint8, device="cuda")
    status = torch.zeros((1,), dtype=torch.int32, device="cuda")
    o, lse = ops.train_forward_varlen(cfg, dev, cu, mx, ws, status=status)
    grads = ops.train_backward_varlen(cfg, dev, cu, mx, o, lse, torch.from_numpy(d_o).cuda(), ws,
                                      status=status)
    torch.cuda.synchronize()
    assert int(status.item()) == 0
    ref = train_reference_varlen(inp, lengths, d_o, eps=cfg.eps, base=cfg.rope_base)
    dv = shape.v_head_dim
    err_o = worst_of(oracle.rowwise_rel_err(o.cpu().numpy().reshape(-1, dv),
                                            ref["o"].reshape(-1, dv)))
    err_l = worst_of(np.abs(lse.cpu().numpy() - ref["lse"]))
    print(f"  o {err_o:.2e} lse {err_l:.2e}", flush=True)
    assert err_o <= tl["o"] and err_l <= max(tl["lse"], 2e-5)
    for n in NAMES:
        r_ = ref["d_" + n]
        scale = float(np.max(np.abs(r_))) if np.any(r_) else 1.0
        e = worst_of(np.abs(grads["d_" + n].cpu().numpy() - r_)) / scale
        assert e <= tl["grad"], (n, e)
