"""GPU parity of the training / prefill path (qkmla_train_forward and
qkmla_train_backward through the C ABI) against the fp64 oracle's forward and
autograd backward.

All device arithmetic is fp32; bf16 storage only rounds the inputs, and the
oracle is given the same rounded values.  Bounds: o per (token, head) row
2e-5 relative to its largest element, lse 2e-5 relative (at least 1), every
gradient tensor 1e-4 of its largest element (fp32 sums of up to a few
thousand terms against fp64)."""
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


def _run(shape, B, T, seed, qk_norm=True, ref_rows=None):
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
    errs = {}
    for n in NAMES:
        r_ = ref["d_" + n]
        scale = float(np.max(np.abs(r_))) if np.any(r_) else 1.0
        errs[n] = worst_of(np.abs(grads["d_" + n].cpu().numpy() - r_)) / scale
    print(f"  o {err_o:.2e} lse {err_l:.2e} " + " ".join(f"{k} {v:.1e}" for k, v in errs.items()),
          flush=True)
    assert err_o <= 2e-5 and err_l <= 2e-5
    for n, e in errs.items():
        assert e <= 1e-4, (n, e)


@pytest.mark.parametrize("qk_norm", [True, False])
def test_train_small_fp32(qk_norm):
    _run(Shape(4, 2, 12, 6, 4, 5, "f32"), 2, 7, 700, qk_norm=qk_norm)


def test_train_bf16_storage_odd_groups():
    _run(Shape(6, 3, 40, 16, 8, 12, "bf16"), 2, 45, 701)


def test_train_sequences_longer_than_a_chunk():
    _run(Shape(4, 2, 32, 16, 8, 16, "f32"), 2, 600, 702)


def test_train_deepseek_like_layer():
    """The DeepSeek-V3-like layer (H=128, G=8, r=512, d_c=128, d_r=64,
    d_v=128) in bf16 storage, two sequences of 96 tokens."""
    _run(DSV3, 2, 96, 703)
