"""qkmla_decode_noalloc (the decode with the library's per-GPU scratch array
instead of a caller workspace) against qkmla_decode on the same inputs: two
calls in a row, the second with a smaller batch and shorter sequences, each
bit-equal to the workspace decode and within the bf16 tolerance of the
oracle; a batch too large for the scratch array is refused before anything
is enqueued."""
import numpy as np
import pytest
import torch

from harness import check_outputs, oracle_decode

pytestmark = pytest.mark.gpu

if torch.cuda.is_available():
    from mla_latent_decode_amd import ops
    from mla_latent_decode_amd.inputs import DSV3, make_inputs
    from mla_latent_decode_amd.runner import DecodeSession


@pytest.mark.parametrize("qk_norm", [True, False])
def test_noalloc_decode_equals_workspace_decode(qk_norm):
    cfg = ops.Config.from_shape(DSV3, qk_norm=qk_norm)
    for label, lens, seed in (("first call", (1000, 333, 64, 1500), 900),
                              ("second call, smaller", (70, 5), 901)):
        print(f"\n[no-alloc decode qk_norm={qk_norm}, {label}] lens={lens}", flush=True)
        inp = make_inputs(DSV3, lens, seed=seed)
        sess = DecodeSession(cfg, inp)
        o_ws, lse_ws = sess.decode()
        o_ws, lse_ws = o_ws.clone(), lse_ws.clone()
        B, H, r = len(lens), cfg.n_heads, cfg.latent_rank
        o_na = torch.full((B, H, r), float("nan"), dtype=torch.float32, device="cuda")
        lse_na = torch.full((B, H), float("nan"), dtype=torch.float32, device="cuda")
        status = torch.zeros((1,), dtype=torch.int32, device="cuda")
        ops.decode_noalloc(cfg, sess.q_c, sess.q_rope, sess.w_qabs, sess.gamma_q_rope, sess.lat,
                           sess.rope, sess.alpha, sess.seq_lens, max(lens), o_na, lse_na, status)
        torch.cuda.synchronize()
        assert int(status.item()) == 0
        assert torch.equal(o_na, o_ws) and torch.equal(lse_na, lse_ws), label
        sess.o_lat.copy_(o_na)
        o = sess.out_proj().cpu().numpy()
        check_outputs(o, o_na.cpu().numpy(), lse_na.cpu().numpy(), oracle_decode(inp, cfg), "bf16",
                      range(B), list(range(H)), f"no-alloc decode, {label}")


def test_noalloc_decode_refuses_a_batch_beyond_the_scratch():
    cfg = ops.Config.from_shape(DSV3)
    B, L = 4096, 64
    need = ops.decode_workspace_size(cfg, B, L)
    assert need > (128 << 20)
    q = torch.zeros((B, 128, 128), dtype=torch.bfloat16, device="cuda")
    qr = torch.zeros((B, 128, 64), dtype=torch.bfloat16, device="cuda")
    w = torch.zeros((8, 512, 128), dtype=torch.bfloat16, device="cuda")
    g = torch.ones((64,), dtype=torch.float32, device="cuda")
    lat = torch.zeros((B, L, 512), dtype=torch.bfloat16, device="cuda")
    rope = torch.zeros((B, L, 64), dtype=torch.bfloat16, device="cuda")
    alpha = torch.zeros((B, L, 8), dtype=torch.float32, device="cuda")
    lens = torch.full((B,), L, dtype=torch.int32, device="cuda")
    o = torch.full((B, 128, 512), 7.0, dtype=torch.float32, device="cuda")
    with pytest.raises(ops.QkmlaError, match="scratch"):
        ops.decode_noalloc(cfg, q, qr, w, g, lat, rope, alpha, lens, L, o)
    torch.cuda.synchronize()
    assert torch.all(o == 7.0)
