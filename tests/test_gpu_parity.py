"""GPU parity of the HIP path (through the C ABI) against the fp64 oracle.

Tolerances (see tests/harness.py): fp32 workload 1e-5 relative; bf16 caches
with fp32 accumulation 2e-2 relative on o and o_lat (per (b,h) infinity norm),
1e-3 elementwise on the alpha cache, 1e-2 per row on the RoPE cache."""
import os

import numpy as np
import pytest
import torch

from harness import TOL, check_caches, check_outputs, heads_of, oracle_decode

pytestmark = pytest.mark.gpu

if torch.cuda.is_available():
    from mla_latent_decode_amd import ops
    from mla_latent_decode_amd.inputs import (DSV3, TINY, Shape, make_inputs, multi_query_rows,
                                              workload_inputs)
    from mla_latent_decode_amd.runner import DecodeSession


def _run(cfg, inp, label, hold_last=False, L_cap=None):
    print(f"\n[{label}] B={len(inp.lengths)} lens={inp.lengths[:6]}{'...' if len(inp.lengths) > 6 else ''}",
          flush=True)
    sess = DecodeSession(cfg, inp, L_cap=L_cap, hold_last=hold_last)
    if hold_last:
        sess.step_append()
    o_lat, lse = sess.decode()
    o = sess.out_proj()
    torch.cuda.synchronize()
    return sess, o.cpu().numpy(), o_lat.cpu().numpy(), lse.cpu().numpy()


def _full_check(cfg, inp, label, **kw):
    sess, o, o_lat, lse = _run(cfg, inp, label, **kw)
    ref = oracle_decode(inp, cfg)
    bs = range(len(inp.lengths))
    check_outputs(o, o_lat, lse, ref, cfg.dtype, bs, list(range(cfg.n_heads)), label)
    check_caches(sess, inp, cfg, bs)
    assert int(sess.status.item()) == 0
    return sess


def test_tiny_fp32_workload_full_parity():
    inp = workload_inputs(0)
    cfg = ops.Config.from_shape(TINY)
    _full_check(cfg, inp, "tiny fp32 B1 L64")


@pytest.mark.parametrize("qk_norm", [True, False])
def test_fp32_generic_shapes(qk_norm):
    for i, (shape, lens) in enumerate([
        (Shape(4, 4, 32, 16, 8, 16, "f32"), (7, 1, 300)),
        (Shape(6, 3, 20, 12, 4, 10, "f32"), (9, 257)),
        (Shape(8, 1, 64, 16, 8, 16, "f32"), (33,)),
    ]):
        inp = make_inputs(shape, lens, seed=200 + i)
        cfg = ops.Config.from_shape(shape, qk_norm=qk_norm)
        _full_check(cfg, inp, f"fp32 generic {i} qk_norm={qk_norm}")


@pytest.mark.parametrize("lens", [(1, 37, 300), (32, 64), (1000,), (31, 33, 95, 97, 1, 2)])
def test_dsv3_bf16_small_parity(lens):
    inp = make_inputs(DSV3, lens, seed=300 + len(lens))
    cfg = ops.Config.from_shape(DSV3)
    _full_check(cfg, inp, f"dsv3 bf16 {lens}")


@pytest.mark.parametrize("n_wg", [1, 3, 6])
def test_dsv3_qk_multi_tile_segments(n_wg, monkeypatch):
    """QK-norm mode through the whole split-KV pipeline: with 1, 3 or 5
    workgroups, segments of 2 to 32 tiles (the three-stage loop turns over
    several times), workgroups holding two or three segments, and the partial
    slot of a workgroup's later segment; every head of every sequence against
    the oracle."""
    lens = (1000, 450, 200)
    rows = ops.plan_segments(lens, max(lens), n_wg)
    assert max(int(r[3] - r[2]) for r in rows) >= 7
    assert max(np.bincount(rows[:, 0])) >= 2
    if n_wg > 1:
        assert (rows[:, 4] == 1).any() and (rows[:, 4] == 0).any()
    inp = make_inputs(DSV3, lens, seed=315)
    cfg = ops.Config.from_shape(DSV3)
    monkeypatch.setenv("QKMLA_NUM_WG", str(n_wg))
    _full_check(cfg, inp, f"dsv3 bf16 QK-norm, {n_wg} workgroups")


def test_dsv3_bf16_plain_mode_parity():
    inp = make_inputs(DSV3, (5, 70, 400), seed=310)
    cfg = ops.Config.from_shape(DSV3, qk_norm=False)
    _full_check(cfg, inp, "dsv3 bf16 plain")


def _plain_logit_error_bound(inp, cfg, b, heads, lat):
    """Bound, from the inputs alone, on how far the kernel's plain-MLA logits
    (natural log) can sit from the oracle's: W~ = W^UK^T and q~ = q^C W~ are
    rounded to bf16 (2^-9 relative each), so the content logit of token t
    moves by at most tau 2^-8 sum_j |c_tj| sum_i |q_i W_ji|; the RoPE query
    and key are bf16 too.  Doubled for the fp32 sums and the P rounding.
    Returns [heads][L]."""
    from oracle import rope
    G, H = cfg.n_groups, cfg.n_heads
    c = np.abs(lat.astype(np.float64))
    L = lat.shape[0]
    kr = np.abs(rope(inp.k_rope_raw[b], np.arange(L), cfg.rope_base))
    out = np.empty((len(heads), L))
    for i, h in enumerate(heads):
        a = np.abs(inp.w_uk[(h * G) // H].astype(np.float64)) @ np.abs(inp.q_c[b, h].astype(np.float64))
        qr = np.abs(rope(inp.q_rope[b, h], L - 1, cfg.rope_base))
        out[i] = cfg.tau * 2.0 ** -7 * (c @ a + kr @ qr)
    return out


def test_dsv3_bf16_plain_planted_restream(monkeypatch):
    """Plain MLA, where logits are not bounded.  Every head h gets one planted
    latent row, along its own content-query direction W^UK_g q^C_h, whose
    logit for h is 100 nats; the rows sit in tiles that are not the first of
    their split-KV segment.  For h that row's logit exceeds every other logit
    of the sequence by more than the kernel's 2^64 reference margin, so the
    segment holding it is streamed again with a raised reference.  Checked on
    the oracle's own logits, with the kernel's logit error bound applied
    against the test: the gap exceeds 64 ln 2 and the other rows' total weight
    stays below 1e-6, so o, o_lat and lse are well posed; lse is compared
    within the planted logit's own error bound."""
    from oracle import explicit_logits
    from mla_latent_decode_amd.inputs import round_bf16
    lens, n_wg = (400, 300), 5
    rows = ops.plan_segments(lens, max(lens), n_wg)
    inp = make_inputs(DSV3, lens, seed=312)
    cfg = ops.Config.from_shape(DSV3, qk_norm=False)
    H, G = cfg.n_heads, cfg.n_groups
    rng = np.random.default_rng(313)
    planted = {}
    for b, L in enumerate(lens):
        cand = [t for r in rows if r[1] == b for t in range((r[2] + 1) * 32, min(r[3] * 32, L))]
        planted[b] = rng.choice(cand, size=H, replace=False)
        for h, t in enumerate(planted[b]):
            u = inp.w_uk[(h * G) // H].astype(np.float64) @ inp.q_c[b, h].astype(np.float64)
            inp.latents[b][t] = round_bf16((u * (100.0 / cfg.tau) / (u @ u)).astype(np.float32))
    bound_lse = {}
    for b in range(len(lens)):
        for g in range(G):
            heads = heads_of([g], H, G)
            lg = explicit_logits(inp.q_c, inp.q_rope, inp.latents[b], inp.k_rope_raw[b], inp.w_uk,
                                 inp.gamma_q, inp.gamma_k, inp.gamma_q_rope, inp.gamma_k_rope,
                                 b, g, qk_norm=False, tau=cfg.tau, base=cfg.rope_base)
            err = _plain_logit_error_bound(inp, cfg, b, heads, inp.latents[b])
            for i, h in enumerate(heads):
                t = planted[b][h]
                low = lg[i, t] - err[i, t]
                others = np.delete(lg[i] + err[i], t)
                assert low - others.max() > 64 * np.log(2.0), (b, h, low - others.max())
                assert np.sum(np.exp(others - low)) < 1e-6, (b, h)
                bound_lse[(b, h)] = err[i, t]
    monkeypatch.setenv("QKMLA_NUM_WG", str(n_wg))
    sess, o, o_lat, lse = _run(cfg, inp, "dsv3 bf16 plain, planted dominant rows")
    ref = oracle_decode(inp, cfg)
    check_outputs(o, o_lat, np.zeros_like(lse), {**ref, "lse": np.zeros_like(ref["lse"])}, "bf16",
                  range(len(lens)), list(range(H)), "plain planted re-stream (o, o_lat)")
    worst = max(abs(lse[b, h] - ref["lse"][b, h]) - e for (b, h), e in bound_lse.items())
    print(f"planted rows: lse error bound up to {max(bound_lse.values()):.2f} nats; "
          f"largest error beyond it {worst:.3e}", flush=True)
    assert worst <= TOL["bf16"]["lse"]
    assert int(sess.status.item()) == 0


def test_dsv3_bf16_log_normal_scales():
    inp = make_inputs(DSV3, (500, 129), seed=311, row_scale_log10_clip=3.0)
    cfg = ops.Config.from_shape(DSV3)
    _full_check(cfg, inp, "dsv3 bf16 log-normal rows")


@pytest.mark.parametrize("heads", [64, 32])
def test_dsv3_fewer_heads(heads):
    shape = Shape(heads, heads // 16, 512, 128, 64, 128, "bf16")
    inp = make_inputs(shape, (45, 200), seed=320 + heads)
    _full_check(ops.Config.from_shape(shape), inp, f"bf16 H={heads}")


@pytest.mark.parametrize("shape_name,lens,s_q", [("tiny", (64, 5), 2), ("dsv3", (300, 70, 2), 3),
                                                  ("dsv3", (1000,), 8)])
def test_multi_query_rows_are_causal_decodes(shape_name, lens, s_q):
    """s_q query rows per sequence (qkmla_decode_multi): row i is the token at
    position L_b - s_q + i over its causal prefix; rows with an empty prefix
    come back as zeros with lse = -inf and the status bit."""
    import oracle
    shape = TINY if shape_name == "tiny" else DSV3
    inp = make_inputs(shape, lens, seed=390 + s_q)
    cfg = ops.Config.from_shape(shape)
    print(f"\n[multi-query {shape_name} s_q={s_q}] lens={lens}", flush=True)
    sess = DecodeSession(cfg, inp)
    q_c, q_rope = multi_query_rows(shape, len(lens), s_q, seed=391 + s_q)
    qc = torch.from_numpy(q_c).to("cuda", cfg.torch_dtype)
    qr = torch.from_numpy(q_rope).to("cuda", cfg.torch_dtype)
    B, H = len(lens), cfg.n_heads
    ws = torch.empty((ops.decode_workspace_size(cfg, B * s_q, max(lens)),), dtype=torch.uint8,
                     device="cuda")
    lse = torch.empty((B, s_q, H), dtype=torch.float32, device="cuda")
    o_lat = ops.decode_multi(cfg, qc, qr, sess.w_qabs, sess.gamma_q_rope, sess.lat, sess.rope,
                             sess.alpha, sess.seq_lens, max(lens), ws, lse=lse, status=sess.status)
    o = ops.out_proj(cfg, o_lat.view(B * s_q, H, -1), sess.w_uv).view(B, s_q, H, -1)
    torch.cuda.synchronize()
    ref = oracle.explicit_decode_multi(q_c, q_rope, inp.latents, inp.k_rope_raw, inp.w_uk,
                                       inp.w_uv, inp.gamma_q, inp.gamma_k, inp.gamma_q_rope,
                                       inp.gamma_k_rope, eps=cfg.eps, tau=cfg.tau,
                                       base=cfg.rope_base)
    flat = lambda x: np.asarray(x).reshape((B * s_q,) + np.asarray(x).shape[2:])  # noqa: E731
    rows = [b * s_q + i for b in range(B) for i in range(s_q) if lens[b] - s_q + i >= 0]
    empty = [b * s_q + i for b in range(B) for i in range(s_q) if lens[b] - s_q + i < 0]
    check_outputs(flat(o.cpu().numpy()), flat(o_lat.cpu().numpy()), flat(lse.cpu().numpy()),
                  {k: flat(v) for k, v in ref.items()}, cfg.dtype, rows, list(range(H)),
                  f"multi-query s_q={s_q}")
    for v in empty:
        assert torch.all(o_lat.view(B * s_q, H, -1)[v] == 0)
        assert torch.all(torch.isneginf(lse.view(B * s_q, H)[v]))
    assert bool(int(sess.status.item()) & ops.QKMLA_DEV_BAD_SEQ_LEN) == bool(empty)


def test_split_count_does_not_change_the_result():
    """The plan (1, 7 or 256 workgroups) only changes which tokens share a
    partial.  P is rounded to bf16 relative to each segment's own reference
    max, so results agree to a few bf16 ulps (2^-9 relative per weight), and
    every plan matches the oracle."""
    inp = make_inputs(DSV3, (700, 333, 64), seed=330)
    cfg = ops.Config.from_shape(DSV3)
    ref = oracle_decode(inp, cfg)
    outs = []
    for nwg in ("1", "7", "256"):
        os.environ["QKMLA_NUM_WG"] = nwg
        try:
            sess = DecodeSession(cfg, inp)
            o_lat, lse = sess.decode()
            o = sess.out_proj()
            outs.append((o_lat.cpu().numpy().copy(), lse.cpu().numpy().copy()))
            check_outputs(o.cpu().numpy(), outs[-1][0], outs[-1][1], ref, "bf16", range(3),
                          list(range(128)), f"plan with {nwg} workgroups")
        finally:
            del os.environ["QKMLA_NUM_WG"]
    for o, l in outs[1:]:
        assert np.max(np.abs(o - outs[0][0])) <= 8e-3 * np.max(np.abs(outs[0][0]))
        assert np.max(np.abs(l - outs[0][1])) <= 2e-3


def test_invalid_sequence_length_gives_zeros_and_status():
    inp = make_inputs(DSV3, (40, 40), seed=340)
    cfg = ops.Config.from_shape(DSV3)
    sess = DecodeSession(cfg, inp)
    sess.seq_lens[1] = 0
    o_lat, lse = sess.decode()
    torch.cuda.synchronize()
    assert int(sess.status.item()) & ops.QKMLA_DEV_BAD_SEQ_LEN
    assert torch.all(o_lat[1] == 0) and torch.all(torch.isinf(lse[1])) and torch.all(lse[1] < 0)
    ref = oracle_decode(inp, cfg, batch_ids=[0])
    check_outputs(sess.out_proj().cpu().numpy(), o_lat.cpu().numpy(), lse.cpu().numpy(), ref,
                  "bf16", [0], list(range(128)), "valid neighbour of an invalid sequence")


def test_bad_append_position_sets_status_and_writes_nothing():
    inp = make_inputs(DSV3, (16,), seed=350)
    cfg = ops.Config.from_shape(DSV3)
    sess = DecodeSession(cfg, inp)
    before = sess.lat.clone()
    c = torch.ones((1, 4, 512), dtype=torch.bfloat16, device="cuda")
    k = torch.ones((1, 4, 64), dtype=torch.bfloat16, device="cuda")
    pos = torch.tensor([14], dtype=torch.int32, device="cuda")  # 14 + 4 > 16
    ops.append(cfg, c, k, sess.w_uk, sess.gamma_k_rope, pos, sess.lat, sess.rope, sess.alpha,
               sess.status)
    torch.cuda.synchronize()
    assert int(sess.status.item()) & ops.QKMLA_DEV_BAD_POSITION
    assert torch.equal(before, sess.lat)


def test_append_one_token_at_a_time_equals_bulk():
    """Forty one-token appends (the decode step's path: alpha^k on the VALU
    with fp32 W^UK) against one bulk append of the same rows (alpha^k on MFMA
    with W^UK split into bf16 high and low parts): latent and RoPE rows are
    bit-equal; alpha agrees to 2^-14 relative, far inside the 1e-3 bound both
    meet against the oracle (the MFMA path carries W^UK to 16 significant
    bits, the VALU path to 24, and they sum in different orders); a repeated
    one-token append is bit-equal to the first."""
    inp = make_inputs(DSV3, (40,), seed=360)
    cfg = ops.Config.from_shape(DSV3)
    bulk = DecodeSession(cfg, inp)
    lat = torch.zeros_like(bulk.lat)
    rope = torch.zeros_like(bulk.rope)
    alpha = torch.zeros_like(bulk.alpha)
    for t in range(40):
        c = bulk.lat[:, t:t + 1].contiguous()
        k = torch.from_numpy(inp.k_rope_raw[0][t:t + 1][None]).to("cuda", torch.bfloat16)
        pos = torch.tensor([t], dtype=torch.int32, device="cuda")
        ops.append(cfg, c, k, bulk.w_uk, bulk.gamma_k_rope, pos, lat, rope, alpha, bulk.status)
    torch.cuda.synchronize()
    assert torch.equal(lat, bulk.lat) and torch.equal(rope, bulk.rope)
    rel = ((alpha[0, :40] - bulk.alpha[0, :40]).abs() / bulk.alpha[0, :40].abs()).max().item()
    assert rel <= 2.0 ** -14, rel
    again = alpha.clone()
    for t in (0, 17, 39):
        c = bulk.lat[:, t:t + 1].contiguous()
        k = torch.from_numpy(inp.k_rope_raw[0][t:t + 1][None]).to("cuda", torch.bfloat16)
        pos = torch.tensor([t], dtype=torch.int32, device="cuda")
        ops.append(cfg, c, k, bulk.w_uk, bulk.gamma_k_rope, pos, lat, rope, again, bulk.status)
    torch.cuda.synchronize()
    assert torch.equal(again, alpha)


def test_scale_invariance_is_bit_exact_on_gpu():
    """eps = 0: scaling latent rows by powers of two leaves every logit's
    rounding unchanged, so lse is bit-identical and alpha scales exactly."""
    inp = make_inputs(DSV3, (90,), seed=370)
    cfg = ops.Config.from_shape(DSV3, eps=0.0)
    a = DecodeSession(cfg, inp)
    _, lse_a = a.decode()
    lse_a = lse_a.clone()
    k = np.random.default_rng(0).integers(-6, 7, size=90)
    inp.latents[0] = (inp.latents[0] * (2.0 ** k)[:, None]).astype(np.float32)
    b = DecodeSession(cfg, inp)
    _, lse_b = b.decode()
    torch.cuda.synchronize()
    assert torch.equal(lse_a, lse_b)
    ratio = (a.alpha[0, :90] / b.alpha[0, :90]).cpu().numpy()
    assert np.array_equal(ratio, np.broadcast_to((2.0 ** k)[:, None], ratio.shape))


def test_permuting_cache_rows_leaves_output_unchanged():
    inp = make_inputs(DSV3, (256,), seed=380)
    cfg = ops.Config.from_shape(DSV3)
    sess = DecodeSession(cfg, inp)
    o1, _ = sess.decode()
    o1 = o1.clone()
    perm = torch.randperm(256, generator=torch.Generator().manual_seed(0)).cuda()
    o2, _ = sess.decode(sess.lat[:, perm].contiguous(), sess.rope[:, perm].contiguous(),
                        sess.alpha[:, perm].contiguous())
    torch.cuda.synchronize()
    # the RoPE keys carry their own positions, so the permuted cache is the same set of tokens
    assert torch.max(torch.abs(o1 - o2)) <= 2e-2 * torch.max(torch.abs(o1))


# --- full-size workloads: sampled sequences and groups, the oracle one by one --------------

@pytest.mark.parametrize("cid,samples", [
    (1, [(0, 0), (7, 5), (15, 7)]),
    (2, [(0, 3), (3, 6)]),
    (3, [(0, 1)]),
    (4, [(0, 0), (31, 4), (63, 7)]),
])
def test_full_size_workloads_sampled(cid, samples):
    from mla_latent_decode_amd.inputs import WORKLOADS
    w = WORKLOADS[cid]
    inp = workload_inputs(cid)
    cfg = ops.Config.from_shape(w.shape)
    sess, o, o_lat, lse = _run(cfg, inp, f"workload {cid}: {w.name}", hold_last=w.append_last)
    assert int(sess.status.item()) == 0
    for b, g in samples:
        ref = oracle_decode(inp, cfg, batch_ids=[b], groups=[g])
        check_outputs(o, o_lat, lse, ref, cfg.dtype, [b], heads_of([g], cfg.n_heads, cfg.n_groups),
                      f"workload {cid} b={b} g={g}")
    check_caches(sess, inp, cfg, sorted({b for b, _ in samples}), max_rows=2048)


def test_maximum_batch_sampled():
    """The largest batch one decode call takes: 4096 sequences of 1..96 tokens
    (one to three tiles; some straddle two workgroups and are merged), caches
    from qkmla_append, the default plan.  Whole and merged sequences sampled
    against the oracle; every lse finite."""
    B = 4096
    lens = tuple(int(x) for x in np.random.default_rng(620).integers(1, 97, size=B))
    inp = make_inputs(DSV3, lens, seed=620)
    cfg = ops.Config.from_shape(DSV3)
    sess, o, o_lat, lse = _run(cfg, inp, "bf16 batch 4096 (maximum)")
    assert int(sess.status.item()) == 0
    assert np.isfinite(lse).all()
    n_cu = torch.cuda.get_device_properties(0).multi_processor_count
    n_wg = ops.plan(cfg, B, max(lens), n_cu)[0]
    rows = ops.plan_segments(lens, max(lens), n_wg)
    split = sorted({int(r[1]) for r in rows if r[4] >= 0})
    whole = sorted({int(r[1]) for r in rows if r[4] < 0})
    assert split and whole
    sample = split[::max(1, len(split) // 24)][:24] + whole[::max(1, len(whole) // 24)][:24]
    ref = oracle_decode(inp, cfg, batch_ids=sample)
    check_outputs(o, o_lat, lse, ref, cfg.dtype, sample, list(range(cfg.n_heads)),
                  f"batch 4096: {len(sample)} sampled of {len(split)} merged, {len(whole)} whole")
    check_caches(sess, inp, cfg, sample)


# --- paged caches: a block table over shared pools ---------------------------------------

def _paged_pools(cfg, inp, page_size, seed, max_blocks=None, chunk=65536):
    """Pools of scattered pages filled through qkmla_append_paged, one append
    per sequence and chunk; returns (block table, latent, rope, alpha pools)."""
    B, dt = len(inp.lengths), cfg.torch_dtype
    max_blocks = max_blocks or -(-max(inp.lengths) // page_size)
    num_pages = B * max_blocks + 5
    perm = np.random.default_rng(seed).permutation(num_pages)[:B * max_blocks]
    table = torch.from_numpy(perm.reshape(B, max_blocks).astype(np.int32)).cuda()
    rows = (num_pages, page_size)
    lat = torch.zeros(rows + (cfg.latent_rank,), dtype=dt, device="cuda")
    rope = torch.zeros(rows + (cfg.rope_dim,), dtype=dt, device="cuda")
    alpha = torch.zeros(rows + (cfg.n_groups,), dtype=torch.float32, device="cuda")
    status = torch.zeros((1,), dtype=torch.int32, device="cuda")
    w_uk = torch.from_numpy(inp.w_uk).cuda()
    gkr = torch.from_numpy(inp.gamma_k_rope).cuda()
    for b, L in enumerate(inp.lengths):
        for s in range(0, L, chunk):
            e = min(L, s + chunk)
            c = torch.from_numpy(np.ascontiguousarray(inp.latents[b][s:e][None])).to("cuda", dt)
            k = torch.from_numpy(np.ascontiguousarray(inp.k_rope_raw[b][s:e][None])).to("cuda", dt)
            pos = torch.full((1,), s, dtype=torch.int32, device="cuda")
            ops.append_paged(cfg, c, k, w_uk, gkr, pos, table[b:b + 1], lat, rope, alpha, status)
    torch.cuda.synchronize()
    assert int(status.item()) == 0
    return table, lat, rope, alpha


def _pool_rows(pool, table, b, L, page_size):
    t = torch.arange(L, device="cuda")
    prow = table[b, t // page_size].long() * page_size + t % page_size
    return pool.view(-1, pool.shape[-1])[prow]


@pytest.mark.parametrize("shape_name,lens,page_size", [
    ("tiny", (64, 5, 37), 5), ("dsv3", (1000, 333, 64, 1), 32), ("dsv3", (700, 90), 64)])
def test_paged_caches_equal_contiguous_bitwise(shape_name, lens, page_size):
    """qkmla_append_paged places exactly the rows qkmla_append writes, and
    qkmla_decode_paged returns the contiguous decode's outputs bit for bit
    (the same tiles and plan read through the block table); the contiguous
    outputs are checked against the oracle."""
    shape = TINY if shape_name == "tiny" else DSV3
    inp = make_inputs(shape, lens, seed=450 + page_size)
    cfg = ops.Config.from_shape(shape)
    sess, o, o_lat, lse = _run(cfg, inp, f"paged {shape_name} page_size={page_size}")
    check_outputs(o, o_lat, lse, oracle_decode(inp, cfg), cfg.dtype, range(len(lens)),
                  list(range(cfg.n_heads)), "contiguous decode")
    table, plat, prope, palpha = _paged_pools(cfg, inp, page_size, seed=451)
    for b, L in enumerate(lens):
        assert torch.equal(_pool_rows(plat, table, b, L, page_size), sess.lat[b, :L])
        assert torch.equal(_pool_rows(prope, table, b, L, page_size), sess.rope[b, :L])
        assert torch.equal(_pool_rows(palpha, table, b, L, page_size), sess.alpha[b, :L])
    B, H = len(lens), cfg.n_heads
    p_lse = torch.empty((B, 1, H), dtype=torch.float32, device="cuda")
    status = torch.zeros((1,), dtype=torch.int32, device="cuda")
    p_lat = ops.decode_paged(cfg, sess.q_c.view(B, 1, H, -1), sess.q_rope.view(B, 1, H, -1),
                             sess.w_qabs, sess.gamma_q_rope, plat, prope, palpha, sess.seq_lens,
                             table, max(lens), sess.workspace, lse=p_lse, status=status)
    torch.cuda.synchronize()
    assert int(status.item()) == 0
    assert np.array_equal(p_lat.view(B, H, -1).cpu().numpy(), o_lat)
    assert np.array_equal(p_lse.view(B, H).cpu().numpy(), lse)


def test_paged_multi_query_and_bad_page():
    """s_q = 3 over 32-row pages equals the contiguous multi-row decode bit for
    bit; a table entry outside the pool sets QKMLA_DEV_BAD_PAGE and leaves the
    other sequences' outputs unchanged."""
    lens, s_q, ps = (300, 70, 2), 3, 32
    inp = make_inputs(DSV3, lens, seed=460)
    cfg = ops.Config.from_shape(DSV3)
    sess = DecodeSession(cfg, inp)
    q_c, q_rope = multi_query_rows(DSV3, len(lens), s_q, seed=461)
    qc = torch.from_numpy(q_c).to("cuda", cfg.torch_dtype)
    qr = torch.from_numpy(q_rope).to("cuda", cfg.torch_dtype)
    B, H = len(lens), cfg.n_heads
    ws = torch.empty((ops.decode_workspace_size(cfg, B * s_q, max(lens)),), dtype=torch.uint8,
                     device="cuda")
    lse_c = torch.empty((B, s_q, H), dtype=torch.float32, device="cuda")
    o_c = ops.decode_multi(cfg, qc, qr, sess.w_qabs, sess.gamma_q_rope, sess.lat, sess.rope,
                           sess.alpha, sess.seq_lens, max(lens), ws, lse=lse_c, status=sess.status)
    table, plat, prope, palpha = _paged_pools(cfg, inp, ps, seed=462)
    lse_p = torch.empty_like(lse_c)
    status = torch.zeros((1,), dtype=torch.int32, device="cuda")
    o_p = ops.decode_paged(cfg, qc, qr, sess.w_qabs, sess.gamma_q_rope, plat, prope, palpha,
                           sess.seq_lens, table, max(lens), ws, lse=lse_p, status=status)
    torch.cuda.synchronize()
    assert int(status.item()) & ops.QKMLA_DEV_BAD_SEQ_LEN  # sequence 2 is shorter than s_q
    assert torch.equal(o_p, o_c) and torch.equal(lse_p, lse_c)
    bad = table.clone()
    bad[1, (lens[1] - 1) // ps] = plat.shape[0] + 3  # outside the pool
    status.zero_()
    o_b = ops.decode_paged(cfg, qc, qr, sess.w_qabs, sess.gamma_q_rope, plat, prope, palpha,
                           sess.seq_lens, bad, max(lens), ws, lse=lse_p, status=status)
    torch.cuda.synchronize()
    assert int(status.item()) & ops.QKMLA_DEV_BAD_PAGE
    assert torch.equal(o_b[0], o_c[0]) and torch.equal(o_b[2], o_c[2])


def test_paged_full_size_long_context():
    """Four 16384-token sequences in 64-row pages of one pool: bit-equal to the
    contiguous decode, and sampled groups against the oracle."""
    lens = (16384, 16384, 9000, 16384)
    inp = make_inputs(DSV3, lens, seed=470)
    cfg = ops.Config.from_shape(DSV3)
    sess, o, o_lat, lse = _run(cfg, inp, "paged long context, contiguous side")
    for b, g in ((0, 0), (2, 5)):
        ref = oracle_decode(inp, cfg, batch_ids=[b], groups=[g])
        check_outputs(o, o_lat, lse, ref, cfg.dtype, [b], heads_of([g], cfg.n_heads, cfg.n_groups),
                      f"long context b={b} g={g}")
    table, plat, prope, palpha = _paged_pools(cfg, inp, 64, seed=471)
    B, H = len(lens), cfg.n_heads
    status = torch.zeros((1,), dtype=torch.int32, device="cuda")
    p_lse = torch.empty((B, 1, H), dtype=torch.float32, device="cuda")
    p_lat = ops.decode_paged(cfg, sess.q_c.view(B, 1, H, -1), sess.q_rope.view(B, 1, H, -1),
                             sess.w_qabs, sess.gamma_q_rope, plat, prope, palpha, sess.seq_lens,
                             table, max(lens), sess.workspace, lse=p_lse, status=status)
    torch.cuda.synchronize()
    assert int(status.item()) == 0
    assert np.array_equal(p_lat.view(B, H, -1).cpu().numpy(), o_lat)
    assert np.array_equal(p_lse.view(B, H).cpu().numpy(), lse)


def test_decode_step_replays_in_a_hip_graph():
    """The decode step (one-token append, decode, out_proj) captured in a HIP
    graph: every replay, with eager work and synchronisations between them,
    reproduces the eager step bit for bit.  The library issues no memset or
    allocation, so nothing in the graph depends on a previous replay."""
    inp = make_inputs(DSV3, (300, 77, 1000), seed=480)
    cfg = ops.Config.from_shape(DSV3)
    print("\n[graph replay] lens=(300, 77, 1000)", flush=True)
    sess = DecodeSession(cfg, inp, hold_last=True)
    sess.step_append()
    o_lat, lse = sess.decode()
    o = sess.out_proj()
    torch.cuda.synchronize()
    ref = (o_lat.clone(), lse.clone(), o.clone())
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):  # warm-up on the capture stream
        sess.step_append()
        sess.decode()
        out = sess.out_proj()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        sess.step_append()
        sess.decode()
        out = sess.out_proj()
    torch.cuda.synchronize()
    for k in range(3):
        sess.o_lat.fill_(float("nan"))
        sess.lse.fill_(float("nan"))
        out.fill_(float("nan"))
        _ = torch.randn(1024, device="cuda").sum()  # eager work between replays
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(sess.o_lat, ref[0]), k
        assert torch.equal(sess.lse, ref[1]), k
        assert torch.equal(out, ref[2]), k
    assert int(sess.status.item()) == 0
