"""Cases run on the emulated device, each compared with the fp64 oracle.

usage: python tests/isa_emu/cases.py RUNTIME_SO [case ...]
Prints one line per check and exits non-zero if any case fails.  Runs in its
own process: the runtime stand-in must be the only HIP runtime loaded.
"""
from __future__ import annotations

import ctypes
import os
import re
import sys
import time
import traceback

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
REPO = os.path.dirname(os.path.dirname(HERE))
sys.path.insert(0, REPO)
sys.path.insert(0, os.path.dirname(HERE))

import oracle  # noqa: E402
from isa_emu.asm import Kernel, parse_inst  # noqa: E402
from isa_emu.device import Device, Session  # noqa: E402
from isa_emu.machine import Emulator, EmuError, Memory  # noqa: E402
from mla_latent_decode_amd.inputs import (DSV3, TINY, Shape, make_inputs,  # noqa: E402
                                          multi_query_rows)

TOL = {"f32": dict(o=1e-5, o_lat=1e-5, lse=1e-5), "bf16": dict(o=2e-2, o_lat=2e-2, lse=5e-2)}
MERGE_HEADS = (0, 37, 127)


def _merge_rows(name, grid, heads=MERGE_HEADS):
    """Block rows (grid y) of merge_kernel<WPH> that hold the given heads: a
    block holds max(4, WPH) / WPH heads."""
    m = re.search(r"merge_kernelILi(\d+)E", name) or re.search(r"merge_kernel<(\d+)>", name)
    wph = int(m.group(1))
    per = max(4, wph) // wph
    return sorted({h // per for h in heads if h // per < grid[1]})


def _qprep_blocks(name, grid, seqs):
    """Blocks of qprep_mfma_kernel<SPB, KS> (or the generic kernel, one
    sequence per block) that hold the given sequences: x = sequence // SPB."""
    m = re.search(r"qprep_mfma_kernelILi(\d+)E", name) or re.search(r"qprep_mfma_kernel<(\d+)", name)
    spb = int(m.group(1)) if m else 1
    xs = sorted({b // spb for b in seqs})
    return [(x, y, z) for x in xs for y in range(grid[1]) for z in range(grid[2])]


def _merge_heads_only(name, grid):
    # the merge kernel has one block per (sequence, head group): run three heads
    if "merge_kernel" in name:
        return [(x, y, z) for z in range(grid[2]) for y in _merge_rows(name, grid)
                for x in range(grid[0])]
    # the wide bulk append: the first and the last (ragged) 128-token chunk
    if "append_bf16_kernelILi4E" in name:
        return [(x, y, z) for z in range(grid[2]) for y in range(grid[1])
                for x in sorted({0, grid[0] - 1})]
    return None


def reference(shape, inp, qk_norm, batch_ids=None):
    tau = 1.0 / np.sqrt(shape.head_dim + shape.rope_dim)
    return oracle.explicit_decode(inp.q_c, inp.q_rope, inp.latents, inp.k_rope_raw, inp.w_uk,
                                  inp.w_uv, inp.gamma_q, inp.gamma_k, inp.gamma_q_rope,
                                  inp.gamma_k_rope, eps=1e-6, tau=tau, base=10000.0,
                                  qk_norm=qk_norm, batch_ids=batch_ids)


def compare(shape, got_o, got_lat, got_lse, ref, bs, hs, label, lse_rel=0.0):
    def worst(x):  # NaN (an output never written) counts as infinitely wrong
        x = np.asarray(x, np.float64)
        return float("inf") if np.isnan(x).any() else float(x.max())

    e = dict(o=0.0, o_lat=0.0, lse=0.0)
    for b in bs:
        e["o"] = max(e["o"], worst(oracle.rowwise_rel_err(got_o[b, hs], ref["o"][b, hs])))
        e["o_lat"] = max(e["o_lat"],
                         worst(oracle.rowwise_rel_err(got_lat[b, hs], ref["o_lat"][b, hs])))
        # lse_rel: unnormalised logits of magnitude |lse| carry bf16 rounding of
        # q~ (2^-9 relative) into the log-sum-exp, so its bound scales with it
        bound = 1.0 + lse_rel * np.abs(ref["lse"][b, hs]) / TOL[shape.dtype]["lse"]
        e["lse"] = max(e["lse"], worst(np.abs(got_lse[b, hs] - ref["lse"][b, hs]) / bound))
    tol = TOL[shape.dtype]
    ok = all(e[k] <= tol[k] for k in tol)
    print(f"[{'ok' if ok else 'FAIL'}] {label}: " + " ".join(f"{k} {v:.2e}" for k, v in e.items()),
          flush=True)
    if not ok:
        raise AssertionError(f"{label}: {e} above {tol}")


def run_layer(dev, shape, lens, seed, label, qk_norm=True, host_fill=True, hold_last=False,
              n_wg=None, heads=None, row_scale=None, lse_rel=0.0):
    inp = make_inputs(shape, lens, seed=seed, row_scale_log10_clip=row_scale)
    if n_wg is not None:
        os.environ["QKMLA_NUM_WG"] = str(n_wg)
    try:
        s = Session(dev, shape, inp, qk_norm=qk_norm, host_fill=host_fill, hold_last=hold_last)
        o_lat, lse = s.decode()
        out = s.out_proj()
    finally:
        os.environ.pop("QKMLA_NUM_WG", None)
    hs = list(range(shape.n_heads)) if heads is None else [h for h in heads if h < shape.n_heads]
    compare(shape, out, o_lat, lse, reference(shape, inp, qk_norm), range(len(lens)), hs, label,
            lse_rel=lse_rel)
    assert s.status[0] == 0, f"{label}: device status {s.status[0]}"
    return s


# ----------------------------------------------------------------------------
CASES = {}


def case(fn):
    CASES[fn.__name__] = fn
    return fn


@case
def fp32_tiny(dev):
    """Every fp32 kernel: absorb, append, generic q-prep and decode, out_proj."""
    run_layer(dev, TINY, (64,), 1000, "fp32 tiny layer, caches from qkmla_append",
              host_fill=False)
    run_layer(dev, Shape(6, 3, 20, 12, 4, 10, "f32"), (9, 257), 201,
              "fp32 odd shape, plain MLA", qk_norm=False, host_fill=False)


@case
def bf16_split(dev):
    """MFMA q-prep, split-KV decode with multi-tile and multi-segment
    workgroups, the merge of partials, MFMA out_proj (three heads merged)."""
    run_layer(dev, DSV3, (70, 33, 1), 500, "bf16 layer over 4 workgroups", n_wg=4,
              heads=MERGE_HEADS)
    # 9 workgroups for 6 tiles: some ranges are empty and the merge skips them
    run_layer(dev, DSV3, (70, 5, 40), 507, "bf16 9 workgroups over 6 tiles (empty ranges)",
              n_wg=9, heads=MERGE_HEADS)
    # a multiple of 8 workgroups: hardware workgroups take plan ranges in XCD order
    run_layer(dev, DSV3, (100, 90, 60), 508, "bf16 8 workgroups over 9 tiles (XCD order)",
              n_wg=8, heads=MERGE_HEADS)


@case
def bf16_many_splits(dev):
    """The merge over many sources: one sequence split over 80 workgroups
    (each source group folds two batches of sources), then 170 tiles of two
    sequences over 300 workgroups, of which 130 hold no tile: the long
    sequence lists more than 256 sources (two passes of the list), many of
    them empty."""
    run_layer(dev, DSV3, (80 * 32,), 509, "bf16 one sequence over 80 workgroups", n_wg=80,
              heads=MERGE_HEADS)
    lens = (150 * 32 - 5, 20 * 32 - 7)
    rows = _plan_rows(dev, list(lens), max(lens), 300)
    p0 = rows[rows[:, 1] == 0][:, 0]
    assert p0.max() - p0.min() + 1 > 256, "want more than one pass of the source list"
    run_layer(dev, DSV3, lens, 511, "bf16 170 tiles over 300 workgroups (empty ranges)",
              n_wg=300, heads=MERGE_HEADS)


@case
def bf16_plain_hold(dev):
    """Plain MLA split-KV and the one-token append of the decode step."""
    run_layer(dev, DSV3, (40, 64), 501, "bf16 plain MLA, last token appended in the step",
              qk_norm=False, host_fill=False, hold_last=True, n_wg=3, heads=MERGE_HEADS)


@case
def bf16_append_caches(dev):
    """The bf16 append path: alpha^k on MFMA (W^UK split into bf16 hi and lo),
    latent copy and RoPE key, filled through qkmla_append (bulk, then the
    step's one-token append), checked element by element against the oracle's
    append, then the decode on those caches."""
    lens = (40, 33, 1)
    s = run_layer(dev, DSV3, lens, 505, "bf16 caches from qkmla_append, step append",
                  host_fill=False, hold_last=True, n_wg=3, heads=MERGE_HEADS)
    inp = s.inp
    wa, wr = 0.0, 0.0
    for b, L in enumerate(lens):
        a_ref, r_ref = oracle.append_ref(inp.latents[b], inp.k_rope_raw[b], np.arange(L), inp.w_uk,
                                         inp.gamma_k_rope, 1e-6, 10000.0, qk_norm=True)
        wa = max(wa, float(np.max(np.abs(s.alpha[b, :L] - a_ref) / np.abs(a_ref))))
        rope = (s.rope[b, :L].astype(np.uint32) << 16).view(np.float32)
        wr = max(wr, float(np.max(oracle.rowwise_rel_err(rope, r_ref))))
        assert np.array_equal(s.lat[b, :L], s.store(inp.latents[b])), "latent rows not copied"
    print(f"[{'ok' if wa <= 1e-3 and wr <= 1e-2 else 'FAIL'}] append caches: alpha {wa:.2e} "
          f"(bound 1e-3) rope {wr:.2e} (bound 1e-2)", flush=True)
    assert wa <= 1e-3 and wr <= 1e-2, (wa, wr)


@case
def bf16_bulk_append_wide(dev):
    """The wide bulk append (4 token blocks per workgroup, from 4096 tokens on):
    4100 tokens of one sequence in one qkmla_append call; the first and the
    last (ragged, 4 tokens) 128-token chunks run and are checked against the
    oracle's append: alpha^k, the RoPE key and the latent copy."""
    lens = (4100,)
    inp = make_inputs(DSV3, lens, seed=508)
    s = Session(dev, DSV3, inp, host_fill=False)
    rows = list(range(128)) + list(range(4096, 4100))
    a_ref, r_ref = oracle.append_ref(inp.latents[0][rows], inp.k_rope_raw[0][rows],
                                     np.array(rows), inp.w_uk, inp.gamma_k_rope, 1e-6, 10000.0,
                                     qk_norm=True)
    wa = float(np.max(np.abs(s.alpha[0, rows] - a_ref) / np.abs(a_ref)))
    rope = (s.rope[0, rows].astype(np.uint32) << 16).view(np.float32)
    wr = float(np.max(oracle.rowwise_rel_err(rope, r_ref)))
    assert np.array_equal(s.lat[0, rows], s.store(inp.latents[0][rows])), "latent rows not copied"
    print(f"[{'ok' if wa <= 1e-3 and wr <= 1e-2 else 'FAIL'}] wide bulk append: alpha {wa:.2e} "
          f"(bound 1e-3) rope {wr:.2e} (bound 1e-2)", flush=True)
    assert wa <= 1e-3 and wr <= 1e-2, (wa, wr)
    assert s.status[0] == 0, f"device status {s.status[0]}"


@case
def bf16_64_heads(dev):
    """The two-wavefront split-KV variant (64 heads in 4 KV groups), caches
    from qkmla_append, 7 tiles over two workgroups."""
    shape = Shape(64, 4, 512, 128, 64, 128, "bf16")
    run_layer(dev, shape, (150, 70), 506, "bf16 H=64 over 2 workgroups", host_fill=False,
              n_wg=2, heads=(0, 37))  # the merge runs heads 0, 37 (and 127)


@case
def bf16_32_heads(dev):
    """The one-wavefront split-KV variant (32 heads in 2 KV groups), caches
    from qkmla_append, 7 tiles over two workgroups (two segments, a slot-1
    partial)."""
    shape = Shape(32, 2, 512, 128, 64, 128, "bf16")
    run_layer(dev, shape, (150, 70), 507, "bf16 H=32 over 2 workgroups", host_fill=False,
              n_wg=2, heads=(0, 3))  # the merge runs the block of heads 0..3 (37, 127 are past H)


def run_multi(dev, shape, lens, s_q, seed, label, n_wg=None, heads=None):
    """Decode of s_q causal query rows per sequence against the oracle; rows
    whose causal prefix is empty must come back as zeros with lse = -inf."""
    inp = make_inputs(shape, lens, seed=seed)
    q_c, q_rope = multi_query_rows(shape, len(lens), s_q, seed=seed + 1)
    if n_wg is not None:
        os.environ["QKMLA_NUM_WG"] = str(n_wg)
    try:
        s = Session(dev, shape, inp, host_fill=True)
        o_lat, lse, out = s.decode_multi(q_c, q_rope)
    finally:
        os.environ.pop("QKMLA_NUM_WG", None)
    tau = 1.0 / np.sqrt(shape.head_dim + shape.rope_dim)
    ref = oracle.explicit_decode_multi(q_c, q_rope, inp.latents, inp.k_rope_raw, inp.w_uk,
                                       inp.w_uv, inp.gamma_q, inp.gamma_k, inp.gamma_q_rope,
                                       inp.gamma_k_rope, eps=1e-6, tau=tau, base=10000.0)
    hs = list(range(shape.n_heads)) if heads is None else [h for h in heads if h < shape.n_heads]
    B = len(lens)
    valid = [(b, i) for b in range(B) for i in range(s_q) if lens[b] - s_q + i >= 0]
    flat = lambda x: x.reshape((B * s_q,) + x.shape[2:])  # noqa: E731
    rows = [b * s_q + i for b, i in valid]
    compare(shape, flat(out), flat(o_lat), flat(lse), {k: flat(v) for k, v in ref.items()}, rows,
            hs, label)
    empty = [b * s_q + i for b in range(B) for i in range(s_q) if lens[b] - s_q + i < 0]
    for v in empty:
        assert np.all(flat(o_lat)[v, hs] == 0) and np.all(np.isneginf(flat(lse)[v, hs])), v
    assert bool(s.status[0] & 1) == bool(empty), s.status[0]


@case
def multi_query(dev):
    """s_q query rows per sequence (causal): fp32 layer with s_q = 2, bf16
    layer with s_q = 3 over split segments, including a sequence shorter than
    s_q whose first row has an empty prefix, and s_q = 8 rows of a 1000-token
    sequence split over 256 workgroups."""
    run_multi(dev, Shape(6, 3, 20, 12, 4, 10, "f32"), (9, 33), 2, 510, "fp32 s_q=2")
    run_multi(dev, DSV3, (70, 40, 2), 3, 511, "bf16 s_q=3 (one row with an empty prefix)",
              n_wg=5, heads=MERGE_HEADS)
    # the GPU test's s_q = 8 case in a 256-CU launch: 8 rows of about 31 tiles
    # over 256 workgroups, so most workgroups stream one tile of one row
    run_multi(dev, DSV3, (1000,), 8, 512, "bf16 s_q=8 over 256 workgroups", n_wg=256,
              heads=MERGE_HEADS)


class CPages(ctypes.Structure):
    _fields_ = [("block_table", ctypes.c_void_p), ("max_blocks", ctypes.c_int32),
                ("page_size", ctypes.c_int32), ("num_pages", ctypes.c_int32)]


def scattered_table(B, max_blocks, num_pages, seed):
    """Block table [B][max_blocks] over a random permutation of the pool's pages."""
    perm = np.random.default_rng(seed).permutation(num_pages)[:B * max_blocks]
    return perm.reshape(B, max_blocks).astype(np.int32)


def run_paged(dev, shape, lens, s_q, page_size, seed, label, n_wg=None, heads=None,
              bad_seq=None):
    """Caches in scattered pages: the paged append must place every row the
    contiguous append writes, bit for bit, and the paged decode must return
    the contiguous decode's outputs bit for bit (same tiles, same plan), which
    are checked against the oracle.  bad_seq: a sequence whose last table
    entry points outside the pool (QKMLA_DEV_BAD_PAGE; the others unaffected)."""
    P = ctypes.c_void_p
    inp = make_inputs(shape, lens, seed=seed)
    q_c, q_rope = multi_query_rows(shape, len(lens), s_q, seed=seed + 1)
    if n_wg is not None:
        os.environ["QKMLA_NUM_WG"] = str(n_wg)
    try:
        s = Session(dev, shape, inp, host_fill=False)  # contiguous, from qkmla_append
        o_ref, lse_ref, out_ref = s.decode_multi(q_c, q_rope)
        B, G, r, dr, H = len(lens), shape.n_groups, shape.latent_rank, shape.rope_dim, shape.n_heads
        max_blocks = -(-s.L_cap // page_size)
        num_pages = B * max_blocks + 3
        table = scattered_table(B, max_blocks, num_pages, seed + 2)
        if bad_seq is not None:
            table[bad_seq, (lens[bad_seq] - 1) // page_size] = num_pages + 7
        bt = dev.put(table, "block table")
        pages = CPages(bt.ctypes.data, max_blocks, page_size, num_pages)
        et = np.uint16 if s.bf else np.float32
        rows = num_pages * page_size
        lat = dev.empty((rows, r), et, "latent pool", fill=0)
        rope = dev.empty((rows, dr), et, "rope pool", fill=0)
        alpha = dev.empty((rows, G), np.float32, "alpha pool", fill=0)
        status = dev.empty((1,), np.int32, "paged status", fill=0)
        # each sequence's rows in one append at position 0, through its table row
        for b, L in enumerate(lens):
            c = dev.put(s.store(inp.latents[b][None]), f"paged new latents {b}")
            k = dev.put(s.store(inp.k_rope_raw[b][None]), f"paged new rope keys {b}")
            pos = dev.put(np.zeros(1, np.int32), f"paged positions {b}")
            one = dev.put(table[b:b + 1], f"block table row {b}")
            pg1 = CPages(one.ctypes.data, max_blocks, page_size, num_pages)
            s.call("qkmla_append_paged", ctypes.byref(s.cfg), 1, L, P(c.ctypes.data),
                   P(k.ctypes.data), P(s.w_uk.ctypes.data), P(s.gamma_k_rope.ctypes.data),
                   P(pos.ctypes.data), ctypes.byref(pg1), P(lat.ctypes.data), P(rope.ctypes.data),
                   P(alpha.ctypes.data), P(status.ctypes.data), None)
        for b, L in enumerate(lens):
            if b == bad_seq:
                L = (L - 1) // page_size * page_size  # rows before the bad page
            t = np.arange(L)
            prow = table[b, t // page_size] * page_size + t % page_size
            assert np.array_equal(lat[prow], s.lat[b, :L]), f"{label}: latent rows of {b}"
            assert np.array_equal(rope[prow], s.rope[b, :L]), f"{label}: rope rows of {b}"
            assert np.array_equal(alpha[prow], s.alpha[b, :L]), f"{label}: alpha rows of {b}"
        qc = dev.put(s.store(q_c), "paged q_c")
        qr = dev.put(s.store(q_rope), "paged q_rope")
        o_lat = dev.empty((B, s_q, H, r), np.float32, "paged o_lat", fill=0xFF)
        lse = dev.empty((B, s_q, H), np.float32, "paged lse", fill=0xFF)
        ws = s.lib.qkmla_decode_workspace_size(ctypes.byref(s.cfg), B * s_q, s.max_len)
        wsb = dev.empty((ws,), np.uint8, "paged workspace", fill=0xCD)
        s.call("qkmla_decode_paged", ctypes.byref(s.cfg), B, s_q, P(qc.ctypes.data),
               P(qr.ctypes.data), P(s.w_qabs.ctypes.data), P(s.gamma_q_rope.ctypes.data),
               P(lat.ctypes.data), P(rope.ctypes.data), P(alpha.ctypes.data),
               P(s.seq_lens.ctypes.data), ctypes.byref(pages), s.max_len, P(wsb.ctypes.data), ws,
               P(o_lat.ctypes.data), P(lse.ctypes.data), P(status.ctypes.data), None)
    finally:
        os.environ.pop("QKMLA_NUM_WG", None)
    hs = list(range(H)) if heads is None else [h for h in heads if h < H]
    good = [b for b in range(B) if b != bad_seq]
    same = all(np.array_equal(o_lat[b][:, hs], o_ref[b][:, hs]) and
               np.array_equal(lse[b][:, hs], lse_ref[b][:, hs]) for b in good)
    print(f"[{'ok' if same else 'FAIL'}] {label}: paged decode bitwise equal to contiguous",
          flush=True)
    assert same, label
    st = int(status[0])
    assert st == (4 if bad_seq is not None else 0), f"{label}: device status {st}"
    tau = 1.0 / np.sqrt(shape.head_dim + shape.rope_dim)
    ref = oracle.explicit_decode_multi(q_c, q_rope, inp.latents, inp.k_rope_raw, inp.w_uk,
                                       inp.w_uv, inp.gamma_q, inp.gamma_k, inp.gamma_q_rope,
                                       inp.gamma_k_rope, eps=1e-6, tau=tau, base=10000.0)
    rows = [b * s_q + i for b in good for i in range(s_q)]
    flat = lambda x: x.reshape((B * s_q,) + x.shape[2:])  # noqa: E731
    compare(shape, flat(out_ref), flat(o_lat), flat(lse), {k: flat(v) for k, v in ref.items()},
            rows, hs, label + " vs oracle")


@case
def paged_caches(dev):
    """Paged latent, RoPE and alpha pools behind a block table: fp32 with
    5-row pages and s_q = 2, bf16 with 32-row pages over split segments (also
    with s_q = 2), each also with one sequence whose table entry lies outside
    the pool, and bf16 with 64-row pages (two tiles per page)."""
    run_paged(dev, Shape(6, 3, 20, 12, 4, 10, "f32"), (9, 33, 17), 2, 5, 520,
              "fp32 5-row pages, s_q=2, bad page in sequence 2", bad_seq=2)
    run_paged(dev, DSV3, (70, 40, 2), 1, 32, 521, "bf16 32-row pages over 4 workgroups",
              n_wg=4, heads=MERGE_HEADS)
    run_paged(dev, DSV3, (70, 40, 2), 1, 32, 522, "bf16 32-row pages, bad page in sequence 0",
              n_wg=3, heads=MERGE_HEADS, bad_seq=0)
    run_paged(dev, DSV3, (45, 33), 2, 32, 523, "bf16 32-row pages, s_q=2", n_wg=3,
              heads=MERGE_HEADS)
    run_paged(dev, DSV3, (150, 64, 97), 1, 64, 524,
              "bf16 64-row pages (two tiles per page) over 5 workgroups", n_wg=5,
              heads=MERGE_HEADS)


TRAIN_IN = ("c", "q_c", "q_rope", "k_rope", "w_uk", "w_uv", "gamma_q", "gamma_k", "gamma_q_rope",
            "gamma_k_rope")
TRAIN_TOL = dict(o=2e-5, lse=2e-5, grad=1e-4)


class CTrainInputs(ctypes.Structure):
    _fields_ = [(n, ctypes.c_void_p) for n in TRAIN_IN]


class CTrainGrads(ctypes.Structure):
    _fields_ = [("d_" + n, ctypes.c_void_p) for n in TRAIN_IN]


def run_train(dev, shape, B, T, seed, label, qk_norm=True, forward_only=False, tol=None,
              rows=None, heads=None):
    """Training forward and backward through the C ABI against the oracle's
    forward and autograd backward.  All arithmetic on the device is fp32 (bf16
    storage only rounds the inputs, which the oracle sees rounded), so o and
    lse are held to 2e-5 relative and every gradient to 1e-4 of its largest
    element."""
    from oracle.qkmla_train_oracle import train_reference
    from mla_latent_decode_amd.inputs import train_inputs
    from isa_emu.device import CConfig, SIGNATURES, bf16_bits
    P = ctypes.c_void_p
    lib = dev.lib
    for n, (rt, at) in SIGNATURES.items():
        if hasattr(lib, n):
            getattr(lib, n).restype, getattr(lib, n).argtypes = rt, at
    bf = shape.dtype == "bf16"
    cfg = CConfig(shape.n_heads, shape.n_groups, shape.latent_rank, shape.head_dim,
                  shape.rope_dim, shape.v_head_dim, 1 if bf else 0, int(qk_norm), 1e-6, 0.0,
                  10000.0)
    inp = train_inputs(shape, B, T, seed)
    d_o = inp.pop("d_o")
    store = (lambda x: bf16_bits(np.asarray(x, np.float32))) if bf else (
        lambda x: np.asarray(x, np.float32))
    dv = {}
    for n in TRAIN_IN:
        fp32 = n.startswith("gamma") or n == "w_uk"
        dv[n] = dev.put(np.asarray(inp[n], np.float32) if fp32 else store(inp[n]), "train " + n)
    ins = CTrainInputs(*[dv[n].ctypes.data for n in TRAIN_IN])
    H, dvh = shape.n_heads, shape.v_head_dim
    o = dev.empty((B, T, H, dvh), np.float32, "train o", fill=0xFF)
    lse = dev.empty((B, T, H), np.float32, "train lse", fill=0xFF)
    gdo = dev.put(d_o.astype(np.float32), "train d_o")
    ws_n = lib.qkmla_train_workspace_size(ctypes.byref(cfg), B, T)
    ws = dev.empty((ws_n,), np.uint8, "train workspace", fill=0xCD)

    def call(name, *args):
        r = getattr(lib, name)(*args)
        if r != 0:
            raise RuntimeError(f"{name} returned {r}: {lib.qkmla_last_error().decode()}")

    call("qkmla_train_forward", ctypes.byref(cfg), B, T, ctypes.byref(ins), P(ws.ctypes.data),
         ws_n, P(o.ctypes.data), P(lse.ctypes.data), None)
    tol = tol or TRAIN_TOL
    if forward_only:
        ref = train_reference(inp, qk_norm=qk_norm, eps=1e-6, base=10000.0)
        # rows, heads: compare only these token rows and heads (a filtered launch)
        sel = (slice(None), slice(None) if rows is None else list(rows))
        hs = slice(None) if heads is None else list(heads)
        go, ro = o[sel][:, :, hs], np.asarray(ref["o"])[sel][:, :, hs]
        eo = float(np.max(oracle.rowwise_rel_err(go.reshape(-1, dvh), ro.reshape(-1, dvh))))
        el = float(np.max(np.abs(lse[sel][:, :, hs] - np.asarray(ref["lse"])[sel][:, :, hs])))
        ok = eo <= tol["o"] and el <= tol["lse"]
        print(f"[{'ok' if ok else 'FAIL'}] {label}: o {eo:.2e} (bound {tol['o']}) lse {el:.2e} "
              f"(bound {tol['lse']})", flush=True)
        if not ok:
            raise AssertionError(f"{label}: o {eo} lse {el}")
        return
    grads = {n: dev.empty(np.shape(inp[n]), np.float32, "train d_" + n, fill=0xFF)
             for n in TRAIN_IN}
    gs = CTrainGrads(*[grads[n].ctypes.data for n in TRAIN_IN])
    call("qkmla_train_backward", ctypes.byref(cfg), B, T, ctypes.byref(ins), P(o.ctypes.data),
         P(lse.ctypes.data), P(gdo.ctypes.data), P(ws.ctypes.data), ws_n, ctypes.byref(gs), None)
    ref = train_reference(inp, d_o, qk_norm=qk_norm, eps=1e-6, base=10000.0)
    err = {"o": float(np.max(oracle.rowwise_rel_err(o.reshape(-1, dvh),
                                                    ref["o"].reshape(-1, dvh)))),
           "lse": float(np.max(np.abs(lse - ref["lse"]) / np.maximum(1.0, np.abs(ref["lse"]))))}
    gerr = {}
    for n in TRAIN_IN:
        r_ = ref["d_" + n]
        scale = float(np.max(np.abs(r_))) if np.any(r_) else 1.0
        gerr[n] = float(np.max(np.abs(grads[n] - r_))) / scale
    ok = (err["o"] <= tol["o"] and err["lse"] <= tol["lse"] and
          all(v <= tol["grad"] for v in gerr.values()))
    print(f"[{'ok' if ok else 'FAIL'}] {label}: o {err['o']:.2e} lse {err['lse']:.2e} grads " +
          " ".join(f"{k} {v:.1e}" for k, v in gerr.items()), flush=True)
    if not ok:
        raise AssertionError(f"{label}: {err} {gerr}")


def run_train_varlen(dev, shape, lengths, seed, label, tol, qk_norm=True, bad_cu=False):
    """Packed sequences through the *_varlen entry points against the oracle's
    per-sequence sum.  bad_cu: cu_seqlens that overrun the packed rows must
    set the status bit and stay in bounds (outputs not compared)."""
    from oracle.qkmla_train_oracle import train_reference_varlen
    from mla_latent_decode_amd.inputs import train_inputs_varlen
    from isa_emu.device import CConfig, SIGNATURES, bf16_bits
    P = ctypes.c_void_p
    lib = dev.lib
    for n, (rt, at) in SIGNATURES.items():
        if hasattr(lib, n):
            getattr(lib, n).restype, getattr(lib, n).argtypes = rt, at
    bf = shape.dtype == "bf16"
    cfg = CConfig(shape.n_heads, shape.n_groups, shape.latent_rank, shape.head_dim,
                  shape.rope_dim, shape.v_head_dim, 1 if bf else 0, int(qk_norm), 1e-6, 0.0,
                  10000.0)
    inp = train_inputs_varlen(shape, lengths, seed)
    d_o = inp.pop("d_o")
    total, n_seq, max_len = int(sum(lengths)), len(lengths), max(max(lengths), 1)
    cu = np.concatenate([[0], np.cumsum(lengths)]).astype(np.int32)
    if bad_cu:
        cu[-1] = total + 5  # overruns the packed rows
    store = (lambda x: bf16_bits(np.asarray(x, np.float32))) if bf else (
        lambda x: np.asarray(x, np.float32))
    dv = {}
    for n in TRAIN_IN:
        fp32 = n.startswith("gamma") or n == "w_uk"
        dv[n] = dev.put(np.asarray(inp[n], np.float32) if fp32 else store(inp[n]), "varlen " + n)
    ins = CTrainInputs(*[dv[n].ctypes.data for n in TRAIN_IN])
    H, dvh = shape.n_heads, shape.v_head_dim
    o = dev.empty((total, H, dvh), np.float32, "varlen o", fill=0xFF)
    lse = dev.empty((total, H), np.float32, "varlen lse", fill=0xFF)
    gdo = dev.put(d_o.astype(np.float32), "varlen d_o")
    cud = dev.put(cu, "cu_seqlens")
    status = dev.empty((1,), np.int32, "varlen status", fill=0)
    ws_n = lib.qkmla_train_workspace_size_varlen(ctypes.byref(cfg), n_seq, total, max_len)
    ws = dev.empty((ws_n,), np.uint8, "varlen workspace", fill=0xCD)

    def call(name, *args):
        r = getattr(lib, name)(*args)
        if r != 0:
            raise RuntimeError(f"{name} returned {r}: {lib.qkmla_last_error().decode()}")

    call("qkmla_train_forward_varlen", ctypes.byref(cfg), n_seq, P(cud.ctypes.data), total,
         max_len, ctypes.byref(ins), P(ws.ctypes.data), ws_n, P(o.ctypes.data),
         P(lse.ctypes.data), P(status.ctypes.data), None)
    grads = {n: dev.empty(np.shape(inp[n]), np.float32, "varlen d_" + n, fill=0xFF)
             for n in TRAIN_IN}
    gs = CTrainGrads(*[grads[n].ctypes.data for n in TRAIN_IN])
    call("qkmla_train_backward_varlen", ctypes.byref(cfg), n_seq, P(cud.ctypes.data), total,
         max_len, ctypes.byref(ins), P(o.ctypes.data), P(lse.ctypes.data), P(gdo.ctypes.data),
         P(ws.ctypes.data), ws_n, ctypes.byref(gs), P(status.ctypes.data), None)
    if bad_cu:
        ok = int(status[0]) == 1
        print(f"[{'ok' if ok else 'FAIL'}] {label}: status {int(status[0])} (expected 1), "
              "all accesses in bounds", flush=True)
        assert ok, label
        return
    assert int(status[0]) == 0, f"{label}: status {int(status[0])}"
    ref = train_reference_varlen(inp, lengths, d_o, qk_norm=qk_norm, eps=1e-6, base=10000.0)
    eo = float(np.max(oracle.rowwise_rel_err(o.reshape(-1, dvh), ref["o"].reshape(-1, dvh))))
    el = float(np.max(np.abs(lse - ref["lse"]) / np.maximum(1.0, np.abs(ref["lse"]))))
    gerr = {}
    for n in TRAIN_IN:
        r_ = ref["d_" + n]
        scale = float(np.max(np.abs(r_))) if np.any(r_) else 1.0
        gerr[n] = float(np.max(np.abs(grads[n] - r_))) / scale
    ok = eo <= tol["o"] and el <= tol["lse"] and all(v <= tol["grad"] for v in gerr.values())
    print(f"[{'ok' if ok else 'FAIL'}] {label}: o {eo:.2e} lse {el:.2e} grads " +
          " ".join(f"{k} {v:.1e}" for k, v in gerr.items()), flush=True)
    if not ok:
        raise AssertionError(f"{label}: o {eo} lse {el} {gerr}")


@case
def train_varlen(dev):
    """Packed sequences of different lengths (one empty) through the
    *_varlen entry points: row-parallel fp32 path and the MFMA path of the
    bf16 layer (sequences spanning key tiles and query blocks), and
    cu_seqlens overrunning the rows (status bit, accesses in bounds)."""
    run_train_varlen(dev, Shape(4, 2, 12, 6, 4, 5, "f32"), [5, 0, 9, 1], 620,
                     "train varlen fp32 (5, 0, 9, 1)", TRAIN_TOL)
    run_train_varlen(dev, DSV3, [19, 0, 34], 621, "train varlen MFMA (19, 0, 34)",
                     dict(o=2e-2, lse=5e-2, grad=2e-2))
    run_train_varlen(dev, Shape(4, 2, 12, 6, 4, 5, "f32"), [3, 4], 622,
                     "train varlen fp32, cu past the rows", TRAIN_TOL, bad_cu=True)
    run_train_varlen(dev, DSV3, [3, 6], 623, "train varlen MFMA, cu past the rows", TRAIN_TOL,
                     bad_cu=True)


@case
def train_fwd_bwd(dev):
    """Training forward and backward (explicit form, causal): fp32 and bf16
    storage on small layers, QK-norm and plain, two sequences, one longer
    than a 256-key chunk."""
    run_train(dev, Shape(4, 2, 12, 6, 4, 5, "f32"), 2, 7, 600, "train fp32 small, QK-norm")
    run_train(dev, Shape(4, 2, 12, 6, 4, 5, "f32"), 2, 7, 601, "train fp32 small, plain",
              qk_norm=False)
    run_train(dev, Shape(6, 3, 40, 16, 8, 12, "bf16"), 1, 19, 602, "train bf16 storage, G=3")
    run_train(dev, Shape(2, 1, 8, 4, 4, 4, "f32"), 1, 300, 603,
              "train fp32, 300 tokens (two chunks)")


@case
def train_mfma(dev):
    """The MFMA attention of the bf16 layer (H=128, G=8, d_c+d_r=192,
    d_v=128), forward and backward, over 70 tokens: two full key tiles and a
    partial one, so the double-buffered tile stages are each refilled, nine
    query blocks (the last partly past the sequence), and key-side waves that
    skip the query steps before their keys.  Q^, K^, V, P, dS and d_o are
    rounded to bf16: bounds 2e-2 on o (per row, relative), 5e-2 on lse and
    2e-2 on every gradient (of its largest element).  Also plain MLA (no
    norms, zero gamma gradients) over 21 tokens."""
    run_train(dev, DSV3, 1, 70, 612, "train MFMA forward + backward, 70 tokens",
              tol=dict(o=2e-2, lse=5e-2, grad=2e-2))
    run_train(dev, DSV3, 1, 21, 613, "train MFMA forward + backward, plain MLA, 21 tokens",
              qk_norm=False, tol=dict(o=2e-2, lse=5e-2, grad=2e-2))


@case
def bf16_long_segments(dev):
    """Segments long enough to run the three-stage tile loop several times:
    one workgroup streaming a 10-tile and a 2-tile sequence (both written
    directly), then two workgroups splitting the 10-tile sequence."""
    run_layer(dev, DSV3, (300, 45), 502, "bf16 one workgroup, 10 + 2 tiles", n_wg=1,
              heads=MERGE_HEADS)
    run_layer(dev, DSV3, (300, 45), 503, "bf16 two workgroups, split sequence", n_wg=2,
              heads=MERGE_HEADS)


def _plan_rows(dev, lens, cap, n_wg):
    """Host replay of the decode plan through the library: rows (workgroup,
    sequence, first tile, end tile, kind), kind -1 = written directly."""
    f = dev.lib.qkmla_plan_segments
    f.restype = ctypes.c_int
    f.argtypes = [ctypes.c_int32, ctypes.c_void_p, ctypes.c_int32, ctypes.c_int32,
                  ctypes.c_void_p, ctypes.c_int32, ctypes.POINTER(ctypes.c_int32)]
    ln = np.ascontiguousarray(lens, np.int32)
    n = ctypes.c_int32()
    assert f(len(ln), ln.ctypes.data, cap, n_wg, None, 0, ctypes.byref(n)) == 0
    out = np.zeros((n.value, 5), np.int32)
    assert f(len(ln), ln.ctypes.data, cap, n_wg, out.ctypes.data, n.value, ctypes.byref(n)) == 0
    return out


def _hw_of_plan(p, n):
    """Hardware workgroup that takes plan range p (the XCD order of the split-KV
    kernel: range (hw mod 8) * n/8 + hw/8 when n is a multiple of 8)."""
    return p if n % 8 else (p % (n // 8)) * 8 + p // (n // 8)


@case
def bf16_max_batch(dev):
    """The largest batch a decode call takes, 4096 sequences of 1..96 tokens,
    in the launch configuration of a 256-CU GPU (256 split-KV workgroups,
    hardware workgroups in XCD order).  The first and the last plan range run
    (each streams about 32 tiles of 16 sequences), with the q-prep blocks of
    the sequences they read; every sequence they complete is checked."""
    B, n_wg = 4096, 256
    lens = [int(x) for x in np.random.default_rng(510).integers(1, 97, size=B)]
    rows = _plan_rows(dev, lens, max(lens), n_wg)
    ranges = (0, n_wg - 1)
    mine = rows[np.isin(rows[:, 0], ranges)]
    read = {int(b) for b in mine[:, 1]}
    whole = sorted({int(b) for b in mine[mine[:, 4] < 0][:, 1]})
    assert len(whole) >= 8 and any(mine[:, 4] >= 0), "want whole and split sequences"
    hws = [_hw_of_plan(p, n_wg) for p in ranges]
    assert hws == [0, n_wg - 1]

    def groups(name, grid):
        if "decode_mfma_kernel" in name:
            assert grid[0] == n_wg, grid
            return [(hw, 0, 0) for hw in hws]
        if "qprep" in name:
            return _qprep_blocks(name, grid, read)
        if "merge_kernel" in name or "out_proj" in name:
            ys = _merge_rows(name, grid) if "merge" in name else range(grid[1])
            return [(b, y, z) for b in whole for y in ys for z in range(grid[2])]
        return None
    inp = make_inputs(DSV3, lens, seed=510)
    keep = dev.group_filter
    dev.group_filter = groups
    os.environ["QKMLA_NUM_WG"] = str(n_wg)
    try:
        s = Session(dev, DSV3, inp, host_fill=True, fill_only=read)
        o_lat, lse = s.decode()
        out = s.out_proj()
    finally:
        os.environ.pop("QKMLA_NUM_WG", None)
        dev.group_filter = keep
    compare(DSV3, out, o_lat, lse, reference(DSV3, inp, True, batch_ids=whole), whole,
            list(MERGE_HEADS), f"bf16 batch 4096, {len(whole)} whole sequences of two workgroups")
    assert s.status[0] == 0


def _partials_offset(B, H, r, dr):
    """Byte offset of the partial slots in the bf16 decode workspace: after
    q~ (bf16 [B][H][r]), alpha^q (f32 [B][H]) and the RoPE query (bf16
    [B][H][d_r]), each region aligned to 256 bytes."""
    def up(x):
        return (x + 255) // 256 * 256
    return up(up(up(B * H * r * 2) + B * H * 4) + B * H * dr * 2)


@case
def bf16_long_context(dev):
    """One sequence of 262144 tokens, the longest decode workload, in the
    launch configuration of a 256-CU GPU: 256 split-KV workgroups of 32 tiles
    each, hardware workgroups in XCD order.  The first and the last plan range
    run, so rows near both ends of a 256 MB latent cache are addressed.  The
    last range's partial (m, l, O) is checked against the oracle over the same
    tokens: a sequence of the range's rows only has the same key-to-query
    position differences, which is all its RoPE logits depend on."""
    L, n_wg = 262144, 256
    H, r = DSV3.n_heads, DSV3.latent_rank
    rows = _plan_rows(dev, [L], L, n_wg)
    ranges = (0, n_wg - 1)
    mine = rows[np.isin(rows[:, 0], ranges)]
    assert len(mine) == 2 and (mine[:, 4] >= 0).all(), mine
    t_first = int(mine[mine[:, 0] == n_wg - 1][0, 2]) * 32
    assert int(mine[mine[:, 0] == n_wg - 1][0, 3]) * 32 == L
    hws = [_hw_of_plan(p, n_wg) for p in ranges]

    def groups(name, grid):
        if "decode_mfma_kernel" in name:
            assert grid[0] == n_wg, grid
            return [(hw, 0, 0) for hw in hws]
        if "merge_kernel" in name:
            return []  # the other 254 partials are not computed
        return None
    inp = make_inputs(DSV3, [L], seed=520)
    keep = dev.group_filter
    dev.group_filter = groups
    os.environ["QKMLA_NUM_WG"] = str(n_wg)
    try:
        s = Session(dev, DSV3, inp, host_fill=True)
        s.decode()
    finally:
        os.environ.pop("QKMLA_NUM_WG", None)
        dev.group_filter = keep
    assert s.status[0] == 0
    # slot 0 of plan range n_wg - 1
    got_lat, got_lse = _slot_partial(np.asarray(s.ws), 2 * (n_wg - 1), H, r, DSV3.rope_dim, 1)
    tail = make_inputs(DSV3, [L], seed=520)
    tail.latents[0] = tail.latents[0][t_first:]
    tail.k_rope_raw[0] = tail.k_rope_raw[0][t_first:]
    tail.lengths[0] = L - t_first
    ref = reference(DSV3, tail, True)
    e_lat = float(np.max(oracle.rowwise_rel_err(got_lat, ref["o_lat"][0])))
    e_lse = float(np.max(np.abs(got_lse - ref["lse"][0])))
    ok = e_lat <= TOL["bf16"]["o_lat"] and e_lse <= TOL["bf16"]["lse"]
    print(f"[{'ok' if ok else 'FAIL'}] bf16 1 x 262144, partial of tokens {t_first}..{L - 1}: "
          f"o_lat {e_lat:.2e} lse {e_lse:.2e}", flush=True)
    assert ok, (e_lat, e_lse)


def _slot_partial(ws, slot, H, r, dr, B):
    """(o_lat, lse) of one partial slot of the bf16 decode workspace:
    m[H], l[H] fp32 in the exp2 domain, then O[H][r] bf16, unnormalised."""
    nbytes = H * 8 + H * r * 2
    start = _partials_offset(B, H, r, dr) + slot * nbytes
    assert start + nbytes <= ws.size
    sp = ws[start:start + nbytes]
    m = sp[:4 * H].view(np.float32).astype(np.float64)
    l_sum = sp[4 * H:8 * H].view(np.float32).astype(np.float64)
    O = (sp[8 * H:].view(np.uint16).astype(np.uint32) << 16).view(np.float32)
    O = O.reshape(H, r).astype(np.float64)
    return O / l_sum[:, None], (m + np.log2(l_sum)) * np.log(2.0)


def _run_plan_ranges(dev, inp, ranges, n_wg, label, regen, hold_last=False):
    """Run the split-KV plan ranges `ranges` of a decode in the launch
    configuration of a GPU with n_wg CUs (hardware workgroups in XCD order),
    with the q-prep of the sequences they read.  Every sequence a range covers
    whole is checked against the oracle; a partial that ends its sequence is
    checked over its own tokens, which keep their key-to-query position
    differences.  regen() draws the same inputs again (for the sliced copy)."""
    H, r, dr = DSV3.n_heads, DSV3.latent_rank, DSV3.rope_dim
    lens = list(inp.lengths)
    B = len(lens)
    rows = _plan_rows(dev, lens, max(lens), n_wg)
    mine = rows[np.isin(rows[:, 0], ranges)]
    read = sorted({int(b) for b in mine[:, 1]})
    whole = sorted({int(b) for b in mine[mine[:, 4] < 0][:, 1]})
    tails = [(int(p), int(b), int(t0) * 32, int(k)) for p, b, t0, t1, k in mine
             if k >= 0 and t1 * 32 >= lens[b]]
    assert tails or whole, mine
    hws = [_hw_of_plan(p, n_wg) for p in ranges]

    def groups(name, grid):
        if "decode_mfma_kernel" in name:
            assert grid[0] == n_wg, grid
            return [(hw, 0, 0) for hw in hws]
        if "qprep" in name:
            return _qprep_blocks(name, grid, read)
        if "merge_kernel" in name:
            return []  # the other ranges' partials are not computed
        return None
    keep = dev.group_filter
    dev.group_filter = groups
    os.environ["QKMLA_NUM_WG"] = str(n_wg)
    try:
        s = Session(dev, DSV3, inp, host_fill=True, hold_last=hold_last, fill_only=set(read))
        o_lat, lse = s.decode()
    finally:
        os.environ.pop("QKMLA_NUM_WG", None)
        dev.group_filter = keep
    assert s.status[0] == 0
    if whole:
        ref = reference(DSV3, inp, True, batch_ids=whole)
        for b in whole:
            e_lat = float(np.max(oracle.rowwise_rel_err(o_lat[b], ref["o_lat"][b])))
            e_lse = float(np.max(np.abs(lse[b] - ref["lse"][b])))
            print(f"  whole sequence {b} ({lens[b]} tokens): o_lat {e_lat:.2e} lse {e_lse:.2e}")
            assert e_lat <= TOL["bf16"]["o_lat"] and e_lse <= TOL["bf16"]["lse"], (b, e_lat, e_lse)
    ws = np.asarray(s.ws)
    for p, b, t_first, kind in tails:
        got_lat, got_lse = _slot_partial(ws, 2 * p + kind, H, r, dr, B)
        tail = regen()
        tail.latents[b] = tail.latents[b][t_first:]
        tail.k_rope_raw[b] = tail.k_rope_raw[b][t_first:]
        tail.lengths[b] = lens[b] - t_first
        ref = reference(DSV3, tail, True, batch_ids=[b])
        e_lat = float(np.max(oracle.rowwise_rel_err(got_lat, ref["o_lat"][b])))
        e_lse = float(np.max(np.abs(got_lse - ref["lse"][b])))
        print(f"  partial of sequence {b}, tokens {t_first}..{lens[b] - 1}: o_lat {e_lat:.2e} "
              f"lse {e_lse:.2e}")
        assert e_lat <= TOL["bf16"]["o_lat"] and e_lse <= TOL["bf16"]["lse"], (b, e_lat, e_lse)
    print(f"[ok] {label}: ranges {list(ranges)}, {len(whole)} whole sequences, {len(tails)} "
          f"ending partials", flush=True)


@case
def bf16_ragged_full(dev):
    """The ragged workload at full size: 64 sequences of 1024..16384 tokens
    (577k in all), latent rows scaled by log-normal factors up to 1e3, in the
    launch configuration of a 256-CU GPU.  The first and the last plan range
    run (about 70 tiles each)."""
    def regen():
        return make_inputs(DSV3, (), 1004, row_scale_log10_clip=3.0, ragged=(1024, 16384),
                           batch=64)
    _run_plan_ranges(dev, regen(), (0, 255), 256, "bf16 ragged 64 sequences", regen)


@case
def bf16_32k_step(dev):
    """The 4 x 32768 workload's step in the launch configuration of a 256-CU
    GPU: each sequence's last token is appended by the library (at row
    32767), then the first plan range and the last ranges of sequences 0 and
    3 run (16 tiles each)."""
    def regen():
        return make_inputs(DSV3, (32768,) * 4, 1002)
    _run_plan_ranges(dev, regen(), (0, 63, 255), 256, "bf16 4 x 32768 with the step's append",
                     regen, hold_last=True)


@case
def bf16_headline_sequence(dev):
    """The 16 x 4096 workload in the launch configuration of a 256-CU GPU:
    every one of sequence 0's 16 split-KV workgroups (8 tiles each, hardware
    workgroups in XCD order), its q-prep, and the merge of its 16 partials,
    checked whole against the oracle."""
    B, L, n_wg = 16, 4096, 256
    lens = [L] * B
    rows = _plan_rows(dev, lens, L, n_wg)
    mine = rows[rows[:, 1] == 0]
    ranges = sorted({int(p) for p in mine[:, 0]})
    assert len(ranges) == 16 and (mine[:, 4] >= 0).all(), mine
    assert not (rows[np.isin(rows[:, 0], ranges)][:, 1] != 0).any()
    hws = [_hw_of_plan(p, n_wg) for p in ranges]

    def groups(name, grid):
        if "decode_mfma_kernel" in name:
            assert grid[0] == n_wg, grid
            return [(hw, 0, 0) for hw in hws]
        if "qprep" in name:
            return _qprep_blocks(name, grid, [0])
        if "merge_kernel" in name:
            return [(0, y, z) for y in _merge_rows(name, grid) for z in range(grid[2])]
        if "out_proj" in name:
            return _qprep_blocks(name, grid, [0])
        return None
    inp = make_inputs(DSV3, lens, seed=530)
    keep = dev.group_filter
    dev.group_filter = groups
    os.environ["QKMLA_NUM_WG"] = str(n_wg)
    try:
        s = Session(dev, DSV3, inp, host_fill=True, fill_only={0})
        o_lat, lse = s.decode()
        out = s.out_proj()
    finally:
        os.environ.pop("QKMLA_NUM_WG", None)
        dev.group_filter = keep
    compare(DSV3, out, o_lat, lse, reference(DSV3, inp, True, batch_ids=[0]), [0],
            list(MERGE_HEADS), "bf16 16 x 4096, sequence 0 over its 16 workgroups and merge")
    assert s.status[0] == 0


@case
def train_mfma_long(dev):
    """The MFMA training forward at 1024 tokens (the training measurement's
    length): the last query block of KV group 0 (8 rows) streams every key
    tile, so the key and value rows at the far end of the sequence are
    addressed; its rows and heads are checked against the oracle.  About 15
    minutes of CPU (the projections and norms run in full), so it is run on
    demand rather than in the test suite."""
    T = 1024

    def groups(name, grid):
        if "flash_fwd_kernel" in name:
            return [(grid[0] - 1, 0, 0)]
        return None
    keep = dev.group_filter
    dev.group_filter = groups
    try:
        run_train(dev, DSV3, 1, T, 614, "train MFMA forward, 1024 tokens, last query block",
                  forward_only=True, tol=dict(o=2e-2, lse=5e-2),
                  rows=range(T - 8, T), heads=range(16))  # 8 query rows per workgroup
    finally:
        dev.group_filter = keep


@case
def bf16_plain_overflow(dev):
    """Plain MLA on latents scaled by up to 1e3: unnormalised logits exceed the
    first tile's reference by far more than 2^64, so segments are streamed
    again with a raised reference; the result must still match the oracle."""
    lens = (200, 70)
    n0 = len(dev.launches)
    run_layer(dev, DSV3, lens, 504, "bf16 plain, log-normal rows (re-stream)",
              qk_norm=False, n_wg=2, heads=MERGE_HEADS, row_scale=3.0, lse_rel=2.0 ** -7)
    # one pass issues 9 loads per wave and tile (8 latent rows + 1 RoPE), 4 waves
    one_pass = 36 * sum((L + 31) // 32 for L in lens)
    dma = sum(r[5] for r in dev.launches[n0:] if "decode_mfma_kernel" in r[0])
    assert dma > one_pass, f"no segment was streamed again ({dma} loads, one pass {one_pass})"
    print(f"[ok] re-stream taken: {dma} tile loads for a one-pass {one_pass}", flush=True)


@case
def hazard_checker(dev):
    """The wait-state check fires on an inline-asm LDS DMA that reads an SGPR a
    VALU instruction wrote one wait state earlier, and not with s_nop 4."""
    def program(nop):
        lines = ["s_mov_b32 m0, 0", "v_readfirstlane_b32 s2, v1", "v_readfirstlane_b32 s3, v2"]
        insts = [parse_inst(t, k) for k, t in enumerate(lines)]
        asm = ([f"s_nop {nop}"] if nop is not None else []) + ["global_load_lds_dword v0, s[2:3]"]
        for t in asm:
            inst = parse_inst(t, len(insts))
            inst.in_asm = True
            insts.append(inst)
        insts += [parse_inst("s_waitcnt vmcnt(0)", 90), parse_inst("s_endpgm", 91)]
        meta = {"group_segment_fixed_size": 256, "user_sgpr_count": 0}
        return Kernel("probe", insts, {}, meta, {})

    buf = np.zeros(1024, np.uint8)
    mem = Memory()
    mem.add(buf.ctypes.data, buf.nbytes, "probe buffer", buf)

    def run(nop):
        emu = Emulator(mem)
        k = program(nop)
        emu.prepare(k)
        from isa_emu.machine import Wave, Workgroup
        wg = Workgroup(256)
        w = Wave(emu, k, wg, 0, (0, 0, 0), (64, 1, 1), 0, 64)
        w.V[1] = buf.ctypes.data & 0xFFFFFFFF
        w.V[2] = buf.ctypes.data >> 32
        w.V[0] = 0
        emu._run_group(k, wg, [w], (0, 0, 0), 100)

    for nop in (None, 0, 3):
        try:
            run(nop)
        except EmuError as e:
            assert "wait states" in str(e), e
        else:
            raise AssertionError(f"hazard with s_nop {nop} not reported")
    run(4)
    print("[ok] wait-state check: reported below 5 wait states, clean at 5", flush=True)

    # An inline-asm MFMA's result read by a VALU instruction: needs
    # XDL_RESULT_WAITS wait states (s_nop N gives N + 1); a VALU write of an
    # MFMA operand needs VALU_TO_XDL_WAITS before the MFMA.
    from isa_emu.machine import VALU_TO_XDL_WAITS, XDL_RESULT_WAITS, Wave, Workgroup

    def run_mfma(nops, valu_first=False, gap=0):
        insts = []
        if valu_first:
            insts.append(parse_inst("v_mov_b32 v0, v1", 0))
            insts += [parse_inst("s_nop 0", 1)] * gap
        asm = ["v_mfma_f32_32x32x16_bf16 v[16:31], v[0:3], v[4:7], 0"] + [f"s_nop {n}" for n in nops]
        for t in asm:
            inst = parse_inst(t, len(insts))
            inst.in_asm = True
            insts.append(inst)
        insts += [parse_inst("v_mov_b32 v40, v16", 80), parse_inst("s_endpgm", 81)]
        k = Kernel("probe", insts, {}, {"group_segment_fixed_size": 0, "user_sgpr_count": 0}, {})
        emu = Emulator(mem)
        emu.prepare(k)
        w = Wave(emu, k, Workgroup(0), 0, (0, 0, 0), (64, 1, 1), 0, 64)
        emu._run_group(k, Workgroup(0), [w], (0, 0, 0), 100)

    for nops in ([], [7], [7, 7]):
        if sum(n + 1 for n in nops) >= XDL_RESULT_WAITS:
            continue
        try:
            run_mfma(nops)
        except EmuError as e:
            assert "wait states after an inline-asm MFMA" in str(e), e
        else:
            raise AssertionError(f"MFMA result read after s_nop {nops} not reported")
    run_mfma([7, 7, 7])
    try:
        run_mfma([7, 7, 7], valu_first=True, gap=VALU_TO_XDL_WAITS - 2)
    except EmuError as e:
        assert "after a VALU wrote it" in str(e), e
    else:
        raise AssertionError("VALU write just before an inline-asm MFMA not reported")
    run_mfma([7, 7, 7], valu_first=True, gap=VALU_TO_XDL_WAITS)
    print("[ok] inline-asm MFMA wait states: result reads and operand writes checked", flush=True)


@case
def isa_semantics(dev):
    """Emulator semantics that the compiled kernels lean on, against numpy on
    random registers: SDWA source selects (word / byte of a VGPR or SGPR
    source) on integer VOP ops, the gfx9 16-bit integer ops (low halves in,
    high half of the destination zeroed), v_bitop3_b32's truth table (bit
    4a + 2b + c) and the half-wave swap of v_permlane32_swap_b32."""
    from isa_emu.machine import Wave, Workgroup
    lines = [
        "v_mul_lo_u16_sdwa v3, v1, v2 dst_sel:DWORD dst_unused:UNUSED_PAD src0_sel:WORD_1 "
        "src1_sel:DWORD",
        "v_or_b32_sdwa v4, v1, v2 dst_sel:DWORD dst_unused:UNUSED_PAD src0_sel:DWORD "
        "src1_sel:WORD_1",
        "v_mul_u32_u24_sdwa v5, v1, v2 dst_sel:DWORD dst_unused:UNUSED_PAD src0_sel:WORD_0 "
        "src1_sel:BYTE_2",
        "v_lshlrev_b16_e32 v6, 3, v1",
        "v_sub_u16_e32 v7, v1, v2",
        "v_mul_lo_u16_e32 v8, v1, v2",
        # SGPR sources in SDWA forms, and the three-input bit table
        "v_and_b32_sdwa v9, s3, v2 dst_sel:DWORD dst_unused:UNUSED_PAD src0_sel:DWORD "
        "src1_sel:WORD_1",
        "v_mul_u32_u24_sdwa v10, v1, s3 dst_sel:DWORD dst_unused:UNUSED_PAD src0_sel:WORD_0 "
        "src1_sel:DWORD",
        "v_or_b32_sdwa v11, s3, v2 dst_sel:DWORD dst_unused:UNUSED_PAD src0_sel:DWORD "
        "src1_sel:WORD_1",
        "v_bitop3_b32 v12, v1, v2, s3 bitop3:0x78",
        # lanes 32..63 of the first operand trade places with lanes 0..31 of the second
        "v_mov_b32_e32 v13, v1",
        "v_mov_b32_e32 v14, v2",
        "v_permlane32_swap_b32_e32 v13, v14",
        "s_endpgm",
    ]
    insts = [parse_inst(t, k) for k, t in enumerate(lines)]
    k = Kernel("isa_semantics", insts, {}, {"group_segment_fixed_size": 0, "user_sgpr_count": 0},
               {})
    emu = Emulator(Memory())
    emu.prepare(k)
    wg = Workgroup(0)
    w = Wave(emu, k, wg, 0, (0, 0, 0), (64, 1, 1), 0, 64)
    rng = np.random.default_rng(7)
    a = rng.integers(0, 2**32, 64, dtype=np.uint64).astype(np.uint32)
    b = rng.integers(0, 2**32, 64, dtype=np.uint64).astype(np.uint32)
    w.V[1], w.V[2] = a, b
    sc = 0x9E3779B9
    w.S[3] = sc
    emu._run_group(k, wg, [w], (0, 0, 0), 100)
    a64, b64 = a.astype(np.uint64), b.astype(np.uint64)
    s64 = np.uint64(sc)
    m16 = np.uint64(0xFFFF)
    expect = {
        3: (((a64 >> np.uint64(16)) & m16) * (b64 & m16)) & m16,
        4: a64 | ((b64 >> np.uint64(16)) & m16),
        5: ((a64 & m16) * ((b64 >> np.uint64(16)) & np.uint64(0xFF))) & np.uint64(0xFFFFFFFF),
        6: ((a64 & m16) << np.uint64(3)) & m16,
        7: ((a64 & m16) - (b64 & m16)) & m16,
        8: ((a64 & m16) * (b64 & m16)) & m16,
        9: s64 & ((b64 >> np.uint64(16)) & m16),
        10: ((a64 & m16) * (s64 & np.uint64(0xFFFFFF))) & np.uint64(0xFFFFFFFF),
        11: s64 | ((b64 >> np.uint64(16)) & m16),
        12: a64 ^ (b64 & s64),  # table 0x78: bit (a b c) set for 011, 100, 101, 110
    }
    for r, e in expect.items():
        assert np.array_equal(w.V[r].astype(np.uint64), e), f"v{r}: {lines[r - 3]}"
    assert np.array_equal(w.V[13], np.concatenate([a[:32], b[:32]])), "permlane32_swap vdst"
    assert np.array_equal(w.V[14], np.concatenate([a[32:], b[32:]])), "permlane32_swap vsrc"
    print("[ok] SDWA source selects (VGPR and SGPR sources), 16-bit integer ops, the "
          "three-input bit table and the half-wave swap match numpy", flush=True)


def main(argv):
    runtime_so = argv[0]
    names = argv[1:] or list(CASES)
    dev = Device(REPO, runtime_so, cu_count=8, group_filter=_merge_heads_only)
    failed = []
    for n in names:
        t0 = time.time()
        try:
            CASES[n](dev)
        except Exception:  # noqa: BLE001 -- every failure is printed and counted
            traceback.print_exc()
            failed.append(n)
        print(f"  -- {n}: {time.time() - t0:.1f} s", flush=True)
    print("FAILED " + " ".join(failed) if failed else "ALL PASSED", flush=True)
    return 1 if failed else 0


if __name__ == "__main__":
    sys.exit(main(sys.argv[1:]))
