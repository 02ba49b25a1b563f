#!/usr/bin/env python3
"""Benchmark of the QK-Normed MLA decode step on one MI355X.

One step = one qkmla_decode call (q-prep, split-KV decode, split merge) over
the latent + RoPE + alpha caches of every sequence; the workload that also
appends the new token in the step (batch 4 x 32k) includes that qkmla_append.
Inputs are resident in HBM before timing starts; caches are rotated over
enough copies that each step streams from HBM rather than the 256 MB
memory-side cache.

Steps are timed as HIP-graph replays of the captured step (one step per cache
copy), which keeps the host's launch overhead off the GPU timeline; each
replay is first checked bit for bit against the eager step, and eager timing
is used (and said) if capture fails or a replay differs.  The eager figures
are reported beside them.

Prints ONE JSON line: value = algorithmic cache bytes per step / step time
(GB/s) for the one-sequence 262 144-token workload (--workload picks
another), with microseconds per step, the overhead against the same kernels
with the normalisation compiled out (plain MLA), the split-KV kernel's
roofline position (its per-launch time from the library's HIP events, each
kernel launched several times back to back between them), the fp64 oracle
timed on the host, and the same figures for the 4k, 32k and ragged workloads
under "sweep".
Under "next_rows": bulk append, s_q = 2 decode, paged-cache decode and the
explicit-form training forward and backward, each timed on its own.

The default run takes the headline (with its sweep) and the next rows from two
child processes (``--part headline`` / ``--part next``, which also run alone,
e.g. under a profiler), so that a failure in a next-row measurement leaves
the headline standing; the parent process never touches the GPU.
"""
from __future__ import annotations

import argparse
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "decode µs/step + cache HBM GB/s at 4k–256k ctx; % overhead vs plain MLA"
HBM_PEAK_GBPS = 8000.0          # MI355X HBM3E
BF16_PEAK_TFLOPS = 2500.0       # MI355X dense bf16 MFMA
MALL_BYTES = 256 << 20
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "decode_splitkv_traffic.json")
KERNEL_SRC = os.path.join(ROOT, "mla_latent_decode_amd", "csrc", "decode_mfma.hip")


def _lengths(w):
    import numpy as np
    if w.lengths:
        return list(w.lengths)
    rng = np.random.default_rng(1000 + w.config_id)
    return [int(x) for x in rng.integers(w.ragged[0], w.ragged[1], size=w.batch, endpoint=True)]


class Bench:
    """Device state of one workload: weights, queries, rotated cache copies."""

    def __init__(self, cid: int):
        import torch
        from mla_latent_decode_amd import ops
        from mla_latent_decode_amd.inputs import WORKLOADS, device_cache_fill_source
        from mla_latent_decode_amd.layout import cache_bytes_per_token, decode_flops_per_token
        self.torch, self.ops = torch, ops
        w = WORKLOADS[cid]
        self.w, self.cid = w, cid
        s = w.shape
        self.lengths = _lengths(w)
        B, L_cap = len(self.lengths), max(self.lengths)
        self.B, self.L_cap = B, L_cap
        self.cfg = ops.Config.from_shape(s)
        self.cfg_plain = ops.Config.from_shape(s, qk_norm=False)
        dev = "cuda"
        g = torch.Generator(device=dev)
        g.manual_seed(2000 + cid)
        f32, dt = torch.float32, self.cfg.torch_dtype
        r, dr, G, H = s.latent_rank, s.rope_dim, s.n_groups, s.n_heads
        self.w_uk = (torch.randn((G, r, s.head_dim), generator=g, device=dev) / math.sqrt(r)).contiguous()
        self.gq = torch.rand((s.head_dim,), generator=g, device=dev) + 0.5
        self.gk = torch.rand((s.head_dim,), generator=g, device=dev) + 0.5
        self.gqr = torch.rand((dr,), generator=g, device=dev) + 0.5
        self.gkr = torch.rand((dr,), generator=g, device=dev) + 0.5
        self.w_qabs = ops.absorb_weights(self.cfg, self.w_uk, self.gq, self.gk)
        self.w_qabs_plain = ops.absorb_weights(self.cfg_plain, self.w_uk, self.gq, self.gk)
        self.q_c = torch.randn((B, H, s.head_dim), generator=g, device=dev).to(dt)
        self.q_rope = torch.randn((B, H, dr), generator=g, device=dev).to(dt)
        lat = torch.zeros((B, L_cap, r), dtype=dt, device=dev)
        rope = torch.zeros((B, L_cap, dr), dtype=dt, device=dev)
        alpha = torch.zeros((B, L_cap, G), dtype=f32, device=dev)
        self.status = torch.zeros((1,), dtype=torch.int32, device=dev)
        for b, start, c, k in device_cache_fill_source(s, self.lengths, 3000 + cid, dev,
                                                       w.row_scale_log10_clip):
            if b is None:
                pos = torch.full((B,), start, dtype=torch.int32, device=dev)
                ops.append(self.cfg, c, k, self.w_uk, self.gkr, pos, lat, rope, alpha, self.status)
            else:
                pos = torch.full((1,), start, dtype=torch.int32, device=dev)
                ops.append(self.cfg, c, k, self.w_uk, self.gkr, pos, lat[b:b + 1], rope[b:b + 1],
                           alpha[b:b + 1], self.status)
        torch.cuda.synchronize()
        self.cache_bytes = lat.numel() * lat.element_size() + rope.numel() * rope.element_size() + \
            alpha.numel() * 4
        n_copies = max(1, math.ceil(2 * MALL_BYTES / self.cache_bytes))
        self.copies = [(lat, rope, alpha)] + [(lat.clone(), rope.clone(), alpha.clone())
                                              for _ in range(n_copies - 1)]
        self.n_copies = n_copies
        self.seq_lens = torch.tensor(self.lengths, dtype=torch.int32, device=dev)
        ws = max(ops.decode_workspace_size(self.cfg, B, L_cap),
                 ops.decode_workspace_size(self.cfg_plain, B, L_cap))
        self.workspace = torch.empty((ws,), dtype=torch.uint8, device=dev)
        self.o_lat = torch.empty((B, H, r), dtype=f32, device=dev)
        self.lse = torch.empty((B, H), dtype=f32, device=dev)
        self.w_uv = (torch.randn((G, r, s.v_head_dim), generator=g, device=dev) / math.sqrt(r)).to(dt)
        self.o_out = torch.empty((B, H, s.v_head_dim), dtype=f32, device=dev)
        self.tokens = sum(self.lengths)
        self.bytes_qk = self.tokens * cache_bytes_per_token(s, True)
        self.bytes_plain = self.tokens * cache_bytes_per_token(s, False)
        self.flops = self.tokens * decode_flops_per_token(s)
        if w.append_last:
            self.step_c = torch.randn((B, 1, r), generator=g, device=dev).to(dt)
            self.step_k = torch.randn((B, 1, dr), generator=g, device=dev).to(dt)
            self.step_pos = torch.tensor([L - 1 for L in self.lengths], dtype=torch.int32, device=dev)
        self.i = 0

    def step(self, plain=False, rotate=True):
        ops = self.ops
        lat, rope, alpha = self.copies[self.i % self.n_copies if rotate else 0]
        self.i += 1
        cfg = self.cfg_plain if plain else self.cfg
        if self.w.append_last:
            ops.append(cfg, self.step_c, self.step_k, self.w_uk, self.gkr, self.step_pos, lat, rope,
                       alpha, self.status)
        ops.decode(cfg, self.q_c, self.q_rope, self.w_qabs_plain if plain else self.w_qabs, self.gqr,
                   lat, rope, alpha, self.seq_lens, self.L_cap, self.workspace, self.o_lat, self.lse,
                   self.status)

    def time_steps(self, steps, warmup, plain=False):
        torch = self.torch
        for _ in range(warmup):
            self.step(plain)
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        t0 = time.perf_counter()
        e0.record()
        for _ in range(steps):
            self.step(plain)
        e1.record()
        torch.cuda.synchronize()
        wall = time.perf_counter() - t0
        return e0.elapsed_time(e1) / steps, wall

    def time_steps_paired(self, steps, warmup, block=5):
        """Eager step times of QK-norm and plain MLA, taken in alternating
        blocks of `block` steps (HIP events around each block), so that both
        modes run under the same clock state: under sustained load the chip
        lowers its clock within a millisecond or two, and two back-to-back
        runs would compare a cool mode with a throttled one.  Returns
        (ms per QK-norm step, ms per plain step)."""
        torch = self.torch
        for _ in range(warmup):
            self.step()
            self.step(plain=True)
        torch.cuda.synchronize()
        n_blocks = max(1, -(-steps // block))
        ev = [[(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
               for _ in range(n_blocks)] for _ in range(2)]
        for k in range(n_blocks):
            for mode in (0, 1):
                e0, e1 = ev[mode][k]
                e0.record()
                for _ in range(block):
                    self.step(plain=bool(mode))
                e1.record()
        torch.cuda.synchronize()
        per = [sum(e0.elapsed_time(e1) for e0, e1 in ev[mode]) / (n_blocks * block)
               for mode in (0, 1)]
        return per[0], per[1]

    def step_spread(self, steps, rotate=True):
        """Per-step times (eager launches, a HIP event pair around each step):
        (p10, p50, p90) in ms.  rotate=False streams one cache copy every
        step, which the memory-side cache may then hold ("warm")."""
        torch = self.torch
        for _ in range(3):
            self.step(rotate=rotate)
        ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
              for _ in range(steps)]
        torch.cuda.synchronize()
        for e0, e1 in ev:
            e0.record()
            self.step(rotate=rotate)
            e1.record()
        torch.cuda.synchronize()
        t = sorted(e0.elapsed_time(e1) for e0, e1 in ev)
        pick = lambda q: t[min(len(t) - 1, int(q * (len(t) - 1) + 0.5))]
        return pick(0.1), pick(0.5), pick(0.9)

    def out_proj_ms(self, steps, per_graph=16):
        """qkmla_out_proj (the V up-projection) on this batch: a HIP graph of
        `per_graph` launches replayed `steps` times between HIP events, so that
        the host's launch cost (more than this short kernel's duration) does
        not enter the figure; the graph's output is checked bit for bit
        against an eager call first.  Falls back to eager launches if the
        capture fails."""
        torch = self.torch
        call = lambda: self.ops.out_proj(self.cfg, self.o_lat, self.w_uv, self.o_out)
        try:
            call()
            torch.cuda.synchronize()
            ref = self.o_out.clone()
            side = torch.cuda.Stream()
            side.wait_stream(torch.cuda.current_stream())
            with torch.cuda.stream(side):
                call()
            torch.cuda.current_stream().wait_stream(side)
            torch.cuda.synchronize()
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g):
                for _ in range(per_graph):
                    call()
            self.o_out.zero_()
            g.replay()
            torch.cuda.synchronize()
            if not torch.equal(self.o_out, ref):
                raise RuntimeError("graph output differs from the eager call")
        except Exception:  # capture unavailable: eager launches (host-bound)
            return _event_ms(torch, call, steps)
        return _event_ms(torch, g.replay, steps) / per_graph

    def _capture(self, plain):
        """One HIP graph of n_copies steps (one per cache copy), checked bit
        for bit against the eager step over three replays.  Returns
        (graph, None) or (None, reason)."""
        torch = self.torch
        try:
            self.i = self.n_copies - 1
            self.step(plain)
            torch.cuda.synchronize()
            ref_lat, ref_lse = self.o_lat.clone(), self.lse.clone()
            side = torch.cuda.Stream()
            side.wait_stream(torch.cuda.current_stream())
            with torch.cuda.stream(side):
                self.i = 0
                for _ in range(self.n_copies):
                    self.step(plain)
            torch.cuda.current_stream().wait_stream(side)
            torch.cuda.synchronize()
            g = torch.cuda.CUDAGraph()
            self.i = 0
            with torch.cuda.graph(g):
                for _ in range(self.n_copies):
                    self.step(plain)
            torch.cuda.synchronize()
            for _ in range(3):
                self.o_lat.fill_(float("nan"))
                self.lse.fill_(float("nan"))
                torch.cuda.synchronize()
                g.replay()
                torch.cuda.synchronize()
                if not (torch.equal(self.o_lat, ref_lat) and torch.equal(self.lse, ref_lse)):
                    return None, "a graph replay differs from the eager step"
            return g, None
        except Exception as ex:  # noqa: BLE001 -- reported in the JSON line, eager timing stands
            return None, f"graph capture failed: {type(ex).__name__}: {ex}"

    def graph_time_paired(self, steps):
        """Graph-replayed step times of QK-norm and plain MLA, replays of the
        two graphs alternating (HIP events around each replay), for the same
        reason as time_steps_paired.  Returns ((ms QK-norm, ms plain), None)
        or (None, reason)."""
        torch = self.torch
        gq, why = self._capture(False)
        if gq is None:
            return None, why
        gp, why = self._capture(True)
        if gp is None:
            return None, why
        reps = max(1, -(-steps // self.n_copies))
        for _ in range(2):
            gq.replay()
            gp.replay()
        ev = [[(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
               for _ in range(reps)] for _ in range(2)]
        torch.cuda.synchronize()
        for k in range(reps):
            for mode, g in ((0, gq), (1, gp)):
                e0, e1 = ev[mode][k]
                e0.record()
                g.replay()
                e1.record()
        torch.cuda.synchronize()
        per = [sum(e0.elapsed_time(e1) for e0, e1 in ev[mode]) / (reps * self.n_copies)
               for mode in (0, 1)]
        return (per[0], per[1]), None

    def kernel_ms(self, steps, plain=False):
        """Average duration of the split-KV kernel over `steps` steps (HIP events
        recorded by the library around each launch on the launch stream)."""
        return self.kernel_breakdown_ms(steps, plain)[1]

    def kernel_breakdown_paired(self, steps, reps=8, block=2):
        """kernel_breakdown_ms for QK-norm and plain MLA in alternating blocks
        of `block` decode calls, for the same reason as time_steps_paired.
        Returns ((q-prep, split-KV, merge) ms QK-norm, the same for plain)."""
        tot = [[0.0, 0.0, 0.0], [0.0, 0.0, 0.0]]
        cnt = [0, 0]
        for _ in range(max(1, -(-steps // block))):
            for mode in (0, 1):
                self.ops.profile_begin(reps)
                for _ in range(block):
                    self.step(plain=bool(mode))
                ms, n = self.ops.profile_end_detail()
                for j in range(3):
                    tot[mode][j] += ms[j]
                cnt[mode] += n
        return tuple(tuple(t / max(c, 1) for t in tot[m]) for m, c in zip((0, 1), cnt))

    def kernel_breakdown_ms(self, steps, plain=False, reps=8):
        """Average (q-prep, split-KV, merge) durations per launch over `steps`
        decode calls, from the library's HIP events on the launch stream, each
        kernel launched `reps` times back to back between its two events (the
        events' own latency, some microseconds, is spread over reps kernels;
        back-to-back kernels have no gap between them)."""
        self.ops.profile_begin(reps)
        for _ in range(steps):
            self.step(plain)
        ms, n = self.ops.profile_end_detail()
        return tuple(m / max(n, 1) for m in ms)


def _kernel_src_hash():
    import hashlib
    return hashlib.sha256(open(KERNEL_SRC, "rb").read()).hexdigest()[:16]


def _traffic(workload_name):
    """HBM bytes per launch of the split-KV kernel from committed rocprofv3 PMC
    counters, if they were taken on the current kernel source."""
    try:
        t = json.load(open(TRAFFIC_FILE))
    except (OSError, ValueError):
        return None
    e = t.get(workload_name)
    if not e or e.get("kernel_src_sha256_16") != _kernel_src_hash():
        return None
    return e.get("hbm_bytes_per_launch")


COPY_BYTES = 1 << 30  # the calibration copy: 1 GiB read, 1 GiB written


def pmc_workload(steps=5, cid=1):
    """What the two rocprofv3 --pmc runs (FETCH_SIZE, then WRITE_SIZE) count:
    `steps` headline decode steps over rotated cache copies, then three plain
    copies of COPY_BYTES (torch's copy kernel) to calibrate the counters.
    Prints one line naming the workload; no timing."""
    import torch
    b = Bench(cid)
    for _ in range(steps):
        b.step()
    torch.cuda.synchronize()
    src = torch.ones(COPY_BYTES // 4, dtype=torch.float32, device="cuda")
    dst = torch.empty_like(src)
    for _ in range(3):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"pmc_workload": b.w.name, "decode_steps": steps, "copy_bytes": COPY_BYTES,
                      "algorithmic_bytes_per_launch": b.bytes_qk}), flush=True)


def _pmc_dispatches(csv_path, counter):
    """[(dispatch id, kernel name, counter value)] in dispatch order from a
    rocprofv3 counter-collection CSV (columns Dispatch_Id, Kernel_Name,
    Counter_Name, Counter_Value; several rows of one dispatch are summed)."""
    import csv
    per = {}
    with open(csv_path, newline="") as f:
        for row in csv.DictReader(f):
            if row.get("Counter_Name", "").split("[")[0] != counter:
                continue
            key = (int(row.get("Dispatch_Id", "0") or 0), row["Kernel_Name"])
            per[key] = per.get(key, 0.0) + float(row["Counter_Value"])
    return [(d, name, v) for (d, name), v in sorted(per.items())]


def _pmc_per_dispatch(csv_path, counter):
    """{kernel name: [counter value of each dispatch, in dispatch order]}."""
    out = {}
    for _, name, v in _pmc_dispatches(csv_path, counter):
        out.setdefault(name, []).append(v)
    return out


def _is_qk_splitkv(name):
    """The QK-norm instantiation of the split-KV kernel, demangled or not."""
    return "decode_mfma_kernel" in name and ("<true" in name or "ILb1E" in name)


def traffic_from_pmc(fetch_csv, write_csv, workload, algorithmic_bytes):
    """HBM bytes per launch of the QK-norm split-KV kernel: its FETCH_SIZE and
    WRITE_SIZE (KiB per dispatch), each scaled by what the same counter reads
    for the plain copy of COPY_BYTES in the same run."""
    fetch_seq = _pmc_dispatches(fetch_csv, "FETCH_SIZE")
    write_seq = _pmc_dispatches(write_csv, "WRITE_SIZE")
    fetch, write = {}, {}
    for seq, d in ((fetch_seq, fetch), (write_seq, write)):
        for _, name, v in seq:
            d.setdefault(name, []).append(v)

    def pick(d, want, what):
        names = [k for k in d if want(k)]
        if len(names) != 1:
            raise ValueError(f"expected one {what} kernel, found {names}")
        return d[names[0]]
    # the calibration copies are the run's last three copy dispatches, whatever
    # kernel torch picks for them (the cache set-up before the decode steps
    # copies too, through other kernels and in other sizes)
    is_copy = lambda k: "copy" in k.lower() and "decode" not in k  # noqa: E731
    mean = lambda v: sum(v) / len(v)  # noqa: E731

    def calibration(seq, what):
        cps = [v for _, name, v in seq if is_copy(name)][-3:]
        if len(cps) != 3:
            raise ValueError(f"expected three calibration copies in the {what} run, found {len(cps)}")
        return mean(cps)
    f_dec, w_dec = mean(pick(fetch, _is_qk_splitkv, "split-KV")), mean(pick(write, _is_qk_splitkv, "split-KV"))
    f_cp, w_cp = calibration(fetch_seq, "FETCH_SIZE"), calibration(write_seq, "WRITE_SIZE")
    kf, kw = COPY_BYTES / (f_cp * 1024.0), COPY_BYTES / (w_cp * 1024.0)
    hbm = f_dec * 1024.0 * kf + w_dec * 1024.0 * kw
    return {workload: {"hbm_bytes_per_launch": round(hbm), "fetch_KiB": f_dec, "write_KiB": w_dec,
                       "copy_fetch_KiB": f_cp, "copy_write_KiB": w_cp,
                       "scale_fetch": kf, "scale_write": kw,
                       "algorithmic_bytes_per_launch": algorithmic_bytes,
                       "traffic_over_algorithmic": round(hbm / algorithmic_bytes, 4),
                       "kernel_src_sha256_16": _kernel_src_hash()}}


def measure(cid, steps, warmup, graph=True):
    b = Bench(cid)
    t0 = time.perf_counter()
    ms_eager, ms_plain_eager = b.time_steps_paired(steps, warmup)
    wall = time.perf_counter() - t0
    (qp_ms, k_ms, mg_ms), (_, k_ms_plain, _) = b.kernel_breakdown_paired(steps)
    p10, p50, p90 = b.step_spread(steps)
    w10, w50, w90 = b.step_spread(steps, rotate=False)
    op_ms = b.out_proj_ms(steps)
    if graph:
        g_pair, g_note = b.graph_time_paired(steps)
    else:
        g_pair, g_note = None, "not requested"
    g_ms, g_ms_plain = g_pair if g_pair else (None, None)
    use_graph = g_pair is not None
    ms_qk = g_ms if use_graph else ms_eager
    ms_plain = g_ms_plain if use_graph else ms_plain_eager
    us = ms_qk * 1e3
    res = {
        "workload": b.w.name,
        "batch": b.B,
        "context": b.lengths[0] if len(set(b.lengths)) == 1 else f"ragged sum={b.tokens}",
        "us_per_step": round(us, 2),
        "step_timing": "graph replay" if use_graph else "eager launches",
        "graph_note": None if use_graph else g_note,
        "us_per_step_eager": round(ms_eager * 1e3, 2),
        "us_per_step_eager_p10_p50_p90": [round(x * 1e3, 2) for x in (p10, p50, p90)],
        "warm_us_per_step_eager_p50": round(w50 * 1e3, 2),
        "out_proj_us": round(op_ms * 1e3, 2),
        "full_step_us": round((ms_qk + op_ms) * 1e3, 2),
        "plain_us_per_step": round(ms_plain * 1e3, 2),
        "plain_us_per_step_eager": round(ms_plain_eager * 1e3, 2),
        "overhead_vs_plain_pct": round(100.0 * (ms_qk / ms_plain - 1.0), 2),
        "cache_GBps": round(b.bytes_qk / (ms_qk * 1e-3) / 1e9, 1),
        "cache_frac_of_8TBps": round(b.bytes_qk / (ms_qk * 1e-3) / 1e9 / HBM_PEAK_GBPS, 4),
        "splitkv_kernel_us": round(k_ms * 1e3, 2),
        "splitkv_kernel_GBps": round(b.bytes_qk / (k_ms * 1e-3) / 1e9, 1),
        "qprep_kernel_us": round(qp_ms * 1e3, 2),
        "merge_kernel_us": round(mg_ms * 1e3, 2),
        "splitkv_kernel_plain_us": round(k_ms_plain * 1e3, 2),
        "splitkv_overhead_vs_plain_pct": round(100.0 * (k_ms / k_ms_plain - 1.0), 2),
        "mfma_TFLOPs": round(b.flops / (k_ms * 1e-3) / 1e12, 1),
        "cache_copies_rotated": b.n_copies,
    }
    status = int(b.status.item())
    if status:
        raise RuntimeError(f"device status {status} during the benchmark")
    return b, res, ms_qk, k_ms, wall


def read_probe(reps=10):
    """The read-stream peak this GPU reaches with a plain kernel: a
    float32-accumulated sum over 4 GiB of bf16 (every byte read once), and a
    1 GiB copy (read + write), both timed with HIP events."""
    import torch
    x = torch.ones((2 << 30,), dtype=torch.bfloat16, device="cuda")
    ms_sum = _event_ms(torch, lambda: torch.sum(x, dtype=torch.float32), reps)
    sum_gbps = x.numel() * 2 / (ms_sum * 1e-3) / 1e9
    del x
    a = torch.empty((1 << 30,), dtype=torch.uint8, device="cuda")
    c = torch.empty_like(a)
    ms_copy = _event_ms(torch, lambda: c.copy_(a), reps)
    copy_gbps = 2 * a.numel() / (ms_copy * 1e-3) / 1e9
    del a, c
    torch.cuda.empty_cache()
    return {"sum_read_GBps": round(sum_gbps, 1), "copy_read_write_GBps": round(copy_gbps, 1),
            "what": "torch sum over 4 GiB bf16 (fp32 accumulation); torch copy of 1 GiB"}


def _event_ms(torch, fn, reps, warmup=2):
    for _ in range(warmup):
        fn()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(reps):
        fn()
    e1.record()
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) / reps


def wg_sweep(b, steps, counts=(128, 256, 384, 512, 768)):
    """Split-KV kernel time (library event hook) for several workgroup counts
    of the plan (QKMLA_NUM_WG), each with a workspace sized for it."""
    from mla_latent_decode_amd import ops
    import torch
    res, keep = {}, b.workspace
    try:
        for n in counts:
            os.environ["QKMLA_NUM_WG"] = str(n)
            b.workspace = torch.empty((ops.decode_workspace_size(b.cfg, b.B, b.L_cap),),
                                      dtype=torch.uint8, device="cuda")
            for _ in range(3):
                b.step()
            k_ms = b.kernel_ms(steps)
            res[str(n)] = {"kernel_us": round(k_ms * 1e3, 2),
                           "GBps": round(b.bytes_qk / (k_ms * 1e-3) / 1e9, 1)}
    finally:
        os.environ.pop("QKMLA_NUM_WG", None)
        b.workspace = keep
    return res


def measure_next_rows(steps):
    """The rows beyond the decode step, each on the batch-16 x 4096 layer
    unless stated: bulk append of every cached token in one call, decode with
    s_q = 2 query rows per sequence, decode over 64-row pages of a shuffled
    pool, the explicit-form training forward and backward (1 x 1024 tokens)
    and a packed prefill forward (16 prompts of 256..2048 tokens).  Eager
    launches timed with HIP events; cache copies rotated as in the
    headline."""
    import torch
    from mla_latent_decode_amd import ops
    from mla_latent_decode_amd.layout import (append_bytes_per_token, cache_bytes_per_token,
                                              train_attention_flops)
    out = {}
    b = Bench(1)
    s, B, L, H = b.w.shape, b.B, b.L_cap, b.w.shape.n_heads
    r, dr, G, dt = s.latent_rank, s.rope_dim, s.n_groups, b.cfg.torch_dtype
    g = torch.Generator(device="cuda")
    g.manual_seed(5000)
    per_tok = cache_bytes_per_token(s, True)
    # N1: bulk append (all 16 x 4096 tokens in one call)
    c_new = torch.randn((B, L, r), generator=g, device="cuda").to(dt)
    k_new = torch.randn((B, L, dr), generator=g, device="cuda").to(dt)
    pos0 = torch.zeros((B,), dtype=torch.int32, device="cuda")
    lat, rope, alpha = b.copies[0]
    ms = _event_ms(torch, lambda: ops.append(b.cfg, c_new, k_new, b.w_uk, b.gkr, pos0, lat, rope,
                                             alpha, b.status), 3)
    out["bulk_append"] = {"tokens": B * L, "us": round(ms * 1e3, 1),
                          "Mtokens_per_s": round(B * L / (ms * 1e-3) / 1e6, 1),
                          "GBps": round(B * L * append_bytes_per_token(s) / (ms * 1e-3) / 1e9, 1)}
    _progress(out, "bulk_append")
    del c_new, k_new
    # N2: s_q = 2 rows per sequence (causal), over the rotated cache copies
    s_q = 2
    qc = torch.randn((B, s_q, H, s.head_dim), generator=g, device="cuda").to(dt)
    qr = torch.randn((B, s_q, H, dr), generator=g, device="cuda").to(dt)
    ws = torch.empty((ops.decode_workspace_size(b.cfg, B * s_q, L),), dtype=torch.uint8,
                     device="cuda")
    o2 = torch.empty((B, s_q, H, r), dtype=torch.float32, device="cuda")
    it = [0]

    def multi():
        la, ro, al = b.copies[it[0] % b.n_copies]
        it[0] += 1
        ops.decode_multi(b.cfg, qc, qr, b.w_qabs, b.gqr, la, ro, al, b.seq_lens, L, ws, o2,
                         status=b.status)
    ms = _event_ms(torch, multi, steps)
    rows_tokens = sum(sum(max(0, Lb - s_q + i + 1) for i in range(s_q)) for Lb in b.lengths)
    out["multi_query_s_q2"] = {"us_per_step": round(ms * 1e3, 2),
                               "cache_GBps_per_row": round(rows_tokens * per_tok / (ms * 1e-3) / 1e9, 1),
                               "note": "each query row streams its own causal prefix"}
    _progress(out, "multi_query_s_q2")
    del qc, qr, o2
    # N3: the same caches in 64-row pages of a shuffled pool (copies rotated)
    ps = 64
    nblk = L // ps
    pools = []
    gen = torch.Generator(device="cpu")
    gen.manual_seed(5001)
    for ci in range(b.n_copies):
        la, ro, al = b.copies[ci]
        perm = torch.randperm(B * nblk, generator=gen).to("cuda")
        table = perm.view(B, nblk).to(torch.int32).contiguous()
        plat = torch.empty((B * nblk, ps, r), dtype=dt, device="cuda")
        prope = torch.empty((B * nblk, ps, dr), dtype=dt, device="cuda")
        palpha = torch.empty((B * nblk, ps, G), dtype=torch.float32, device="cuda")
        plat[perm] = la.view(B * nblk, ps, r)
        prope[perm] = ro.view(B * nblk, ps, dr)
        palpha[perm] = al.view(B * nblk, ps, G)
        pools.append((table, plat, prope, palpha))
    o1 = torch.empty((B, 1, H, r), dtype=torch.float32, device="cuda")
    q1c, q1r = b.q_c.view(B, 1, H, -1), b.q_rope.view(B, 1, H, -1)

    def paged():
        t_, pl, pr, pa = pools[it[0] % len(pools)]
        it[0] += 1
        ops.decode_paged(b.cfg, q1c, q1r, b.w_qabs, b.gqr, pl, pr, pa, b.seq_lens, t_, L,
                         b.workspace, o1, status=b.status)
    ms_p = _event_ms(torch, paged, steps)
    ms_c, _ = b.time_steps(steps, 3)
    out["paged_64"] = {"us_per_step": round(ms_p * 1e3, 2),
                       "contiguous_us_per_step_eager": round(ms_c * 1e3, 2),
                       "cache_GBps": round(b.bytes_qk / (ms_p * 1e-3) / 1e9, 1)}
    _progress(out, "paged_64")
    status = int(b.status.item())
    del pools
    # split-KV workgroup count: the plan's default is one per CU
    out["splitkv_wg_sweep"] = {b.w.name: wg_sweep(b, steps)}
    del b
    torch.cuda.empty_cache()
    b3 = Bench(3)
    out["splitkv_wg_sweep"][b3.w.name] = wg_sweep(b3, max(5, steps // 2))
    _progress(out, "splitkv_wg_sweep")
    status |= int(b3.status.item())
    del b3
    torch.cuda.empty_cache()
    if status:
        raise RuntimeError(f"device status {status} in the next-row measurements")
    # N4: training forward and backward, DeepSeek-V3-like layer, 1 x 1024 tokens
    Bt, T = 1, 1024
    cfg = ops.Config.from_shape(s)
    shp = {"c": (Bt, T, r), "q_c": (Bt, T, H, s.head_dim), "q_rope": (Bt, T, H, dr),
           "k_rope": (Bt, T, dr), "w_uk": (G, r, s.head_dim), "w_uv": (G, r, s.v_head_dim),
           "gamma_q": (s.head_dim,), "gamma_k": (s.head_dim,), "gamma_q_rope": (dr,),
           "gamma_k_rope": (dr,)}
    ins = {}
    for n, sh in shp.items():
        x = torch.randn(sh, generator=g, device="cuda")
        if n.startswith("gamma"):
            x = x.abs() * 0.5 + 0.5
        elif n.startswith("w_"):
            x = x / math.sqrt(r)
        ins[n] = x if (n == "w_uk" or n.startswith("gamma")) else x.to(dt)
    wst = torch.empty((ops.train_workspace_size(cfg, Bt, T),), dtype=torch.uint8, device="cuda")
    o, lse = ops.train_forward(cfg, ins, wst)
    d_o = torch.randn(tuple(o.shape), generator=g, device="cuda")
    grads = ops.train_backward(cfg, ins, o, lse, d_o, wst)
    ms_f = _event_ms(torch, lambda: ops.train_forward(cfg, ins, wst, o, lse), 3, warmup=1)
    ms_b = _event_ms(torch, lambda: ops.train_backward(cfg, ins, o, lse, d_o, wst, grads), 3,
                     warmup=1)
    ff, fb = train_attention_flops(s, Bt, T)
    # packed prefill: 16 prompts of 256..2048 tokens, forward only
    import numpy as np
    lens = [int(x) for x in np.random.default_rng(5002).integers(256, 2048, size=16,
                                                                 endpoint=True)]
    total = sum(lens)
    cu = torch.tensor(np.concatenate([[0], np.cumsum(lens)]), dtype=torch.int32, device="cuda")
    pre = {n: (torch.randn((total,) + sh[2:], generator=g, device="cuda").to(dt)
               if n in ("c", "q_c", "q_rope", "k_rope") else ins[n]) for n, sh in shp.items()}
    wsv = torch.empty((ops.train_workspace_size_varlen(cfg, len(lens), total, max(lens)),),
                      dtype=torch.uint8, device="cuda")
    stv = torch.zeros((1,), dtype=torch.int32, device="cuda")
    ov, lv = ops.train_forward_varlen(cfg, pre, cu, max(lens), wsv, status=stv)
    ms_v = _event_ms(torch, lambda: ops.train_forward_varlen(cfg, pre, cu, max(lens), wsv, ov, lv,
                                                            stv), 3, warmup=1)
    pairs_flops = sum(2 * H * L * (L + 1) // 2 * (s.head_dim + dr + s.v_head_dim) for L in lens)
    out["prefill_packed_fwd"] = {"sequences": len(lens), "tokens": total, "ms": round(ms_v, 3),
                                 "Mtokens_per_s": round(total / (ms_v * 1e-3) / 1e6, 2),
                                 "attention_TFLOPs": round(pairs_flops / (ms_v * 1e-3) / 1e12, 2)}
    _progress(out, "prefill_packed_fwd")
    if int(stv.item()):
        raise RuntimeError(f"device status {int(stv.item())} in the packed prefill")
    del pre, wsv, ov, lv
    out["train_fwd_bwd"] = {"batch": Bt, "seq_len": T, "fwd_ms": round(ms_f, 3),
                            "bwd_ms": round(ms_b, 3),
                            "fwd_attention_TFLOPs": round(ff / (ms_f * 1e-3) / 1e12, 2),
                            "bwd_attention_TFLOPs": round(fb / (ms_b * 1e-3) / 1e12, 2),
                            "kernels": "MFMA attention and projection GEMMs (bf16 operands), row-parallel norms"}
    _progress(out, "train_fwd_bwd")
    return out


def _progress(out, name):
    print(f"[bench] {name} {out[name]}", file=sys.stderr, flush=True)


def cpu_baseline(cid, budget_s=15.0, max_rounds=64):
    """The fp64 oracle on the host: the workload's sequences, whole, one at a
    time with fresh seeds (going round the workload again when it has fewer
    sequences than the budget takes), until about `budget_s` seconds of oracle
    decode time; returns its cache GB/s."""
    import numpy as np
    from threadpoolctl import threadpool_info

    import oracle
    from mla_latent_decode_amd.inputs import WORKLOADS, make_inputs
    from mla_latent_decode_amd.layout import cache_bytes_per_token
    w = WORKLOADS[cid]
    lengths = _lengths(w)
    done_tokens, elapsed, n, t_alpha = 0, 0.0, 0, 0.0
    for i in range(max_rounds):
        L = lengths[i % len(lengths)]
        inp = make_inputs(w.shape, [L], seed=4000 + i, row_scale_log10_clip=w.row_scale_log10_clip)
        t0 = time.perf_counter()
        oracle.explicit_decode(inp.q_c, inp.q_rope, inp.latents, inp.k_rope_raw, inp.w_uk, inp.w_uv,
                               inp.gamma_q, inp.gamma_k, inp.gamma_q_rope, inp.gamma_k_rope)
        elapsed += time.perf_counter() - t0
        # the alpha / RoPE-key part (what qkmla_append computes), timed on its own
        t0 = time.perf_counter()
        oracle.append_ref(inp.latents[0], inp.k_rope_raw[0], np.arange(L), inp.w_uk,
                          inp.gamma_k_rope, 1e-6, 10000.0)
        t_alpha += time.perf_counter() - t0
        done_tokens += L
        n += 1
        if elapsed >= budget_s:
            break
    info = threadpool_info()
    threads = max([p.get("num_threads", 1) for p in info] + [1])
    blas = sorted({f"{p.get('internal_api')} {p.get('version')}" for p in info
                   if p.get("user_api") == "blas"})
    cpu = "unknown"
    try:
        cpu = next(ln.split(":", 1)[1].strip() for ln in open("/proc/cpuinfo")
                   if ln.startswith("model name"))
    except (OSError, StopIteration):
        pass
    gbps = done_tokens * cache_bytes_per_token(w.shape, True) / elapsed / 1e9
    return {"value": round(gbps, 4), "unit": "GB/s", "cores": threads, "kind": "oracle",
            "sample": f"{n} whole sequences of the workload's {len(lengths)} (fresh seeds; "
                      f"{done_tokens} cached tokens), fp64 explicit form, {elapsed:.1f} s",
            "us_per_step_extrapolated": round(elapsed / done_tokens * sum(lengths) * 1e6, 1),
            "alpha_append_us_per_step_extrapolated":
                round(t_alpha / done_tokens * sum(lengths) * 1e6, 1),
            "affinity_cpus": len(os.sched_getaffinity(0)), "cpu_model": cpu, "blas": blas}


def main():
    ap = argparse.ArgumentParser(description=__doc__.splitlines()[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", type=int, default=3, help="headline workload (1-4)")
    ap.add_argument("--no-sweep", action="store_true")
    ap.add_argument("--no-cpu", action="store_true")
    ap.add_argument("--no-next", action="store_true",
                    help="skip the bulk-append, s_q=2, paged and training measurements")
    ap.add_argument("--no-graph", action="store_true",
                    help="time eager launches only (no HIP-graph replay of the step)")
    ap.add_argument("--pmc-workload", action="store_true",
                    help="run only what the rocprofv3 --pmc passes count (decode steps and a "
                         "calibration copy)")
    ap.add_argument("--traffic", nargs=3, metavar=("FETCH_CSV", "WRITE_CSV", "ALGO_BYTES"),
                    help="write the split-KV kernel's HBM traffic from two --pmc runs' CSVs "
                         "into profiles/decode_splitkv_traffic.json (no GPU needed)")
    ap.add_argument("--part", choices=("all", "headline", "next"), default="all",
                    help="all: run the headline (with its sweep) and the next-row measurements "
                         "each in a child process and print the combined line; headline / next: "
                         "run only that part in this process and print its JSON")
    args = ap.parse_args()
    if args.traffic:
        from mla_latent_decode_amd.inputs import WORKLOADS
        t = traffic_from_pmc(args.traffic[0], args.traffic[1], WORKLOADS[args.workload].name,
                             int(args.traffic[2]))
        try:
            prev = json.load(open(TRAFFIC_FILE))
        except (OSError, ValueError):
            prev = {}
        prev.update(t)
        json.dump(prev, open(TRAFFIC_FILE, "w"), indent=1)
        print(json.dumps(t))
        return
    if args.gpus != 1:
        print(f"bench.py measures one GPU only; --gpus {args.gpus} is not supported "
              "(the decode path is a single-GPU kernel library)", file=sys.stderr)
        sys.exit(2)
    if args.part == "all" and not args.pmc_workload:
        run_parts(args)
        return
    import torch
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(2)
    if args.pmc_workload:
        pmc_workload(cid=args.workload)
        return
    if args.part == "next":
        try:
            nxt = measure_next_rows(max(10, args.steps // 2))
        except Exception as ex:  # noqa: BLE001 -- reported in the JSON line
            nxt = {"error": f"{type(ex).__name__}: {ex}"}
        print(json.dumps({"next_rows": nxt}), flush=True)
        return
    b, res, ms_qk, k_ms, _ = measure(args.workload, args.steps, args.warmup, not args.no_graph)
    print(f"[bench] headline {res}", file=sys.stderr, flush=True)
    achieved = b.bytes_qk / (k_ms * 1e-3) / 1e9
    line = {
        "metric": METRIC,
        "value": res["cache_GBps"],
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_qk, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": res["workload"], "batch": b.B, "context": res["context"],
                   "heads": b.w.shape.n_heads, "kv_groups": b.w.shape.n_groups,
                   "latent_rank": b.w.shape.latent_rank, "rope_dim": b.w.shape.rope_dim,
                   "caches": "bf16 latent + bf16 rope + fp32 alpha", "parallelism": "single GPU"},
        "us_per_step": res["us_per_step"],
        "plain_us_per_step": res["plain_us_per_step"],
        "overhead_vs_plain_pct": res["overhead_vs_plain_pct"],
        "roofline": {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBPS,
                     "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBPS, 4),
                     "traffic": _traffic(res["workload"]),
                     "kernel": "decode_mfma_kernel<true,4> (split-KV)",
                     "kernel_us": res["splitkv_kernel_us"],
                     "algorithmic_bytes_per_launch": b.bytes_qk,
                     "mfma_TFLOPs": res["mfma_TFLOPs"],
                     "mfma_frac": round(res["mfma_TFLOPs"] / BF16_PEAK_TFLOPS, 4)},
        "headline": res,
    }
    del b
    torch.cuda.empty_cache()
    probe = read_probe()
    line["read_probe"] = probe
    line["roofline"]["frac_of_read_probe"] = round(achieved / probe["sum_read_GBps"], 4)
    print(f"[bench] read probe {probe}", file=sys.stderr, flush=True)
    if not args.no_sweep:
        sweep = []
        for cid in (1, 2, 3, 4):
            if cid == args.workload:
                continue
            _b, r, *_ = measure(cid, max(10, args.steps // 2), max(3, args.warmup // 2),
                                not args.no_graph)
            print(f"[bench] sweep {r}", file=sys.stderr, flush=True)
            sweep.append(r)
            del _b
            torch.cuda.empty_cache()
        line["sweep"] = sweep
        # mean QK-norm overhead over the 4k, 32k and 256k workloads
        from mla_latent_decode_amd.inputs import WORKLOADS
        over = [r["overhead_vs_plain_pct"] for r in [res] + sweep
                if r["workload"] in {WORKLOADS[c].name for c in (1, 2, 3)}]
        if len(over) == 3:
            line["overhead_vs_plain_pct_mean_4k_32k_256k"] = round(sum(over) / 3, 2)
    print(json.dumps(line), flush=True)


def _run_child(part, args, timeout_s):
    """Run one part of the benchmark in a child process.  Its stderr (the
    progress lines) passes through; its last JSON line on stdout is the
    result.  Returns (result or None, error text)."""
    import subprocess
    cmd = [sys.executable, os.path.abspath(__file__), "--part", part, "--steps", str(args.steps),
           "--warmup", str(args.warmup), "--workload", str(args.workload)]
    if args.no_sweep:
        cmd.append("--no-sweep")
    if args.no_graph:
        cmd.append("--no-graph")
    try:
        p = subprocess.run(cmd, stdout=subprocess.PIPE, text=True, timeout=timeout_s)
    except subprocess.TimeoutExpired:
        return None, f"the {part} part did not finish within {timeout_s} s"
    lines = [ln for ln in p.stdout.splitlines() if ln.startswith("{")]
    if p.returncode != 0 or not lines:
        return None, f"the {part} part exited with status {p.returncode}"
    return json.loads(lines[-1]), None


def run_parts(args):
    """The default run.  The headline (and its sweep) and the next-row
    measurements each run in a child process, so that a failure in one of the
    next rows cannot take the headline with it; this process never touches
    the GPU and adds the host baseline."""
    line, err = _run_child("headline", args, 900)
    if line is None:
        print(f"bench.py: {err}", file=sys.stderr)
        sys.exit(1)
    if not args.no_next:
        nxt, err = _run_child("next", args, 900)
        line["next_rows"] = nxt["next_rows"] if nxt else {"error": err}
        print(f"[bench] next rows {line['next_rows']}", file=sys.stderr, flush=True)
    if not args.no_cpu:
        line["cpu_baseline"] = cpu_baseline(args.workload)
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
