"""Device-side decode session: weights, the three caches and a workspace, all
held as torch tensors on one GPU, driven through the C ABI in ops.py.

The caches are filled with qkmla_append, so the alpha and RoPE caches the
decode reads are the library's own.  Host numpy inputs come from
mla_latent_decode_amd.inputs.
"""
from __future__ import annotations

from typing import Optional

import numpy as np
import torch

from . import ops
from .inputs import Inputs


def _dev(x: np.ndarray, dtype, device) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(x)).to(device=device, dtype=dtype)


class DecodeSession:
    """One decode layer for one batch of sequences.

    ``hold_last`` keeps the last token of every sequence out of the initial
    fill so that the decode step can append it itself (step_append)."""

    def __init__(self, cfg: ops.Config, inp: Inputs, *, device="cuda", L_cap: Optional[int] = None,
                 hold_last: bool = False, fill_chunk: int = 65536):
        self.cfg, self.inp, self.device = cfg, inp, device
        dt = cfg.torch_dtype
        B = len(inp.lengths)
        self.B = B
        self.lengths = list(inp.lengths)
        self.max_len = max(self.lengths) if self.lengths else 1
        self.L_cap = L_cap or self.max_len
        f32 = torch.float32
        self.w_uk = _dev(inp.w_uk, f32, device)
        self.w_uv = _dev(inp.w_uv, dt, device)
        self.gamma_q = _dev(inp.gamma_q, f32, device)
        self.gamma_k = _dev(inp.gamma_k, f32, device)
        self.gamma_q_rope = _dev(inp.gamma_q_rope, f32, device)
        self.gamma_k_rope = _dev(inp.gamma_k_rope, f32, device)
        self.w_qabs = ops.absorb_weights(cfg, self.w_uk, self.gamma_q, self.gamma_k)
        r, dr, G = cfg.latent_rank, cfg.rope_dim, cfg.n_groups
        self.lat = torch.zeros((B, self.L_cap, r), dtype=dt, device=device)
        self.rope = torch.zeros((B, self.L_cap, dr), dtype=dt, device=device)
        self.alpha = torch.zeros((B, self.L_cap, G), dtype=f32, device=device)
        self.status = torch.zeros((1,), dtype=torch.int32, device=device)
        self.q_c = _dev(inp.q_c, dt, device)
        self.q_rope = _dev(inp.q_rope, dt, device)
        self.hold_last = hold_last
        fill = [L - 1 if hold_last else L for L in self.lengths]
        self._fill(fill, fill_chunk)
        self.seq_lens = torch.tensor(self.lengths, dtype=torch.int32, device=device)
        if hold_last:
            self.step_c = _dev(np.stack([c[-1:] for c in inp.latents]), dt, device)
            self.step_kr = _dev(np.stack([k[-1:] for k in inp.k_rope_raw]), dt, device)
            self.step_pos = torch.tensor(fill, dtype=torch.int32, device=device)
        ws = ops.decode_workspace_size(cfg, B, self.max_len)
        self.workspace = torch.empty((ws,), dtype=torch.uint8, device=device)
        self.o_lat = torch.empty((B, cfg.n_heads, r), dtype=f32, device=device)
        self.lse = torch.empty((B, cfg.n_heads), dtype=f32, device=device)

    def _fill(self, fill, chunk):
        cfg, inp, dt = self.cfg, self.inp, self.cfg.torch_dtype
        uniform = len(set(fill)) == 1
        if uniform and fill[0] > 0:
            n = fill[0]
            for s in range(0, n, chunk):
                e = min(n, s + chunk)
                c = _dev(np.stack([x[s:e] for x in inp.latents]), dt, self.device)
                k = _dev(np.stack([x[s:e] for x in inp.k_rope_raw]), dt, self.device)
                pos = torch.full((self.B,), s, dtype=torch.int32, device=self.device)
                ops.append(cfg, c, k, self.w_uk, self.gamma_k_rope, pos, self.lat, self.rope,
                           self.alpha, self.status)
            return
        for b, n in enumerate(fill):
            for s in range(0, n, chunk):
                e = min(n, s + chunk)
                c = _dev(inp.latents[b][s:e][None], dt, self.device)
                k = _dev(inp.k_rope_raw[b][s:e][None], dt, self.device)
                pos = torch.full((1,), s, dtype=torch.int32, device=self.device)
                ops.append(cfg, c, k, self.w_uk, self.gamma_k_rope, pos, self.lat[b:b + 1],
                           self.rope[b:b + 1], self.alpha[b:b + 1], self.status)

    def step_append(self):
        """Append the held-back last token of every sequence (the decode step's append)."""
        ops.append(self.cfg, self.step_c, self.step_kr, self.w_uk, self.gamma_k_rope,
                   self.step_pos, self.lat, self.rope, self.alpha, self.status)

    def decode(self, lat=None, rope=None, alpha=None):
        ops.decode(self.cfg, self.q_c, self.q_rope, self.w_qabs, self.gamma_q_rope,
                   self.lat if lat is None else lat, self.rope if rope is None else rope,
                   self.alpha if alpha is None else alpha, self.seq_lens, self.max_len,
                   self.workspace, self.o_lat, self.lse, self.status)
        return self.o_lat, self.lse

    def out_proj(self, o_lat=None):
        return ops.out_proj(self.cfg, self.o_lat if o_lat is None else o_lat, self.w_uv)
