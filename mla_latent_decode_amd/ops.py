"""ctypes binding of libqkmla.so for torch tensors.

Argument marshalling only: every step of the decode runs in the library's HIP
kernels.  Importing this module loads the library and raises if it has not
been built (python -m mla_latent_decode_amd.build); there is no fallback.

Function names and argument order follow include/qkmla.h.  Tensors must be
contiguous; device tensors must live on the current CUDA (HIP) device; work is
enqueued on torch's current stream.
"""
from __future__ import annotations

import ctypes
import dataclasses
import math
import os
from typing import Optional

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libqkmla.so")

QKMLA_F32, QKMLA_BF16 = 0, 1
QKMLA_DEV_BAD_SEQ_LEN, QKMLA_DEV_BAD_POSITION, QKMLA_DEV_BAD_PAGE = 1, 2, 4


class QkmlaError(RuntimeError):
    pass


class _Config(ctypes.Structure):
    _fields_ = [("n_heads", ctypes.c_int32), ("n_groups", ctypes.c_int32),
                ("latent_rank", ctypes.c_int32), ("head_dim", ctypes.c_int32),
                ("rope_dim", ctypes.c_int32), ("v_head_dim", ctypes.c_int32),
                ("dtype", ctypes.c_int32), ("qk_norm", ctypes.c_int32),
                ("eps", ctypes.c_float), ("softmax_scale", ctypes.c_float),
                ("rope_base", ctypes.c_float)]


class _Pages(ctypes.Structure):
    _fields_ = [("block_table", ctypes.c_void_p), ("max_blocks", ctypes.c_int32),
                ("page_size", ctypes.c_int32), ("num_pages", ctypes.c_int32)]


class _TrainInputs(ctypes.Structure):
    _fields_ = [(n, ctypes.c_void_p) for n in ("c", "q_c", "q_rope", "k_rope", "w_uk", "w_uv",
                                               "gamma_q", "gamma_k", "gamma_q_rope",
                                               "gamma_k_rope")]


TRAIN_GRAD_NAMES = ("d_c", "d_q_c", "d_q_rope", "d_k_rope", "d_w_uk", "d_w_uv", "d_gamma_q",
                    "d_gamma_k", "d_gamma_q_rope", "d_gamma_k_rope")


class _TrainGrads(ctypes.Structure):
    _fields_ = [(n, ctypes.c_void_p) for n in TRAIN_GRAD_NAMES]


def _load():
    if not os.path.exists(LIB_PATH):
        raise QkmlaError(f"{LIB_PATH} is missing: build it with "
                         "`python -m mla_latent_decode_amd.build` (no fallback path exists)")
    lib = ctypes.CDLL(LIB_PATH)
    P, I32, SZ = ctypes.c_void_p, ctypes.c_int32, ctypes.c_size_t
    C = ctypes.POINTER(_Config)
    PG = ctypes.POINTER(_Pages)
    sig = {
        "qkmla_absorb_weights": (I32, [C, P, P, P, P, P]),
        "qkmla_append": (I32, [C, I32, I32, P, P, P, P, P, I32, P, P, P, P, P]),
        "qkmla_decode_workspace_size": (SZ, [C, I32, I32]),
        "qkmla_decode": (I32, [C, I32, P, P, P, P, P, P, P, P, I32, I32, P, SZ, P, P, P, P]),
        "qkmla_decode_multi": (I32, [C, I32, I32, P, P, P, P, P, P, P, P, I32, I32, P, SZ, P, P,
                                     P, P]),
        "qkmla_decode_noalloc": (I32, [C, I32, P, P, P, P, P, P, P, P, I32, I32, P, P, P, P]),
        "qkmla_append_paged": (I32, [C, I32, I32, P, P, P, P, P, PG, P, P, P, P, P]),
        "qkmla_decode_paged": (I32, [C, I32, I32, P, P, P, P, P, P, P, P, PG, I32, P, SZ, P, P,
                                     P, P]),
        "qkmla_train_workspace_size": (SZ, [C, I32, I32]),
        "qkmla_train_forward": (I32, [C, I32, I32, ctypes.POINTER(_TrainInputs), P, SZ, P, P, P]),
        "qkmla_train_backward": (I32, [C, I32, I32, ctypes.POINTER(_TrainInputs), P, P, P, P, SZ,
                                       ctypes.POINTER(_TrainGrads), P]),
        "qkmla_train_workspace_size_varlen": (SZ, [C, I32, I32, I32]),
        "qkmla_train_forward_varlen": (I32, [C, I32, P, I32, I32, ctypes.POINTER(_TrainInputs), P,
                                             SZ, P, P, P, P]),
        "qkmla_train_backward_varlen": (I32, [C, I32, P, I32, I32, ctypes.POINTER(_TrainInputs),
                                              P, P, P, P, SZ, ctypes.POINTER(_TrainGrads), P, P]),
        "qkmla_out_proj": (I32, [C, I32, P, P, P, P]),
        "qkmla_plan": (I32, [C, I32, I32, I32, ctypes.POINTER(I32), ctypes.POINTER(I32)]),
        "qkmla_status_string": (ctypes.c_char_p, [ctypes.c_int]),
        "qkmla_last_error": (ctypes.c_char_p, []),
        "qkmla_abi_version": (ctypes.c_int, []),
        "qkmla_plan_segments": (I32, [I32, P, I32, I32, P, I32, ctypes.POINTER(I32)]),
        "qkmla_plan_merge_sources": (I32, [I32, P, I32, I32, I32, P, I32, ctypes.POINTER(I32)]),
        "qkmla_profile_begin": (I32, []),
        "qkmla_profile_begin_reps": (I32, [I32]),
        "qkmla_profile_end": (I32, [ctypes.POINTER(ctypes.c_double), ctypes.POINTER(I32)]),
        "qkmla_profile_end_detail": (I32, [ctypes.POINTER(ctypes.c_double), ctypes.POINTER(I32)]),
    }
    for name, (res, args) in sig.items():
        f = getattr(lib, name)
        f.restype, f.argtypes = res, args
    return lib


_lib = _load()


@dataclasses.dataclass(frozen=True)
class Config:
    """Mirror of qkmla_config."""
    n_heads: int
    n_groups: int
    latent_rank: int
    head_dim: int
    rope_dim: int
    v_head_dim: int
    dtype: str = "bf16"        # "bf16" or "f32"
    qk_norm: bool = True
    eps: float = 1e-6
    softmax_scale: float = 0.0  # <= 0: 1/sqrt(head_dim + rope_dim)
    rope_base: float = 10000.0

    @classmethod
    def from_shape(cls, shape, **kw):
        return cls(shape.n_heads, shape.n_groups, shape.latent_rank, shape.head_dim,
                   shape.rope_dim, shape.v_head_dim, shape.dtype, **kw)

    @property
    def torch_dtype(self):
        return torch.bfloat16 if self.dtype == "bf16" else torch.float32

    @property
    def tau(self) -> float:
        return self.softmax_scale if self.softmax_scale > 0 else 1.0 / math.sqrt(
            self.head_dim + self.rope_dim)

    def c(self) -> _Config:
        return _Config(self.n_heads, self.n_groups, self.latent_rank, self.head_dim,
                       self.rope_dim, self.v_head_dim,
                       QKMLA_BF16 if self.dtype == "bf16" else QKMLA_F32, int(self.qk_norm),
                       self.eps, self.softmax_scale, self.rope_base)


def _check(status: int, what: str):
    if status != 0:
        msg = _lib.qkmla_last_error().decode()
        raise QkmlaError(f"{what}: {_lib.qkmla_status_string(status).decode()}: {msg}")


def _ptr(t: Optional[torch.Tensor], shape=None, dtype=None, name="tensor"):
    """Device address of a contiguous tensor on the current GPU, after checking
    its dtype and shape (the library reads and writes exactly that extent)."""
    if t is None:
        return None
    if t.device.type != "cuda" or t.device.index != torch.cuda.current_device():
        raise QkmlaError(f"{name} must be a tensor on the current GPU, got {t.device}")
    if not t.is_contiguous():
        raise QkmlaError(f"{name} must be contiguous")
    if dtype is not None and t.dtype != dtype:
        raise QkmlaError(f"{name} must be {dtype}, got {t.dtype}")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise QkmlaError(f"{name} must have shape {tuple(shape)}, got {tuple(t.shape)}")
    return ctypes.c_void_p(t.data_ptr())


def _stream():
    return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)


def abi_version() -> int:
    return _lib.qkmla_abi_version()


def profile_begin(reps: int = 1):
    """Start recording HIP events around the q-prep, split-KV and merge
    launches of each decode call; with reps > 1 each kernel is launched reps
    times back to back between its events and the figures are per launch."""
    _check(_lib.qkmla_profile_begin_reps(int(reps)), "qkmla_profile_begin_reps")


def profile_end():
    """Stop recording; returns (summed split-KV kernel ms, decode calls)."""
    ms, n = ctypes.c_double(), ctypes.c_int32()
    _check(_lib.qkmla_profile_end(ctypes.byref(ms), ctypes.byref(n)), "qkmla_profile_end")
    return ms.value, n.value


def profile_end_detail():
    """Stop recording; returns ((q-prep ms, split-KV ms, merge ms) summed,
    decode calls)."""
    ms, n = (ctypes.c_double * 3)(), ctypes.c_int32()
    _check(_lib.qkmla_profile_end_detail(ms, ctypes.byref(n)), "qkmla_profile_end_detail")
    return (ms[0], ms[1], ms[2]), n.value


def plan(cfg: Config, batch: int, max_seq_len: int, n_cu: int):
    """Host-only planner: (decode workgroups, tile tokens)."""
    nwg, tile = ctypes.c_int32(), ctypes.c_int32()
    _check(_lib.qkmla_plan(ctypes.byref(cfg.c()), batch, max_seq_len, n_cu, ctypes.byref(nwg),
                           ctypes.byref(tile)), "qkmla_plan")
    return nwg.value, tile.value


def _host_i32(values):
    import numpy as np
    return np.ascontiguousarray(np.asarray(values, dtype=np.int32))


def plan_segments(seq_lens, cache_capacity: int, n_workgroups: int):
    """Host replay of the decode plan: array of rows (workgroup, sequence,
    first tile, end tile, kind) with kind -1 = whole sequence written directly,
    0/1 = partial in that workgroup slot."""
    import numpy as np
    lens = _host_i32(seq_lens)
    n = ctypes.c_int32()
    _check(_lib.qkmla_plan_segments(len(lens), lens.ctypes.data_as(ctypes.c_void_p), cache_capacity,
                                    n_workgroups, None, 0, ctypes.byref(n)), "qkmla_plan_segments")
    out = np.zeros((max(n.value, 1), 5), dtype=np.int32)
    _check(_lib.qkmla_plan_segments(len(lens), lens.ctypes.data_as(ctypes.c_void_p), cache_capacity,
                                    n_workgroups, out.ctypes.data_as(ctypes.c_void_p), n.value,
                                    ctypes.byref(n)), "qkmla_plan_segments")
    return out[:n.value]


def plan_merge_sources(seq_lens, cache_capacity: int, n_workgroups: int, b: int):
    """(workgroup, slot) pairs the merge reads for sequence b."""
    import numpy as np
    lens = _host_i32(seq_lens)
    n = ctypes.c_int32()
    cap = n_workgroups + 2
    out = np.zeros((cap, 2), dtype=np.int32)
    _check(_lib.qkmla_plan_merge_sources(len(lens), lens.ctypes.data_as(ctypes.c_void_p),
                                         cache_capacity, n_workgroups, b,
                                         out.ctypes.data_as(ctypes.c_void_p), cap, ctypes.byref(n)),
           "qkmla_plan_merge_sources")
    return out[:n.value]


def decode_workspace_size(cfg: Config, batch: int, max_seq_len: int) -> int:
    n = _lib.qkmla_decode_workspace_size(ctypes.byref(cfg.c()), batch, max_seq_len)
    if n == 0:
        raise QkmlaError("qkmla_decode_workspace_size: " + _lib.qkmla_last_error().decode())
    return n


def absorb_weights(cfg: Config, w_uk, gamma_q, gamma_k, out=None):
    G, r, dc = cfg.n_groups, cfg.latent_rank, cfg.head_dim
    if out is None:
        out = torch.empty((G, r, dc), dtype=cfg.torch_dtype, device=w_uk.device)
    _check(_lib.qkmla_absorb_weights(
        ctypes.byref(cfg.c()), _ptr(w_uk, (G, r, dc), torch.float32, "w_uk"),
        _ptr(gamma_q, (dc,), torch.float32, "gamma_q"), _ptr(gamma_k, (dc,), torch.float32, "gamma_k"),
        _ptr(out, (G, r, dc), cfg.torch_dtype, "w_qabs"), _stream()), "qkmla_absorb_weights")
    return out


def append(cfg: Config, c_new, k_rope_new, w_uk, gamma_k_rope, positions, latent_cache,
           rope_cache, alpha_cache=None, status=None):
    """c_new [B][n_new][r], k_rope_new [B][n_new][d_r], positions [B] int32 (device)."""
    B, n_new = c_new.shape[0], c_new.shape[1]
    L_cap = latent_cache.shape[1]
    dt = cfg.torch_dtype
    _check(_lib.qkmla_append(
        ctypes.byref(cfg.c()), B, n_new, _ptr(c_new, (B, n_new, cfg.latent_rank), dt, "c_new"),
        _ptr(k_rope_new, (B, n_new, cfg.rope_dim), dt, "k_rope_new"),
        _ptr(w_uk, (cfg.n_groups, cfg.latent_rank, cfg.head_dim), torch.float32, "w_uk"),
        _ptr(gamma_k_rope, (cfg.rope_dim,), torch.float32, "gamma_k_rope"),
        _ptr(positions, (B,), torch.int32, "positions"), L_cap,
        _ptr(latent_cache, (B, L_cap, cfg.latent_rank), dt, "latent_cache"),
        _ptr(rope_cache, (B, L_cap, cfg.rope_dim), dt, "rope_cache"),
        _ptr(alpha_cache, (B, L_cap, cfg.n_groups), torch.float32, "alpha_cache"),
        _ptr(status, (1,), torch.int32, "status"), _stream()), "qkmla_append")


def decode(cfg: Config, q_c, q_rope, w_qabs, gamma_q_rope, latent_cache, rope_cache, alpha_cache,
           seq_lens, max_seq_len: int, workspace, o_lat=None, lse=None, status=None):
    B = q_c.shape[0]
    L_cap = latent_cache.shape[1]
    H, r, dt = cfg.n_heads, cfg.latent_rank, cfg.torch_dtype
    if o_lat is None:
        o_lat = torch.empty((B, H, r), dtype=torch.float32, device=q_c.device)
    _check(_lib.qkmla_decode(
        ctypes.byref(cfg.c()), B, _ptr(q_c, (B, H, cfg.head_dim), dt, "q_c"),
        _ptr(q_rope, (B, H, cfg.rope_dim), dt, "q_rope"),
        _ptr(w_qabs, (cfg.n_groups, r, cfg.head_dim), dt, "w_qabs"),
        _ptr(gamma_q_rope, (cfg.rope_dim,), torch.float32, "gamma_q_rope"),
        _ptr(latent_cache, (B, L_cap, r), dt, "latent_cache"),
        _ptr(rope_cache, (B, L_cap, cfg.rope_dim), dt, "rope_cache"),
        _ptr(alpha_cache, (B, L_cap, cfg.n_groups), torch.float32, "alpha_cache"),
        _ptr(seq_lens, (B,), torch.int32, "seq_lens"), L_cap, max_seq_len,
        _ptr(workspace, (workspace.numel(),), torch.uint8, "workspace"), workspace.numel(),
        _ptr(o_lat, (B, H, r), torch.float32, "o_lat"),
        _ptr(lse, (B, H), torch.float32, "lse"), _ptr(status, (1,), torch.int32, "status"),
        _stream()), "qkmla_decode")
    return o_lat


def decode_noalloc(cfg: Config, q_c, q_rope, w_qabs, gamma_q_rope, latent_cache, rope_cache,
                   alpha_cache, seq_lens, max_seq_len: int, o_lat, lse=None, status=None):
    """qkmla_decode without a workspace argument (the library's per-GPU scratch
    array); o_lat must be given, so the call allocates nothing."""
    B = q_c.shape[0]
    L_cap = latent_cache.shape[1]
    H, r, dt = cfg.n_heads, cfg.latent_rank, cfg.torch_dtype
    _check(_lib.qkmla_decode_noalloc(
        ctypes.byref(cfg.c()), B, _ptr(q_c, (B, H, cfg.head_dim), dt, "q_c"),
        _ptr(q_rope, (B, H, cfg.rope_dim), dt, "q_rope"),
        _ptr(w_qabs, (cfg.n_groups, r, cfg.head_dim), dt, "w_qabs"),
        _ptr(gamma_q_rope, (cfg.rope_dim,), torch.float32, "gamma_q_rope"),
        _ptr(latent_cache, (B, L_cap, r), dt, "latent_cache"),
        _ptr(rope_cache, (B, L_cap, cfg.rope_dim), dt, "rope_cache"),
        _ptr(alpha_cache, (B, L_cap, cfg.n_groups), torch.float32, "alpha_cache"),
        _ptr(seq_lens, (B,), torch.int32, "seq_lens"), L_cap, max_seq_len,
        _ptr(o_lat, (B, H, r), torch.float32, "o_lat"),
        _ptr(lse, (B, H), torch.float32, "lse"), _ptr(status, (1,), torch.int32, "status"),
        _stream()), "qkmla_decode_noalloc")
    return o_lat


def decode_multi(cfg: Config, q_c, q_rope, w_qabs, gamma_q_rope, latent_cache, rope_cache,
                 alpha_cache, seq_lens, max_seq_len: int, workspace, o_lat=None, lse=None,
                 status=None):
    """s_q query rows per sequence: q_c [B][s_q][H][d_c], q_rope [B][s_q][H][d_r];
    row i is the token at position seq_lens[b] - s_q + i (causal).  Returns
    o_lat [B][s_q][H][r].  Workspace: decode_workspace_size(cfg, B * s_q, ...)."""
    B, s_q = q_c.shape[0], q_c.shape[1]
    L_cap = latent_cache.shape[1]
    H, r, dt = cfg.n_heads, cfg.latent_rank, cfg.torch_dtype
    if o_lat is None:
        o_lat = torch.empty((B, s_q, H, r), dtype=torch.float32, device=q_c.device)
    _check(_lib.qkmla_decode_multi(
        ctypes.byref(cfg.c()), B, s_q, _ptr(q_c, (B, s_q, H, cfg.head_dim), dt, "q_c"),
        _ptr(q_rope, (B, s_q, H, cfg.rope_dim), dt, "q_rope"),
        _ptr(w_qabs, (cfg.n_groups, r, cfg.head_dim), dt, "w_qabs"),
        _ptr(gamma_q_rope, (cfg.rope_dim,), torch.float32, "gamma_q_rope"),
        _ptr(latent_cache, (B, L_cap, r), dt, "latent_cache"),
        _ptr(rope_cache, (B, L_cap, cfg.rope_dim), dt, "rope_cache"),
        _ptr(alpha_cache, (B, L_cap, cfg.n_groups), torch.float32, "alpha_cache"),
        _ptr(seq_lens, (B,), torch.int32, "seq_lens"), L_cap, max_seq_len,
        _ptr(workspace, (workspace.numel(),), torch.uint8, "workspace"), workspace.numel(),
        _ptr(o_lat, (B, s_q, H, r), torch.float32, "o_lat"),
        _ptr(lse, (B, s_q, H), torch.float32, "lse"), _ptr(status, (1,), torch.int32, "status"),
        _stream()), "qkmla_decode_multi")
    return o_lat


def _pages(block_table, latent_pool):
    """qkmla_pages for a device block table [B][max_blocks] and a latent pool
    [num_pages][page_size][r]."""
    if block_table.dim() != 2:
        raise QkmlaError("block_table must be [B][max_blocks]")
    return _Pages(_ptr(block_table, None, torch.int32, "block_table"), block_table.shape[1],
                  latent_pool.shape[1], latent_pool.shape[0])


def append_paged(cfg: Config, c_new, k_rope_new, w_uk, gamma_k_rope, positions, block_table,
                 latent_pool, rope_pool, alpha_pool=None, status=None):
    """qkmla_append into paged pools: latent_pool [num_pages][page_size][r],
    rope_pool [num_pages][page_size][d_r], alpha_pool [num_pages][page_size][G],
    block_table [B][max_blocks] int32 (device)."""
    B, n_new = c_new.shape[0], c_new.shape[1]
    NP, PS = latent_pool.shape[0], latent_pool.shape[1]
    dt = cfg.torch_dtype
    pg = _pages(block_table, latent_pool)
    _check(_lib.qkmla_append_paged(
        ctypes.byref(cfg.c()), B, n_new, _ptr(c_new, (B, n_new, cfg.latent_rank), dt, "c_new"),
        _ptr(k_rope_new, (B, n_new, cfg.rope_dim), dt, "k_rope_new"),
        _ptr(w_uk, (cfg.n_groups, cfg.latent_rank, cfg.head_dim), torch.float32, "w_uk"),
        _ptr(gamma_k_rope, (cfg.rope_dim,), torch.float32, "gamma_k_rope"),
        _ptr(positions, (B,), torch.int32, "positions"), ctypes.byref(pg),
        _ptr(latent_pool, (NP, PS, cfg.latent_rank), dt, "latent_pool"),
        _ptr(rope_pool, (NP, PS, cfg.rope_dim), dt, "rope_pool"),
        _ptr(alpha_pool, (NP, PS, cfg.n_groups), torch.float32, "alpha_pool"),
        _ptr(status, (1,), torch.int32, "status"), _stream()), "qkmla_append_paged")


def decode_paged(cfg: Config, q_c, q_rope, w_qabs, gamma_q_rope, latent_pool, rope_pool,
                 alpha_pool, seq_lens, block_table, max_seq_len: int, workspace, o_lat=None,
                 lse=None, status=None):
    """qkmla_decode_paged: q_c [B][s_q][H][d_c], q_rope [B][s_q][H][d_r]; pools and
    block table as for append_paged.  Returns o_lat [B][s_q][H][r]."""
    B, s_q = q_c.shape[0], q_c.shape[1]
    NP, PS = latent_pool.shape[0], latent_pool.shape[1]
    H, r, dt = cfg.n_heads, cfg.latent_rank, cfg.torch_dtype
    if o_lat is None:
        o_lat = torch.empty((B, s_q, H, r), dtype=torch.float32, device=q_c.device)
    pg = _pages(block_table, latent_pool)
    _check(_lib.qkmla_decode_paged(
        ctypes.byref(cfg.c()), B, s_q, _ptr(q_c, (B, s_q, H, cfg.head_dim), dt, "q_c"),
        _ptr(q_rope, (B, s_q, H, cfg.rope_dim), dt, "q_rope"),
        _ptr(w_qabs, (cfg.n_groups, r, cfg.head_dim), dt, "w_qabs"),
        _ptr(gamma_q_rope, (cfg.rope_dim,), torch.float32, "gamma_q_rope"),
        _ptr(latent_pool, (NP, PS, r), dt, "latent_pool"),
        _ptr(rope_pool, (NP, PS, cfg.rope_dim), dt, "rope_pool"),
        _ptr(alpha_pool, (NP, PS, cfg.n_groups), torch.float32, "alpha_pool"),
        _ptr(seq_lens, (B,), torch.int32, "seq_lens"), ctypes.byref(pg), max_seq_len,
        _ptr(workspace, (workspace.numel(),), torch.uint8, "workspace"), workspace.numel(),
        _ptr(o_lat, (B, s_q, H, r), torch.float32, "o_lat"),
        _ptr(lse, (B, s_q, H), torch.float32, "lse"), _ptr(status, (1,), torch.int32, "status"),
        _stream()), "qkmla_decode_paged")
    return o_lat


def out_proj(cfg: Config, o_lat, w_uv, out=None):
    B, H = o_lat.shape[0], o_lat.shape[1]
    if out is None:
        out = torch.empty((B, H, cfg.v_head_dim), dtype=torch.float32, device=o_lat.device)
    _check(_lib.qkmla_out_proj(
        ctypes.byref(cfg.c()), B, _ptr(o_lat, (B, H, cfg.latent_rank), torch.float32, "o_lat"),
        _ptr(w_uv, (cfg.n_groups, cfg.latent_rank, cfg.v_head_dim), cfg.torch_dtype, "w_uv"),
        _ptr(out, (B, H, cfg.v_head_dim), torch.float32, "out"), _stream()), "qkmla_out_proj")
    return out


# --- training / prefill (explicit form) ---------------------------------------------------

def train_workspace_size(cfg: Config, batch: int, seq_len: int) -> int:
    n = _lib.qkmla_train_workspace_size(ctypes.byref(cfg.c()), batch, seq_len)
    if n == 0:
        raise QkmlaError("qkmla_train_workspace_size: " + _lib.qkmla_last_error().decode())
    return n


def _train_inputs(cfg: Config, t: dict, lead: tuple) -> _TrainInputs:
    """lead: the token dims, (B, T) or (total,) for packed sequences."""
    H, G, r, dc, dr, dv = (cfg.n_heads, cfg.n_groups, cfg.latent_rank, cfg.head_dim,
                           cfg.rope_dim, cfg.v_head_dim)
    dt, f32 = cfg.torch_dtype, torch.float32
    spec = {"c": (lead + (r,), dt), "q_c": (lead + (H, dc), dt), "q_rope": (lead + (H, dr), dt),
            "k_rope": (lead + (dr,), dt), "w_uk": ((G, r, dc), f32), "w_uv": ((G, r, dv), dt),
            "gamma_q": ((dc,), f32), "gamma_k": ((dc,), f32), "gamma_q_rope": ((dr,), f32),
            "gamma_k_rope": ((dr,), f32)}
    return _TrainInputs(*[_ptr(t.get(n), shp, dtp, n) for n, (shp, dtp) in spec.items()])


def train_forward(cfg: Config, inputs: dict, workspace, o=None, lse=None):
    """Causal explicit-form forward over inputs["c"] [B][T][r] etc. (dict of
    device tensors named as in qkmla_train_inputs).  Returns (o, lse)."""
    B, T = inputs["c"].shape[:2]
    H, dev = cfg.n_heads, inputs["c"].device
    if o is None:
        o = torch.empty((B, T, H, cfg.v_head_dim), dtype=torch.float32, device=dev)
    if lse is None:
        lse = torch.empty((B, T, H), dtype=torch.float32, device=dev)
    ins = _train_inputs(cfg, inputs, (B, T))
    _check(_lib.qkmla_train_forward(
        ctypes.byref(cfg.c()), B, T, ctypes.byref(ins),
        _ptr(workspace, (workspace.numel(),), torch.uint8, "workspace"), workspace.numel(),
        _ptr(o, (B, T, H, cfg.v_head_dim), torch.float32, "o"),
        _ptr(lse, (B, T, H), torch.float32, "lse"), _stream()), "qkmla_train_forward")
    return o, lse


def train_backward(cfg: Config, inputs: dict, o, lse, d_o, workspace, grads: Optional[dict] = None):
    """Gradients of sum(o * d_o) with respect to every input: dict
    d_<name> -> fp32 tensor of that input's shape."""
    B, T = inputs["c"].shape[:2]
    H, dev = cfg.n_heads, inputs["c"].device
    if grads is None:
        grads = {"d_" + n: torch.empty(tuple(inputs[n].shape), dtype=torch.float32, device=dev)
                 for n in ("c", "q_c", "q_rope", "k_rope", "w_uk", "w_uv", "gamma_q", "gamma_k",
                           "gamma_q_rope", "gamma_k_rope")}
    ins = _train_inputs(cfg, inputs, (B, T))
    gs = _TrainGrads(*[_ptr(grads[n], tuple(inputs[n[2:]].shape), torch.float32, n)
                       for n in TRAIN_GRAD_NAMES])
    _check(_lib.qkmla_train_backward(
        ctypes.byref(cfg.c()), B, T, ctypes.byref(ins),
        _ptr(o, (B, T, H, cfg.v_head_dim), torch.float32, "o"),
        _ptr(lse, (B, T, H), torch.float32, "lse"),
        _ptr(d_o, (B, T, H, cfg.v_head_dim), torch.float32, "d_o"),
        _ptr(workspace, (workspace.numel(),), torch.uint8, "workspace"), workspace.numel(), ctypes.byref(gs),
        _stream()), "qkmla_train_backward")
    return grads


def train_workspace_size_varlen(cfg: Config, n_seqs: int, total_tokens: int,
                                max_seq_len: int) -> int:
    n = _lib.qkmla_train_workspace_size_varlen(ctypes.byref(cfg.c()), n_seqs, total_tokens,
                                               max_seq_len)
    if n == 0:
        raise QkmlaError("qkmla_train_workspace_size_varlen: " + _lib.qkmla_last_error().decode())
    return n


def train_forward_varlen(cfg: Config, inputs: dict, cu_seqlens, max_seq_len: int, workspace,
                         o=None, lse=None, status=None):
    """Packed sequences: per-token inputs [total][...], cu_seqlens device int32
    [n_seqs + 1].  Returns (o [total][H][d_v], lse [total][H])."""
    total = inputs["c"].shape[0]
    n_seqs = cu_seqlens.numel() - 1
    H, dev = cfg.n_heads, inputs["c"].device
    if o is None:
        o = torch.empty((total, H, cfg.v_head_dim), dtype=torch.float32, device=dev)
    if lse is None:
        lse = torch.empty((total, H), dtype=torch.float32, device=dev)
    ins = _train_inputs(cfg, inputs, (total,))
    _check(_lib.qkmla_train_forward_varlen(
        ctypes.byref(cfg.c()), n_seqs, _ptr(cu_seqlens, (n_seqs + 1,), torch.int32, "cu_seqlens"), total,
        max_seq_len, ctypes.byref(ins), _ptr(workspace, (workspace.numel(),), torch.uint8, "workspace"),
        workspace.numel(), _ptr(o, (total, H, cfg.v_head_dim), torch.float32, "o"),
        _ptr(lse, (total, H), torch.float32, "lse"), _ptr(status, (1,), torch.int32, "status"),
        _stream()), "qkmla_train_forward_varlen")
    return o, lse


def train_backward_varlen(cfg: Config, inputs: dict, cu_seqlens, max_seq_len: int, o, lse, d_o,
                          workspace, grads: Optional[dict] = None, status=None):
    total = inputs["c"].shape[0]
    n_seqs = cu_seqlens.numel() - 1
    H, dev = cfg.n_heads, inputs["c"].device
    if grads is None:
        grads = {"d_" + n: torch.empty(tuple(inputs[n].shape), dtype=torch.float32, device=dev)
                 for n in ("c", "q_c", "q_rope", "k_rope", "w_uk", "w_uv", "gamma_q", "gamma_k",
                           "gamma_q_rope", "gamma_k_rope")}
    ins = _train_inputs(cfg, inputs, (total,))
    gs = _TrainGrads(*[_ptr(grads[n], tuple(inputs[n[2:]].shape), torch.float32, n)
                       for n in TRAIN_GRAD_NAMES])
    _check(_lib.qkmla_train_backward_varlen(
        ctypes.byref(cfg.c()), n_seqs, _ptr(cu_seqlens, (n_seqs + 1,), torch.int32, "cu_seqlens"), total,
        max_seq_len, ctypes.byref(ins), _ptr(o, (total, H, cfg.v_head_dim), torch.float32, "o"),
        _ptr(lse, (total, H), torch.float32, "lse"),
        _ptr(d_o, (total, H, cfg.v_head_dim), torch.float32, "d_o"),
        _ptr(workspace, (workspace.numel(),), torch.uint8, "workspace"), workspace.numel(), ctypes.byref(gs),
        _ptr(status, (1,), torch.int32, "status"), _stream()), "qkmla_train_backward_varlen")
    return grads
