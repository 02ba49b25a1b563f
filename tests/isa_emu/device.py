"""The emulated device: the library's real host code over the runtime stand-in,
numpy arrays as device memory, and a driver for the four C-ABI calls.

Must run in a process that has not loaded the real HIP runtime (no torch):
the stand-in takes its place by soname.
"""
from __future__ import annotations

import ctypes
import glob
import os
import subprocess
import time
from typing import Optional

import numpy as np

from .asm import load_kernels
from .machine import Emulator, EmuError, Memory

HERE = os.path.dirname(os.path.abspath(__file__))
LAUNCH_CB = ctypes.CFUNCTYPE(ctypes.c_int, ctypes.c_char_p, ctypes.c_uint32, ctypes.c_uint32,
                             ctypes.c_uint32, ctypes.c_uint32, ctypes.c_uint32, ctypes.c_uint32,
                             ctypes.c_size_t, ctypes.POINTER(ctypes.c_void_p), ctypes.c_void_p)


def build_runtime(out_dir: str) -> str:
    """Compile the runtime stand-in; returns the path of libamdhip64.so.7."""
    os.makedirs(out_dir, exist_ok=True)
    out = os.path.join(out_dir, "libamdhip64.so.7")
    subprocess.run(["gcc", "-O2", "-shared", "-fPIC",
                    "-Wl,--version-script=" + os.path.join(HERE, "runtime.map"),
                    "-Wl,-soname,libamdhip64.so.7", os.path.join(HERE, "runtime.c"), "-o", out],
                   check=True)
    return out


# gfx950 limits a launch must respect, or the runtime rejects it
GFX950_LDS_BYTES = 160 * 1024      # LDS per workgroup (static + dynamic)
GFX950_REGS_PER_SIMD_LANE = 512    # unified VGPR + AGPR file, per lane of a SIMD
GFX950_SIMDS_PER_CU = 4


def check_launch_fits(name, md, static_lds, grid, block, dyn_lds):
    """Raise EmuError for a launch configuration that the device would refuse:
    a workgroup above the kernel's compiled maximum size, more LDS than a
    workgroup can have, registers that do not fit one CU, or grid dimensions
    out of range.  The emulator itself would run such a launch."""
    short = name[:60]
    threads = block[0] * block[1] * block[2]
    if min(block) < 1 or min(grid) < 1:
        raise EmuError(f"{short}: empty grid {grid} or block {block}")
    if grid[0] >= 2 ** 31 or grid[1] > 65535 or grid[2] > 65535:
        raise EmuError(f"{short}: grid {grid} out of range")
    maxw = md.get(".max_flat_workgroup_size", 1024)
    if threads > maxw:
        raise EmuError(f"{short}: block of {threads} threads above the compiled maximum {maxw}")
    if static_lds + dyn_lds > GFX950_LDS_BYTES:
        raise EmuError(f"{short}: {static_lds} + {dyn_lds} B of LDS above {GFX950_LDS_BYTES}")
    waves = -(-threads // 64)
    per_simd = -(-waves // GFX950_SIMDS_PER_CU)
    vg = md.get(".vgpr_count", 0)
    if per_simd * vg > GFX950_REGS_PER_SIMD_LANE:
        raise EmuError(f"{short}: {waves} waves of {vg} registers do not fit one CU")

class Device:
    def __init__(self, repo: str, runtime_so: str, cu_count: int = 8, verbose: bool = False,
                 group_filter=None):
        self.hip = ctypes.CDLL(runtime_so, mode=ctypes.RTLD_GLOBAL)
        lib_path = os.path.join(repo, "mla_latent_decode_amd", "libqkmla.so")
        asm = sorted(glob.glob(os.path.join(repo, "mla_latent_decode_amd", "_build",
                                            "*-gfx950.s")))
        if not asm:
            raise FileNotFoundError("no device assembly next to the library; build it first")
        newest_asm = max(os.path.getmtime(a) for a in asm)
        if os.path.getmtime(lib_path) + 1 < newest_asm:
            raise RuntimeError("device assembly is newer than the library; rebuild")
        self.lib = ctypes.CDLL(lib_path)
        self.hip.emu_set_cu_count(cu_count)
        self.hip.emu_var_info.argtypes = [ctypes.c_int, ctypes.POINTER(ctypes.c_char_p),
                                          ctypes.POINTER(ctypes.c_void_p),
                                          ctypes.POINTER(ctypes.c_size_t)]
        self.mem = Memory()
        self.emu = Emulator(self.mem)
        self.kernels = {}
        for a in asm:
            self.kernels.update(load_kernels(a))
        self._keep = []
        self.verbose = verbose
        self.launches = []
        self.error: Optional[BaseException] = None
        self.group_filter = group_filter
        self._cb = LAUNCH_CB(self._launch)
        self.hip.emu_set_launch_callback(self._cb)

    # -- memory --------------------------------------------------------------
    def alloc(self, nbytes: int, name: str) -> np.ndarray:
        raw = np.zeros(nbytes + 512, np.uint8)
        off = (-raw.ctypes.data) % 256
        buf = raw[off:off + nbytes]
        self._keep.append(raw)
        if nbytes:
            self.mem.add(buf.ctypes.data, nbytes, name, buf)
        return buf

    def put(self, x: np.ndarray, name: str) -> np.ndarray:
        x = np.ascontiguousarray(x)
        b = self.alloc(x.nbytes, name)
        b[:] = x.view(np.uint8).reshape(-1)
        return b.view(x.dtype).reshape(x.shape)

    def empty(self, shape, dtype, name: str, fill: Optional[int] = None) -> np.ndarray:
        b = self.alloc(int(np.prod(shape)) * np.dtype(dtype).itemsize, name)
        if fill is not None:
            b[:] = fill
        return b.view(dtype).reshape(shape)

    def _refresh_vars(self):
        for i in range(self.hip.emu_var_count()):
            nm, dv, sz = ctypes.c_char_p(), ctypes.c_void_p(), ctypes.c_size_t()
            self.hip.emu_var_info(i, ctypes.byref(nm), ctypes.byref(dv), ctypes.byref(sz))
            if dv.value and dv.value not in self.mem.allocs:
                self.mem.add(dv.value, sz.value, "device variable " + nm.value.decode())

    # -- launches ------------------------------------------------------------
    def _launch(self, name, gx, gy, gz, bx, by, bz, shmem, args, stream):
        name = name.decode()
        try:
            self._refresh_vars()
            k = self.kernels[name]
            md = k.md
            check_launch_fits(name, md, k.lds_bytes, (gx, gy, gz), (bx, by, bz), shmem)
            ksz = md[".kernarg_segment_size"]
            # the runtime pads the argument segment; kernels may load past its end
            kab = self.alloc(((ksz + 63) // 64) * 64 + 64, "kernel arguments of " + name[:40])
            hidden = {
                "hidden_block_count_x": gx, "hidden_block_count_y": gy, "hidden_block_count_z": gz,
                "hidden_group_size_x": bx, "hidden_group_size_y": by, "hidden_group_size_z": bz,
                "hidden_grid_dims": 1 + (gy > 1 or gz > 1) + (gz > 1),
                "hidden_dynamic_lds_size": shmem,
            }
            ai = 0
            for a in md[".args"]:
                off, sz, kind = a[".offset"], a[".size"], a[".value_kind"]
                if kind.startswith("hidden"):
                    v = hidden.get(kind, 0)
                    kab[off:off + sz] = np.frombuffer(int(v).to_bytes(8, "little")[:sz], np.uint8)
                    continue
                src = ctypes.cast(args[ai], ctypes.POINTER(ctypes.c_uint8 * sz)).contents
                kab[off:off + sz] = np.frombuffer(bytes(src), np.uint8)
                ai += 1
            groups = self.group_filter(name, (gx, gy, gz)) if self.group_filter else None
            t0, n0, d0 = time.time(), self.emu.stats.insts, self.emu.stats.lds_dma
            self.emu.run(k, (gx, gy, gz), (bx, by, bz), shmem, kab.ctypes.data, groups)
            rec = (name, (gx, gy, gz), (bx, by, bz), self.emu.stats.insts - n0, time.time() - t0,
                   self.emu.stats.lds_dma - d0)
            self.launches.append(rec)
            if self.verbose:
                print(f"  [emu] {name[:70]} grid {rec[1]} block {rec[2]}: {rec[3]} instructions, "
                      f"{rec[4]:.1f} s", flush=True)
            return 0
        except EmuError as e:
            self.error = e
            print(f"  [emu] {name}:\n{e}", flush=True)
            return 1
        except Exception as e:  # noqa: BLE001 -- reported through the library's status
            import traceback
            traceback.print_exc()
            self.error = e
            return 1


class CConfig(ctypes.Structure):
    _fields_ = [("n_heads", ctypes.c_int32), ("n_groups", ctypes.c_int32),
                ("latent_rank", ctypes.c_int32), ("head_dim", ctypes.c_int32),
                ("rope_dim", ctypes.c_int32), ("v_head_dim", ctypes.c_int32),
                ("dtype", ctypes.c_int32), ("qk_norm", ctypes.c_int32),
                ("eps", ctypes.c_float), ("softmax_scale", ctypes.c_float),
                ("rope_base", ctypes.c_float)]


def bf16_bits(x: np.ndarray) -> np.ndarray:
    u = np.ascontiguousarray(x, np.float32).view(np.uint32)
    return ((u + 0x7FFF + ((u >> 16) & 1)) >> 16).astype(np.uint16)


_P, _I32, _SZ = ctypes.c_void_p, ctypes.c_int32, ctypes.c_size_t
_C = ctypes.POINTER(CConfig)
SIGNATURES = {
    "qkmla_absorb_weights": (_I32, [_C, _P, _P, _P, _P, _P]),
    "qkmla_append": (_I32, [_C, _I32, _I32, _P, _P, _P, _P, _P, _I32, _P, _P, _P, _P, _P]),
    "qkmla_decode_workspace_size": (_SZ, [_C, _I32, _I32]),
    "qkmla_decode": (_I32, [_C, _I32, _P, _P, _P, _P, _P, _P, _P, _P, _I32, _I32, _P, _SZ, _P, _P,
                            _P, _P]),
    "qkmla_decode_multi": (_I32, [_C, _I32, _I32, _P, _P, _P, _P, _P, _P, _P, _P, _I32, _I32, _P,
                                  _SZ, _P, _P, _P, _P]),
    "qkmla_append_paged": (_I32, [_C, _I32, _I32, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P]),
    "qkmla_decode_paged": (_I32, [_C, _I32, _I32, _P, _P, _P, _P, _P, _P, _P, _P, _P, _I32, _P,
                                  _SZ, _P, _P, _P, _P]),
    "qkmla_train_workspace_size": (_SZ, [_C, _I32, _I32]),
    "qkmla_train_forward": (_I32, [_C, _I32, _I32, _P, _P, _SZ, _P, _P, _P]),
    "qkmla_train_backward": (_I32, [_C, _I32, _I32, _P, _P, _P, _P, _P, _SZ, _P, _P]),
    "qkmla_train_workspace_size_varlen": (_SZ, [_C, _I32, _I32, _I32]),
    "qkmla_train_forward_varlen": (_I32, [_C, _I32, _P, _I32, _I32, _P, _P, _SZ, _P, _P, _P,
                                          _P]),
    "qkmla_train_backward_varlen": (_I32, [_C, _I32, _P, _I32, _I32, _P, _P, _P, _P, _P, _SZ,
                                           _P, _P, _P]),
    "qkmla_out_proj": (_I32, [_C, _I32, _P, _P, _P, _P]),
    "qkmla_last_error": (ctypes.c_char_p, []),
}


class Session:
    """Weights, caches and outputs of one decode layer on the emulated device,
    driven through the C ABI exactly as the GPU tests drive it.

    ``host_fill`` writes the caches from the oracle's append instead of
    running the append kernel (to keep long cases short); ``fill_only``
    limits that to the listed sequences (the others keep zero rows)."""

    def __init__(self, dev: Device, shape, inp, qk_norm: bool = True, host_fill: bool = False,
                 hold_last: bool = False, fill_only=None):
        self.dev, self.shape, self.inp = dev, shape, inp
        s = shape
        self.bf = s.dtype == "bf16"
        self.cfg = CConfig(s.n_heads, s.n_groups, s.latent_rank, s.head_dim, s.rope_dim,
                           s.v_head_dim, 1 if self.bf else 0, int(qk_norm), 1e-6, 0.0, 10000.0)
        self.qk_norm = qk_norm
        lib = dev.lib
        for n, (r, a) in SIGNATURES.items():
            if hasattr(lib, n):
                f = getattr(lib, n)
                f.restype, f.argtypes = r, a
        self.lib = lib
        B = len(inp.lengths)
        self.B = B
        self.lengths = list(inp.lengths)
        self.max_len = max(self.lengths)
        self.L_cap = self.max_len
        H, G, r, dc, dr, dv = s.n_heads, s.n_groups, s.latent_rank, s.head_dim, s.rope_dim, s.v_head_dim
        st = self.store
        P = _P
        self.w_uk = dev.put(inp.w_uk.astype(np.float32), "w_uk")
        self.w_uv = dev.put(st(inp.w_uv), "w_uv")
        self.gamma_q = dev.put(inp.gamma_q.astype(np.float32), "gamma_q")
        self.gamma_k = dev.put(inp.gamma_k.astype(np.float32), "gamma_k")
        self.gamma_q_rope = dev.put(inp.gamma_q_rope.astype(np.float32), "gamma_q_rope")
        self.gamma_k_rope = dev.put(inp.gamma_k_rope.astype(np.float32), "gamma_k_rope")
        et = np.uint16 if self.bf else np.float32
        self.w_qabs = dev.empty((G, r, dc), et, "w_qabs")
        self.call("qkmla_absorb_weights", ctypes.byref(self.cfg), P(self.w_uk.ctypes.data),
                  P(self.gamma_q.ctypes.data), P(self.gamma_k.ctypes.data),
                  P(self.w_qabs.ctypes.data), None)
        self.lat = dev.empty((B, self.L_cap, r), et, "latent cache", fill=0)
        self.rope = dev.empty((B, self.L_cap, dr), et, "rope cache", fill=0)
        self.alpha = dev.empty((B, self.L_cap, G), np.float32, "alpha cache", fill=0)
        self.status = dev.empty((1,), np.int32, "status", fill=0)
        self.q_c = dev.put(st(inp.q_c), "q_c")
        self.q_rope = dev.put(st(inp.q_rope), "q_rope")
        fill = [L - 1 if hold_last else L for L in self.lengths]
        if host_fill:
            import oracle
            for b, n in enumerate(fill):
                if n > 0 and (fill_only is None or b in fill_only):
                    a_ref, r_ref = oracle.append_ref(inp.latents[b][:n], inp.k_rope_raw[b][:n],
                                                     np.arange(n), inp.w_uk, inp.gamma_k_rope, 1e-6,
                                                     10000.0, qk_norm=qk_norm)
                    self.lat[b, :n] = st(inp.latents[b][:n])
                    self.rope[b, :n] = st(r_ref)
                    if qk_norm:
                        self.alpha[b, :n] = a_ref.astype(np.float32)
        else:
            for b, n in enumerate(fill):
                if n <= 0:
                    continue
                c = dev.put(st(inp.latents[b][:n][None]), f"new latents {b}")
                k = dev.put(st(inp.k_rope_raw[b][:n][None]), f"new rope keys {b}")
                pos = dev.put(np.zeros(1, np.int32), f"positions {b}")
                self.call("qkmla_append", ctypes.byref(self.cfg), 1, n, P(c.ctypes.data),
                          P(k.ctypes.data), P(self.w_uk.ctypes.data),
                          P(self.gamma_k_rope.ctypes.data), P(pos.ctypes.data), self.L_cap,
                          P(self.lat[b:b + 1].ctypes.data), P(self.rope[b:b + 1].ctypes.data),
                          P(self.alpha[b:b + 1].ctypes.data), P(self.status.ctypes.data), None)
        if hold_last:
            c = dev.put(st(np.stack([x[-1:] for x in inp.latents])), "step latents")
            k = dev.put(st(np.stack([x[-1:] for x in inp.k_rope_raw])), "step rope keys")
            pos = dev.put(np.array(fill, np.int32), "step positions")
            self.call("qkmla_append", ctypes.byref(self.cfg), B, 1, P(c.ctypes.data),
                      P(k.ctypes.data), P(self.w_uk.ctypes.data), P(self.gamma_k_rope.ctypes.data),
                      P(pos.ctypes.data), self.L_cap, P(self.lat.ctypes.data),
                      P(self.rope.ctypes.data), P(self.alpha.ctypes.data),
                      P(self.status.ctypes.data), None)
        self.seq_lens = dev.put(np.array(self.lengths, np.int32), "seq_lens")
        self.o_lat = dev.empty((B, H, r), np.float32, "o_lat", fill=0xFF)
        self.lse = dev.empty((B, H), np.float32, "lse", fill=0xFF)
        self.out = dev.empty((B, H, dv), np.float32, "out", fill=0xFF)

    def store(self, x):
        x = np.asarray(x, np.float32)
        return bf16_bits(x) if self.bf else x

    def call(self, name: str, *args):
        r = getattr(self.lib, name)(*args)
        if r != 0:
            raise RuntimeError(f"{name} returned {r}: {self.lib.qkmla_last_error().decode()}\n"
                               f"{self.dev.error}")
        return r

    def decode(self):
        P = _P
        ws = self.lib.qkmla_decode_workspace_size(ctypes.byref(self.cfg), self.B, self.max_len)
        self.ws = self.dev.empty((ws,), np.uint8, "workspace", fill=0xCD)
        self.call("qkmla_decode", ctypes.byref(self.cfg), self.B, P(self.q_c.ctypes.data),
                  P(self.q_rope.ctypes.data), P(self.w_qabs.ctypes.data),
                  P(self.gamma_q_rope.ctypes.data), P(self.lat.ctypes.data),
                  P(self.rope.ctypes.data), P(self.alpha.ctypes.data),
                  P(self.seq_lens.ctypes.data), self.L_cap, self.max_len, P(self.ws.ctypes.data),
                  ws, P(self.o_lat.ctypes.data), P(self.lse.ctypes.data),
                  P(self.status.ctypes.data), None)
        return self.o_lat.copy(), self.lse.copy()

    def decode_multi(self, q_c, q_rope):
        """s_q query rows per sequence (q_c [B][s_q][H][d_c], q_rope
        [B][s_q][H][d_r], host arrays); returns (o_lat [B][s_q][H][r],
        lse [B][s_q][H], out [B][s_q][H][d_v])."""
        P = _P
        B, s_q = q_c.shape[:2]
        s = self.shape
        qc = self.dev.put(self.store(q_c), "q_c (several rows)")
        qr = self.dev.put(self.store(q_rope), "q_rope (several rows)")
        o_lat = self.dev.empty((B, s_q, s.n_heads, s.latent_rank), np.float32, "o_lat rows",
                               fill=0xFF)
        lse = self.dev.empty((B, s_q, s.n_heads), np.float32, "lse rows", fill=0xFF)
        out = self.dev.empty((B, s_q, s.n_heads, s.v_head_dim), np.float32, "o rows", fill=0xFF)
        ws = self.lib.qkmla_decode_workspace_size(ctypes.byref(self.cfg), B * s_q, self.max_len)
        self.ws = self.dev.empty((ws,), np.uint8, "workspace", fill=0xCD)
        self.call("qkmla_decode_multi", ctypes.byref(self.cfg), B, s_q, P(qc.ctypes.data),
                  P(qr.ctypes.data), P(self.w_qabs.ctypes.data),
                  P(self.gamma_q_rope.ctypes.data), P(self.lat.ctypes.data),
                  P(self.rope.ctypes.data), P(self.alpha.ctypes.data),
                  P(self.seq_lens.ctypes.data), self.L_cap, self.max_len, P(self.ws.ctypes.data),
                  ws, P(o_lat.ctypes.data), P(lse.ctypes.data), P(self.status.ctypes.data), None)
        self.call("qkmla_out_proj", ctypes.byref(self.cfg), B * s_q, P(o_lat.ctypes.data),
                  P(self.w_uv.ctypes.data), P(out.ctypes.data), None)
        return o_lat.copy(), lse.copy(), out.copy()

    def out_proj(self):
        self.call("qkmla_out_proj", ctypes.byref(self.cfg), self.B, _P(self.o_lat.ctypes.data),
                  _P(self.w_uv.ctypes.data), _P(self.out.ctypes.data), None)
        return self.out.copy()
