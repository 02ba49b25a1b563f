"""Machine state of the emulator: memory, workgroups, wavefronts, dispatch.

A wavefront keeps its VGPRs (v0..v255, then a0..a255) as uint32[512, 64] and
its SGPRs as Python ints: s0..s105, VCC at 106/107, M0 at 124 and EXEC at
126/127.  Workgroups run their wavefronts one after another up to each
barrier, then release them together; the LDS race checks (semantics.lds_mark)
treat everything between two barriers as unordered across wavefronts.
"""
from __future__ import annotations

import bisect
import collections
import os
from typing import Dict, List, Optional

import numpy as np

from .asm import Kernel, Op

U32 = np.uint32
M32 = 0xFFFFFFFF
M64 = 0xFFFFFFFFFFFFFFFF
FULL = M64
LANES = np.arange(64)
SHARED_BASE = 0x0001_0000_0000_0000      # flat-address aperture of LDS
PRIVATE_BASE = 0x0002_0000_0000_0000     # flat-address aperture of scratch
VCC, M0, EXEC = 106, 124, 126
LDS_LIMIT = 160 * 1024                   # bytes of LDS per workgroup on gfx950


# Wait states between an MFMA writing VGPRs and a VALU access to them (the
# 16-pass figure with margin), and between a VALU write and an MFMA reading it.
XDL_RESULT_WAITS = 19
VALU_TO_XDL_WAITS = 2


class EmuError(Exception):
    """A kernel did something the hardware would fault on or race on."""


_MASK_CACHE: Dict[int, np.ndarray] = {}
_SHIFTS = LANES.astype(np.uint64)


def mask_to_bool(m: int) -> np.ndarray:
    """Read-only bool[64] of a lane mask (cached)."""
    r = _MASK_CACHE.get(m)
    if r is None:
        r = ((np.uint64(m) >> _SHIFTS) & np.uint64(1)).astype(bool)
        r.flags.writeable = False
        if len(_MASK_CACHE) < 100000:
            _MASK_CACHE[m] = r
    return r


def bool_to_mask(b: np.ndarray) -> int:
    return int(np.packbits(b.astype(np.uint8), bitorder="little").view("<u8")[0])


def f32(x: np.ndarray) -> np.ndarray:
    return x.view(np.float32)


def sext32(v: int) -> int:
    v &= M32
    return v - (1 << 32) if v & 0x80000000 else v


def bf16_rne(x: np.ndarray) -> np.ndarray:
    """float32 -> uint32 holding bf16 bits, round to nearest even (NaN kept quiet)."""
    u = x.astype(np.float32).view(U32).astype(np.uint64)
    r = ((u + 0x7FFF + ((u >> 16) & 1)) >> 16) & 0xFFFF
    r = np.where(np.isnan(x), (u >> 16) | 0x40, r)
    return r.astype(U32)


def bf16_to_f32(h: np.ndarray) -> np.ndarray:
    return (h.astype(U32) << 16).view(np.float32)


# ----------------------------------------------------------------------------
class Memory:
    """Registered global allocations (process memory) with bounds checks."""

    def __init__(self):
        self.bases: List[int] = []
        self.allocs: Dict[int, tuple] = {}

    def add(self, addr: int, size: int, name: str, arr: Optional[np.ndarray] = None):
        if arr is None:
            import ctypes
            arr = np.ctypeslib.as_array((ctypes.c_uint8 * size).from_address(addr))
        i = bisect.bisect_right(self.bases, addr)
        for j in (i - 1, i):
            if 0 <= j < len(self.bases):
                b = self.bases[j]
                s = self.allocs[b][0]
                if addr < b + s and b < addr + size:
                    raise EmuError(f"overlapping allocations {name} and {self.allocs[b][1]}")
        self.bases.insert(i, addr)
        self.allocs[addr] = (size, name, arr)

    def _nearest(self, ad: int) -> str:
        best = None
        for b in self.bases:
            size, name, _ = self.allocs[b]
            d = ad - (b + size) if ad >= b + size else b - ad
            if best is None or abs(d) < best[0]:
                best = (abs(d), f"{name}[{b:#x}, +{size}) at distance {d}")
        return best[1] if best else "none"

    def locate(self, addrs: np.ndarray, nbytes: int, what: str):
        """[(buffer, offsets, lane selection)] covering every address."""
        a = addrs.astype(np.uint64)
        lo, hi = int(a.min()), int(a.max())
        i = bisect.bisect_right(self.bases, lo) - 1
        if i >= 0:
            b = self.bases[i]
            size, _, arr = self.allocs[b]
            if lo >= b and hi + nbytes <= b + size:
                return [(arr, (a - np.uint64(b)).astype(np.int64), np.ones(len(a), bool))]
        groups: Dict[int, list] = {}
        for k, ad in enumerate(a.tolist()):
            j = bisect.bisect_right(self.bases, ad) - 1
            if not (j >= 0 and ad + nbytes <= self.bases[j] + self.allocs[self.bases[j]][0]):
                raise EmuError(f"{what}: address {ad:#x} (+{nbytes} B, lane {k}) is outside "
                               f"every allocation; nearest: {self._nearest(ad)}")
            groups.setdefault(self.bases[j], []).append(k)
        out = []
        for b, lanes in groups.items():
            sel = np.zeros(len(a), bool)
            sel[lanes] = True
            out.append((self.allocs[b][2], (a - np.uint64(b)).astype(np.int64), sel))
        return out

    def read(self, addrs: np.ndarray, nbytes: int, what: str) -> np.ndarray:
        """uint8[len(addrs), nbytes]"""
        out = np.zeros((len(addrs), nbytes), np.uint8)
        if len(addrs):
            for arr, off, sel in self.locate(addrs, nbytes, what):
                out[sel] = arr[off[sel][:, None] + np.arange(nbytes)[None, :]]
        return out

    def read_scalar(self, addr: int, nbytes: int, what: str) -> bytes:
        return self.read(np.array([addr], np.uint64), nbytes, what)[0].tobytes()

    def write(self, addrs: np.ndarray, data: np.ndarray, what: str):
        n = data.shape[1]
        if len(addrs):
            for arr, off, sel in self.locate(addrs, n, what):
                offs, d = off[sel], data[sel]
                for k in range(len(offs)):   # lane order: the highest lane wins an overlap
                    arr[offs[k]:offs[k] + n] = d[k]


class Stats:
    def __init__(self):
        self.insts = 0
        self.lds_dma = 0                    # global->LDS load instructions issued
        self.by_op: collections.Counter = collections.Counter()
        self.warnings: List[str] = []


# ----------------------------------------------------------------------------
class Workgroup:
    """LDS bytes plus per-dword bookkeeping for DMA and race checks."""

    def __init__(self, lds_bytes: int):
        n = max(lds_bytes, 4)
        nd = (n + 3) // 4
        self.lds = np.zeros(n, np.uint8)
        self.lds_size = lds_bytes
        self.dma_pending = np.zeros(nd, np.int32)
        self.w_wave = np.full(nd, -1, np.int16)
        self.w_epoch = np.full(nd, -1, np.int64)
        self.r_epoch = np.full(nd, -1, np.int64)
        self.r_mask = np.zeros(nd, np.int64)
        self.epoch = 0


class Wave:
    def __init__(self, emu: "Emulator", kern: Kernel, wg: Workgroup, wave_id: int, group_id,
                 block, kernarg_addr: int, n_threads: int):
        self.emu, self.k, self.wg, self.wid = emu, kern, wg, wave_id
        self.V = np.zeros((512, 64), U32)
        self.S = [0] * 128
        self.scc = 0
        self.pc = 0
        self.done = False
        self.at_barrier = False
        self.clock = 0                      # wait states issued so far
        self.valu_sgpr_write: Dict[int, int] = {}
        self.salu_m0_write = -100
        # Hazards of MFMAs written as inline asm, which the compiler does not
        # see as MFMAs: register -> wait-state clock of the MFMA that wrote it,
        # and of the last VALU write (MFMA operands need wait states after one)
        self.xdl_write = {}
        self.valu_vgpr_write = {}
        self.cur_inst = None
        self.in_mfma_srcc = False
        self.vm_q: collections.deque = collections.deque()
        self.lgkm_q: collections.deque = collections.deque()
        self.pend_v: Dict[int, int] = {}
        self.pend_s: Dict[int, int] = {}
        self.priv = np.zeros((64, max(kern.private_bytes, 4)), np.uint8)
        md = kern.meta
        si = 0
        for key, n in (("user_sgpr_private_segment_buffer", 4), ("user_sgpr_dispatch_ptr", 2),
                       ("user_sgpr_queue_ptr", 2)):
            if md.get(key, 0):
                si += n
        if md.get("user_sgpr_kernarg_segment_ptr", 0):
            self.S[si] = kernarg_addr & M32
            self.S[si + 1] = kernarg_addr >> 32
        si = md.get("user_sgpr_count", 0)
        for d, key in enumerate(("x", "y", "z")):
            if md.get("system_sgpr_workgroup_id_" + key, 0):
                self.S[si] = group_id[d]
                si += 1
        tid = wave_id * 64 + LANES
        bx, by, _ = block
        self.V[0] = ((tid % bx) | (((tid // bx) % by) << 10) | ((tid // (bx * by)) << 20)).astype(U32)
        self.set_exec(bool_to_mask(tid < n_threads))

    # -- scalar registers ----------------------------------------------------
    def set_exec(self, m: int):
        self.S[EXEC] = m & M32
        self.S[EXEC + 1] = (m >> 32) & M32

    @property
    def exec(self) -> int:
        return self.S[EXEC] | (self.S[EXEC + 1] << 32)

    def exec_mask(self) -> np.ndarray:
        return mask_to_bool(self.exec)

    @property
    def vcc(self) -> int:
        return self.S[VCC] | (self.S[VCC + 1] << 32)

    def _check_pend_s(self, idx: int, n: int, what: str):
        for r in range(idx, idx + n):
            if r in self.pend_s:
                raise EmuError(f"{what} s{r} while its load is still in flight")

    def sget(self, o: Op, ty: str = "b32") -> int:
        """Scalar operand as an int; ty in b64/u64/i64/f64 reads a register pair."""
        wide = ty in ("b64", "u64", "i64", "f64")
        if o.kind == "s":
            n = 2 if wide else 1
            self._check_pend_s(o.idx, n, "read of")
            v = self.S[o.idx]
            return v | (self.S[o.idx + 1] << 32) if wide else v
        if o.kind == "imm":
            if ty == "f64":
                return o.imm_bits("f64")
            return o.ival & (M64 if wide else M32)
        if o.kind == "fimm":
            return o.imm_bits("f64" if ty == "f64" else "f32")
        if o.kind == "shared_base":
            return SHARED_BASE
        if o.kind == "private_base":
            return PRIVATE_BASE
        raise EmuError(f"bad scalar operand {o.text}")

    def sset(self, o: Op, v: int, n: Optional[int] = None):
        n = n or o.n
        if o.kind != "s":
            raise EmuError(f"bad scalar destination {o.text}")
        for r in range(o.idx, o.idx + n):
            if r in self.pend_s:
                raise EmuError(f"write of s{r} while its load is still in flight")
        self.S[o.idx] = v & M32
        if n == 2:
            self.S[o.idx + 1] = (v >> 32) & M32
        if o.idx == M0:
            self.salu_m0_write = self.clock

    def note_valu_sgpr(self, o: Op, n: int = 1):
        for r in range(o.idx, o.idx + max(o.n, n)):
            self.valu_sgpr_write[r] = self.clock

    # -- vector registers ----------------------------------------------------
    @staticmethod
    def vrow(o: Op, i: int = 0) -> int:
        return (256 if o.kind == "a" else 0) + o.idx + i

    def check_pend_v(self, row: int, what: str):
        if row in self.pend_v:
            name = f"a{row - 256}" if row >= 256 else f"v{row}"
            raise EmuError(f"{what} {name} while its load is still in flight")

    def check_xdl_result(self, r: int, what: str):
        t = self.xdl_write.get(r)
        if t is not None and not self.in_mfma_srcc and self.clock - t - 1 < XDL_RESULT_WAITS:
            raise EmuError(f"{what} v{r} {self.clock - t - 1} wait states after an inline-asm "
                           f"MFMA wrote it (needs {XDL_RESULT_WAITS})")

    def vget(self, o: Op, ty: str = "b32", i: int = 0) -> np.ndarray:
        """Dword i of operand o for all 64 lanes."""
        k = o.kind
        if k == "v" or k == "a":
            r = (256 if k == "a" else 0) + o.idx + i
            if r in self.pend_v:
                self.check_pend_v(r, "read of")
            if self.xdl_write:
                self.check_xdl_result(r, "read of")
            return self.V[r]
        if k == "s":
            self._check_pend_s(o.idx + i, 1, "read of")
            return np.full(64, self.S[o.idx + i], U32)
        if k in ("imm", "fimm"):
            b = o.imm_bits(ty)
            b = (b >> (32 * i)) & M32 if ty in ("f64", "b64", "u64", "i64") else (0 if i else b)
            return np.full(64, b, U32)
        raise EmuError(f"bad vector operand {o.text}")

    def vget64(self, o: Op, ty: str = "b64") -> np.ndarray:
        lo = self.vget(o, ty, 0).astype(np.uint64)
        hi = self.vget(o, ty, 1).astype(np.uint64)
        return lo | (hi << np.uint64(32))

    def vset(self, o: Op, val: np.ndarray, i: int = 0, mask: Optional[np.ndarray] = None):
        r = (256 if o.kind == "a" else 0) + o.idx + i
        if r in self.pend_v:
            self.check_pend_v(r, "write of")
        op = self.cur_inst.op if self.cur_inst is not None else ""
        if not op.startswith("v_mfma"):
            if self.xdl_write:
                self.check_xdl_result(r, "write of")
            if op.startswith("v_"):
                self.valu_vgpr_write[r] = self.clock
        if mask is None:
            e = self.exec
            if e == FULL:
                self.V[r] = val
                return
            mask = mask_to_bool(e)
        np.copyto(self.V[r], val.astype(U32, copy=False), where=mask)

    def vset64(self, o: Op, val: np.ndarray, mask: Optional[np.ndarray] = None):
        v = val.astype(np.uint64)
        self.vset(o, (v & np.uint64(M32)).astype(U32), 0, mask)
        self.vset(o, (v >> np.uint64(32)).astype(U32), 1, mask)

    def fget(self, o: Op, i: int = 0) -> np.ndarray:
        x = f32(self.vget(o, "f32", i)).copy()
        if o.abs:
            x = np.abs(x)
        return -x if o.neg else x

    def dget(self, o: Op) -> np.ndarray:
        x = self.vget64(o, "f64").view(np.float64).copy()
        if o.abs:
            x = np.abs(x)
        return -x if o.neg else x

    def dset(self, o: Op, x: np.ndarray, mask: Optional[np.ndarray] = None):
        self.vset64(o, np.asarray(x, np.float64).view(np.uint64), mask)

    def lanemask_get(self, o: Op) -> np.ndarray:
        return mask_to_bool(self.sget(o, "b64"))

    def lanemask_set(self, o: Op, b: np.ndarray):
        """A per-lane condition written by VALU; inactive lanes read as 0."""
        self.sset(o, bool_to_mask(b & self.exec_mask()), 2)
        self.note_valu_sgpr(o, 2)


# ----------------------------------------------------------------------------
def _sdwa_wrap(h, base, inst):
    """SDWA form of a plain integer VOP handler: its src0_sel / src1_sel pick a
    byte or word of the source (zero-extended) before the operation.  Only
    handlers that read their sources through vget (the integer VOP table) and
    a full-dword destination are modelled; anything else stops the run."""
    from .semantics import _V
    sels = {}
    for k, key in ((1, "src0_sel"), (2, "src1_sel")):
        sel = inst.mods.get(key, "DWORD")
        if sel != "DWORD":
            sels[k] = sel
    if inst.mods.get("dst_sel", "DWORD") != "DWORD" or "sext(" in inst.text:
        raise EmuError(f"sdwa dst_sel / sext not modelled (line {inst.line}: {inst.text})")
    if not sels:
        return h
    if base not in _V:
        raise EmuError(f"sdwa source select on {base} not modelled (line {inst.line}: {inst.text})")

    def pick(x, sel):
        x = x.astype(np.uint32)
        if sel == "WORD_0":
            return x & np.uint32(0xFFFF)
        if sel == "WORD_1":
            return (x >> np.uint32(16)) & np.uint32(0xFFFF)
        if sel.startswith("BYTE_"):
            return (x >> np.uint32(8 * int(sel[5:]))) & np.uint32(0xFF)
        raise EmuError(f"sdwa sel {sel}")

    def run(w, i):
        ops = {id(i.ops[k]): sel for k, sel in sels.items() if k < len(i.ops)}
        orig = w.vget

        def vget(o, ty="b32", idx=0):
            v = orig(o, ty, idx)
            sel = ops.get(id(o))
            return v if sel is None else pick(v, sel)
        w.vget = vget
        try:
            h(w, i)
        finally:
            del w.vget
    return run


class Emulator:
    def __init__(self, mem: Memory):
        from .semantics import HANDLERS
        self.mem = mem
        self.stats = Stats()
        self.handlers = HANDLERS
        self.max_vm_inflight = 0
        self.trace = os.environ.get("QKMLA_EMU_TRACE")   # kernel-name substring
        self.opcount = os.environ.get("QKMLA_EMU_OPCOUNT")

    def prepare(self, kern: Kernel):
        for inst in kern.insts:
            if inst.handler is None:
                base = inst.op
                for suf in ("_e32", "_e64", "_sdwa"):
                    if base.endswith(suf):
                        base = base[: -len(suf)]
                        break
                h = self.handlers.get(base)
                if h is None:
                    raise EmuError(f"no semantics for {inst.op} (line {inst.line}: {inst.text})")
                if inst.op.endswith("_sdwa") and base != "v_and_b32":  # v_and_b32 does its own
                    h = _sdwa_wrap(h, base, inst)
                inst.handler = h

    def run(self, kern: Kernel, grid, block, shmem: int, kernarg_addr: int,
            groups: Optional[List[tuple]] = None, max_insts: int = 200_000_000):
        self.prepare(kern)
        nthreads = block[0] * block[1] * block[2]
        nwaves = (nthreads + 63) // 64
        lds_total = kern.lds_bytes + shmem
        if lds_total > LDS_LIMIT:
            raise EmuError(f"LDS {lds_total} B exceeds {LDS_LIMIT} B")
        if groups is None:
            groups = [(x, y, z) for z in range(grid[2]) for y in range(grid[1])
                      for x in range(grid[0])]
        for g in groups:
            wg = Workgroup(lds_total)
            waves = [Wave(self, kern, wg, w, g, block, kernarg_addr, nthreads)
                     for w in range(nwaves)]
            self._run_group(kern, wg, waves, g, max_insts)

    def _trace(self, w: Wave, inst):
        desc = ""
        if inst.ops:
            d = inst.ops[0]
            if d.kind in ("v", "a"):
                vals = [int(w.V[w.vrow(d, k), 0]) for k in range(min(d.n, 4))]
                desc = " ".join(f"{v:08x}" for v in vals)
            elif d.kind == "s":
                desc = " ".join(f"{w.S[d.idx + k]:08x}" for k in range(min(d.n, 4)))
        print(f"{inst.line:6d} {inst.text[:70]:70s} | {desc} scc={w.scc}")

    def _run_group(self, kern: Kernel, wg: Workgroup, waves: List[Wave], g, max_insts: int):
        insts = kern.insts
        n = 0
        trace = self.trace and self.trace in kern.name and g == (0, 0, 0)
        count = self.opcount and self.opcount in kern.name and g == (0, 0, 0)
        while True:
            for w in waves:
                while not w.done and not w.at_barrier:
                    if w.pc >= len(insts):
                        raise EmuError(f"wave {w.wid} ran past the end of {kern.name}")
                    inst = insts[w.pc]
                    w.pc += 1
                    w.cur_inst = inst
                    try:
                        inst.handler(w, inst)
                    except EmuError as e:
                        raise EmuError(f"[{kern.name[:60]} group {g} wave {w.wid}] asm line "
                                       f"{inst.line}: {inst.text}\n    {e}") from None
                    if trace and w.wid == 0:
                        self._trace(w, inst)
                    if count and w.wid == 0:
                        self.stats.by_op[inst.op] += 1
                    w.clock += 1
                    n += 1
                    if n > max_insts:
                        raise EmuError(f"{kern.name}: instruction limit reached (a hang?)")
            live = [w for w in waves if not w.done]
            if not live:
                break
            # every live wavefront waits at the barrier (ended ones do not count)
            wg.epoch += 1
            for w in live:
                w.at_barrier = False
        self.stats.insts += n
        for w in waves:
            if w.pend_v or w.pend_s:
                self.stats.warnings.append(f"{kern.name}: a wave ended with loads never waited for")
            for q in (w.vm_q, w.lgkm_q):
                while q:
                    q.popleft().pop(w)
