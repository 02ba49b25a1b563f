"""Instruction semantics of the emulator: the gfx950 subset the library's
kernels compile to.  Each handler takes (wave, instruction).  Unknown opcodes
are reported by the emulator before a kernel starts (Emulator.prepare)."""
from __future__ import annotations

import numpy as np

from .machine import (M32, M64, SHARED_BASE, U32, VALU_TO_XDL_WAITS, EmuError, bf16_rne, bf16_to_f32, f32,
                      mask_to_bool, sext32)

HANDLERS = {}
F32 = np.float32
F64 = np.float64
I32 = np.int32
U64 = np.uint64
LANES = np.arange(64)


def h(*names):
    def deco(fn):
        for n in names:
            HANDLERS[n] = fn
        return fn
    return deco


def _err_np():
    return np.errstate(all="ignore")


# ============================================================================
# pending-result queue entries
class Pend:
    __slots__ = ("vrows", "srows", "apply", "dma", "queues", "what")

    def __init__(self, w, vrows=(), srows=(), apply=None, dma=None, queues=1, what=""):
        self.vrows, self.srows, self.apply, self.dma = list(vrows), list(srows), apply, dma
        self.queues = queues
        self.what = what
        for r in self.vrows:
            if r in w.pend_v:
                raise EmuError(f"{what}: destination row {r} already has a load in flight")
            w.pend_v[r] = 1
        for r in self.srows:
            if r in w.pend_s:
                raise EmuError(f"{what}: destination s{r} already has a load in flight")
            w.pend_s[r] = 1

    def pop(self, w):
        self.queues -= 1
        if self.queues == 0:
            self.retire(w)

    def retire(self, w):
        for r in self.vrows:
            w.pend_v.pop(r, None)
        for r in self.srows:
            w.pend_s.pop(r, None)
        if self.apply is not None:
            self.apply()
        if self.dma is not None:
            idx, data = self.dma
            wg = w.wg
            wg.dma_pending[idx] -= 1
            lds_mark(w, idx, "w", "LDS DMA completion")
            # write bytes
            b = (idx[:, None] * 4 + np.arange(4)[None, :]).reshape(-1)
            wg.lds[b] = data.reshape(-1)


def push_vm(w, p):
    w.vm_q.append(p)
    if len(w.vm_q) > 63:
        w.emu.stats.warnings.append(f"more than 63 vector memory ops in flight ({w.k.name[:40]} pc {w.pc})")
    w.emu.max_vm_inflight = max(w.emu.max_vm_inflight, len(w.vm_q))


def push_lgkm(w, p):
    w.lgkm_q.append(p)


@h("s_waitcnt")
def _waitcnt(w, inst):
    vm = inst.mods.get("vmcnt", 63)
    lg = inst.mods.get("lgkmcnt", 15)
    while len(w.vm_q) > vm:
        w.vm_q.popleft().pop(w)
    while len(w.lgkm_q) > lg:
        w.lgkm_q.popleft().pop(w)


@h("s_nop")
def _nop(w, inst):
    w.clock += inst.ops[0].ival  # s_nop N gives N+1 wait states (1 added by the loop)


@h("s_barrier")
def _barrier(w, inst):
    w.at_barrier = True


@h("s_endpgm")
def _endpgm(w, inst):
    w.done = True


@h("s_setprio", "s_sleep")
def _ignore(w, inst):
    pass


# ============================================================================
# hazards the compiler cannot see through inline asm
def check_vmem_sgpr_hazard(w, inst, sops):
    for o in sops:
        if o is None or o.kind != "s":
            continue
        for r in range(o.idx, o.idx + o.n):
            t = w.valu_sgpr_write.get(r)
            if t is not None and w.clock - t - 1 < 5:
                msg = (f"VMEM reads s{r} {w.clock - t - 1} wait states after a VALU wrote it "
                       f"(needs 5)")
                if inst.in_asm:
                    raise EmuError(msg)
                w.emu.stats.warnings.append(msg + f" [compiler code, line {inst.line}]")


# ============================================================================
# SALU
def _s2(w, inst, ty="b32"):
    return [w.sget(o, ty) for o in inst.ops[1:]]


def _setscc(w, c):
    w.scc = 1 if c else 0


@h("s_mov_b32")
def _(w, i):
    w.sset(i.ops[0], w.sget(i.ops[1]))


@h("s_mov_b64")
def _(w, i):
    w.sset(i.ops[0], w.sget(i.ops[1], "b64"), 2)


@h("s_movk_i32")
def _(w, i):
    v = i.ops[1].ival & 0xFFFF
    w.sset(i.ops[0], (v - 0x10000 if v & 0x8000 else v) & M32)


@h("s_add_u32")
def _(w, i):
    a, b = _s2(w, i)
    r = a + b
    w.sset(i.ops[0], r)
    _setscc(w, r >> 32)


@h("s_addc_u32")
def _(w, i):
    a, b = _s2(w, i)
    r = a + b + w.scc
    w.sset(i.ops[0], r)
    _setscc(w, r >> 32)


@h("s_sub_u32")
def _(w, i):
    a, b = _s2(w, i)
    w.sset(i.ops[0], (a - b) & M32)
    _setscc(w, b > a)


@h("s_subb_u32")
def _(w, i):
    a, b = _s2(w, i)
    c = w.scc
    w.sset(i.ops[0], (a - b - c) & M32)
    _setscc(w, b + c > a)


@h("s_add_i32")
def _(w, i):
    a, b = [sext32(x) for x in _s2(w, i)]
    r = a + b
    w.sset(i.ops[0], r & M32)
    _setscc(w, r != sext32(r))


@h("s_sub_i32")
def _(w, i):
    a, b = [sext32(x) for x in _s2(w, i)]
    r = a - b
    w.sset(i.ops[0], r & M32)
    _setscc(w, r != sext32(r))


@h("s_addk_i32")
def _(w, i):
    a = sext32(w.sget(i.ops[0]))
    k = i.ops[1].ival & 0xFFFF
    k = k - 0x10000 if k & 0x8000 else k
    r = a + k
    w.sset(i.ops[0], r & M32)
    _setscc(w, r != sext32(r))


@h("s_mul_i32")
def _(w, i):
    a, b = _s2(w, i)
    w.sset(i.ops[0], (sext32(a) * sext32(b)) & M32)


@h("s_mulk_i32")
def _(w, i):
    k = i.ops[1].ival & 0xFFFF
    k = k - 0x10000 if k & 0x8000 else k
    w.sset(i.ops[0], (sext32(w.sget(i.ops[0])) * k) & M32)


@h("s_mul_hi_u32")
def _(w, i):
    a, b = _s2(w, i)
    w.sset(i.ops[0], ((a * b) >> 32) & M32)


@h("s_mul_hi_i32")
def _(w, i):
    a, b = _s2(w, i)
    w.sset(i.ops[0], ((sext32(a) * sext32(b)) >> 32) & M32)


@h("s_lshl_b32")
def _(w, i):
    a, b = _s2(w, i)
    r = (a << (b & 31)) & M32
    w.sset(i.ops[0], r)
    _setscc(w, r)


@h("s_lshl_b64")
def _(w, i):
    a = w.sget(i.ops[1], "b64")
    b = w.sget(i.ops[2])
    r = (a << (b & 63)) & M64
    w.sset(i.ops[0], r, 2)
    _setscc(w, r)


@h("s_bfe_u32")
def _(w, i):
    a, b = _s2(w, i)
    off, width = b & 31, (b >> 16) & 127
    r = (a >> off) & ((1 << width) - 1) if width else 0
    r &= M32
    w.sset(i.ops[0], r)
    _setscc(w, r)


@h("s_bfe_i64")
def _(w, i):
    a = w.sget(i.ops[1], "b64")
    b = w.sget(i.ops[2])
    off, width = b & 63, (b >> 16) & 127
    r = 0
    if width:
        r = (a >> off) & ((1 << width) - 1)
        if (r >> (width - 1)) & 1:
            r -= 1 << width
        r &= M64
    w.sset(i.ops[0], r, 2)
    _setscc(w, r)


@h("s_lshr_b32")
def _(w, i):
    a, b = _s2(w, i)
    r = a >> (b & 31)
    w.sset(i.ops[0], r)
    _setscc(w, r)


@h("s_lshr_b64")
def _(w, i):
    a = w.sget(i.ops[1], "b64")
    b = w.sget(i.ops[2])
    r = a >> (b & 63)
    w.sset(i.ops[0], r, 2)
    _setscc(w, r)


@h("s_ashr_i32")
def _(w, i):
    a, b = _s2(w, i)
    r = (sext32(a) >> (b & 31)) & M32
    w.sset(i.ops[0], r)
    _setscc(w, r)


def _bitop(fn, wide):
    def run(w, i):
        ty = "b64" if wide else "b32"
        a = w.sget(i.ops[1], ty)
        b = w.sget(i.ops[2], ty)
        r = fn(a, b) & (M64 if wide else M32)
        w.sset(i.ops[0], r, 2 if wide else 1)
        _setscc(w, r)
    return run


for _n, _f in (("and", lambda a, b: a & b), ("or", lambda a, b: a | b),
               ("xor", lambda a, b: a ^ b), ("andn2", lambda a, b: a & ~b),
               ("orn2", lambda a, b: a | ~b), ("nand", lambda a, b: ~(a & b)),
               ("nor", lambda a, b: ~(a | b))):
    HANDLERS[f"s_{_n}_b32"] = _bitop(_f, False)
    HANDLERS[f"s_{_n}_b64"] = _bitop(_f, True)


@h("s_not_b32")
def _(w, i):
    r = ~w.sget(i.ops[1]) & M32
    w.sset(i.ops[0], r)
    _setscc(w, r)


@h("s_not_b64")
def _(w, i):
    r = ~w.sget(i.ops[1], "b64") & M64
    w.sset(i.ops[0], r, 2)
    _setscc(w, r)


@h("s_min_i32")
def _(w, i):
    a, b = [sext32(x) for x in _s2(w, i)]
    w.sset(i.ops[0], min(a, b) & M32)
    _setscc(w, a < b)


@h("s_max_i32")
def _(w, i):
    a, b = [sext32(x) for x in _s2(w, i)]
    w.sset(i.ops[0], max(a, b) & M32)
    _setscc(w, a > b)


@h("s_min_u32")
def _(w, i):
    a, b = _s2(w, i)
    w.sset(i.ops[0], min(a, b))
    _setscc(w, a < b)


@h("s_max_u32")
def _(w, i):
    a, b = _s2(w, i)
    w.sset(i.ops[0], max(a, b))
    _setscc(w, a > b)


@h("s_abs_i32")
def _(w, i):
    a = sext32(w.sget(i.ops[1]))
    r = abs(a) & M32
    w.sset(i.ops[0], r)
    _setscc(w, r)


@h("s_cselect_b32")
def _(w, i):
    a, b = _s2(w, i)
    w.sset(i.ops[0], a if w.scc else b)


@h("s_cselect_b64")
def _(w, i):
    a = w.sget(i.ops[1], "b64")
    b = w.sget(i.ops[2], "b64")
    w.sset(i.ops[0], a if w.scc else b, 2)


def _scmp(fn, signed, wide=False):
    def run(w, i):
        ty = "b64" if wide else "b32"
        a = w.sget(i.ops[0], ty)
        b = w.sget(i.ops[1], ty)
        if signed:
            a, b = sext32(a), sext32(b)
        _setscc(w, fn(a, b))
    return run


_CMP = {"eq": lambda a, b: a == b, "lg": lambda a, b: a != b, "gt": lambda a, b: a > b,
        "ge": lambda a, b: a >= b, "lt": lambda a, b: a < b, "le": lambda a, b: a <= b}
for _c, _f in _CMP.items():
    HANDLERS[f"s_cmp_{_c}_i32"] = _scmp(_f, True)
    HANDLERS[f"s_cmp_{_c}_u32"] = _scmp(_f, False)
    HANDLERS[f"s_cmp_{_c}_u64"] = _scmp(_f, False, True)


def _scmpk(fn, signed):
    def run(w, i):
        a = w.sget(i.ops[0])
        k = i.ops[1].ival & 0xFFFF
        if signed:
            a = sext32(a)
            k = k - 0x10000 if k & 0x8000 else k
        _setscc(w, fn(a, k))
    return run


for _c, _f in _CMP.items():
    HANDLERS[f"s_cmpk_{_c}_i32"] = _scmpk(_f, True)
    HANDLERS[f"s_cmpk_{_c}_u32"] = _scmpk(_f, False)


@h("s_bitcmp0_b32")
def _(w, i):
    a, b = w.sget(i.ops[0]), w.sget(i.ops[1])
    _setscc(w, ((a >> (b & 31)) & 1) == 0)


@h("s_bitcmp1_b32")
def _(w, i):
    a, b = w.sget(i.ops[0]), w.sget(i.ops[1])
    _setscc(w, ((a >> (b & 31)) & 1) == 1)


@h("s_bitset1_b32")
def _(w, i):
    d = w.sget(i.ops[0])
    b = w.sget(i.ops[1])
    w.sset(i.ops[0], d | (1 << (b & 31)))


@h("s_bitset0_b32")
def _(w, i):
    d = w.sget(i.ops[0])
    b = w.sget(i.ops[1])
    w.sset(i.ops[0], d & ~(1 << (b & 31)) & M32)


@h("s_brev_b32")
def _(w, i):
    a = w.sget(i.ops[1])
    w.sset(i.ops[0], int(f"{a:032b}"[::-1], 2))


@h("s_ff1_i32_b64")
def _(w, i):
    a = w.sget(i.ops[1], "b64")
    r = (a & -a).bit_length() - 1 if a else -1
    w.sset(i.ops[0], r & M32)


@h("s_ff1_i32_b32")
def _(w, i):
    a = w.sget(i.ops[1])
    r = (a & -a).bit_length() - 1 if a else -1
    w.sset(i.ops[0], r & M32)


@h("s_bcnt1_i32_b64")
def _(w, i):
    r = bin(w.sget(i.ops[1], "b64")).count("1")
    w.sset(i.ops[0], r)
    _setscc(w, r)


def _saveexec(fn):
    def run(w, i):
        old = w.exec
        s = w.sget(i.ops[1], "b64")
        new = fn(s, old) & M64
        w.sset(i.ops[0], old, 2)
        w.set_exec(new)
        _setscc(w, new)
    return run


HANDLERS["s_and_saveexec_b64"] = _saveexec(lambda s, e: s & e)
HANDLERS["s_or_saveexec_b64"] = _saveexec(lambda s, e: s | e)
HANDLERS["s_andn2_saveexec_b64"] = _saveexec(lambda s, e: s & ~e)
HANDLERS["s_xor_saveexec_b64"] = _saveexec(lambda s, e: s ^ e)


def _branch(cond):
    def run(w, i):
        if cond(w):
            w.pc = i.target
    return run


HANDLERS["s_branch"] = _branch(lambda w: True)
HANDLERS["s_cbranch_scc0"] = _branch(lambda w: w.scc == 0)
HANDLERS["s_cbranch_scc1"] = _branch(lambda w: w.scc == 1)
HANDLERS["s_cbranch_vccz"] = _branch(lambda w: w.vcc == 0)
HANDLERS["s_cbranch_vccnz"] = _branch(lambda w: w.vcc != 0)
HANDLERS["s_cbranch_execz"] = _branch(lambda w: w.exec == 0)
HANDLERS["s_cbranch_execnz"] = _branch(lambda w: w.exec != 0)


def _sload(nd):
    def run(w, i):
        d, base, off = i.ops
        check_vmem_sgpr_hazard(w, i, [])
        b = w.sget(base, "b64")
        o = off.ival if off.kind == "imm" else w.sget(off)
        addr = (b + o) & ~3
        data = np.frombuffer(w.emu.mem.read_scalar(addr, 4 * nd, "s_load"), "<u4")
        vals = [int(x) for x in data]
        rows = list(range(d.idx, d.idx + nd))

        def apply():
            for k, r in enumerate(rows):
                w.S[r] = vals[k]
        push_lgkm(w, Pend(w, srows=rows, apply=apply, what=i.text))
    return run


for _n, _k in (("s_load_dword", 1), ("s_load_dwordx2", 2), ("s_load_dwordx4", 4),
               ("s_load_dwordx8", 8), ("s_load_dwordx16", 16)):
    HANDLERS[_n] = _sload(_k)


# ============================================================================
# VALU: lane-select / cross-lane moves
@h("v_readlane_b32")
def _(w, i):
    d, src, sel = i.ops
    if sel.kind == "s":
        t = w.valu_sgpr_write.get(sel.idx)
        if t is not None and w.clock - t - 1 < 4 and i.in_asm:
            raise EmuError("readlane lane select written by VALU < 4 wait states before")
        lane = w.sget(sel) & 63
    else:
        lane = sel.ival & 63
    v = int(w.vget(src)[lane])
    w.sset(d, v)
    w.note_valu_sgpr(d)


@h("v_permlane32_swap_b32")
def _(w, i):
    """Swap lanes 32..63 of the destination with lanes 0..31 of the source
    (both operands are written)."""
    d, src = i.ops
    if not w.exec_mask().all():
        raise EmuError("v_permlane32_swap with partial exec not modelled")
    if i.mods.get("bound_ctrl") or i.mods.get("fi"):
        raise EmuError(f"v_permlane32_swap modifiers not modelled: {i.text}")
    vd, vs = w.vget(d).copy(), w.vget(src).copy()
    nd, ns = vd.copy(), vs.copy()
    nd[32:] = vs[:32]
    ns[:32] = vd[32:]
    w.vset(d, nd)
    w.vset(src, ns)


@h("v_readfirstlane_b32")
def _(w, i):
    d, src = i.ops
    m = w.exec_mask()
    lane = int(np.argmax(m)) if m.any() else 0
    v = int(w.vget(src)[lane])
    w.sset(d, v)
    w.note_valu_sgpr(d)


@h("v_writelane_b32")
def _(w, i):
    d, src, sel = i.ops
    lane = (w.sget(sel) if sel.kind == "s" else sel.ival) & 63
    v = w.sget(src) if src.kind == "s" else src.imm_bits("b32")
    row = w.vrow(d)
    w.check_pend_v(row, "write of")
    w.V[row, lane] = v


@h("v_mbcnt_lo_u32_b32")
def _(w, i):
    d, a, b = i.ops
    m = w.sget(a) if a.kind == "s" else a.imm_bits("b32")
    if a.kind == "v":
        raise EmuError("mbcnt with VGPR mask")
    bits = mask_to_bool(m & M32)[:32]
    pre = np.concatenate([[0], np.cumsum(bits)])   # count of bits below lane, lanes 0..32
    cnt = np.where(LANES < 32, pre[np.minimum(LANES, 32)], pre[32])
    w.vset(d, (cnt + w.vget(b).astype(np.int64)).astype(U32))


@h("v_mbcnt_hi_u32_b32")
def _(w, i):
    d, a, b = i.ops
    m = w.sget(a) if a.kind == "s" else a.imm_bits("b32")
    bits = mask_to_bool(m & M32)[:32]
    pre = np.concatenate([[0], np.cumsum(bits)])
    cnt = np.where(LANES < 32, 0, pre[np.clip(LANES - 32, 0, 32)])
    w.vset(d, (cnt + w.vget(b).astype(np.int64)).astype(U32))


@h("v_mov_b32")
def _(w, i):
    w.vset(i.ops[0], w.vget(i.ops[1]))


@h("v_mov_b64")
def _(w, i):
    w.vset64(i.ops[0], w.vget64(i.ops[1]))


@h("v_accvgpr_write_b32", "v_accvgpr_read_b32", "v_accvgpr_mov_b32")
def _(w, i):
    w.vset(i.ops[0], w.vget(i.ops[1]))


@h("v_cndmask_b32")
def _(w, i):
    d, a, b = i.ops[:3]
    sel = w.lanemask_get(i.ops[3]) if len(i.ops) > 3 else mask_to_bool(w.vcc)
    if a.abs or a.neg or b.abs or b.neg:
        x = np.where(sel, w.fget(b), w.fget(a))
        w.vset(d, x.view(U32))
    else:
        w.vset(d, np.where(sel, w.vget(b), w.vget(a)))


# ============================================================================
# VALU integer
def _u(w, o):
    return w.vget(o).astype(np.uint64)


def _i(w, o):
    return w.vget(o).view(I32).astype(np.int64)


def _wrap(r):
    return (np.asarray(r).astype(np.int64) & M32).astype(U32) if np.asarray(r).dtype != np.uint64 \
        else (r & U64(M32)).astype(U32)


def _vop(fn, nsrc):
    def run(w, i):
        srcs = [_u(w, o) for o in i.ops[1:1 + nsrc]]
        w.vset(i.ops[0], _wrap(fn(*srcs)))
    return run


_V = {
    "v_add_u32": (lambda a, b: a + b, 2),
    "v_sub_u32": (lambda a, b: a - b, 2),
    "v_subrev_u32": (lambda a, b: b - a, 2),
    "v_and_b32": (lambda a, b: a & b, 2),
    "v_or_b32": (lambda a, b: a | b, 2),
    "v_xor_b32": (lambda a, b: a ^ b, 2),
    "v_not_b32": (lambda a: ~a, 1),
    "v_lshlrev_b32": (lambda a, b: b << (a & U64(31)), 2),
    "v_lshrrev_b32": (lambda a, b: b >> (a & U64(31)), 2),
    "v_lshl_add_u32": (lambda a, b, c: (a << (b & U64(31))) + c, 3),
    "v_add_lshl_u32": (lambda a, b, c: ((a + b) & U64(M32)) << (c & U64(31)), 3),
    "v_lshl_or_b32": (lambda a, b, c: ((a << (b & U64(31))) & U64(M32)) | c, 3),
    "v_add3_u32": (lambda a, b, c: a + b + c, 3),
    "v_or3_b32": (lambda a, b, c: a | b | c, 3),
    "v_and_or_b32": (lambda a, b, c: (a & b) | c, 3),
    "v_xad_u32": (lambda a, b, c: (a ^ b) + c, 3),
    "v_bfi_b32": (lambda a, b, c: (a & b) | (~a & c), 3),
    "v_mul_lo_u32": (lambda a, b: a * b, 2),
    "v_mul_hi_u32": (lambda a, b: (a * b) >> U64(32), 2),
    "v_mul_u32_u24": (lambda a, b: (a & U64(0xFFFFFF)) * (b & U64(0xFFFFFF)), 2),
    # 16-bit integer ops (gfx9 family): low halves in, the high half of the
    # destination zeroed
    "v_mul_lo_u16": (lambda a, b: ((a & U64(0xFFFF)) * (b & U64(0xFFFF))) & U64(0xFFFF), 2),
    "v_add_u16": (lambda a, b: ((a & U64(0xFFFF)) + (b & U64(0xFFFF))) & U64(0xFFFF), 2),
    "v_sub_u16": (lambda a, b: ((a & U64(0xFFFF)) - (b & U64(0xFFFF))) & U64(0xFFFF), 2),
    "v_subrev_u16": (lambda a, b: ((b & U64(0xFFFF)) - (a & U64(0xFFFF))) & U64(0xFFFF), 2),
    "v_lshlrev_b16": (lambda a, b: ((b & U64(0xFFFF)) << (a & U64(15))) & U64(0xFFFF), 2),
    "v_lshrrev_b16": (lambda a, b: (b & U64(0xFFFF)) >> (a & U64(15)), 2),
    "v_max_u16": (lambda a, b: np.maximum(a & U64(0xFFFF), b & U64(0xFFFF)), 2),
    "v_min_u16": (lambda a, b: np.minimum(a & U64(0xFFFF), b & U64(0xFFFF)), 2),
    "v_mad_u16": (lambda a, b, c: ((a & U64(0xFFFF)) * (b & U64(0xFFFF)) + (c & U64(0xFFFF)))
                  & U64(0xFFFF), 3),
    "v_mad_u32_u24": (lambda a, b, c: (a & U64(0xFFFFFF)) * (b & U64(0xFFFFFF)) + c, 3),
    "v_min_u32": (lambda a, b: np.minimum(a, b), 2),
    "v_max_u32": (lambda a, b: np.maximum(a, b), 2),
    "v_bfe_u32": (lambda a, b, c: (a >> (b & U64(31))) & ((U64(1) << (c & U64(31))) - U64(1)), 3),
    "v_alignbit_b32": (lambda a, b, c: ((a << U64(32)) | b) >> (c & U64(31)), 3),
}
for _n, (_f, _k) in _V.items():
    HANDLERS[_n] = _vop(_f, _k)


@h("v_mul_hi_i32")
def _(w, i):
    d, a, b = i.ops
    w.vset(d, ((_i(w, a) * _i(w, b)) >> 32) & M32)


@h("v_ashrrev_i32")
def _(w, i):
    d, a, b = i.ops
    w.vset(d, (_i(w, b) >> (_u(w, a) & U64(31)).astype(np.int64)).astype(np.int64) & M32)


@h("v_mul_i32_i24")
def _(w, i):
    def s24(x):
        x = x & 0xFFFFFF
        return np.where(x & 0x800000, x - (1 << 24), x)
    r = s24(_i(w, i.ops[1])) * s24(_i(w, i.ops[2]))
    w.vset(i.ops[0], (r & M32).astype(U32))


@h("v_mad_i32_i24")
def _(w, i):
    def s24(x):
        x = x & 0xFFFFFF
        return np.where(x & 0x800000, x - (1 << 24), x)
    r = s24(_i(w, i.ops[1])) * s24(_i(w, i.ops[2])) + _i(w, i.ops[3])
    w.vset(i.ops[0], (r & M32).astype(U32))


@h("v_min_i32")
def _(w, i):
    w.vset(i.ops[0], (np.minimum(_i(w, i.ops[1]), _i(w, i.ops[2])) & M32).astype(U32))


@h("v_max_i32")
def _(w, i):
    w.vset(i.ops[0], (np.maximum(_i(w, i.ops[1]), _i(w, i.ops[2])) & M32).astype(U32))


@h("v_med3_i32")
def _(w, i):
    a, b, c = [_i(w, o) for o in i.ops[1:4]]
    r = np.maximum(np.minimum(a, b), np.minimum(np.maximum(a, b), c))
    w.vset(i.ops[0], (r & M32).astype(U32))


@h("v_bfrev_b32")
def _(w, i):
    a = w.vget(i.ops[1]).copy()
    r = np.zeros(64, np.uint64)
    for k in range(32):
        r |= ((a.astype(np.uint64) >> U64(k)) & U64(1)) << U64(31 - k)
    w.vset(i.ops[0], r.astype(U32))


@h("v_ffbh_u32")
def _(w, i):
    a = w.vget(i.ops[1]).astype(np.uint64)
    r = np.full(64, M32, np.uint64)
    for k in range(32):
        bit = (a >> U64(31 - k)) & U64(1)
        r = np.where((r == M32) & (bit == 1), U64(k), r)
    w.vset(i.ops[0], r.astype(U32))


@h("v_perm_b32")
def _(w, i):
    d, a, b, s = i.ops
    comb = (_u(w, a) << U64(32)) | _u(w, b)
    sel = _u(w, s)
    out = np.zeros(64, np.uint64)
    for k in range(4):
        sk = (sel >> U64(8 * k)) & U64(0xFF)
        byte = (comb >> (U64(8) * np.minimum(sk, U64(7)))) & U64(0xFF)
        byte = np.where(sk >= 13, U64(0xFF), np.where(sk == 12, U64(0), byte))
        if ((sk >= 8) & (sk <= 11)).any():
            raise EmuError("v_perm sign-replicate selectors not implemented")
        out |= byte << U64(8 * k)
    w.vset(d, out.astype(U32))


@h("v_bitop3_b32")
def _(w, i):
    d, a, b, c = i.ops
    tt = i.mods["bitop3"]
    A, B, C = _u(w, a), _u(w, b), _u(w, c)
    out = np.zeros(64, np.uint64)
    for k in range(8):
        if (tt >> k) & 1:
            ta = A if k & 4 else ~A
            tb = B if k & 2 else ~B
            tc = C if k & 1 else ~C
            out |= ta & tb & tc
    w.vset(d, (out & U64(M32)).astype(U32))


@h("v_and_b32")  # also the sdwa form
def _(w, i):
    a = _sdwa_src(w, i, 1, "src0_sel")
    b = _sdwa_src(w, i, 2, "src1_sel")
    if i.mods.get("dst_sel", "DWORD") != "DWORD":
        raise EmuError("sdwa dst_sel not implemented")
    w.vset(i.ops[0], (a & b).astype(U32))


def _sdwa_src(w, i, k, key):
    x = _u(w, i.ops[k])
    sel = i.mods.get(key, "DWORD")
    if sel == "DWORD":
        return x
    if sel == "WORD_0":
        return x & U64(0xFFFF)
    if sel == "WORD_1":
        return (x >> U64(16)) & U64(0xFFFF)
    if sel.startswith("BYTE_"):
        return (x >> U64(8 * int(sel[5:]))) & U64(0xFF)
    raise EmuError(f"sdwa sel {sel}")


# carry ops: (dst, carry-out, src0, src1[, carry-in])
@h("v_add_co_u32")
def _(w, i):
    d, cd, a, b = i.ops[:4]
    r = _u(w, a) + _u(w, b)
    w.vset(d, (r & U64(M32)).astype(U32))
    w.lanemask_set(cd, (r >> U64(32)) != 0)


@h("v_addc_co_u32")
def _(w, i):
    d, cd, a, b, ci = i.ops[:5]
    c = w.lanemask_get(ci).astype(np.uint64)
    r = _u(w, a) + _u(w, b) + c
    w.vset(d, (r & U64(M32)).astype(U32))
    w.lanemask_set(cd, (r >> U64(32)) != 0)


@h("v_sub_co_u32")
def _(w, i):
    d, cd, a, b = i.ops[:4]
    A, B = _u(w, a), _u(w, b)
    w.vset(d, ((A - B) & U64(M32)).astype(U32))
    w.lanemask_set(cd, B > A)


@h("v_subrev_co_u32")
def _(w, i):
    d, cd, a, b = i.ops[:4]
    A, B = _u(w, b), _u(w, a)
    w.vset(d, ((A - B) & U64(M32)).astype(U32))
    w.lanemask_set(cd, B > A)


@h("v_subb_co_u32")
def _(w, i):
    d, cd, a, b, ci = i.ops[:5]
    c = w.lanemask_get(ci).astype(np.int64)
    A, B = _u(w, a).astype(np.int64), _u(w, b).astype(np.int64)
    r = A - B - c
    w.vset(d, (r & M32).astype(U32))
    w.lanemask_set(cd, r < 0)


@h("v_subbrev_co_u32")
def _(w, i):
    d, cd, a, b, ci = i.ops[:5]
    c = w.lanemask_get(ci).astype(np.int64)
    A, B = _u(w, b).astype(np.int64), _u(w, a).astype(np.int64)
    r = A - B - c
    w.vset(d, (r & M32).astype(U32))
    w.lanemask_set(cd, r < 0)


@h("v_mad_u64_u32")
def _(w, i):
    d, cd, a, b, c = i.ops
    A = [int(x) for x in w.vget(a)]
    B = [int(x) for x in w.vget(b)]
    C = [int(x) for x in w.vget64(c)]
    r = [A[k] * B[k] + C[k] for k in range(64)]
    w.vset64(d, np.array([x & M64 for x in r], np.uint64))
    w.lanemask_set(cd, np.array([x >> 64 != 0 for x in r]))


@h("v_mad_i64_i32")
def _(w, i):
    d, cd, a, b, c = i.ops
    A = [sext32(int(x)) for x in w.vget(a)]
    B = [sext32(int(x)) for x in w.vget(b)]
    C64 = w.vget64(c) if c.kind in "va" else np.full(
        64, w.sget(c, "b64") if c.kind == "s" else c.imm_bits("b64"), np.uint64)
    C = [int(x) - (1 << 64) if int(x) >> 63 else int(x) for x in C64]
    r = [A[k] * B[k] + C[k] for k in range(64)]
    w.vset64(d, np.array([x & M64 for x in r], np.uint64))
    w.lanemask_set(cd, np.array([not (-(1 << 63) <= x < (1 << 63)) for x in r]))


@h("v_lshlrev_b64")
def _(w, i):
    d, a, b = i.ops
    s = _u(w, a) & U64(63)
    w.vset64(d, w.vget64(b) << s)


@h("v_lshrrev_b64")
def _(w, i):
    d, a, b = i.ops
    s = _u(w, a) & U64(63)
    w.vset64(d, w.vget64(b) >> s)


@h("v_lshl_add_u64")
def _(w, i):
    d, a, b, c = i.ops
    A = w.vget64(a)
    s = _u(w, b) & U64(7)
    C = w.vget64(c) if c.kind != "imm" else np.full(64, c.imm_bits("b64"), np.uint64)
    with _err_np():
        w.vset64(d, (A << s) + C)


# ============================================================================
# VOPC
def _vcmp(fn, ty):
    def run(w, i):
        d, a, b = i.ops[0], i.ops[1], i.ops[2]
        if ty == "f32":
            A, B = w.fget(a), w.fget(b)
        elif ty == "f64":
            A, B = w.dget(a), w.dget(b)
        elif ty == "i32":
            A, B = _i(w, a), _i(w, b)
        elif ty == "u32":
            A, B = _u(w, a), _u(w, b)
        elif ty == "i64":
            A, B = w.vget64(a, "i64").view(np.int64), w.vget64(b, "i64").view(np.int64)
        elif ty == "u64":
            A, B = w.vget64(a, "u64"), w.vget64(b, "u64")
        with _err_np():
            r = fn(A, B)
        w.lanemask_set(d, r)
    return run


_FCMP = {
    "eq": lambda a, b: a == b, "lt": lambda a, b: a < b, "le": lambda a, b: a <= b,
    "gt": lambda a, b: a > b, "ge": lambda a, b: a >= b, "lg": lambda a, b: (a < b) | (a > b),
    "neq": lambda a, b: ~(a == b), "nlt": lambda a, b: ~(a < b), "nle": lambda a, b: ~(a <= b),
    "ngt": lambda a, b: ~(a > b), "nge": lambda a, b: ~(a >= b), "nlg": lambda a, b: ~((a < b) | (a > b)),
    "o": lambda a, b: ~(np.isnan(a) | np.isnan(b)), "u": lambda a, b: np.isnan(a) | np.isnan(b),
}
_ICMP = {"eq": lambda a, b: a == b, "ne": lambda a, b: a != b, "lt": lambda a, b: a < b,
         "le": lambda a, b: a <= b, "gt": lambda a, b: a > b, "ge": lambda a, b: a >= b}
for _c, _f in _FCMP.items():
    for _t in ("f32", "f64"):
        HANDLERS[f"v_cmp_{_c}_{_t}"] = _vcmp(_f, _t)
for _c, _f in _ICMP.items():
    for _t in ("i32", "u32", "i64", "u64"):
        HANDLERS[f"v_cmp_{_c}_{_t}"] = _vcmp(_f, _t)


def _fclass(x, mask):
    x = np.asarray(x)
    r = np.zeros(x.shape, bool)
    fin = np.isfinite(x)
    tiny = np.finfo(x.dtype).tiny
    sign = np.signbit(x)
    nan = np.isnan(x)
    tests = [
        nan & False,                                   # 0 signaling NaN (treated as none)
        nan,                                           # 1 quiet NaN
        np.isinf(x) & sign,                            # 2 -inf
        fin & sign & (np.abs(x) >= tiny),              # 3 -normal
        fin & sign & (np.abs(x) < tiny) & (x != 0),    # 4 -denorm
        (x == 0) & sign,                               # 5 -0
        (x == 0) & ~sign,                              # 6 +0
        fin & ~sign & (np.abs(x) < tiny) & (x != 0),   # 7 +denorm
        fin & ~sign & (np.abs(x) >= tiny),             # 8 +normal
        np.isinf(x) & ~sign,                           # 9 +inf
    ]
    for k, t in enumerate(tests):
        r |= t & (((mask >> k) & 1) != 0)
    return r


def _vcmp_class(ty):
    def run(w, i):
        d, a, b = i.ops[0], i.ops[1], i.ops[2]
        x = w.fget(a) if ty == "f32" else w.dget(a)
        m = _u(w, b)
        w.lanemask_set(d, _fclass(x, m))
    return run


HANDLERS["v_cmp_class_f32"] = _vcmp_class("f32")
HANDLERS["v_cmp_class_f64"] = _vcmp_class("f64")


# ============================================================================
# VALU float32
def _fop(fn, nsrc):
    def run(w, i):
        srcs = [w.fget(o) for o in i.ops[1:1 + nsrc]]
        with _err_np():
            r = np.asarray(fn(*srcs), dtype=np.float64).astype(F32)
        if i.mods.get("clamp"):
            r = np.clip(r, 0, 1).astype(F32)
        w.vset(i.ops[0], r.view(U32))
    return run


def _fma(a, b, c):
    return a.astype(F64) * b.astype(F64) + c.astype(F64)


def _maxf(a, b):
    return np.fmax(a, b)


_F = {
    "v_add_f32": (lambda a, b: a + b, 2),
    "v_sub_f32": (lambda a, b: a - b, 2),
    "v_subrev_f32": (lambda a, b: b - a, 2),
    "v_mul_f32": (lambda a, b: a * b, 2),
    "v_max_f32": (_maxf, 2),
    "v_min_f32": (lambda a, b: np.fmin(a, b), 2),
    "v_max3_f32": (lambda a, b, c: np.fmax(np.fmax(a, b), c), 3),
    "v_min3_f32": (lambda a, b, c: np.fmin(np.fmin(a, b), c), 3),
    "v_fma_f32": (_fma, 3),
    "v_exp_f32": (lambda a: np.exp2(a.astype(F64)), 1),
    "v_log_f32": (lambda a: np.log2(a.astype(F64)), 1),
    "v_rcp_f32": (lambda a: 1.0 / a.astype(F64), 1),
    "v_rcp_iflag_f32": (lambda a: 1.0 / a.astype(F64), 1),
    "v_rsq_f32": (lambda a: 1.0 / np.sqrt(a.astype(F64)), 1),
    "v_sqrt_f32": (lambda a: np.sqrt(a.astype(F64)), 1),
    "v_trunc_f32": (lambda a: np.trunc(a), 1),
    "v_floor_f32": (lambda a: np.floor(a), 1),
    "v_rndne_f32": (lambda a: np.rint(a), 1),
    "v_fract_f32": (lambda a: a - np.floor(a), 1),
}
for _n, (_f, _k) in _F.items():
    HANDLERS[_n] = _fop(_f, _k)


# the f32 add/sub/mul must round once in f32: numpy f32 arithmetic does
def _fop32(fn):
    def run(w, i):
        a, b = w.fget(i.ops[1]), w.fget(i.ops[2])
        with _err_np():
            r = fn(a, b).astype(F32)
        w.vset(i.ops[0], r.view(U32))
    return run


HANDLERS["v_add_f32"] = _fop32(lambda a, b: a + b)
HANDLERS["v_sub_f32"] = _fop32(lambda a, b: a - b)
HANDLERS["v_subrev_f32"] = _fop32(lambda a, b: b - a)
HANDLERS["v_mul_f32"] = _fop32(lambda a, b: a * b)


@h("v_fmac_f32")
def _(w, i):
    d, a, b = i.ops
    c = w.fget(d)
    r = _fma(w.fget(a), w.fget(b), c).astype(F32)
    w.vset(d, r.view(U32))


@h("v_fmamk_f32")
def _(w, i):
    d, a, k, b = i.ops
    kk = np.full(64, k.imm_bits("f32"), U32).view(F32)
    r = _fma(w.fget(a), kk, w.fget(b)).astype(F32)
    w.vset(d, r.view(U32))


@h("v_fmaak_f32")
def _(w, i):
    d, a, b, k = i.ops
    kk = np.full(64, k.imm_bits("f32"), U32).view(F32)
    r = _fma(w.fget(a), w.fget(b), kk).astype(F32)
    w.vset(d, r.view(U32))


@h("v_ldexp_f32")
def _(w, i):
    d, a, b = i.ops
    with _err_np():
        r = np.ldexp(w.fget(a).astype(F64), np.clip(_i(w, b), -400, 400)).astype(F32)
    w.vset(d, r.view(U32))


@h("v_cvt_f32_u32")
def _(w, i):
    w.vset(i.ops[0], _u(w, i.ops[1]).astype(F32).view(U32))


@h("v_cvt_f32_i32")
def _(w, i):
    w.vset(i.ops[0], _i(w, i.ops[1]).astype(F32).view(U32))


def _f2int(x, lo, hi):
    x = np.asarray(x, F64)
    r = np.where(np.isnan(x), 0, np.clip(np.trunc(np.nan_to_num(x)), lo, hi))
    return r.astype(np.int64)


@h("v_cvt_u32_f32")
def _(w, i):
    w.vset(i.ops[0], (_f2int(w.fget(i.ops[1]), 0, M32) & M32).astype(U32))


@h("v_cvt_i32_f32")
def _(w, i):
    w.vset(i.ops[0], (_f2int(w.fget(i.ops[1]), -2**31, 2**31 - 1) & M32).astype(U32))


@h("v_cvt_pk_bf16_f32")
def _(w, i):
    d, a, b = i.ops
    lo = bf16_rne(w.fget(a))
    hi = bf16_rne(w.fget(b))
    w.vset(d, (lo | (hi << 16)).astype(U32))


@h("v_div_scale_f32")
def _(w, i):
    d, cd, a, b, c = i.ops
    A, B, C = w.fget(a), w.fget(b), w.fget(c)
    m = w.exec_mask()
    _check_div_range(np.abs(B[m]), np.abs(C[m]), "f32")
    w.vset(d, A.view(U32))
    w.lanemask_set(cd, np.zeros(64, bool))


@h("v_div_fmas_f32")
def _(w, i):
    d, a, b, c = i.ops
    r = _fma(w.fget(a), w.fget(b), w.fget(c)).astype(F32)
    w.vset(d, r.view(U32))


def _check_div_range(den, num, ty):
    lo, hi = (2.0 ** -60, 2.0 ** 60)
    bad_den = (den < lo) | (den > hi) | ~np.isfinite(den)
    bad_num = ((num != 0) & ((num < lo) | (num > hi))) | ~np.isfinite(num)
    if bad_den.any() or bad_num.any():
        raise EmuError(f"division operands outside the emulated range ({ty}): "
                       f"den {den[bad_den][:3]} num {num[bad_num][:3]}")


def _div_fixup(q, den, num, dt):
    sign = np.signbit(den) ^ np.signbit(num)
    r = np.abs(q).astype(dt)
    r = np.where(sign, -r, r)
    r = np.where(num == 0, np.where(sign, -0.0, 0.0).astype(dt), r)
    r = np.where(np.isnan(num), num, r)
    r = np.where(np.isnan(den), den, r)
    return r.astype(dt)


@h("v_div_fixup_f32")
def _(w, i):
    d, a, b, c = i.ops
    r = _div_fixup(w.fget(a), w.fget(b), w.fget(c), F32)
    w.vset(d, r.view(U32))


# ============================================================================
# VALU float64
def _dop(fn, nsrc):
    def run(w, i):
        srcs = [w.dget(o) for o in i.ops[1:1 + nsrc]]
        with _err_np():
            r = np.asarray(fn(*srcs), F64)
        w.dset(i.ops[0], r)
    return run


def _fma64(a, b, c):
    # fused multiply-add in extended precision, then rounded to float64
    return (a.astype(np.longdouble) * b.astype(np.longdouble) + c.astype(np.longdouble)).astype(F64)


_D = {
    "v_add_f64": (lambda a, b: a + b, 2),
    "v_mul_f64": (lambda a, b: a * b, 2),
    "v_fma_f64": (_fma64, 3),
    "v_rcp_f64": (lambda a: 1.0 / a, 1),
    "v_rsq_f64": (lambda a: 1.0 / np.sqrt(a), 1),
    "v_sqrt_f64": (lambda a: np.sqrt(a), 1),
    "v_floor_f64": (lambda a: np.floor(a), 1),
    "v_trunc_f64": (lambda a: np.trunc(a), 1),
    "v_rndne_f64": (lambda a: np.rint(a), 1),
    "v_fract_f64": (lambda a: a - np.floor(a), 1),
    "v_max_f64": (lambda a, b: np.fmax(a, b), 2),
    "v_min_f64": (lambda a, b: np.fmin(a, b), 2),
}
for _n, (_f, _k) in _D.items():
    HANDLERS[_n] = _dop(_f, _k)


@h("v_fmac_f64")
def _(w, i):
    d, a, b = i.ops
    w.dset(d, _fma64(w.dget(a), w.dget(b), w.dget(d)))


@h("v_ldexp_f64")
def _(w, i):
    d, a, b = i.ops
    with _err_np():
        w.dset(d, np.ldexp(w.dget(a), np.clip(_i(w, b), -3000, 3000)))


@h("v_frexp_mant_f64")
def _(w, i):
    x = w.dget(i.ops[1])
    m, e = np.frexp(x)
    m = np.where(np.isfinite(x), m, x)
    w.dset(i.ops[0], m)


@h("v_frexp_exp_i32_f64")
def _(w, i):
    x = w.dget(i.ops[1])
    m, e = np.frexp(np.where(np.isfinite(x), x, 0))
    w.vset(i.ops[0], (e.astype(np.int64) & M32).astype(U32))


@h("v_cvt_f64_f32")
def _(w, i):
    w.dset(i.ops[0], w.fget(i.ops[1]).astype(F64))


@h("v_cvt_f32_f64")
def _(w, i):
    with _err_np():
        w.vset(i.ops[0], w.dget(i.ops[1]).astype(F32).view(U32))


@h("v_cvt_f64_i32")
def _(w, i):
    w.dset(i.ops[0], _i(w, i.ops[1]).astype(F64))


@h("v_cvt_f64_u32")
def _(w, i):
    w.dset(i.ops[0], _u(w, i.ops[1]).astype(F64))


@h("v_cvt_i32_f64")
def _(w, i):
    w.vset(i.ops[0], (_f2int(w.dget(i.ops[1]), -2**31, 2**31 - 1) & M32).astype(U32))


@h("v_cvt_u32_f64")
def _(w, i):
    w.vset(i.ops[0], (_f2int(w.dget(i.ops[1]), 0, M32) & M32).astype(U32))


@h("v_div_scale_f64")
def _(w, i):
    d, cd, a, b, c = i.ops
    A, B, C = w.dget(a), w.dget(b), w.dget(c)
    m = w.exec_mask()
    _check_div_range(np.abs(B[m]), np.abs(C[m]), "f64")
    w.dset(d, A)
    w.lanemask_set(cd, np.zeros(64, bool))


@h("v_div_fmas_f64")
def _(w, i):
    d, a, b, c = i.ops
    w.dset(d, _fma64(w.dget(a), w.dget(b), w.dget(c)))


@h("v_div_fixup_f64")
def _(w, i):
    d, a, b, c = i.ops
    w.dset(d, _div_fixup(w.dget(a), w.dget(b), w.dget(c), F64))


# ============================================================================
# MFMA
def _mfma_idx(M):
    """Lane/element -> (row, k) of A (also (col, k) of B) and (row, col) of D for
    the bf16 MFMA shapes 32x32x16 (M = 32) and 16x16x32 (M = 16)."""
    if M == 32:
        a_m = np.repeat(LANES % 32, 8).reshape(64, 8)
        a_k = (8 * (LANES // 32))[:, None] + np.arange(8)[None, :]
        d_m = np.array([[8 * (r // 4) + 4 * (l // 32) + r % 4 for r in range(16)] for l in range(64)])
        d_n = np.repeat(LANES % 32, 16).reshape(64, 16)
    else:
        a_m = np.repeat(LANES % 16, 8).reshape(64, 8)
        a_k = (8 * (LANES // 16))[:, None] + np.arange(8)[None, :]
        d_m = np.array([[4 * (l // 16) + r for r in range(4)] for l in range(64)])
        d_n = np.repeat(LANES % 16, 4).reshape(64, 4)
    return a_m, a_k, d_m, d_n


_MF = {32: _mfma_idx(32), 16: _mfma_idx(16)}


def _read_bf16x8(w, o):
    regs = [w.vget(o, "b32", k) for k in range(4)]
    r = np.stack(regs, 1).astype(U32)           # [64, 4]
    lo = r & 0xFFFF
    hi = r >> 16
    h16 = np.stack([lo, hi], 2).reshape(64, 8)  # element 2k = low half of reg k
    return bf16_to_f32(h16).astype(F64)


def _mfma(M):
    N, K, nreg = (32, 16, 16) if M == 32 else (16, 32, 4)
    a_m, a_k, d_m, d_n = _MF[M]

    def run(w, i):
        d, a, b, c = i.ops
        if w.exec != (1 << 64) - 1:
            w.emu.stats.warnings.append(f"MFMA with partial exec at line {i.line}")
        if i.in_asm:
            # operands written by a VALU too recently; the accumulator may be
            # the previous MFMA's result only when it is exactly that range
            for o, n in ((a, 4), (b, 4), (c, nreg)):
                if o.kind not in ("v", "a"):
                    continue
                for k in range(n):
                    r = w.vrow(o, k)
                    t = w.valu_vgpr_write.get(r)
                    if t is not None and w.clock - t - 1 < VALU_TO_XDL_WAITS:
                        raise EmuError(f"MFMA reads v{r} {w.clock - t - 1} wait states after a "
                                       f"VALU wrote it (needs {VALU_TO_XDL_WAITS})")
        Av = _read_bf16x8(w, a)
        Bv = _read_bf16x8(w, b)
        Am = np.zeros((M, K))
        Bm = np.zeros((K, N))
        Am[a_m, a_k] = Av
        Bm[a_k, a_m] = Bv          # B[k][n]: same lane pattern with n = lane % M
        if c.kind == "imm" and c.ival == 0:
            Cm = np.zeros((M, N))
        else:
            w.in_mfma_srcc = c.kind == d.kind and c.idx == d.idx
            try:
                Cl = np.stack([f32(w.vget(c, "b32", r)) for r in range(nreg)], 1).astype(F64)
            finally:
                w.in_mfma_srcc = False
            Cm = np.zeros((M, N))
            Cm[d_m, d_n] = Cl
        D = (Am @ Bm + Cm).astype(F32)
        out = D[d_m, d_n]       # [64, nreg]
        full = np.ones(64, bool)
        for r in range(nreg):
            w.vset(d, out[:, r].view(U32), r, mask=full)
        if i.in_asm:
            for r in range(nreg):
                w.xdl_write[w.vrow(d, r)] = w.clock
        else:
            for r in range(nreg):
                w.xdl_write.pop(w.vrow(d, r), None)
    return run


HANDLERS["v_mfma_f32_32x32x16_bf16"] = _mfma(32)
HANDLERS["v_mfma_f32_16x16x32_bf16"] = _mfma(16)


# ============================================================================
# LDS
def lds_mark(w, idx, kind, what):
    wg = w.wg
    me = w.wid
    ep = wg.epoch
    if kind == "r":
        bad = (wg.w_epoch[idx] == ep) & (wg.w_wave[idx] != me) & (wg.w_wave[idx] >= 0)
        if bad.any():
            j = idx[bad][0]
            raise EmuError(f"{what}: LDS race, dword {j} written by wave {wg.w_wave[j]} "
                           f"and read by wave {me} in the same barrier interval")
        same = wg.r_epoch[idx] == ep
        wg.r_mask[idx] = np.where(same, wg.r_mask[idx], 0) | (1 << me)
        wg.r_epoch[idx] = ep
    else:
        bad = (wg.w_epoch[idx] == ep) & (wg.w_wave[idx] != me) & (wg.w_wave[idx] >= 0)
        if bad.any():
            j = idx[bad][0]
            raise EmuError(f"{what}: LDS race, dword {j} written by waves {wg.w_wave[j]} "
                           f"and {me} in the same barrier interval")
        bad = (wg.r_epoch[idx] == ep) & ((wg.r_mask[idx] & ~(1 << me)) != 0)
        if bad.any():
            j = idx[bad][0]
            raise EmuError(f"{what}: LDS race, dword {j} read by waves mask "
                           f"{int(wg.r_mask[j]):#x} and written by wave {me} in the same "
                           f"barrier interval")
        wg.w_wave[idx] = me
        wg.w_epoch[idx] = ep


def lds_check(w, offs, nbytes, kind, what):
    """offs: int64 byte offsets of active lanes -> dword index array."""
    wg = w.wg
    if len(offs) == 0:
        return np.zeros(0, np.int64)
    if (offs < 0).any() or (offs + nbytes > wg.lds_size).any():
        bad = offs[(offs < 0) | (offs + nbytes > wg.lds_size)]
        raise EmuError(f"{what}: LDS access at {int(bad[0])} (+{nbytes}) outside the "
                       f"{wg.lds_size}-byte allocation")
    nd = max(nbytes // 4, 1)
    idx = (offs[:, None] // 4 + np.arange(nd)[None, :]).reshape(-1)
    if (wg.dma_pending[idx] > 0).any():
        raise EmuError(f"{what}: LDS bytes touched while an LDS DMA into them is in flight")
    if kind != "atomic":
        lds_mark(w, np.unique(idx), kind, what)
    return idx


def _lds_addr(w, i, aop, key="offset"):
    base = w.vget(aop).astype(np.int64)
    return base + int(i.mods.get(key, 0))


def _dsread(nb):
    def run(w, i):
        d, a = i.ops
        m = w.exec_mask()
        offs = _lds_addr(w, i, a)[m]
        lds_check(w, offs, nb, "r", i.text)
        data = w.wg.lds[offs[:, None] + np.arange(nb)[None, :]].copy()
        nd = nb // 4
        vals = data.view("<u4").reshape(-1, nd) if len(offs) else np.zeros((0, nd), U32)
        rows = [w.vrow(d, k) for k in range(nd)]

        def apply():
            for k, r in enumerate(rows):
                w.V[r, m] = vals[:, k]
        push_lgkm(w, Pend(w, vrows=rows, apply=apply, what=i.text))
    return run


HANDLERS["ds_read_b32"] = _dsread(4)
HANDLERS["ds_read_b64"] = _dsread(8)
HANDLERS["ds_read_b128"] = _dsread(16)


def _dsread2(nb, stride):
    """ds_read2[st64]_b32/b64: two nb-byte elements at addr + offset0*stride
    and addr + offset1*stride (stride = element size, times 64 for st64)."""
    def run(w, i):
        d, a = i.ops
        m = w.exec_mask()
        base = w.vget(a).astype(np.int64)[m]
        nd = nb // 4
        vals = []
        for key in ("offset0", "offset1"):
            o = base + stride * int(i.mods.get(key, 0))
            lds_check(w, o, nb, "r", i.text)
            vals.append(w.wg.lds[o[:, None] + np.arange(nb)].copy().view("<u4").reshape(-1, nd))
        rows = [w.vrow(d, k) for k in range(2 * nd)]

        def apply():
            for k in range(nd):
                w.V[rows[k], m] = vals[0][:, k]
                w.V[rows[nd + k], m] = vals[1][:, k]
        push_lgkm(w, Pend(w, vrows=rows, apply=apply, what=i.text))
    return run


HANDLERS["ds_read2_b32"] = _dsread2(4, 4)
HANDLERS["ds_read2st64_b32"] = _dsread2(4, 256)
HANDLERS["ds_read2_b64"] = _dsread2(8, 8)
HANDLERS["ds_read2st64_b64"] = _dsread2(8, 512)


def _dswrite(nb, hi16=False):
    """ds_write_b32/b64/b128 and the 16-bit forms (ds_write_b16 stores bits
    15:0 of the data VGPR, ds_write_b16_d16_hi bits 31:16)."""
    def run(w, i):
        a, d = i.ops
        m = w.exec_mask()
        offs = _lds_addr(w, i, a)[m]
        lds_check(w, offs, nb, "w", i.text)
        if nb >= 4:
            vals = np.stack([w.vget(d, "b32", k)[m] for k in range(nb // 4)], 1).astype("<u4")
            b = vals.view(np.uint8).reshape(-1, nb)
        else:
            x = w.vget(d)[m]
            x = (x >> 16) if hi16 else x
            b = (x & 0xFFFF).astype("<u2").view(np.uint8).reshape(-1, 2)
        # lane order: later lanes win on overlap
        for k in range(len(offs)):
            w.wg.lds[offs[k]:offs[k] + nb] = b[k]
        push_lgkm(w, Pend(w, what=i.text))
    return run


def _dswrite2(nb, stride):
    """ds_write2[st64]_b32/b64: data0 at addr + offset0*stride, data1 at
    addr + offset1*stride (stride = element size, times 64 for st64)."""
    def run(w, i):
        a, d0, d1 = i.ops
        m = w.exec_mask()
        base = w.vget(a).astype(np.int64)[m]
        nd = nb // 4
        for key, d in (("offset0", d0), ("offset1", d1)):
            offs = base + stride * int(i.mods.get(key, 0))
            lds_check(w, offs, nb, "w", i.text)
            vals = np.stack([w.vget(d, "b32", k)[m] for k in range(nd)], 1).astype("<u4")
            b = vals.view(np.uint8).reshape(-1, nb)
            for k in range(len(offs)):
                w.wg.lds[offs[k]:offs[k] + nb] = b[k]
        push_lgkm(w, Pend(w, what=i.text))
    return run


HANDLERS["ds_write2_b32"] = _dswrite2(4, 4)
HANDLERS["ds_write2_b64"] = _dswrite2(8, 8)
HANDLERS["ds_write2st64_b32"] = _dswrite2(4, 256)
HANDLERS["ds_write2st64_b64"] = _dswrite2(8, 512)
HANDLERS["ds_write_b32"] = _dswrite(4)
HANDLERS["ds_write_b64"] = _dswrite(8)
HANDLERS["ds_write_b128"] = _dswrite(16)
HANDLERS["ds_write_b16"] = _dswrite(2)
HANDLERS["ds_write_b16_d16_hi"] = _dswrite(2, hi16=True)


@h("ds_add_f32")
def _(w, i):
    a, d = i.ops
    m = w.exec_mask()
    offs = _lds_addr(w, i, a)[m]
    idx = lds_check(w, offs, 4, "atomic", i.text)
    vals = f32(w.vget(d))[m]
    lds = w.wg.lds
    for k in range(len(offs)):
        o = offs[k]
        cur = lds[o:o + 4].view(F32)[0]
        lds[o:o + 4] = np.array([F32(cur + vals[k])], F32).view(np.uint8)
    push_lgkm(w, Pend(w, what=i.text))


@h("ds_bpermute_b32")
def _(w, i):
    d, a, s = i.ops
    m = w.exec_mask()
    addr = (w.vget(a).astype(np.int64) + int(i.mods.get("offset", 0)))
    src_lane = (addr // 4) % 64
    data = w.vget(s).copy()
    if (~m[src_lane[m]]).any():
        w.emu.stats.warnings.append(f"bpermute reads an inactive lane (line {i.line})")
    vals = data[src_lane]
    row = w.vrow(d)

    def apply():
        w.V[row, m] = vals[m]
    push_lgkm(w, Pend(w, vrows=[row], apply=apply, what=i.text))


@h("ds_read_b64_tr_b16")
def _(w, i):
    d, a = i.ops
    m = w.exec_mask()
    if not m.all():
        raise EmuError("ds_read_b64_tr_b16 with partial exec not modelled")
    offs = _lds_addr(w, i, a)
    if (offs % 8).any():
        raise EmuError("ds_read_b64_tr_b16 address not 8-byte aligned")
    lds_check(w, offs, 8, "r", i.text)
    blocks = w.wg.lds[offs[:, None] + np.arange(8)].copy().view("<u2").reshape(64, 4)
    res = np.zeros((64, 4), np.uint16)
    for lane in range(64):
        g, li = divmod(lane, 16)
        for e in range(4):
            res[lane, e] = blocks[16 * g + 4 * e + li // 4, li % 4]
    r32 = res.view("<u4").reshape(64, 2)
    rows = [w.vrow(d, 0), w.vrow(d, 1)]

    def apply():
        w.V[rows[0]] = r32[:, 0]
        w.V[rows[1]] = r32[:, 1]
    push_lgkm(w, Pend(w, vrows=rows, apply=apply, what=i.text))


# ============================================================================
# global / flat / scratch
def _gaddr(w, i, vop, sop):
    """Per-lane 64-bit addresses for global_* with vaddr/saddr forms."""
    off = int(i.mods.get("offset", 0))
    if sop is None or sop.kind == "off":
        a = w.vget64(vop).astype(np.int64)
    else:
        base = w.sget(sop, "b64")
        a = np.int64(base) + w.vget(vop).astype(np.int64)
    return (a + off).astype(np.uint64)


def _gload(nb, signed=False):
    def run(w, i):
        d, v, s = i.ops[0], i.ops[1], i.ops[2]
        check_vmem_sgpr_hazard(w, i, [s])
        m = w.exec_mask()
        addrs = _gaddr(w, i, v, s)[m]
        data = w.emu.mem.read(addrs, nb, i.text)
        if nb >= 4:
            vals = data.view("<u4").reshape(-1, nb // 4)
        else:
            vals = data.view("<u2" if nb == 2 else "u1").reshape(-1, 1).astype(U32)
        nd = max(nb // 4, 1)
        rows = [w.vrow(d, k) for k in range(nd)]

        def apply():
            for k, r in enumerate(rows):
                w.V[r, m] = vals[:, k]
        push_vm(w, Pend(w, vrows=rows, apply=apply, what=i.text))
    return run


HANDLERS["global_load_dword"] = _gload(4)
HANDLERS["global_load_dwordx2"] = _gload(8)
HANDLERS["global_load_dwordx3"] = _gload(12)
HANDLERS["global_load_dwordx4"] = _gload(16)
HANDLERS["global_load_ushort"] = _gload(2)
HANDLERS["global_load_ubyte"] = _gload(1)


def _gstore(nb, hi16=False):
    def run(w, i):
        v, d, s = i.ops[0], i.ops[1], i.ops[2]
        check_vmem_sgpr_hazard(w, i, [s])
        m = w.exec_mask()
        addrs = _gaddr(w, i, v, s)[m]
        if nb >= 4:
            vals = np.stack([w.vget(d, "b32", k)[m] for k in range(nb // 4)], 1).astype("<u4")
            b = vals.view(np.uint8).reshape(-1, nb)
        else:
            x = w.vget(d)[m]
            x = (x >> 16) if hi16 else x
            b = (x & 0xFFFF).astype("<u2").view(np.uint8).reshape(-1, 2)
        w.emu.mem.write(addrs, b, i.text)
        push_vm(w, Pend(w, what=i.text))
    return run


HANDLERS["global_store_dword"] = _gstore(4)
HANDLERS["global_store_dwordx2"] = _gstore(8)
HANDLERS["global_store_dwordx3"] = _gstore(12)
HANDLERS["global_store_dwordx4"] = _gstore(16)
HANDLERS["global_store_short"] = _gstore(2)
HANDLERS["global_store_short_d16_hi"] = _gstore(2, hi16=True)


@h("global_atomic_or")
def _(w, i):
    v, d, s = i.ops[:3]
    if i.mods.get("sc0") or i.mods.get("glc"):
        raise EmuError("returning atomics not modelled")
    check_vmem_sgpr_hazard(w, i, [s])
    m = w.exec_mask()
    addrs = _gaddr(w, i, v, s)[m]
    vals = w.vget(d)[m]
    for k in range(len(addrs)):
        cur = np.frombuffer(w.emu.mem.read(addrs[k:k + 1], 4, i.text)[0].tobytes(), "<u4")[0]
        nv = np.array([cur | vals[k]], "<u4").view(np.uint8).reshape(1, 4)
        w.emu.mem.write(addrs[k:k + 1], nv, i.text)
    push_vm(w, Pend(w, what=i.text))


def _gload_lds(nb):
    def run(w, i):
        v, s = i.ops[0], i.ops[1]
        check_vmem_sgpr_hazard(w, i, [s])
        if w.clock - w.salu_m0_write - 1 < 1 and i.in_asm:
            raise EmuError("LDS DMA issued right after an M0 write (needs 1 wait state)")
        m = w.exec_mask()
        addrs = _gaddr(w, i, v, s)
        data = w.emu.mem.read(addrs[m], nb, i.text)
        m0 = w.S[124] & 0x3FFFF
        ioff = int(i.mods.get("offset", 0))
        lds_off = (m0 + ioff + nb * np.arange(64))[m].astype(np.int64)
        wg = w.wg
        if (lds_off + nb > wg.lds_size).any() or (lds_off < 0).any():
            raise EmuError(f"LDS DMA target {int(lds_off.max())}+{nb} outside "
                           f"{wg.lds_size}-byte LDS (M0={m0:#x})")
        idx = (lds_off[:, None] // 4 + np.arange(nb // 4)[None, :]).reshape(-1)
        if (wg.dma_pending[idx] > 0).any():
            raise EmuError("LDS DMA into bytes with another DMA still in flight")
        lds_mark(w, np.unique(idx), "w", i.text + " (issue)")
        wg.dma_pending[idx] += 1
        w.emu.stats.lds_dma += 1
        push_vm(w, Pend(w, dma=(idx, data.reshape(-1, 4)), what=i.text))
    return run


HANDLERS["global_load_lds_dword"] = _gload_lds(4)
HANDLERS["global_load_lds_dwordx4"] = _gload_lds(16)


def _bload_lds(nb):
    """buffer_load_dword{,x4} vaddr, s[r:r+3], soffset offen lds: a raw
    (stride 0) buffer load into LDS at M0 + nb * lane.  Only the forms the
    kernels use are accepted; an access that leaves the descriptor's range is
    an error here (the hardware would return zeros), as is a descriptor with
    the zero data format (which reads zeros)."""
    def run(w, i):
        if not i.mods.get("lds"):
            raise EmuError(f"buffer load without lds is not modelled: {i.text}")
        if i.mods.get("idxen") or int(i.mods.get("offset", 0)) != 0:
            raise EmuError(f"buffer load form not modelled (idxen / offset): {i.text}")
        v, rs, so = i.ops[0], i.ops[1], i.ops[2]
        if rs.kind != "s" or rs.n != 4:
            raise EmuError(f"buffer descriptor must be 4 SGPRs: {i.text}")
        check_vmem_sgpr_hazard(w, i, [rs, so])
        if w.clock - w.salu_m0_write - 1 < 1 and i.in_asm:
            raise EmuError("LDS DMA issued right after an M0 write (needs 1 wait state)")
        w._check_pend_s(rs.idx, 4, "read of")
        d = [int(w.S[rs.idx + k]) for k in range(4)]
        base = d[0] | ((d[1] & 0xFFFF) << 32)
        stride = (d[1] >> 16) & 0x3FFF
        num_records = d[2]
        if stride != 0:
            raise EmuError(f"strided buffer descriptor not modelled ({stride}): {i.text}")
        if ((d[3] >> 15) & 0xF) == 0:
            raise EmuError(f"buffer descriptor with data format 0 reads zeros: {i.text}")
        m = w.exec_mask()
        soff = np.int64(w.sget(so))
        voff = (w.vget(v).astype(np.int64) if i.mods.get("offen")
                else np.zeros(64, np.int64))
        off = voff + soff
        if ((off + nb > num_records) | (off < 0))[m].any():
            raise EmuError(f"buffer load outside its descriptor's {num_records} bytes "
                           f"(offset up to {int(off[m].max())}): {i.text}")
        addrs = (np.int64(base) + off).astype(np.uint64)
        data = w.emu.mem.read(addrs[m], nb, i.text)
        m0 = w.S[124] & 0x3FFFF
        lds_off = (m0 + nb * np.arange(64))[m].astype(np.int64)
        wg = w.wg
        if (lds_off + nb > wg.lds_size).any() or (lds_off < 0).any():
            raise EmuError(f"LDS DMA target {int(lds_off.max())}+{nb} outside "
                           f"{wg.lds_size}-byte LDS (M0={m0:#x})")
        idx = (lds_off[:, None] // 4 + np.arange(nb // 4)[None, :]).reshape(-1)
        if (wg.dma_pending[idx] > 0).any():
            raise EmuError("LDS DMA into bytes with another DMA still in flight")
        lds_mark(w, np.unique(idx), "w", i.text + " (issue)")
        wg.dma_pending[idx] += 1
        w.emu.stats.lds_dma += 1
        push_vm(w, Pend(w, dma=(idx, data.reshape(-1, 4)), what=i.text))
    return run


HANDLERS["buffer_load_dword"] = _bload_lds(4)
HANDLERS["buffer_load_dwordx4"] = _bload_lds(16)


def _flat_split(w, addrs):
    lds = (addrs >= np.uint64(SHARED_BASE)) & (addrs < np.uint64(SHARED_BASE + (1 << 32)))
    return lds


@h("flat_load_dword")
def _(w, i):
    d, v = i.ops[0], i.ops[1]
    m = w.exec_mask()
    addrs = (w.vget64(v) + np.uint64(int(i.mods.get("offset", 0))))[m]
    is_lds = _flat_split(w, addrs)
    vals = np.zeros(len(addrs), U32)
    if is_lds.any():
        offs = (addrs[is_lds] - np.uint64(SHARED_BASE)).astype(np.int64)
        lds_check(w, offs, 4, "r", i.text)
        vals[is_lds] = w.wg.lds[offs[:, None] + np.arange(4)].copy().view("<u4").reshape(-1)
    if (~is_lds).any():
        vals[~is_lds] = w.emu.mem.read(addrs[~is_lds], 4, i.text).view("<u4").reshape(-1)
    row = w.vrow(d)

    def apply():
        w.V[row, m] = vals
    p = Pend(w, vrows=[row], apply=apply, queues=2, what=i.text)
    push_vm(w, p)
    push_lgkm(w, p)


@h("flat_store_dword")
def _(w, i):
    v, d = i.ops[0], i.ops[1]
    m = w.exec_mask()
    addrs = (w.vget64(v) + np.uint64(int(i.mods.get("offset", 0))))[m]
    vals = w.vget(d)[m].astype("<u4")
    is_lds = _flat_split(w, addrs)
    if is_lds.any():
        offs = (addrs[is_lds] - np.uint64(SHARED_BASE)).astype(np.int64)
        lds_check(w, offs, 4, "w", i.text)
        b = vals[is_lds].view(np.uint8).reshape(-1, 4)
        for k in range(len(offs)):
            w.wg.lds[offs[k]:offs[k] + 4] = b[k]
    if (~is_lds).any():
        w.emu.mem.write(addrs[~is_lds], vals[~is_lds].view(np.uint8).reshape(-1, 4), i.text)
    p = Pend(w, queues=2, what=i.text)
    push_vm(w, p)
    push_lgkm(w, p)


def _scr_addr(w, i, vop, sop):
    off = int(i.mods.get("offset", 0))
    a = np.full(64, off, np.int64)
    if vop is not None and vop.kind == "v":
        a += w.vget(vop).astype(np.int64)
    if sop is not None and sop.kind == "s":
        a += w.sget(sop)
    return a


def _sload_priv(nb):
    def run(w, i):
        d, v, s = i.ops
        m = w.exec_mask()
        a = _scr_addr(w, i, v, s)[m]
        P = w.priv.shape[1]
        if (a < 0).any() or (a + nb > P).any():
            raise EmuError(f"scratch access {int(a.max())}+{nb} outside {P}-byte private segment")
        lanes = np.nonzero(m)[0]
        data = w.priv[lanes[:, None], a[:, None] + np.arange(nb)[None, :]].copy()
        vals = data.view("<u4").reshape(-1, nb // 4)
        rows = [w.vrow(d, k) for k in range(nb // 4)]

        def apply():
            for k, r in enumerate(rows):
                w.V[r, m] = vals[:, k]
        push_vm(w, Pend(w, vrows=rows, apply=apply, what=i.text))
    return run


def _sstore_priv(nb):
    def run(w, i):
        v, d, s = i.ops
        m = w.exec_mask()
        a = _scr_addr(w, i, v, s)[m]
        P = w.priv.shape[1]
        if (a < 0).any() or (a + nb > P).any():
            raise EmuError(f"scratch access {int(a.max())}+{nb} outside {P}-byte private segment")
        lanes = np.nonzero(m)[0]
        vals = np.stack([w.vget(d, "b32", k)[m] for k in range(nb // 4)], 1).astype("<u4")
        w.priv[lanes[:, None], a[:, None] + np.arange(nb)[None, :]] = vals.view(np.uint8).reshape(-1, nb)
        push_vm(w, Pend(w, what=i.text))
    return run


HANDLERS["scratch_load_dword"] = _sload_priv(4)
HANDLERS["scratch_load_dwordx2"] = _sload_priv(8)
HANDLERS["scratch_load_dwordx3"] = _sload_priv(12)
HANDLERS["scratch_load_dwordx4"] = _sload_priv(16)
HANDLERS["scratch_store_dword"] = _sstore_priv(4)
HANDLERS["scratch_store_dwordx2"] = _sstore_priv(8)
HANDLERS["scratch_store_dwordx3"] = _sstore_priv(12)
HANDLERS["scratch_store_dwordx4"] = _sstore_priv(16)
