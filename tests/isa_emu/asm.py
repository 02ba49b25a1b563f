"""Parse the gfx950 assembly that hipcc -save-temps writes into kernels of
decoded instructions (operands, modifiers, branch targets, inline-asm marks)
plus each kernel's launch metadata."""
from __future__ import annotations

import re
import struct
from dataclasses import dataclass, field
from typing import Dict, List

import yaml

SPECIAL = {
    "vcc": (106, 2), "vcc_lo": (106, 1), "vcc_hi": (107, 1),
    "exec": (126, 2), "exec_lo": (126, 1), "exec_hi": (127, 1),
    "m0": (124, 1), "flat_scratch": (102, 2), "flat_scratch_lo": (102, 1),
    "flat_scratch_hi": (103, 1),
}
INLINE_F = {"0.5": 0.5, "-0.5": -0.5, "1.0": 1.0, "-1.0": -1.0, "2.0": 2.0, "-2.0": -2.0,
            "4.0": 4.0, "-4.0": -4.0, "0.15915494": 0.15915494309189535}


@dataclass
class Op:
    kind: str            # v a s imm fimm label off shared_base private_base
    idx: int = 0
    n: int = 1
    neg: bool = False
    abs: bool = False
    ival: int = 0        # integer literal
    fval: float = 0.0    # float inline constant
    text: str = ""

    def imm_bits(self, ty: str) -> int:
        """Bit pattern of an immediate for an operand of type ty."""
        if self.kind == "imm":
            v = self.ival
            if ty == "f64":
                # a 32-bit hex literal supplies the high half; small ints are
                # inline integers
                if -16 <= v <= 64:
                    return v & 0xFFFFFFFFFFFFFFFF
                return (v & 0xFFFFFFFF) << 32
            if ty in ("b64", "u64", "i64"):
                return v & 0xFFFFFFFFFFFFFFFF
            return v & 0xFFFFFFFF
        if self.kind == "fimm":
            if ty == "f64":
                return struct.unpack("<Q", struct.pack("<d", self.fval))[0]
            if ty == "f16":
                raise NotImplementedError
            return struct.unpack("<I", struct.pack("<f", self.fval))[0]
        raise ValueError(f"not an immediate: {self.text}")


@dataclass
class Inst:
    op: str
    ops: List[Op]
    mods: Dict[str, object]
    line: int
    text: str
    in_asm: bool = False
    target: int = -1     # branch target index
    handler: object = None


@dataclass
class Kernel:
    name: str
    insts: List[Inst]
    labels: Dict[str, int]
    meta: Dict[str, int]
    md: dict = field(default_factory=dict)

    @property
    def lds_bytes(self):
        return self.meta.get("group_segment_fixed_size", 0)

    @property
    def private_bytes(self):
        return self.meta.get("private_segment_fixed_size", 0)


_reg = re.compile(r"^([vsa])(\d+)$")
_regr = re.compile(r"^([vsa])\[(\d+):(\d+)\]$")


def parse_operand(tok: str) -> Op:
    t = tok.strip()
    neg = ab = False
    if t.startswith("-") and len(t) > 1 and (t[1] in "vsa|" or t[1:].startswith("abs(")):
        neg, t = True, t[1:]
    if t.startswith("|") and t.endswith("|"):
        ab, t = True, t[1:-1]
    m = _reg.match(t)
    if m:
        return Op(m.group(1), int(m.group(2)), 1, neg, ab, text=tok)
    m = _regr.match(t)
    if m:
        lo, hi = int(m.group(2)), int(m.group(3))
        return Op(m.group(1), lo, hi - lo + 1, neg, ab, text=tok)
    if t in SPECIAL:
        i, n = SPECIAL[t]
        return Op("s", i, n, neg, ab, text=tok)
    if t == "off":
        return Op("off", text=tok)
    if t == "src_shared_base":
        return Op("shared_base", n=2, text=tok)
    if t == "src_private_base":
        return Op("private_base", n=2, text=tok)
    if t in INLINE_F:
        return Op("fimm", fval=INLINE_F[t], text=tok)
    if re.match(r"^-?0x[0-9a-fA-F]+$", t):
        v = int(t, 16)
        return Op("imm", ival=v, text=tok)
    if re.match(r"^-?\d+$", t):
        return Op("imm", ival=int(t), text=tok)
    if t.startswith(".L") or t.startswith("_Z"):
        return Op("label", text=t)
    raise ValueError(f"cannot parse operand {tok!r}")


def _split_top(s: str) -> List[str]:
    out, depth, cur = [], 0, []
    for ch in s:
        if ch in "[(":
            depth += 1
        elif ch in "])":
            depth -= 1
        if ch == "," and depth == 0:
            out.append("".join(cur))
            cur = []
        else:
            cur.append(ch)
    if cur:
        out.append("".join(cur))
    return out


_MOD = re.compile(r"^(offset|offset0|offset1|bitop3|dst_sel|dst_unused|src0_sel|src1_sel|"
                  r"op_sel|op_sel_hi|cbsz|abid|blgp|neg_lo|neg_hi):(.+)$")
_FLAGS = {"sc0", "sc1", "nt", "glc", "slc", "dlc", "clamp", "lds", "gds", "offen", "idxen"}


def parse_inst(line: str, lineno: int) -> Inst:
    body = line.split(";", 1)[0].strip()
    parts = body.split(None, 1)
    op = parts[0]
    rest = parts[1] if len(parts) > 1 else ""
    mods: Dict[str, object] = {}
    if op == "s_waitcnt":
        for m in re.finditer(r"(vmcnt|lgkmcnt|expcnt)\((\d+)\)", rest):
            mods[m.group(1)] = int(m.group(2))
        if not mods and rest.strip():
            v = int(rest.strip(), 0)
            mods = {"vmcnt": (v & 0xF) | ((v >> 10) & 0x30), "expcnt": (v >> 4) & 7,
                    "lgkmcnt": (v >> 8) & 0xF}
        return Inst(op, [], mods, lineno, line.strip())
    toks = _split_top(rest) if rest else []
    ops: List[Op] = []
    for i, tk in enumerate(toks):
        tk = tk.strip()
        if i == len(toks) - 1:
            words = tk.split()
            # modifiers follow the last operand, separated by spaces
            first = words[0] if words else ""
            trail = words[1:]
            if _MOD.match(first) or first in _FLAGS:
                trail = words
                first = ""
            for w in trail:
                m = _MOD.match(w)
                if m:
                    k, v = m.group(1), m.group(2)
                    if v.startswith("["):
                        mods[k] = [int(x, 0) for x in v.strip("[]").split(",")]
                    else:
                        try:
                            mods[k] = int(v, 0)
                        except ValueError:
                            mods[k] = v
                elif w in _FLAGS:
                    mods[w] = True
                else:
                    raise ValueError(f"unknown modifier {w!r} in {line.strip()!r}")
            if first:
                ops.append(parse_operand(first))
        else:
            ops.append(parse_operand(tk))
    return Inst(op, ops, mods, lineno, line.strip())


def _parse_md(text: str) -> Dict[str, dict]:
    m = re.search(r"\.amdgpu_metadata\n(.*?)\n\s*\.end_amdgpu_metadata", text, re.S)
    if not m:
        return {}
    doc = yaml.safe_load(m.group(1))
    return {k[".name"]: k for k in doc.get("amdhsa.kernels", [])}


def load_kernels(path: str) -> Dict[str, Kernel]:
    text = open(path).read()
    lines = text.splitlines()
    md = _parse_md(text)
    kernels: Dict[str, Kernel] = {}
    i = 0
    while i < len(lines):
        ln = lines[i]
        m = re.match(r"^(_Z\S+|[A-Za-z_][\w.]*):\s*(;.*)?$", ln)
        if m and m.group(1) in md:
            name = m.group(1)
            insts: List[Inst] = []
            labels: Dict[str, int] = {}
            in_asm = False
            i += 1
            while i < len(lines) and not lines[i].startswith(".Lfunc_end"):
                raw = lines[i]
                s = raw.strip()
                i += 1
                if not s:
                    continue
                if s.startswith(";;#ASMSTART"):
                    in_asm = True
                    continue
                if s.startswith(";;#ASMEND"):
                    in_asm = False
                    continue
                if s.startswith(";") or s.startswith("."):
                    lm = re.match(r"^(\.L[\w.$]+):", s)
                    if lm:
                        labels[lm.group(1)] = len(insts)
                    continue
                inst = parse_inst(s, i)
                inst.in_asm = in_asm
                insts.append(inst)
            for inst in insts:
                for o in inst.ops:
                    if o.kind == "label":
                        inst.target = labels[o.text]
            mm = re.search(r"\.amdhsa_kernel " + re.escape(name) + r"\n(.*?)\.end_amdhsa_kernel",
                           text, re.S)
            meta = {k: int(v) for k, v in re.findall(r"\.amdhsa_(\w+)\s+(\d+)", mm.group(1))}
            kernels[name] = Kernel(name, insts, labels, meta, md[name])
        else:
            i += 1
    return kernels
