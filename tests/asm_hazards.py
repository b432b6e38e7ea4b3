"""Wait-state checks on the gfx950 code of the built library, for the MFMAs written as inline assembly.

The compiler inserts the wait states that the matrix core needs around the MFMAs it emits itself, but
its hazard checks do not look inside an asm statement. The kernels that keep their dK/dV sums in the
accumulator registers (AGPRs) issue those MFMAs as inline assembly, and the register allocator may put
its own copies (v_accvgpr_write, v_accvgpr_mov, v_accvgpr_read) next to them. Two rules of the CDNA
instruction set are checked on every MFMA whose destination is an AGPR tuple (the compiler's own
MFMAs in these libraries write VGPR tuples):

  - before: no VALU instruction writes a register that the MFMA reads (A, B or the accumulator)
    fewer than 2 wait states earlier (the count the compiler itself keeps for its MFMAs on gfx950);
  - after: no instruction other than an MFMA accumulating into the very same tuple reads or writes
    the MFMA's destination fewer than 12 wait states later (an 8-pass 32x32 MFMA; again the count
    the compiler keeps after its own MFMAs).

A wait state is one instruction, or N + 1 for ``s_nop N``. Paths are followed through fall-through and
branches, so a copy placed at a loop exit or entry is seen. The code objects are taken from the
library's offload section and disassembled with the ROCm llvm-objdump.
"""
import os
import re
import subprocess
import tempfile

LLVM = "/opt/rocm/llvm/bin"
BEFORE_WS = 2
AFTER_WS = 12
_MAGIC = b"__CLANG_OFFLOAD_BUNDLE__"
_TARGET = "hipv4-amdgcn-amd-amdhsa--gfx950"


def code_objects(lib_path):
    """The gfx950 code objects of a shared library built by hipcc (one per compilation unit)."""
    with tempfile.TemporaryDirectory() as tmp:
        fat = os.path.join(tmp, "fat.bin")
        subprocess.run([f"{LLVM}/llvm-objcopy", f"--dump-section=.hip_fatbin={fat}", lib_path, os.devnull],
                       check=True, capture_output=True)
        data = open(fat, "rb").read()
        starts = [m.start() for m in re.finditer(re.escape(_MAGIC), data)]
        objs = []
        for n, s in enumerate(starts):
            e = starts[n + 1] if n + 1 < len(starts) else len(data)
            bundle, obj = os.path.join(tmp, f"b{n}"), os.path.join(tmp, f"co{n}.o")
            with open(bundle, "wb") as f:
                f.write(data[s:e])
            subprocess.run([f"{LLVM}/clang-offload-bundler", "--unbundle", "--type=o", f"--targets={_TARGET}",
                            f"--input={bundle}", f"--output={obj}"], check=True, capture_output=True)
            objs.append(open(obj, "rb").read())
        return objs


def disassemble(obj_bytes):
    with tempfile.NamedTemporaryFile(suffix=".o") as f:
        f.write(obj_bytes)
        f.flush()
        return subprocess.run([f"{LLVM}/llvm-objdump", "-d", "--mcpu=gfx950", f.name], check=True,
                              capture_output=True, text=True).stdout


_FUNC = re.compile(r"^([0-9a-f]+) <(.+)>:$")
_INST = re.compile(r"^\s+(\S+)\s*(.*?)\s*//\s*([0-9A-F]+):")
_TGT = re.compile(r"<(.+)\+0x([0-9a-f]+)>")
_REG = re.compile(r"\b([va])(?:\[(\d+):(\d+)\]|(\d+)\b)")


def parse(text):
    """{function: [(address, mnemonic, operand text, branch target address or None)]} from objdump text."""
    funcs, cur, base = {}, None, 0
    for line in text.splitlines():
        m = _FUNC.match(line)
        if m:
            base, cur = int(m.group(1), 16), m.group(2)
            funcs[cur] = []
            continue
        m = _INST.match(line)
        if cur is None or not m:
            continue
        ops = m.group(2)
        tgt = None
        if m.group(1).startswith(("s_branch", "s_cbranch")):
            t = _TGT.search(line)
            if t and t.group(1) == cur:
                tgt = base + int(t.group(2), 16)
        funcs[cur].append((int(m.group(3), 16), m.group(1), ops, tgt))
    return funcs


def regs(text):
    """Registers named in an operand text, as a set of ('v' | 'a', index)."""
    out = set()
    for m in _REG.finditer(text):
        lo, hi = (int(m.group(2)), int(m.group(3))) if m.group(2) else (int(m.group(4)), int(m.group(4)))
        out.update((m.group(1), i) for i in range(lo, hi + 1))
    return out


def operands(ops):
    return [o.strip() for o in ops.split(",")] if ops else []


def is_mfma(mn):
    return mn.startswith("v_mfma") or mn.startswith("v_smfmac")


def valu_writes(mn, ops):
    """Vector registers a VALU instruction writes (its first operand); none for other instructions."""
    if not mn.startswith("v_") or is_mfma(mn) or mn.startswith(("v_cmp", "v_readlane", "v_readfirstlane")):
        return set()
    ops = operands(ops)
    return regs(ops[0]) if ops else set()


def wait_states(mn, ops):
    if mn == "s_nop":
        return int(ops, 0) + 1
    return 1


def check_function(insts):
    """Hazards of the AGPR-destination MFMAs of one function, as readable strings."""
    index = {addr: i for i, (addr, _, _, _) in enumerate(insts)}
    sources = {}  # branch target index -> indices of the branches to it
    for i, (_, mn, _, tgt) in enumerate(insts):
        if tgt is not None and tgt in index:
            sources.setdefault(index[tgt], []).append(i)
    problems = []

    def back(i, budget, reads, origin, seen):
        # instructions before index i (exclusive), within `budget` wait states, on every path into i
        preds = list(sources.get(i, []))
        if i > 0 and insts[i - 1][1] != "s_branch" and not insts[i - 1][1].startswith("s_endpgm"):
            preds.append(i - 1)
        for j in preds:
            if (j, budget) in seen:
                continue
            seen.add((j, budget))
            _, mn, ops, _ = insts[j]
            hit = valu_writes(mn, ops) & reads
            if hit:
                problems.append(f"{insts[origin][1]} {insts[origin][2]} at {insts[origin][0]:#x}: "
                                f"{mn} {ops} at {insts[j][0]:#x} writes {sorted(hit)[:4]} "
                                f"fewer than {BEFORE_WS} wait states before")
            ws = budget - wait_states(mn, ops)
            if ws > 0:
                back(j, ws, reads, origin, seen)

    def fwd(i, budget, dest, tuple_text, origin, seen):
        # instructions after index i, within `budget` wait states, on every path out of i
        _, mn_i, _, tgt = insts[i]
        succ = []
        if mn_i != "s_branch" and not mn_i.startswith("s_endpgm") and i + 1 < len(insts):
            succ.append(i + 1)
        if tgt is not None and tgt in index:
            succ.append(index[tgt])
        for j in succ:
            if (j, budget) in seen:
                continue
            seen.add((j, budget))
            _, mn, ops, _ = insts[j]
            touched = regs(ops) & dest
            if touched:
                o = operands(ops)
                chain = is_mfma(mn) and len(o) >= 4 and o[0] == tuple_text and o[3] == tuple_text \
                    and not (regs(o[1]) | regs(o[2])) & dest
                if not chain:
                    problems.append(f"{insts[origin][1]} {insts[origin][2]} at {insts[origin][0]:#x}: "
                                    f"{mn} {ops} at {insts[j][0]:#x} touches {sorted(touched)[:4]} "
                                    f"fewer than {AFTER_WS} wait states after")
            ws = budget - wait_states(mn, ops)
            if ws > 0:
                fwd(j, ws, dest, tuple_text, origin, seen)

    for i, (_, mn, ops, _) in enumerate(insts):
        if not is_mfma(mn):
            continue
        o = operands(ops)
        if not o or not o[0].startswith("a"):
            continue
        reads = set().union(*(regs(x) for x in o[1:4]))
        back(i, BEFORE_WS, reads, i, set())
        fwd(i, AFTER_WS, regs(o[0]), o[0], i, set())
    return problems


def check_library(lib_path):
    """({function: [problems]}, number of AGPR-destination MFMAs seen) over every code object."""
    found, count = {}, 0
    for obj in code_objects(lib_path):
        for name, insts in parse(disassemble(obj)).items():
            count += sum(1 for _, mn, ops, _ in insts if is_mfma(mn) and ops.startswith("a"))
            p = check_function(insts)
            if p:
                found[name] = p
    return found, count
