"""Register hazards of inline-assembly memory instructions, checked in the
compiled gfx950 code of every kernel (CPU only: hipcc cross-compiles).

The compiler does not know what an `asm` statement does to memory: it takes
the output registers of an `asm` load as written when the statement ends and
the data registers of an `asm` store as free at that point.  The hardware
does neither: a load's registers are written when the data returns, and a
store may still read its data after the next instructions have issued.  Both
are safe only behind an `s_waitcnt vmcnt` that retires the instruction.
This scan walks each kernel's straight-line code, tracks the outstanding
vector-memory instructions issued from `asm` statements, and fails when any
instruction touches the registers of an outstanding `asm` load, or writes
the data registers of an outstanding `asm` store, before a `vmcnt` wait
retires it.  Both patterns have produced wrong results on the GPU (a
register copied before a read-back landed; partial sums stored from
registers the next instruction reused for an address).
"""
import os
import re
import shutil
import subprocess
import tempfile

import pytest

from tiled_dense_gemm_09_amd import build

KERNEL_FILES = ["gemm_async.hip", "gemm_skinny.hip", "attention.hip", "gemm_mx.hip"]

_REG = re.compile(r"\b([va])(?:\[(\d+):(\d+)\]|(\d+)\b)")


def _regs(text):
    out = set()
    for m in _REG.finditer(text):
        if m.group(2):
            out |= {(m.group(1), i) for i in range(int(m.group(2)), int(m.group(3)) + 1)}
        else:
            out.add((m.group(1), int(m.group(4))))
    return out


def scan(asm_text):
    """[(function, outstanding instruction, offending instruction)]"""
    found = []
    objects = set(re.findall(r"^\s*\.type\s+(_ZN2tg\w+),\s*@object", asm_text, re.M))
    for fn in re.findall(r"^(_ZN2tg\w+):", asm_text, re.M):
        if fn in objects:  # data symbols (e.g. a zero granule) carry no code
            continue
        a = asm_text.index(fn + ":")
        b = asm_text.index(".Lfunc_end", a)
        in_asm = False
        pending = []  # vector-memory instructions in issue order: (kind, registers, text)
        for raw in asm_text[a:b].splitlines():
            line = raw.strip()
            if line.startswith(";;#ASMSTART"):
                in_asm = True
                continue
            if line.startswith(";;#ASMEND"):
                in_asm = False
                continue
            if not line or line.startswith((";", ".")) or line.endswith(":"):
                continue
            op = line.split()[0]
            operands = line[len(op):].split(",")
            if op == "s_waitcnt":
                m = re.search(r"vmcnt\((\d+)\)", line)
                if m:
                    keep = int(m.group(1))
                    pending = pending[len(pending) - keep:] if 0 < keep < len(pending) else (
                        [] if keep == 0 else pending)
                continue
            touched = _regs(line)
            written = set()
            if operands and not op.startswith(("global_store", "buffer_store", "flat_store", "s_")):
                written = _regs(operands[0])
            for kind, regs, text in pending:
                if (kind == "load" and touched & regs) or (kind == "store" and written & regs):
                    found.append((fn, text, line))
            if op.startswith(("global_", "buffer_", "flat_", "scratch_")):
                if in_asm and "load" in op and "lds" not in op:
                    pending.append(("load", _regs(operands[0]), line))
                elif in_asm and "store" in op and len(operands) > 1:
                    pending.append(("store", _regs(operands[1]), line))
                else:
                    pending.append(("other", set(), line))
    return found


# The store sequence of an earlier split-K build (one `asm` statement per
# store): the second instruction after the first store overwrites its data.
BAD_STORES = """
_ZN2tg4testEv:
\t;;#ASMSTART
\tglobal_store_dwordx4 v[68:69], v[18:21], off sc1
\t;;#ASMEND
\ts_mov_b64 s[0:1], 0x400
\tv_lshl_add_u64 v[18:19], v[68:69], 0, s[0:1]
\t;;#ASMSTART
\tglobal_store_dwordx4 v[18:19], v[22:25], off sc1
\t;;#ASMEND
\ts_waitcnt vmcnt(0)
.Lfunc_end0:
"""

# A read-back whose register is copied before its wait.
BAD_LOADS = """
_ZN2tg4testEv:
\t;;#ASMSTART
\tglobal_load_dwordx4 v[4:7], v[0:1], off sc1
\t;;#ASMEND
\tv_mov_b32_e32 v20, v5
\t;;#ASMSTART
\ts_waitcnt vmcnt(0)
\t;;#ASMEND
.Lfunc_end0:
"""

# The same instructions with the waits where they belong.
GOOD = """
_ZN2tg4testEv:
\t;;#ASMSTART
\tglobal_store_dwordx4 v[68:69], v[18:21], off sc1
\tglobal_store_dwordx4 v[68:69], v[22:25], off offset:1024 sc1
\ts_waitcnt vmcnt(0)
\t;;#ASMEND
\tv_lshl_add_u64 v[18:19], v[68:69], 0, s[0:1]
\t;;#ASMSTART
\tglobal_load_dwordx4 v[4:7], v[0:1], off sc1
\tglobal_load_dwordx4 v[8:11], v[0:1], off offset:1024 sc1
\t;;#ASMEND
\t;;#ASMSTART
\ts_waitcnt vmcnt(1)
\t;;#ASMEND
\tv_mov_b32_e32 v20, v5
\t;;#ASMSTART
\ts_waitcnt vmcnt(0)
\t;;#ASMEND
\tv_mov_b32_e32 v21, v9
.Lfunc_end0:
"""


def test_scan_finds_both_hazard_patterns():
    assert len(scan(BAD_STORES)) == 1
    assert len(scan(BAD_LOADS)) == 1
    assert scan(GOOD) == []


@pytest.fixture(scope="module")
def device_asm():
    hipcc = build.hipcc()
    if not os.path.exists(hipcc) and shutil.which(hipcc) is None:
        pytest.skip("hipcc not available")
    tmp = tempfile.mkdtemp(prefix="tg_asm_")
    procs = {}
    for f in KERNEL_FILES:
        out = os.path.join(tmp, f + ".s")
        cmd = [hipcc] + build.FLAGS + ["--cuda-device-only", "-S",
                                       os.path.join(build.CSRC, f), "-o", out]
        procs[f] = (subprocess.Popen(cmd, stdout=subprocess.DEVNULL, stderr=subprocess.PIPE), out)
    texts = {}
    for f, (p, out) in procs.items():
        _, err = p.communicate(timeout=600)
        assert p.returncode == 0, err.decode()[-2000:]
        texts[f] = open(out).read()
    shutil.rmtree(tmp, ignore_errors=True)
    return texts


@pytest.mark.parametrize("src", KERNEL_FILES)
def test_no_asm_register_hazards(device_asm, src):
    text = device_asm[src]
    assert "_ZN2tg" in text
    found = scan(text)
    assert not found, "\n".join("%s: %s -> %s" % h for h in found[:10])
