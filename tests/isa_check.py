"""Static checks on the gfx950 code object inside the built libtim.so.

The MFMA kernels issue matrix instructions from inline asm (tied
accumulators, hand-placed waits).  The compiler's hazard recognizer does not
look into asm, so the wait states that an MFMA's result needs before any other
instruction touches its destination registers are provided by the kernels
themselves, and the register allocator could in principle place a copy of an
accumulator where the kernel's author did not expect one.  This module reads
the disassembly of the library as built (AMD assembly of code built here:
``llvm-objcopy`` pulls the offload bundle out of the ``.hip_fatbin`` section,
``clang-offload-bundler`` unbundles the gfx950 code object and
``llvm-objdump`` disassembles it) and walks every control-flow path from every
MFMA:

* no instruction other than an MFMA whose accumulator operand is exactly the
  same register range (the hardware's own chaining case) may read or write a
  register of the MFMA's destination within the number of wait states the
  compiler's own hazard recognizer inserts between that MFMA shape and a
  VALU read of its result (measured by compiling a three-kernel probe with
  hipcc: 8 for 16x16x32 bf16, 12 for 32x32x16 bf16, 18 for 32x32x2 f32 with
  this toolchain; 19, more than any of them, for a shape not probed);
* no MFMA may read a register that a non-MFMA vector instruction wrote
  within ``VALU_TO_MFMA_WAIT`` wait states.

Wait states are counted as the hazard recognizer counts them: one per
instruction, ``n + 1`` for ``s_nop n``.

One idiom is interpreted rather than walked blindly: a conditional branch
over a block of ``s_nop`` (the wait after a K loop's last MFMA, skipped while
the loop continues).  A path that takes such a skip is followed only around
the loop (it takes the next backward branch), because the kernels skip the
wait exactly when another iteration follows.
"""
from __future__ import annotations

import functools
import os
import re
import shutil
import subprocess
import tempfile

MFMA_WAIT = 19
VALU_TO_MFMA_WAIT = 2
LLVM_BIN = "/opt/rocm/llvm/bin"

# one kernel per MFMA shape the library uses: the result is read by a VALU
# instruction right away, so the compiler must put the full wait between
_PROBE = r"""
#include <hip/hip_runtime.h>
typedef __attribute__((__vector_size__(8 * sizeof(__bf16)))) __bf16 bf16x8;
typedef __attribute__((__vector_size__(4 * sizeof(float)))) float f32x4;
typedef __attribute__((__vector_size__(16 * sizeof(float)))) float f32x16;
extern "C" __global__ void p_v_mfma_f32_16x16x32_bf16(const bf16x8* a, float* o) {
    f32x4 c = {0, 0, 0, 0};
    c = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a[threadIdx.x], a[threadIdx.x + 64], c, 0, 0, 0);
    o[threadIdx.x] = c[0] * 3.0f;
}
extern "C" __global__ void p_v_mfma_f32_32x32x16_bf16(const bf16x8* a, float* o) {
    f32x16 c = {};
    c = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[threadIdx.x], a[threadIdx.x + 64], c, 0, 0, 0);
    o[threadIdx.x] = c[0] * 3.0f;
}
extern "C" __global__ void p_v_mfma_f32_32x32x2_f32(const float* a, float* o) {
    f32x16 c = {};
    c = __builtin_amdgcn_mfma_f32_32x32x2f32(a[threadIdx.x], a[threadIdx.x + 64], c, 0, 0, 0);
    o[threadIdx.x] = c[0] * 3.0f;
}
"""


@functools.lru_cache(maxsize=1)
def required_waits():
    """{mfma opcode: wait states} as the compiler's hazard recognizer places
    them before a VALU read of the result (the s_nop right after the MFMA in
    each probe kernel)."""
    tmp = tempfile.mkdtemp(prefix="tim_hz_")
    src, asm = os.path.join(tmp, "probe.hip"), os.path.join(tmp, "probe.s")
    with open(src, "w") as f:
        f.write(_PROBE)
    subprocess.run(["hipcc", "--offload-arch=gfx950", "-O3", "-S", "--cuda-device-only", src,
                    "-o", asm], check=True, capture_output=True)
    out, cur, waits = {}, None, None
    for line in open(asm):
        m = re.match(r"^p_(v_mfma_\w+):", line)
        if m:
            cur, waits = m.group(1), None
            continue
        if cur is None:
            continue
        t = line.split()
        if not t:
            continue
        if t[0] == cur:
            waits = 0
        elif waits is not None and t[0] == "s_nop":
            waits += int(t[1], 0) + 1
        elif waits is not None:
            out[cur], cur = waits, None
    return out


def mfma_wait(op):
    return required_waits().get(op, MFMA_WAIT)


_INSN = re.compile(r"^\s+([a-z_0-9]+)(?:\s+(.*?))?\s*//\s*([0-9A-Fa-f]+):")
_FUNC = re.compile(r"^([0-9a-f]+) <(.+)>:$")
_TARGET = re.compile(r"<(.+)\+0x([0-9a-f]+)>\s*$")
_REG = re.compile(r"\b([va])(?:\[(\d+):(\d+)\]|(\d+)(?!\d))")


def tool(name):
    path = os.path.join(LLVM_BIN, name)
    return path if os.path.exists(path) else shutil.which(name)


def tools_available():
    return all(tool(t) for t in ("llvm-objcopy", "clang-offload-bundler", "llvm-objdump",
                                 "llvm-readelf"))


_BUNDLE_MAGIC = b"__CLANG_OFFLOAD_BUNDLE__"


@functools.lru_cache(maxsize=4)
def code_objects(lib_path):
    """Paths of the gfx950 code objects unbundled from ``lib_path`` (a shared
    library: one offload bundle per translation unit, concatenated in its
    ``.hip_fatbin`` section; or a device-only object, one bundle)."""
    tmp = tempfile.mkdtemp(prefix="tim_isa_")
    with open(lib_path, "rb") as f:
        data = f.read(len(_BUNDLE_MAGIC))
    if data == _BUNDLE_MAGIC:            # a device-only object: one bundle
        fat = lib_path
    else:
        fat = os.path.join(tmp, "fat.bin")
        subprocess.run([tool("llvm-objcopy"), "-O", "binary", "--only-section=.hip_fatbin",
                        lib_path, fat], check=True)
    data = open(fat, "rb").read()
    starts = []
    k = data.find(_BUNDLE_MAGIC)
    while k >= 0:
        starts.append(k)
        k = data.find(_BUNDLE_MAGIC, k + 1)
    out = []
    for n, (a, b) in enumerate(zip(starts, starts[1:] + [len(data)])):
        part = os.path.join(tmp, f"bundle{n}.bin")
        with open(part, "wb") as f:
            f.write(data[a:b])
        co = os.path.join(tmp, f"gfx950_{n}.co")
        subprocess.run([tool("clang-offload-bundler"), "--unbundle", "--type=o",
                        f"--input={part}", "--targets=hipv4-amdgcn-amd-amdhsa--gfx950",
                        f"--output={co}"], check=True)
        if os.path.getsize(co) > 0:
            out.append(co)
    return tuple(out)


def regs(text):
    """Set of (file, index) of every v/a register named in an operand string."""
    out = set()
    for f, lo, hi, one in _REG.findall(text or ""):
        if one:
            out.add((f, int(one)))
        else:
            out.update((f, i) for i in range(int(lo), int(hi) + 1))
    return out


class Insn:
    __slots__ = ("addr", "op", "args", "target", "regs", "dst", "srcc")

    def __init__(self, addr, op, args, target):
        self.addr, self.op, self.args, self.target = addr, op, args or "", target
        self.regs = regs(self.args)
        parts = [p.strip() for p in self.args.split(",")] if self.args else []
        self.dst = regs(parts[0]) if parts else set()
        self.srcc = regs(parts[3]) if self.is_mfma and len(parts) > 3 else set()

    @property
    def is_mfma(self):
        return self.op.startswith("v_mfma") or self.op.startswith("v_smfmac")

    @property
    def is_vector(self):
        return self.op.startswith(("v_", "buffer_", "global_", "flat_", "ds_", "scratch_"))

    def wait_states(self):
        if self.op == "s_nop":
            return int(self.args.strip(), 0) + 1
        return 1


@functools.lru_cache(maxsize=4)
def kernels(lib_path):
    """{kernel symbol: [Insn, ...]} from the disassembly."""
    dis = "\n".join(subprocess.run([tool("llvm-objdump"), "-d", co], check=True,
                                   capture_output=True, text=True).stdout
                    for co in code_objects(lib_path))
    funcs, cur, start = {}, None, 0
    for line in dis.splitlines():
        m = _FUNC.match(line)
        if m:
            start, cur = int(m.group(1), 16), m.group(2)
            funcs[cur] = []
            continue
        if cur is None:
            continue
        m = _INSN.match(line)
        if not m:
            continue
        op, args, addr = m.group(1), m.group(2), int(m.group(3), 16)
        target = None
        if op.startswith("s_branch") or op.startswith("s_cbranch"):
            t = _TARGET.search(line)
            if t and t.group(1) == cur:
                target = start + int(t.group(2), 16)
            args = None
        funcs[cur].append(Insn(addr, op, args, target))
    return funcs


def successors(code, i, index_of):
    ins = code[i]
    if ins.op in ("s_endpgm", "s_setpc_b64", "s_trap"):
        return []
    if ins.op == "s_branch":
        return [index_of[ins.target]]
    if ins.op.startswith("s_cbranch"):
        nxt = [i + 1] if i + 1 < len(code) else []
        return nxt + ([index_of[ins.target]] if ins.target in index_of else [])
    return [i + 1] if i + 1 < len(code) else []


def _skips_wait(code, i, index_of):
    """A forward conditional branch whose fall-through is a block of s_nop
    ending at its target: the skippable wait after a loop's last MFMA."""
    ins = code[i]
    if not ins.op.startswith("s_cbranch") or ins.target not in index_of:
        return False
    j = index_of[ins.target]
    return j > i + 1 and all(code[k].op == "s_nop" for k in range(i + 1, j))


def check_kernel(code):
    """List of human-readable violations in one kernel's instruction list."""
    index_of = {ins.addr: k for k, ins in enumerate(code)}
    bad = []
    for i, ins in enumerate(code):
        if ins.is_mfma and ins.dst:
            dst = ins.dst
            need = mfma_wait(ins.op)
            # (index, wait states so far, skipped-wait flag)
            stack = [(j, 0, False) for j in successors(code, i, index_of)]
            seen = set()
            while stack:
                j, dist, skipped = stack.pop()
                if dist >= need or (j, dist, skipped) in seen:
                    continue
                seen.add((j, dist, skipped))
                nxt = code[j]
                if nxt.is_mfma and nxt.dst == dst and nxt.srcc == dst and \
                        not (nxt.regs - nxt.srcc - nxt.dst) & dst:
                    continue        # the chained MFMA: its own walk covers what follows
                if nxt.regs & dst:
                    bad.append(f"{nxt.op} {nxt.args} at {nxt.addr:#x}: {dist} wait states "
                               f"after {ins.op} {ins.args} at {ins.addr:#x}")
                    continue
                d2 = dist + nxt.wait_states()
                if _skips_wait(code, j, index_of):
                    stack.append((index_of[nxt.target], d2, True))
                    stack.append((j + 1, d2, skipped))
                    continue
                succ = successors(code, j, index_of)
                if skipped and nxt.op.startswith("s_cbranch") and nxt.target is not None \
                        and nxt.target <= nxt.addr:
                    succ = [index_of[nxt.target]]          # a skipped wait: the loop continues
                for s in succ:
                    stack.append((s, d2, skipped))
        elif ins.is_vector and not ins.is_mfma and ins.dst and ins.op.startswith("v_"):
            written = ins.dst
            stack = [(j, 0) for j in successors(code, i, index_of)]
            seen = set()
            while stack:
                j, dist = stack.pop()
                if dist >= VALU_TO_MFMA_WAIT or (j, dist) in seen:
                    continue
                seen.add((j, dist))
                nxt = code[j]
                if nxt.is_mfma and (nxt.regs - nxt.dst) & written:
                    bad.append(f"{nxt.op} {nxt.args} at {nxt.addr:#x}: {dist} wait states "
                               f"after {ins.op} {ins.args} at {ins.addr:#x}")
                    continue
                for s in successors(code, j, index_of):
                    stack.append((s, dist + nxt.wait_states()))
    return bad


def check_lds_reads(code):
    """Violations of one rule in one kernel: no instruction reads a register
    that an LDS read (ds_read*) writes before an s_waitcnt that counts LDS
    operations has followed that read.  The MFMA kernels issue their LDS
    reads from asm and wait for them with counted waits of their own; a
    copy of a read's destination that the compiler places in between (for
    instance to join the two halves of a transposed fragment) would read
    registers whose data has not arrived."""
    index_of = {ins.addr: k for k, ins in enumerate(code)}
    bad = []
    for i, ins in enumerate(code):
        if not ins.op.startswith("ds_read") or not ins.dst:
            continue
        dst = ins.dst
        stack = list(successors(code, i, index_of))
        seen = set()
        while stack:
            j = stack.pop()
            if j in seen:
                continue
            seen.add(j)
            nxt = code[j]
            if nxt.op == "s_waitcnt" and "lgkmcnt" in nxt.args:
                continue
            srcs = nxt.regs - nxt.dst if not nxt.op.startswith(("ds_", "buffer_", "global_")) \
                else nxt.regs - (nxt.dst if nxt.op.startswith("ds_read") else set())
            if srcs & dst:
                bad.append(f"{nxt.op} {nxt.args} at {nxt.addr:#x} reads the destination of "
                           f"{ins.op} {ins.args} at {ins.addr:#x} before any LDS wait")
                continue
            if nxt.dst and dst <= nxt.dst and not nxt.op.startswith("ds_read"):
                continue        # overwritten: the pending value is no longer read
            stack.extend(successors(code, j, index_of))
    return bad


@functools.lru_cache(maxsize=4)
def private_segment_sizes(lib_path):
    """{kernel symbol: private (scratch) bytes per work-item} from the code
    object's metadata note."""
    notes = "\n".join(subprocess.run([tool("llvm-readelf"), "--notes", co], check=True,
                                     capture_output=True, text=True).stdout
                      for co in code_objects(lib_path))
    sizes, name, pss = {}, None, None
    for line in notes.splitlines():
        s = line.strip().lstrip("- ").strip()
        if s.startswith(".name:"):
            name = s.split(":", 1)[1].strip()
        elif s.startswith(".private_segment_fixed_size:"):
            pss = int(s.split(":", 1)[1])
        elif s.startswith(".symbol:"):
            sym = s.split(":", 1)[1].strip()
            if sym.endswith(".kd"):
                sym = sym[:-3]
            if pss is not None:
                sizes[sym] = pss
            name, pss = None, None
    return sizes
