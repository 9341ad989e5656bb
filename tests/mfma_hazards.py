"""Static check of the built library's gfx950 code for matrix-product results
that are touched too soon.

Some kernels issue their matrix products (v_mfma) from inline assembly.  The
compiler then does not know that the instruction is a matrix product: it may
read, copy or overwrite the accumulator registers right after it (for example
when it moves accumulators between registers at a loop's exit), before the
product has written them.  The hardware does not interlock these accesses.
The compiler's own products are covered by its hazard pass, which never leaves
fewer than 12 wait states between a 32x32x16 product and the first access of
its result; this check asks the same of every product.

The check disassembles the library (llvm-objdump on the gfx950 code object),
builds each kernel's control-flow edges (fall-through and branch targets), and
walks backwards from every non-product instruction that reads or writes a
register: a product writing that register fewer than MIN_WAIT wait states
earlier on some path is reported.  An instruction counts one wait state and
s_nop N counts N + 1, a lower bound on the cycles between them.  Products that
feed other products are left to the hardware, which orders dependent products.
"""
import os
import re
import shutil
import subprocess
import tempfile

MIN_WAIT = 12
ROCM_LLVM = "/opt/rocm/llvm/bin"


def tools_available():
    return all(os.path.exists(os.path.join(ROCM_LLVM, t)) for t in ("llvm-objdump", "clang-offload-bundler")) and \
        shutil.which("objcopy") is not None


def code_objects(so_path, tmp, arch="gfx950"):
    """Paths of the library's gfx950 code objects, one per compiled source: the
    .hip_fatbin section holds one offload bundle per translation unit, each
    starting with the bundle magic."""
    fat = os.path.join(tmp, "fatbin")
    subprocess.run(["objcopy", "-O", "binary", "--only-section=.hip_fatbin", so_path, fat], check=True)
    data = open(fat, "rb").read()
    magic = b"__CLANG_OFFLOAD_BUNDLE__"
    starts = []
    i = data.find(magic)
    while i >= 0:
        starts.append(i)
        i = data.find(magic, i + 1)
    out = []
    for n, (a, b) in enumerate(zip(starts, starts[1:] + [len(data)])):
        part = os.path.join(tmp, f"bundle{n}")
        with open(part, "wb") as f:
            f.write(data[a:b])
        co = os.path.join(tmp, f"code{n}.o")
        subprocess.run([os.path.join(ROCM_LLVM, "clang-offload-bundler"), "--unbundle", "--type=o",
                        f"--input={part}", f"--targets=hipv4-amdgcn-amd-amdhsa--{arch}", f"--output={co}"],
                       check=True)
        out.append(co)
    return out


def disassemble(so_path, arch="gfx950"):
    """Disassembly text of all of the library's device code objects."""
    with tempfile.TemporaryDirectory() as tmp:
        texts = []
        for co in code_objects(so_path, tmp, arch):
            out = subprocess.run([os.path.join(ROCM_LLVM, "llvm-objdump"), "-d", "--no-show-raw-insn", co],
                                 check=True, capture_output=True, text=True)
            texts.append(out.stdout)
    return "\n".join(texts)


def parse(text):
    """{kernel name: [(address, instruction text)]} from llvm-objdump output."""
    funcs, cur = {}, None
    for line in text.splitlines():
        m = re.match(r"^([0-9a-f]+) <(.*)>:", line)
        if m:
            cur = m.group(2)
            funcs[cur] = []
            continue
        m = re.match(r"^\s+(\S.*?)\s*//\s*([0-9A-Fa-f]+):", line)
        if m and cur is not None:
            funcs[cur].append((int(m.group(2), 16), m.group(1).strip()))
    return funcs


def _regs(tok):
    out = set()
    for m in re.finditer(r"\b([av])\[(\d+):(\d+)\]", tok):
        out |= {(m.group(1), r) for r in range(int(m.group(2)), int(m.group(3)) + 1)}
    for m in re.finditer(r"(?<![\w\[])([av])(\d+)\b", tok):
        out.add((m.group(1), int(m.group(2))))
    return out


def _operands(ins):
    parts = ins.split(None, 1)
    return [o.strip() for o in parts[1].split(",")] if len(parts) > 1 else []


def _wait(ins):
    m = re.match(r"s_nop (\d+)", ins)
    return int(m.group(1)) + 1 if m else 1


def _predecessors(ins):
    index = {a: i for i, (a, _) in enumerate(ins)}
    preds = {i: [] for i in range(len(ins))}
    for i, (a, t) in enumerate(ins):
        op = t.split()[0]
        m = re.match(r"s_c?branch\S*\s+(-?\d+)", t)
        if m:
            off = int(m.group(1))
            if off > 32767:
                off -= 65536
            tgt = a + 4 + 4 * off
            if tgt in index:
                preds[index[tgt]].append(i)
        if op not in ("s_branch", "s_endpgm", "s_setpc_b64") and i + 1 < len(ins):
            preds[i + 1].append(i)
    return preds


def close_accesses(ins, min_wait=MIN_WAIT):
    """[(access, product, wait states)] for one kernel's instruction list."""
    preds = _predecessors(ins)
    found = []
    for i, (_, t) in enumerate(ins):
        op = t.split()[0]
        if op.startswith("v_mfma") or op.startswith("s_"):
            continue
        ops = _operands(t)
        touched = set()
        for o in ops:
            touched |= _regs(o)
        if not touched:
            continue
        stack, seen = [(p, 0) for p in preds[i]], set()
        while stack:
            j, w = stack.pop()
            if (j, w) in seen or w >= min_wait:
                continue
            seen.add((j, w))
            tj = ins[j][1]
            if tj.startswith("v_mfma"):
                dst = _regs(_operands(tj)[0])
                if dst & touched:
                    found.append((t, tj, w))
                    continue
            for p in preds[j]:
                stack.append((p, w + _wait(tj)))
    return found


def scan_library(so_path, min_wait=MIN_WAIT):
    """{kernel: [(access, product, wait states)]} for kernels with findings."""
    funcs = parse(disassemble(so_path))
    return {name: hits for name, ins in funcs.items() if (hits := close_accesses(ins, min_wait))}
