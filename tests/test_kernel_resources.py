"""Register spills of the built library's gfx950 kernels.

Every kernel is built to a register budget (two waves per SIMD for the
prefill, decode and backward kernels).  A kernel that overflows it keeps
registers in per-lane scratch memory, and a scratch access inside a loop costs
a memory round trip on every iteration.  The checks read the code object's
metadata (spill counts) and its disassembly (where the scratch accesses sit).
"""
import os
import re
import subprocess
import tempfile

import pytest

import mfma_hazards as H
from exact_attention_72_amd import api

# Kernels allowed to spill, with the most VGPRs they may keep in scratch: the
# varlen prefill with ALiBi at head_dim 128 (packed and unpacked GQA rows)
# keeps values the epilogue needs there, outside its key loop.
ALLOWED_SPILLS = {
    "_ZN12_GLOBAL__N_117fa_prefill_kernelILi128ELb1ELb0ELb0ELb0ELb1E7FaNoModEEv8FaParams": 16,
    "_ZN12_GLOBAL__N_117fa_prefill_kernelILi128ELb1ELb1ELb0ELb0ELb1E7FaNoModEEv8FaParams": 16,
}


def kernel_notes(so_path, arch="gfx950"):
    """{kernel symbol: {field: int}} from the AMDGPU metadata of every code object."""
    with tempfile.TemporaryDirectory() as tmp:
        text = "\n".join(
            subprocess.run([os.path.join(H.ROCM_LLVM, "llvm-readelf"), "--notes", co], check=True,
                           capture_output=True, text=True).stdout
            for co in H.code_objects(so_path, tmp, arch))
    out, cur = {}, None
    for line in text.splitlines():
        m = re.match(r"\s+\.name:\s+(\S+)", line)
        if m:
            cur = m.group(1)
            out[cur] = {}
            continue
        m = re.match(r"\s+\.(vgpr_count|agpr_count|vgpr_spill_count|sgpr_spill_count):\s+(\d+)", line)
        if m and cur is not None:
            out[cur][m.group(1)] = int(m.group(2))
    return out


def _successors(ins):
    """Instruction-level control-flow successors (fall-through and branch targets)."""
    index = {a: i for i, (a, _) in enumerate(ins)}
    succ = [[] for _ in ins]
    for i, (a, t) in enumerate(ins):
        op = t.split()[0]
        m = re.match(r"s_c?branch\S*\s+(-?\d+)", t)
        if m:
            off = int(m.group(1))
            if off > 32767:
                off -= 65536
            tgt = a + 4 + 4 * off
            if tgt in index:
                succ[i].append(index[tgt])
        if op not in ("s_branch", "s_endpgm", "s_setpc_b64") and i + 1 < len(ins):
            succ[i].append(i + 1)
    return succ


def scratch_in_loops(ins):
    """Scratch instructions of one kernel that lie on a cycle of its control flow."""
    succ = _successors(ins)
    found = []
    for i, (a, t) in enumerate(ins):
        if not t.startswith("scratch_"):
            continue
        stack, seen = list(succ[i]), set()
        while stack:
            j = stack.pop()
            if j == i:
                found.append((a, t))
                break
            if j in seen:
                continue
            seen.add(j)
            stack.extend(succ[j])
    return found


def test_loop_finder_sees_a_scratch_access_in_a_loop():
    base = 0x1000
    ins = [(base, "scratch_store_dword off, v1, off"), (base + 4, "v_add_f32_e32 v0, v0, v1"),
           (base + 8, "scratch_load_dword v2, off, off"), (base + 12, "s_cbranch_scc1 65533"),
           (base + 16, "scratch_load_dword v3, off, off")]
    # the branch at base + 12 jumps back 3 instructions to base + 4
    assert [a for a, _ in scratch_in_loops(ins)] == [base + 8]


needs_tools = pytest.mark.skipif(
    not (H.tools_available() and os.path.exists(os.path.join(H.ROCM_LLVM, "llvm-readelf"))),
    reason="ROCm llvm tools not found")


@needs_tools
def test_kernels_do_not_spill_beyond_the_allowed():
    if not os.path.exists(api.LIB_PATH):
        pytest.skip("library not built")
    notes = kernel_notes(api.LIB_PATH)
    assert any("fa_prefill_kernel" in k for k in notes) and any("fa_fp8_fwd_kernel" in k for k in notes), \
        "every code object's metadata is read"
    bad = [f"{k}: {v.get('vgpr_spill_count')} VGPRs spilled" for k, v in notes.items()
           if v.get("vgpr_spill_count", 0) > ALLOWED_SPILLS.get(k, 0)]
    assert not bad, "\n".join(bad)


@needs_tools
def test_no_scratch_access_inside_a_loop():
    if not os.path.exists(api.LIB_PATH):
        pytest.skip("library not built")
    funcs = H.parse(H.disassemble(api.LIB_PATH))
    bad = {k: hits for k, ins in funcs.items() if (hits := scratch_in_loops(ins))}
    assert not bad, "\n".join(f"{k[:80]}: {t}" for k, v in bad.items() for _, t in v[:3])
