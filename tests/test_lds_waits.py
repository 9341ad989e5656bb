"""The built library touches no LDS result before a wait covers it (see
lds_waits.py), and the checker itself finds planted cases."""
import os

import pytest

import lds_waits as L
import mfma_hazards as H
from exact_attention_72_amd import api


def uses(*lines, base=0x1000):
    out = [f"{base:016x} <k>:"]
    for i, t in enumerate(lines):
        out.append(f"\t{t} // {base + 4 * i:012X}: 0")
    return L.early_lds_uses(H.parse("\n".join(out))["k"])


def test_checker_flags_a_copy_before_the_wait():
    assert uses("ds_read_b128 v[4:7], v1", "v_mov_b32_e32 v20, v5", "s_waitcnt lgkmcnt(0)") == \
        ["v_mov_b32_e32 v20, v5"]


def test_checker_accepts_a_use_after_the_wait():
    assert uses("ds_read_b128 v[4:7], v1", "s_waitcnt lgkmcnt(0)", "v_mov_b32_e32 v20, v5") == []


def test_checker_counts_in_order_completion():
    # two reads, lgkmcnt(1): the first has landed, the second has not
    lines = ("ds_read_b128 v[4:7], v1", "ds_read_b128 v[8:11], v2", "s_waitcnt lgkmcnt(1)")
    assert uses(*lines, "v_mov_b32_e32 v20, v5") == []
    assert uses(*lines, "v_mov_b32_e32 v20, v9") == ["v_mov_b32_e32 v20, v9"]


def test_checker_flags_an_overwrite_and_follows_branches():
    assert uses("ds_read_b64 v[4:5], v1", "v_mov_b32_e32 v4, 0", "s_waitcnt lgkmcnt(0)") == ["v_mov_b32_e32 v4, 0"]
    # a branch over the wait straight to the use
    found = uses("ds_read_b64 v[4:5], v1", "s_cbranch_scc1 1", "s_waitcnt lgkmcnt(0)", "v_add_f32_e32 v6, v4, v4")
    assert found == ["v_add_f32_e32 v6, v4, v4"]


@pytest.mark.skipif(not H.tools_available(), reason="ROCm llvm-objdump / clang-offload-bundler not found")
def test_built_library_waits_for_every_lds_result():
    if not os.path.exists(api.LIB_PATH):
        pytest.skip("library not built")
    funcs = H.parse(H.disassemble(api.LIB_PATH))
    assert any("fa_fp8_fwd_kernel" in k for k in funcs), "every code object of the library is checked"
    bad = {k: v for k, ins in funcs.items() if (v := L.early_lds_uses(ins))}
    assert not bad, "\n".join(f"{k[:80]}: {t}" for k, v in bad.items() for t in v[:3])
