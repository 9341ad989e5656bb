"""The built library leaves every matrix-product result alone for at least 12
wait states (see mfma_hazards.py), and the checker itself finds planted cases."""
import os

import pytest

import mfma_hazards as H
from exact_attention_72_amd import api


def listing(*lines, base=0x1000):
    """objdump-style text for one kernel from instruction strings (4 bytes each)."""
    out = [f"{base:016x} <k>:"]
    for i, t in enumerate(lines):
        out.append(f"\t{t} // {base + 4 * i:012X}: 0")
    return "\n".join(out)


MFMA = "v_mfma_f32_32x32x16_bf16 a[0:15], v[0:3], v[4:7], a[0:15]"


def hits(*lines):
    return H.close_accesses(H.parse(listing(*lines))["k"])


def test_checker_flags_a_read_right_after_the_product():
    found = hits(MFMA, "s_nop 3", "v_accvgpr_read_b32 v8, a5")
    assert len(found) == 1 and found[0][2] == 4


def test_checker_accepts_a_read_after_enough_wait_states():
    assert hits(MFMA, "s_nop 7", "s_nop 3", "v_accvgpr_read_b32 v8, a5") == []


def test_checker_ignores_registers_the_product_does_not_write():
    assert hits(MFMA, "v_accvgpr_read_b32 v8, a16", "v_add_f32_e32 v9, v0, v4") == []


def test_checker_flags_an_overwrite_of_the_accumulator():
    assert len(hits(MFMA, "s_nop 1", "v_accvgpr_write_b32 a15, v2")) == 1


def test_checker_follows_a_branch_to_the_reader():
    # the product, then a branch over 8 nops straight to the read: 1 wait state
    found = hits(MFMA, "s_branch 8", *(["s_nop 0"] * 8), "v_accvgpr_read_b32 v8, a0")
    assert len(found) == 1 and found[0][2] == 1


@pytest.mark.skipif(not H.tools_available(), reason="ROCm llvm-objdump / clang-offload-bundler not found")
def test_built_library_has_no_early_accumulator_access():
    if not os.path.exists(api.LIB_PATH):
        pytest.skip("library not built")
    bad = H.scan_library(api.LIB_PATH)
    lines = [f"{k[:70]}: {t} after {w} wait states from {m}" for k, v in bad.items() for t, m, w in v[:3]]
    assert not bad, "\n".join(lines)
