"""The compiled gfx950 kernels never read an MFMA result too soon (see mfma_hazards)."""

import os
import shutil
import subprocess

import pytest

import mfma_hazards
from tree_attention_verify_ancestor_amd import build as tvbuild

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")


@pytest.mark.skipif(not (os.path.exists(HIPCC) or shutil.which("hipcc")), reason="hipcc missing")
@pytest.mark.parametrize("src", [os.path.basename(p) for p in tvbuild.sources()])
def test_no_mfma_read_hazard(src, tmp_path):
    path = os.path.join(tvbuild.PKG, "csrc", src)
    out = tmp_path / (src + ".s")
    flags = [f for f in tvbuild.HIPCC_FLAGS if f not in ("-shared", "-fPIC")]
    subprocess.run([HIPCC, "-S", "--offload-device-only", *flags, "-I",
                    os.path.join(tvbuild.ROOT, "include"), path, "-o", str(out)],
                   check=True, capture_output=True)
    found = mfma_hazards.scan(out.read_text())
    assert not found, "\n".join(found[:5])


def test_scanner_catches_a_short_branch_path():
    """A hand-written shape of the miscompile: MFMA, taken branch, 4 nops, read."""
    asm = "\n".join([
        "kern:",
        "v_mfma_f32_32x32x16_bf16 a[64:79], v[72:75], v[112:115], a[64:79]",
        "s_cbranch_vccnz .LBB1_54",
        "v_mov_b32 v1, v2", "v_mov_b32 v1, v2", "v_mov_b32 v1, v2", "v_mov_b32 v1, v2",
        "v_mov_b32 v1, v2", "v_mov_b32 v1, v2", "v_mov_b32 v1, v2",
        ".LBB1_54:",
        "s_nop 3",
        "v_accvgpr_read_b32 v83, a79",
    ])
    assert len(mfma_hazards.scan(asm)) == 1
    safe = asm.replace("s_nop 3", "s_nop 7\ns_nop 3")
    assert mfma_hazards.scan(safe) == []
