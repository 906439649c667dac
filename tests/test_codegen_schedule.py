"""The compiled schedule of the eight-wave attention step is the one the source pins
(CPU: compiles attn.hip for gfx950 and reads the assembly).

The step interleaves each QK product of the next subtile with two of this subtile's
weights (fma, exp2).  Without the pins the optimiser gathers every exp2 of a step
behind the last product, and the softmax no longer overlaps the matrix core; this
test fails if that happens again."""

import os
import re
import shutil
import subprocess

import pytest

from tree_attention_verify_ancestor_amd import build as tvbuild

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
KERNEL = "_ZN2tv9attn_bf16ILi128ELi8ELi1ELi1EEEvNS_8AttnArgsE"


def _function_asm(tmp_path):
    src = os.path.join(tvbuild.PKG, "csrc", "attn.hip")
    out = tmp_path / "attn.s"
    flags = [f for f in tvbuild.HIPCC_FLAGS if f not in ("-shared", "-fPIC")]
    subprocess.run([HIPCC, "-S", "--offload-device-only", *flags, "-I",
                    os.path.join(tvbuild.ROOT, "include"), src, "-o", str(out)],
                   check=True, capture_output=True)
    lines = out.read_text().split("\n")
    start = next(i for i, l in enumerate(lines) if l.startswith(KERNEL + ":"))
    end = next(i for i in range(start, len(lines)) if "s_endpgm" in lines[i])
    return lines[start:end]


def _blocks(lines):
    """Basic blocks as lists of instruction mnemonics."""
    blocks, cur = [], []
    for l in lines:
        if re.match(r"^\.LBB\d+_\d+:", l):
            blocks.append(cur)
            cur = []
        elif l.strip() and not l.strip().startswith((";", ".")):
            cur.append(l.split()[0])
    blocks.append(cur)
    return blocks


@pytest.mark.skipif(not (os.path.exists(HIPCC) or shutil.which("hipcc")), reason="hipcc missing")
def test_softmax_interleaves_with_the_products(tmp_path):
    check_interleaved(_blocks(_function_asm(tmp_path)))


def check_interleaved(blocks):
    # blocks holding whole steps: 16 products (8 QK, 8 PV), 16 exponentials and 16 V^T
    # reads from LDS each (the exact fallback path reads global memory and is not
    # pipelined)
    steps = [b for b in blocks if b.count("v_mfma_f32_32x32x16_bf16") >= 16 and b.count("v_exp_f32_e32") >= 16
             and b.count("ds_read_b64_tr_b16") >= 16]
    assert steps, "no block with a whole step of the pipeline"
    for b in steps:
        mf = [i for i, op in enumerate(b) if op == "v_mfma_f32_32x32x16_bf16"]
        gaps_with_exp = sum(any(op == "v_exp_f32_e32" for op in b[x + 1:y]) for x, y in zip(mf, mf[1:]))
        # each step has 7 gaps between its 8 QK products, each carrying two weights
        n_steps = min(len(mf), b.count("v_exp_f32_e32")) // 16
        assert gaps_with_exp >= 6 * n_steps, (gaps_with_exp, len(mf))
