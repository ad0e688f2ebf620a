"""Checks of the compiled gfx950 code (CPU only: hipcc cross-compiles).

The grouped GEMMs copy operands global -> LDS with inline-asm
global_load_lds_dwordx4 / buffer_load_dwordx4 ... lds instructions whose LDS
address the asm writes into m0 itself.
That is sound only while no compiler-generated instruction of those kernels
reads m0 (the compiler would not know the asm changed it).  This test
compiles every source that includes the copy helper and checks the code:
every m0 reference is the asm's own write, directly followed by its copy,
and no instruction that reads m0 implicitly appears anywhere else.
"""
import importlib.util
import os
import re
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "sparsely_gated_mixture_amd", "csrc")

# Instructions that read m0 without naming it (besides buffer loads carrying
# the lds modifier, matched on the whole line below).
IMPLICIT_M0 = re.compile(r"^(s_movrel|v_movrel|s_sendmsg|ds_gws|ds_append|ds_consume|"
                         r"ds_ordered_count|s_set_gpr_idx|v_interp|ds_param|ds_direct|"
                         r"buffer_load_\w*lds|global_load_lds|scratch_load_lds|"
                         r"\w+_addtid)")


def _build_flags():
    spec = importlib.util.spec_from_file_location(
        "_moe_build", os.path.join(ROOT, "sparsely_gated_mixture_amd", "build.py"))
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    return mod


def _dma_sources():
    return sorted(f for f in os.listdir(CSRC) if f.endswith(".hip")
                  and '#include "lds_dma.h"' in open(os.path.join(CSRC, f)).read())


@pytest.mark.skipif(shutil.which("hipcc") is None and not os.path.exists("/opt/rocm/bin/hipcc"),
                    reason="hipcc not available")
@pytest.mark.parametrize("src", _dma_sources())
def test_m0_is_written_only_by_the_copy_helper(src, tmp_path):
    b = _build_flags()
    out = tmp_path / (src + ".s")
    cmd = [b._hipcc()] + b.COMMON + b.DEVICE + ["--cuda-device-only", "-S",
                                                 os.path.join(CSRC, src), "-o", str(out)]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-2000:]
    lines = [l.split(";")[0].strip() for l in out.read_text().splitlines()]
    code = [l for l in lines if l and not l.startswith(".") and not l.endswith(":")]
    copies = 0
    for i, ins in enumerate(code):
        op = ins.split()[0]
        if re.search(r"\bm0\b", ins):
            assert op == "s_mov_b32" and ins.split()[1].rstrip(",") == "m0", (
                f"{src}: compiler-generated use of m0: {ins}")
            nxt = code[i + 2]
            assert code[i + 1] == "s_nop 0" and (
                nxt.startswith("global_load_lds_dwordx4") or
                (nxt.startswith("buffer_load_dwordx4") and nxt.endswith(" lds"))), (
                f"{src}: m0 write not followed by its copy: {ins}")
        elif IMPLICIT_M0.match(op) or (op.startswith("buffer_load") and ins.endswith(" lds")):
            is_copy = op == "global_load_lds_dwordx4" or (op == "buffer_load_dwordx4" and
                                                          ins.endswith(" lds"))
            assert is_copy and code[i - 2].startswith("s_mov_b32 m0"), (
                f"{src}: instruction reading m0 outside the copy helper: {ins}")
            copies += 1
    assert copies > 0, f"{src}: no global->LDS copies found"
