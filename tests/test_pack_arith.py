"""Exhaustive host checks of the fp32 identities behind the packer's exact arithmetic and the
FP8 decode.

radiance_drafthead.py, _quantize_head_now: the scale is (hi - lo) / 3 and the codes come from
w / sc, each an IEEE fp32 division. The packer forms the first with an FMA-corrected product by
RN(1/3) and each w / sc with an FMA-corrected product by RN(1/sc); pack_arith_check.c checks both
against IEEE division over every input that matters (see its header).
"""
import os
import shutil
import subprocess
import tempfile

import pytest

HERE = os.path.dirname(os.path.abspath(__file__))


def _cc():
    for c in ("gcc", "cc", "clang"):
        if shutil.which(c):
            return c
    pytest.skip("no C compiler on this host")


def test_exhaustive_division_identities():
    cc = _cc()
    with tempfile.TemporaryDirectory() as tmp:
        exe = os.path.join(tmp, "pack_arith_check")
        src = os.path.join(HERE, "pack_arith_check.c")
        cmd = [cc, "-O2", "-ffp-contract=off", "-fopenmp", src, "-o", exe, "-lm"]
        if subprocess.run(cmd, capture_output=True).returncode != 0:
            cmd.remove("-fopenmp")
            subprocess.run(cmd, check=True, capture_output=True)
        p = subprocess.run([exe], capture_output=True, text=True, timeout=600)
    assert "fp8 checked 256 mismatches 0" in p.stdout, p.stdout
    assert "div3 checked 2139095040 mismatches 0" in p.stdout, p.stdout
    assert "quot checked 1073741824 mismatches 0" in p.stdout, p.stdout
    assert p.returncode == 0
