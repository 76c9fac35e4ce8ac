"""Compiled-code check: no SCC reader whose condition was overwritten.

Compiles every library source to gfx950 assembly (hipcc, no GPU needed) and
scans it with tests/isa_scc.py; the scanner itself is checked on fixtures of
a bad and a good instruction sequence from gfx950 builds.
"""
import os
import shutil
import subprocess
import tempfile
from concurrent.futures import ThreadPoolExecutor

import pytest

from tests.isa_scc import suspicious_scc_reads

HERE = os.path.dirname(os.path.abspath(__file__))
GOLDEN = os.path.join(HERE, "golden")


def test_scanner_flags_select_after_clobbered_scc():
    with open(os.path.join(GOLDEN, "scc_select_after_clobber.s")) as f:
        found = suspicious_scc_reads(f.read())
    assert [f[1] for f in found] == ["s_cselect_b32 s8, 0, s34"]
    assert found[0][3].startswith("s_lshr_b64")


def test_scanner_accepts_compare_and_carry_selects():
    with open(os.path.join(GOLDEN, "scc_select_ok.s")) as f:
        assert suspicious_scc_reads(f.read()) == []


@pytest.mark.timeout(600)
def test_library_assembly_has_no_select_after_clobbered_scc():
    from exact_attention_45_amd import build as B
    try:
        cc = B.hipcc()
    except RuntimeError:
        pytest.skip("hipcc not available")
    tmp = tempfile.mkdtemp(prefix="miattn_isa_")
    try:
        def compile_one(src):
            out = os.path.join(tmp, src.replace(".hip", ".s"))
            cmd = [cc, *B.HIP_FLAGS, "-I", B.INCLUDE, "-I", B.CSRC, *B.SOURCE_FLAGS.get(src, []),
                   "--cuda-device-only", "-S", os.path.join(B.CSRC, src), "-o", out]
            r = subprocess.run(cmd, capture_output=True, text=True)
            assert r.returncode == 0, r.stderr[-2000:]
            with open(out) as f:
                return src, suspicious_scc_reads(f.read())

        with ThreadPoolExecutor(max_workers=4) as ex:
            results = list(ex.map(compile_one, B.SOURCES))
    finally:
        shutil.rmtree(tmp, ignore_errors=True)
    bad = {src: found[:3] for src, found in results if found}
    assert not bad, f"SCC read after a clobbering writer: {bad}"
