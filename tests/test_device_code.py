"""Checks of the compiled gfx950 device code (no GPU needed; needs hipcc).

Regressions these guard against, both found in this library's own kernels:
  * an inline-asm block that writes SCC while the compiler keeps SCC live
    across it: a 64-bit address add split around the block (s_add_u32 before,
    s_addc_u32 after) loses its carry and the load faults; every block that
    writes SCC must be followed by a fresh SCC write before any SCC read;
  * buffer descriptors that the compiler treats as divergent: each load then
    sits in a waterfall loop (a nested loop around a buffer load); the chunk
    loops of the kernels must have none.
"""
import os
import re
import shutil
import subprocess

import pytest

from kda_chunked_delta_amd import build as kbuild

SCC_WRITERS = re.compile(r"^\s*(s_add_u32|s_sub_u32|s_add_i32|s_sub_i32|s_addk_i32|s_cmp\w*|s_max_\w+|s_min_\w+|"
                         r"s_and_b\d+|s_or_b\d+|s_xor_b\d+|s_andn2_\w+|s_orn2_\w+|s_lshl\w*|s_lshr\w*|s_ashr\w*|"
                         r"s_bfe\w*|s_abs\w*|s_not_\w+|s_\w+_saveexec_\w+)\b")
SCC_READERS = re.compile(r"^\s*(s_addc_u32|s_subb_u32|s_cselect_\w+|s_cbranch_scc[01]|s_cmov\w*)\b")


@pytest.fixture(scope="module")
def device_asm(tmp_path_factory):
    if not os.path.exists(kbuild.HIPCC) and shutil.which("hipcc") is None:
        pytest.skip("hipcc not available")
    out = tmp_path_factory.mktemp("isa")
    flags = [f for f in kbuild.FLAGS if f not in ("-shared", "-fPIC")]
    texts = {}
    for src in ("kda_kernels.hip", "kda_decode.hip"):
        dst = str(out / (src + ".s"))
        subprocess.run([kbuild.HIPCC, *flags, "--cuda-device-only", "-S", "-o", dst,
                        os.path.join(kbuild.HERE, "csrc", src)], check=True,
                       stdout=subprocess.DEVNULL, stderr=subprocess.DEVNULL)
        texts[src] = open(dst).read().split("\n")
    return texts


def test_inline_asm_does_not_break_live_scc(device_asm):
    checked = 0
    for src, lines in device_asm.items():
        for i, line in enumerate(lines):
            if ";;#ASMSTART" not in line:
                continue
            j = i + 1
            while ";;#ASMEND" not in lines[j]:
                j += 1
            if not any(SCC_WRITERS.match(x) for x in lines[i + 1:j]):
                continue
            checked += 1
            for k in range(j + 1, len(lines)):
                if SCC_READERS.match(lines[k]):
                    raise AssertionError("%s line %d: SCC read after an SCC-writing asm block (line %d) with "
                                         "no fresh SCC write between: %s" % (src, k + 1, i + 1, lines[k].strip()))
                if SCC_WRITERS.match(lines[k]) or lines[k].startswith(".LBB") or "s_branch" in lines[k]:
                    break
    assert checked > 0


def test_chunk_loops_have_no_waterfall_loads(device_asm):
    lines = device_asm["kda_kernels.hip"]
    fn, depth2 = None, False
    for line in lines:
        if re.match(r"^_ZN3kda\w+:", line):
            fn = line
        if "Inner Loop Header: Depth=2" in line:
            depth2 = True
        elif line.startswith(".LBB") or line.startswith(".Lfunc_end"):
            depth2 = "Depth=2" in line
        if depth2 and "buffer_load" in line:
            raise AssertionError("a buffer load inside a nested (waterfall) loop in %s" % fn)
