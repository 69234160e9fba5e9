"""Checks of the compiled gfx950 device code (no GPU needed; needs hipcc).

Regressions these guard against, found in this library's own kernels:
  * an inline-asm block that writes SCC while the compiler keeps SCC live
    across it: a 64-bit address add split around the block (s_add_u32 before,
    s_addc_u32 after) loses its carry and the load faults; every block that
    writes SCC must be followed by a fresh SCC write before any SCC read;
  * buffer descriptors that the compiler treats as divergent: each load then
    sits in a waterfall loop (a nested loop around a buffer load); the chunk
    loops of the kernels must have none;
  * an MFMA accumulator handed from one MFMA shape to another (a 16x16x16
    product chained onto a 16x16x32 accumulator lost a contribution): every
    MFMA's accumulator is last written by an MFMA of its own shape, or by
    something other than an MFMA.
It also checks two properties the fused kernel's speed or correctness
rests on: the order of its direct-to-LDS g loads against the register
loads whose wait covers them, and no spill reloads inside its output loops.
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


MFMA = re.compile(r"^\s*(v_mfma_\w+)\s+(.*)$")
REG = re.compile(r"^([va])(?:\[(\d+):(\d+)\]|(\d+))$")


def _reg_range(tok):
    m = REG.match(tok.strip())
    if not m:
        return None
    lo = int(m.group(2) if m.group(2) is not None else m.group(4))
    hi = int(m.group(3) if m.group(3) is not None else m.group(4))
    return m.group(1), lo, hi


def mfma_shape_changes(lines):
    """(line, mfma, accumulator, writer, writer line) for every MFMA whose
    accumulator (C operand) an MFMA of another shape wrote last in the same
    basic block, and the number of MFMAs with a register accumulator."""
    found, checked = [], 0
    for i, line in enumerate(lines):
        m = MFMA.match(line)
        if not m:
            continue
        ops = [o.strip() for o in m.group(2).split(",")]
        if len(ops) < 4:
            continue
        c = _reg_range(ops[3].split()[0])
        if c is None:
            continue  # an inline constant accumulator (0)
        checked += 1
        for k in range(i - 1, -1, -1):
            prev = lines[k].strip()
            if prev.endswith(":"):
                break  # start of the basic block
            if not prev or prev.startswith(";") or prev.startswith("."):
                continue
            mnem = prev.split()[0]
            if "store" in mnem or "write" in mnem or mnem.startswith("s_"):
                continue
            rest = prev[len(mnem):].strip()
            dst = _reg_range(rest.split(",")[0]) if rest else None
            if dst is None or dst[0] != c[0] or dst[2] < c[1] or dst[1] > c[2]:
                continue
            pm = MFMA.match(lines[k])
            if pm and pm.group(1) != m.group(1):
                found.append((i + 1, m.group(1), ops[3], pm.group(1), k + 1))
            break
    return found, checked


def test_mfma_accumulators_keep_their_shape(device_asm):
    """No MFMA takes as its accumulator (C operand) a register tile that an
    MFMA of another shape wrote last. A 16x16x16 product chained onto a
    16x16x32 accumulator was seen to lose the last 16x16x32 contribution in
    two of the four output rows; each shape must start from a fresh
    accumulator (or a VALU-written one) instead."""
    total = 0
    for src, lines in device_asm.items():
        found, checked = mfma_shape_changes(lines)
        assert not found, "%s: %s" % (src, found[:3])
        total += checked
    assert total > 0


PLANTED = r"""
#include <hip/hip_runtime.h>
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
__global__ void planted(const bf16x8* a, const i16x4* b, f32x4* o) {
    const int l = threadIdx.x;
    f32x4 acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a[l], a[l + 64], f32x4{0.f, 0.f, 0.f, 0.f}, 0, 0, 0);
    acc = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(b[l], b[l + 64], acc, 0, 0, 0);
    o[l] = acc;
}
"""


def test_mfma_shape_check_catches_a_planted_chain(tmp_path):
    """The check above flags a kernel (compiled only, never run) that hands a
    16x16x32 accumulator to a 16x16x16 product."""
    if not os.path.exists(kbuild.HIPCC) and shutil.which("hipcc") is None:
        pytest.skip("hipcc not available")
    src = tmp_path / "planted.hip"
    src.write_text(PLANTED)
    dst = tmp_path / "planted.s"
    flags = [f for f in kbuild.FLAGS if f not in ("-shared", "-fPIC") and not f.startswith("-I")]
    subprocess.run([kbuild.HIPCC, *flags, "--cuda-device-only", "-S", "-o", str(dst), str(src)], check=True,
                   stdout=subprocess.DEVNULL, stderr=subprocess.DEVNULL)
    found, checked = mfma_shape_changes(dst.read_text().split("\n"))
    assert checked == 1 and len(found) == 1 and "16x16x16" in found[0][1] and "16x16x32" in found[0][3]


def _function_body(lines, name_prefix):
    """Lines of the first function whose symbol starts with name_prefix."""
    start = next(i for i, l in enumerate(lines) if re.match(re.escape(name_prefix) + r"\w*:", l))
    end = next(i for i in range(start, len(lines)) if "s_endpgm" in lines[i])
    return lines[start:end + 1]


def test_direct_to_lds_g_loads_precede_their_register_loads(device_asm):
    """The fused kernel's K1 wavefronts load each chunk's g rows straight into
    LDS and rely on the compiler's wait for the same chunk's register loads,
    issued later, to cover them (loads complete in order). In the start-up
    batches each chunk's g load opens its batch; in the chunk loop it is
    issued at the start of an interval and the register loads at its end,
    and no register load may have moved above it within the interval."""
    body = _function_body(device_asm["kda_kernels.hip"], "_ZN3kda9kda_fusedILb0EEEvNS_6K2ArgsE")
    blocks, cur = [], []
    for line in body:
        if re.match(r"^\.LBB\d+_\d+:", line) or re.match(r"^\s*s_(cbranch_\w+|branch)\b", line):
            blocks.append(cur)
            cur = []
        elif "s_barrier" in line:
            cur.append("barrier")
        elif "buffer_load" in line:
            cur.append("lds" if re.search(r"\blds\b", line) else "reg")
    blocks.append(cur)
    # barrier-delimited pieces (within a basic block): one interval's loads
    pieces = []
    for b in blocks:
        piece = []
        for e in b + ["barrier"]:
            if e == "barrier":
                if piece:
                    pieces.append(piece)
                piece = []
            else:
                piece.append(e)
    with_dma = [p for p in pieces if "lds" in p]
    assert sum(p.count("lds") for p in with_dma) >= 4, "direct-to-LDS loads not found"
    # the start-up piece issues whole batches, each opening with its g load
    start = with_dma[0]
    assert start[0] == "lds" and all(start[i + 1] == "reg" for i, e in enumerate(start[:-1]) if e == "lds"), start
    # in the chunk loop each interval issues the g load before any register load
    for p in with_dma[1:]:
        assert "reg" not in p[:p.index("lds")], p


def test_fused_chunk_loops_reload_no_spills(device_asm):
    """Spill reloads (scratch loads) inside the fused kernel's chunk loops
    that store output cost a memory round trip per chunk (one such reload in
    a Gram wavefront's loop made the 16 x 8192, 64-head batch 3% slower)."""
    body = _function_body(device_asm["kda_kernels.hip"], "_ZN3kda9kda_fusedILb0EEEvNS_6K2ArgsE")
    heads = {}
    for i, line in enumerate(body):
        m = re.match(r"^(\.LBB\d+_\d+):.*Loop Header", line)
        if m:
            heads[m.group(1)] = i
    checked = 0
    for label, h in heads.items():
        ends = [i for i, l in enumerate(body) if re.search(r"s_(cbranch_\w+|branch)\s+" + re.escape(label) + r"\s*$", l)]
        if not ends or max(ends) < h:
            continue
        loop = body[h:max(ends) + 1]
        if not any("buffer_store" in l or "global_store" in l for l in loop):
            continue
        checked += 1
        assert not any("scratch_load" in l for l in loop), "spill reload in an output loop at line %d" % h
    assert checked >= 3
