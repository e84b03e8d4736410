"""Checks on the gfx950 assembly of every kernel source (CPU only: hipcc
cross-compiles).

* Loads that copy HBM straight into LDS are written as inline asm, which the
  compiler's hazard checks do not see into.  The ISA requires 5 wait states
  between a VALU write of an SGPR (readlane, readfirstlane) and a
  vector-memory instruction that reads it, and 1 between an M0 write and an
  LDS-DMA load; a missing wait lets the load use a stale address.  Every
  such load must have them.
* No kernel may touch scratch memory or use flat addressing (a sign that
  values spilled or that a pointer lost its address space).
"""
import os
import re
import shutil
import subprocess
from concurrent.futures import ThreadPoolExecutor

import pytest

from compressed_sparse_attention_06_amd import build as B

HIP_SOURCES = [s for s in B.SOURCES if s.endswith(".hip")]


def _asm(src, tmp_path):
    out = tmp_path / (os.path.splitext(src)[0] + ".s")
    cmd = [B.HIPCC, *B.CFLAGS, *B.EXTRA.get(src, []), "--cuda-device-only", "-S", os.path.join(B.CSRC, src),
           "-o", str(out)]
    res = subprocess.run(cmd, capture_output=True, text=True)
    assert res.returncode == 0, res.stderr[-2000:]
    return out.read_text()


@pytest.fixture(scope="module")
def asm(tmp_path_factory):
    if shutil.which(B.HIPCC) is None and not os.path.exists(B.HIPCC):
        pytest.skip("hipcc not available")
    tmp = tmp_path_factory.mktemp("asm")
    with ThreadPoolExecutor(max_workers=len(HIP_SOURCES)) as ex:
        texts = list(ex.map(lambda s: _asm(s, tmp), HIP_SOURCES))
    return dict(zip(HIP_SOURCES, texts))


def _instructions(text):
    """(kernel, instruction) pairs in program order; labels, directives and
    comments dropped."""
    kernel, out = None, []
    for raw in text.splitlines():
        line = raw.split(";")[0].strip()
        if not line:
            continue
        m = re.match(r"^(_Z\w+):", line)
        if m:
            kernel = m.group(1)
            continue
        if line.startswith(".") or line.endswith(":"):
            continue
        out.append((kernel, line))
    return out


def _sgprs(operand):
    m = re.fullmatch(r"s\[(\d+):(\d+)\]", operand)
    if m:
        return {f"s{k}" for k in range(int(m.group(1)), int(m.group(2)) + 1)}
    return {operand} if re.fullmatch(r"s\d+", operand) else set()


def lds_dma_hazards(text):
    """Violations before every LDS-DMA load of `text` (see module docstring)."""
    ins = _instructions(text)
    bad = []
    for i, (kernel, line) in enumerate(ins):
        if not line.startswith("global_load_lds") and not re.match(r"buffer_load_\w+ .*\blds\b", line):
            continue
        ops = [o.strip() for o in line.split(None, 1)[1].split(",")] if " " in line else []
        regs = set().union(*[_sgprs(o) for o in ops]) if ops else set()
        waits = 0
        for back in range(1, 6):
            if i - back < 0 or waits >= 5:
                break
            prev = ins[i - back][1]
            if prev.startswith("s_nop"):
                waits += int(prev.split()[1]) + 1
                continue
            dst = prev.split(None, 1)[1].split(",")[0].strip() if " " in prev else ""
            if prev.startswith("v_") and _sgprs(dst) & regs:
                bad.append((kernel, f"VALU writes {dst} {waits} wait states before: {line}"))
                break
            if back == 1 and dst == "m0":
                bad.append((kernel, f"M0 written right before: {line}"))
            waits += 1
    return bad


def test_hazard_scanner_flags_known_patterns():
    """The scanner itself: each violation is caught, the padded forms pass."""
    k = "_Zkernel:\n"
    assert lds_dma_hazards(k + "v_readlane_b32 s4, v4, 0\nv_readlane_b32 s5, v5, 0\n"
                               "global_load_lds_dwordx4 v1, s[4:5]\n")
    assert lds_dma_hazards(k + "s_mov_b32 m0, s3\nglobal_load_lds_dwordx4 v1, s[4:5]\n")
    assert not lds_dma_hazards(k + "v_readlane_b32 s4, v4, 0\ns_mov_b32 m0, s3\ns_nop 4\n"
                                   "global_load_lds_dwordx4 v1, s[4:5]\n")
    assert not lds_dma_hazards(k + "v_readlane_b32 s6, v4, 0\ns_mov_b32 m0, s3\ns_nop 0\n"
                                   "global_load_lds_dwordx4 v1, s[4:5]\n")


@pytest.mark.parametrize("src", HIP_SOURCES)
def test_lds_dma_wait_states(asm, src):
    bad = lds_dma_hazards(asm[src])
    assert not bad, f"{src}: {len(bad)} LDS-DMA hazards, first: {bad[:3]}"


@pytest.mark.parametrize("src", HIP_SOURCES)
def test_no_scratch_or_flat(asm, src):
    hits = [(k, l) for k, l in _instructions(asm[src]) if re.match(r"(scratch|flat)_", l)]
    assert not hits, f"{src}: {len(hits)} scratch/flat instructions, first: {hits[:3]}"
