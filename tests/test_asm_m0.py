"""Host check on the generated gfx950 code (no GPU needed).

The direct global -> LDS tile copy (csrc/lds_copy.h) sets M0 to the LDS
destination inside inline assembly and lists M0 as clobbered.  M0 is one of
the compiler's reserved registers, and hipcc warns that a clobber of a
reserved register is not guaranteed to be honoured: a value the compiler kept
in M0 across the copy would be corrupted.  The kernels are therefore correct
only while the compiler itself never uses M0 in them.  This test compiles
every kernel source that includes the helper to assembly, with the library's
own flags, and fails if any instruction outside the helper's inline-assembly
blocks names M0, or if a block differs from the helper's three instructions (the copy takes
a 64-bit address, or a 32-bit offset from a base in scalar registers).
"""
import os
import re
import subprocess
import tempfile
from concurrent.futures import ThreadPoolExecutor

import pytest

from exact_attention_77_amd import build as B

HELPER_BLOCK = [r"s_mov_b32 m0, s\d+", r"s_nop 0",
                r"global_load_lds_dword(x4)? (v\[\d+:\d+\], off|v\d+, s\[\d+:\d+\])"]


def _sources_using_helper():
    out = []
    for src in B.sources():
        if not src.endswith(".hip"):
            continue
        text = open(os.path.join(B.CSRC, src), encoding="utf-8").read()
        if '#include "lds_copy.h"' in text:
            out.append(src)
    return out


def _device_asm(src, tmp):
    path = os.path.join(tmp, src + ".s")
    cmd = [B.HIPCC, *B.COMMON, *B.PER_FILE.get(src, []), "-x", "hip", "--cuda-device-only", "-S",
           os.path.join(B.CSRC, src), "-o", path]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-2000:]
    return open(path, encoding="utf-8").read()


def _m0_violations(asm):
    """Lines naming m0 outside the helper's blocks, and malformed blocks."""
    bad, block, n_blocks = [], None, 0
    for ln in asm.splitlines():
        s = ln.split(";")[0].strip()
        if ln.strip() == ";;#ASMSTART":
            block = []
            continue
        if ln.strip() == ";;#ASMEND":
            if any(re.search(r"\bm0\b", x) for x in block):
                n_blocks += 1
                if len(block) != 3 or not all(re.fullmatch(p, x) for p, x in zip(HELPER_BLOCK, block)):
                    bad.append("block: " + " | ".join(block))
            block = None
            continue
        if not s:
            continue
        if block is not None:
            block.append(re.sub(r"\s+", " ", s))
        elif re.search(r"\bm0\b", s):
            bad.append(s)
    return bad, n_blocks


def test_m0_only_in_copy_helper():
    srcs = _sources_using_helper()
    assert srcs, "no kernel source includes the copy helper"
    with tempfile.TemporaryDirectory() as tmp:
        with ThreadPoolExecutor(max_workers=min(4, len(srcs))) as ex:
            asms = list(ex.map(lambda s: _device_asm(s, tmp), srcs))
    for src, asm in zip(srcs, asms):
        bad, n_blocks = _m0_violations(asm)
        assert n_blocks > 0, f"{src}: no tile copy found in the generated code"
        assert not bad, f"{src}: M0 used outside the copy helper: {bad[:5]}"


def test_checker_flags_foreign_m0_use():
    """The checker itself: an M0 write by the compiler, or an extra
    instruction inside a helper block, must be reported."""
    ok = ";;#ASMSTART\n\ts_mov_b32 m0, s2\n\ts_nop 0\n\tglobal_load_lds_dwordx4 v[4:5], off\n;;#ASMEND\n"
    assert _m0_violations(ok) == ([], 1)
    bad, _ = _m0_violations(ok + "\ts_mov_b32 m0, -1\n\tds_read_b32 v1, v2\n")
    assert bad == ["s_mov_b32 m0, -1"]
    extra = ok.replace("s_nop 0\n", "s_nop 0\n\ts_mov_b32 s3, m0\n")
    bad, _ = _m0_violations(extra)
    assert len(bad) == 1 and bad[0].startswith("block:")
