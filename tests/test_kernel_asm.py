"""Static checks on the gfx950 machine code of the HIP kernels (CPU only).

Every kernel source is compiled to device assembly with the library's own
flags and scanned for MFMA instructions whose destination registers partially
overlap their accumulator input (C) registers.  Such an instruction is not a
valid MFMA encoding, and the compiler has produced one (from a partially
unrolled loop carrying two accumulators, which it rotated through AGPR moves);
the result was silently wrong values.  Exact overlap (accumulate in place) and
disjoint ranges are both fine.
"""
import concurrent.futures as cf
import os
import re
import shutil
import subprocess

import pytest

from looped_hybrid_attention_amd import build as B

HIP_SOURCES = sorted(f for f in os.listdir(B.CSRC) if f.endswith(".hip"))

_REG = re.compile(r"([av])\[(\d+):(\d+)\]$|([av])(\d+)$")


def _range(tok):
    m = _REG.match(tok.strip())
    if not m:
        return None
    if m.group(1):
        return m.group(1), int(m.group(2)), int(m.group(3))
    return m.group(4), int(m.group(5)), int(m.group(5))


def partial_overlaps(asm: str):
    """(function, instruction) for each MFMA whose D and C ranges partially overlap."""
    out, func = [], None
    for line in asm.splitlines():
        m = re.match(r"^(_Z\S+):", line)
        if m:
            func = m.group(1)
        if "v_mfma" not in line:
            continue
        ops = line.split(None, 1)[1].split(",")
        if len(ops) < 4:
            continue
        d, c = _range(ops[0]), _range(ops[3])
        if d and c and d[0] == c[0] and (d[1], d[2]) != (c[1], c[2]) and d[1] <= c[2] and c[1] <= d[2]:
            out.append((func, line.strip()))
    return out


def test_checker_flags_partial_overlap():
    asm = ("_Zfoo:\n"
           "\tv_mfma_f32_16x16x4_f32 a[0:3], v1, v2, a[2:5]\n"
           "\tv_mfma_f32_16x16x4_f32 a[4:7], v1, v2, a[4:7]\n"
           "\tv_mfma_f32_16x16x4_f32 a[8:11], v1, v2, a[12:15]\n"
           "\tv_mfma_f32_32x32x16_bf16 v[0:15], v[16:19], v[20:23], 0\n")
    bad = partial_overlaps(asm)
    assert len(bad) == 1 and "a[0:3]" in bad[0][1]


def _asm(src, tmp):
    out = os.path.join(tmp, os.path.basename(src) + ".s")
    cmd = [B.HIPCC, *[f for f in B.FLAGS if f != "-fPIC"], "--cuda-device-only", "-S", src, "-o", out]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-2000:]
    with open(out) as fh:
        return fh.read()


@pytest.mark.skipif(not shutil.which(B.HIPCC) and not os.path.exists(B.HIPCC), reason="hipcc not available")
def test_no_partially_overlapping_mfma(tmp_path):
    srcs = [os.path.join(B.CSRC, f) for f in HIP_SOURCES]
    with cf.ThreadPoolExecutor(max_workers=min(8, len(srcs))) as ex:
        asms = list(ex.map(lambda s: _asm(s, str(tmp_path)), srcs))
    bad = [(os.path.basename(s), f, i) for s, a in zip(srcs, asms) for f, i in partial_overlaps(a)]
    assert not bad, "MFMA destination partially overlaps its C operand:\n" + "\n".join(map(str, bad[:10]))
