"""Static check of the gfx950 assembly of every kernel source (CPU only: hipcc
cross-compiles).  An MFMA does not honour the lane mask, so an MFMA inside a
lane-masked block that the compiler emits without an execz skip branch still
writes its accumulator in a wave whose lanes are all masked off.  Every such
block must therefore be absent: wave-uniform conditions around MFMAs belong in
scalar registers (readfirstlane) or in compile-time loop bounds."""
import concurrent.futures as cf
import os
import re
import subprocess

import pytest

from chunked_gated_delta_06_amd import build as b

SRC = os.path.join(os.path.dirname(b.__file__), "csrc")
SOURCES = sorted(f for f in os.listdir(SRC) if f.endswith(".hip"))


def unskipped_mfma_blocks(asm: str):
    lines = asm.split("\n")
    fn, start, bad = None, None, []
    for i, line in enumerate(lines):
        t = line.strip()
        m = re.match(r"^(_Z\S+):", line)
        if m:
            fn = m.group(1)
        if t.startswith("s_and_saveexec"):
            start, mf = i, 0
            skip = any("execz" in lines[k] for k in range(i + 1, min(i + 3, len(lines))))
        elif start is not None and "v_mfma" in t:
            mf += 1
        elif start is not None and re.match(r"s_(or|andn2|xor|mov)_b64 exec", t):
            if mf and not skip:
                bad.append(f"{fn}: lines {start + 1}-{i + 1}, {mf} MFMA")
            start = None
    return bad


def compile_asm(src, tmp):
    out = os.path.join(tmp, src + ".s")
    cmd = [b.HIPCC, *[f for f in b.CFLAGS if f != "-fPIC"], "--cuda-device-only", "-S",
           os.path.join(SRC, src), "-o", out]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-2000:]
    return open(out).read()


@pytest.mark.skipif(not os.path.exists(b.HIPCC), reason="hipcc not installed")
def test_no_mfma_in_unskipped_masked_blocks(tmp_path):
    with cf.ThreadPoolExecutor(min(8, os.cpu_count() or 1)) as ex:
        asms = dict(zip(SOURCES, ex.map(lambda s: compile_asm(s, str(tmp_path)), SOURCES)))
    bad = {s: unskipped_mfma_blocks(a) for s, a in asms.items()}
    bad = {s: v for s, v in bad.items() if v}
    assert not bad, bad


def test_checker_flags_the_pattern():
    """The scanner itself: a masked block holding an MFMA and no skip branch is
    reported; the same block behind s_cbranch_execz is not."""
    body = "\n".join([
        "_ZN3gdr4testEv:",
        "\ts_and_saveexec_b64 s[4:5], vcc",
        "\tv_mfma_f32_16x16x32_bf16 v[0:3], v[4:7], v[8:11], 0",
        "\ts_or_b64 exec, exec, s[4:5]",
    ])
    assert len(unskipped_mfma_blocks(body)) == 1
    skipped = body.replace("vcc\n", "vcc\n\ts_cbranch_execz .LBB0_2\n")
    assert unskipped_mfma_blocks(skipped) == []
