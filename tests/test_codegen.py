"""Code generation of the MFMA attention kernel (CPU: hipcc cross-compiles
gfx950).  The kernel keeps its whole accumulator tile in AGPRs and its query
operands in VGPRs, at the register file's limit; the row pipeline relies on
explicit vmcnt waits for LDS DMAs issued several tiles ahead.  A register
spill inside the tile loop brings a scratch reload and a full vmcnt(0) wait
into every tile, which drains that pipeline (a 40 % slowdown when it last
happened, with identical results), so it is checked here rather than by the
timing."""
import os
import re
import shutil
import subprocess

import pytest

from long_context_attention_15_amd import build as B

SRC = os.path.join(B.CSRC, "attn_m32.hip")


def _tile_loops(asm):
    """{label: body lines} of the innermost loops (backward branches) whose
    body holds at least 96 MFMA instructions: the tile loops, one per pass
    of each instantiation."""
    lines = asm.split("\n")
    labels = {}
    for i, line in enumerate(lines):
        m = re.match(r"^(\.LBB\d+_\d+):", line)
        if m:
            labels[m.group(1)] = i
    spans = []
    for i, line in enumerate(lines):
        m = re.search(r"s_c?branch\w*\s+(\.LBB\d+_\d+)", line)
        if m and m.group(1) in labels and labels[m.group(1)] < i:
            a = labels[m.group(1)]
            if sum("v_mfma" in x for x in lines[a: i + 1]) >= 96:
                spans.append((a, i, m.group(1)))
    inner = [s for s in spans if not any(o != s and s[0] <= o[0] and o[1] <= s[1] and (o[0], o[1]) != (s[0], s[1])
                                         for o in spans)]
    return {name: lines[a: e + 1] for a, e, name in inner}


@pytest.mark.skipif(not os.path.exists(B.HIPCC) and shutil.which("hipcc") is None, reason="hipcc not available")
def test_attention_tile_loops_have_no_spills_or_full_waits(tmp_path):
    out = tmp_path / "attn_m32.s"
    cmd = [B.HIPCC] + B.FLAGS + ["--offload-device-only", "-S", SRC, "-o", str(out)]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-2000:]
    loops = _tile_loops(out.read_text())
    assert len(loops) >= 4, f"expected the tile loops of both instantiations, found {len(loops)}"
    for name, body in loops.items():
        scratch = [x.strip() for x in body if "scratch_" in x]
        full = [x.strip() for x in body if re.search(r"s_waitcnt\s+vmcnt\(0\)", x)]
        assert not scratch, f"{name}: scratch accesses in the tile loop: {scratch[:4]}"
        assert not full, f"{name}: full vmcnt waits in the tile loop: {full[:4]}"
