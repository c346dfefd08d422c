"""Machine-code check of the HIP sources: every workgroup barrier must be
preceded by a wait for the wave's LDS operations (lgkmcnt 0), so that LDS
data handed between waves across a barrier has landed. The compiler has been
seen to drop that wait where the barrier heads a loop, which let a vote flag
written at the end of one step be read stale in the next."""

import os
import re
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "sparse_attention_long_skip_amd", "csrc")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

_LDS_WRITE = re.compile(r"^\s*(ds_write|ds_store|ds_add|ds_sub|ds_max|ds_min|ds_and|ds_or|ds_xor|ds_inc|"
                        r"ds_dec|ds_cmpst|ds_wrxchg)")


def _unwaited_barriers(asm: str):
    bad = []
    lines = asm.splitlines()
    for i, l in enumerate(lines):
        if l.strip() != "s_barrier":
            continue
        j = i - 1
        while j >= 0:
            s = lines[j].strip()
            if s.startswith("s_waitcnt") and "lgkmcnt(0)" in s:
                break
            if _LDS_WRITE.match(s) or lines[j].startswith(".LBB") or re.match(r"^_Z\w+:", lines[j]):
                bad.append((i + 1, lines[j].strip()))
                break
            j -= 1
    return bad


@pytest.mark.skipif(not os.path.exists(HIPCC), reason="hipcc not available")
@pytest.mark.parametrize("src", ["prefill.hip", "mask.hip", "vslash.hip", "calibrate.hip"])
def test_every_barrier_waits_for_lds(src, tmp_path):
    out = tmp_path / (src + ".s")
    cmd = [HIPCC, "--offload-arch=gfx950", "-O3", "-std=c++17", "-Xclang", "-target-feature", "-Xclang",
           "-packed-fp32-ops", "-I", CSRC, "--cuda-device-only", "-S", "-o", str(out),
           os.path.join(CSRC, src)]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-2000:]
    bad = _unwaited_barriers(out.read_text())
    assert not bad, f"{src}: barriers without a preceding LDS wait at {bad[:5]}"
