"""Code-generation guards on the library's gfx950 assembly (CPU, cross-compiled).

- No kernel uses scratch memory: register spills of these kernels go to
  per-lane scratch in HBM, on the hot path.
- No kernel wraps a memory access in a loop over the distinct values of an
  operand that must be wave-uniform (a buffer resource or scalar offset the
  compiler could not prove uniform): such a loop reads the operand lane by lane
  (v_readfirstlane), runs the access for the matching lanes and repeats, which
  multiplies the instructions around every access.
"""
import os
import re
import subprocess

import pytest

from hyper_connection_residual_mixes_amd import build as hip_build

SOURCES = ["hc_kernels.hip", "hc_generic.hip", "hc_noalloc.hip"]


def _asm(src, tmp_path):
    out = tmp_path / (src + ".s")
    cmd = [hip_build.hipcc(), *hip_build.HIP_FLAGS, "--cuda-device-only", "-S",
           "-I", os.path.join(hip_build.ROOT, "include"), "-I", hip_build.CSRC,
           os.path.join(hip_build.CSRC, src), "-o", str(out)]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-2000:]
    return out.read_text()


def kernels(asm: str):
    """(name, body) of every kernel in an assembly listing."""
    parts = re.split(r"\n(_Z\w+):[^\n]*\n", asm)
    return [(parts[i], parts[i + 1].split(".Lfunc_end")[0]) for i in range(1, len(parts), 2)]


def waterfall_loops(body: str) -> int:
    """Backward s_cbranch_execnz whose loop ends by flipping exec (s_xor exec) and
    reads a lane's value into a scalar register."""
    lines = [l.split(";")[0].strip() for l in body.split("\n")]
    lines = [l for l in lines if l]
    labels = {m.group(1): i for i, l in enumerate(lines) for m in [re.match(r"^(\.LBB\w+):", l)] if m}
    count = 0
    for i, l in enumerate(lines):
        m = re.match(r"s_cbranch_execnz\s+(\.LBB\w+)$", l)
        if not m or labels.get(m.group(1), i) >= i:
            continue
        loop = lines[labels[m.group(1)]:i]
        if any(re.match(r"s_xor_b(32|64)\s+exec,\s*exec", x) for x in lines[max(0, i - 2):i]) \
                and any(x.startswith("v_readfirstlane") for x in loop):
            count += 1
    return count


def test_detector_finds_a_waterfall_loop():
    body = "\n".join([".LBB0_1:", "v_readfirstlane_b32 s4, v10", "v_cmp_eq_u32_e32 vcc, s4, v10",
                      "s_and_saveexec_b64 s[0:1], vcc", "buffer_load_dwordx4 v[2:5], v1, s[4:7], 0 offen",
                      "s_xor_b64 exec, exec, s[0:1]", "s_cbranch_execnz .LBB0_1"])
    assert waterfall_loops(body) == 1
    assert waterfall_loops(body.replace("v_readfirstlane_b32 s4, v10", "s_mov_b32 s4, 0")) == 0


@pytest.mark.parametrize("src", SOURCES)
def test_no_scratch_and_no_waterfall_loops(src, tmp_path):
    asm = _asm(src, tmp_path)
    ks = kernels(asm)
    if src != "hc_noalloc.hip":
        assert ks, "no kernels found"
    scratch = re.findall(r"\.amdhsa_kernel (\S+)\n(?:.*\n)*?\s*\.amdhsa_private_segment_fixed_size (\d+)", asm)
    assert [k for k, v in scratch if int(v) != 0] == []
    assert [(name[:80], n) for name, body in ks for n in [waterfall_loops(body)] if n] == []
