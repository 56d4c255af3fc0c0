"""The MFMA-rate ceiling measures MFMAs only.

bench_ceilings.hip's MFMA loop must compile to back-to-back
v_mfma_f32_16x16x32_bf16 with nothing but the loop's scalar count between them:
register moves of the accumulators inside the loop wait on each result and
halve the rate it reports. Compiles the file to gfx950 assembly with the
flags the benchmark's build uses; runs on the CPU.
"""
import os
import re
import subprocess

from hyper_connection_residual_mixes_amd import build as hip_build


def _mfma_loop(asm: str):
    """The instructions of the innermost loop of mfma_kernel."""
    start = asm.index("_Z11mfma_kernelPfi:")
    body = asm[start:asm.index("s_endpgm", start)].split("\n")
    ins = [l.split(";")[0].strip() for l in body]
    loops = [i for i, l in enumerate(body) if "Inner Loop Header" in l]
    assert len(loops) == 1, "expected one loop in mfma_kernel"
    head = body[loops[0]].split(":")[0].strip()
    end = next(i for i in range(loops[0], len(ins)) if re.match(r"s_cbranch_\w+\s+" + re.escape(head) + r"$", ins[i]))
    return [l for l in ins[loops[0] + 1:end + 1] if l]


def test_mfma_loop_has_no_register_moves(tmp_path):
    out = tmp_path / "bench_ceilings.s"
    cmd = [hip_build.hipcc(), *hip_build.HIP_FLAGS, *hip_build.CEILINGS_FLAGS, "--cuda-device-only", "-S",
           os.path.join(hip_build.ROOT, "bench_ceilings.hip"), "-o", str(out)]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-2000:]
    loop = _mfma_loop(out.read_text())
    mfma = [l for l in loop if l.startswith("v_mfma_f32_16x16x32_bf16")]
    assert len(mfma) == 8, loop
    other_vector = [l for l in loop if l.startswith("v_") and not l.startswith("v_mfma")]
    assert other_vector == [], other_vector
    # eight distinct accumulators, each its own source and destination
    dst = [re.match(r"v_mfma_\w+\s+(v\[\d+:\d+\]),.*,\s*(v\[\d+:\d+\])$", l) for l in mfma]
    assert all(m and m.group(1) == m.group(2) for m in dst), mfma
    assert len({m.group(1) for m in dst}) == 8
