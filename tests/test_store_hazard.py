"""gfx950 store-data hazard: no VALU write to a wide store's data registers within
two wait states after the store.

A 16-byte buffer store reads its data registers after issue; a VALU write to them
in the next instruction corrupted stored values (the guarded helper in
hc_kernels.hip keeps two wait states after its 16-byte stores). Every other wide
store relies on the compiler's schedule, so this test compiles the device code of
the library's sources to gfx950 assembly (hipcc -S, the library's own flags) and
scans every 8-, 12- and 16-byte vector store. Runs on the CPU (cross-compilation).
"""
import os
import re
import subprocess

import pytest

from hyper_connection_residual_mixes_amd import build as hip_build

STORE = re.compile(r"((?:global|buffer|flat)_store_dwordx[234])\s+(.*)")


def _regs(spec: str):
    m = re.match(r"v\[(\d+):(\d+)\]", spec)
    if m:
        return set(range(int(m.group(1)), int(m.group(2)) + 1))
    m = re.match(r"v(\d+)$", spec)
    return {int(m.group(1))} if m else set()


def hazards(asm: str):
    """(store, next instruction) pairs where a VALU instruction within two wait
    states of a wide store writes one of the store's data registers."""
    ins = [l.strip() for l in asm.split("\n")]
    ins = [l for l in ins if l and not l.startswith((";", ".")) and not re.match(r"^[\w.$]+:", l)]
    found, stores = [], 0
    for i, t in enumerate(ins):
        m = STORE.match(t)
        if not m:
            continue
        stores += 1
        ops = [o.strip() for o in m.group(2).split(",")]
        data = _regs(ops[0] if m.group(1).startswith("buffer") else ops[1])
        waits = 0
        for nt in ins[i + 1:i + 4]:
            if waits >= 2:
                break
            if nt.startswith("s_nop"):
                parts = nt.split()
                waits += (int(parts[1]) + 1) if len(parts) > 1 else 1
                continue
            mm = re.match(r"(v_\w+)\s+([^,\s]+)", nt)
            if mm and not nt.startswith("v_nop") and _regs(mm.group(2)) & data:
                found.append((t, nt))
            waits += 1
    return stores, found


def test_scanner_finds_a_planted_hazard():
    asm = "global_store_dwordx4 v2, v[4:7], s[0:1]\nv_mov_b32 v4, 0\n"
    assert hazards(asm) == (1, [("global_store_dwordx4 v2, v[4:7], s[0:1]", "v_mov_b32 v4, 0")])
    assert hazards("buffer_store_dwordx4 v[8:11], v1, s[4:7], 0 offen\ns_nop 1\nv_mov_b32 v8, 0\n")[1] == []


@pytest.mark.parametrize("src", ["hc_kernels.hip", "hc_generic.hip", "hc_noalloc.hip"])
def test_no_valu_write_after_wide_store(src, tmp_path):
    out = tmp_path / (src + ".s")
    cmd = [hip_build.hipcc(), *hip_build.HIP_FLAGS, "--cuda-device-only", "-S",
           "-I", os.path.join(hip_build.ROOT, "include"), "-I", hip_build.CSRC,
           os.path.join(hip_build.CSRC, src), "-o", str(out)]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-2000:]
    stores, found = hazards(out.read_text())
    assert found == [], found[:5]
    if src != "hc_noalloc.hip":
        assert stores > 0
