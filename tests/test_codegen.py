"""Code-generation guard for the GEMM kernels (host-only: hipcc cross-compiles
gfx950 assembly without a GPU).

The K pipeline stages operand tiles with global->LDS copies and orders them
before the LDS reads with its own partial waits (vmcnt(N)) and one barrier
per K block.  If the compiler cannot tell the LDS reads apart from the
in-flight copies, it inserts a full drain (s_waitcnt vmcnt(0)) before the
reads in every K block, which serialises the pipeline (a 1.5x slowdown of the
grouped MoE product was traced to exactly this).  This test counts the full
drains per kernel: one after the loop for the three-stage tiles, and one more
for the two-stage tiles (256x256, 256x192: their wait at the top of each
chunk is a full drain by design, since their copies are one chunk ahead) and
for the fused gate_up kernel (its epilogue waits once for its m_indices
loads).  The persistent walk of a
three-stage tile adds one drain, taken once per tile before its stores leave
the counter.
"""

import os
import re
import shutil
import subprocess

import pytest

from fine_grained_block_fp8_amd import build as fgbuild

GEMM_SRC = os.path.join(fgbuild.CSRC, "gemm.hip")


def kernel_drains(asm: str) -> dict[str, int]:
    out: dict[str, int] = {}
    cur = None
    for line in asm.splitlines():
        m = re.match(r"^(_Z\S+):", line)
        if m:
            cur = m.group(1)
            out[cur] = 0
            continue
        if cur is not None and "s_waitcnt vmcnt(0)" in line:
            out[cur] += 1
    return out


@pytest.mark.skipif(shutil.which("hipcc") is None and not os.path.exists("/opt/rocm/bin/hipcc"),
                    reason="HIP toolchain not installed")
def test_gemm_loops_have_no_full_drain(tmp_path):
    asm_path = tmp_path / "gemm.s"
    cmd = [fgbuild.hipcc(), *[a for a in fgbuild.COMMON if a != "-fPIC"], "--cuda-device-only", "-S", GEMM_SRC,
           "-o", str(asm_path)]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-2000:]
    drains = kernel_drains(asm_path.read_text())
    gemm = {k: v for k, v in drains.items()
            if "gemm_nt_kernel" in k or "gemm_nt_persistent_kernel" in k or "gemm_silu_kernel" in k}
    assert len(gemm) >= 15 and any("gemm_silu_kernel" in k for k in gemm), sorted(drains)
    for name, n in gemm.items():
        tile = re.search(r"TileILi(\d+)ELi(\d+)ELi(\d+)ELi(\d+)ELi(\d+)E", name)
        assert tile, name
        two_stage = tile.group(5) == "2"
        allowed = 2 if two_stage or "persistent" in name or "gemm_silu_kernel" in name else 1
        assert n <= allowed, f"{name}: {n} full vmcnt drains"
