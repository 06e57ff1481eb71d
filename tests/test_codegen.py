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
loads), and for the 128x512 tile (before its loop, once for the first
chunk's scale loads into registers).  The persistent walk of a
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
    asm = asm_path.read_text()
    for name, n in gemm.items():
        tile = re.search(r"TileILi(\d+)ELi(\d+)ELi(\d+)ELi(\d+)ELi(\d+)E", name)
        assert tile, name
        two_stage = tile.group(5) == "2"
        allowed = 2 if two_stage or "persistent" in name or "gemm_silu_kernel" in name else 1
        # with 8 or more waves the K loop is written twice (copying waves 0-3
        # and the others), each copy with its own drains
        waves = int(tile.group(3)) * int(tile.group(4))
        if waves >= 8 and (two_stage or "persistent" in name):
            allowed += 1
        # the 128x512 tile keeps its scales in registers: before one copy of
        # its loop the compiler waits for the first chunk's scale loads, which
        # the first chunk-top wait of the loop waits for anyway
        if tile.group(1, 2) == ("128", "512"):
            allowed += 1
        assert n <= allowed, f"{name}: {n} full vmcnt drains"
        loops = mfma_loop_drains(asm, name)
        assert loops and max(loops) <= (1 if two_stage or "persistent" in name else 0), (name, loops)


def mfma_loop_drains(asm: str, kernel_prefix: str) -> list[int]:
    """Full drains inside each loop that contains MFMAs, for the kernels
    whose symbol starts with kernel_prefix.  A loop is its header block (the
    label the compiler marks "Loop Header") and every block it annotates as
    "in Loop: Header=<that block>" (the compiler may place them before the
    header)."""
    out = []
    cur = None
    blocks: list[tuple[str, list[str]]] = []
    for line in asm.splitlines() + ["_Zend:"]:
        m = re.match(r"^(_Z\S+):", line)
        if m:
            if cur is not None and cur.startswith(kernel_prefix):
                headers = [lab for lab, body in blocks if body and "Loop Header" in body[0]]
                for h in headers:
                    key = h.lstrip(".L")  # BB0_11
                    loop = [l for lab, body in blocks
                            if lab == h or (body and f"in Loop: Header={key}" in body[0]) for l in body]
                    if any("v_mfma" in l for l in loop):
                        out.append(sum("s_waitcnt vmcnt(0)" in l for l in loop))
            cur, blocks = m.group(1), [("", [])]
            continue
        b = re.match(r"^(\.LBB\w+):|^; %(bb\.\w+):", line)
        if b:
            blocks.append((b.group(1) or b.group(2), [line]))
        elif blocks:
            blocks[-1][1].append(line)
    return out


@pytest.mark.skipif(shutil.which("hipcc") is None and not os.path.exists("/opt/rocm/bin/hipcc"),
                    reason="HIP toolchain not installed")
def test_split_k_loop_has_one_full_drain(tmp_path):
    """The K-split kernel's K loops (the two-stage 256x256 tile, written once
    for the copying waves and once for the others) keep their one full drain
    per chunk; the waits of its partial-sum exchange come after the loops."""
    asm_path = tmp_path / "gemm.s"
    cmd = [fgbuild.hipcc(), *[a for a in fgbuild.COMMON if a != "-fPIC"], "--cuda-device-only", "-S", GEMM_SRC,
           "-o", str(asm_path)]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-2000:]
    loops = mfma_loop_drains(asm_path.read_text(), "_ZN5fgfp821gemm_nt_splitk_kernel")
    assert loops == [1, 1], loops  # the loop of the copying waves and that of the others
