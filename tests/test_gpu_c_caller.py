"""The C ABI from C: a program with no Python or PyTorch in its process
(tests/c_caller/c_caller.c, built here with gcc against include/fgfp8.h,
libfgfp8.so and the HIP runtime) quantizes, multiplies and runs the fused
decode linear; its outputs meet the oracle (bytes and scales bit-exact,
products within the product criteria)."""

import os
import shutil
import subprocess

import numpy as np
import pytest

import fine_grained_block_fp8_amd as fg
import oracle
import workloads
from tests.parity import check_gemm, magnitude_sum

pytestmark = pytest.mark.gpu

HERE = os.path.dirname(os.path.abspath(__file__))
ROCM = os.environ.get("ROCM_PATH", "/opt/rocm")


def build_c_caller(tmp_path) -> str:
    cc = shutil.which("gcc") or shutil.which("cc")
    if cc is None:
        pytest.skip("no C compiler")
    exe = str(tmp_path / "c_caller")
    lib_dir = os.path.dirname(fg.LIBRARY_PATH)
    cmd = [cc, "-std=c11", "-O2", "-Wall", "-Werror", "-I", os.path.dirname(fg.HEADER_PATH), "-I",
           os.path.join(ROCM, "include"), os.path.join(HERE, "c_caller", "c_caller.c"), "-o", exe, "-L", lib_dir,
           "-lfgfp8", "-L", os.path.join(ROCM, "lib"), "-lamdhip64", f"-Wl,-rpath,{lib_dir}",
           f"-Wl,-rpath,{os.path.join(ROCM, 'lib')}"]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr
    return exe


def test_c_program_through_the_abi(tmp_path):
    exe = build_c_caller(tmp_path)
    m, n, k = 300, 520, 768
    lin = workloads.random_linear(m, n, k, seed=77)
    (tmp_path / "a.bin").write_bytes(lin.a.tobytes())
    (tmp_path / "b.bin").write_bytes(lin.b.tobytes())
    out = str(tmp_path / "out")
    print(f"c_caller {m}x{n}x{k}", flush=True)
    r = subprocess.run([exe, str(tmp_path / "a.bin"), str(tmp_path / "b.bin"), str(m), str(n), str(k), out],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 0, r.stdout + r.stderr
    assert "c_caller ok" in r.stdout

    def load(name, dtype, shape):
        return np.fromfile(f"{out}.{name}.bin", dtype=dtype).reshape(shape)

    sa_ld = -(-m // 4) * 4
    q = load("q", np.uint8, (m, k))
    sa = load("sa", np.float32, (k // 128, sa_ld))
    qb = load("qb", np.uint8, (n, k))
    sb = load("sb", np.float32, (-(-n // 128), k // 128))
    d = workloads.bf16_bits_to_f32(load("d", np.uint16, (m, n))).astype(np.float64)
    d1 = workloads.bf16_bits_to_f32(load("d1", np.uint16, (1, n))).astype(np.float64)

    oq, osa = oracle.quantize_groups(lin.a)
    oqb, osb = oracle.quantize_blocks(lin.b)
    assert np.array_equal(q, oq)
    assert np.array_equal(sa[:, :m].view(np.uint32), osa[:, :m].view(np.uint32))
    assert np.array_equal(qb, oqb)
    assert np.array_equal(sb.view(np.uint32), osb.view(np.uint32))
    check_gemm(d, oracle.gemm_nt(oq, osa, oqb, osb), magnitude_sum(oq, osa, oqb, osb), k, "C caller product")
    check_gemm(d1, oracle.gemm_nt(oq[:1], osa[:, :1], oqb, osb), magnitude_sum(oq[:1], osa[:, :1], oqb, osb), k,
               "C caller fused decode")
