"""Host-side checks of the C ABI (no GPU needed, no compute calls).

* the library loads and exports every function include/fgfp8.h declares;
* the header is valid C and C++;
* argument validation returns FGFP8_EINVAL with a message, before any device
  is touched;
* without a usable GPU, well-formed calls return FGFP8_ENODEV instead of
  crashing (skipped where a GPU is present);
* the kernel plan chooser is a pure host function and is deterministic.
"""

import ctypes
import os
import shutil
import subprocess

import pytest
import torch

import fine_grained_block_fp8_amd as fg

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "fgfp8.h")
P = 0x10000  # a 16-byte aligned, never dereferenced pointer value


def test_library_exports_every_declared_function():
    names = fg.declared_functions()
    assert set(names) == {
        "quantize_fp8_groups",
        "quantize_fp8_blocks",
        "fp8_gemm_nt",
        "m_grouped_fp8_gemm_nt_contiguous",
        "fgfp8_last_error",
        "fgfp8_describe_gemm",
        "fgfp8_describe_grouped",
        "fgfp8_describe_linear",
        "fp8_linear_nt",
        "m_grouped_fp8_gemm_nt_masked",
        "fp8_gemm_nt_fp8_out",
        "quantize_fp8_groups_ue8m0",
        "quantize_fp8_blocks_ue8m0",
        "fp8_gemm_nt_ue8m0",
        "moe_max_padded_rows",
        "moe_route_workspace_bytes",
        "moe_route_contiguous",
        "moe_gather_quantize",
        "silu_mul_quantize",
        "moe_combine",
        "quantize_fp8_mx",
        "fp8_gemm_nt_mx",
        "moe_gate_up_silu_quantize",
        "quantize_fp8_groups_masked",
        "moe_gather_quantize_tokens",
        "moe_route_contiguous_noalloc",
        "moe_route_noalloc_max_workspace_bytes",
        "fp8_gemm_nt_ws",
        "fp8_gemm_nt_workspace_bytes",
        "m_grouped_fp8_gemm_nt_masked_ws",
        "m_grouped_fp8_gemm_nt_masked_workspace_bytes",
        "fgfp8_stream_read",
    }
    lib = fg.library()
    for n in names:
        assert hasattr(lib, n), n
    nm = shutil.which("nm")
    if nm:
        out = subprocess.run([nm, "-D", "--defined-only", fg.LIBRARY_PATH], capture_output=True, text=True).stdout
        exported = {line.split()[-1] for line in out.splitlines() if " T " in line}
        assert set(names) <= exported


@pytest.mark.parametrize("compiler,lang", [("gcc", "c"), ("g++", "c++")])
def test_header_compiles(compiler, lang, tmp_path):
    cc = shutil.which(compiler)
    if cc is None:
        pytest.skip(f"{compiler} not available")
    src = tmp_path / ("t.c" if lang == "c" else "t.cpp")
    src.write_text('#include "fgfp8.h"\nint main(void) { return fgfp8_last_error() == 0; }\n')
    r = subprocess.run([cc, "-fsyntax-only", "-Wall", "-Werror", "-x", lang, "-I", os.path.dirname(HEADER), str(src)],
                       capture_output=True, text=True)
    assert r.returncode == 0, r.stderr


def _lib():
    return fg.library()


@pytest.mark.parametrize(
    "args,needle",
    [
        ((P, 4, 100, P, P, 4, None), "multiple of 128"),
        ((P, 4, 0, P, P, 4, None), "multiple of 128"),
        ((P, 5, 128, P, P, 5, None), "sa_ld"),
        ((P, 5, 128, P, P, 4, None), "sa_ld"),
        ((None, 4, 128, P, P, 4, None), "null"),
        ((P + 8, 4, 128, P, P, 4, None), "aligned"),
        ((P, -1, 128, P, P, 4, None), "out of range"),
    ],
)
def test_quantize_groups_rejects(args, needle):
    rc = _lib().quantize_fp8_groups(*args)
    assert rc == fg.FGFP8_EINVAL
    assert needle in fg.last_error()


def test_ue8m0_calls_validate_like_the_fp32_ones():
    lib = _lib()
    assert lib.quantize_fp8_groups_ue8m0(P, 4, 100, P, P, 4, None) == fg.FGFP8_EINVAL
    assert "multiple of 128" in fg.last_error()
    assert lib.quantize_fp8_blocks_ue8m0(P, 10, 128, None, P, None) == fg.FGFP8_EINVAL
    assert lib.fp8_gemm_nt_ue8m0(P, P, 6, P, P, P, 8, 16, 256, None) == fg.FGFP8_EINVAL
    assert "fp8_gemm_nt_ue8m0" in fg.last_error()
    assert lib.fp8_gemm_nt_ue8m0(P, P, 8, P, P, P, 0, 16, 256, None) == fg.FGFP8_OK


def test_quantize_blocks_rejects():
    lib = _lib()
    assert lib.quantize_fp8_blocks(P, 10, 130, P, P, None) == fg.FGFP8_EINVAL
    assert lib.quantize_fp8_blocks(P, 10, 128, None, P, None) == fg.FGFP8_EINVAL
    assert lib.quantize_fp8_blocks(P, 10, 128, P, P + 4, None) == fg.FGFP8_EINVAL


def test_gemm_rejects():
    lib = _lib()
    ok = dict(a=P, sa=P, sa_ld=8, b=P, sb=P, d=P, m=8, n=16, k=256)

    def call(**kw):
        a = {**ok, **kw}
        return lib.fp8_gemm_nt(a["a"], a["sa"], a["sa_ld"], a["b"], a["sb"], a["d"], a["m"], a["n"], a["k"], None)

    assert call(k=200) == fg.FGFP8_EINVAL
    assert call(sa_ld=6) == fg.FGFP8_EINVAL
    assert call(sa_ld=4) == fg.FGFP8_EINVAL
    assert call(d=None) == fg.FGFP8_EINVAL
    assert call(b=P + 2) == fg.FGFP8_EINVAL
    assert call(n=-3) == fg.FGFP8_EINVAL
    assert call(k=1 << 25) == fg.FGFP8_EINVAL
    assert call(k=1 << 24) == fg.FGFP8_EINVAL  # 256 rows * K would wrap the 32-bit buffer size
    assert "exceeds" in fg.last_error()
    # empty problems are a valid no-op, even without a device
    assert call(m=0) == fg.FGFP8_OK
    assert call(n=0) == fg.FGFP8_OK


def test_grouped_rejects():
    lib = _lib()

    def call(m=256, g=4, n=128, k=256, sa_ld=256, idx=P):
        return lib.m_grouped_fp8_gemm_nt_contiguous(P, P, sa_ld, idx, P, P, g, P, m, n, k, None)

    assert call(m=200, sa_ld=200) == fg.FGFP8_EINVAL
    assert "multiple of 128" in fg.last_error()
    assert call(g=0) == fg.FGFP8_EINVAL
    assert call(idx=None) == fg.FGFP8_EINVAL
    assert call(k=64) == fg.FGFP8_EINVAL
    assert call(m=0, sa_ld=4) == fg.FGFP8_OK


def test_masked_rejects():
    lib = _lib()

    def call(g=4, max_m=64, n=128, k=256, sa_ld=256, mm=P, em=32):
        return lib.m_grouped_fp8_gemm_nt_masked(P, P, sa_ld, mm, P, P, g, max_m, em, P, n, k, None)

    assert call(max_m=62) == fg.FGFP8_EINVAL
    assert "multiple of 4" in fg.last_error()
    assert call(g=0) == fg.FGFP8_EINVAL
    assert call(sa_ld=252) == fg.FGFP8_EINVAL  # sa_ld < num_groups * max_m
    assert call(mm=None) == fg.FGFP8_EINVAL
    assert call(k=200) == fg.FGFP8_EINVAL
    assert call(max_m=0, sa_ld=4) == fg.FGFP8_OK
    assert call(n=0) == fg.FGFP8_OK


def test_masked_workspace_size_and_rejects():
    """m_grouped_fp8_gemm_nt_masked_ws: the workspace query (1 KB of counters
    and 256 slots of one 128 x 256 FP32 tile) and the checks that come before
    any device work."""
    lib = fg.library()
    want = 256 * 4 + 256 * 128 * 256 * 4
    assert lib.m_grouped_fp8_gemm_nt_masked_workspace_bytes(32, 128, 4096, 7168) == want
    assert fg.m_grouped_fp8_gemm_nt_masked_workspace_bytes(1, 4, 16, 128) == want
    assert lib.m_grouped_fp8_gemm_nt_masked_workspace_bytes(0, 128, 4096, 7168) == 0
    assert lib.m_grouped_fp8_gemm_nt_masked_workspace_bytes(4, 128, 4096, 100) == 0
    assert lib.m_grouped_fp8_gemm_nt_masked_workspace_bytes(4, -4, 4096, 256) == 0

    def call(ws=P, nbytes=want, g=4, max_m=64, k=256):
        return lib.m_grouped_fp8_gemm_nt_masked_ws(P, P, 256, P, P, P, g, max_m, 32, P, 128, k, ws, nbytes, None)

    assert call(ws=P + 16) == fg.FGFP8_EINVAL
    assert "256-byte" in fg.last_error()
    assert call(ws=None) == fg.FGFP8_EINVAL
    assert call(nbytes=-1) == fg.FGFP8_EINVAL
    assert call(max_m=62) == fg.FGFP8_EINVAL  # the masked call's own checks apply
    assert "m_grouped_fp8_gemm_nt_masked_ws" in fg.last_error()
    assert call(k=200) == fg.FGFP8_EINVAL
    assert call(max_m=0) == fg.FGFP8_OK


def test_masked_quantizer_rejects():
    lib = _lib()

    def call(g=4, max_m=64, k=256, sa_ld=256, mm=P, x=P):
        return lib.quantize_fp8_groups_masked(x, mm, g, max_m, k, P, P, sa_ld, None)

    assert call(max_m=62) == fg.FGFP8_EINVAL
    assert "quantize_fp8_groups_masked" in fg.last_error() and "multiple of 4" in fg.last_error()
    assert call(g=0) == fg.FGFP8_EINVAL
    assert call(sa_ld=252) == fg.FGFP8_EINVAL  # sa_ld < num_groups * max_m
    assert call(mm=None) == fg.FGFP8_EINVAL
    assert call(x=P + 4) == fg.FGFP8_EINVAL  # misaligned
    assert call(k=200) == fg.FGFP8_EINVAL
    assert call(max_m=0, sa_ld=4, mm=None, x=None) == fg.FGFP8_OK


def test_fp8_out_rejects():
    lib = _lib()

    def call(m=8, n=256, k=256, sa_ld=8, sd_ld=8, q=P, sd=P, d=None):
        return lib.fp8_gemm_nt_fp8_out(P, P, sa_ld, P, P, q, sd, sd_ld, d, m, n, k, None)

    assert call(n=200) == fg.FGFP8_EINVAL
    assert "multiple of 128" in fg.last_error()
    assert call(sd_ld=4) == fg.FGFP8_EINVAL
    assert call(q=None) == fg.FGFP8_EINVAL
    assert call(d=P + 4) == fg.FGFP8_EINVAL
    assert call(m=0) == fg.FGFP8_OK


def test_mx_calls_validate():
    lib = _lib()
    assert lib.quantize_fp8_mx(P, 4, 100, P, P, 4, None) == fg.FGFP8_EINVAL
    assert lib.quantize_fp8_mx(P, 5, 128, P, P, 5, None) == fg.FGFP8_EINVAL
    assert lib.quantize_fp8_mx(None, 0, 128, None, None, 0, None) == fg.FGFP8_OK
    assert lib.fp8_gemm_nt_mx(P, P, 8, P, P, 12, P, 8, 16, 256, None) == fg.FGFP8_EINVAL  # sb_ld % 4
    assert "sb_ld" in fg.last_error()
    assert lib.fp8_gemm_nt_mx(P, P, 8, P, P, 8, P, 8, 16, 256, None) == fg.FGFP8_EINVAL  # sb_ld < n
    assert lib.fp8_gemm_nt_mx(P, P, 8, P, P, 16, P, 8, 16, 200, None) == fg.FGFP8_EINVAL
    assert lib.fp8_gemm_nt_mx(None, None, 0, None, None, 16, None, 0, 16, 256, None) == fg.FGFP8_OK


def test_moe_sizes():
    lib = _lib()
    assert lib.moe_max_padded_rows(8192, 4, 32) == (8192 * 4 + 32 * 127 + 127) // 128 * 128
    assert lib.moe_max_padded_rows(0, 1, 1) == 128
    assert lib.moe_max_padded_rows(-1, 4, 32) == -1
    assert lib.moe_route_workspace_bytes(257, 32) == 2 * 32 * 4 + 32 * 4
    assert lib.moe_route_workspace_bytes(0, 3) == 12
    assert lib.moe_route_workspace_bytes(4, 0) == -1


def test_moe_calls_reject():
    lib = _lib()
    mpm = lib.moe_max_padded_rows(100, 4, 8)
    ws = lib.moe_route_workspace_bytes(100, 8)

    def route(tokens=100, topk=4, g=8, m_pad_max=mpm, wsb=ws, idx=P):
        return lib.moe_route_contiguous(idx, tokens, topk, g, P, P, P, P, m_pad_max, P, wsb, None)

    assert route(topk=9) == fg.FGFP8_EINVAL
    assert "topk" in fg.last_error()
    assert route(g=0) == fg.FGFP8_EINVAL
    assert route(g=4096) == fg.FGFP8_EINVAL
    assert route(m_pad_max=mpm - 128) == fg.FGFP8_EINVAL
    assert "m_pad_max" in fg.last_error()
    assert route(m_pad_max=mpm + 4) == fg.FGFP8_EINVAL
    assert route(wsb=ws - 4) == fg.FGFP8_EINVAL
    assert "workspace" in fg.last_error()
    assert route(idx=None) == fg.FGFP8_EINVAL

    assert lib.moe_gather_quantize(P, 10, 100, P, 256, P, P, 256, None) == fg.FGFP8_EINVAL
    assert lib.moe_gather_quantize(P, 10, 128, P, 256, P, P, 252, None) == fg.FGFP8_EINVAL
    assert lib.moe_gather_quantize(P, 10, 128, None, 256, P, P, 256, None) == fg.FGFP8_EINVAL
    assert lib.moe_gather_quantize(P, -1, 128, P, 256, P, P, 256, None) == fg.FGFP8_EINVAL
    assert lib.moe_gather_quantize(P, 10, 128, P, 0, P, P, 4, None) == fg.FGFP8_OK
    tok = lib.moe_gather_quantize_tokens
    assert tok(P, 10, 128, 0, P, P, 256, P, P, 256, None) == fg.FGFP8_EINVAL  # topk
    assert tok(P, 10, 128, 9, P, P, 256, P, P, 256, None) == fg.FGFP8_EINVAL
    assert tok(P, 10, 100, 4, P, P, 256, P, P, 256, None) == fg.FGFP8_EINVAL  # k
    assert tok(P, 10, 128, 4, P, P, 256, P, P, 252, None) == fg.FGFP8_EINVAL  # sa_ld
    assert tok(P, 10, 128, 4, None, P, 256, P, P, 256, None) == fg.FGFP8_EINVAL  # row_of
    assert tok(P, 10, 128, 4, P, None, 256, P, P, 256, None) == fg.FGFP8_EINVAL  # token_of_row
    assert tok(P, 10, 128, 4, P, P, 0, P, P, 4, None) == fg.FGFP8_OK
    assert lib.silu_mul_quantize(P, 256, 64, P, P, P, 256, None) == fg.FGFP8_EINVAL
    assert lib.silu_mul_quantize(P + 2, 256, 128, P, P, P, 256, None) == fg.FGFP8_EINVAL
    assert lib.silu_mul_quantize(P, 0, 128, P, P, P, 4, None) == fg.FGFP8_OK
    assert lib.moe_combine(P, 64, 100, P, P, 8, 4, P, None) == fg.FGFP8_EINVAL
    assert "multiple of 8" in fg.last_error()
    assert lib.moe_combine(P, 64, 128, P, P, 8, 0, P, None) == fg.FGFP8_EINVAL
    assert lib.moe_combine(P, 64, 128, None, P, 8, 4, P, None) == fg.FGFP8_EINVAL
    assert lib.moe_combine(P, -1, 128, P, P, 8, 4, P, None) == fg.FGFP8_EINVAL
    assert lib.moe_combine(P, 64, 128, P, P, 0, 4, P, None) == fg.FGFP8_OK


def test_empty_problems_accept_null_pointers():
    """An empty problem validates its sizes, then returns FGFP8_OK without
    looking at its (possibly null) pointers -- what an empty tensor passes."""
    lib = _lib()
    N = None
    assert lib.quantize_fp8_groups(N, 0, 256, N, N, 0, None) == fg.FGFP8_OK
    assert lib.quantize_fp8_groups_ue8m0(N, 0, 256, N, N, 0, None) == fg.FGFP8_OK
    assert lib.quantize_fp8_groups(N, 0, 200, N, N, 0, None) == fg.FGFP8_EINVAL  # sizes still checked
    assert lib.quantize_fp8_blocks(N, 0, 256, N, N, None) == fg.FGFP8_OK
    assert lib.fp8_gemm_nt(N, N, 0, N, N, N, 0, 16, 256, None) == fg.FGFP8_OK
    assert lib.fp8_gemm_nt(N, N, 8, N, N, N, 8, 0, 256, None) == fg.FGFP8_OK
    assert lib.fp8_gemm_nt_ue8m0(N, N, 0, N, N, N, 0, 16, 256, None) == fg.FGFP8_OK
    assert lib.m_grouped_fp8_gemm_nt_contiguous(N, N, 0, N, N, N, 4, N, 0, 128, 256, None) == fg.FGFP8_OK
    assert lib.m_grouped_fp8_gemm_nt_masked(N, N, 0, N, N, N, 4, 0, 0, N, 128, 256, None) == fg.FGFP8_OK
    assert lib.fp8_gemm_nt_fp8_out(N, N, 0, N, N, N, N, 0, N, 0, 256, 256, None) == fg.FGFP8_OK
    assert lib.fp8_linear_nt(N, 0, 256, N, N, 128, N, N, N, 0, None) == fg.FGFP8_OK
    assert lib.moe_gather_quantize(N, 0, 256, N, 0, N, N, 0, None) == fg.FGFP8_OK
    assert lib.silu_mul_quantize(N, 0, 128, N, N, N, 0, None) == fg.FGFP8_OK
    assert lib.moe_combine(N, 0, 128, N, N, 0, 4, N, None) == fg.FGFP8_OK


def test_linear_rejects():
    lib = _lib()

    def call(m=2, k=256, n=128, q=None, sa=None, sa_ld=0, x=P):
        return lib.fp8_linear_nt(x, m, k, P, P, n, P, q, sa, sa_ld, None)

    assert call(k=100) == fg.FGFP8_EINVAL
    assert call(m=17) == fg.FGFP8_EINVAL  # above 16 rows the workspace is required
    assert "workspace" in fg.last_error()
    assert call(q=P) == fg.FGFP8_EINVAL  # q without sa
    assert call(m=8, q=P, sa=P, sa_ld=6) == fg.FGFP8_EINVAL
    assert call(x=None) == fg.FGFP8_EINVAL
    assert call(m=0) == fg.FGFP8_OK


def test_python_binding_rejects_cpu_tensors():
    x = torch.zeros((4, 128), dtype=torch.bfloat16)
    with pytest.raises(ValueError):
        fg.quantize_fp8_groups(x)


@pytest.mark.skipif(torch.cuda.is_available(), reason="a GPU is present")
def test_no_device_is_reported_not_crashed():
    lib = _lib()
    assert lib.quantize_fp8_groups(P, 4, 128, P, P, 4, None) == fg.FGFP8_ENODEV
    assert "device" in fg.last_error()
    assert lib.fp8_gemm_nt(P, P, 8, P, P, P, 8, 16, 256, None) == fg.FGFP8_ENODEV
    assert lib.quantize_fp8_blocks(P, 16, 256, P, P, None) == fg.FGFP8_ENODEV
    assert lib.m_grouped_fp8_gemm_nt_contiguous(P, P, 128, P, P, P, 2, P, 128, 64, 128, None) == fg.FGFP8_ENODEV
    assert lib.fp8_linear_nt(P, 1, 256, P, P, 128, P, None, None, 0, None) == fg.FGFP8_ENODEV
    assert lib.m_grouped_fp8_gemm_nt_masked(P, P, 256, P, P, P, 4, 64, 32, P, 128, 256, None) == fg.FGFP8_ENODEV
    assert lib.m_grouped_fp8_gemm_nt_masked_ws(P, P, 256, P, P, P, 4, 64, 32, P, 128, 256, P, 1 << 26,
                                               None) == fg.FGFP8_ENODEV
    assert lib.quantize_fp8_groups_masked(P, P, 4, 64, 256, P, P, 256, None) == fg.FGFP8_ENODEV
    assert lib.fp8_gemm_nt_fp8_out(P, P, 8, P, P, P, P, 8, None, 8, 256, 256, None) == fg.FGFP8_ENODEV
    mpm, ws = lib.moe_max_padded_rows(100, 4, 8), lib.moe_route_workspace_bytes(100, 8)
    assert lib.moe_route_contiguous(P, 100, 4, 8, P, P, P, P, mpm, P, ws, None) == fg.FGFP8_ENODEV
    assert lib.moe_gather_quantize(P, 10, 128, P, 256, P, P, 256, None) == fg.FGFP8_ENODEV
    assert lib.moe_gather_quantize_tokens(P, 10, 128, 4, P, P, 256, P, P, 256, None) == fg.FGFP8_ENODEV
    assert lib.silu_mul_quantize(P, 256, 128, P, P, P, 256, None) == fg.FGFP8_ENODEV
    assert lib.moe_combine(P, 64, 128, P, P, 8, 4, P, None) == fg.FGFP8_ENODEV


def test_describe_grouped_plans(monkeypatch):
    """The grouped product's tile: 128x512 where it takes fewer rounds of the
    256 CUs per unit of work (the 32-expert MoE layout: 273 blocks x 8 such
    tiles against 16 of 128x256), 128x256 for narrow N, the override, and the
    shape checks."""
    assert fg.describe_grouped(34944, 4096, 7168) == "tile128x512_w2x4"
    assert fg.describe_grouped(34944, 7168, 2048) == "tile128x512_w2x4"
    assert fg.describe_grouped(34944, 14336, 1024) == "tile128x256_w2x4 persistent"  # short K: the walk
    assert fg.describe_grouped(256, 384, 512).startswith("tile128x256_w2x4")
    monkeypatch.setenv("FGFP8_GROUPED_TILE", "tile128x256_w2x4")
    assert fg.describe_grouped(34944, 4096, 7168) == "tile128x256_w2x4"
    monkeypatch.setenv("FGFP8_PERSISTENT", "1")
    assert fg.describe_grouped(34944, 4096, 7168) == "tile128x256_w2x4 persistent"
    monkeypatch.setenv("FGFP8_GROUPED_TILE", "tile128x512_w2x4")
    assert fg.describe_grouped(256, 384, 512) == "tile128x512_w2x4"  # the wide tile has no walk
    # its 512-row weight panel must stay within 32-bit buffer offsets, forced or not
    assert fg.describe_grouped(256, 4096, (1 << 23) - 128) == "tile128x512_w2x4"
    assert fg.describe_grouped(256, 4096, 1 << 23).startswith("tile128x256_w2x4")
    monkeypatch.delenv("FGFP8_GROUPED_TILE")
    assert fg.describe_grouped(34944, 4096, (1 << 24) - 128).startswith("tile128x256_w2x4")
    buf = ctypes.create_string_buffer(64)
    lib = fg.library()
    for m, n, k in [(100, 4096, 7168), (0, 4096, 7168), (256, 0, 128), (256, 128, 100)]:
        assert lib.fgfp8_describe_grouped(m, n, k, buf, 64) == fg.FGFP8_EINVAL, (m, n, k)
    assert lib.fgfp8_describe_grouped(256, 128, 128, None, 64) == fg.FGFP8_EINVAL


def test_describe_gemm_plans():
    assert fg.describe_gemm(1, 12288, 4096).startswith("decode")
    assert fg.describe_gemm(16, 4096, 12288).startswith("decode")
    assert fg.describe_gemm(8192, 8192, 8192).startswith("tile256x256")
    assert fg.describe_gemm(2048, 4096, 4096) == fg.describe_gemm(2048, 4096, 4096)
    # the calibrated planner: fewest rounds of tiles weighted by each tile's
    # measured rate (shapes where the fastest forced tile was the one named)
    for (m, n, k), tile in [((2048, 6144, 4096), "tile256x192_w4x3"), ((4096, 6144, 4096), "tile256x192_w4x3"),
                            ((2048, 12288, 4096), "tile256x192_w4x3"), ((2048, 24576, 4096), "tile256x256_w4x2"),
                            ((2048, 3072, 4096), "tile128x256_w2x4"), ((8192, 7168, 2048), "tile256x256_w4x2"),
                            ((512, 4096, 4096), "tile128x128_w2x2")]:
        assert fg.describe_gemm(m, n, k).split()[0] == tile, (m, n, k)
    buf = ctypes.create_string_buffer(4)
    assert _lib().fgfp8_describe_gemm(8192, 8192, 8192, buf, 4) == fg.FGFP8_OK
    assert len(buf.value) == 3  # truncated, NUL-terminated
    assert _lib().fgfp8_describe_gemm(8, 8, 100, buf, 4) == fg.FGFP8_EINVAL


def test_persistent_walk_plan(monkeypatch):
    """The persistent walk is the default for two or more rounds of 256x256
    tiles (host-only); FGFP8_PERSISTENT forces or forbids it."""
    monkeypatch.delenv("FGFP8_PERSISTENT", raising=False)
    monkeypatch.delenv("FGFP8_GEMM_TILE", raising=False)
    assert fg.describe_gemm(2048, 24576, 4096) == "tile256x256_w4x2 split=0 persistent"  # 768 tiles
    assert fg.describe_gemm(8192, 8192, 8192).endswith(" persistent")
    assert fg.describe_gemm(4096, 4096, 4096) == "tile256x256_w4x2 split=0"  # one round
    assert fg.describe_gemm(2048, 4096, 4096) == "tile128x256_w2x4 split=0"
    assert fg.describe_gemm(2048, 6144, 4096) == "tile256x192_w4x3 split=0"  # not whole 128-column blocks
    assert fg.describe_gemm(8192, 8192, 128) == "tile256x256_w4x2 split=0"  # one chunk: no walk
    monkeypatch.setenv("FGFP8_PERSISTENT", "0")
    assert fg.describe_gemm(2048, 24576, 4096) == "tile256x256_w4x2 split=0"
    monkeypatch.setenv("FGFP8_PERSISTENT", "1")
    assert fg.describe_gemm(4096, 4096, 4096) == "tile256x256_w4x2 split=0 persistent"
    assert fg.describe_gemm(2048, 4096, 4096) == "tile128x256_w2x4 split=0 persistent"


def test_decode_slab_plan(monkeypatch):
    """The m <= 16 product's plan (host-only): three slabs per workgroup
    (with a split of 8 waves) for m > 4 where K <= 16384, the split comes to
    8 and the three-slab workgroups still number at least the 256 CUs, else
    one; FGFP8_DECODE_SLABS forces it where the shape allows."""
    monkeypatch.delenv("FGFP8_DECODE_SLABS", raising=False)
    assert fg.describe_gemm(16, 12288, 4096) == "decode_splitk_slab16 split=8 slabs=3"
    assert fg.describe_gemm(5, 12288, 4096) == "decode_splitk_slab16 split=8 slabs=3"
    assert fg.describe_gemm(4, 12288, 4096) == "decode_splitk_slab16 split=4"
    assert fg.describe_gemm(1, 12288, 4096) == "decode_splitk_slab16 split=4"
    # fewer three-slab workgroups than CUs: one slab per workgroup
    assert fg.describe_gemm(16, 8192, 4096) == "decode_splitk_slab16 split=4"
    assert fg.describe_gemm(16, 2048, 4096) == "decode_splitk_slab16 split=8"
    # 256 slabs at K = 12288: sixteen waves per slab, no room for three slabs
    assert fg.describe_gemm(16, 4096, 12288) == "decode_splitk_slab16 split=16"
    # K past 16384: the fused form's activation and three slabs' sums exceed LDS
    assert "slabs" not in fg.describe_gemm(16, 12288, 32768)
    monkeypatch.setenv("FGFP8_DECODE_SLABS", "1")
    assert fg.describe_gemm(16, 12288, 4096) == "decode_splitk_slab16 split=4"
    monkeypatch.setenv("FGFP8_DECODE_SLABS", "3")
    assert fg.describe_gemm(1, 12288, 4096) == "decode_splitk_slab16 split=8 slabs=3"
    assert fg.describe_gemm(1, 1040, 4096) == "decode_splitk_slab16 split=8 slabs=3"


def test_describe_linear_paths(monkeypatch):
    """fp8_linear_nt's path (host-only): the LDS fused form up to 4 rows, the
    three-slab LDS form above that on wide weights while the quantize tasks
    per lane fit (8 with the activation outputs, 16 without), the register
    form without a workspace elsewhere, quantize + product with one."""
    for v in ("FGFP8_DECODE_SLABS", "FGFP8_DECODE_XQ"):
        monkeypatch.delenv(v, raising=False)
    d = fg.describe_linear
    assert d(1, 12288, 4096, False) == "fused act-quant + decode_splitk_slab16 split=4 slabs=1 form=lds4"
    assert d(4, 12288, 4096, True) == "fused act-quant + decode_splitk_slab16 split=4 slabs=1 form=lds4"
    assert d(8, 12288, 4096, True) == "fused act-quant + decode_splitk_slab16 split=8 slabs=3 form=lds16"
    assert d(16, 12288, 4096, False) == "fused act-quant + decode_splitk_slab16 split=8 slabs=3 form=lds16"
    assert d(16, 12288, 4096, True) == "quantize_fp8_groups + decode_splitk_slab16 split=8 slabs=3"
    assert d(16, 4096, 12288, False) == "fused act-quant + decode_splitk_slab16 split=16 slabs=1 form=registers"
    assert d(16, 4096, 12288, True) == "quantize_fp8_groups + decode_splitk_slab16 split=16"
    # too few slabs for three per workgroup on every CU
    assert d(16, 2048, 4096, False).endswith("slabs=1 form=registers")
    assert d(2048, 4096, 4096, True).startswith("quantize_fp8_groups + tile")
    buf = ctypes.create_string_buffer(64)
    assert _lib().fgfp8_describe_linear(2048, 4096, 4096, 0, buf, 64) == fg.FGFP8_EINVAL  # needs the workspace
    assert _lib().fgfp8_describe_linear(8, 8, 100, 1, buf, 64) == fg.FGFP8_EINVAL
    assert _lib().fgfp8_describe_linear(8, 8, 128, 1, None, 64) == fg.FGFP8_EINVAL
    monkeypatch.setenv("FGFP8_DECODE_XQ", "1")
    assert d(8, 12288, 4096, False).endswith("slabs=1 form=registers")
    assert d(4, 12288, 4096, True).endswith("form=registers")


def test_fused_gate_up_rejects():
    lib = _lib()

    def call(a=P, m_indices=P, q=P, m=256, inter=256, k=512, groups=4, sa_ld=256, sq_ld=256):
        return lib.moe_gate_up_silu_quantize(a, P, sa_ld, m_indices, P, P, groups, q, P, sq_ld, m, inter, k, None)

    assert call(m=200) == fg.FGFP8_EINVAL  # m is a multiple of the 128-row blocks
    assert call(inter=200) == fg.FGFP8_EINVAL
    assert call(k=100) == fg.FGFP8_EINVAL
    assert call(groups=0) == fg.FGFP8_EINVAL
    assert call(sq_ld=6) == fg.FGFP8_EINVAL
    assert call(sa_ld=128) == fg.FGFP8_EINVAL
    assert call(inter=(1 << 20), k=(1 << 11)) == fg.FGFP8_EINVAL  # (inter + 128) * k beyond 2^31
    assert "2^31" in fg.last_error()
    assert call(m_indices=None) == fg.FGFP8_EINVAL
    assert call(q=None) == fg.FGFP8_EINVAL
    assert call(m=0, a=None, m_indices=None, q=None, sa_ld=0, sq_ld=0) == fg.FGFP8_OK  # empty: nothing to do


def test_gemm_workspace_sizes_and_rejects():
    """fp8_gemm_nt_ws: the workspace query (K split where 256x256 tiles fill
    at most half the compute units and K has at least 64 chunks), and the
    argument checks that come before any device work."""
    lib = fg.library()
    tiles = 8 * 16  # 2048 x 4096 in 256x256 tiles
    assert lib.fp8_gemm_nt_workspace_bytes(2048, 4096, 12288) == (2 * tiles * 4 + 255) // 256 * 256 + tiles * 256 * 256 * 4
    assert lib.fp8_gemm_nt_workspace_bytes(2048, 4096, 4096) == 0  # too few chunks per half
    assert lib.fp8_gemm_nt_workspace_bytes(2048, 24576, 4096) == 0  # whole tiles fill the CUs
    assert lib.fp8_gemm_nt_workspace_bytes(16, 4096, 12288) == 0  # decode shapes
    assert lib.fp8_gemm_nt_workspace_bytes(2048, 4096, 100) == 0  # invalid K
    assert lib.fp8_gemm_nt_workspace_bytes(-1, 4096, 12288) == 0
    # a workspace that is not 256-byte aligned
    assert lib.fp8_gemm_nt_ws(P, P, 2048, P, P, P, 2048, 4096, 12288, P + 16, 1 << 26, None) == fg.FGFP8_EINVAL
    assert "256-byte" in fg.last_error()
    assert lib.fp8_gemm_nt_ws(P, P, 2048, P, P, P, 2048, 4096, 12288, P, -1, None) == fg.FGFP8_EINVAL
    # the fp8_gemm_nt checks apply
    assert lib.fp8_gemm_nt_ws(P, P, 2048, P, P, P, 2048, 4096, 100, P, 1 << 26, None) == fg.FGFP8_EINVAL
    assert lib.fp8_gemm_nt_ws(None, None, 0, None, None, None, 0, 4096, 12288, None, 0, None) == fg.FGFP8_OK
