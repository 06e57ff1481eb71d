"""GPU parity of fp8_gemm_nt_fp8_out (product with FP8 output for the next
layer).  Its bytes and scales must equal, bit for bit, the GPU quantizer and
the oracle's quantize_groups applied to the call's own bf16 product, whose
values are checked against the oracle's FP64 result; above 16 rows they must
also equal the two-call path quantize_fp8_groups(fp8_gemm_nt(a, b)).  Every
tile configuration, ragged M, and M <= 16."""

import numpy as np
import pytest
import torch

import fine_grained_block_fp8_amd as fg
import oracle
import workloads
from tests.parity import bits32, check_full, check_sampled, codes, gpu_hot_path

pytestmark = pytest.mark.gpu

TILES = ["tile256x256_w4x2", "tile256x192_w4x3", "tile256x128_w4x2", "tile128x256_w2x4", "tile128x128_w2x2"]


def run_and_check(lin, label):
    q, sa, qb, sb, d = gpu_hot_path(lin)
    m, n = lin.m, lin.n
    q_out = torch.full((m, n), 0x7F, dtype=torch.uint8, device="cuda").view(torch.float8_e4m3fn)
    sd = torch.full((n // 128, fg.padded_rows(m)), float("nan"), dtype=torch.float32, device="cuda")
    d2 = torch.full((m, n), float("nan"), dtype=torch.bfloat16, device="cuda")
    fg.fp8_gemm_nt_fp8_out((q, sa), (qb, sb), out=(q_out, sd), d=d2)
    torch.cuda.synchronize()
    # q is the quantizer applied to this call's own bf16 product (the GPU
    # quantizer and the oracle's, bit for bit)
    q_ref, sd_ref = fg.quantize_fp8_groups(d2)
    torch.cuda.synchronize()
    assert torch.equal(q_out.view(torch.uint8), q_ref.view(torch.uint8)), f"{label}: FP8 output differs"
    assert np.array_equal(bits32(sd[:, :m]), bits32(sd_ref[:, :m])), f"{label}: output scales differ"
    d_bits = d2.view(torch.int16).cpu().numpy().view(np.uint16)
    oq, osd = oracle.quantize_groups(d_bits)
    assert np.array_equal(codes(q_out), oq), f"{label}: FP8 output differs from the oracle quantizer"
    assert np.array_equal(bits32(sd[:, :m]), bits32(osd[:, :m]))
    # above 16 rows fp8_gemm_nt runs the same tile kernel: the two-call path is
    # the same bits (at most 16 rows it runs the decode kernel, whose K split
    # sums in another order)
    if m > 16:
        assert torch.equal(d2.view(torch.int16), d.view(torch.int16)), f"{label}: bf16 output differs from fp8_gemm_nt"
    d = d2
    # and the product itself against the oracle (sampled)
    rng = np.random.default_rng(3)
    rows = np.unique(np.concatenate([[0, m - 1], rng.integers(0, m, size=min(m, 16))]))
    check_sampled(lin, q, sa, qb, sb, d, rows, np.arange(n // 128), label)


@pytest.mark.parametrize("tile", TILES)
@pytest.mark.parametrize("m,n,k", [(300, 512, 384), (129, 256, 256), (17, 384, 640)])
def test_fp8_out_every_tile(tile, m, n, k, monkeypatch):
    monkeypatch.setenv("FGFP8_GEMM_TILE", tile)
    run_and_check(workloads.random_linear(m, n, k, seed=m + n + k), f"{tile} {m}x{n}x{k}")


@pytest.mark.parametrize("m", [1, 4, 16])
def test_fp8_out_small_m(m):
    run_and_check(workloads.random_linear(m, 1024, 512, seed=m), f"m={m}")


def test_fp8_out_prefill_o():
    """The o projection's output shape (2048 x 4096) with outlier activations:
    the FP8 output equals the oracle's quantizer applied to the call's own
    bf16 product (and the GPU quantizer's, bit for bit), and every output of
    that product meets the product criteria against the oracle."""
    (lin,) = workloads.prefill_linears(names=["o"])
    q, sa, qb, sb, d = gpu_hot_path(lin)
    m, n = lin.m, lin.n
    q_out = torch.full((m, n), 0x7F, dtype=torch.uint8, device="cuda").view(torch.float8_e4m3fn)
    sd = torch.full((n // 128, fg.padded_rows(m)), float("nan"), dtype=torch.float32, device="cuda")
    d2 = torch.full((m, n), float("nan"), dtype=torch.bfloat16, device="cuda")
    fg.fp8_gemm_nt_fp8_out((q, sa), (qb, sb), out=(q_out, sd), d=d2)
    q_ref, sd_ref = fg.quantize_fp8_groups(d2)
    torch.cuda.synchronize()
    assert torch.equal(q_out.view(torch.uint8), q_ref.view(torch.uint8))
    assert np.array_equal(bits32(sd[:, :m]), bits32(sd_ref[:, :m]))
    oq, osd = oracle.quantize_groups(d2.view(torch.int16).cpu().numpy().view(np.uint16))
    assert np.array_equal(codes(q_out), oq), "FP8 output differs from the oracle quantizer"
    assert np.array_equal(bits32(sd[:, :m]), bits32(osd[:, :m])), "output scales differ from the oracle's"
    assert torch.equal(d2.view(torch.int16), d.view(torch.int16)), "bf16 output differs from fp8_gemm_nt"
    check_full(lin, q, sa, qb, sb, d2, "fp8-out o")
