"""GPU parity of the UE8M0 recipe: quantize_fp8_groups_ue8m0 /
quantize_fp8_blocks_ue8m0 bit-exact against the oracle's power-of-two
quantizers, and fp8_gemm_nt_ue8m0 (scales applied by the matrix cores,
accumulation across chunks inside the MFMA) against the oracle product on the
same quantized operands, for every tile configuration and decode shapes."""

import numpy as np
import pytest
import torch

import fine_grained_block_fp8_amd as fg
import oracle
import workloads
from tests.parity import bits32, check_gemm, check_sampled, codes, d_to_f64, magnitude_sum, sample_col_blocks, sample_rows, to_dev_bf16

pytestmark = pytest.mark.gpu

TILES = ["tile256x256_w4x2", "tile256x192_w4x3", "tile256x128_w4x2", "tile128x256_w2x4", "tile128x128_w2x2"]


def ue8m0_path(lin):
    x, w = to_dev_bf16(lin.a), to_dev_bf16(lin.b)
    q, sa = fg.quantize_fp8_groups(x, ue8m0=True)
    qb, sb = fg.quantize_fp8_blocks(w, ue8m0=True)
    d = torch.full((lin.m, lin.n), float("nan"), dtype=torch.bfloat16, device="cuda")
    fg.fp8_gemm_nt((q, sa), (qb, sb), d, ue8m0=True)
    torch.cuda.synchronize()
    return q, sa, qb, sb, d


def check_all(lin, q, sa, qb, sb, d, label):
    oq, osa = oracle.quantize_groups_ue8m0(lin.a)
    oqb, osb = oracle.quantize_blocks_ue8m0(lin.b)
    assert np.array_equal(codes(q), oq), f"{label}: activation codes"
    assert np.array_equal(bits32(sa[:, : lin.m]), bits32(osa[:, : lin.m])), f"{label}: activation scales"
    assert np.array_equal(codes(qb), oqb), f"{label}: weight codes"
    assert np.array_equal(bits32(sb), bits32(osb)), f"{label}: weight scales"
    ref = oracle.gemm_nt(oq, osa, oqb, osb)
    return check_gemm(d_to_f64(d), ref, magnitude_sum(oq, osa, oqb, osb), lin.k, label)


@pytest.mark.parametrize("tile", TILES)
@pytest.mark.parametrize("m,n,k", [(17, 136, 128), (129, 1000, 384), (300, 520, 768)])
def test_ue8m0_every_tile(tile, m, n, k, monkeypatch):
    monkeypatch.setenv("FGFP8_GEMM_TILE", tile)
    lin = workloads.random_linear(m, n, k, seed=m * 3 + n + k)
    check_all(lin, *ue8m0_path(lin), f"ue8m0 {tile} {m}x{n}x{k}")


@pytest.mark.parametrize("m", [1, 4, 16])
def test_ue8m0_decode_shapes(m):
    lin = workloads.decode_linear(m, 4096, 12288)
    q, sa, qb, sb, d = ue8m0_path(lin)
    rng = np.random.default_rng(4)
    check_sampled(lin, q, sa, qb, sb, d, np.arange(m), sample_col_blocks(lin.n, 12, rng), f"ue8m0 decode m={m}",
                  quantizers=(oracle.quantize_groups_ue8m0, oracle.quantize_blocks_ue8m0))


def test_ue8m0_prefill_with_outliers_sampled():
    (lin,) = workloads.prefill_linears(names=["qkv"])
    q, sa, qb, sb, d = ue8m0_path(lin)
    rng = np.random.default_rng(5)
    check_sampled(lin, q, sa, qb, sb, d, sample_rows(lin.m, 32, rng), sample_col_blocks(lin.n, 8, rng), "ue8m0 qkv",
                  quantizers=(oracle.quantize_groups_ue8m0, oracle.quantize_blocks_ue8m0))


def test_promote_path_agrees_on_power_of_two_scales():
    """fp8_gemm_nt (FP32 promotion) on the same power-of-two operands: both
    products meet the criteria against the oracle, so they agree to FP32
    summation order."""
    lin = workloads.random_linear(256, 512, 1024, seed=61)
    q, sa, qb, sb, d = ue8m0_path(lin)
    d2 = torch.full_like(d, float("nan"))
    fg.fp8_gemm_nt((q, sa), (qb, sb), d2)
    torch.cuda.synchronize()
    oq, osa = oracle.quantize_groups_ue8m0(lin.a)
    oqb, osb = oracle.quantize_blocks_ue8m0(lin.b)
    ref = oracle.gemm_nt(oq, osa, oqb, osb)
    s = magnitude_sum(oq, osa, oqb, osb)
    check_gemm(d_to_f64(d), ref, s, lin.k, "ue8m0 product")
    check_gemm(d_to_f64(d2), ref, s, lin.k, "promote product")
