"""GPU parity of the MXFP8 recipe (quantize_fp8_mx, fp8_gemm_nt_mx) against
the oracle: quantized bytes and packed E8M0 scale words bit-exact; products
within the product criteria (the FP64 oracle, normwise 2e-3 and the
elementwise FP32-order bound), at every tile configuration, at decode shapes
and sampled at a prefill shape; and, where the MX scales are uniform over
each 128x128 block, bit-identical to the gran-128 UE8M0 product (the same
MFMAs with the same scale operands)."""

import numpy as np
import pytest
import torch

import fine_grained_block_fp8_amd as fg
import oracle
import workloads
from tests.parity import check_gemm, codes, d_to_f64, sample_col_blocks, sample_rows, to_dev_bf16, to_dev_u8_fp8

pytestmark = pytest.mark.gpu

TILES = ["tile256x256_w4x2", "tile256x192_w4x3", "tile256x128_w4x2", "tile128x256_w2x4", "tile128x128_w2x2"]


def mag_sum_mx(qa, sa, qb, sb):
    """S[m, n] = sum_k |dequant(a)[m, k] * dequant(b)[n, k]| (FP64)."""
    t = np.abs(oracle.e4m3_table())
    m, n = qa.shape[0], qb.shape[0]
    da = t[qa] * np.exp2(np.repeat(oracle.unpack_mx_scales(sa, m) - 127, 32, axis=1))
    db = t[qb] * np.exp2(np.repeat(oracle.unpack_mx_scales(sb, n) - 127, 32, axis=1))
    return da @ db.T


def gpu_mx(lin, sa_ld=None):
    x, w = to_dev_bf16(lin.a), to_dev_bf16(lin.b)
    q, sa = fg.quantize_fp8_mx(x, s_ld=sa_ld)
    qb, sb = fg.quantize_fp8_mx(w)
    d = torch.full((lin.m, lin.n), float("nan"), dtype=torch.bfloat16, device="cuda")
    fg.fp8_gemm_nt_mx((q, sa), (qb, sb), d)
    torch.cuda.synchronize()
    return q, sa, qb, sb, d


def ints(t):
    return t.cpu().numpy()


@pytest.mark.parametrize("m,k", [(1, 128), (5, 256), (300, 768), (2048, 4096), (129, 12288)])
def test_quantize_mx_bit_exact(m, k):
    x = workloads.activation_bf16(np.random.default_rng(m + k), m, k, outliers=True)
    q, s = fg.quantize_fp8_mx(to_dev_bf16(x))
    oq, os_ = oracle.quantize_mx(x)
    assert np.array_equal(codes(q), oq)
    assert np.array_equal(ints(s)[:, :m], os_[:, :m])


def test_quantize_mx_weight_and_edge_values():
    rng = np.random.default_rng(2)
    w = workloads.gaussian_bf16(rng, (130, 512), 0.02)
    x = workloads.bf16_bits_to_f32(w).copy()
    x[0, :32] = 0.0  # zero block
    x[1, 32:64] = np.float32(2.0 ** -133)  # tiny block
    x[2, 64] = np.float32(-0.0)
    x[3, 96:128] = np.float32(3.0e38)  # largest scales
    w = workloads.f32_to_bf16_bits(x)
    q, s = fg.quantize_fp8_mx(to_dev_bf16(w))
    oq, os_ = oracle.quantize_mx(w)
    assert np.array_equal(codes(q), oq)
    assert np.array_equal(ints(s)[:, :130], os_[:, :130])


@pytest.mark.parametrize("tile", TILES)
@pytest.mark.parametrize("m,n,k", [(17, 136, 128), (300, 520, 768), (129, 1000, 384)])
def test_mx_product_every_tile(tile, m, n, k, monkeypatch):
    monkeypatch.setenv("FGFP8_GEMM_TILE", tile)
    lin = workloads.random_linear(m, n, k, seed=m + 7 * n + k)
    q, sa, qb, sb, d = gpu_mx(lin)
    oq, osa = oracle.quantize_mx(lin.a)
    oqb, osb = oracle.quantize_mx(lin.b)
    assert np.array_equal(codes(q), oq) and np.array_equal(codes(qb), oqb)
    ref = oracle.gemm_nt_mx(oq, osa, oqb, osb)
    check_gemm(d_to_f64(d), ref, mag_sum_mx(oq, osa, oqb, osb), k, f"mx {tile} {m}x{n}x{k}")


@pytest.mark.parametrize("m", [1, 4, 16])
def test_mx_product_decode_shapes(m):
    lin = workloads.decode_linear(m, 4096, 1024)
    q, sa, qb, sb, d = gpu_mx(lin)
    oq, osa = oracle.quantize_mx(lin.a)
    oqb, osb = oracle.quantize_mx(lin.b)
    check_gemm(d_to_f64(d), oracle.gemm_nt_mx(oq, osa, oqb, osb), mag_sum_mx(oq, osa, oqb, osb), lin.k, f"mx m={m}")


def test_mx_prefill_gate_up_sampled():
    (lin,) = workloads.prefill_linears(names=["gate_up"])
    q, sa, qb, sb, d = gpu_mx(lin)
    rng = np.random.default_rng(8)
    rows = sample_rows(lin.m, 16, rng)
    cols = np.concatenate([np.arange(c * 128, c * 128 + 128) for c in sample_col_blocks(lin.n, 4, rng)])
    oq, osa = oracle.quantize_mx(lin.a[rows])
    oqb, osb = oracle.quantize_mx(lin.b[cols])
    ri, ci = torch.as_tensor(rows, device="cuda"), torch.as_tensor(cols, device="cuda")
    assert np.array_equal(codes(q.view(torch.uint8).index_select(0, ri)), oq)
    assert np.array_equal(ints(sa.index_select(1, ri)), osa[:, : rows.size])
    got = d_to_f64(d.index_select(0, ri).index_select(1, ci))
    check_gemm(got, oracle.gemm_nt_mx(oq, osa, oqb, osb), mag_sum_mx(oq, osa, oqb, osb), lin.k, "mx gate_up")


def test_uniform_block_scales_equal_gran128_ue8m0_bitwise():
    """Activation groups whose four 32-blocks share the amax, and weight
    scales spread from 128x128 blocks: the MX product and the UE8M0 product
    run the same MFMAs with the same scale bytes."""
    rng = np.random.default_rng(12)
    m, n, k = 300, 384, 512
    x = rng.uniform(-1, 1, size=(m, k)).astype(np.float32)
    x[:, ::32] = np.float32(2.5)
    a = workloads.f32_to_bf16_bits(x)
    w = workloads.gaussian_bf16(rng, (n, k), 0.02)
    qa8, sa8 = fg.quantize_fp8_groups(to_dev_bf16(a), ue8m0=True)
    qb8, sb8 = fg.quantize_fp8_blocks(to_dev_bf16(w), ue8m0=True)
    d8 = torch.empty((m, n), dtype=torch.bfloat16, device="cuda")
    fg.fp8_gemm_nt((qa8, sa8), (qb8, sb8), d8, ue8m0=True)
    qam, sam = fg.quantize_fp8_mx(to_dev_bf16(a))
    torch.cuda.synchronize()
    assert torch.equal(qam.view(torch.uint8), qa8.view(torch.uint8))
    # weight scale words from the oracle's 128x128 UE8M0 block scales, one word per column and chunk
    _, osb = oracle.quantize_blocks_ue8m0(w)
    c = oracle.quantize.e8m0_code(osb)[np.arange(n) // 128]  # [n][k/128]
    words = (c | (c << 8) | (c << 16) | (c << 24)).astype(np.uint32).view(np.int32).T.copy()  # [k/128][n]
    sbm = torch.from_numpy(words).cuda()
    dm = torch.empty((m, n), dtype=torch.bfloat16, device="cuda")
    fg.fp8_gemm_nt_mx((qam, sam), (to_dev_u8_fp8(codes(qb8)), sbm), dm)
    torch.cuda.synchronize()
    assert torch.equal(dm.view(torch.int16), d8.view(torch.int16))
