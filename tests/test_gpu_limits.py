"""GPU parity at the largest K the library accepts (2^24 - 128): the 256-row
tile's copy range is then 256 * K = 2^32 - 32768 bytes, the edge of the
32-bit buffer-resource offsets every copy uses; the decode kernels split
131071 chunks over their waves.  The operands are drawn on the device
(workloads.device_fp8_operand) and the oracle computes sampled outputs from
the sampled rows, copied back.  The activation quantizer is checked
bit-exact at that K on a few rows."""

import numpy as np
import pytest
import torch

import fine_grained_block_fp8_amd as fg
import oracle
import workloads
from tests.parity import bits32, check_gemm, codes, d_to_f64, magnitude_sum, to_dev_bf16

pytestmark = pytest.mark.gpu

K_MAX = (1 << 24) - 128
KB = K_MAX // 128


def operands(m, n, seed):
    qa, sa = workloads.device_fp8_operand(m, K_MAX, seed, (KB, fg.padded_rows(m)))
    qb, sb = workloads.device_fp8_operand(n, K_MAX, seed + 1, (-(-n // 128), KB))
    return qa, sa, qb, sb


def check_sampled_outputs(qa, sa, qb, sb, d, rows, cols, label, normwise=True):
    """Sampled outputs against the oracle, the samples pooled into one
    check: the normwise criterion is a whole-matrix statistic (a perfect bf16
    rounding alone scores ~1.6e-3), so it needs a few hundred elements.  The
    magnitude sum S is additive over K and taken slice by slice to bound host
    memory."""
    ri = torch.as_tensor(rows, device="cuda")
    oqa, osa = codes(qa.index_select(0, ri)), sa.index_select(1, ri).cpu().numpy()
    osb_all = sb.cpu().numpy()
    got_all, ref_all, s_all = [], [], []
    for blk in sorted(set(c // 128 for c in cols)):
        cs = [c for c in cols if c // 128 == blk]
        oqb = codes(qb.index_select(0, torch.as_tensor(cs, device="cuda")))
        osb = osb_all[blk : blk + 1]
        ref_all.append(oracle.gemm_nt(oqa, osa, oqb, osb))
        got_all.append(d_to_f64(d.index_select(0, ri).index_select(1, torch.as_tensor(cs, device="cuda"))))
        step = 1 << 20
        s_all.append(sum(magnitude_sum(oqa[:, k0 : k0 + step], osa[k0 // 128 : (k0 + step) // 128],
                                       oqb[:, k0 : k0 + step], osb[:, k0 // 128 : (k0 + step) // 128])
                         for k0 in range(0, K_MAX, step)))
    got, ref, s = (np.concatenate([x.reshape(-1) for x in xs])[None, :] for xs in (got_all, ref_all, s_all))
    if normwise:
        assert got.size >= 256
        check_gemm(got, ref, s, K_MAX, label)
    else:  # too few samples for the normwise statistic: the elementwise bound alone
        assert np.all(np.isfinite(got))
        assert np.all(np.abs(got - ref) <= 2.0**-8 * np.abs(ref) + 2.0 * (K_MAX + KB) * 2.0**-24 * s), label


@pytest.mark.parametrize("tile", ["tile256x256_w4x2", "tile128x128_w2x2"])
def test_largest_k_tile_path(tile, monkeypatch):
    monkeypatch.setenv("FGFP8_GEMM_TILE", tile)
    m = n = 256
    qa, sa, qb, sb = operands(m, n, seed=31)
    d = torch.full((m, n), float("nan"), dtype=torch.bfloat16, device="cuda")
    fg.fp8_gemm_nt((qa, sa), (qb, sb), d)
    torch.cuda.synchronize()
    assert torch.isfinite(d.float()).all()
    cols = list(range(0, 128, 4)) + list(range(131, 256, 4))
    check_sampled_outputs(qa, sa, qb, sb, d, [0, 77, 129, 255], cols, f"K max {tile}")


@pytest.mark.parametrize("m", [1, 8, 16])
def test_largest_k_decode_path(m):
    n = 32
    qa, sa, qb, sb = operands(m, n, seed=37 + m)
    d = torch.full((m, n), float("nan"), dtype=torch.bfloat16, device="cuda")
    fg.fp8_gemm_nt((qa, sa), (qb, sb), d)
    torch.cuda.synchronize()
    assert torch.isfinite(d.float()).all()
    check_sampled_outputs(qa, sa, qb, sb, d, list(range(m)), list(range(n)), f"K max decode m={m}", normwise=m > 1)


def test_largest_k_quantizer_and_fused_linear():
    rng = np.random.default_rng(41)
    x = workloads.activation_bf16(rng, 2, K_MAX, outliers=True)
    xd = to_dev_bf16(x)
    q, sa = fg.quantize_fp8_groups(xd)
    oq, osa = oracle.quantize_groups(x)
    assert np.array_equal(codes(q), oq)
    assert np.array_equal(bits32(sa)[:, :2], bits32(osa[:, :2]))
    # the fused linear (activation quantized inside the product kernel) gives
    # the bits of the two calls
    qb, sb = workloads.device_fp8_operand(16, K_MAX, 43, (1, KB))
    d1 = torch.empty((2, 16), dtype=torch.bfloat16, device="cuda")
    fg.fp8_gemm_nt((q, sa), (qb, sb), d1)
    d2 = fg.fp8_linear(xd, (qb, sb))
    torch.cuda.synchronize()
    assert torch.equal(d1.view(torch.int16), d2.view(torch.int16))
