"""GPU parity of m_grouped_fp8_gemm_nt_contiguous against the oracle."""

import numpy as np
import pytest
import torch

import fine_grained_block_fp8_amd as fg
import oracle
import workloads
from tests import oracle_workers
from tests.parity import (
    assert_stats,
    bits32,
    block_rows,
    check_gemm,
    codes,
    d_to_f64,
    magnitude_sum,
    one_row_per_band,
    to_dev_bf16,
)

pytestmark = pytest.mark.gpu


def gpu_grouped(g: workloads.Grouped):
    x = to_dev_bf16(g.a)
    q, sa = fg.quantize_fp8_groups(x)
    w = to_dev_bf16(g.b.reshape(g.num_groups * g.n, g.k))
    if g.n % 128 == 0:
        qb, sb = fg.quantize_fp8_blocks(w)
        qb = qb.view(g.num_groups, g.n, g.k)
        sb = sb.view(g.num_groups, g.n // 128, g.k // 128)
    else:  # blocks must not straddle two experts: quantize expert by expert
        qb = torch.empty((g.num_groups, g.n, g.k), dtype=torch.float8_e4m3fn, device="cuda")
        sb = torch.empty((g.num_groups, -(-g.n // 128), g.k // 128), dtype=torch.float32, device="cuda")
        for e in range(g.num_groups):
            fg.quantize_fp8_blocks(w[e * g.n : (e + 1) * g.n], out=(qb[e], sb[e]))
    idx = torch.from_numpy(g.m_indices).cuda()
    d = torch.full((g.m, g.n), float("nan"), dtype=torch.bfloat16, device="cuda")
    fg.m_grouped_fp8_gemm_nt_contiguous((q, sa), (qb, sb), d, idx)
    torch.cuda.synchronize()
    return q, sa, qb, sb, d


def check_groups(g, q, sa, qb, sb, d, groups=None, rows_per_group=None, cblocks=None, rng=None):
    rng = rng or np.random.default_rng(0)
    groups = range(g.num_groups) if groups is None else groups
    cblocks = np.arange(-(-g.n // 128)) if cblocks is None else cblocks
    cols = block_rows(g.n, cblocks)
    out = []
    for e in groups:
        rows = np.nonzero(g.m_indices == e)[0]
        if rows.size == 0:
            continue
        if rows_per_group and rows.size > rows_per_group:
            rows = np.unique(np.concatenate([rows[[0, -1]], rng.choice(rows, rows_per_group - 2, replace=False)]))
        oq, osa = oracle.quantize_groups(g.a[rows])
        oqb, osb = oracle.quantize_blocks(g.b[e][cols])
        ri = torch.as_tensor(rows, device="cuda")
        ci = torch.as_tensor(cols, device="cuda")
        assert np.array_equal(codes(q.view(torch.uint8).index_select(0, ri)), oq)
        assert np.array_equal(bits32(sa[:, : g.m].index_select(1, ri)), bits32(osa[:, : rows.size]))
        assert np.array_equal(codes(qb[e].view(torch.uint8).index_select(0, ci)), oqb)
        assert np.array_equal(bits32(sb[e][torch.as_tensor(cblocks, device="cuda")]), bits32(osb))
        ref = oracle.gemm_nt(oq, osa, oqb, osb)
        got = d_to_f64(d.index_select(0, ri).index_select(1, ci))
        out.append(check_gemm(got, ref, magnitude_sum(oq, osa, oqb, osb), g.k, f"group {e}"))
    return out


@pytest.mark.parametrize(
    "sizes,n,k",
    [
        ([5, 0, 130, 1, 128], 256, 256),
        ([0, 0, 7], 128, 384),
        ([300, 129, 64, 0, 1], 200, 512),
        ([128], 384, 256),
        ([1] * 9, 128, 128),
        ([700, 1000, 260, 0, 513], 512, 384),
    ],
)
def test_small_grouped_cases(sizes, n, k):
    g = workloads.small_grouped(sizes, n, k, seed=sum(sizes) + n + k)
    q, sa, qb, sb, d = gpu_grouped(g)
    check_groups(g, q, sa, qb, sb, d)
    # padding rows are unspecified, but every real row must be finite
    real = torch.from_numpy(g.m_indices >= 0).cuda()
    assert torch.isfinite(d[real].float()).all()


def test_one_group_equals_dense():
    lin = workloads.random_linear(256, 384, 512, seed=41)
    g = workloads.Grouped("g1", 1, 384, 512, np.array([256]), np.array([0]), np.zeros(256, np.int32), lin.a,
                          lin.b[None], np.arange(256))
    q, sa, qb, sb, d = gpu_grouped(g)
    dd = torch.empty_like(d)
    fg.fp8_gemm_nt((q, sa), (qb[0], sb[0]), dd)
    torch.cuda.synchronize()
    check_groups(g, q, sa, qb, sb, d)
    # same arithmetic per output tile: identical bits
    assert torch.equal(dd.view(torch.int16), d.view(torch.int16))


def test_moe_zipf_32_experts_every_tile():
    """The 32-expert Zipf case (K = 7168, N = 4096): every output column of
    one real row from each 64-row band of the layout (the height of a wave's
    tile) that holds real rows, so every workgroup tile of every expert (128
    rows, 512 or 256 columns as planned) -- and every 64-row wave tile with
    real rows -- is compared with the oracle, with each expert's whole weight
    quantized by the oracle."""
    g = workloads.moe_grouped()
    assert g.num_groups == 32 and g.k == 7168 and g.n == 4096
    assert np.all(g.starts % 128 == 0) and g.m % 128 == 0
    assert int(g.sizes.sum()) == 8192 * 4
    print(f"grouped {g.name}: m_pad={g.m}", flush=True)
    q, sa, qb, sb, d = gpu_grouped(g)
    real = torch.from_numpy(g.m_indices >= 0).cuda()
    assert torch.isfinite(d[real].float()).all()
    rows = one_row_per_band(np.nonzero(g.m_indices >= 0)[0], 64, np.random.default_rng(4))
    assert set(g.m_indices[rows // 128 * 128]) == set(range(32)), "a sampled band in every expert"
    oqb, osb = oracle_workers.quantize_blocks(g.b.reshape(g.num_groups * g.n, g.k))
    assert np.array_equal(codes(qb.view(torch.uint8).reshape(-1, g.k)), oqb), "weight codes differ"
    assert np.array_equal(bits32(sb.reshape(-1, g.k // 128)), bits32(osb)), "weight scales differ"
    oqb = oqb.reshape(g.num_groups, g.n, g.k)
    osb = osb.reshape(g.num_groups, g.n // 128, g.k // 128)
    oq, osa = oracle.quantize_groups(g.a[rows])
    ri = torch.as_tensor(rows, device="cuda")
    assert np.array_equal(codes(q.view(torch.uint8).index_select(0, ri)), oq), "activation codes differ"
    assert np.array_equal(bits32(sa[:, : g.m].index_select(1, ri)), bits32(osa[:, : rows.size])), "scales differ"
    got = d_to_f64(d.index_select(0, ri))
    parts = []
    for e in range(g.num_groups):
        sel = np.nonzero(g.m_indices[rows] == e)[0]
        if sel.size == 0:
            continue
        parts.append(oracle_workers.product_stats(oq[sel], osa[:, sel], oqb[e], osb[e], got[sel], g.k, piece=64))
        assert_stats(parts[-1], f"expert {e}")
    assert_stats(oracle_workers.merge(parts), "all experts")


def test_grouped_deterministic():
    g = workloads.small_grouped([200, 333, 0, 90], 256, 512, seed=3)
    _, _, _, _, d1 = gpu_grouped(g)
    _, _, _, _, d2 = gpu_grouped(g)
    real = torch.from_numpy(g.m_indices >= 0).cuda()
    assert torch.equal(d1[real].view(torch.int16), d2[real].view(torch.int16))


@pytest.mark.parametrize(
    "sizes,n,k",
    [([300, 129, 64, 0, 1], 512, 256), ([700, 1000, 260, 0, 513], 768, 384), ([5, 0, 2000, 1, 128, 900], 4096, 640)],
)
def test_persistent_walk_matches_per_block_kernel(sizes, n, k, monkeypatch):
    """The persistent walk over the grouped layout (padding blocks skipped,
    several tiles per workgroup) gives the same bits as one workgroup per
    block."""
    g = workloads.small_grouped(sizes, n, k, seed=sum(sizes) + 7)
    monkeypatch.setenv("FGFP8_GROUPED_TILE", "tile128x256_w2x4")  # the walk's tile
    monkeypatch.setenv("FGFP8_PERSISTENT", "0")
    _, _, _, _, d1 = gpu_grouped(g)
    monkeypatch.setenv("FGFP8_PERSISTENT", "1")
    q, sa, qb, sb, d2 = gpu_grouped(g)
    real = torch.from_numpy(g.m_indices >= 0).cuda()
    assert torch.equal(d1[real].view(torch.int16), d2[real].view(torch.int16))
    check_groups(g, q, sa, qb, sb, d2, rows_per_group=16)


@pytest.mark.parametrize(
    "sizes,n,k",
    [
        ([5, 0, 130, 1, 128], 512, 128),
        ([300, 129, 64, 0, 1], 700, 256),
        ([700, 1000, 260, 0, 513], 1000, 384),
        ([5, 0, 2000, 1, 128, 900], 4224, 640),
        ([1] * 9, 128, 128),
    ],
)
def test_wide_tile_matches_128x256(sizes, n, k, monkeypatch):
    """The 128x512 grouped tile (its scales loaded into registers, not staged
    through LDS) gives the same bits as the 128x256 tile on every real row:
    ragged N inside and across 512-column tiles, a one-chunk K, empty and
    one-row groups.  It also meets the oracle."""
    g = workloads.small_grouped(sizes, n, k, seed=sum(sizes) + n + 11)
    print(f"wide tile {sizes} n={n} k={k}", flush=True)
    monkeypatch.setenv("FGFP8_PERSISTENT", "0")
    monkeypatch.setenv("FGFP8_GROUPED_TILE", "tile128x256_w2x4")
    _, _, _, _, d1 = gpu_grouped(g)
    monkeypatch.setenv("FGFP8_GROUPED_TILE", "tile128x512_w2x4")
    q, sa, qb, sb, d2 = gpu_grouped(g)
    real = torch.from_numpy(g.m_indices >= 0).cuda()
    assert torch.equal(d1[real].view(torch.int16), d2[real].view(torch.int16))
    check_groups(g, q, sa, qb, sb, d2, rows_per_group=16)
