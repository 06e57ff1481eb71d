"""Pins for the oracle's block-scaled product and its grouped variant.

Anchors: exact rational brute force (fractions.Fraction), exact integer
arithmetic for the FP8 partial products, the invariant the pages state (two
such products differ only by summation order: Linnet "Backend plugins"
page, module docstring of the DeepGEMM plugin source), the constant-scale
quick start of the deepgemm-rust README (a closed form), and reductions to a
plain matrix product.
"""

import json
import os
from fractions import Fraction

import numpy as np
import pytest

import oracle
import workloads
from tests.exact import to_bf16

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")
FINITE = np.array([c for c in range(256) if c not in (0x7F, 0xFF)], dtype=np.uint8)


def random_operands(rng, m, n, k, extreme=False):
    qa = rng.choice(FINITE, size=(m, k)).astype(np.uint8)
    qb = rng.choice(FINITE, size=(n, k)).astype(np.uint8)
    if extreme:
        qa[:, ::3] = 0x7E
        qb[:, ::3] = 0xFE
    sa = np.full((k // 128, -(-m // 4) * 4), np.nan, dtype=np.float32)
    sa[:, :m] = (rng.random((k // 128, m)) * 2.0 ** rng.integers(-12, 4, size=(k // 128, m))).astype(np.float32)
    sb = (rng.random((-(-n // 128), k // 128)) * 2.0 ** rng.integers(-12, 4, size=(-(-n // 128), k // 128))).astype(np.float32)
    return qa, sa, qb, sb


def fraction_gemm(qa, sa, qb, sb):
    """D = sum_k dec(qa[m,k]) dec(qb[n,k]) sa[k//128][m] sb[n//128][k//128], exactly."""
    t = oracle.e4m3_table()
    m, k = qa.shape
    n = qb.shape[0]
    fa = [[Fraction(float(t[c])) for c in row] for row in qa]
    fb = [[Fraction(float(t[c])) for c in row] for row in qb]
    out = [[Fraction(0)] * n for _ in range(m)]
    for i in range(m):
        for j in range(n):
            acc = Fraction(0)
            for kb in range(k // 128):
                s = Fraction(float(sa[kb, i])) * Fraction(float(sb[j // 128, kb]))
                acc += s * sum(fa[i][kk] * fb[j][kk] for kk in range(kb * 128, (kb + 1) * 128))
            out[i][j] = acc
    return out


@pytest.mark.parametrize("m,n,k", [(1, 1, 128), (3, 5, 256), (8, 8, 384), (2, 130, 256)])
def test_gemm_matches_rational_brute_force(m, n, k):
    rng = np.random.default_rng(m * 100 + n + k)
    qa, sa, qb, sb = random_operands(rng, m, n, k)
    d = oracle.gemm_nt(qa, sa, qb, sb)
    exact = fraction_gemm(qa, sa, qb, sb)
    t = oracle.e4m3_table()
    for i in range(m):
        for j in range(n):
            # error bound: K/128 roundings of terms bounded by sum |terms|
            mag = sum(
                abs(float(t[qa[i, kk]]) * float(t[qb[j, kk]])) * float(sa[kk // 128, i]) * float(sb[j // 128, kk // 128])
                for kk in range(k)
            )
            assert abs(Fraction(d[i, j]) - exact[i][j]) <= Fraction(2.0**-50) * Fraction(mag) + Fraction(2.0**-1000)


def test_partial_products_are_exact_integers():
    """dec(code) * 2^9 is an integer for every finite code, so 2^18 * P is an
    integer sum that int64 computes exactly; the FP64 matrix product must equal it."""
    rng = np.random.default_rng(5)
    qa, _, qb, _ = random_operands(rng, 64, 48, 128, extreme=True)
    t = oracle.e4m3_table()
    ia = np.round(t[qa] * 512).astype(np.int64)
    ib = np.round(t[qb] * 512).astype(np.int64)
    p_int = ia @ ib.T
    d = oracle.gemm_nt(qa, np.ones((1, 64), np.float32), qb, np.ones((1, 1), np.float32))
    assert np.array_equal(d * 2.0**18, p_int.astype(np.float64))
    assert np.abs(p_int).max() < 2**53


def test_chunk_order_and_dequantized_form_agree():
    """Reordering the K chunks, or dequantizing first and doing one FP64
    product, only changes the summation order: results agree to FP64 rounding."""
    rng = np.random.default_rng(9)
    m, n, k = 37, 300, 1024
    qa, sa, qb, sb = random_operands(rng, m, n, k)
    d = oracle.gemm_nt(qa, sa, qb, sb)
    perm = rng.permutation(k // 128)
    cols = np.concatenate([np.arange(p * 128, (p + 1) * 128) for p in perm])
    d_perm = oracle.gemm_nt(qa[:, cols], sa[perm], qb[:, cols], sb[:, perm])
    d_deq = oracle.gemm_nt_dequantized(qa, sa, qb, sb)
    for other in (d_perm, d_deq):
        assert np.linalg.norm(other - d) <= 1e-12 * np.linalg.norm(d)


def test_constant_scales_quick_start_closed_form():
    """deepgemm-rust quick start: every activation scale 0.01 and every weight
    scale 0.02.  Then D = fl32(0.01) * fl32(0.02) * (Qa . Qb^T), with the code
    product computed exactly in integers."""
    with open(os.path.join(GOLDEN, "quickstart_constant_scales.json")) as f:
        g = json.load(f)
    assert g["k"] % g["k_multiple"] == 0
    rng = np.random.default_rng(17)
    m, n, k = 24, 136, 512  # a reduced shape of the quick start's (m, n, k)
    qa, _, qb, _ = random_operands(rng, m, n, k)
    sa = np.full((k // 128, 24), np.float32(g["sfa"]), dtype=np.float32)
    sb = np.full((-(-n // 128), k // 128), np.float32(g["sfb"]), dtype=np.float32)
    d = oracle.gemm_nt(qa, sa, qb, sb)
    t = oracle.e4m3_table()
    p_int = np.round(t[qa] * 512).astype(np.int64) @ np.round(t[qb] * 512).astype(np.int64).T
    c = float(np.float32(g["sfa"])) * float(np.float32(g["sfb"]))
    expect = c * p_int.astype(np.float64) * 2.0**-18
    # the oracle rounds once per 128-chunk term: bound by the sum of |chunk terms|
    ia, ib = np.round(t[qa] * 512).astype(np.int64), np.round(t[qb] * 512).astype(np.int64)
    mag = sum(np.abs(ia[:, j : j + 128] @ ib[:, j : j + 128].T) for j in range(0, k, 128)) * c * 2.0**-18
    assert np.all(np.abs(d - expect) <= (k // 128 + 1) * 2.0**-53 * mag)


def test_unit_scales_reduce_to_plain_matmul():
    rng = np.random.default_rng(19)
    qa, _, qb, _ = random_operands(rng, 16, 40, 256)
    d = oracle.gemm_nt(qa, np.ones((2, 16), np.float32), qb, np.ones((1, 2), np.float32))
    t = oracle.e4m3_table()
    assert np.array_equal(d, t[qa] @ t[qb].T)  # exact on both sides


def test_scale_indexing_is_per_row_and_per_column_block():
    """Scale only one (chunk, row) of sa or one (column block, chunk) of sb:
    exactly that row / that 128-column block changes, by the expected factor."""
    rng = np.random.default_rng(29)
    m, n, k = 6, 260, 384
    qa, sa, qb, sb = random_operands(rng, m, n, k)
    d0 = oracle.gemm_nt(qa, sa, qb, sb)
    sa2 = sa.copy()
    sa2[1, 4] *= 2
    d1 = oracle.gemm_nt(qa, sa2, qb, sb)
    changed = np.any(d1 != d0, axis=1)
    assert changed.tolist() == [False, False, False, False, True, False]
    sb2 = sb.copy()
    sb2[2, 0] *= 4
    d2 = oracle.gemm_nt(qa, sa, qb, sb2)
    cols = np.nonzero(np.any(d2 != d0, axis=0))[0]
    assert cols.min() >= 256 and cols.max() <= 259


def test_grouped_reduces_to_dense_per_group():
    sizes = [5, 0, 130, 1, 128]
    rng = np.random.default_rng(31)
    starts, padded, m_idx = workloads.grouped_layout(sizes)
    assert np.all(starts % 128 == 0) and m_idx.shape[0] == padded.sum()
    G, n, k = len(sizes), 200, 256
    m = m_idx.shape[0]
    qa, sa, _, _ = random_operands(rng, m, n, k)
    qb = rng.choice(FINITE, size=(G, n, k)).astype(np.uint8)
    sb = (rng.random((G, 2, 2)) + 0.5).astype(np.float32)
    d = oracle.grouped_gemm_nt(qa, sa, m_idx, qb, sb, G)
    for g in range(G):
        rows = np.nonzero(m_idx == g)[0]
        assert rows.size == sizes[g]
        if rows.size:
            assert np.all(rows >= starts[g]) and np.all(rows < starts[g] + padded[g])
            ref = oracle.gemm_nt(qa[rows], sa[:, rows], qb[g], sb[g])
            assert np.array_equal(d[rows], ref)
    assert np.all(np.isnan(d[m_idx < 0]))
    # the flat (num_groups * n, k) weight form of the quick start gives the same result
    d_flat = oracle.grouped_gemm_nt(qa, sa, m_idx, qb.reshape(G * n, k), sb.reshape(G * 2, 2), G)
    assert np.array_equal(np.nan_to_num(d_flat, nan=7.0), np.nan_to_num(d, nan=7.0))


def test_grouped_layout_matches_the_quickstart_fixture():
    """The grouped layout and operand shapes against the deepgemm-rust
    "Quick start" grouped example (tests/golden/grouped_quickstart_layout.json):
    every group starts at a multiple of the fixture's alignment, b is
    (num_groups * n, k) and sfb (num_groups * ceil(n/128), ceil(k/128));
    the oracle accepts exactly those flat forms, and refuses a weight whose
    rows are not a multiple of num_groups."""
    with open(os.path.join(GOLDEN, "grouped_quickstart_layout.json")) as f:
        fx = json.load(f)
    align = fx["alignment"]
    assert align == 128 and fx["b_shape"] == ["num_groups * n", "k"]
    assert fx["sfb_shape"] == ["num_groups * ceil(n/128)", "ceil(k/128)"]
    sizes = [3, 0, 200, 128, 1]
    starts, padded, m_idx = workloads.grouped_layout(sizes)
    assert np.all(starts % align == 0) and np.all(padded % align == 0)
    assert starts.tolist() == [0, 128, 128, 384, 512] and m_idx.shape[0] == 640
    G, n, k = len(sizes), 136, 256  # n not a multiple of 128: ceil(n/128) = 2 blocks per group
    rng = np.random.default_rng(43)
    qa, sa, _, _ = random_operands(rng, m_idx.shape[0], n, k)
    qb = rng.choice(FINITE, size=(G * n, k)).astype(np.uint8)  # (num_groups * n, k)
    sb = (rng.random((G * -(-n // 128), -(-k // 128))) + 0.5).astype(np.float32)
    d = oracle.grouped_gemm_nt(qa, sa, m_idx, qb, sb, G)
    for g in range(G):
        rows = np.nonzero(m_idx == g)[0]
        if rows.size:
            nb = -(-n // 128)
            ref = oracle.gemm_nt(qa[rows], sa[:, rows], qb[g * n:(g + 1) * n], sb[g * nb:(g + 1) * nb])
            assert np.array_equal(d[rows], ref)
    with pytest.raises(ValueError):
        oracle.grouped_gemm_nt(qa, sa, m_idx, qb[:-1], sb, G)


def test_grouped_with_one_group_equals_dense():
    rng = np.random.default_rng(37)
    m, n, k = 256, 136, 384
    qa, sa, qb, sb = random_operands(rng, m, n, k)
    d = oracle.grouped_gemm_nt(qa, sa, np.zeros(m, np.int32), qb[None], sb[None], 1)
    assert np.array_equal(d, oracle.gemm_nt(qa, sa, qb, sb))


def test_round_to_bf16_matches_exact_rounding():
    rng = np.random.default_rng(41)
    vals = np.concatenate(
        [
            rng.standard_normal(2000) * 10.0 ** rng.integers(-40, 38, size=2000),
            (np.arange(1, 300) * 2.0**-140),  # bf16 subnormal range, ties included
            [0.0, -0.0, 1.0 + 2.0**-8, 1.0 + 3 * 2.0**-8, 3.3895313892515355e38, 3.4e38],
        ]
    )
    bits = oracle.round_to_bf16(vals)
    got = workloads.bf16_bits_to_f32(bits).astype(np.float64)
    for v, gv in zip(vals, got):
        r = to_bf16(Fraction(float(v)))
        if r is None:
            assert np.isinf(gv)
        else:
            assert Fraction(float(gv)) == r, v


def _masked_operands(rng, g_count, max_m, n, k):
    qa = rng.choice(FINITE, size=(g_count, max_m, k)).astype(np.uint8)
    qb = rng.choice(FINITE, size=(g_count, n, k)).astype(np.uint8)
    sa = (rng.random((k // 128, g_count * max_m)) * 2.0 ** rng.integers(-8, 4, size=(k // 128, g_count * max_m))).astype(np.float32)
    sb = (rng.random((g_count, -(-n // 128), k // 128)) + 0.25).astype(np.float32)
    return qa, sa, qb, sb


def test_masked_matches_rational_brute_force():
    """Tiny masked case against exact rationals, element by element: the
    group's weight and scale block, the folded activation-scale column
    g*max_m + r, and the row mask."""
    rng = np.random.default_rng(43)
    g_count, max_m, n, k = 3, 4, 3, 256
    qa, sa, qb, sb = _masked_operands(rng, g_count, max_m, n, k)
    masked = np.array([2, 0, 4])
    d = oracle.masked_grouped_gemm_nt(qa, sa, masked, qb, sb)
    t = oracle.e4m3_table()
    for g in range(g_count):
        for r in range(max_m):
            if r >= masked[g]:
                assert np.all(np.isnan(d[g, r]))
                continue
            for j in range(n):
                exact = Fraction(0)
                mag = 0.0
                for kb in range(k // 128):
                    s = Fraction(float(sa[kb, g * max_m + r])) * Fraction(float(sb[g, j // 128, kb]))
                    part = sum(Fraction(float(t[qa[g, r, kk]])) * Fraction(float(t[qb[g, j, kk]])) for kk in range(kb * 128, (kb + 1) * 128))
                    exact += s * part
                    mag += float(s) * sum(abs(float(t[qa[g, r, kk]]) * float(t[qb[g, j, kk]])) for kk in range(kb * 128, (kb + 1) * 128))
                assert abs(Fraction(d[g, r, j]) - exact) <= Fraction(2.0**-50) * Fraction(mag) + Fraction(2.0**-1000)


def test_masked_full_groups_equal_contiguous_layout():
    """With every group full (masked_m = max_m, max_m a multiple of 128) the
    dispatch buffer is exactly the contiguous layout with m_indices = g on
    group g's rows: the independently pinned contiguous form must agree."""
    rng = np.random.default_rng(47)
    g_count, max_m, n, k = 3, 128, 136, 256
    qa, sa, qb, sb = _masked_operands(rng, g_count, max_m, n, k)
    d = oracle.masked_grouped_gemm_nt(qa, sa, np.full(g_count, max_m), qb, sb)
    m_idx = np.repeat(np.arange(g_count, dtype=np.int32), max_m)
    d_c = oracle.grouped_gemm_nt(qa.reshape(g_count * max_m, k), sa, m_idx, qb, sb, g_count)
    assert np.array_equal(d.reshape(g_count * max_m, n), d_c)


def test_masked_groups_are_isolated_and_mask_is_a_prefix():
    """Changing one group's weight or its rows past masked_m changes nothing
    in the other groups, nor in the masked-off rows."""
    rng = np.random.default_rng(53)
    g_count, max_m, n, k = 4, 8, 130, 128
    qa, sa, qb, sb = _masked_operands(rng, g_count, max_m, n, k)
    masked = np.array([8, 3, 0, 5])
    d = oracle.masked_grouped_gemm_nt(qa, sa, masked, qb, sb)
    qb2, qa2 = qb.copy(), qa.copy()
    qb2[1] = rng.choice(FINITE, size=(n, k))
    qa2[3, 5:] = rng.choice(FINITE, size=(max_m - 5, k))
    d2 = oracle.masked_grouped_gemm_nt(qa2, sa, masked, qb2, sb)
    for g in (0, 2, 3):
        assert np.array_equal(np.nan_to_num(d[g], nan=7.0), np.nan_to_num(d2[g], nan=7.0))
    assert not np.array_equal(d[1, :3], d2[1, :3])
    assert np.all(np.isnan(d[2])) and np.all(np.isnan(d[3, 5:]))
