"""The block-scaled FP8 product D = A.B^T, dense and M-grouped (contiguous and
masked), in FP64.

Test infrastructure (see the package docstring): not part of the product path.

Definition (deepgemm-rust README, "What's implemented" table, fp8_gemm_nt row:
activation scales per 1x128 group, weight scales per 128x128 block, partials
promoted to FP32, bfloat16 output; and the kernel notes on applying the scales
per 128-wide block): for every
128-wide chunk kb of K, the FP8 operands give a partial product

    P[m, n, kb] = sum_{k in chunk kb} dec(qa[m, k]) * dec(qb[n, k])

which is then scaled by sa[kb][m] * sb[n // 128][kb] and accumulated:

    D[m, n] = sum_kb sa[kb][m] * sb[n // 128][kb] * P[m, n, kb].

In FP64 the partial products are exact (every E4M3 product is a multiple of
2^-18 and |P| < 128 * 448^2 < 2^25, well inside 53 bits) and so is each scale
product (float32 x float32), so the only roundings are one per accumulated
term.  The pages note that two such block-scaled products differ only by the
order of their sums (Linnet "Backend plugins" page, module docstring of the
plugin source): ``gemm_nt_dequantized`` is that other order (dequantize both operands,
then one FP64 matrix product) and the tests check the two agree.

Output rounding (bfloat16 output): ``round_to_bf16`` rounds the FP64 result once,
to nearest-even, to a bfloat16 bit pattern.  It is used only for diagnostics;
parity is judged against the FP64 result.
"""

from __future__ import annotations

import numpy as np

from .e4m3 import e4m3_decode
from .quantize import unpack_mx_scales

GROUP = 128


def _check(qa, sa, qb, sb):
    m, k = qa.shape
    n, k2 = qb.shape
    if k != k2 or k % GROUP:
        raise ValueError("A and B must share K, a multiple of 128")
    if sa.shape[0] != k // GROUP or sa.shape[1] < m:
        raise ValueError("sa must be [K/128][>= M]")
    if sb.shape != (-(-n // GROUP), k // GROUP):
        raise ValueError("sb must be [ceil(N/128)][K/128]")
    return m, n, k


def gemm_nt(qa, sa, qb, sb) -> np.ndarray:
    """FP64 D[M][N] from E4M3 codes qa [M][K], qb [N][K], activation scales
    sa float32 [K/128][>=M] (MN-major) and weight scales sb float32
    [ceil(N/128)][K/128], one 128-chunk at a time as the definition reads."""
    qa = np.asarray(qa, dtype=np.uint8)
    qb = np.asarray(qb, dtype=np.uint8)
    sa = np.asarray(sa, dtype=np.float32)
    sb = np.asarray(sb, dtype=np.float32)
    m, n, k = _check(qa, sa, qb, sb)
    a = e4m3_decode(qa)
    b = e4m3_decode(qb)
    d = np.zeros((m, n), dtype=np.float64)
    col_block = np.arange(n) // GROUP
    for kb in range(k // GROUP):
        chunk = slice(kb * GROUP, (kb + 1) * GROUP)
        p = a[:, chunk] @ b[:, chunk].T  # exact partial products
        scale = sa[kb, :m].astype(np.float64)[:, None] * sb[col_block, kb].astype(np.float64)[None, :]
        d += scale * p
    return d


def gemm_nt_dequantized(qa, sa, qb, sb) -> np.ndarray:
    """The same product summed in another order: dequantize each operand
    (code value times its scale, exact in FP64), then one FP64 matrix product."""
    qa = np.asarray(qa, dtype=np.uint8)
    qb = np.asarray(qb, dtype=np.uint8)
    sa = np.asarray(sa, dtype=np.float32)
    sb = np.asarray(sb, dtype=np.float32)
    m, n, k = _check(qa, sa, qb, sb)
    a = e4m3_decode(qa) * np.repeat(sa[:, :m].T.astype(np.float64), GROUP, axis=1)
    b_scale = np.repeat(np.repeat(sb.astype(np.float64), GROUP, axis=0)[:n], GROUP, axis=1)
    b = e4m3_decode(qb) * b_scale
    return a @ b.T


def grouped_gemm_nt(qa, sa, m_indices, qb, sb, num_groups: int) -> np.ndarray:
    """M-grouped contiguous product (deepgemm-rust README, "Quick start",
    grouped example: tokens of all experts concatenated, each group's start
    128-aligned, b of shape (num_groups * n, k), sfb of shape
    (num_groups * ceil(n/128), k/128)).

    qa [M][K]; sa [K/128][>=M]; m_indices int32 [M], the group of each row or
    -1 for a padding row; qb [num_groups * N][K] (or [G][N][K]); sb
    [num_groups * ceil(N/128)][K/128] (or [G][ceil(N/128)][K/128]).
    Row r with g = m_indices[r] >= 0 is the dense product of A's row r with
    group g's weight; padding rows are NaN (they carry no defined value).
    """
    qa = np.asarray(qa, dtype=np.uint8)
    m, k = qa.shape
    qb = np.asarray(qb, dtype=np.uint8).reshape(num_groups, -1, k)
    n = qb.shape[1]
    nb = -(-n // GROUP)
    sb = np.asarray(sb, dtype=np.float32).reshape(num_groups, nb, k // GROUP)
    sa = np.asarray(sa, dtype=np.float32)
    m_indices = np.asarray(m_indices, dtype=np.int64)
    d = np.full((m, n), np.nan, dtype=np.float64)
    for g in range(num_groups):
        rows = np.nonzero(m_indices == g)[0]
        if rows.size == 0:
            continue
        d[rows] = gemm_nt(qa[rows], sa[:, rows], qb[g], sb[g])
    return d


def masked_grouped_gemm_nt(qa, sa, masked_m, qb, sb) -> np.ndarray:
    """M-grouped masked product (deepgemm-rust README, "What's implemented",
    m_grouped_fp8_gemm_nt_masked row: the same product with a masked_m
    scheduler, for a dispatch buffer that holds every group's rows at a fixed
    stride; only the first masked_m[g] rows of group g are real).

    qa [G][max_m][K]; sa [K/128][>= G*max_m], the activation scales of the
    buffer viewed as one (G*max_m) x K matrix (the group folded into the
    scale column: row r of group g is column g*max_m + r); masked_m [G];
    qb [G][N][K]; sb [G][ceil(N/128)][K/128].  Returns D [G][max_m][N] with
    row r < masked_m[g] of group g the dense product of that row with group
    g's weight, and NaN elsewhere (those rows carry no defined value).
    """
    qa = np.asarray(qa, dtype=np.uint8)
    g_count, max_m, k = qa.shape
    qb = np.asarray(qb, dtype=np.uint8).reshape(g_count, -1, k)
    n = qb.shape[1]
    sb = np.asarray(sb, dtype=np.float32).reshape(g_count, -(-n // GROUP), k // GROUP)
    sa = np.asarray(sa, dtype=np.float32)
    masked_m = np.asarray(masked_m, dtype=np.int64)
    d = np.full((g_count, max_m, n), np.nan, dtype=np.float64)
    for g in range(g_count):
        rows = int(masked_m[g])
        if rows <= 0:
            continue
        cols = g * max_m + np.arange(rows)
        d[g, :rows] = gemm_nt(qa[g, :rows], sa[:, cols], qb[g], sb[g])
    return d


def round_to_bf16(d: np.ndarray) -> np.ndarray:
    """Round FP64 values once, to nearest-even, to bfloat16 bit patterns (uint16)."""
    d = np.asarray(d, dtype=np.float64)
    finite = np.isfinite(d)
    with np.errstate(over="ignore", invalid="ignore"):
        safe = np.where(finite, d, 0.0)
        mant, expo = np.frexp(safe)  # d = mant * 2^expo, 0.5 <= |mant| < 1
        # normal bf16: 8 significant bits -> mant * 2^8 rounded to an integer
        normal = np.rint(mant * 256.0) * np.exp2(expo - 8.0)
        # subnormal bf16 (|d| < 2^-126): quantum 2^-133
        sub = np.rint(np.where(np.abs(safe) < 2.0**-126, safe, 0.0) * 2.0**133) * 2.0**-133
        out = np.where(np.abs(safe) < 2.0**-126, sub, normal)
        out = np.where(np.abs(out) > 3.3895313892515355e38, np.copysign(np.inf, d), out)  # past bf16 max
        out = np.where(finite, out, d)
    bits = (out.astype(np.float32).view(np.uint32) >> 16).astype(np.uint16)
    return bits


def gemm_nt_mx(qa, sa_packed, qb, sb_packed) -> np.ndarray:
    """The MXFP8 product in FP64: with one power-of-two scale per 1x32 block
    of each row of A and of B (E8M0 codes packed four to an int32, see
    quantize_mx),

        D[m, n] = sum_b 2^(ea[m, b] - 127) * 2^(eb[n, b] - 127) * P[m, n, b],
        P[m, n, b] = sum_{k in block b} dec(qa[m, k]) * dec(qb[n, k]).

    Every term is exact in FP64 (a block partial is a multiple of 2^-18 below
    2^23, the scales are powers of two), so the only roundings are one per
    accumulated term."""
    qa = np.asarray(qa, dtype=np.uint8)
    qb = np.asarray(qb, dtype=np.uint8)
    m, k = qa.shape
    n, k2 = qb.shape
    if k != k2 or k % GROUP:
        raise ValueError("A and B must share K, a multiple of 128")
    ea = unpack_mx_scales(sa_packed, m)
    eb = unpack_mx_scales(sb_packed, n)
    a = e4m3_decode(qa)
    b = e4m3_decode(qb)
    d = np.zeros((m, n), dtype=np.float64)
    for blk in range(k // 32):
        cols = slice(32 * blk, 32 * blk + 32)
        p = a[:, cols] @ b[:, cols].T  # exact
        d += np.ldexp(p, (ea[:, blk] - 127)[:, None] + (eb[:, blk] - 127)[None, :])
    return d
