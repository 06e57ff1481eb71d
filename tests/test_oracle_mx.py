"""Pins for the oracle's MXFP8 recipe: one power-of-two scale per 1x32 block
of each row, E8M0 codes packed four to an int32 (deepgemm-rust README, "Full
recipes", gran-32 with UE8M0 scale factors).

Anchors: exact rational arithmetic (tests/exact.py) for the scale rule and the
codes; a packed word worked out by hand; the reduction to the gran-128 UE8M0
recipe when a 128-group's four blocks share their amax; rational brute force
for the product, its agreement with the dequantized FP64 product (the two
orders of summation), and its reduction to the FP32-scale product when every
scale of a 128x128 block is the same power of two.
"""

from fractions import Fraction

import numpy as np
import pytest

import oracle
import workloads
from tests.exact import e4m3_code, f32_fraction, to_f32


def bf16(values) -> np.ndarray:
    f = np.asarray(values, dtype=np.float32)
    bits = workloads.f32_to_bf16_bits(f)
    assert np.array_equal(workloads.bf16_bits_to_f32(bits), f)
    return bits


def exact_mx_block(xs):
    """Power-of-two scale and codes of one 32-block with exact rationals:
    s32 = RN32(amax / 448) (1 if amax == 0), s = the least power of two >= s32
    (within [2^-127, 2^127]); code_i = E4M3(RN32(x_i / s))."""
    amax = max(abs(f32_fraction(x)) for x in xs)
    s32 = Fraction(1) if amax == 0 else to_f32(amax / 448)
    e = -127
    while Fraction(2) ** e < s32 and e < 127:
        e += 1
    s = Fraction(2) ** e
    codes = [e4m3_code(to_f32(f32_fraction(x) / s), bool(np.signbit(x))) for x in xs]
    return e + 127, codes


def test_blocks_match_exact_rationals():
    rng = np.random.default_rng(21)
    for trial in range(12):
        scale = float(2.0 ** rng.integers(-40, 40))
        x = workloads.bf16_bits_to_f32(workloads.f32_to_bf16_bits(rng.standard_normal(256).astype(np.float32) * np.float32(scale)))
        x[rng.integers(0, 256, 3)] = 0.0
        q, s = oracle.quantize_mx(workloads.f32_to_bf16_bits(x)[None, :])
        codes = oracle.unpack_mx_scales(s, 1)[0]
        for b in range(8):
            want_code, want_q = exact_mx_block(x[32 * b: 32 * b + 32])
            assert codes[b] == want_code, (trial, b)
            assert q[0, 32 * b: 32 * b + 32].tolist() == want_q, (trial, b)


def test_zero_and_tiny_blocks():
    x = np.zeros(128, dtype=np.float32)
    x[32:64] = np.float32(2.0 ** -133)  # bf16 subnormal: amax/448 underflows to the smallest E8M0 scale
    x[64] = np.float32(-0.0)
    q, s = oracle.quantize_mx(bf16(x)[None, :])
    codes = oracle.unpack_mx_scales(s, 1)[0]
    assert codes[0] == 127 and codes[2] == 127 and codes[3] == 127  # zero blocks: s = 1
    assert codes[1] == 0  # 2^-127
    assert np.all(q[0, :32] == 0) and q[0, 64] == 0x80


def test_packed_word_by_hand():
    # blocks with amax 448 (s = 1, code 127), 896 (s = 2, 128), 1 (s = 2^-8
    # since 1/448 is just below 2^-8: code 119) and 0 (s = 1, 127)
    x = np.zeros(128, dtype=np.float32)
    x[0], x[32], x[64] = 448.0, 896.0, 1.0
    q, s = oracle.quantize_mx(bf16(x)[None, :])
    assert int(s[0, 0]) & 0xFFFFFFFF == 127 | (128 << 8) | (119 << 16) | (127 << 24)
    assert q[0, 0] == 0x7E and q[0, 32] == 0x7E  # 448 / 1 and 896 / 2 both encode 448
    assert q[0, 64] == 0x78  # 1 / 2^-8 = 256 = 2^8: exponent 15, mantissa 0
    assert s.shape == (1, 4) and np.all(s[0, 1:] == -1)


def test_reduces_to_gran128_ue8m0_when_blocks_share_amax():
    rng = np.random.default_rng(5)
    x = rng.uniform(-1, 1, size=(6, 512)).astype(np.float32)
    x[:, ::32] = np.float32(3.0)  # every 32-block holds its 128-group's amax
    bits = bf16(workloads.bf16_bits_to_f32(workloads.f32_to_bf16_bits(x)))
    q, s = oracle.quantize_mx(bits)
    q128, s128 = oracle.quantize_groups_ue8m0(bits)
    assert np.array_equal(q, q128)
    codes = oracle.unpack_mx_scales(s, 6).reshape(6, 4, 4)
    want = oracle.quantize.e8m0_code(s128[:, :6].T)
    assert np.array_equal(codes, np.repeat(want[:, :, None], 4, axis=2))


def test_product_brute_force_rationals():
    rng = np.random.default_rng(9)
    finite = np.array([c for c in range(256) if c not in (0x7F, 0xFF)], dtype=np.uint8)
    m, n, k = 3, 4, 128
    qa = rng.choice(finite, size=(m, k)).astype(np.uint8)
    qb = rng.choice(finite, size=(n, k)).astype(np.uint8)
    ca = rng.integers(100, 150, size=(m, 4))
    cb = rng.integers(100, 150, size=(n, 4))
    pack = lambda c: (c[:, 0] | (c[:, 1] << 8) | (c[:, 2] << 16) | (c[:, 3] << 24)).astype(np.uint32).view(np.int32)
    sa = np.full((1, 4), -1, dtype=np.int32)
    sa[0, :m] = pack(ca)
    sb = pack(cb)[None, :]
    got = oracle.gemm_nt_mx(qa, sa, qb, sb)
    t = oracle.e4m3_table()
    for i in range(m):
        for j in range(n):
            terms = [Fraction(float(t[qa[i, kk]])) * Fraction(float(t[qb[j, kk]]))
                     * Fraction(2) ** (int(ca[i, kk // 32]) - 127 + int(cb[j, kk // 32]) - 127) for kk in range(k)]
            ref = sum(terms)
            # four FP64 accumulations of exact block terms
            bound = sum(abs(x) for x in terms) * Fraction(4, 2**53) + Fraction(1, 2**1074)
            assert abs(Fraction(got[i, j]) - ref) <= bound


def test_product_equals_dequantized_fp64_product():
    rng = np.random.default_rng(3)
    a = workloads.gaussian_bf16(rng, (40, 384), 1.0)
    b = workloads.gaussian_bf16(rng, (56, 384), 0.02)
    qa, sa = oracle.quantize_mx(a)
    qb, sb = oracle.quantize_mx(b)
    d = oracle.gemm_nt_mx(qa, sa, qb, sb)
    t = oracle.e4m3_table()
    da = t[qa] * np.exp2(np.repeat(oracle.unpack_mx_scales(sa, 40) - 127, 32, axis=1))
    db = t[qb] * np.exp2(np.repeat(oracle.unpack_mx_scales(sb, 56) - 127, 32, axis=1))
    ref = da @ db.T
    assert np.allclose(d, ref, rtol=1e-12, atol=1e-12 * np.abs(ref).max())


def test_product_reduces_to_fp32_scale_product():
    """Every 32-block of a 128-chunk with the same power-of-two scale, and one
    scale per 128x128 weight block: the MX product equals gemm_nt with those
    scales."""
    rng = np.random.default_rng(4)
    finite = np.array([c for c in range(256) if c not in (0x7F, 0xFF)], dtype=np.uint8)
    m, n, k = 20, 130, 256
    qa = rng.choice(finite, size=(m, k)).astype(np.uint8)
    qb = rng.choice(finite, size=(n, k)).astype(np.uint8)
    ea = rng.integers(110, 140, size=(m, 2))
    eb = rng.integers(110, 140, size=(2, 2))  # per 128x128 weight block
    pack = lambda c: (c | (c << 8) | (c << 16) | (c << 24)).astype(np.uint32).view(np.int32)
    sa = np.full((2, 20), -1, np.int32)
    sa[:, :m] = pack(ea.T)
    sb = np.stack([pack(eb[np.arange(n) // 128, c]) for c in range(2)])
    d_mx = oracle.gemm_nt_mx(qa, sa, qb, sb)
    sa32 = np.ldexp(1.0, ea.T - 127).astype(np.float32)
    sb32 = np.ldexp(1.0, eb - 127).astype(np.float32)
    d = oracle.gemm_nt(qa, sa32, qb, sb32)
    t = np.abs(oracle.e4m3_table())
    mag = (t[qa] * np.repeat(sa32.T.astype(np.float64), 128, axis=1)) @ (
        t[qb] * np.repeat(np.repeat(sb32.astype(np.float64), 128, axis=0)[:n], 128, axis=1)).T
    assert np.all(np.abs(d_mx - d) <= 16 * 2.0**-53 * mag)
