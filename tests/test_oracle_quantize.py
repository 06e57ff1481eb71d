"""Pins for the oracle's group (1x128) and block (128x128) quantizers.

Anchors: exact rational arithmetic (tests/exact.py) for the float32 scale and
quotient roundings, closed-form constructions whose result is known without
running any quantizer, and invariants between the two quantizers.
"""

from fractions import Fraction

import numpy as np
import pytest

import oracle
import workloads
from tests.exact import e4m3_code, f32_fraction, to_f32


def bf16(values) -> np.ndarray:
    """bf16 bits of values that are exactly representable in bf16."""
    f = np.asarray(values, dtype=np.float32)
    bits = workloads.f32_to_bf16_bits(f)
    assert np.array_equal(workloads.bf16_bits_to_f32(bits), f), "value not exact in bf16"
    return bits


def exact_group(xs):
    """Scale and codes of one group computed with exact rationals:
    s = RN32(amax / 448) (1 if amax == 0); code_i = E4M3(RN32(x_i / s))."""
    amax = max(abs(f32_fraction(x)) for x in xs)
    s = Fraction(1) if amax == 0 else to_f32(amax / 448)
    codes = [e4m3_code(to_f32(f32_fraction(x) / s), bool(np.signbit(x))) for x in xs]
    return s, codes


def test_random_groups_match_exact_rationals():
    rng = np.random.default_rng(11)
    for trial in range(40):
        scale = float(2.0 ** rng.integers(-30, 30))
        x = workloads.bf16_bits_to_f32(workloads.f32_to_bf16_bits(rng.standard_normal(128).astype(np.float32) * np.float32(scale)))
        q, sa = oracle.quantize_groups(workloads.f32_to_bf16_bits(x)[None, :])
        s, codes = exact_group(x)
        assert Fraction(float(sa[0, 0])) == s
        assert list(q[0]) == codes


def test_subnormal_groups_match_exact_rationals():
    # bf16 subnormals (below 2^-126) down to the smallest, 2^-133
    rng = np.random.default_rng(12)
    for trial in range(10):
        mags = rng.integers(0, 128, size=128).astype(np.float64) * 2.0**-133
        sign = np.where(rng.random(128) < 0.5, -1.0, 1.0)
        x = (mags * sign).astype(np.float32)
        q, sa = oracle.quantize_groups(bf16(x)[None, :])
        s, codes = exact_group(x)
        assert Fraction(float(sa[0, 0])) == s
        assert list(q[0]) == codes


@pytest.mark.parametrize("j", [-20, -3, 0, 5, 40])
def test_power_of_two_construction(j):
    """Group x_i = dec(c_i) * 2^j with one element equal to +-448 * 2^j:
    then amax/448 = 2^j exactly, s = 2^j, and every code comes back unchanged."""
    rng = np.random.default_rng(100 + j)
    t = oracle.e4m3_table()
    finite = np.array([c for c in range(256) if c not in (0x7F, 0xFF)], dtype=np.uint8)
    codes = rng.choice(finite, size=128)
    codes[rng.integers(0, 128)] = 0xFE if j % 2 else 0x7E
    x = (t[codes] * 2.0**j).astype(np.float32)
    q, sa = oracle.quantize_groups(bf16(x)[None, :])
    assert sa[0, 0] == np.float32(2.0**j)
    assert np.array_equal(q[0], codes)


@pytest.mark.parametrize("c", [1.0, 0.02, 3.0e-5, 17.25, -2.5, 6.0e4])
def test_constant_group(c):
    """A constant group c: s = RN32(|c|/448), every element rounds to the
    largest code of its sign (|c|/s lies within a float32 ulp of 448)."""
    x = workloads.bf16_bits_to_f32(workloads.f32_to_bf16_bits(np.full(128, c, np.float32)))
    q, sa = oracle.quantize_groups(workloads.f32_to_bf16_bits(x)[None, :])
    assert Fraction(float(sa[0, 0])) == to_f32(abs(f32_fraction(x[0])) / 448)
    assert np.all(q == (0xFE if c < 0 else 0x7E))


def test_zero_and_negative_zero_groups():
    x = np.zeros((2, 256), dtype=np.float32)
    x[1, :128] = -0.0
    x[1, 128:] = -0.0
    x[0, 128:] = -0.0
    q, sa = oracle.quantize_groups(workloads.f32_to_bf16_bits(x))
    assert np.all(sa[:, :2] == 1.0)
    assert np.all(q[0, :128] == 0x00) and np.all(q[0, 128:] == 0x80) and np.all(q[1] == 0x80)


def test_hand_derived_group():
    """One element 7 (= 448 * 2^-6) and the rest 1.0: s = 2^-6 exactly;
    7/s = 448 -> 0x7E; 1/s = 64 = 2^6 -> exponent field 13, mantissa 0 -> 0x68."""
    x = np.ones(128, dtype=np.float32)
    x[5] = 7.0
    x[6] = -1.0
    q, sa = oracle.quantize_groups(bf16(x)[None, :])
    assert sa[0, 0] == np.float32(2.0**-6)
    expect = np.full(128, 0x68, dtype=np.uint8)
    expect[5] = 0x7E
    expect[6] = 0xE8
    assert np.array_equal(q[0], expect)


def test_scale_layout_mn_major_and_padding():
    rng = np.random.default_rng(3)
    for m in (1, 3, 4, 5, 9):
        x = workloads.gaussian_bf16(rng, (m, 384), 1.0)
        q, sa = oracle.quantize_groups(x)
        assert sa.shape == (3, -(-m // 4) * 4)
        for r in range(m):
            q1, sa1 = oracle.quantize_groups(x[r : r + 1])
            assert np.array_equal(q1[0], q[r])
            assert np.array_equal(sa1[:, 0], sa[:, r])
        # group g of row r is scaled by sa[g][r]: its largest element maps to +-448
        t = oracle.e4m3_table()
        dec = np.abs(t[q]).reshape(m, 3, 128)
        assert np.all(dec.max(axis=2) == 448.0)
    q, sa = oracle.quantize_groups(workloads.gaussian_bf16(rng, (5, 128), 1.0), sa_ld=12)
    assert sa.shape == (1, 12)


def test_quotient_never_reaches_saturation_on_workloads():
    """|x / s| < 464 for every element of the workload activations, so the
    saturation branch is never what decides a code (reading of the pages'
    'satfinite')."""
    for lin in workloads.prefill_linears(m=64):
        x = workloads.bf16_bits_to_f32(lin.a).reshape(lin.m, -1, 128)
        amax = np.abs(x).max(axis=2)
        s = np.where(amax == 0, np.float32(1), (amax / np.float32(448)).astype(np.float32))
        y = (x / s[:, :, None]).astype(np.float32)
        assert np.abs(y).max() < 464.0


def test_block_quantizer_equals_group_quantizer_when_rows_share_amax():
    """A 128x128 block whose every row has the same amax (and the same sign of
    that element) quantizes to the same codes as per-row 1x128 groups, and its
    block scale equals each row's group scale."""
    rng = np.random.default_rng(21)
    n, k = 256, 256
    w = rng.standard_normal((n, k)).astype(np.float32) * np.float32(0.02)
    w = workloads.bf16_bits_to_f32(workloads.f32_to_bf16_bits(w))
    w[:, 7] = 0.125  # every row's amax in group 0 and therefore in block (i, 0)
    w[:, 128 + 9] = -0.25  # group 1 / block column 1
    wb = workloads.f32_to_bf16_bits(w)
    qb, sb = oracle.quantize_blocks(wb)
    qg, sg = oracle.quantize_groups(wb)
    assert np.array_equal(qb, qg)
    for i in range(2):
        for j in range(2):
            assert np.all(sg[j, i * 128 : (i + 1) * 128] == sb[i, j])


def test_block_quantizer_partial_last_block_and_closed_forms():
    rng = np.random.default_rng(22)
    n, k = 200, 256
    t = oracle.e4m3_table()
    finite = np.array([c for c in range(256) if c not in (0x7F, 0xFF)], dtype=np.uint8)
    codes = rng.choice(finite, size=(n, k))
    # block (0,0) scale 2^-3, (0,1) 2^4, (1,0) 2^0, (1,1) 2^-10 -- rows 128..199 form block row 1
    exps = np.array([[-3, 4], [0, -10]])
    codes[3, 5] = 0x7E
    codes[100, 200] = 0xFE
    codes[150, 0] = 0x7E
    codes[199, 255] = 0xFE
    scale = np.repeat(np.repeat(2.0 ** exps, 128, axis=0)[:n], 128, axis=1)
    w = (t[codes] * scale).astype(np.float32)
    qb, sb = oracle.quantize_blocks(bf16(w))
    assert sb.shape == (2, 2)
    assert np.array_equal(sb, (2.0**exps).astype(np.float32))
    assert np.array_equal(qb, codes)


def test_block_quantizer_random_blocks_match_exact_rationals():
    rng = np.random.default_rng(23)
    w = workloads.gaussian_bf16(rng, (130, 128), 0.02)
    qb, sb = oracle.quantize_blocks(w)
    x = workloads.bf16_bits_to_f32(w)
    for i, rows in enumerate((slice(0, 128), slice(128, 130))):
        block = x[rows]
        amax = max(abs(f32_fraction(v)) for v in block.reshape(-1))
        s = to_f32(amax / 448)
        assert Fraction(float(sb[i, 0])) == s
        sample = rng.integers(0, block.size, size=300)
        for idx in sample:
            r, c = divmod(int(idx), 128)
            v = block[r, c]
            assert int(qb[rows][r, c]) == e4m3_code(to_f32(f32_fraction(v) / s), bool(np.signbit(v)))


def test_rejects_k_not_multiple_of_128():
    with pytest.raises(ValueError):
        oracle.quantize_groups(np.zeros((2, 100), np.uint16))
    with pytest.raises(ValueError):
        oracle.quantize_blocks(np.zeros((2, 100), np.uint16))


# ------------------------------------------------------------- UE8M0 scales
def exact_group_ue8m0(xs):
    """Power-of-two scale and codes with exact rationals: s32 = RN32(amax/448)
    (1 if amax == 0), s = the least power of two >= s32 within [2^-127, 2^127];
    code_i = E4M3(RN32(x_i / s))."""
    amax = max(abs(f32_fraction(x)) for x in xs)
    s32 = Fraction(1) if amax == 0 else to_f32(amax / 448)
    s = Fraction(2) ** -127
    while s < s32 and s < Fraction(2) ** 127:
        s *= 2
    codes = [e4m3_code(to_f32(f32_fraction(x) / s), bool(np.signbit(x))) for x in xs]
    return s, codes


def test_ue8m0_random_groups_match_exact_rationals():
    rng = np.random.default_rng(111)
    for trial in range(40):
        scale = float(2.0 ** rng.integers(-40, 40))
        x = workloads.bf16_bits_to_f32(workloads.f32_to_bf16_bits(rng.standard_normal(128).astype(np.float32) * np.float32(scale)))
        q, sa = oracle.quantize_groups_ue8m0(workloads.f32_to_bf16_bits(x)[None, :])
        s, codes = exact_group_ue8m0(x)
        assert Fraction(float(sa[0, 0])) == s
        assert list(q[0]) == codes


def test_ue8m0_subnormal_and_zero_groups():
    rng = np.random.default_rng(112)
    mags = rng.integers(0, 128, size=128).astype(np.float64) * 2.0**-133
    x = (mags * np.where(rng.random(128) < 0.5, -1.0, 1.0)).astype(np.float32)
    q, sa = oracle.quantize_groups_ue8m0(bf16(x)[None, :])
    s, codes = exact_group_ue8m0(x)
    assert Fraction(float(sa[0, 0])) == s == Fraction(2) ** -127  # clamped to the E8M0 minimum
    assert list(q[0]) == codes
    q0, s0 = oracle.quantize_groups_ue8m0(np.zeros((1, 128), np.uint16))
    assert s0[0, 0] == 1.0 and not q0.any()


@pytest.mark.parametrize("j", [-20, 0, 7])
def test_ue8m0_equals_fp32_recipe_when_the_scale_is_a_power_of_two(j):
    """With amax = 448 * 2^j the FP32 scale is already 2^j: both recipes agree."""
    rng = np.random.default_rng(200 + j)
    t = oracle.e4m3_table()
    finite = np.array([c for c in range(256) if c not in (0x7F, 0xFF)], dtype=np.uint8)
    codes = rng.choice(finite, size=(4, 128))
    codes[:, 5] = 0x7E
    x = (t[codes] * 2.0**j).astype(np.float32)
    q1, s1 = oracle.quantize_groups(bf16(x))
    q2, s2 = oracle.quantize_groups_ue8m0(bf16(x))
    assert np.array_equal(q1, q2) and np.array_equal(s1[:, :4], s2[:, :4])


def test_ue8m0_scales_are_powers_of_two_bounding_amax():
    (lin,) = workloads.prefill_linears(names=["o"])
    q, sa = oracle.quantize_groups_ue8m0(lin.a[:64])
    s = sa[:, :64].astype(np.float64)
    mant, _ = np.frexp(s)
    assert np.all(mant == 0.5), "scales must be powers of two"
    x = workloads.bf16_bits_to_f32(lin.a[:64]).reshape(64, -1, 128)
    amax = np.abs(x).max(axis=2).T.astype(np.float64)
    assert np.all(amax / 448 <= s * (1 + 2.0**-23)) and np.all(s < 2 * amax / 448 * (1 + 2.0**-23))


def test_ue8m0_blocks_match_exact_rationals():
    rng = np.random.default_rng(113)
    w = (rng.standard_normal((130, 256)) * 0.02).astype(np.float32)
    bits = workloads.f32_to_bf16_bits(w)
    q, sb = oracle.quantize_blocks_ue8m0(bits)
    wf = workloads.bf16_bits_to_f32(bits)
    for i, rows in enumerate([slice(0, 128), slice(128, 130)]):
        for j in range(2):
            block = wf[rows, j * 128 : (j + 1) * 128]
            s, codes = exact_group_ue8m0(block.ravel())
            assert Fraction(float(sb[i, j])) == s
            assert list(q[rows, j * 128 : (j + 1) * 128].ravel()) == codes
