"""Pins for the oracle's MoE layer (deepgemm-rust README, "What's implemented",
moe_fp8_layer row).

Anchors:
* routing: a layout worked out by hand from the definition, a brute force of
  nested Python loops (experts, then tokens, then slots) on random small
  inputs with dropped and repeated slots, and invariants at workload scale;
* SiLU-times-up: closed forms (silu(0) = 0, silu(1) = 1/(1+e^-1)), the FP64
  logistic function of scipy, and the identity silu(g) - silu(-g) = g;
* combine: exact rational sums (fractions.Fraction) on small inputs;
* the whole layer: with one expert and one slot of weight one it reduces to the
  chain of dense products (the oracle's pinned gemm_nt, not the grouped one);
  it is equivariant under a permutation of the tokens and a relabelling of the
  experts; and it tracks an unquantized FP64 MoE within the FP8 error.
"""

from fractions import Fraction

import numpy as np
import pytest
from scipy.special import expit

import oracle
import workloads
from oracle import moe
from tests.exact import to_bf16


def bf16(bits):
    return workloads.bf16_bits_to_f32(bits).astype(np.float64)


# --------------------------------------------------------------------- route
def test_route_hand_example():
    # tokens 0..2, two slots each: t0 -> (1, 0), t1 -> (1, 2), t2 -> (0, 1).
    # expert 0 holds (t0, j1), (t2, j0) at rows 0, 1; expert 1 holds (t0, j0),
    # (t1, j0), (t2, j1) at rows 128..130; expert 2 holds (t1, j1) at row 256.
    counts, m_idx, tok, row_of = moe.route_contiguous([[1, 0], [1, 2], [0, 1]], 3, 512)
    assert counts.tolist() == [2, 3, 1]
    assert row_of.tolist() == [[128, 0], [129, 256], [1, 130]]
    expect_idx = np.full(512, -1)
    expect_idx[[0, 1]] = 0
    expect_idx[[128, 129, 130]] = 1
    expect_idx[256] = 2
    assert np.array_equal(m_idx, expect_idx)
    expect_tok = np.full(512, -1)
    expect_tok[[0, 1, 128, 129, 130, 256]] = [0, 2, 0, 1, 2, 1]
    assert np.array_equal(tok, expect_tok)
    assert moe.max_padded_rows(3, 2, 3) == 512


def brute_route(topk_idx, g, m_pad_max):
    tokens, topk = len(topk_idx), len(topk_idx[0])
    m_idx = [-1] * m_pad_max
    tok = [-1] * m_pad_max
    row_of = [[-1] * topk for _ in range(tokens)]
    counts = [0] * g
    row = 0
    for e in range(g):
        start = row
        for t in range(tokens):
            for j in range(topk):
                if topk_idx[t][j] == e:
                    m_idx[row], tok[row], row_of[t][j] = e, t, row
                    row += 1
        counts[e] = row - start
        while row % 128:
            row += 1
    return counts, m_idx, tok, row_of


@pytest.mark.parametrize("seed", range(6))
def test_route_matches_loop_brute_force(seed):
    rng = np.random.default_rng(seed)
    g = int(rng.integers(1, 9))
    tokens = int(rng.integers(0, 300))
    topk = int(rng.integers(1, 9))
    idx = rng.integers(-2, g + 2, size=(tokens, topk))  # out-of-range slots drop; repeats allowed
    mpm = moe.max_padded_rows(tokens, topk, g)
    got = moe.route_contiguous(idx, g, mpm)
    want = brute_route(idx.tolist(), g, mpm)
    assert got[0].tolist() == want[0]
    assert got[1].tolist() == want[1]
    assert got[2].tolist() == want[2]
    assert got[3].reshape(tokens, topk).tolist() == want[3]


def test_route_invariants_at_workload_scale():
    rng = np.random.default_rng(7)
    idx = workloads.zipf_topk_routing(rng, 2000, 32, 4, 1.1)
    counts, m_idx, tok, row_of = moe.route_contiguous(idx, 32)
    assert counts.sum() == idx.size
    assert np.array_equal(m_idx[row_of], idx)
    assert np.array_equal(tok[row_of], np.repeat(np.arange(2000)[:, None], 4, axis=1))
    rows = np.sort(row_of.reshape(-1))
    assert np.unique(rows).size == rows.size
    starts = np.nonzero(np.diff(np.concatenate(([-1], m_idx))) != 0)[0]
    for e in range(32):
        r = np.nonzero(m_idx == e)[0]
        assert r.size == counts[e]
        if r.size:
            assert r[0] % 128 == 0 and np.all(np.diff(r) == 1)
            assert np.all(np.diff(tok[r]) > 0)  # distinct experts per token: tokens strictly ascend
    assert starts.size > 0
    assert (m_idx >= 0).sum() == idx.size


# ------------------------------------------------------------------ silu_mul
def test_silu_mul_closed_forms():
    gate = np.array([[0.0, 1.0, -1.0, 2.0, -200.0, 200.0]], dtype=np.float32)
    up = np.array([[3.0, 1.0, 1.0, -0.5, 1.0, 1.0]], dtype=np.float32)
    h = workloads.f32_to_bf16_bits(np.concatenate([gate, up], axis=1))
    a = bf16(moe.silu_mul(h))[0]
    e1 = 1.0 / (1.0 + np.exp(-1.0))
    want = [0.0, float(to_bf16(Fraction(e1))), float(to_bf16(Fraction(-1.0 * (1 - e1)))),
            float(to_bf16(Fraction(-0.5 * 2.0 / (1 + np.exp(-2.0))))), 0.0, 200.0]
    assert a.tolist() == want
    assert np.all(np.isfinite(a))


def test_silu_mul_tracks_fp64_logistic():
    rng = np.random.default_rng(3)
    h = workloads.gaussian_bf16(rng, (64, 512), 3.0)
    a = bf16(moe.silu_mul(h))
    hg, hu = bf16(h[:, :256]), bf16(h[:, 256:])
    exact = hg * expit(hg) * hu
    ulp = np.exp2(np.floor(np.log2(np.maximum(np.abs(exact), 2.0**-126))) - 7)
    # one bf16 rounding of a value within a few float32 ulps of the exact one
    assert np.all(np.abs(a - exact) <= 0.5 * ulp + 2.0**-20 * np.abs(exact))
    # swapped halves would fail the check above; the gate must be the first half
    swapped = hu * expit(hu) * hg
    assert np.max(np.abs(a - swapped)) > 0.1


def test_silu_odd_part_identity():
    rng = np.random.default_rng(4)
    g = workloads.gaussian_bf16(rng, (1, 256), 2.0)
    ones = workloads.f32_to_bf16_bits(np.ones((1, 256), dtype=np.float32))
    neg = g ^ np.uint16(0x8000)
    a_pos = bf16(moe.silu_mul(np.concatenate([g, ones], axis=1)))
    a_neg = bf16(moe.silu_mul(np.concatenate([neg, ones], axis=1)))
    x = bf16(g)
    tol = 2.0**-8 * (np.abs(a_pos) + np.abs(a_neg)) + 1e-30
    assert np.all(np.abs((a_pos - a_neg) - x) <= tol)


def test_silu_mul_quantize_zeroes_padding_rows():
    rng = np.random.default_rng(5)
    h = workloads.gaussian_bf16(rng, (8, 512), 1.0)
    m_idx = np.array([0, 0, -1, 1, -1, 2, 2, -1], dtype=np.int32)
    q, sa = moe.silu_mul_quantize(h, m_idx)
    pad = m_idx < 0
    assert np.all(q[pad] == 0)
    assert np.all(sa[:, :8][:, pad] == 1.0)
    assert np.all(np.any(q[~pad] != 0, axis=1))


# ------------------------------------------------------------------- combine
def test_combine_exact_rational():
    rng = np.random.default_rng(6)
    y = workloads.gaussian_bf16(rng, (20, 16), 1.0)
    row_of = rng.integers(-1, 20, size=(5, 3)).astype(np.int32)
    w = rng.random((5, 3)).astype(np.float32)
    got = moe.combine(y, row_of, w)
    yv = bf16(y)
    for t in range(5):
        for c in range(16):
            s = Fraction(0)
            for j in range(3):
                if row_of[t, j] >= 0:
                    s += Fraction(float(w[t, j])) * Fraction(float(yv[row_of[t, j], c]))
            assert abs(Fraction(got[t, c]) - s) <= abs(s) * Fraction(1, 2**50) + Fraction(1, 2**1000)


def test_combine_single_slot_weight_one_is_identity():
    rng = np.random.default_rng(8)
    y = workloads.gaussian_bf16(rng, (10, 24), 1.0)
    row_of = np.array([[3], [0], [9], [-1]], dtype=np.int32)
    out = moe.combine(y, row_of, np.ones((4, 1), dtype=np.float32))
    assert np.array_equal(oracle.round_to_bf16(out)[:3], y[[3, 0, 9]])
    assert np.all(out[3] == 0)


# ---------------------------------------------------------------- the layer
def small_layer(seed, tokens=64, experts=4, topk=2, hidden=256, inter=256):
    return workloads.moe_layer(seed=seed, experts=experts, tokens=tokens, topk=topk, hidden=hidden, inter=inter)


def quantized_weights(c):
    w1 = [oracle.quantize_blocks(c.w1[g]) for g in range(c.experts)]
    w2 = [oracle.quantize_blocks(c.w2[g]) for g in range(c.experts)]
    return ((np.stack([q for q, _ in w1]), np.stack([s for _, s in w1])),
            (np.stack([q for q, _ in w2]), np.stack([s for _, s in w2])))


def test_layer_with_one_expert_reduces_to_dense_products():
    c = small_layer(11, tokens=40, experts=1, topk=1)
    (q1, s1), (q2, s2) = quantized_weights(c)
    r = moe.moe_layer(c.x, c.topk_idx, np.ones((40, 1), dtype=np.float32), (q1, s1), (q2, s2), 1)
    qa, sa = oracle.quantize_groups(c.x)
    h = oracle.round_to_bf16(oracle.gemm_nt(qa, sa, q1[0], s1[0]))
    g, u = bf16(h[:, :c.inter]), bf16(h[:, c.inter:])
    # the activation from its FP64 definition, then one bf16 rounding; differs
    # from the float32 steps only at rounding boundaries
    act64 = g * expit(g) * u
    act = moe.silu_mul(h)
    assert np.mean(act != oracle.round_to_bf16(act64)) < 0.01
    qa2, sa2 = oracle.quantize_groups(act)
    y = oracle.round_to_bf16(oracle.gemm_nt(qa2, sa2, q2[0], s2[0]))
    assert np.array_equal(r["out_bf16"], y)
    assert np.array_equal(r["h"][:40], h)


def test_layer_token_permutation_and_expert_relabel_equivariance():
    c = small_layer(12)
    w1, w2 = quantized_weights(c)
    base = moe.moe_layer(c.x, c.topk_idx, c.topk_weights, w1, w2, c.experts)["out_bf16"]
    rng = np.random.default_rng(1)
    perm = rng.permutation(c.tokens)
    p = moe.moe_layer(c.x[perm], c.topk_idx[perm], c.topk_weights[perm], w1, w2, c.experts)["out_bf16"]
    assert np.array_equal(p, base[perm])
    relabel = rng.permutation(c.experts)  # expert e becomes relabel[e]
    inv = np.argsort(relabel)
    w1r = (w1[0][inv], w1[1][inv])
    w2r = (w2[0][inv], w2[1][inv])
    r = moe.moe_layer(c.x, relabel[c.topk_idx], c.topk_weights, w1r, w2r, c.experts)["out_bf16"]
    assert np.array_equal(r, base)


def test_layer_tracks_unquantized_fp64_moe():
    c = small_layer(13, tokens=48, experts=3, topk=2, hidden=384, inter=256)
    w1, w2 = quantized_weights(c)
    out = moe.moe_layer(c.x, c.topk_idx, c.topk_weights, w1, w2, c.experts)["out"]
    x = bf16(c.x)
    ref = np.zeros_like(out)
    for t in range(c.tokens):
        for j in range(c.topk):
            e = c.topk_idx[t, j]
            hh = bf16(c.w1[e]) @ x[t]
            g, u = hh[:c.inter], hh[c.inter:]
            ref[t] += c.topk_weights[t, j] * (bf16(c.w2[e]) @ (g * expit(g) * u))
    rel = np.linalg.norm(out - ref) / np.linalg.norm(ref)
    assert rel < 0.08, rel  # FP8 E4M3 keeps 3 fraction bits: a few percent per product
    assert rel > 1e-4  # and the quantization is really there
