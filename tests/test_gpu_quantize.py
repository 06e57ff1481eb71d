"""GPU parity of the quantizers against the oracle: bit-exact E4M3 bytes and
FP32 scale bit patterns (the quantization result is unique)."""

import numpy as np
import pytest
import torch

import fine_grained_block_fp8_amd as fg
import oracle
import workloads
from tests.parity import bits32, codes, to_dev_bf16

pytestmark = pytest.mark.gpu


def run_groups(a_bits: np.ndarray, sa_ld=None, guard=4096):
    """GPU quantize with poisoned, guarded outputs; returns (q, sa) numpy and
    asserts the guard bytes and the padding scale rows stay untouched."""
    m, k = a_bits.shape
    sa_ld = fg.padded_rows(m) if sa_ld is None else sa_ld
    x = to_dev_bf16(a_bits)
    qbuf = torch.full((m * k + guard,), 0xA5, dtype=torch.uint8, device="cuda")
    sbuf = torch.full(((k // 128) * sa_ld + guard,), float("nan"), dtype=torch.float32, device="cuda")
    q = qbuf[: m * k].view(m, k)
    sa = sbuf[: (k // 128) * sa_ld].view(k // 128, sa_ld)
    fg.quantize_fp8_groups(x, sa_ld=sa_ld, out=(q, sa))
    torch.cuda.synchronize()
    assert torch.all(qbuf[m * k :] == 0xA5), "write past the end of q"
    assert torch.all(torch.isnan(sbuf[(k // 128) * sa_ld :])), "write past the end of sa"
    if sa_ld > m:
        assert torch.all(torch.isnan(sa[:, m:])), "scale padding rows were written"
    return q.cpu().numpy(), sa[:, :m].cpu().numpy()


def assert_groups_match(a_bits, sa_ld=None, label=""):
    gq, gsa = run_groups(a_bits, sa_ld)
    oq, osa = oracle.quantize_groups(a_bits, sa_ld)
    m = a_bits.shape[0]
    assert np.array_equal(gq, oq), f"{label}: {np.sum(gq != oq)} codes differ"
    assert np.array_equal(bits32(gsa), bits32(osa[:, :m])), f"{label}: scales differ"


def test_single_linear_activation():
    assert_groups_match(workloads.single_linear().a, label="128x512")


@pytest.mark.parametrize("m,k", [(2048, 4096), (2048, 12288)])
def test_prefill_activations(m, k):
    rng = np.random.default_rng(2)
    a = workloads.activation_bf16(rng, m, k, outliers=True)
    assert_groups_match(a, label=f"prefill {m}x{k}")


@pytest.mark.parametrize("m", [1, 4, 16])
@pytest.mark.parametrize("n,k", workloads.DECODE_SHAPES)
def test_decode_activations(m, n, k):
    assert_groups_match(workloads.decode_linear(m, n, k).a, label=f"decode {m}x{k}")


@pytest.mark.parametrize("m", [1, 2, 3, 5, 127, 129, 300])
def test_ragged_rows(m):
    rng = np.random.default_rng(m)
    assert_groups_match(workloads.gaussian_bf16(rng, (m, 384), 1.0), label=f"m={m}")


def test_wider_scale_leading_dimension():
    rng = np.random.default_rng(9)
    assert_groups_match(workloads.gaussian_bf16(rng, (10, 256), 1.0), sa_ld=24, label="sa_ld=24")


def test_edge_case_groups():
    """Zero and negative-zero groups, bf16 subnormals, one-hot groups, huge
    outliers, groups whose amax is a power of two times 448, mixed signs."""
    k = 128 * 12
    rows = []
    z = np.zeros(k, np.float32)
    rows.append(z.copy())
    nz = z.copy()
    nz[:] = -0.0
    rows.append(nz)
    rng = np.random.default_rng(3)
    sub = (rng.integers(-127, 128, size=k) * 2.0**-133).astype(np.float32)  # bf16 subnormals
    rows.append(sub)
    oh = z.copy()
    oh[5::128] = 3.0
    oh[77::128] = -1e-30
    rows.append(oh)
    big = rng.standard_normal(k).astype(np.float32)
    big[::97] *= 1e30
    rows.append(big)
    p2 = rng.standard_normal(k).astype(np.float32)
    p2[::128] = 448.0 * 2.0**-20
    rows.append(p2)
    tiny = rng.standard_normal(k).astype(np.float32) * np.float32(1e-36)
    rows.append(tiny)
    a = workloads.f32_to_bf16_bits(np.stack(rows))
    assert_groups_match(a, label="edge groups")


def test_every_bf16_magnitude_pattern():
    """Groups built from every positive and negative bf16 finite bit pattern
    (65024 values), in two orders, so every exponent/mantissa combination is
    quantized under many different scales."""
    bits = np.arange(0, 0x7F80, dtype=np.uint16)
    allv = np.concatenate([bits, bits | 0x8000])
    rng = np.random.default_rng(4)
    a1 = allv[: (allv.size // 1024) * 1024].reshape(-1, 1024)
    a2 = rng.permutation(allv)[: a1.size].reshape(-1, 1024)
    assert_groups_match(np.ascontiguousarray(a1), label="ordered bf16 patterns")
    assert_groups_match(np.ascontiguousarray(a2), label="shuffled bf16 patterns")


def test_moe_activation_sample():
    g = workloads.moe_grouped(with_weights=False)
    rng = np.random.default_rng(0)
    rows = np.unique(np.concatenate([rng.choice(g.m, 1500, replace=False), np.nonzero(g.m_indices < 0)[0][:20]]))
    sub = np.ascontiguousarray(g.a[rows])
    assert_groups_match(sub, label="moe rows")


def test_groups_deterministic():
    rng = np.random.default_rng(5)
    a = workloads.gaussian_bf16(rng, (333, 1024), 1.0)
    q1, s1 = run_groups(a)
    q2, s2 = run_groups(a)
    assert np.array_equal(q1, q2) and np.array_equal(bits32(s1), bits32(s2))


# ------------------------------------------------------------------ blocks
def assert_blocks_match(w_bits, label=""):
    n, k = w_bits.shape
    w = to_dev_bf16(w_bits)
    guard = 4096
    qbuf = torch.full((n * k + guard,), 0x5A, dtype=torch.uint8, device="cuda")
    nb = -(-n // 128)
    sbuf = torch.full((nb * (k // 128) + guard,), float("nan"), dtype=torch.float32, device="cuda")
    q = qbuf[: n * k].view(n, k)
    sb = sbuf[: nb * (k // 128)].view(nb, k // 128)
    fg.quantize_fp8_blocks(w, out=(q, sb))
    torch.cuda.synchronize()
    assert torch.all(qbuf[n * k :] == 0x5A) and torch.all(torch.isnan(sbuf[nb * (k // 128) :]))
    oq, osb = oracle.quantize_blocks(w_bits)
    assert np.array_equal(codes(q), oq), f"{label}: weight codes differ"
    assert np.array_equal(bits32(sb), bits32(osb)), f"{label}: weight scales differ"


@pytest.mark.parametrize("n,k", [(256, 512), (1, 128), (200, 384), (129, 256), (6144, 4096)])
def test_weight_blocks(n, k):
    rng = np.random.default_rng(n + k)
    assert_blocks_match(workloads.gaussian_bf16(rng, (n, k), 0.02), label=f"{n}x{k}")


def test_weight_blocks_edge_values():
    rng = np.random.default_rng(8)
    w = rng.standard_normal((256, 256)).astype(np.float32) * np.float32(0.02)
    w[:128, :128] = 0.0  # all-zero block
    w[128:, :128] = -0.0
    w[:128, 128:] = (rng.integers(-127, 128, size=(128, 128)) * 2.0**-133).astype(np.float32)
    w[200, 200] = 3e38
    assert_blocks_match(workloads.f32_to_bf16_bits(w), label="edge blocks")
