"""Seeded synthetic inputs for the block-scaled FP8 linear, shared by the
tests, the benchmark and the oracle's callers.

This module holds input generation only: Gaussian draws, outlier planting,
top-k expert routing and the 128-row-aligned grouped layout.  It contains none
of the method's arithmetic (no quantization, scaling or products) and imports
neither the oracle nor the HIP library, so both sides can consume its arrays.

Every value is drawn in float32 from numpy's PCG64 and rounded to the nearest
bfloat16 (ties to even); the bfloat16 bit patterns (uint16) are what both
sides receive.  Workload shapes are the ones the pages' model uses (Qwen3-8B
linears, Linnet "Backend plugins" page, DeepGEMM section; the M=1, N=12288,
K=4096 decode linear of the AReno FP8 decode pull request, "Testing" section)
and a 32-expert MoE layer with K=7168, N=4096 per expert.  No trained weights
or real prompts are involved.
"""

from __future__ import annotations

from dataclasses import dataclass, field

import numpy as np

ALIGN = 128  # grouped layout: every group starts at a multiple of 128 rows


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 values to the nearest bfloat16 (ties to even), as uint16 bits.
    Inputs here are finite Gaussian draws; NaN/inf are not produced."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    lsb = (u >> 16) & 1
    return ((u + 0x7FFF + lsb) >> 16).astype(np.uint16)


def bf16_bits_to_f32(bits: np.ndarray) -> np.ndarray:
    return (np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


def _rngs(seed: int, n: int) -> list[np.random.Generator]:
    return [np.random.Generator(np.random.PCG64(s)) for s in np.random.SeedSequence(seed).spawn(n)]


def gaussian_bf16(rng: np.random.Generator, shape, std: float) -> np.ndarray:
    x = rng.standard_normal(size=shape, dtype=np.float32)
    if std != 1.0:
        x *= np.float32(std)
    return f32_to_bf16_bits(x)


def activation_bf16(rng: np.random.Generator, m: int, k: int, outliers: bool, outlier_rng=None) -> np.ndarray:
    """A ~ N(0, 1) in float32; with ``outliers``, exactly round(0.001*M*K)
    distinct uniformly chosen positions are multiplied by 20 before the
    bfloat16 rounding."""
    x = rng.standard_normal(size=(m, k), dtype=np.float32)
    if outliers:
        n_out = int(round(0.001 * m * k))
        if n_out:
            orng = outlier_rng if outlier_rng is not None else rng
            pos = orng.choice(m * k, size=n_out, replace=False)
            x.reshape(-1)[pos] *= np.float32(20.0)
    return f32_to_bf16_bits(x)


# --------------------------------------------------------------------- dense
@dataclass
class Linear:
    name: str
    m: int
    n: int
    k: int
    a: np.ndarray  # uint16 [M][K] bf16 bits
    b: np.ndarray  # uint16 [N][K] bf16 bits

    @property
    def flops(self) -> int:
        return 2 * self.m * self.n * self.k


def single_linear(seed: int = 1) -> Linear:
    """Single linear: A 128x512 ~ N(0,1), B 256x512 ~ N(0,0.02)."""
    ra, rb = _rngs(seed, 2)
    return Linear("single_128x256x512", 128, 256, 512, gaussian_bf16(ra, (128, 512), 1.0), gaussian_bf16(rb, (256, 512), 0.02))


PREFILL_SHAPES = (("qkv", 6144, 4096), ("o", 4096, 4096), ("gate_up", 24576, 4096), ("down", 4096, 12288))


def prefill_linears(seed: int = 2, m: int = 2048, names=None) -> list[Linear]:
    """Qwen3-8B-shaped prefill linears at M tokens: activations N(0,1) with
    0.1% outliers x20, weights N(0,0.02)."""
    rngs = _rngs(seed, 3 * len(PREFILL_SHAPES))
    out = []
    for i, (name, n, k) in enumerate(PREFILL_SHAPES):
        if names is not None and name not in names:
            continue
        ra, rb, ro = rngs[3 * i : 3 * i + 3]
        a = activation_bf16(ra, m, k, outliers=True, outlier_rng=ro)
        b = gaussian_bf16(rb, (n, k), 0.02)
        out.append(Linear(f"prefill_{name}_{m}x{n}x{k}", m, n, k, a, b))
    return out


DECODE_SHAPES = ((12288, 4096), (4096, 12288))


def decode_linear(m: int, n: int, k: int, seed: int = 3) -> Linear:
    """Decode-shaped linear (M in {1,4,16}); same distributions as prefill."""
    sub = {(12288, 4096): 0, (4096, 12288): 1}.get((n, k), 2)
    ra, rb, ro = _rngs(seed * 1000 + sub * 100 + m, 3)
    a = activation_bf16(ra, m, k, outliers=True, outlier_rng=ro)
    b = gaussian_bf16(rb, (n, k), 0.02)
    return Linear(f"decode_{m}x{n}x{k}", m, n, k, a, b)


def square_linear(m: int, n: int, k: int, seed: int = 5) -> Linear:
    ra, rb = _rngs(seed * 1000 + (m >> 10), 2)
    return Linear(f"square_{m}x{n}x{k}", m, n, k, gaussian_bf16(ra, (m, k), 1.0), gaussian_bf16(rb, (n, k), 0.02))


def random_linear(m: int, n: int, k: int, seed: int, a_std: float = 1.0, b_std: float = 0.02) -> Linear:
    ra, rb = _rngs(seed, 2)
    return Linear(f"rand_{m}x{n}x{k}", m, n, k, gaussian_bf16(ra, (m, k), a_std), gaussian_bf16(rb, (n, k), b_std))


# ------------------------------------------------------------------- grouped
def zipf_topk_routing(rng: np.random.Generator, tokens: int, experts: int, topk: int, alpha: float) -> np.ndarray:
    """Each token picks ``topk`` distinct experts, drawn one after another
    without replacement with probability proportional to rank^-alpha
    (rank r = 1..experts is expert r-1).  Returns int64 [tokens][topk]."""
    p = np.arange(1, experts + 1, dtype=np.float64) ** -alpha
    p /= p.sum()
    return np.stack([rng.choice(experts, size=topk, replace=False, p=p) for _ in range(tokens)])


def grouped_layout(group_sizes, align: int = ALIGN):
    """128-row-aligned contiguous layout: group g occupies rows
    [start[g], start[g] + size[g]) and is zero-padded to a multiple of
    ``align``; m_indices[r] = g for a real row of group g and -1 for padding.
    Returns (starts int64[G], padded_sizes int64[G], m_indices int32[M_pad])."""
    sizes = np.asarray(group_sizes, dtype=np.int64)
    padded = -(-sizes // align) * align
    starts = np.concatenate([[0], np.cumsum(padded)[:-1]]).astype(np.int64)
    m_indices = np.full(int(padded.sum()), -1, dtype=np.int32)
    for g, (s, n) in enumerate(zip(starts, sizes)):
        m_indices[s : s + n] = g
    return starts, padded, m_indices


@dataclass
class Grouped:
    name: str
    num_groups: int
    n: int
    k: int
    sizes: np.ndarray  # real rows per group
    starts: np.ndarray
    m_indices: np.ndarray  # int32 [M_pad]
    a: np.ndarray  # uint16 [M_pad][K]; padding rows are +0
    b: np.ndarray  # uint16 [G][N][K]
    token_of_row: np.ndarray = field(default=None)  # int64 [M_pad], -1 on padding

    @property
    def m(self) -> int:
        return int(self.m_indices.shape[0])

    @property
    def useful_flops(self) -> int:
        return 2 * int(self.sizes.sum()) * self.n * self.k


def moe_grouped(
    seed: int = 4,
    experts: int = 32,
    tokens: int = 8192,
    topk: int = 4,
    alpha: float = 1.1,
    n: int = 4096,
    k: int = 7168,
    with_weights: bool = True,
) -> Grouped:
    """MoE grouped workload: tokens x_t ~ N(0,1), routed top-k by a seeded
    Zipf(alpha) expert choice; rows grouped by expert in ascending token order
    and zero-padded to 128-row multiples; expert weights [G][N][K] ~ N(0,0.02)."""
    r_route, r_x, r_w = _rngs(seed, 3)
    choice = zipf_topk_routing(r_route, tokens, experts, topk, alpha)
    sizes = np.array([(choice == g).any(axis=1).sum() for g in range(experts)], dtype=np.int64)
    starts, _padded, m_indices = grouped_layout(sizes)
    x = gaussian_bf16(r_x, (tokens, k), 1.0)
    a = np.zeros((m_indices.shape[0], k), dtype=np.uint16)
    token_of_row = np.full(m_indices.shape[0], -1, dtype=np.int64)
    for g in range(experts):
        toks = np.nonzero((choice == g).any(axis=1))[0]  # ascending token order
        a[starts[g] : starts[g] + toks.size] = x[toks]
        token_of_row[starts[g] : starts[g] + toks.size] = toks
    if with_weights:
        b = np.empty((experts, n, k), dtype=np.uint16)
        for g in range(experts):
            b[g] = gaussian_bf16(r_w, (n, k), 0.02)
    else:
        b = None
    return Grouped(f"moe_{experts}x{n}x{k}_zipf{alpha}_top{topk}", experts, n, k, sizes, starts, m_indices, a, b, token_of_row)


def small_grouped(sizes, n: int, k: int, seed: int) -> Grouped:
    """A small grouped case with given real group sizes (zeros allowed)."""
    r_x, r_w = _rngs(seed, 2)
    sizes = np.asarray(sizes, dtype=np.int64)
    starts, _padded, m_indices = grouped_layout(sizes)
    a = np.zeros((m_indices.shape[0], k), dtype=np.uint16)
    for g, (s, c) in enumerate(zip(starts, sizes)):
        a[s : s + c] = gaussian_bf16(r_x, (int(c), k), 1.0)
    b = gaussian_bf16(r_w, (len(sizes), n, k), 0.02)
    token_of_row = np.where(m_indices >= 0, np.arange(m_indices.shape[0]), -1)
    return Grouped(f"grouped_{len(sizes)}x{n}x{k}", len(sizes), n, k, sizes, starts, m_indices, a, b, token_of_row)


# -------------------------------------------------------------------- masked
@dataclass
class Masked:
    """A masked grouped (dispatch-buffer) case: group g's rows are buffer rows
    g*max_m .. g*max_m + max_m - 1, the first masked_m[g] of them real."""

    name: str
    num_groups: int
    max_m: int
    n: int
    k: int
    masked_m: np.ndarray  # int32 [G]
    expected_m: int
    a: np.ndarray  # uint16 [G][max_m][K]; rows past masked_m hold unrelated values
    b: np.ndarray  # uint16 [G][N][K]


def small_masked(masked_m, max_m: int, n: int, k: int, seed: int) -> Masked:
    """Given per-group counts; every row of the buffer (real or not) ~ N(0,1),
    so rows past the count carry values a kernel must ignore."""
    r_x, r_w = _rngs(seed, 2)
    masked_m = np.asarray(masked_m, dtype=np.int32)
    g = masked_m.shape[0]
    a = gaussian_bf16(r_x, (g, max_m, k), 1.0)
    b = gaussian_bf16(r_w, (g, n, k), 0.02)
    em = int(np.clip(masked_m, 0, max_m).mean()) if g else 0
    return Masked(f"masked_{g}x{max_m}x{n}x{k}", g, max_m, n, k, masked_m, em, a, b)


def moe_masked(seed: int = 5, experts: int = 32, tokens: int = 1024, topk: int = 4, alpha: float = 1.1,
               n: int = 4096, k: int = 7168, with_weights: bool = True) -> Masked:
    """Decode-time MoE dispatch buffer: `tokens` tokens routed top-k by the
    seeded Zipf(alpha) expert choice (as moe_grouped); expert g receives
    masked_m[g] of them; max_m is the largest count rounded up to 128;
    expected_m the mean count (the hint a dispatcher knows ahead of time).
    Rows past a group's count are zero, as a freshly cleared buffer."""
    r_route, r_x, r_w = _rngs(seed, 3)
    choice = zipf_topk_routing(r_route, tokens, experts, topk, alpha)
    counts = np.array([(choice == g).any(axis=1).sum() for g in range(experts)], dtype=np.int32)
    max_m = int(-(-counts.max() // ALIGN) * ALIGN)
    x = gaussian_bf16(r_x, (tokens, k), 1.0)
    a = np.zeros((experts, max_m, k), dtype=np.uint16)
    for g in range(experts):
        toks = np.nonzero((choice == g).any(axis=1))[0]
        a[g, : toks.size] = x[toks]
    b = gaussian_bf16(r_w, (experts, n, k), 0.02) if with_weights else np.zeros((0,), np.uint16)
    return Masked(f"moe_masked_{experts}x{n}x{k}_zipf{alpha}_top{topk}_{tokens}tok", experts, max_m, n, k, counts,
                  int(round(counts.mean())), a, b)


# ----------------------------------------------------------------- MoE layer
@dataclass
class MoeLayer:
    name: str
    tokens: int
    experts: int
    topk: int
    hidden: int  # H
    inter: int  # I: w1 is [G][2I][H] (gate rows, then up rows), w2 [G][H][I]
    x: np.ndarray  # uint16 [T][H]
    topk_idx: np.ndarray  # int32 [T][topk]
    topk_weights: np.ndarray  # float32 [T][topk]
    w1: np.ndarray = field(default=None)  # uint16 [G][2I][H]
    w2: np.ndarray = field(default=None)  # uint16 [G][H][I]

    @property
    def useful_flops(self) -> int:
        """Both products over the routed pairs (padding rows excluded)."""
        pairs = int(((self.topk_idx >= 0) & (self.topk_idx < self.experts)).sum())
        return 2 * pairs * (2 * self.inter) * self.hidden + 2 * pairs * self.hidden * self.inter


def moe_layer(seed: int = 6, experts: int = 32, tokens: int = 8192, topk: int = 4, hidden: int = 7168,
              inter: int = 2048, alpha: float = 1.1, with_weights: bool = True) -> MoeLayer:
    """A MoE layer input: tokens x_t ~ N(0, 1) [T][H]; top-k distinct experts
    per token by the seeded Zipf(alpha) choice; routing weights = softmax of
    N(0, 1) logits over the token's k slots (float32, positive, summing to one);
    expert weights w1 [G][2I][H] and w2 [G][H][I] ~ N(0, 0.02)."""
    r_route, r_x, r_w1, r_w2, r_p = _rngs(seed, 5)
    choice = zipf_topk_routing(r_route, tokens, experts, topk, alpha).astype(np.int32)
    x = gaussian_bf16(r_x, (tokens, hidden), 1.0)
    logits = r_p.standard_normal(size=(tokens, topk)).astype(np.float64)
    p = np.exp(logits - logits.max(axis=1, keepdims=True))
    weights = (p / p.sum(axis=1, keepdims=True)).astype(np.float32)
    w1 = w2 = None
    if with_weights:
        w1 = np.empty((experts, 2 * inter, hidden), dtype=np.uint16)
        w2 = np.empty((experts, hidden, inter), dtype=np.uint16)
        for g in range(experts):
            w1[g] = gaussian_bf16(r_w1, (2 * inter, hidden), 0.02)
            w2[g] = gaussian_bf16(r_w2, (hidden, inter), 0.02)
    return MoeLayer(f"moe_layer_{experts}e_top{topk}_{tokens}tok_h{hidden}_i{inter}", tokens, experts, topk, hidden,
                    inter, x, choice, weights, w1, w2)


def device_fp8_operand(rows: int, k: int, seed: int, scale_shape, device: str = "cuda"):
    """Random E4M3 codes [rows][k] drawn on the device (operands too large to
    draw on the host: the largest K the library accepts), with float32 scales
    of shape ``scale_shape`` drawn uniformly in [2^-9, 2^-7].  Codes are
    uniform over the finite codes: magnitude code 0..0x7E with a random sign
    bit (never 0x7F / 0xFF, the NaNs).  torch's seeded device generator; the
    oracle sees the same bytes by copying the sampled rows back."""
    import torch

    gen = torch.Generator(device=device)
    gen.manual_seed(seed)
    q = torch.randint(0, 127, (rows, k), dtype=torch.uint8, device=device, generator=gen)
    q |= torch.randint(0, 2, (rows, k), dtype=torch.uint8, device=device, generator=gen) << 7
    s = torch.rand(scale_shape, dtype=torch.float32, device=device, generator=gen) * (2.0**-7 - 2.0**-9) + 2.0**-9
    return q.view(torch.float8_e4m3fn), s
