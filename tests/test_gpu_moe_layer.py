"""GPU parity of the MoE layer calls (deepgemm-rust README, "What's
implemented", moe_fp8_layer row) against the oracle, step by step and end to
end.

Criteria:
* routing (counts, m_indices, token_of_row, row_of) and the gather+quantize
  step: bit-exact (integer work and quantization of identical inputs);
* the first grouped product inside the layer: the product criteria of the
  dense product (its operands are bit-identical on both sides);
* SiLU-times-up + quantize on one seeded input: both sides decide each code in
  float32, but the kernel's expf and numpy's exp may differ in the last float32
  bit, which can move a bf16 rounding; one such move changes the element by one
  bf16 ulp and the group scale by at most 2^-7 relative, far below one E4M3 step
  (2^-3), so every code may differ by at most one step and the scales by at most
  2^-7 relative, and such differences must be rare;
* combine on one seeded input: the FP32 sum in slot order is within topk * 2^-24
  * sum|w y| of the exact sum, and its bf16 rounding within half a bf16 ulp more;
* inside the whole layer, the first product on the two sides may differ within
  the product tolerance (2e-3 normwise; about 1% of its bf16 outputs round the
  other way), so the activation that follows may round to the neighbouring
  E4M3 code: a relative change of about 2e-3 moves a rounding (step 2^-4 to
  2^-3 relative) with probability about 2e-3 / 2^-4 = 3%, each move changes
  that element by one step, normwise about sqrt(0.03) * 2^-3.5 = 1.6e-2, which
  passes through the second product and the convex combine (weights summing
  to one) unchanged.  The dequantized activation, y and out take a normwise
  tolerance of twice that, 2^-5.  The exactness of each step on identical
  inputs is what the step tests above check.
"""

import numpy as np
import pytest
import torch

import fine_grained_block_fp8_amd as fg
import oracle
import workloads
from oracle import moe
from tests.parity import bits32, check_gemm, codes, d_to_f64, magnitude_sum, to_dev_bf16

pytestmark = pytest.mark.gpu

TOL_LAYER = 2.0**-5


def dev_i32(a):
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.int32)).cuda()


def host(t):
    torch.cuda.synchronize()
    return t.cpu().numpy()


# --------------------------------------------------------------------- route
@pytest.mark.parametrize(
    "tokens,topk,experts,seed",
    [(0, 4, 8, 0), (1, 1, 1, 1), (255, 2, 3, 2), (256, 8, 16, 3), (257, 4, 32, 4), (1000, 6, 256, 5),
     (700, 8, 2048, 6), (3000, 4, 32, 7),
     # expert counts that split unevenly over the offsets scan's 256 threads
     # (runs of ceil(E/256) experts, the last threads' runs short or empty)
     (900, 4, 257, 8), (1200, 6, 300, 9), (2500, 8, 1000, 10), (4000, 3, 2047, 11)],
)
def test_route_bit_exact(tokens, topk, experts, seed):
    rng = np.random.default_rng(seed)
    idx = rng.integers(-1, experts + 1, size=(tokens, topk)).astype(np.int32)  # dropped and repeated slots
    print(f"route tokens={tokens} topk={topk} experts={experts} seed={seed}", flush=True)
    got = fg.moe_route_contiguous(dev_i32(idx), experts)
    want = moe.route_contiguous(idx, experts)
    for name, g, w in zip(("counts", "m_indices", "token_of_row", "row_of"), got, want):
        assert np.array_equal(host(g), w), name


def test_route_zipf_workload_and_larger_buffer():
    c = workloads.moe_layer(seed=6, tokens=8192, with_weights=False)
    mpm = moe.max_padded_rows(c.tokens, c.topk, c.experts) + 256
    got = fg.moe_route_contiguous(dev_i32(c.topk_idx), c.experts, m_pad_max=mpm)
    want = moe.route_contiguous(c.topk_idx, c.experts, mpm)
    for name, g, w in zip(("counts", "m_indices", "token_of_row", "row_of"), got, want):
        assert np.array_equal(host(g), w), name


# ------------------------------------------------------------ gather + quant
@pytest.mark.parametrize("tokens,hidden,seed", [(100, 256, 0), (333, 640, 1), (64, 7168, 2)])
def test_gather_quantize_bit_exact(tokens, hidden, seed):
    rng = np.random.default_rng(seed)
    x = workloads.activation_bf16(rng, tokens, hidden, outliers=True)
    idx = workloads.zipf_topk_routing(rng, tokens, 8, 3, 1.1).astype(np.int32)
    _, _, tok, _ = moe.route_contiguous(idx, 8)
    q, sa = fg.moe_gather_quantize(to_dev_bf16(x), dev_i32(tok))
    oq, osa = moe.gather_quantize(x, tok)
    m = tok.size
    assert np.array_equal(codes(q), oq)
    assert np.array_equal(bits32(sa[:, :m]), bits32(osa[:, :m]))


@pytest.mark.parametrize(
    "tokens,hidden,experts,topk,seed",
    [(0, 256, 4, 2, 0), (1, 128, 1, 1, 1), (100, 256, 8, 3, 2), (333, 640, 16, 8, 3), (257, 7168, 32, 4, 4)],
)
def test_gather_by_token_equals_gather_by_row(tokens, hidden, experts, topk, seed):
    """The token-major gather (each token read and quantized once, written to
    its rows; the other rows zero codes and scale 1) writes the bytes of the
    row-major gather and of the oracle over every row of the buffer, with
    dropped slots (expert ids outside the range) in the routing."""
    rng = np.random.default_rng(seed)
    x = workloads.activation_bf16(rng, max(tokens, 1), hidden, outliers=True)[:tokens]
    idx = rng.integers(-1, experts + 1, size=(tokens, topk)).astype(np.int32)
    print(f"gather by token: tokens={tokens} hidden={hidden} experts={experts} topk={topk}", flush=True)
    _, _, tok, row_of = fg.moe_route_contiguous(dev_i32(idx), experts)
    xd = to_dev_bf16(x)
    m = tok.shape[0]
    poison = lambda: (torch.full((m, hidden), 0x7F, dtype=torch.uint8, device="cuda").view(torch.float8_e4m3fn),
                      torch.full((hidden // 128, fg.padded_rows(m)), float("nan"), dtype=torch.float32, device="cuda"))
    q1, s1 = fg.moe_gather_quantize(xd, tok, out=poison())
    q2, s2 = fg.moe_gather_quantize_tokens(xd, row_of, tok, out=poison())
    torch.cuda.synchronize()
    assert torch.equal(q2.view(torch.uint8), q1.view(torch.uint8))
    assert np.array_equal(bits32(s2[:, :m]), bits32(s1[:, :m]))
    oq, osa = moe.gather_quantize(x, host(tok))
    assert np.array_equal(codes(q2), oq)
    assert np.array_equal(bits32(s2[:, :m]), bits32(osa[:, :m]))


# ------------------------------------------------------------------ silu_mul
def ordinal(c):
    c = c.astype(np.int32)
    return np.where(c & 0x80, -(c & 0x7F), c & 0x7F)


def check_act(q, sa, oq, osa, m, label):
    kq, ks = codes(q), host(sa)[:, :m]
    os_ = osa[:, :m]
    step = np.abs(ordinal(kq) - ordinal(oq))
    assert step.max(initial=0) <= 1, f"{label}: a code differs by more than one step"
    srel = np.abs(ks.astype(np.float64) - os_) / os_
    assert srel.max(initial=0) <= 2.0**-7, f"{label}: scale off by {srel.max():.2e}"
    frac_codes = float(np.mean(step != 0)) if step.size else 0.0
    frac_scales = float(np.mean(ks != os_)) if ks.size else 0.0
    print(f"{label}: codes differing {frac_codes:.2e}, scales differing {frac_scales:.2e}", flush=True)
    assert frac_codes <= 1e-3 and frac_scales <= 1e-3
    return frac_codes, frac_scales


@pytest.mark.parametrize("m,inter,seed", [(256, 128, 0), (512, 384, 1), (1024, 2048, 2)])
def test_silu_mul_quantize(m, inter, seed):
    rng = np.random.default_rng(seed)
    h = workloads.gaussian_bf16(rng, (m, 2 * inter), 1.7)
    h[:, :7] = workloads.f32_to_bf16_bits(np.array([0.0, -0.0, 90.0, -90.0, 1e-30, 3.0e4, -3.0e4], np.float32))
    m_idx = rng.integers(-1, 4, size=m).astype(np.int32)
    q, sa = fg.silu_mul_quantize(to_dev_bf16(h), dev_i32(m_idx))
    oq, osa = moe.silu_mul_quantize(h, m_idx)
    pad = m_idx < 0
    assert np.all(codes(q)[pad] == 0)
    check_act(q, sa, oq, osa, m, f"silu m={m} I={inter}")


# ------------------------------------------------------------------- combine
@pytest.mark.parametrize("tokens,topk,hidden,seed", [(1, 1, 8, 0), (37, 4, 520, 1), (300, 8, 7168, 2)])
def test_combine_bound(tokens, topk, hidden, seed):
    rng = np.random.default_rng(seed)
    rows = tokens * topk + 5
    y = workloads.gaussian_bf16(rng, (rows, hidden), 1.0)
    row_of = rng.integers(-1, rows, size=(tokens, topk)).astype(np.int32)
    w = rng.random((tokens, topk)).astype(np.float32)
    out = host(fg.moe_combine(to_dev_bf16(y), dev_i32(row_of), torch.from_numpy(w).cuda()).view(torch.int16))
    got = workloads.bf16_bits_to_f32(out.view(np.uint16)).astype(np.float64)
    ref = moe.combine(y, row_of, w)
    yv = workloads.bf16_bits_to_f32(y).astype(np.float64)
    mag = np.zeros_like(ref)
    for j in range(topk):
        live = row_of[:, j] >= 0
        mag[live] += np.abs(w[live, j, None]) * np.abs(yv[row_of[live, j]])
    err = topk * 2.0**-24 * mag
    big = np.abs(ref) + err
    ulp = np.exp2(np.floor(np.log2(np.maximum(big, 2.0**-126))) - 7)
    assert np.all(np.abs(got - ref) <= 0.5 * ulp + err)
    assert np.all(got[row_of.max(axis=1) < 0] == 0)


# ----------------------------------------------------------------- the layer
def device_weights(c):
    q1 = torch.empty((c.experts, 2 * c.inter, c.hidden), dtype=torch.float8_e4m3fn, device="cuda")
    s1 = torch.empty((c.experts, 2 * c.inter // 128, c.hidden // 128), dtype=torch.float32, device="cuda")
    q2 = torch.empty((c.experts, c.hidden, c.inter), dtype=torch.float8_e4m3fn, device="cuda")
    s2 = torch.empty((c.experts, c.hidden // 128, c.inter // 128), dtype=torch.float32, device="cuda")
    for e in range(c.experts):  # per-expert slices of the scales need not be 16-byte aligned: copy
        qa, sa = fg.quantize_fp8_blocks(to_dev_bf16(c.w1[e]))
        q1[e].copy_(qa)
        s1[e].copy_(sa)
        qa, sa = fg.quantize_fp8_blocks(to_dev_bf16(c.w2[e]))
        q2[e].copy_(qa)
        s2[e].copy_(sa)
    return (q1, s1), (q2, s2)


def run_layer_steps(c, w1, w2):
    x = to_dev_bf16(c.x)
    idx = dev_i32(c.topk_idx)
    wts = torch.from_numpy(c.topk_weights).cuda()
    counts, m_idx, tok, row_of = fg.moe_route_contiguous(idx, c.experts)
    a1 = fg.moe_gather_quantize(x, tok)
    m = m_idx.shape[0]
    h = torch.full((m, 2 * c.inter), float("nan"), dtype=torch.bfloat16, device="cuda")
    fg.m_grouped_fp8_gemm_nt_contiguous(a1, w1, h, m_idx)
    a2 = fg.silu_mul_quantize(h, m_idx)
    y = torch.full((m, c.hidden), float("nan"), dtype=torch.bfloat16, device="cuda")
    fg.m_grouped_fp8_gemm_nt_contiguous(a2, w2, y, m_idx)
    out = fg.moe_combine(y, row_of, wts)
    fused = fg.moe_fp8_layer(x, idx, wts, w1, w2)
    # the gate_up product fused with SiLU.mul + quantize, on poisoned outputs
    qf = torch.full((m, c.inter), 0x7F, dtype=torch.uint8, device="cuda").view(torch.float8_e4m3fn)
    sf = torch.full((c.inter // 128, fg.padded_rows(m)), float("nan"), dtype=torch.float32, device="cuda")
    a2f = fg.moe_gate_up_silu_quantize(a1, w1, m_idx, out=(qf, sf))
    torch.cuda.synchronize()
    return dict(counts=counts, m_indices=m_idx, token_of_row=tok, row_of=row_of, a1=a1, h=h, a2=a2, y=y, out=out,
                fused=fused, a2f=a2f)


def check_fused_gate_up(r, m):
    """The fused kernel's activation codes and scales equal the two-step
    path's (grouped product, then silu_mul_quantize) on every row, padding
    blocks included."""
    assert torch.equal(r["a2f"][0].view(torch.uint8), r["a2"][0].view(torch.uint8)), "fused act codes differ"
    assert np.array_equal(bits32(r["a2f"][1][:, :m]), bits32(r["a2"][1][:, :m])), "fused act scales differ"


@pytest.mark.parametrize(
    "tokens,experts,topk,hidden,inter,seed",
    [(256, 8, 4, 512, 256, 0), (77, 5, 2, 384, 384, 1), (300, 16, 6, 256, 128, 2)],
)
def test_layer_parity(tokens, experts, topk, hidden, inter, seed):
    print(f"layer T={tokens} G={experts} top{topk} H={hidden} I={inter}", flush=True)
    c = workloads.moe_layer(seed=100 + seed, experts=experts, tokens=tokens, topk=topk, hidden=hidden, inter=inter)
    w1, w2 = device_weights(c)
    r = run_layer_steps(c, w1, w2)
    ow1 = [oracle.quantize_blocks(c.w1[e]) for e in range(experts)]
    ow2 = [oracle.quantize_blocks(c.w2[e]) for e in range(experts)]
    ow1 = (np.stack([q for q, _ in ow1]), np.stack([s for _, s in ow1]))
    ow2 = (np.stack([q for q, _ in ow2]), np.stack([s for _, s in ow2]))
    assert np.array_equal(codes(w1[0]), ow1[0]) and np.array_equal(bits32(w1[1]), bits32(ow1[1]))
    assert np.array_equal(codes(w2[0]), ow2[0]) and np.array_equal(bits32(w2[1]), bits32(ow2[1]))
    o = moe.moe_layer(c.x, c.topk_idx, c.topk_weights, ow1, ow2, experts)
    for name in ("counts", "m_indices", "token_of_row", "row_of"):
        assert np.array_equal(host(r[name]), o[name]), name
    m = o["m_indices"].size
    assert np.array_equal(codes(r["a1"][0]), o["qa1"])
    assert np.array_equal(bits32(r["a1"][1][:, :m]), bits32(o["sa1"][:, :m]))
    # first product: operands identical on both sides, the product criteria hold per expert
    h = d_to_f64(r["h"])
    for e in range(experts):
        rows = np.nonzero(o["m_indices"] == e)[0]
        if rows.size:
            s = magnitude_sum(o["qa1"][rows], o["sa1"][:, rows], ow1[0][e], ow1[1][e])
            check_gemm(h[rows], o["h64"][rows], s, hidden, f"gate_up expert {e}")
    live = o["m_indices"] >= 0
    kh = host(r["h"].view(torch.int16)).view(np.uint16)
    frac_h = float(np.mean(kh[live] != o["h"][live]))
    # the activation, dequantized (code value times its group's scale)
    t = oracle.e4m3_table()
    ks = host(r["a2"][1])[:, :m]
    deq_k = t[codes(r["a2"][0])] * np.repeat(ks.T.astype(np.float64), 128, axis=1)
    deq_o = t[o["qa2"]] * np.repeat(o["sa2"][:, :m].T.astype(np.float64), 128, axis=1)
    assert np.all(deq_k[~live] == 0)
    rel_a = np.linalg.norm(deq_k - deq_o) / np.linalg.norm(deq_o)
    y = d_to_f64(r["y"])[live]
    rel_y = np.linalg.norm(y - o["y64"][live]) / np.linalg.norm(o["y64"][live])
    out = d_to_f64(r["out"])
    rel = np.linalg.norm(out - o["out"]) / np.linalg.norm(o["out"])
    print(f"layer: h rounded differently {frac_h:.2e}; normwise act {rel_a:.2e}, y {rel_y:.2e}, out {rel:.2e}",
          flush=True)
    assert rel_a <= TOL_LAYER and rel_y <= TOL_LAYER and rel <= TOL_LAYER, (rel_a, rel_y, rel)
    assert torch.equal(r["fused"].view(torch.int16), r["out"].view(torch.int16))
    check_fused_gate_up(r, m)


@pytest.mark.parametrize("tokens,experts,topk,hidden,inter,seed",
                         [(64, 3, 2, 128, 128, 3), (500, 12, 4, 1024, 640, 4), (160, 4, 4, 7168, 2048, 5)])
def test_fused_gate_up_bit_identical(tokens, experts, topk, hidden, inter, seed):
    """moe_gate_up_silu_quantize against the grouped product followed by
    silu_mul_quantize, bit for bit, over expert widths of one to sixteen
    128-column blocks and K of one to 56 chunks."""
    print(f"fused gate_up T={tokens} G={experts} top{topk} H={hidden} I={inter}", flush=True)
    c = workloads.moe_layer(seed=200 + seed, experts=experts, tokens=tokens, topk=topk, hidden=hidden, inter=inter)
    w1, w2 = device_weights(c)
    r = run_layer_steps(c, w1, w2)
    check_fused_gate_up(r, r["m_indices"].shape[0])
    assert torch.equal(r["fused"].view(torch.int16), r["out"].view(torch.int16))


def test_layer_graph_replay():
    """The whole layer captured once in a HIP graph (no host synchronisation
    inside), replayed with new inputs copied into the same buffers."""
    c = workloads.moe_layer(seed=120, experts=8, tokens=256, topk=4, hidden=256, inter=256)
    c2 = workloads.moe_layer(seed=121, experts=8, tokens=256, topk=4, hidden=256, inter=256)
    w1, w2 = device_weights(c)
    x = to_dev_bf16(c.x)
    idx = dev_i32(c.topk_idx)
    wts = torch.from_numpy(c.topk_weights).cuda()
    eager = fg.moe_fp8_layer(x, idx, wts, w1, w2)
    torch.cuda.synchronize()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        fg.moe_fp8_layer(x, idx, wts, w1, w2)  # allocator warm-up on the side stream
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        out = fg.moe_fp8_layer(x, idx, wts, w1, w2)
    for rep in range(3):
        src = c if rep % 2 == 0 else c2
        x.copy_(to_dev_bf16(src.x))
        idx.copy_(dev_i32(src.topk_idx))
        wts.copy_(torch.from_numpy(src.topk_weights).cuda())
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        want = fg.moe_fp8_layer(x, idx, wts, w1, w2)
        torch.cuda.synchronize()
        assert torch.equal(out.view(torch.int16), want.view(torch.int16)), rep
        if rep == 0:
            assert torch.equal(out.view(torch.int16), eager.view(torch.int16))


def test_layer_full_size_sampled():
    """The layer at its workload size (8192 tokens, 32 experts, top-4 by
    Zipf(1.1), H = 7168, I = 2048), in the launch configuration the benchmark
    times: routing bit-exact in full; the gathered operand bit-exact on sampled
    rows; the first product, the activation, y and out on sampled tokens whose
    experts all lie among the six most loaded (so the oracle quantizes six
    experts' weights, not 32)."""
    c = workloads.moe_layer(seed=6)
    print(f"full-size layer {c.name}", flush=True)
    w1, w2 = device_weights(c)
    r = run_layer_steps(c, w1, w2)
    want = moe.route_contiguous(c.topk_idx, c.experts)
    for name, w in zip(("counts", "m_indices", "token_of_row", "row_of"), want):
        assert np.array_equal(host(r[name]), w), name
    counts, m_idx, tok, row_of = want
    m = m_idx.size
    assert torch.equal(r["fused"].view(torch.int16), r["out"].view(torch.int16))
    check_fused_gate_up(r, m)
    rng = np.random.default_rng(0)
    # gathered operand on sampled rows (real and padding)
    rows = np.unique(np.concatenate([rng.choice(m, 64, replace=False), [0, m - 1]]))
    oq, osa = moe.gather_quantize(c.x, tok[rows])
    ri = torch.as_tensor(rows, device="cuda")
    assert np.array_equal(codes(r["a1"][0].view(torch.uint8).index_select(0, ri)), oq)
    assert np.array_equal(bits32(r["a1"][1][:, :m].index_select(1, ri)), bits32(osa[:, : rows.size]))
    # sampled tokens through the whole chain
    experts = 6
    cand = np.nonzero(np.all(c.topk_idx < experts, axis=1))[0]
    toks = np.sort(rng.choice(cand, 12, replace=False))
    ow1 = {e: oracle.quantize_blocks(c.w1[e]) for e in range(experts)}
    ow2 = {e: oracle.quantize_blocks(c.w2[e]) for e in range(experts)}
    t = oracle.e4m3_table()
    out_ref = np.zeros((toks.size, c.hidden))
    out_got = d_to_f64(r["out"].index_select(0, torch.as_tensor(toks, device="cuda")))
    h_all = d_to_f64(r["h"])
    a2q, a2s = codes(r["a2"][0]), host(r["a2"][1])
    y_all = d_to_f64(r["y"])
    act_k, act_o, y_k, y_o = [], [], [], []
    for i, tkn in enumerate(toks):
        for j in range(c.topk):
            e, row = int(c.topk_idx[tkn, j]), int(row_of[tkn, j])
            qa, sa = oracle.quantize_groups(c.x[tkn : tkn + 1])
            h64 = oracle.gemm_nt(qa, sa, *ow1[e])
            check_gemm(h_all[row : row + 1], h64, magnitude_sum(qa, sa, *ow1[e]), c.hidden, f"token {tkn} slot {j}")
            h = oracle.round_to_bf16(h64)
            qa2, sa2 = moe.silu_mul_quantize(h, np.array([e], dtype=np.int32))
            act_o.append(t[qa2[0]] * np.repeat(sa2[:, 0].astype(np.float64), 128))
            act_k.append(t[a2q[row]] * np.repeat(a2s[:, row].astype(np.float64), 128))
            y64 = oracle.gemm_nt(qa2, sa2, *ow2[e])
            y_o.append(y64[0])
            y_k.append(y_all[row])
            out_ref[i] += float(c.topk_weights[tkn, j]) * workloads.bf16_bits_to_f32(
                oracle.round_to_bf16(y64[0])).astype(np.float64)
    rel_a = np.linalg.norm(np.array(act_k) - np.array(act_o)) / np.linalg.norm(np.array(act_o))
    rel_y = np.linalg.norm(np.array(y_k) - np.array(y_o)) / np.linalg.norm(np.array(y_o))
    rel = np.linalg.norm(out_got - out_ref) / np.linalg.norm(out_ref)
    print(f"full-size sampled: normwise act {rel_a:.2e}, y {rel_y:.2e}, out {rel:.2e}", flush=True)
    assert rel_a <= TOL_LAYER and rel_y <= TOL_LAYER and rel <= TOL_LAYER, (rel_a, rel_y, rel)
