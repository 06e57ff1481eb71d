"""GPU parity of m_grouped_fp8_gemm_nt_masked against the oracle.

The activation buffer [G][max_m][K] is quantized as one (G*max_m) x K matrix
(checked bit-exact), the weights expert by expert; every computed row is held
to the product criteria of tests/parity.py, rows past a group's count must
stay untouched (NaN-poisoned output), and a full-groups case must equal the
contiguous grouped kernel bit for bit (same MFMA chunks, same promotion
order)."""

import numpy as np
import pytest
import torch

import fine_grained_block_fp8_amd as fg
import oracle
import workloads
from tests.parity import bits32, check_gemm, codes, d_to_f64, magnitude_sum, to_dev_bf16

pytestmark = pytest.mark.gpu


def gpu_masked(c: workloads.Masked, masked_dev=None, expected_m=None, workspace=None):
    g, mm, n, k = c.num_groups, c.max_m, c.n, c.k
    x = to_dev_bf16(c.a.reshape(g * mm, k))
    q, sa = fg.quantize_fp8_groups(x)
    w = to_dev_bf16(c.b.reshape(g * n, k))
    if n % 128 == 0:
        qb, sb = fg.quantize_fp8_blocks(w)
        qb, sb = qb.view(g, n, k), sb.view(g, n // 128, k // 128)
    else:
        qb = torch.empty((g, n, k), dtype=torch.float8_e4m3fn, device="cuda")
        sb = torch.empty((g, -(-n // 128), k // 128), dtype=torch.float32, device="cuda")
        for e in range(g):  # per expert (a block must not straddle two experts), via aligned temporaries
            qe, se = fg.quantize_fp8_blocks(w[e * n : (e + 1) * n])
            qb[e].copy_(qe)
            sb[e].copy_(se)
    if masked_dev is None:
        masked_dev = torch.from_numpy(c.masked_m.astype(np.int32)).cuda()
    d = torch.full((g, mm, n), float("nan"), dtype=torch.bfloat16, device="cuda")
    fg.m_grouped_fp8_gemm_nt_masked((q.view(g, mm, k), sa), (qb, sb), d, masked_dev,
                                    c.expected_m if expected_m is None else expected_m, workspace=workspace)
    torch.cuda.synchronize()
    return q, sa, qb, sb, d


def check_masked(c, q, sa, qb, sb, d, groups=None, rows_per_group=None, cblocks=None, rng=None):
    rng = rng or np.random.default_rng(0)
    g_all, mm, n, k = c.num_groups, c.max_m, c.n, c.k
    groups = range(g_all) if groups is None else groups
    cblocks = np.arange(-(-n // 128)) if cblocks is None else np.asarray(cblocks)
    cols = np.concatenate([np.arange(b * 128, min(n, b * 128 + 128)) for b in cblocks])
    counts = np.clip(c.masked_m, 0, mm)
    for e in groups:
        rows = np.arange(int(counts[e]))
        if rows_per_group and rows.size > rows_per_group:
            rows = np.unique(np.concatenate([rows[[0, -1]], rng.choice(rows, rows_per_group - 2, replace=False)]))
        buf_rows = e * mm + rows
        if rows.size:
            oq, osa = oracle.quantize_groups(c.a[e][rows])
            oqb, osb = oracle.quantize_blocks(c.b[e][cols])
            ri = torch.as_tensor(buf_rows, device="cuda")
            assert np.array_equal(codes(q.view(torch.uint8).index_select(0, ri)), oq)
            assert np.array_equal(bits32(sa.index_select(1, ri)), bits32(osa[:, : rows.size]))
            assert np.array_equal(codes(qb[e].view(torch.uint8).index_select(0, torch.as_tensor(cols, device="cuda"))), oqb)
            ref = oracle.gemm_nt(oq, osa, oqb, osb)
            got = d_to_f64(d[e].index_select(0, torch.as_tensor(rows, device="cuda")).index_select(1, torch.as_tensor(cols, device="cuda")))
            check_gemm(got, ref, magnitude_sum(oq, osa, oqb, osb), k, f"group {e}")
        # rows past the count are never written
        assert torch.isnan(d[e, int(counts[e]):].float()).all(), f"group {e}: rows past masked_m written"


@pytest.mark.parametrize(
    "counts,max_m,n,k",
    [
        ([0, 137, 200], 200, 264, 384),
        ([64, 1, 17, 0, 33], 64, 128, 256),
        ([300, 129, 128, 256], 300, 512, 640),
        ([5], 8, 16, 128),
    ],
)
def test_small_masked_cases(counts, max_m, n, k):
    c = workloads.small_masked(counts, max_m, n, k, seed=sum(counts) + max_m + n + k)
    q, sa, qb, sb, d = gpu_masked(c)
    check_masked(c, q, sa, qb, sb, d)


@pytest.mark.parametrize("tile", ["tile128x256_w2x4", "tile128x128_w2x2"])
@pytest.mark.parametrize("counts,max_m,n,k", [([0, 137, 200], 200, 264, 384), ([300, 129, 128, 256], 300, 520, 640)])
def test_each_masked_tile(tile, counts, max_m, n, k, monkeypatch, capfd):
    """Both 128-row tiles forced on ragged shapes (N not a multiple of the
    tile width, counts that end inside a tile)."""
    monkeypatch.setenv("FGFP8_MASKED_TILE", tile)
    monkeypatch.setenv("FGFP8_PRINT_CONFIG", "1")
    c = workloads.small_masked(counts, max_m, n, k, seed=sum(counts) + n + 3)
    q, sa, qb, sb, d = gpu_masked(c)
    lines = [ln for ln in capfd.readouterr().err.splitlines() if "m_grouped_fp8_gemm_nt_masked" in ln]
    assert lines and lines[-1].endswith(tile), lines
    check_masked(c, q, sa, qb, sb, d)


def test_oracle_function_agrees_on_a_small_case():
    """The oracle's masked form itself (folded scale columns) on the GPU's
    quantized bytes."""
    c = workloads.small_masked([3, 0, 8], 8, 136, 256, seed=71)
    q, sa, qb, sb, d = gpu_masked(c)
    g, mm, n, k = c.num_groups, c.max_m, c.n, c.k
    ref = oracle.masked_grouped_gemm_nt(codes(q).reshape(g, mm, k), sa.cpu().numpy(), c.masked_m,
                                        codes(qb).reshape(g, n, k), sb.cpu().numpy())
    got = d_to_f64(d.reshape(g * mm, n)).reshape(g, mm, n)
    qa_all, sa_all = codes(q).reshape(g, mm, k), sa.cpu().numpy()
    qb_all, sb_all = codes(qb).reshape(g, n, k), sb.cpu().numpy()
    for e in range(g):
        r = int(c.masked_m[e])
        if r:
            s = magnitude_sum(qa_all[e, :r], sa_all[:, e * mm : e * mm + r], qb_all[e], sb_all[e])
            check_gemm(got[e, :r], ref[e, :r], s, k, f"group {e}")


def test_counts_outside_range_are_clamped():
    c = workloads.small_masked([-3, 40, 7], 32, 128, 256, seed=73)
    q, sa, qb, sb, d = gpu_masked(c)
    c2 = workloads.Masked(c.name, c.num_groups, c.max_m, c.n, c.k, np.array([0, 32, 7], np.int32), c.expected_m, c.a, c.b)
    check_masked(c2, q, sa, qb, sb, d)


@pytest.mark.parametrize("expected_m", [1, 128, 4096])
def test_full_groups_equal_contiguous_bitwise(expected_m):
    """max_m a multiple of 128 and every group full: the buffer is the
    contiguous layout, and the results must be the same bits whatever tile the
    hint selects."""
    c = workloads.small_masked([256, 256, 256], 256, 384, 512, seed=79)
    q, sa, qb, sb, d = gpu_masked(c, expected_m=expected_m)
    idx = torch.repeat_interleave(torch.arange(3, dtype=torch.int32, device="cuda"), 256)
    d2 = torch.full((768, c.n), float("nan"), dtype=torch.bfloat16, device="cuda")
    fg.m_grouped_fp8_gemm_nt_contiguous((q, sa), (qb, sb), d2, idx)
    torch.cuda.synchronize()
    assert torch.equal(d.reshape(768, c.n).view(torch.int16), d2.view(torch.int16))


def test_decode_moe_dispatch_buffer_sampled():
    """The 32-expert, K = 7168, N = 4096 decode dispatch buffer (1024 tokens,
    Zipf(1.1) top-4): sampled rows of several groups against the oracle."""
    c = workloads.moe_masked()
    q, sa, qb, sb, d = gpu_masked(c)
    rng = np.random.default_rng(11)
    check_masked(c, q, sa, qb, sb, d, groups=[0, 1, 7, 20, 31], rows_per_group=6, cblocks=[0, 13, 31], rng=rng)
    for e in range(c.num_groups):
        assert torch.isfinite(d[e, : int(c.masked_m[e])].float()).all()


# ------------------------------------------------ the workspace (tail-split) form


def tail_split_tiles(counts, max_m, n, k, bn, grid):
    """The tiles the workspace form splits along K, by the rule its header
    states: live tiles (128-row tiles below each count, group order, column
    tile fastest) dealt to `grid` workgroups; the last round's r tiles split
    into min(grid // r, 8, K/128) parts when that is at least 2."""
    tiles_n = -(-n // bn)
    rows = np.clip(np.asarray(counts), 0, max_m)
    order = [(g, tm, tn) for g in range(len(rows)) for tm in range(-(-int(rows[g]) // 128)) for tn in range(tiles_n)]
    rem = len(order) % grid
    parts = min(grid // rem if rem else 1, 8, k // 128)
    return (set(order[len(order) - rem:]) if parts >= 2 else set()), parts


def masked_grid():
    return min(torch.cuda.get_device_properties(0).multi_processor_count, 256)


@pytest.mark.parametrize(
    "counts,max_m,n,k",
    [
        ([0, 137, 200], 200, 264, 384),
        ([64, 1, 17, 0, 33], 64, 128, 256),
        ([300, 129, 128, 256], 300, 512, 640),
        ([5], 8, 16, 128),
        ([900, 0, 3, 894, 260], 900, 4096, 1024),  # several whole rounds before the split one
        (np.random.default_rng(5).integers(-3, 200, 70).tolist(), 196, 384, 512),
    ],
)
def test_tail_split_matches_oracle_and_is_deterministic(counts, max_m, n, k, capfd, monkeypatch):
    """The split walk (forced) against the oracle on ragged cases (few live
    tiles, so the whole launch is one split round; several whole rounds
    before the split one; 70 groups, past the 64 held in registers), twice
    in a row on one workspace: the same bits both times, and every tile the
    rule does not split equal to the plain call bit for bit."""
    monkeypatch.setenv("FGFP8_PRINT_CONFIG", "1")
    monkeypatch.setenv("FGFP8_MASKED_SPLIT", "1")
    c = workloads.small_masked(counts, max_m, n, k, seed=sum(counts) + max_m + n + k + 1)
    ws = fg.masked_workspace(c.num_groups, c.max_m, c.n, c.k)
    q, sa, qb, sb, d = gpu_masked(c, workspace=ws)
    line = [ln for ln in capfd.readouterr().err.splitlines() if "m_grouped_fp8_gemm_nt_masked_ws" in ln][-1]
    assert "tail-split" in line, line
    check_masked(c, q, sa, qb, sb, d)
    masked_dev = torch.from_numpy(c.masked_m.astype(np.int32)).cuda()
    d2 = torch.full_like(d, float("nan"))
    fg.m_grouped_fp8_gemm_nt_masked((q.view(c.num_groups, c.max_m, c.k), sa), (qb, sb), d2, masked_dev, c.expected_m,
                                    workspace=ws)
    d3 = torch.full_like(d, float("nan"))
    fg.m_grouped_fp8_gemm_nt_masked((q.view(c.num_groups, c.max_m, c.k), sa), (qb, sb), d3, masked_dev, c.expected_m)
    torch.cuda.synchronize()
    assert torch.equal(d.view(torch.int16), d2.view(torch.int16)), "the workspace form is not deterministic"
    bn = 256 if line.endswith("tile128x256_w2x4") else 128
    split, parts = tail_split_tiles(c.masked_m, c.max_m, c.n, c.k, bn, masked_grid())
    same = torch.ones(d.shape, dtype=torch.bool, device="cuda")
    for g, tm, tn in split:
        same[g, tm * 128 : tm * 128 + 128, tn * bn : tn * bn + bn] = False
    a, b = d.view(torch.int16), d3.view(torch.int16)
    assert torch.equal(a[same], b[same]), "a tile that is not split differs from the plain call"


def test_tail_split_zipf_dispatch_buffer(monkeypatch):
    """The split walk (forced) on the 32-expert, K = 7168, N = 4096 decode
    dispatch buffer (1024 tokens, Zipf(1.1) top-4): 800 live tiles, so three
    whole rounds and 32 tiles split in 8.  Every split tile against the
    oracle (all its columns, sampled rows), sampled rows of other groups, the
    untouched rows past the counts, and the tiles that are not split equal to
    the plain call bit for bit."""
    monkeypatch.setenv("FGFP8_MASKED_SPLIT", "1")
    c = workloads.moe_masked()
    ws = fg.masked_workspace(c.num_groups, c.max_m, c.n, c.k)
    q, sa, qb, sb, d = gpu_masked(c, workspace=ws)
    split, parts = tail_split_tiles(c.masked_m, c.max_m, c.n, c.k, 256, masked_grid())
    if masked_grid() == 256:
        assert len(split) == 32 and parts == 8
    groups = sorted({g for g, _, _ in split} | {0, 7})
    rng = np.random.default_rng(13)
    check_masked(c, q, sa, qb, sb, d, groups=groups, rows_per_group=8, rng=rng)
    d3 = torch.full_like(d, float("nan"))
    masked_dev = torch.from_numpy(c.masked_m.astype(np.int32)).cuda()
    fg.m_grouped_fp8_gemm_nt_masked((q.view(c.num_groups, c.max_m, c.k), sa), (qb, sb), d3, masked_dev, c.expected_m)
    torch.cuda.synchronize()
    same = torch.ones(d.shape, dtype=torch.bool, device="cuda")
    for g, tm, tn in split:
        same[g, tm * 128 : tm * 128 + 128, tn * 256 : tn * 256 + 256] = False
    assert torch.equal(d.view(torch.int16)[same], d3.view(torch.int16)[same])
    for e in range(c.num_groups):
        assert torch.isfinite(d[e, : int(c.masked_m[e])].float()).all()


def test_tail_split_workspace_reused_by_a_smaller_call(monkeypatch):
    """One workspace for two different calls in a row (the second smaller):
    each call leaves the counters at zero for the next."""
    monkeypatch.setenv("FGFP8_MASKED_SPLIT", "1")
    ws = fg.masked_workspace(4, 300, 512, 640)
    for counts, max_m, n, k in (([300, 129, 128, 256], 300, 512, 640), ([0, 37, 5], 40, 136, 256)):
        c = workloads.small_masked(counts, max_m, n, k, seed=max_m + n)
        q, sa, qb, sb, d = gpu_masked(c, workspace=ws)
        check_masked(c, q, sa, qb, sb, d)
    assert int(ws[:1024].view(torch.int32).abs().sum().item()) == 0


def test_workspace_form_walks_only_small_dispatches(capfd, monkeypatch):
    """By default the workspace form walks and splits only where the expected
    live tiles fill at most a quarter of the CUs: 2 groups of 16 expected rows
    at N = 4096 (32 tiles) walk, 32 groups of 128 (512 tiles) run the plain
    kernel -- with the plain call's bits."""
    monkeypatch.setenv("FGFP8_PRINT_CONFIG", "1")
    for groups, em, walk in ((2, 16, True), (32, 128, False)):
        c = workloads.small_masked([em] * groups, 128, 4096, 256, seed=groups)
        c = workloads.Masked(c.name, c.num_groups, c.max_m, c.n, c.k, c.masked_m, em, c.a, c.b)
        ws = fg.masked_workspace(c.num_groups, c.max_m, c.n, c.k)
        q, sa, qb, sb, d = gpu_masked(c, workspace=ws)
        line = [ln for ln in capfd.readouterr().err.splitlines() if "m_grouped_fp8_gemm_nt_masked_ws" in ln][-1]
        assert ("tail-split" in line) == walk, line
        check_masked(c, q, sa, qb, sb, d, rows_per_group=6, cblocks=[0, 17, 31])
        if not walk:
            d3 = torch.full_like(d, float("nan"))
            fg.m_grouped_fp8_gemm_nt_masked((q.view(c.num_groups, c.max_m, c.k), sa), (qb, sb), d3,
                                            torch.from_numpy(c.masked_m.astype(np.int32)).cuda(), em)
            torch.cuda.synchronize()
            assert torch.equal(d.view(torch.int16), d3.view(torch.int16))


# ------------------------------------------- quantizing the real rows only


@pytest.mark.parametrize(
    "counts,max_m,k",
    [([0, 137, 200], 200, 384), ([64, 1, 17, 0, 33], 64, 256), ([-3, 40, 7, 32], 32, 640), ([5], 8, 128),
     ([896, 0, 3, 894], 896, 7168),
     # 1024 groups: the most the prefix-sum form takes; 1100: the one-wave-per-block form
     (np.random.default_rng(6).integers(-2, 7, 1024).tolist(), 4, 128),
     (np.random.default_rng(7).integers(-2, 11, 1100).tolist(), 8, 256)],
)
def test_masked_quantizer_bit_exact_and_leaves_other_rows(counts, max_m, k):
    g = len(counts)
    rng = np.random.default_rng(g + max_m + k)
    x = workloads.activation_bf16(rng, g * max_m, k, outliers=True)
    xd = to_dev_bf16(x).view(g, max_m, k)
    mm = torch.tensor(counts, dtype=torch.int32, device="cuda")
    sa_ld = fg.padded_rows(g * max_m)
    q = torch.full((g, max_m, k), 0x7F, dtype=torch.uint8, device="cuda").view(torch.float8_e4m3fn)
    sa = torch.full((k // 128, sa_ld), float("nan"), dtype=torch.float32, device="cuda")
    fg.quantize_fp8_groups_masked(xd, mm, out=(q, sa))
    torch.cuda.synchronize()
    qc, sc = codes(q).reshape(g, max_m, k), sa.cpu().numpy()
    for e, c in enumerate(np.clip(counts, 0, max_m)):
        if c:
            oq, osa = oracle.quantize_groups(x[e * max_m : e * max_m + c])
            assert np.array_equal(qc[e, :c], oq), f"group {e}"
            assert np.array_equal(bits32(sc[:, e * max_m : e * max_m + c]), bits32(osa[:, :c])), f"group {e}"
        assert np.all(qc[e, c:] == 0x7F), f"group {e}: rows past the count written"
        assert np.all(np.isnan(sc[:, e * max_m + c : (e + 1) * max_m])), f"group {e}: scales past the count written"


def test_masked_quantizer_then_product_equals_full_buffer_path():
    """The decode dispatch buffer: quantizing only the real rows gives the
    masked product the same bits as quantizing the whole buffer."""
    c = workloads.moe_masked()
    q, sa, qb, sb, d = gpu_masked(c)
    g, mm, n, k = c.num_groups, c.max_m, c.n, c.k
    masked_dev = torch.from_numpy(c.masked_m.astype(np.int32)).cuda()
    x = to_dev_bf16(c.a.reshape(g * mm, k)).view(g, mm, k)
    q2, sa2 = fg.quantize_fp8_groups_masked(x, masked_dev)
    d2 = torch.full((g, mm, n), float("nan"), dtype=torch.bfloat16, device="cuda")
    fg.m_grouped_fp8_gemm_nt_masked((q2, sa2), (qb, sb), d2, masked_dev, c.expected_m)
    torch.cuda.synchronize()
    assert torch.equal(d2.view(torch.int16), d.view(torch.int16))
    for e in (0, 9, 31):
        r = int(c.masked_m[e])
        assert torch.equal(q2[e, :r].view(torch.uint8), q.view(g, mm, k)[e, :r].view(torch.uint8))
