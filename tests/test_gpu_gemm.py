"""GPU parity of fp8_gemm_nt against the oracle run on the same quantized
inputs (the quantized bytes are first checked bit-exact).  Criteria: the
normwise relative error <= 2e-3 and the elementwise FP32-order bound
(tests/parity.py); determinism; NaN-poisoned outputs and guard bands."""

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
    check_full,
    check_gemm,
    check_sampled,
    codes,
    d_to_f64,
    gpu_hot_path,
    magnitude_sum,
    one_row_per_band,
    sample_col_blocks,
    sample_rows,
    to_dev_bf16,
    to_dev_u8_fp8,
)

pytestmark = pytest.mark.gpu


def full_check(lin, label):
    q, sa, qb, sb, d = gpu_hot_path(lin)
    rows = np.arange(lin.m)
    cblocks = np.arange(-(-lin.n // 128))
    return check_sampled(lin, q, sa, qb, sb, d, rows, cblocks, label)


def test_single_linear_128x256x512():
    r = full_check(workloads.single_linear(), "128x256x512")
    assert r["frac_not_bf16_rne"] < 0.05


@pytest.mark.parametrize("seed", [11, 12])
def test_single_linear_other_seeds(seed):
    full_check(workloads.single_linear(seed), f"single seed {seed}")


@pytest.mark.parametrize(
    "m,n,k",
    [
        (1, 128, 128),
        (3, 200, 768),
        (5, 16, 256),
        (16, 1, 128),
        (17, 136, 128),
        (127, 264, 384),
        (129, 520, 768),
        (256, 512, 768),
        (300, 384, 1024),
        (520, 1000, 512),
    ],
)
def test_odd_shapes(m, n, k):
    full_check(workloads.random_linear(m, n, k, seed=m * 7 + n + k), f"{m}x{n}x{k}")


@pytest.mark.parametrize("name", ["qkv", "o", "gate_up", "down"])
def test_prefill_linears_full(name):
    """Every output of each prefill linear against the oracle (all tiles of
    the launch the bench times)."""
    (lin,) = workloads.prefill_linears(names=[name])
    print(f"prefill {lin.name}: {fg.describe_gemm(lin.m, lin.n, lin.k)}", flush=True)
    q, sa, qb, sb, d = gpu_hot_path(lin)
    r = check_full(lin, q, sa, qb, sb, d, lin.name)
    assert r["frac_not_bf16_rne"] < 0.05


@pytest.mark.parametrize("m", [1, 4, 16])
@pytest.mark.parametrize("n,k", workloads.DECODE_SHAPES)
def test_decode_linears_full(m, n, k):
    lin = workloads.decode_linear(m, n, k)
    q, sa, qb, sb, d = gpu_hot_path(lin)
    check_full(lin, q, sa, qb, sb, d, lin.name)


def test_square_8192_full():
    """Every output of the 8192^3 product against the oracle."""
    lin = workloads.square_linear(8192, 8192, 8192)
    print(f"square {lin.name}: {fg.describe_gemm(lin.m, lin.n, lin.k)}", flush=True)
    q, sa, qb, sb, d = gpu_hot_path(lin)
    check_full(lin, q, sa, qb, sb, d, lin.name)


def test_square_16384_every_tile():
    """M = N = 16384, K = 8192: every output column of one row from each
    64-row band (the height of a wave's tile), so every output tile of the
    launch -- every 256x256 workgroup tile and every 64-row wave tile in it --
    is compared with the oracle; every output is checked to be written."""
    m = n = 16384
    k = 8192
    lin = workloads.square_linear(m, n, k)
    print(f"square {lin.name}: {fg.describe_gemm(m, n, k)}", flush=True)
    q, sa, qb, sb, d = gpu_hot_path(lin)
    assert torch.isfinite(d.float()).all(), "unwritten or non-finite outputs"
    rows = one_row_per_band(np.arange(m), 64, np.random.default_rng(3))
    assert rows.size == m // 64
    oqb, osb = oracle_workers.quantize_blocks(lin.b)
    assert np.array_equal(codes(qb), oqb), "weight codes differ"
    assert np.array_equal(bits32(sb), bits32(osb)), "weight scales differ"
    oq, osa = oracle.quantize_groups(lin.a[rows])
    ri = torch.as_tensor(rows, device=d.device)
    assert np.array_equal(codes(q.view(torch.uint8).index_select(0, ri)), oq), "activation codes differ"
    assert np.array_equal(bits32(sa[:, :m].index_select(1, ri)), bits32(osa[:, : rows.size])), "scales differ"
    got = d_to_f64(d.index_select(0, ri))
    assert_stats(oracle_workers.product_stats(oq, osa, oqb, osb, got, k, piece=32), lin.name)


def test_constant_scales_closed_form():
    """Hand-set scales (0.01 / 0.02, deepgemm-rust quick start) on random codes:
    exercises the GEMM alone with scales the quantizer did not produce."""
    rng = np.random.default_rng(17)
    m, n, k = 96, 272, 640
    finite = np.array([c for c in range(256) if c not in (0x7F, 0xFF)], dtype=np.uint8)
    qa = rng.choice(finite, size=(m, k)).astype(np.uint8)
    qb = rng.choice(finite, size=(n, k)).astype(np.uint8)
    sa = np.full((k // 128, m), 0.01, np.float32)
    sb = np.full((-(-n // 128), k // 128), 0.02, np.float32)
    d = torch.full((m, n), float("nan"), dtype=torch.bfloat16, device="cuda")
    fg.fp8_gemm_nt((to_dev_u8_fp8(qa), torch.from_numpy(sa).cuda()), (to_dev_u8_fp8(qb), torch.from_numpy(sb).cuda()), d)
    ref = oracle.gemm_nt(qa, sa, qb, sb)
    check_gemm(d_to_f64(d), ref, magnitude_sum(qa, sa, qb, sb), k, "constant scales")


def test_distinct_scales_per_row_chunk_and_block():
    """Random scales spanning 2^-12..2^4, different for every (chunk, row) and
    (column block, chunk): a transposed or shifted scale index fails."""
    rng = np.random.default_rng(23)
    m, n, k = 200, 392, 1024
    finite = np.array([c for c in range(256) if c not in (0x7F, 0xFF)], dtype=np.uint8)
    qa = rng.choice(finite, size=(m, k)).astype(np.uint8)
    qb = rng.choice(finite, size=(n, k)).astype(np.uint8)
    sa = (rng.random((k // 128, 200)) * 2.0 ** rng.integers(-12, 4, size=(k // 128, 200))).astype(np.float32)
    sb = (rng.random((4, k // 128)) * 2.0 ** rng.integers(-12, 4, size=(4, k // 128))).astype(np.float32)
    d = torch.full((m, n), float("nan"), dtype=torch.bfloat16, device="cuda")
    fg.fp8_gemm_nt((to_dev_u8_fp8(qa), torch.from_numpy(sa).cuda()), (to_dev_u8_fp8(qb), torch.from_numpy(sb).cuda()), d)
    ref = oracle.gemm_nt(qa, sa, qb, sb)
    check_gemm(d_to_f64(d), ref, magnitude_sum(qa, sa, qb, sb), k, "distinct scales")


def test_deterministic_and_guarded():
    lin = workloads.random_linear(300, 520, 768, seed=99)
    q, sa, qb, sb, d1 = gpu_hot_path(lin)
    guard = 8192
    buf = torch.full((lin.m * lin.n + guard,), float("nan"), dtype=torch.bfloat16, device="cuda")
    d2 = buf[: lin.m * lin.n].view(lin.m, lin.n)
    fg.fp8_gemm_nt((q, sa), (qb, sb), d2)
    torch.cuda.synchronize()
    assert torch.isnan(buf[lin.m * lin.n :].float()).all(), "write past the end of d"
    assert torch.equal(d1.view(torch.int16), d2.view(torch.int16)), "two runs differ"


def test_linear_helper_matches_two_calls():
    lin = workloads.random_linear(33, 256, 512, seed=5)
    q, sa, qb, sb, d = gpu_hot_path(lin)
    x = torch.from_numpy(lin.a.view(np.int16)).view(torch.bfloat16).cuda()
    y = fg.fp8_linear(x.view(3, 11, 512), (qb, sb))
    torch.cuda.synchronize()
    assert torch.equal(y.reshape(33, 256).view(torch.int16), d.view(torch.int16))


def test_runs_on_a_side_stream():
    lin = workloads.random_linear(64, 256, 256, seed=6)
    q, sa, qb, sb, d = gpu_hot_path(lin)
    s = torch.cuda.Stream()
    d2 = torch.empty_like(d)
    with torch.cuda.stream(s):
        fg.fp8_gemm_nt((q, sa), (qb, sb), d2)
    s.synchronize()
    assert torch.equal(d.view(torch.int16), d2.view(torch.int16))


@pytest.mark.parametrize("m", [1, 2, 3, 4, 5, 8, 13, 16])
@pytest.mark.parametrize("n,k", [(12288, 4096), (4096, 12288), (200, 384), (1000, 128)])
def test_fused_linear_matches_two_calls_and_oracle(m, n, k):
    """fp8_linear_nt (one fused kernel for m <= 4, and for m <= 16 without the
    activation outputs) writes the same quantized activation as
    quantize_fp8_groups (checked bit-exact against the oracle) and the same
    output bits as quantize_fp8_groups + fp8_gemm_nt."""
    lin = workloads.decode_linear(m, n, k) if (n, k) in workloads.DECODE_SHAPES else workloads.random_linear(m, n, k, seed=m + n)
    q, sa, qb, sb, d_two = gpu_hot_path(lin)
    x = torch.from_numpy(lin.a.view(np.int16)).view(torch.bfloat16).cuda()
    d = torch.full((m, n), float("nan"), dtype=torch.bfloat16, device="cuda")
    q2 = torch.full((m, k), 0x7F, dtype=torch.uint8, device="cuda").view(torch.float8_e4m3fn)
    sa2 = torch.full((k // 128, fg.padded_rows(m)), float("nan"), dtype=torch.float32, device="cuda")
    fg.fp8_linear_nt(x, (qb, sb), d, (q2, sa2))
    torch.cuda.synchronize()
    oq, osa = oracle.quantize_groups(lin.a)
    assert np.array_equal(codes(q2), oq)
    assert np.array_equal(sa2[:, :m].cpu().numpy().view(np.uint32), osa[:, :m].view(np.uint32))
    assert torch.equal(d.view(torch.int16), d_two.view(torch.int16)), "fused output differs from the two-call path"
    # and without the optional activation outputs (for m > 4 the
    # register-quantizing fused kernel)
    d3 = torch.full((m, n), float("nan"), dtype=torch.bfloat16, device="cuda")
    fg.fp8_linear_nt(x, (qb, sb), d3)
    torch.cuda.synchronize()
    assert torch.equal(d3.view(torch.int16), d_two.view(torch.int16))
    rng = np.random.default_rng(5)
    check_sampled(lin, q, sa, qb, sb, d, np.arange(m), sample_col_blocks(n, 8, rng), f"fused {m}x{n}x{k}")


@pytest.mark.parametrize("m", [1, 3, 4, 8, 16])
@pytest.mark.parametrize("n,k", [(12288, 4096), (4096, 12288), (1000, 384)])
def test_register_quantizing_kernel_at_small_m(m, n, k, monkeypatch):
    """The register-quantizing fused kernel forced at m <= 4 (where the LDS
    form is the default): its quantized activation outputs (written by
    workgroup 0) are the oracle's bit for bit, and its product is the
    two-call path's bits."""
    monkeypatch.setenv("FGFP8_DECODE_XQ", "1")
    lin = workloads.decode_linear(m, n, k) if (n, k) in workloads.DECODE_SHAPES else workloads.random_linear(m, n, k, seed=m + n)
    q, sa, qb, sb, d_two = gpu_hot_path(lin)
    x = to_dev_bf16(lin.a)
    d = torch.full((m, n), float("nan"), dtype=torch.bfloat16, device="cuda")
    q2 = torch.full((m, k), 0x7F, dtype=torch.uint8, device="cuda").view(torch.float8_e4m3fn)
    sa2 = torch.full((k // 128, fg.padded_rows(m)), float("nan"), dtype=torch.float32, device="cuda")
    fg.fp8_linear_nt(x, (qb, sb), d, (q2, sa2))
    torch.cuda.synchronize()
    oq, osa = oracle.quantize_groups(lin.a)
    assert np.array_equal(codes(q2), oq)
    assert np.array_equal(sa2[:, :m].cpu().numpy().view(np.uint32), osa[:, :m].view(np.uint32))
    assert torch.equal(d.view(torch.int16), d_two.view(torch.int16))


@pytest.mark.parametrize("m", [1, 4, 13, 16])
@pytest.mark.parametrize("n,k", [(12288, 4096), (1040, 4096), (1000, 2048)])
def test_decode_three_slabs_per_workgroup(m, n, k, monkeypatch):
    """Three 16-column slabs per workgroup (FGFP8_DECODE_SLABS=3; 1040
    columns leave the last workgroup one slab past N, 1000 end in a slab of
    8 columns): every output against the oracle, and the fused forms (with
    the activation outputs for m <= 4, and the fused kernel fp8_linear_nt
    picks without them) give the two-call path's bits."""
    monkeypatch.setenv("FGFP8_DECODE_SLABS", "3")
    desc = fg.describe_gemm(m, n, k)
    print(f"decode {m}x{n}x{k}: {desc}", flush=True)
    assert "slabs=3" in desc
    lin = workloads.decode_linear(m, n, k) if (n, k) in workloads.DECODE_SHAPES else workloads.random_linear(m, n, k, seed=m + n)
    q, sa, qb, sb, d_two = gpu_hot_path(lin)
    check_full(lin, q, sa, qb, sb, d_two, f"slabs3 {m}x{n}x{k}")
    x = to_dev_bf16(lin.a)
    if m <= 4:
        d = torch.full((m, n), float("nan"), dtype=torch.bfloat16, device="cuda")
        q2 = torch.full((m, k), 0x7F, dtype=torch.uint8, device="cuda").view(torch.float8_e4m3fn)
        sa2 = torch.full((k // 128, fg.padded_rows(m)), float("nan"), dtype=torch.float32, device="cuda")
        fg.fp8_linear_nt(x, (qb, sb), d, (q2, sa2))
        torch.cuda.synchronize()
        assert np.array_equal(codes(q2), codes(q))
        assert torch.equal(d.view(torch.int16), d_two.view(torch.int16))
    d3 = torch.full((m, n), float("nan"), dtype=torch.bfloat16, device="cuda")
    fg.fp8_linear_nt(x, (qb, sb), d3)
    torch.cuda.synchronize()
    assert torch.equal(d3.view(torch.int16), d_two.view(torch.int16))


@pytest.mark.parametrize("m,n,k,force3", [(5, 12288, 4096, False), (8, 12288, 4096, False), (16, 12288, 4096, False),
                                           (13, 1040, 4096, True), (16, 1040, 2048, True), (6, 1040, 8192, True),
                                           (11, 1000, 2048, True),
                                           (16, 2048, 4096, False), (16, 4096, 12288, False)])
def test_fused_three_slab_lds_form(m, n, k, force3, monkeypatch, capfd):
    """fp8_linear_nt at 4 < m <= 16, with and without the activation
    outputs: the path it takes is the one describe_linear names (the
    three-slab kernel that quantizes all rows into LDS where it applies,
    FGFP8_DECODE_SLABS=3 forcing three slabs on the ragged 1040-column
    weights), its output is the oracle's element by element and the two-call
    path's bit for bit, and the activation outputs (each (row, group) written
    by one workgroup) are the oracle's quantizer's."""
    monkeypatch.setenv("FGFP8_PRINT_CONFIG", "1")
    if force3:
        monkeypatch.setenv("FGFP8_DECODE_SLABS", "3")
    lin = workloads.decode_linear(m, n, k) if (n, k) in workloads.DECODE_SHAPES else workloads.random_linear(m, n, k, seed=m + n + k)
    q, sa, qb, sb, d_two = gpu_hot_path(lin)
    x = to_dev_bf16(lin.a)
    oq, osa = oracle.quantize_groups(lin.a)
    for act in (True, False):
        form = fg.describe_linear(m, n, k, act)
        d = torch.full((m, n), float("nan"), dtype=torch.bfloat16, device="cuda")
        out = None
        if act:
            out = (torch.full((m, k), 0x7F, dtype=torch.uint8, device="cuda").view(torch.float8_e4m3fn),
                   torch.full((k // 128, fg.padded_rows(m)), float("nan"), dtype=torch.float32, device="cuda"))
        capfd.readouterr()
        fg.fp8_linear_nt(x, (qb, sb), d, out)
        torch.cuda.synchronize()
        err = capfd.readouterr().err
        print(f"fused {m}x{n}x{k} act={act}: {form} | {err.strip()}", flush=True)
        if form.startswith("fused"):
            assert form.split("form=")[1] in err, (form, err)
        wide = "form=lds16" in form
        assert wide == ("slabs=3" in fg.describe_gemm(m, n, k) and m * k // 128 <= (256 if act else 512)), form
        if act:
            assert np.array_equal(codes(out[0]), oq)
            assert np.array_equal(out[1][:, :m].cpu().numpy().view(np.uint32), osa[:, :m].view(np.uint32))
        assert torch.equal(d.view(torch.int16), d_two.view(torch.int16)), f"{form}: output differs from the two-call path"
        if wide and act:
            check_full(lin, q, sa, qb, sb, d, f"fused lds16 {m}x{n}x{k}")


TILES = ["tile256x256_w4x2", "tile256x192_w4x3", "tile256x128_w4x2", "tile128x256_w2x4", "tile128x128_w2x2"]
# the persistent walk takes tiles of whole 128-column blocks
PERSISTENT_TILES = [t for t in TILES if t != "tile256x192_w4x3"]


@pytest.mark.parametrize("tile", TILES)
@pytest.mark.parametrize("m,n,k", [(17, 136, 128), (200, 300, 256), (129, 1000, 384), (300, 520, 768), (513, 264, 1152)])
def test_every_tile_config(tile, m, n, k, monkeypatch):
    """Each tile configuration, forced through FGFP8_GEMM_TILE, on shapes with
    ragged M, N edges and several K chunks."""
    monkeypatch.setenv("FGFP8_GEMM_TILE", tile)
    assert fg.describe_gemm(m, n, k).startswith(tile)
    full_check(workloads.random_linear(m, n, k, seed=m + 3 * n + k), f"{tile} {m}x{n}x{k}")


@pytest.mark.parametrize("m,n,k", [(300, 520, 768), (512, 768, 512)])
def test_tiles_give_identical_bits(m, n, k, monkeypatch):
    """Every output element takes the same MFMA chunks and the same promotion
    order whatever the tile, so all tile configurations give the same bits
    (a staging or indexing slip in one of them breaks this at once)."""
    lin = workloads.random_linear(m, n, k, seed=7)
    outs = {}
    for tile in TILES:
        monkeypatch.setenv("FGFP8_GEMM_TILE", tile)
        outs[tile] = gpu_hot_path(lin)[-1]
    for tile in TILES[1:]:
        assert torch.equal(outs[tile].view(torch.int16), outs[TILES[0]].view(torch.int16)), tile


@pytest.mark.parametrize("tile", TILES)
def test_every_tile_config_prefill_o(tile, monkeypatch):
    monkeypatch.setenv("FGFP8_GEMM_TILE", tile)
    (lin,) = workloads.prefill_linears(names=["o"])
    q, sa, qb, sb, d = gpu_hot_path(lin)
    rng = np.random.default_rng(7)
    check_sampled(lin, q, sa, qb, sb, d, sample_rows(lin.m, 24, rng), sample_col_blocks(lin.n, 6, rng), f"o {tile}")


def test_graph_replays_match_eager():
    """The calls are legal under HIP graph capture (no allocation, no host
    synchronisation, no memset nodes): capture the fused decode linear and the
    quantize + product pair, replay several times with eager work and
    synchronisations in between, and compare every replay with the eager
    result bit for bit."""
    dec = workloads.decode_linear(1, 4096, 12288)
    big = workloads.random_linear(300, 520, 768, seed=123)
    xs, ws, outs, eager = [], [], [], []
    for lin in (dec, big):
        x = torch.from_numpy(lin.a.view(np.int16)).view(torch.bfloat16).cuda()
        w = torch.from_numpy(lin.b.view(np.int16)).view(torch.bfloat16).cuda()
        qb, sb = fg.quantize_fp8_blocks(w)
        xs.append(x)
        ws.append((qb, sb))
    q = torch.empty((big.m, big.k), dtype=torch.float8_e4m3fn, device="cuda")
    sa = torch.empty((big.k // 128, fg.padded_rows(big.m)), dtype=torch.float32, device="cuda")
    d_dec = torch.empty((1, dec.n), dtype=torch.bfloat16, device="cuda")
    d_big = torch.empty((big.m, big.n), dtype=torch.bfloat16, device="cuda")

    def work():
        fg.fp8_linear_nt(xs[0], ws[0], d_dec)
        fg.quantize_fp8_groups(xs[1], out=(q, sa))
        fg.fp8_gemm_nt((q, sa), ws[1], d_big)

    work()
    torch.cuda.synchronize()
    ref_dec, ref_big = d_dec.clone(), d_big.clone()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    g = torch.cuda.CUDAGraph()
    with torch.cuda.stream(s):
        work()
        torch.cuda.synchronize()
        with torch.cuda.graph(g, stream=s):
            work()
    torch.cuda.synchronize()
    for i in range(4):
        d_dec.fill_(float("nan"))
        d_big.fill_(float("nan"))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(d_dec.view(torch.int16), ref_dec.view(torch.int16)), f"replay {i}: decode differs"
        assert torch.equal(d_big.view(torch.int16), ref_big.view(torch.int16)), f"replay {i}: gemm differs"
        work()  # eager work between replays
        torch.cuda.synchronize()


def _product(lin, env, monkeypatch):
    for key, val in env.items():
        monkeypatch.setenv(key, val)
    _q, _sa, _qb, _sb, d = gpu_hot_path(lin)
    return d


@pytest.mark.parametrize("tile", PERSISTENT_TILES)
@pytest.mark.parametrize("m,n,k", [(200, 300, 256), (2100, 1800, 384), (513, 4000, 640), (4096, 3000, 1280)])
def test_persistent_walk_matches_per_tile_kernel(tile, m, n, k, monkeypatch):
    """The persistent tile walk (several tiles per workgroup, the next tile's
    chunks fetched during the current tile's last ones, ragged M and N edges,
    the minimum K of two chunks) gives the same bits as one workgroup per
    tile, and meets the oracle on sampled rows."""
    lin = workloads.random_linear(m, n, k, seed=m + n + k + len(tile))
    print(f"persistent {tile} {m}x{n}x{k}", flush=True)
    base = _product(lin, {"FGFP8_GEMM_TILE": tile, "FGFP8_PERSISTENT": "0"}, monkeypatch)
    monkeypatch.setenv("FGFP8_PERSISTENT", "1")
    q, sa, qb, sb, d = gpu_hot_path(lin)
    assert torch.equal(base.view(torch.int16), d.view(torch.int16))
    rng = np.random.default_rng(m)
    check_sampled(lin, q, sa, qb, sb, d, sample_rows(m, 16, rng), sample_col_blocks(n, 4, rng), f"persistent {tile}")


def test_empty_problems_through_the_binding():
    """Zero rows (or columns) through every call: nothing is written, no error."""
    dev = "cuda"
    x = torch.empty((0, 256), dtype=torch.bfloat16, device=dev)
    q, sa = fg.quantize_fp8_groups(x)
    assert q.shape == (0, 256) and sa.shape == (2, 0)
    q8, sa8 = fg.quantize_fp8_groups(x, ue8m0=True)
    assert q8.shape == (0, 256)
    qb, sb = fg.quantize_fp8_blocks(torch.empty((0, 256), dtype=torch.bfloat16, device=dev))
    assert qb.shape == (0, 256)
    lin = workloads.random_linear(8, 128, 256, seed=5)
    wq, ws = fg.quantize_fp8_blocks(to_dev_bf16(lin.b))
    d = torch.empty((0, 128), dtype=torch.bfloat16, device=dev)
    fg.fp8_gemm_nt((q, sa), (wq, ws), d)
    fg.fp8_gemm_nt((q, sa), (wq, ws), d, ue8m0=True)
    assert fg.fp8_linear(x, (wq, ws)).shape == (0, 128)
    qo, so = fg.fp8_gemm_nt_fp8_out((q, sa), (wq, ws))
    assert qo.shape == (0, 128)
    xa = to_dev_bf16(lin.a)
    qa, saa = fg.quantize_fp8_groups(xa)
    d0 = torch.empty((8, 0), dtype=torch.bfloat16, device=dev)
    fg.fp8_gemm_nt((qa, saa), (wq[:0], ws[:0]), d0)
    # the MoE layer with no tokens
    idx = torch.empty((0, 2), dtype=torch.int32, device=dev)
    wts = torch.empty((0, 2), dtype=torch.float32, device=dev)
    w1 = fg.quantize_fp8_blocks(torch.zeros((2 * 256, 256), dtype=torch.bfloat16, device=dev))
    w2 = fg.quantize_fp8_blocks(torch.zeros((2 * 256, 128), dtype=torch.bfloat16, device=dev))
    w1 = (w1[0].view(2, 256, 256), w1[1].view(2, 2, 2))
    w2 = (w2[0].view(2, 256, 128), w2[1].view(2, 2, 1))
    out = fg.moe_fp8_layer(torch.empty((0, 256), dtype=torch.bfloat16, device=dev), idx, wts, w1, w2)
    torch.cuda.synchronize()
    assert out.shape == (0, 256)


# ------------------------------------------------ K split (fp8_gemm_nt_ws)
def _split_run(q, sa, qb, sb, m, n, ws):
    d = torch.full((m, n), float("nan"), dtype=torch.bfloat16, device="cuda")
    fg.fp8_gemm_nt((q, sa), (qb, sb), d, workspace=ws)
    return d


def _counters_zero(ws, m, n):
    tiles = -(-m // 256) * -(-n // 256)
    return bool((ws[: 8 * tiles].view(torch.int32) == 0).all())


def test_split_k_down_projection_full():
    """The down projection (2048 x 4096 x 12288) through fp8_gemm_nt_ws, whose
    plan splits K over two workgroups per 256x256 tile: every output against
    the oracle, the same bits on a second call, and the workspace's counters
    back to zero after each call."""
    (lin,) = workloads.prefill_linears(names=["down"])
    assert "splitk2" in fg.describe_gemm(lin.m, lin.n, lin.k)
    x = to_dev_bf16(lin.a)
    w = to_dev_bf16(lin.b)
    q, sa = fg.quantize_fp8_groups(x)
    qb, sb = fg.quantize_fp8_blocks(w)
    ws = fg.gemm_workspace(lin.m, lin.n, lin.k)
    assert ws is not None
    d1 = _split_run(q, sa, qb, sb, lin.m, lin.n, ws)
    torch.cuda.synchronize()
    assert _counters_zero(ws, lin.m, lin.n)
    d2 = _split_run(q, sa, qb, sb, lin.m, lin.n, ws)
    torch.cuda.synchronize()
    assert torch.equal(d1.view(torch.int16), d2.view(torch.int16)), "two calls differ"
    assert _counters_zero(ws, lin.m, lin.n)
    check_full(lin, q, sa, qb, sb, d1, "down, K split")


@pytest.mark.parametrize("m,n,k", [(300, 520, 768), (256, 256, 256), (513, 1000, 1408), (17, 384, 640),
                                   (1000, 136, 2304)])
def test_split_k_forced_ragged_shapes(m, n, k, monkeypatch):
    """The K split forced (FGFP8_SPLITK=1) on ragged M, N and on K of two
    chunks (one per half): every output against the oracle, twice, with the
    counters back to zero; a workspace below the required size runs the
    unsplit plan, bit for bit."""
    monkeypatch.setenv("FGFP8_SPLITK", "1")
    lin = workloads.random_linear(m, n, k, seed=m * 3 + n + k)
    print(f"split {m}x{n}x{k}: {fg.describe_gemm(m, n, k)}", flush=True)
    q, sa, qb, sb, d0 = gpu_hot_path(lin)
    nbytes = fg.fp8_gemm_nt_workspace_bytes(m, n, k)
    assert nbytes > 0
    ws = torch.zeros(nbytes, dtype=torch.uint8, device="cuda")
    d1 = _split_run(q, sa, qb, sb, m, n, ws)
    d2 = _split_run(q, sa, qb, sb, m, n, ws)
    torch.cuda.synchronize()
    assert torch.equal(d1.view(torch.int16), d2.view(torch.int16))
    assert _counters_zero(ws, m, n)
    check_sampled(lin, q, sa, qb, sb, d1, np.arange(m), np.arange(-(-n // 128)), f"split {m}x{n}x{k}")
    small = torch.zeros(nbytes - 256, dtype=torch.uint8, device="cuda")
    d3 = _split_run(q, sa, qb, sb, m, n, small)
    torch.cuda.synchronize()
    assert torch.equal(d3.view(torch.int16), d0.view(torch.int16)), "an undersized workspace must run fp8_gemm_nt"


def test_workspace_forms_replay_in_graphs(monkeypatch):
    """The two workspace protocols under HIP graph capture: the K-split dense
    product (pairs meeting through arrival counts and ready flags) and the
    masked product's split walk (forced; parts counted in, the last one sums)
    each reset their counters inside the kernel and record no memset, so
    every replay -- with eager calls on the same workspaces in between --
    gives the eager result bit for bit."""
    monkeypatch.setenv("FGFP8_MASKED_SPLIT", "1")
    lin = workloads.random_linear(512, 1024, 8192, seed=321)
    x = torch.from_numpy(lin.a.view(np.int16)).view(torch.bfloat16).cuda()
    w = torch.from_numpy(lin.b.view(np.int16)).view(torch.bfloat16).cuda()
    qa, sa = fg.quantize_fp8_groups(x)
    qb, sb = fg.quantize_fp8_blocks(w)
    ws_dense = fg.gemm_workspace(lin.m, lin.n, lin.k)
    assert ws_dense is not None, fg.describe_gemm(lin.m, lin.n, lin.k)
    d_dense = torch.empty((lin.m, lin.n), dtype=torch.bfloat16, device="cuda")
    c = workloads.small_masked([300, 129, 128, 256], 300, 512, 640, seed=99)
    g_, mm, n, k = c.num_groups, c.max_m, c.n, c.k
    mq, msa = fg.quantize_fp8_groups(torch.from_numpy(c.a.reshape(g_ * mm, k).view(np.int16)).view(torch.bfloat16).cuda())
    mqb, msb = fg.quantize_fp8_blocks(torch.from_numpy(c.b.reshape(g_ * n, k).view(np.int16)).view(torch.bfloat16).cuda())
    mqb, msb = mqb.view(g_, n, k), msb.view(g_, n // 128, k // 128)
    counts = torch.from_numpy(c.masked_m.astype(np.int32)).cuda()
    ws_masked = fg.masked_workspace(g_, mm, n, k)
    d_masked = torch.full((g_, mm, n), float("nan"), dtype=torch.bfloat16, device="cuda")

    def work():
        fg.fp8_gemm_nt((qa, sa), (qb, sb), d_dense, workspace=ws_dense)
        fg.m_grouped_fp8_gemm_nt_masked((mq.view(g_, mm, k), msa), (mqb, msb), d_masked, counts, c.expected_m,
                                        workspace=ws_masked)

    work()
    torch.cuda.synchronize()
    ref_dense, ref_masked = d_dense.clone(), d_masked.clone()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.stream(s):
        work()
        torch.cuda.synchronize()
        with torch.cuda.graph(graph, stream=s):
            work()
    torch.cuda.synchronize()
    for i in range(4):
        d_dense.fill_(float("nan"))
        d_masked.fill_(float("nan"))
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(d_dense.view(torch.int16), ref_dense.view(torch.int16)), f"replay {i}: K-split product differs"
        assert torch.equal(d_masked.view(torch.int16), ref_masked.view(torch.int16)), f"replay {i}: masked differs"
        work()  # eager calls on the same workspaces between replays
        torch.cuda.synchronize()
    assert int(ws_masked[:1024].view(torch.int32).abs().sum().item()) == 0
