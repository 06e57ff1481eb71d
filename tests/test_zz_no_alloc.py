"""The allocation-free routing call, moe_route_contiguous_noalloc, through the
C ABI: its outputs equal those of moe_route_contiguous (the same routing
with a workspace the caller allocates) bit for bit, on two calls in a row
where the second is smaller (the library's fixed workspace keeps the first
call's contents), and sizes beyond the fixed workspace are refused on the
host before anything is enqueued."""

import numpy as np
import pytest
import torch

import fine_grained_block_fp8_amd as fg
import workloads

pytestmark = pytest.mark.gpu

POISON = -7  # every output entry is written, so none may keep this value


def _routing_case(tokens, experts, topk, seed):
    """Zipf-routed experts with some slots dropped (-1 or >= experts) and
    some repeated within a token."""
    rng = np.random.default_rng(seed)
    idx = workloads.zipf_topk_routing(rng, tokens, experts, topk, 1.1).astype(np.int32)
    flat = idx.reshape(-1)
    drop = rng.choice(flat.size, size=flat.size // 50, replace=False)
    flat[drop[: drop.size // 2]] = -1
    flat[drop[drop.size // 2 :]] = experts
    if topk > 1:
        rep = rng.choice(tokens, size=max(1, tokens // 40), replace=False)
        idx[rep, 1] = idx[rep, 0]
    return torch.from_numpy(idx).cuda()


def _buffers(tokens, topk, experts):
    m = fg.moe_max_padded_rows(tokens, topk, experts)
    dev = "cuda"
    return (torch.full((experts,), POISON, dtype=torch.int32, device=dev),
            torch.full((m,), POISON, dtype=torch.int32, device=dev),
            torch.full((m,), POISON, dtype=torch.int32, device=dev),
            torch.full((tokens, topk), POISON, dtype=torch.int32, device=dev))


def test_noalloc_route_equals_workspace_route_twice():
    # the second call is smaller than the first
    for tokens, experts, topk, seed in ((8192, 256, 8, 1), (1000, 33, 4, 2)):
        print(f"noalloc route tokens={tokens} experts={experts} topk={topk}", flush=True)
        idx = _routing_case(tokens, experts, topk, seed)
        want = fg.moe_route_contiguous(idx, experts)
        got = fg.moe_route_contiguous_noalloc(idx, experts, out=_buffers(tokens, topk, experts))
        torch.cuda.synchronize()
        for name, g, w in zip(("counts", "m_indices", "token_of_row", "row_of"), got, want):
            assert torch.equal(g, w), f"{name} differs (tokens={tokens}, experts={experts})"
            assert not torch.any(g == POISON), f"{name} not fully written"


def test_noalloc_route_refuses_sizes_beyond_its_workspace():
    cap = fg.moe_route_noalloc_max_workspace_bytes()
    experts = 2048
    # the smallest token count whose routing workspace exceeds the fixed one
    tokens = 256 * (cap // (4 * experts))
    assert fg.moe_route_workspace_bytes(tokens, experts) > cap
    idx = torch.zeros((tokens, 1), dtype=torch.int32, device="cuda")
    with pytest.raises(fg.Fgfp8Error) as e:
        fg.moe_route_contiguous_noalloc(idx, experts, out=_buffers(tokens, 1, experts))
    assert e.value.code == fg.FGFP8_EINVAL
    assert "fixed" in str(e.value)
    # one block fewer fits
    tokens -= 256
    assert fg.moe_route_workspace_bytes(tokens, experts) <= cap
    idx = torch.zeros((tokens, 1), dtype=torch.int32, device="cuda")
    got = fg.moe_route_contiguous_noalloc(idx, experts, out=_buffers(tokens, 1, experts))
    want = fg.moe_route_contiguous(idx, experts)
    torch.cuda.synchronize()
    for g, w in zip(got, want):
        assert torch.equal(g, w)
