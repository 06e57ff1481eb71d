"""Fine-grained block-scaled FP8 linear for AMD MI355X (gfx950).

A thin Python binding over libfgfp8.so, the C-ABI library declared in
include/fgfp8.h.  Every step of the path runs in the library's HIP kernels;
this module only checks tensor dtypes/shapes, passes device pointers and the
current torch stream, and turns error codes into exceptions.  torch provides
device memory and streams and nothing else.  Importing the package fails
loudly if the library has not been built (there is no fallback path).

Calls (names as on the deepgemm-rust README, "What's implemented", and the
Linnet DeepGEMM plugin source):

    q, sa = quantize_fp8_groups(x)                   # x: bf16 [M, K]
    qb, sb = quantize_fp8_blocks(w)                  # w: bf16 [N, K]
    fp8_gemm_nt((q, sa), (qb, sb), d)                # d: bf16 [M, N], in place
    m_grouped_fp8_gemm_nt_contiguous((q, sa), (qb, sb), d, m_indices)
    m_grouped_fp8_gemm_nt_masked((q, sa), (qb, sb), d, masked_m, expected_m)
    out = moe_fp8_layer(x, topk_idx, topk_weights, w1, w2)   # the MoE layer
"""

from __future__ import annotations

import ctypes
import os
import re

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIBRARY_PATH = os.path.join(_HERE, "libfgfp8.so")
HEADER_PATH = os.path.join(os.path.dirname(_HERE), "include", "fgfp8.h")

FGFP8_OK, FGFP8_EINVAL, FGFP8_ENODEV, FGFP8_ELAUNCH = 0, 1, 2, 3
GROUP = 128

if not os.path.exists(LIBRARY_PATH):
    raise ImportError(
        f"{LIBRARY_PATH} is missing: build it with `python fine_grained_block_fp8_amd/build.py` "
        "(the FP8 linear has no path other than its HIP kernels)"
    )

_lib = ctypes.CDLL(LIBRARY_PATH)
_i64, _vp, _fp, _i32 = ctypes.c_int64, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int32
_lib.quantize_fp8_groups.argtypes = [_vp, _i64, _i64, _vp, _fp, _i64, _vp]
_lib.quantize_fp8_blocks.argtypes = [_vp, _i64, _i64, _vp, _fp, _vp]
_lib.fp8_gemm_nt.argtypes = [_vp, _fp, _i64, _vp, _fp, _vp, _i64, _i64, _i64, _vp]
_lib.m_grouped_fp8_gemm_nt_contiguous.argtypes = [_vp, _fp, _i64, _vp, _vp, _fp, _i32, _vp, _i64, _i64, _i64, _vp]
_lib.fp8_linear_nt.argtypes = [_vp, _i64, _i64, _vp, _fp, _i64, _vp, _vp, _fp, _i64, _vp]
_lib.fp8_gemm_nt_fp8_out.argtypes = [_vp, _fp, _i64, _vp, _fp, _vp, _fp, _i64, _vp, _i64, _i64, _i64, _vp]
_lib.m_grouped_fp8_gemm_nt_masked.argtypes = [_vp, _fp, _i64, _vp, _vp, _fp, _i32, _i64, _i64, _vp, _i64, _i64, _vp]
_lib.m_grouped_fp8_gemm_nt_masked_ws.argtypes = [_vp, _fp, _i64, _vp, _vp, _fp, _i32, _i64, _i64, _vp, _i64, _i64, _vp,
                                                 _i64, _vp]
_lib.m_grouped_fp8_gemm_nt_masked_workspace_bytes.argtypes = [_i32, _i64, _i64, _i64]
_lib.m_grouped_fp8_gemm_nt_masked_workspace_bytes.restype = ctypes.c_int64
_lib.quantize_fp8_groups_masked.argtypes = [_vp, _vp, _i32, _i64, _i64, _vp, _fp, _i64, _vp]
_lib.quantize_fp8_groups_ue8m0.argtypes = [_vp, _i64, _i64, _vp, _fp, _i64, _vp]
_lib.quantize_fp8_blocks_ue8m0.argtypes = [_vp, _i64, _i64, _vp, _fp, _vp]
_lib.fp8_gemm_nt_ue8m0.argtypes = [_vp, _fp, _i64, _vp, _fp, _vp, _i64, _i64, _i64, _vp]
_lib.fgfp8_stream_read.argtypes = [_vp, _i64, _vp, _i64, _vp]
_lib.fp8_gemm_nt_ws.argtypes = [_vp, _fp, _i64, _vp, _fp, _vp, _i64, _i64, _i64, _vp, _i64, _vp]
_lib.fp8_gemm_nt_workspace_bytes.argtypes = [_i64, _i64, _i64]
_lib.fp8_gemm_nt_workspace_bytes.restype = ctypes.c_int64
_lib.quantize_fp8_mx.argtypes = [_vp, _i64, _i64, _vp, _vp, _i64, _vp]
_lib.fp8_gemm_nt_mx.argtypes = [_vp, _vp, _i64, _vp, _vp, _i64, _vp, _i64, _i64, _i64, _vp]
_lib.moe_max_padded_rows.argtypes = [_i64, _i32, _i32]
_lib.moe_max_padded_rows.restype = ctypes.c_int64
_lib.moe_route_workspace_bytes.argtypes = [_i64, _i32]
_lib.moe_route_workspace_bytes.restype = ctypes.c_int64
_lib.moe_route_contiguous.argtypes = [_vp, _i64, _i32, _i32, _vp, _vp, _vp, _vp, _i64, _vp, _i64, _vp]
_lib.moe_route_contiguous_noalloc.argtypes = [_vp, _i64, _i32, _i32, _vp, _vp, _vp, _vp, _i64, _vp]
_lib.moe_route_noalloc_max_workspace_bytes.argtypes = []
_lib.moe_route_noalloc_max_workspace_bytes.restype = ctypes.c_int64
_lib.moe_gather_quantize.argtypes = [_vp, _i64, _i64, _vp, _i64, _vp, _fp, _i64, _vp]
_lib.silu_mul_quantize.argtypes = [_vp, _i64, _i64, _vp, _vp, _fp, _i64, _vp]
_lib.moe_gather_quantize_tokens.argtypes = [_vp, _i64, _i64, _i32, _vp, _vp, _i64, _vp, _fp, _i64, _vp]
_lib.moe_combine.argtypes = [_vp, _i64, _i64, _vp, _fp, _i64, _i32, _vp, _vp]
_lib.moe_gate_up_silu_quantize.argtypes = [_vp, _fp, _i64, _vp, _vp, _fp, _i32, _vp, _fp, _i64, _i64, _i64, _i64, _vp]
_lib.fgfp8_last_error.argtypes = []
_lib.fgfp8_last_error.restype = ctypes.c_char_p
_lib.fgfp8_describe_gemm.argtypes = [_i64, _i64, _i64, ctypes.c_char_p, _i64]
_lib.fgfp8_describe_linear.argtypes = [_i64, _i64, _i64, ctypes.c_int, ctypes.c_char_p, _i64]
_lib.fgfp8_describe_grouped.argtypes = [_i64, _i64, _i64, ctypes.c_char_p, _i64]
for _name in ("quantize_fp8_groups", "quantize_fp8_blocks", "fp8_gemm_nt", "m_grouped_fp8_gemm_nt_contiguous",
              "m_grouped_fp8_gemm_nt_masked", "m_grouped_fp8_gemm_nt_masked_ws", "fp8_gemm_nt_fp8_out", "fp8_linear_nt", "fgfp8_describe_gemm",
              "fgfp8_describe_linear", "fgfp8_describe_grouped",
              "quantize_fp8_groups_ue8m0", "quantize_fp8_blocks_ue8m0", "fp8_gemm_nt_ue8m0", "moe_route_contiguous",
              "moe_gather_quantize", "silu_mul_quantize", "moe_combine", "quantize_fp8_mx", "fp8_gemm_nt_mx",
              "moe_gate_up_silu_quantize", "quantize_fp8_groups_masked",
              "moe_gather_quantize_tokens", "moe_route_contiguous_noalloc", "fp8_gemm_nt_ws", "fgfp8_stream_read"):
    getattr(_lib, _name).restype = ctypes.c_int


class Fgfp8Error(RuntimeError):
    def __init__(self, code: int, message: str):
        super().__init__(f"[fgfp8 error {code}] {message}")
        self.code = code


def last_error() -> str:
    return (_lib.fgfp8_last_error() or b"").decode()


def _check(rc: int) -> None:
    if rc != FGFP8_OK:
        raise Fgfp8Error(rc, last_error())


def declared_functions() -> list[str]:
    """Names of the functions include/fgfp8.h declares."""
    with open(HEADER_PATH) as f:
        text = f.read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return re.findall(r"^\s*(?:int|int64_t|const char\*)\s+(\w+)\s*\(", text, flags=re.M)


def library() -> ctypes.CDLL:
    return _lib


_raw_stream = getattr(torch._C, "_cuda_getCurrentRawStream", None)


def _stream(t: torch.Tensor) -> int:
    """torch's current stream on t's device, as a raw hipStream_t."""
    if _raw_stream is not None:
        return _raw_stream(t.device.index)
    return torch.cuda.current_stream(t.device).cuda_stream


def _ptr(t: torch.Tensor) -> int:
    return t.data_ptr()


def _need(t: torch.Tensor, name: str, dtypes, ndim: int) -> None:
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.device.type != "cuda":
        raise ValueError(f"{name} must be on a GPU (got {t.device})")
    if t.dtype not in dtypes:
        raise ValueError(f"{name} must have dtype in {dtypes} (got {t.dtype})")
    if t.dim() != ndim:
        raise ValueError(f"{name} must be {ndim}-D (got shape {tuple(t.shape)})")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


_FP8 = (torch.float8_e4m3fn, torch.uint8)


def padded_rows(m: int) -> int:
    """Scale leading dimension: rows padded to a multiple of four."""
    return -(-m // 4) * 4


def quantize_fp8_groups(x: torch.Tensor, sa_ld: int | None = None, out=None, ue8m0: bool = False):
    """Per-(1x128) activation quantization.  x: bf16 [M, K].  Returns
    (q float8_e4m3fn [M, K], sa float32 [K/128, sa_ld]), sa MN-major.
    ue8m0=True rounds every scale up to a power of two (the UE8M0 recipe)."""
    _need(x, "x", (torch.bfloat16,), 2)
    m, k = x.shape
    sa_ld = padded_rows(m) if sa_ld is None else int(sa_ld)
    if out is None:
        q = torch.empty((m, k), dtype=torch.float8_e4m3fn, device=x.device)
        sa = torch.empty((k // GROUP if k % GROUP == 0 else 0, sa_ld), dtype=torch.float32, device=x.device)
    else:
        q, sa = out
        _need(q, "q", _FP8, 2)
        _need(sa, "sa", (torch.float32,), 2)
        if tuple(q.shape) != (m, k) or tuple(sa.shape) != (k // GROUP, sa_ld):
            raise ValueError("output shapes must be q [M, K] and sa [K/128, sa_ld]")
    fn = _lib.quantize_fp8_groups_ue8m0 if ue8m0 else _lib.quantize_fp8_groups
    _check(fn(_ptr(x), m, k, _ptr(q), _ptr(sa), sa_ld, _stream(x)))
    return q, sa


def quantize_fp8_groups_masked(x: torch.Tensor, masked_m: torch.Tensor, sa_ld: int | None = None, out=None):
    """quantize_fp8_groups over a dispatch buffer x bf16 [G, max_m, K] whose
    group g holds masked_m[g] real rows (int32 [G], on the device): only
    those rows are quantized.  Returns (q float8_e4m3fn [G, max_m, K], sa
    float32 [K/128, sa_ld]) with group g's row r in scale column g*max_m + r,
    the operand the masked product takes; rows past a count keep whatever q
    and sa held."""
    _need(x, "x", (torch.bfloat16,), 3)
    _need(masked_m, "masked_m", (torch.int32,), 1)
    g, max_m, k = x.shape
    if masked_m.shape[0] != g:
        raise ValueError("masked_m must be [G]")
    sa_ld = padded_rows(g * max_m) if sa_ld is None else int(sa_ld)
    if out is None:
        q = torch.empty((g, max_m, k), dtype=torch.float8_e4m3fn, device=x.device)
        sa = torch.empty((k // GROUP if k % GROUP == 0 else 0, sa_ld), dtype=torch.float32, device=x.device)
    else:
        q, sa = out
        _need(q, "q", _FP8, 3)
        _need(sa, "sa", (torch.float32,), 2)
        if tuple(q.shape) != (g, max_m, k) or tuple(sa.shape) != (k // GROUP, sa_ld):
            raise ValueError("output shapes must be q [G, max_m, K] and sa [K/128, sa_ld]")
    _check(_lib.quantize_fp8_groups_masked(_ptr(x), _ptr(masked_m), g, max_m, k, _ptr(q), _ptr(sa), sa_ld,
                                           _stream(x)))
    return q, sa


def quantize_fp8_blocks(w: torch.Tensor, out=None, ue8m0: bool = False):
    """Per-(128x128) weight quantization.  w: bf16 [N, K].  Returns
    (q float8_e4m3fn [N, K], sb float32 [ceil(N/128), K/128]); ue8m0=True:
    power-of-two scales."""
    _need(w, "w", (torch.bfloat16,), 2)
    n, k = w.shape
    if out is None:
        q = torch.empty((n, k), dtype=torch.float8_e4m3fn, device=w.device)
        sb = torch.empty((-(-n // GROUP), k // GROUP if k % GROUP == 0 else 0), dtype=torch.float32, device=w.device)
    else:
        q, sb = out
        _need(q, "q", _FP8, 2)
        _need(sb, "sb", (torch.float32,), 2)
        if tuple(q.shape) != (n, k):
            raise ValueError(f"q must be [{n}, {k}]")
        if k % GROUP == 0 and tuple(sb.shape) != (-(-n // GROUP), k // GROUP):
            raise ValueError(f"sb must be [{-(-n // GROUP)}, {k // GROUP}]")
        if q.device != w.device or sb.device != w.device:
            raise ValueError("q and sb must be on w's device")
    fn = _lib.quantize_fp8_blocks_ue8m0 if ue8m0 else _lib.quantize_fp8_blocks
    _check(fn(_ptr(w), n, k, _ptr(q), _ptr(sb), _stream(w)))
    return q, sb


def fp8_gemm_nt(a, b, d: torch.Tensor, ue8m0: bool = False, workspace: torch.Tensor | None = None) -> torch.Tensor:
    """d[M, N] (bf16, written in place) = A . B^T with A = (q [M, K], sa
    [K/128, sa_ld]) and B = (q [N, K], sb [ceil(N/128), K/128]).  ue8m0=True
    runs fp8_gemm_nt_ue8m0 (every scale must be a power of two).  With
    `workspace` (a uint8 device tensor from gemm_workspace, zero-filled when
    allocated) it runs fp8_gemm_nt_ws, which splits K over two workgroups per
    tile on shapes whose tiles would leave compute units idle."""
    (qa, sa), (qb, sb) = a, b
    _need(qa, "a", _FP8, 2)
    _need(qb, "b", _FP8, 2)
    _need(sa, "sa", (torch.float32,), 2)
    _need(sb, "sb", (torch.float32,), 2)
    _need(d, "d", (torch.bfloat16,), 2)
    m, k = qa.shape
    n = qb.shape[0]
    if qb.shape[1] != k:
        raise ValueError("a and b must share K")
    if tuple(d.shape) != (m, n):
        raise ValueError(f"d must be [{m}, {n}]")
    if k % GROUP == 0 and (sa.shape[0] != k // GROUP or tuple(sb.shape) != (-(-n // GROUP), k // GROUP)):
        raise ValueError("scale shapes must be sa [K/128, sa_ld] and sb [ceil(N/128), K/128]")
    if workspace is not None:
        if ue8m0:
            raise ValueError("the workspace form is for FP32 scales")
        _need(workspace, "workspace", (torch.uint8,), 1)
        _check(_lib.fp8_gemm_nt_ws(_ptr(qa), _ptr(sa), sa.shape[1], _ptr(qb), _ptr(sb), _ptr(d), m, n, k,
                                   _ptr(workspace), workspace.numel(), _stream(d)))
        return d
    fn = _lib.fp8_gemm_nt_ue8m0 if ue8m0 else _lib.fp8_gemm_nt
    _check(fn(_ptr(qa), _ptr(sa), sa.shape[1], _ptr(qb), _ptr(sb), _ptr(d), m, n, k, _stream(d)))
    return d


def fp8_gemm_nt_workspace_bytes(m: int, n: int, k: int) -> int:
    """Bytes of workspace fp8_gemm_nt_ws uses for this shape (0: none)."""
    return int(_lib.fp8_gemm_nt_workspace_bytes(m, n, k))


def gemm_workspace(m: int, n: int, k: int, device="cuda") -> torch.Tensor | None:
    """A zero-filled workspace for fp8_gemm_nt(..., workspace=) at this
    shape, or None when the shape's plan needs none.  Reusable by any later
    call on the same stream (each call leaves it ready for the next)."""
    nbytes = fp8_gemm_nt_workspace_bytes(m, n, k)
    return torch.zeros(nbytes, dtype=torch.uint8, device=device) if nbytes else None


def fp8_gemm_nt_fp8_out(a, b, out=None, d: torch.Tensor | None = None):
    """The product of fp8_gemm_nt, quantized per 1x128 group of each row for
    the next layer: returns (q float8_e4m3fn [M, N], sd float32 [N/128,
    sd_ld]), bit-identical to quantize_fp8_groups(fp8_gemm_nt(a, b)); d, if
    given, also receives the bf16 product.  N must be a multiple of 128."""
    (qa, sa), (qb, sb) = a, b
    _need(qa, "a", _FP8, 2)
    _need(qb, "b", _FP8, 2)
    _need(sa, "sa", (torch.float32,), 2)
    _need(sb, "sb", (torch.float32,), 2)
    m, k = qa.shape
    n = qb.shape[0]
    if qb.shape[1] != k:
        raise ValueError("a and b must share K")
    if out is None:
        q = torch.empty((m, n), dtype=torch.float8_e4m3fn, device=qa.device)
        sd = torch.empty((n // GROUP if n % GROUP == 0 else 0, padded_rows(m)), dtype=torch.float32, device=qa.device)
    else:
        q, sd = out
        _need(q, "q", _FP8, 2)
        _need(sd, "sd", (torch.float32,), 2)
        if tuple(q.shape) != (m, n):
            raise ValueError(f"q must be [{m}, {n}]")
    d_ptr = None
    if d is not None:
        _need(d, "d", (torch.bfloat16,), 2)
        if tuple(d.shape) != (m, n):
            raise ValueError(f"d must be [{m}, {n}]")
        d_ptr = _ptr(d)
    _check(
        _lib.fp8_gemm_nt_fp8_out(
            _ptr(qa), _ptr(sa), sa.shape[1], _ptr(qb), _ptr(sb), _ptr(q), _ptr(sd), sd.shape[1], d_ptr, m, n, k,
            _stream(qa),
        )
    )
    return q, sd


def m_grouped_fp8_gemm_nt_contiguous(a, b, d: torch.Tensor, m_indices: torch.Tensor) -> torch.Tensor:
    """Grouped product: A = (q [M, K], sa), B = (q [G, N, K], sb [G, ceil(N/128), K/128]),
    m_indices int32 [M] (group of each row, -1 for padding), d bf16 [M, N]."""
    (qa, sa), (qb, sb) = a, b
    _need(qa, "a", _FP8, 2)
    _need(qb, "b", _FP8, 3)
    _need(sa, "sa", (torch.float32,), 2)
    _need(sb, "sb", (torch.float32,), 3)
    _need(d, "d", (torch.bfloat16,), 2)
    _need(m_indices, "m_indices", (torch.int32,), 1)
    m, k = qa.shape
    g, n, k2 = qb.shape
    if k2 != k or tuple(d.shape) != (m, n) or m_indices.shape[0] != m:
        raise ValueError("shape mismatch among a [M, K], b [G, N, K], d [M, N], m_indices [M]")
    if k % GROUP == 0 and tuple(sb.shape) != (g, -(-n // GROUP), k // GROUP):
        raise ValueError("sb must be [G, ceil(N/128), K/128]")
    _check(
        _lib.m_grouped_fp8_gemm_nt_contiguous(
            _ptr(qa), _ptr(sa), sa.shape[1], _ptr(m_indices), _ptr(qb), _ptr(sb), g, _ptr(d), m, n, k, _stream(d)
        )
    )
    return d


def m_grouped_fp8_gemm_nt_masked(a, b, d: torch.Tensor, masked_m: torch.Tensor, expected_m: int | None = None,
                                 workspace: torch.Tensor | None = None):
    """Masked grouped product: A = (q [G, max_m, K], sa [K/128, sa_ld]) with the
    group folded into the scale column (row g*max_m + r), B = (q [G, N, K], sb
    [G, ceil(N/128), K/128]), masked_m int32 [G] on the device, d bf16
    [G, max_m, N] (rows past masked_m[g] are not written).  expected_m is a
    host-side hint for the tile choice.  workspace (masked_workspace()): one
    workgroup per CU walks the live tiles and splits the last round's tiles
    along K where that round would leave CUs idle (deterministic; split tiles
    round differently from the plain call, within the same bounds)."""
    (qa, sa), (qb, sb) = a, b
    _need(qa, "a", _FP8, 3)
    _need(qb, "b", _FP8, 3)
    _need(sa, "sa", (torch.float32,), 2)
    _need(sb, "sb", (torch.float32,), 3)
    _need(d, "d", (torch.bfloat16,), 3)
    _need(masked_m, "masked_m", (torch.int32,), 1)
    g, max_m, k = qa.shape
    g2, n, k2 = qb.shape
    if g2 != g or k2 != k or tuple(d.shape) != (g, max_m, n) or masked_m.shape[0] != g:
        raise ValueError("shape mismatch among a [G, max_m, K], b [G, N, K], d [G, max_m, N], masked_m [G]")
    if k % GROUP == 0 and tuple(sb.shape) != (g, -(-n // GROUP), k // GROUP):
        raise ValueError("sb must be [G, ceil(N/128), K/128]")
    if k % GROUP == 0 and sa.shape[0] != k // GROUP:
        raise ValueError("sa must be [K/128, sa_ld]")
    em = 0 if expected_m is None else int(expected_m)
    if workspace is None:
        _check(
            _lib.m_grouped_fp8_gemm_nt_masked(
                _ptr(qa), _ptr(sa), sa.shape[1], _ptr(masked_m), _ptr(qb), _ptr(sb), g, max_m, em, _ptr(d), n, k,
                _stream(d)
            )
        )
        return d
    _need(workspace, "workspace", (torch.uint8,), 1)
    _check(
        _lib.m_grouped_fp8_gemm_nt_masked_ws(
            _ptr(qa), _ptr(sa), sa.shape[1], _ptr(masked_m), _ptr(qb), _ptr(sb), g, max_m, em, _ptr(d), n, k,
            _ptr(workspace), workspace.numel(), _stream(d)
        )
    )
    return d


def m_grouped_fp8_gemm_nt_masked_workspace_bytes(num_groups: int, max_m: int, n: int, k: int) -> int:
    """Bytes of workspace the masked product's workspace form uses (0: invalid arguments)."""
    return int(_lib.m_grouped_fp8_gemm_nt_masked_workspace_bytes(num_groups, max_m, n, k))


def masked_workspace(num_groups: int, max_m: int, n: int, k: int, device="cuda") -> torch.Tensor | None:
    """A zero-filled workspace for m_grouped_fp8_gemm_nt_masked(..., workspace=),
    reusable by every later call on the same stream (each call leaves it ready
    for the next)."""
    nbytes = m_grouped_fp8_gemm_nt_masked_workspace_bytes(num_groups, max_m, n, k)
    return torch.zeros(nbytes, dtype=torch.uint8, device=device) if nbytes else None


# fp8_linear_nt: one fused kernel up to FUSED_MAX_M rows when no workspace is
# given; up to FUSED_FAST_MAX_M rows that kernel is the fastest path.  Above
# it, passing the workspace is never slower: the library then runs the fused
# three-slab kernel where it wins, else quantize + product
# (describe_linear names the choice).
FUSED_MAX_M, FUSED_FAST_MAX_M = 16, 4


def fp8_linear_nt(x: torch.Tensor, weight, d: torch.Tensor, act_out=None) -> torch.Tensor:
    """d[M, N] = quantize_groups(x) . B^T for bf16 x [M, K] and the stored
    weight (q [N, K], sb).  `act_out` = (q [M, K], sa [K/128, sa_ld])
    optionally receives the quantized activation.  One fused kernel for
    M <= 4; for 4 < M <= 16 a fused kernel, or with `act_out` the quantizer
    and the product where they are faster (describe_linear says which);
    above 16 rows `act_out` is required.  Every path gives the same bits."""
    qb, sb = weight
    _need(x, "x", (torch.bfloat16,), 2)
    _need(qb, "b", _FP8, 2)
    _need(sb, "sb", (torch.float32,), 2)
    _need(d, "d", (torch.bfloat16,), 2)
    m, k = x.shape
    n = qb.shape[0]
    if qb.shape[1] != k or tuple(d.shape) != (m, n):
        raise ValueError("shape mismatch among x [M, K], b [N, K], d [M, N]")
    if act_out is None:
        q_ptr, sa_ptr, sa_ld = None, None, 0
    else:
        q, sa = act_out
        _need(q, "q", _FP8, 2)
        _need(sa, "sa", (torch.float32,), 2)
        q_ptr, sa_ptr, sa_ld = _ptr(q), _ptr(sa), sa.shape[1]
    _check(_lib.fp8_linear_nt(_ptr(x), m, k, _ptr(qb), _ptr(sb), n, _ptr(d), q_ptr, sa_ptr, sa_ld, _stream(d)))
    return d


def fp8_linear(x: torch.Tensor, weight) -> torch.Tensor:
    """The pages' linear (Linnet DeepGEMM plugin, _BlockProduct.execute): round
    the bf16 input per 1x128 group, then the block-scaled product with the
    pre-quantized weight (q [N, K], sb).  x: bf16 [..., K]; returns bf16 [..., N]."""
    qb, sb = weight
    flat = x.reshape(-1, x.shape[-1])
    m, k = flat.shape
    d = torch.empty((m, qb.shape[0]), dtype=torch.bfloat16, device=x.device)
    act = None
    if m > FUSED_FAST_MAX_M:  # the two-launch path is the faster one here
        act = (torch.empty((m, k), dtype=torch.float8_e4m3fn, device=x.device),
               torch.empty((k // GROUP, padded_rows(m)), dtype=torch.float32, device=x.device))
    fp8_linear_nt(flat, (qb, sb), d, act)
    return d.reshape(*x.shape[:-1], qb.shape[0])


# ---------------------------------------------------------------- MX recipe
def quantize_fp8_mx(x: torch.Tensor, s_ld: int | None = None, out=None):
    """MXFP8 quantization: one power-of-two scale per 1x32 block of each row.
    x: bf16 [M, K] (an activation, or a weight [N, K]).  Returns (q
    float8_e4m3fn [M, K], s int32 [K/128, s_ld]) with the four E8M0 codes of
    a 128-column chunk packed in each int32."""
    _need(x, "x", (torch.bfloat16,), 2)
    m, k = x.shape
    s_ld = padded_rows(m) if s_ld is None else int(s_ld)
    if out is None:
        out = (torch.empty((m, k), dtype=torch.float8_e4m3fn, device=x.device),
               torch.empty((k // GROUP, s_ld), dtype=torch.int32, device=x.device))
    q, sc = out
    _need(q, "q", _FP8, 2)
    _need(sc, "s", (torch.int32,), 2)
    _check(_lib.quantize_fp8_mx(_ptr(x), m, k, _ptr(q), _ptr(sc), sc.shape[1], _stream(x)))
    return q, sc


def fp8_gemm_nt_mx(a, b, d: torch.Tensor) -> torch.Tensor:
    """MXFP8 product: a = (q [M, K], s int32 [K/128, sa_ld]), b = (q [N, K],
    s int32 [K/128, sb_ld]) from quantize_fp8_mx; d bf16 [M, N] in place."""
    (qa, sa), (qb, sb) = a, b
    _need(qa, "a", _FP8, 2)
    _need(qb, "b", _FP8, 2)
    _need(sa, "sa", (torch.int32,), 2)
    _need(sb, "sb", (torch.int32,), 2)
    _need(d, "d", (torch.bfloat16,), 2)
    m, k = qa.shape
    n = qb.shape[0]
    if qb.shape[1] != k or tuple(d.shape) != (m, n):
        raise ValueError("shape mismatch among a [M, K], b [N, K], d [M, N]")
    _check(_lib.fp8_gemm_nt_mx(_ptr(qa), _ptr(sa), sa.shape[1], _ptr(qb), _ptr(sb), sb.shape[1], _ptr(d), m, n, k,
                               _stream(d)))
    return d


# ----------------------------------------------------------------- MoE layer
def moe_max_padded_rows(tokens: int, topk: int, num_experts: int) -> int:
    """Upper bound of the contiguous layout's rows: roundup(T*topk + G*127, 128)."""
    r = _lib.moe_max_padded_rows(tokens, topk, num_experts)
    if r < 0:
        raise ValueError("bad MoE sizes")
    return r


def moe_route_contiguous(topk_idx: torch.Tensor, num_experts: int, m_pad_max: int | None = None, out=None):
    """Routing layout from topk_idx int32 [T, topk].  Returns (counts [G],
    m_indices [m_pad_max], token_of_row [m_pad_max], row_of [T, topk]), all
    int32 on the device and computed without a host synchronisation.  `out`
    optionally holds those four tensors plus a uint8 workspace of at least
    moe_route_workspace_bytes(T, G) bytes, to be reused across calls."""
    _need(topk_idx, "topk_idx", (torch.int32,), 2)
    tokens, topk = topk_idx.shape
    dev = topk_idx.device
    if out is None:
        if m_pad_max is None:
            m_pad_max = moe_max_padded_rows(tokens, topk, num_experts)
        ws_bytes = _lib.moe_route_workspace_bytes(tokens, num_experts)
        if ws_bytes < 0:
            raise ValueError("bad MoE sizes")
        out = (torch.empty(num_experts, dtype=torch.int32, device=dev),
               torch.empty(m_pad_max, dtype=torch.int32, device=dev),
               torch.empty(m_pad_max, dtype=torch.int32, device=dev),
               torch.empty((tokens, topk), dtype=torch.int32, device=dev),
               torch.empty(max(ws_bytes, 16), dtype=torch.uint8, device=dev))
    counts, m_indices, token_of_row, row_of, ws = out
    for t, name in ((counts, "counts"), (m_indices, "m_indices"), (token_of_row, "token_of_row")):
        _need(t, name, (torch.int32,), 1)
    _need(row_of, "row_of", (torch.int32,), 2)
    if counts.shape[0] != num_experts or token_of_row.shape != m_indices.shape or tuple(row_of.shape) != (tokens, topk):
        raise ValueError("routing buffers do not match (G, m_pad_max, [T, topk])")
    _check(
        _lib.moe_route_contiguous(
            _ptr(topk_idx), tokens, topk, num_experts, _ptr(counts), _ptr(m_indices), _ptr(token_of_row),
            _ptr(row_of), m_indices.shape[0], _ptr(ws), ws.numel(), _stream(topk_idx)
        )
    )
    return counts, m_indices, token_of_row, row_of


def moe_route_contiguous_noalloc(topk_idx: torch.Tensor, num_experts: int, out) -> tuple:
    """moe_route_contiguous with the library's fixed routing workspace instead
    of a caller's: nothing is allocated.  `out` = (counts [G], m_indices
    [m_pad_max], token_of_row [m_pad_max], row_of [T, topk]), int32 device
    tensors the caller owns.  Calls on one device share the workspace: calls
    that overlap in time race."""
    _need(topk_idx, "topk_idx", (torch.int32,), 2)
    tokens, topk = topk_idx.shape
    counts, m_indices, token_of_row, row_of = out
    for t, name in ((counts, "counts"), (m_indices, "m_indices"), (token_of_row, "token_of_row")):
        _need(t, name, (torch.int32,), 1)
    _need(row_of, "row_of", (torch.int32,), 2)
    if counts.shape[0] != num_experts or token_of_row.shape != m_indices.shape or tuple(row_of.shape) != (tokens, topk):
        raise ValueError("routing buffers do not match (G, m_pad_max, [T, topk])")
    _check(
        _lib.moe_route_contiguous_noalloc(
            _ptr(topk_idx), tokens, topk, num_experts, _ptr(counts), _ptr(m_indices), _ptr(token_of_row),
            _ptr(row_of), m_indices.shape[0], _stream(topk_idx)
        )
    )
    return counts, m_indices, token_of_row, row_of


def moe_route_noalloc_max_workspace_bytes() -> int:
    return int(_lib.moe_route_noalloc_max_workspace_bytes())


def moe_route_workspace_bytes(tokens: int, num_experts: int) -> int:
    r = _lib.moe_route_workspace_bytes(tokens, num_experts)
    if r < 0:
        raise ValueError("bad MoE sizes")
    return r


def moe_gather_quantize(x: torch.Tensor, token_of_row: torch.Tensor, out=None):
    """Rows x[token_of_row[r]] (zeros for an index outside [0, T)) quantized per 1x128 group.
    x: bf16 [T, K].  Returns (q float8_e4m3fn [m_pad_max, K], sa float32
    [K/128, m_pad_max'] with the rows padded to a multiple of four)."""
    _need(x, "x", (torch.bfloat16,), 2)
    _need(token_of_row, "token_of_row", (torch.int32,), 1)
    k = x.shape[1]
    m = token_of_row.shape[0]
    if out is None:
        out = (torch.empty((m, k), dtype=torch.float8_e4m3fn, device=x.device),
               torch.empty((k // GROUP, padded_rows(m)), dtype=torch.float32, device=x.device))
    q, sa = out
    _need(q, "q", _FP8, 2)
    _need(sa, "sa", (torch.float32,), 2)
    if tuple(q.shape) != (m, k):
        raise ValueError("q must be [m_pad_max, K]")
    _check(_lib.moe_gather_quantize(_ptr(x), x.shape[0], k, _ptr(token_of_row), m, _ptr(q), _ptr(sa), sa.shape[1],
                                    _stream(x)))
    return q, sa


def moe_gather_quantize_tokens(x: torch.Tensor, row_of: torch.Tensor, token_of_row: torch.Tensor, out=None):
    """moe_gather_quantize for the routing layout (row_of int32 [T, topk] and
    token_of_row int32 [m_pad_max] as moe_route_contiguous writes them): each
    token's row is read and quantized once and written to its rows; rows no
    token maps to get zero codes and scale 1.  Same bytes as
    moe_gather_quantize."""
    _need(x, "x", (torch.bfloat16,), 2)
    _need(row_of, "row_of", (torch.int32,), 2)
    _need(token_of_row, "token_of_row", (torch.int32,), 1)
    tokens, k = x.shape
    if row_of.shape[0] != tokens:
        raise ValueError("row_of must be [T, topk]")
    m = token_of_row.shape[0]
    if out is None:
        out = (torch.empty((m, k), dtype=torch.float8_e4m3fn, device=x.device),
               torch.empty((k // GROUP, padded_rows(m)), dtype=torch.float32, device=x.device))
    q, sa = out
    _need(q, "q", _FP8, 2)
    _need(sa, "sa", (torch.float32,), 2)
    if tuple(q.shape) != (m, k):
        raise ValueError("q must be [m_pad_max, K]")
    _check(_lib.moe_gather_quantize_tokens(_ptr(x), tokens, k, row_of.shape[1], _ptr(row_of), _ptr(token_of_row), m,
                                           _ptr(q), _ptr(sa), sa.shape[1], _stream(x)))
    return q, sa


def silu_mul_quantize(h: torch.Tensor, m_indices: torch.Tensor, out=None):
    """act = bf16(silu(h[:, :I]) * h[:, I:]) quantized per 1x128 group (rows
    with m_indices < 0 give zeros).  h: bf16 [M, 2I].  Returns (q [M, I], sa
    [I/128, roundup(M, 4)])."""
    _need(h, "h", (torch.bfloat16,), 2)
    _need(m_indices, "m_indices", (torch.int32,), 1)
    m, two_i = h.shape
    if two_i % 2 or m_indices.shape[0] != m:
        raise ValueError("h must be [M, 2I] and m_indices [M]")
    inter = two_i // 2
    if out is None:
        out = (torch.empty((m, inter), dtype=torch.float8_e4m3fn, device=h.device),
               torch.empty((inter // GROUP, padded_rows(m)), dtype=torch.float32, device=h.device))
    q, sa = out
    _need(q, "q", _FP8, 2)
    _need(sa, "sa", (torch.float32,), 2)
    if tuple(q.shape) != (m, inter):
        raise ValueError("q must be [M, I]")
    _check(_lib.silu_mul_quantize(_ptr(h), m, inter, _ptr(m_indices), _ptr(q), _ptr(sa), sa.shape[1], _stream(h)))
    return q, sa


def moe_gate_up_silu_quantize(a, w1, m_indices: torch.Tensor, out=None):
    """The gate_up grouped product with SiLU.mul and the 1x128 quantizer in
    its epilogue: a = (q [M, K], sa), w1 = (q [G, 2I, K], sb [G, 2I/128,
    K/128]) with the gate rows first; returns (q [M, I], sa [I/128,
    roundup(M, 4)]), the bits m_grouped_fp8_gemm_nt_contiguous followed by
    silu_mul_quantize give."""
    (qa, sa), (qw, sw) = a, w1
    _need(qa, "a", _FP8, 2)
    _need(sa, "sa", (torch.float32,), 2)
    _need(qw, "w1", _FP8, 3)
    _need(sw, "sb1", (torch.float32,), 3)
    _need(m_indices, "m_indices", (torch.int32,), 1)
    m, k = qa.shape
    g, two_i, k2 = qw.shape
    if k2 != k or two_i % 2 or m_indices.shape[0] != m:
        raise ValueError("shape mismatch among a [M, K], w1 [G, 2I, K], m_indices [M]")
    if k % GROUP == 0 and two_i % GROUP == 0 and tuple(sw.shape) != (g, two_i // GROUP, k // GROUP):
        raise ValueError("sb1 must be [G, 2I/128, K/128]")
    inter = two_i // 2
    if out is None:
        out = (torch.empty((m, inter), dtype=torch.float8_e4m3fn, device=qa.device),
               torch.empty((inter // GROUP, padded_rows(m)), dtype=torch.float32, device=qa.device))
    q, sq = out
    _need(q, "q", _FP8, 2)
    _need(sq, "sq", (torch.float32,), 2)
    if tuple(q.shape) != (m, inter):
        raise ValueError("q must be [M, I]")
    _check(_lib.moe_gate_up_silu_quantize(_ptr(qa), _ptr(sa), sa.shape[1], _ptr(m_indices), _ptr(qw), _ptr(sw), g,
                                          _ptr(q), _ptr(sq), sq.shape[1], m, inter, k, _stream(qa)))
    return q, sq


def moe_combine(y: torch.Tensor, row_of: torch.Tensor, topk_weights: torch.Tensor, out=None) -> torch.Tensor:
    """out[t] = bf16(sum_j topk_weights[t, j] * y[row_of[t, j]]) in FP32, slot
    order; slots whose row lies outside [0, rows) are skipped.  y bf16 [rows, H], row_of int32 [T, topk], topk_weights float32 [T, topk]."""
    _need(y, "y", (torch.bfloat16,), 2)
    _need(row_of, "row_of", (torch.int32,), 2)
    _need(topk_weights, "topk_weights", (torch.float32,), 2)
    tokens, topk = row_of.shape
    if tuple(topk_weights.shape) != (tokens, topk):
        raise ValueError("topk_weights must match row_of [T, topk]")
    hdim = y.shape[1]
    if out is None:
        out = torch.empty((tokens, hdim), dtype=torch.bfloat16, device=y.device)
    _need(out, "out", (torch.bfloat16,), 2)
    if tuple(out.shape) != (tokens, hdim):
        raise ValueError("out must be [T, H]")
    _check(_lib.moe_combine(_ptr(y), y.shape[0], hdim, _ptr(row_of), _ptr(topk_weights), tokens, topk, _ptr(out),
                            _stream(y)))
    return out


def moe_fp8_layer(x: torch.Tensor, topk_idx: torch.Tensor, topk_weights: torch.Tensor, w1, w2,
                  fused: bool = True) -> torch.Tensor:
    """The FP8 MoE layer (deepgemm-rust README, "What's implemented",
    moe_fp8_layer row), every step on the device with no host synchronisation:
    route -> gather+quantize -> grouped product with w1 -> SiLU.mul+quantize ->
    grouped product with w2 -> weighted combine.  With `fused` the w1 product
    and SiLU.mul+quantize are one kernel (same bits).

    x bf16 [T, H]; topk_idx int32 [T, topk]; topk_weights float32 [T, topk];
    w1 = (q [G, 2I, H], sb [G, 2I/128, H/128]) with the gate rows first, then
    the up rows; w2 = (q [G, H, I], sb [G, H/128, I/128]).  Returns bf16 [T, H]."""
    (q1, s1), (q2, s2) = w1, w2
    _need(q1, "w1", _FP8, 3)
    _need(q2, "w2", _FP8, 3)
    tokens, hdim = x.shape
    g, two_i, h1 = q1.shape
    if h1 != hdim or tuple(q2.shape) != (g, hdim, two_i // 2):
        raise ValueError("w1 must be [G, 2I, H] and w2 [G, H, I]")
    counts, m_indices, token_of_row, row_of = moe_route_contiguous(topk_idx, g)
    m = m_indices.shape[0]
    a1 = moe_gather_quantize_tokens(x, row_of, token_of_row)
    if fused:
        a2 = moe_gate_up_silu_quantize(a1, (q1, s1), m_indices)
    else:
        hbuf = torch.empty((m, two_i), dtype=torch.bfloat16, device=x.device)
        m_grouped_fp8_gemm_nt_contiguous(a1, (q1, s1), hbuf, m_indices)
        a2 = silu_mul_quantize(hbuf, m_indices)
    y = torch.empty((m, hdim), dtype=torch.bfloat16, device=x.device)
    m_grouped_fp8_gemm_nt_contiguous(a2, (q2, s2), y, m_indices)
    return moe_combine(y, row_of, topk_weights)


def stream_read(src: torch.Tensor, out: torch.Tensor) -> None:
    """Measurement aid: read all of src (a contiguous device tensor whose
    size is a multiple of 32 KiB) once; out (uint8, >= 4096 bytes) receives
    XORs of what was read."""
    if not (src.is_cuda and src.is_contiguous() and out.is_cuda and out.dtype == torch.uint8):
        raise ValueError("src must be a contiguous device tensor and out a uint8 device tensor")
    _check(_lib.fgfp8_stream_read(_ptr(src), src.numel() * src.element_size(), _ptr(out), out.numel(), _stream(src)))


def describe_gemm(m: int, n: int, k: int) -> str:
    buf = ctypes.create_string_buffer(128)
    _check(_lib.fgfp8_describe_gemm(m, n, k, buf, 128))
    return buf.value.decode()


def describe_grouped(m: int, n: int, k: int) -> str:
    """The kernel m_grouped_fp8_gemm_nt_contiguous runs for m padded rows."""
    buf = ctypes.create_string_buffer(128)
    _check(_lib.fgfp8_describe_grouped(m, n, k, buf, 128))
    return buf.value.decode()


def describe_linear(m: int, n: int, k: int, act_out: bool) -> str:
    """The path fp8_linear_nt takes (act_out: whether the quantized
    activation is passed too)."""
    buf = ctypes.create_string_buffer(256)
    _check(_lib.fgfp8_describe_linear(m, n, k, int(bool(act_out)), buf, 256))
    return buf.value.decode()


__all__ = [
    "FGFP8_EINVAL",
    "FGFP8_ELAUNCH",
    "FGFP8_ENODEV",
    "FGFP8_OK",
    "Fgfp8Error",
    "declared_functions",
    "describe_gemm",
    "describe_linear",
    "fp8_gemm_nt",
    "fp8_gemm_nt_fp8_out",
    "fp8_gemm_nt_mx",
    "fp8_linear",
    "fp8_linear_nt",
    "fp8_gemm_nt_workspace_bytes",
    "gemm_workspace",
    "stream_read",
    "last_error",
    "m_grouped_fp8_gemm_nt_contiguous",
    "m_grouped_fp8_gemm_nt_masked",
    "m_grouped_fp8_gemm_nt_masked_workspace_bytes",
    "masked_workspace",
    "moe_combine",
    "moe_fp8_layer",
    "moe_gate_up_silu_quantize",
    "moe_gather_quantize",
    "moe_gather_quantize_tokens",
    "moe_max_padded_rows",
    "moe_route_contiguous",
    "moe_route_contiguous_noalloc",
    "moe_route_noalloc_max_workspace_bytes",
    "moe_route_workspace_bytes",
    "padded_rows",
    "quantize_fp8_blocks",
    "quantize_fp8_groups",
    "quantize_fp8_groups_masked",
    "quantize_fp8_mx",
    "silu_mul_quantize",
]
