"""ctypes binding of libattn_varlen.so (include/attn_varlen.h).

Argument marshalling only: tensors become device pointers, strides and token
extents; the stream is torch's current stream. Every step of the computation
runs in the library's HIP kernels. If the library is missing this module
raises instead of computing anything another way.
"""
from __future__ import annotations

import ctypes
import math
from pathlib import Path

_PKG = Path(__file__).resolve().parent
LIB_PATH = _PKG / "libattn_varlen.so"

OK = 0
ENULL, EINVAL, EUNSUPPORTED, EALIGN, ECU, EMAXSEQ, EHIP = -1, -2, -3, -4, -5, -6, -7
ERROR_NAMES = {ENULL: "ENULL", EINVAL: "EINVAL", EUNSUPPORTED: "EUNSUPPORTED", EALIGN: "EALIGN",
               ECU: "ECU", EMAXSEQ: "EMAXSEQ", EHIP: "EHIP"}

#: every symbol include/attn_varlen.h declares
EXPORTED_SYMBOLS = (
    "attn_varlen_fwd", "attn_varlen_fwd_hostcu", "attn_varlen_validate", "attn_varlen_block_m",
    "attn_varlen_count_tiles", "attn_varlen_grid_plan", "attn_varlen_segments_per_launch",
    "attn_varlen_decode_tile", "attn_varlen_element_offset", "attn_varlen_last_error",
    "attn_varlen_fwd_ex", "attn_varlen_fwd_hostcu_ex", "attn_varlen_validate_ex",
    "attn_fwd_batched", "attn_fwd_batched_validate",
    "attn_varlen_bwd_preprocess", "attn_varlen_bwd", "attn_varlen_bwd_hostcu", "attn_varlen_bwd_validate",
    "attn_varlen_bwd_grid_plan", "attn_varlen_async_workspace_bytes", "attn_varlen_fwd_async",
    "attn_varlen_async_status", "attn_varlen_async_grid", "attn_varlen_fp8_workspace_bytes",
    "attn_varlen_fp8_workspace_offsets", "attn_varlen_fwd_fp8", "attn_varlen_fwd_fp8_hostcu",
    "attn_varlen_block_m_for", "attn_varlen_one_stage_keys", "attn_varlen_short_stage_keys",
    "attn_varlen_num_tiles", "attn_varlen_fwd_async_noalloc",
)

CAUSAL = 1  # ATTN_VARLEN_CAUSAL


class AttnVarlenError(RuntimeError):
    def __init__(self, code: int, message: str):
        super().__init__(f"{ERROR_NAMES.get(code, code)}: {message}")
        self.code = code


class Layout(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int64) for n in (
        "q_row", "q_head", "k_row", "k_head", "v_row", "v_head", "o_row", "o_head",
        "lse_head", "q_tokens", "k_tokens")]


class BatchedLayout(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int64) for n in (
        "q_batch", "q_row", "q_head", "k_batch", "k_row", "k_head", "v_batch", "v_row", "v_head",
        "o_batch", "o_row", "o_head", "lse_batch", "lse_head")]


class BwdLayout(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int64) for n in (
        "q_row", "q_head", "k_row", "k_head", "v_row", "v_head", "o_row", "o_head", "do_row", "do_head",
        "dq_row", "dq_head", "dk_row", "dk_head", "dv_row", "dv_head", "lse_head", "delta_head",
        "q_tokens", "k_tokens")]


_lib = None
_i32p = ctypes.POINTER(ctypes.c_int32)
_i64p = ctypes.POINTER(ctypes.c_int64)
_vp = ctypes.c_void_p


def lib():
    """Load libattn_varlen.so (raises if it has not been built)."""
    global _lib
    if _lib is None:
        if not LIB_PATH.exists():
            raise RuntimeError(
                f"{LIB_PATH} is missing: build it with `python -m varlen_flashattention_forward_amd.build` "
                "(there is no fallback implementation)")
        L = ctypes.CDLL(str(LIB_PATH))
        fwd_args = [_vp, _vp, _vp, _vp, _vp, ctypes.c_int32, ctypes.c_int32, ctypes.c_int32,
                    ctypes.c_int32, ctypes.c_int32, ctypes.POINTER(Layout), ctypes.c_float, _vp, _vp, _vp]
        for name in ("attn_varlen_fwd", "attn_varlen_fwd_hostcu"):
            f = getattr(L, name)
            f.restype = ctypes.c_int32
            f.argtypes = fwd_args
        L.attn_varlen_validate.restype = ctypes.c_int32
        L.attn_varlen_validate.argtypes = fwd_args[:-1]
        ex_args = fwd_args[:12] + [ctypes.c_uint32] + fwd_args[12:]
        for name in ("attn_varlen_fwd_ex", "attn_varlen_fwd_hostcu_ex"):
            f = getattr(L, name)
            f.restype = ctypes.c_int32
            f.argtypes = ex_args
        L.attn_varlen_validate_ex.restype = ctypes.c_int32
        L.attn_varlen_validate_ex.argtypes = ex_args[:-1]
        b_args = [_vp, _vp, _vp] + [ctypes.c_int32] * 5 + [ctypes.POINTER(BatchedLayout), ctypes.c_float,
                                                          ctypes.c_uint32, _vp, _vp, _vp]
        L.attn_fwd_batched.restype = ctypes.c_int32
        L.attn_fwd_batched.argtypes = b_args
        L.attn_fwd_batched_validate.restype = ctypes.c_int32
        L.attn_fwd_batched_validate.argtypes = b_args[:-1]
        L.attn_varlen_bwd_preprocess.restype = ctypes.c_int32
        L.attn_varlen_bwd_preprocess.argtypes = [_vp, _vp, ctypes.c_int64, ctypes.c_int32, ctypes.c_int32] + \
            [ctypes.c_int64] * 4 + [_vp, ctypes.c_int64, _vp]
        bwd_args = [_vp] * 8 + [ctypes.c_int32] * 5 + [ctypes.POINTER(BwdLayout), ctypes.c_float, ctypes.c_uint32,
                                                      _vp, _vp, _vp, _vp, _vp]
        for name in ("attn_varlen_bwd", "attn_varlen_bwd_hostcu"):
            f = getattr(L, name)
            f.restype = ctypes.c_int32
            f.argtypes = bwd_args
        L.attn_varlen_bwd_validate.restype = ctypes.c_int32
        L.attn_varlen_bwd_validate.argtypes = bwd_args[:-1]
        L.attn_varlen_bwd_grid_plan.restype = ctypes.c_int32
        L.attn_varlen_bwd_grid_plan.argtypes = [_i32p, _i32p, ctypes.c_int32, ctypes.c_int32, ctypes.c_int32,
                                                _i64p, _i64p, _i64p, _i64p]
        L.attn_varlen_async_workspace_bytes.restype = ctypes.c_int64
        L.attn_varlen_async_workspace_bytes.argtypes = [ctypes.c_int32]
        L.attn_varlen_fwd_async.restype = ctypes.c_int32
        L.attn_varlen_fwd_async.argtypes = fwd_args[:12] + [ctypes.c_uint32, _vp, ctypes.c_int64] + fwd_args[12:]
        L.attn_varlen_fwd_async_noalloc.restype = ctypes.c_int32
        L.attn_varlen_fwd_async_noalloc.argtypes = fwd_args[:12] + [ctypes.c_uint32] + fwd_args[12:] + \
            [ctypes.POINTER(ctypes.c_void_p)]
        L.attn_varlen_async_status.restype = ctypes.c_int32
        L.attn_varlen_async_status.argtypes = [_vp, _vp, _i32p]
        L.attn_varlen_async_grid.restype = ctypes.c_int32
        L.attn_varlen_async_grid.argtypes = [ctypes.c_int64] + [ctypes.c_int32] * 5 + [_i64p]
        L.attn_varlen_fp8_workspace_bytes.restype = ctypes.c_int64
        L.attn_varlen_fp8_workspace_bytes.argtypes = [ctypes.c_int64, ctypes.c_int64, ctypes.c_int32, ctypes.c_int32]
        L.attn_varlen_fp8_workspace_offsets.restype = ctypes.c_int32
        L.attn_varlen_fp8_workspace_offsets.argtypes = [ctypes.c_int64, ctypes.c_int64, ctypes.c_int32,
                                                        ctypes.c_int32, _i64p, _i64p]
        for name in ("attn_varlen_fwd_fp8", "attn_varlen_fwd_fp8_hostcu"):
            f = getattr(L, name)
            f.restype = ctypes.c_int32
            f.argtypes = fwd_args[:12] + [ctypes.c_uint32, _vp, ctypes.c_int64] + fwd_args[12:]
        L.attn_varlen_block_m.restype = ctypes.c_int32
        L.attn_varlen_block_m.argtypes = [ctypes.c_int32]
        L.attn_varlen_block_m_for.restype = ctypes.c_int32
        L.attn_varlen_block_m_for.argtypes = [ctypes.c_int32, ctypes.c_int32]
        L.attn_varlen_one_stage_keys.restype = ctypes.c_int32
        L.attn_varlen_one_stage_keys.argtypes = []
        L.attn_varlen_short_stage_keys.restype = ctypes.c_int32
        L.attn_varlen_short_stage_keys.argtypes = []
        L.attn_varlen_count_tiles.restype = ctypes.c_int64
        L.attn_varlen_count_tiles.argtypes = [_i32p, ctypes.c_int32, ctypes.c_int32, ctypes.c_int32]
        L.attn_varlen_num_tiles.restype = ctypes.c_int64
        L.attn_varlen_num_tiles.argtypes = [_i32p, ctypes.c_int32, ctypes.c_int32, ctypes.c_int32,
                                            ctypes.c_int32]
        L.attn_varlen_grid_plan.restype = ctypes.c_int32
        L.attn_varlen_grid_plan.argtypes = [_i32p, ctypes.c_int32, ctypes.c_int32, ctypes.c_int32, ctypes.c_int32,
                                            _i64p, _i64p]
        L.attn_varlen_segments_per_launch.restype = ctypes.c_int32
        L.attn_varlen_segments_per_launch.argtypes = []
        L.attn_varlen_decode_tile.restype = ctypes.c_int32
        L.attn_varlen_decode_tile.argtypes = [_i32p, ctypes.c_int32, ctypes.c_int32, ctypes.c_int32,
                                              ctypes.c_int64, _i32p, _i32p, _i32p]
        L.attn_varlen_element_offset.restype = ctypes.c_int64
        L.attn_varlen_element_offset.argtypes = [ctypes.c_int64] * 4
        L.attn_varlen_last_error.restype = ctypes.c_char_p
        L.attn_varlen_last_error.argtypes = []
        _lib = L
    return _lib


def last_error() -> str:
    return lib().attn_varlen_last_error().decode()


def _check(rc: int) -> None:
    if rc != OK:
        raise AttnVarlenError(rc, last_error())


def _cu_array(cu):
    vals = [int(x) for x in cu]
    return (ctypes.c_int32 * max(1, len(vals)))(*vals), len(vals) - 1


# ---- host-only helpers (no GPU needed) -------------------------------------------------

def block_m(head_dim: int, max_seqlen_k: int | None = None) -> int:
    """Query rows per tile: of the general configuration, or, given the call's
    max_seqlen_k, of the configuration the bf16 forward picks for it."""
    if max_seqlen_k is None:
        r = lib().attn_varlen_block_m(head_dim)
    else:
        r = lib().attn_varlen_block_m_for(head_dim, max_seqlen_k)
    _check(min(r, 0))
    return r


def one_stage_keys() -> int:
    """Longest key segment (max_seqlen_k) the one-stage configuration takes."""
    return lib().attn_varlen_one_stage_keys()


def short_stage_keys() -> int:
    """Longest key segment (max_seqlen_k) the 64-key-stage configuration takes."""
    return lib().attn_varlen_short_stage_keys()


def count_tiles(cu_q, num_heads: int, block_m_: int) -> int:
    arr, B = _cu_array(cu_q)
    r = lib().attn_varlen_count_tiles(arr, B, num_heads, block_m_)
    if r < 0:
        _check(int(r))
    return int(r)


def num_tiles(cu_q, num_heads: int, head_dim: int, max_seqlen_k: int) -> int:
    """Exact workgroup total of one attn_varlen_fwd call with these host
    cu_seqlens_q, head count, head_dim and max_seqlen_k."""
    arr, B = _cu_array(cu_q)
    r = lib().attn_varlen_num_tiles(arr, B, num_heads, head_dim, max_seqlen_k)
    if r < 0:
        _check(int(r))
    return int(r)


def grid_plan(cu_q, num_heads: int, head_dim: int, max_seqlen_k: int):
    """(launches, workgroups) of attn_varlen_fwd for these cu_seqlens_q and max_seqlen_k."""
    arr, B = _cu_array(cu_q)
    nl, nw = ctypes.c_int64(), ctypes.c_int64()
    _check(lib().attn_varlen_grid_plan(arr, B, num_heads, head_dim, max_seqlen_k, ctypes.byref(nl),
                                       ctypes.byref(nw)))
    return nl.value, nw.value


def segments_per_launch() -> int:
    return lib().attn_varlen_segments_per_launch()


def decode_tile(cu_q, num_heads: int, block_m_: int, wg: int):
    arr, B = _cu_array(cu_q)
    s, m, h = ctypes.c_int32(), ctypes.c_int32(), ctypes.c_int32()
    _check(lib().attn_varlen_decode_tile(arr, B, num_heads, block_m_, wg, ctypes.byref(s), ctypes.byref(m),
                                         ctypes.byref(h)))
    return s.value, m.value, h.value


def element_offset(row: int, row_stride: int, head: int, head_stride: int) -> int:
    return lib().attn_varlen_element_offset(row, row_stride, head, head_stride)


def validate(q_ptr, k_ptr, v_ptr, cu_q, cu_k, num_heads, head_dim, max_q, max_k, layout: Layout,
             scale: float, out_ptr, lse_ptr, flags: int | None = None) -> int:
    """Return code of the host-side argument check (no HIP call); flags=None
    uses the flag-less entry point."""
    cq, B = _cu_array(cu_q)
    ck, Bk = _cu_array(cu_k)
    if Bk != B:
        raise ValueError("cu_q and cu_k differ in length")
    if flags is None:
        return lib().attn_varlen_validate(q_ptr, k_ptr, v_ptr, cq, ck, B, num_heads, head_dim, max_q,
                                          max_k, ctypes.byref(layout), scale, out_ptr, lse_ptr)
    return lib().attn_varlen_validate_ex(q_ptr, k_ptr, v_ptr, cq, ck, B, num_heads, head_dim, max_q,
                                         max_k, ctypes.byref(layout), scale, flags, out_ptr, lse_ptr)


def validate_batched(q_ptr, k_ptr, v_ptr, batch, seqlen_q, seqlen_k, num_heads, head_dim,
                     layout: BatchedLayout, scale: float, flags: int, out_ptr, lse_ptr) -> int:
    """Return code of the batched entry point's argument check (no HIP call)."""
    return lib().attn_fwd_batched_validate(q_ptr, k_ptr, v_ptr, batch, seqlen_q, seqlen_k, num_heads,
                                           head_dim, ctypes.byref(layout), scale, flags, out_ptr, lse_ptr)


# ---- torch front end ----------------------------------------------------------------

def _layout_of(q, k, v, out, lse, lse_head):
    for name, t in (("q", q), ("k", k), ("v", v), ("out", out)):
        if t.dim() != 3 or t.stride(2) != 1:
            raise ValueError(f"{name} must be [tokens, H, D] with a contiguous D dimension")
    return Layout(q.stride(0), q.stride(1), k.stride(0), k.stride(1), v.stride(0), v.stride(1),
                  out.stride(0), out.stride(1), lse_head, q.shape[0], k.shape[0])


def _fwd_tensors(q, k, v, out, lse, return_lse: bool):
    """Check the forward's q, k, v (and a caller-supplied out / lse) and
    allocate what is missing. Returns (total_q, H, D, out, lse, lse_head)."""
    import torch

    if q.dtype != torch.bfloat16 or k.dtype != torch.bfloat16 or v.dtype != torch.bfloat16:
        raise TypeError("q, k, v must be bfloat16")
    if not (q.is_cuda and k.is_cuda and v.is_cuda):
        raise ValueError("q, k, v must be device tensors")
    if q.dim() != 3 or k.dim() != 3:
        raise ValueError("q must be [total_q, H, D] and k, v [total_k, H, D]")
    total_q, H, D = q.shape
    if k.shape[1:] != (H, D) or v.shape != k.shape:
        raise ValueError("k and v must be [total_k, H, D] matching q's H and D")
    if out is None:
        out = torch.empty((total_q, H, D), dtype=torch.bfloat16, device=q.device)
    elif out.dtype != torch.bfloat16 or out.shape != q.shape or not out.is_cuda or out.device != q.device:
        raise ValueError("out must be a bf16 device tensor with q's shape on q's device")
    lse_head = 0
    if lse is None and return_lse:
        lse = torch.empty((H, total_q), dtype=torch.float32, device=q.device)
    if lse is not None:
        if lse.dtype != torch.float32 or lse.dim() != 2 or lse.shape[0] != H or lse.stride(1) != 1 \
                or lse.shape[1] < total_q or not lse.is_cuda or lse.device != q.device:
            raise ValueError("lse must be an fp32 device tensor [H, >= total_q] with unit inner stride")
        lse_head = lse.stride(0)
    return total_q, H, D, out, lse, lse_head


def attn_varlen_fwd(q, k, v, cu_seqlens_q, cu_seqlens_k, max_seqlen_q: int, max_seqlen_k: int,
                    softmax_scale: float | None = None, out=None, lse=None, return_lse: bool = True,
                    cu_seqlens_q_host=None, cu_seqlens_k_host=None, stream=None, causal: bool = False):
    """Varlen attention forward on torch's current stream.

    q: [total_q, H, D], k/v: [total_k, H, D] bf16 CUDA tensors (any token and
    head strides, contiguous D). cu_seqlens_q/k: int32 CUDA tensors [B+1].
    When host copies of cu_seqlens are given, the synchronisation-free entry
    point is used. causal: row r of a segment sees keys j <= r + Lk - Lq.
    Returns (out [total_q, H, D] bf16, lse [H, total_q] fp32 or None).
    """
    import torch

    total_q, H, D, out, lse, lse_head = _fwd_tensors(q, k, v, out, lse, return_lse)
    if softmax_scale is None:
        softmax_scale = 1.0 / math.sqrt(D)
    layout = _layout_of(q, k, v, out, lse, lse_head)
    if stream is None:
        stream = torch.cuda.current_stream(q.device).cuda_stream
    L = lib()
    lse_ptr = lse.data_ptr() if lse is not None else None
    if cu_seqlens_q_host is not None or cu_seqlens_k_host is not None:
        cq, B = _cu_array(cu_seqlens_q_host)
        ck, Bk = _cu_array(cu_seqlens_k_host)
        if B != Bk:
            raise ValueError("cu_seqlens_q and cu_seqlens_k differ in length")
        rc = L.attn_varlen_fwd_hostcu_ex(q.data_ptr(), k.data_ptr(), v.data_ptr(), cq, ck, B, H, D,
                                         int(max_seqlen_q), int(max_seqlen_k), ctypes.byref(layout),
                                         float(softmax_scale), CAUSAL if causal else 0, out.data_ptr(),
                                         lse_ptr, stream)
    else:
        for name, cu in (("cu_seqlens_q", cu_seqlens_q), ("cu_seqlens_k", cu_seqlens_k)):
            if cu.dtype != torch.int32 or not cu.is_cuda or cu.dim() != 1 or not cu.is_contiguous():
                raise ValueError(f"{name} must be a contiguous int32 device tensor")
        B = cu_seqlens_q.numel() - 1
        if cu_seqlens_k.numel() != B + 1:
            raise ValueError("cu_seqlens_q and cu_seqlens_k differ in length")
        rc = L.attn_varlen_fwd_ex(q.data_ptr(), k.data_ptr(), v.data_ptr(), cu_seqlens_q.data_ptr(),
                                  cu_seqlens_k.data_ptr(), B, H, D, int(max_seqlen_q), int(max_seqlen_k),
                                  ctypes.byref(layout), float(softmax_scale), CAUSAL if causal else 0,
                                  out.data_ptr(), lse_ptr, stream)
    _check(rc)
    return out, lse


def async_workspace_bytes(num_segments: int) -> int:
    r = lib().attn_varlen_async_workspace_bytes(num_segments)
    if r < 0:
        _check(int(r))
    return int(r)


def async_grid(q_tokens: int, num_segments: int, num_heads: int, head_dim: int, max_seqlen_q: int,
               max_seqlen_k: int) -> int:
    g = ctypes.c_int64()
    _check(lib().attn_varlen_async_grid(q_tokens, num_segments, num_heads, head_dim, max_seqlen_q, max_seqlen_k,
                                        ctypes.byref(g)))
    return g.value


def async_workspace(num_segments: int, device):
    """A workspace tensor for attn_varlen_fwd_async (caller-owned device memory)."""
    import torch

    return torch.empty(async_workspace_bytes(num_segments) // 4, dtype=torch.int32, device=device)


def async_status(workspace, stream=None) -> int:
    """The planner's status word of the last call that used `workspace` (waits
    for the stream). `workspace` is a workspace tensor, or the integer plan
    address that attn_varlen_fwd_async_noalloc returns (current device)."""
    import torch

    if isinstance(workspace, int):
        ptr, dev = workspace, torch.device("cuda", torch.cuda.current_device())
    else:
        ptr, dev = workspace.data_ptr(), workspace.device
    if stream is None:
        stream = torch.cuda.current_stream(dev).cuda_stream
    st = ctypes.c_int32()
    _check(lib().attn_varlen_async_status(ptr, stream, ctypes.byref(st)))
    return st.value


def attn_varlen_fwd_async(q, k, v, cu_seqlens_q, cu_seqlens_k, max_seqlen_q: int, max_seqlen_k: int,
                          workspace=None, softmax_scale: float | None = None, out=None, lse=None,
                          return_lse: bool = True, stream=None, causal: bool = False):
    """Sync-free varlen attention forward (device planner; no host wait).

    Same tensors as attn_varlen_fwd; cu_seqlens_q/k must be int32 device
    tensors. `workspace` (from async_workspace) is allocated when not given.
    Errors in the cu values are reported through async_status(workspace).
    Returns (out, lse, workspace).
    """
    import torch

    total_q, H, D, out, lse, lse_head = _fwd_tensors(q, k, v, out, lse, return_lse)
    for name, cu in (("cu_seqlens_q", cu_seqlens_q), ("cu_seqlens_k", cu_seqlens_k)):
        if cu.dtype != torch.int32 or not cu.is_cuda or cu.dim() != 1 or not cu.is_contiguous():
            raise ValueError(f"{name} must be a contiguous int32 device tensor")
    B = cu_seqlens_q.numel() - 1
    if cu_seqlens_k.numel() != B + 1:
        raise ValueError("cu_seqlens_q and cu_seqlens_k differ in length")
    if softmax_scale is None:
        softmax_scale = 1.0 / math.sqrt(D)
    if workspace is None:
        workspace = async_workspace(B, q.device)
    elif not workspace.is_cuda or workspace.device != q.device or not workspace.is_contiguous():
        raise ValueError("workspace must be a contiguous device tensor on q's device")
    layout = _layout_of(q, k, v, out, lse, lse_head)
    if stream is None:
        stream = torch.cuda.current_stream(q.device).cuda_stream
    rc = lib().attn_varlen_fwd_async(q.data_ptr(), k.data_ptr(), v.data_ptr(), cu_seqlens_q.data_ptr(),
                                     cu_seqlens_k.data_ptr(), B, H, D, int(max_seqlen_q), int(max_seqlen_k),
                                     ctypes.byref(layout), float(softmax_scale), CAUSAL if causal else 0,
                                     workspace.data_ptr(), workspace.numel() * workspace.element_size(),
                                     out.data_ptr(), lse.data_ptr() if lse is not None else None, stream)
    _check(rc)
    return out, lse, workspace


def attn_varlen_fwd_async_noalloc(q, k, v, cu_seqlens_q, cu_seqlens_k, max_seqlen_q: int, max_seqlen_k: int,
                                  softmax_scale: float | None = None, out=None, lse=None, return_lse: bool = True,
                                  stream=None, causal: bool = False):
    """attn_varlen_fwd_async with the plan in the library's static device
    array instead of a workspace (the C entry point allocates nothing; pass
    out and lse to allocate nothing here either). At most 65536 segments.
    Returns (out, lse, plan): plan is the integer device address of the
    static plan for async_status, or None when nothing was enqueued."""
    import torch

    total_q, H, D, out, lse, lse_head = _fwd_tensors(q, k, v, out, lse, return_lse)
    for name, cu in (("cu_seqlens_q", cu_seqlens_q), ("cu_seqlens_k", cu_seqlens_k)):
        if cu.dtype != torch.int32 or not cu.is_cuda or cu.dim() != 1 or not cu.is_contiguous():
            raise ValueError(f"{name} must be a contiguous int32 device tensor")
    B = cu_seqlens_q.numel() - 1
    if cu_seqlens_k.numel() != B + 1:
        raise ValueError("cu_seqlens_q and cu_seqlens_k differ in length")
    if softmax_scale is None:
        softmax_scale = 1.0 / math.sqrt(D)
    layout = _layout_of(q, k, v, out, lse, lse_head)
    if stream is None:
        stream = torch.cuda.current_stream(q.device).cuda_stream
    plan = ctypes.c_void_p()
    with torch.cuda.device(q.device):
        rc = lib().attn_varlen_fwd_async_noalloc(q.data_ptr(), k.data_ptr(), v.data_ptr(), cu_seqlens_q.data_ptr(),
                                                 cu_seqlens_k.data_ptr(), B, H, D, int(max_seqlen_q),
                                                 int(max_seqlen_k), ctypes.byref(layout), float(softmax_scale),
                                                 CAUSAL if causal else 0, out.data_ptr(),
                                                 lse.data_ptr() if lse is not None else None, stream,
                                                 ctypes.byref(plan))
    _check(rc)
    return out, lse, plan.value


def fp8_workspace_bytes(total_q: int, total_k: int, num_heads: int, head_dim: int) -> int:
    r = lib().attn_varlen_fp8_workspace_bytes(total_q, total_k, num_heads, head_dim)
    if r < 0:
        _check(int(r))
    return int(r)


def fp8_workspace_offsets(total_q: int, total_k: int, num_heads: int, head_dim: int):
    """(q8 offset, k8 offset) in bytes; the 2*H amax words sit at offset 0."""
    a, b = ctypes.c_int64(), ctypes.c_int64()
    _check(lib().attn_varlen_fp8_workspace_offsets(total_q, total_k, num_heads, head_dim, ctypes.byref(a),
                                                   ctypes.byref(b)))
    return a.value, b.value


def attn_varlen_fwd_fp8(q, k, v, cu_seqlens_q, cu_seqlens_k, max_seqlen_q: int, max_seqlen_k: int,
                        workspace=None, softmax_scale: float | None = None, out=None, lse=None,
                        return_lse: bool = True, cu_seqlens_q_host=None, cu_seqlens_k_host=None, stream=None,
                        causal: bool = False):
    """Forward with per-head E4M3 q and k and the 8-bit score product
    (head_dim 64 or 128). Same tensors as attn_varlen_fwd; `workspace` (uint8
    device tensor of fp8_workspace_bytes) is allocated when not given.
    Returns (out, lse, workspace)."""
    import torch

    total_q, H, D, out, lse, lse_head = _fwd_tensors(q, k, v, out, lse, return_lse)
    if softmax_scale is None:
        softmax_scale = 1.0 / math.sqrt(D)
    if workspace is None:
        workspace = torch.empty(fp8_workspace_bytes(total_q, k.shape[0], H, D), dtype=torch.uint8, device=q.device)
    elif not workspace.is_cuda or workspace.device != q.device or not workspace.is_contiguous():
        raise ValueError("workspace must be a contiguous device tensor on q's device")
    layout = _layout_of(q, k, v, out, lse, lse_head)
    if stream is None:
        stream = torch.cuda.current_stream(q.device).cuda_stream
    tail = (ctypes.byref(layout), float(softmax_scale), CAUSAL if causal else 0, workspace.data_ptr(),
            workspace.numel() * workspace.element_size(), out.data_ptr(),
            lse.data_ptr() if lse is not None else None, stream)
    L = lib()
    if cu_seqlens_q_host is not None or cu_seqlens_k_host is not None:
        cq, B = _cu_array(cu_seqlens_q_host)
        ck, Bk = _cu_array(cu_seqlens_k_host)
        if B != Bk:
            raise ValueError("cu_seqlens_q and cu_seqlens_k differ in length")
        rc = L.attn_varlen_fwd_fp8_hostcu(q.data_ptr(), k.data_ptr(), v.data_ptr(), cq, ck, B, H, D,
                                          int(max_seqlen_q), int(max_seqlen_k), *tail)
    else:
        for name, cu in (("cu_seqlens_q", cu_seqlens_q), ("cu_seqlens_k", cu_seqlens_k)):
            if cu.dtype != torch.int32 or not cu.is_cuda or cu.dim() != 1 or not cu.is_contiguous():
                raise ValueError(f"{name} must be a contiguous int32 device tensor")
        B = cu_seqlens_q.numel() - 1
        if cu_seqlens_k.numel() != B + 1:
            raise ValueError("cu_seqlens_q and cu_seqlens_k differ in length")
        rc = L.attn_varlen_fwd_fp8(q.data_ptr(), k.data_ptr(), v.data_ptr(), cu_seqlens_q.data_ptr(),
                                   cu_seqlens_k.data_ptr(), B, H, D, int(max_seqlen_q), int(max_seqlen_k), *tail)
    _check(rc)
    return out, lse, workspace


def attn_fwd(q, k, v, softmax_scale: float | None = None, causal: bool = False, out=None, lse=None,
             return_lse: bool = True, stream=None):
    """Batched dense attention forward (the flash_attn_func form) on torch's
    current stream: q [W, Sq, H, D], k/v [W, Sk, H, D] bf16 CUDA tensors with
    any batch, row and head strides and a contiguous D. Returns
    (out [W, Sq, H, D] bf16, lse [W, H, Sq] fp32 or None)."""
    import torch

    if q.dtype != torch.bfloat16 or k.dtype != torch.bfloat16 or v.dtype != torch.bfloat16:
        raise TypeError("q, k, v must be bfloat16")
    if not (q.is_cuda and k.is_cuda and v.is_cuda):
        raise ValueError("q, k, v must be device tensors")
    if q.dim() != 4 or k.dim() != 4 or v.shape != k.shape:
        raise ValueError("q must be [W, Sq, H, D] and k, v [W, Sk, H, D]")
    W, Sq, H, D = q.shape
    if k.shape[0] != W or k.shape[2:] != (H, D):
        raise ValueError("k and v must match q's batch, head count and head dim")
    Sk = k.shape[1]
    if softmax_scale is None:
        softmax_scale = 1.0 / math.sqrt(D)
    if out is None:
        out = torch.empty((W, Sq, H, D), dtype=torch.bfloat16, device=q.device)
    elif out.dtype != torch.bfloat16 or out.shape != q.shape:
        raise ValueError("out must be bf16 with q's shape")
    if lse is None and return_lse:
        lse = torch.empty((W, H, Sq), dtype=torch.float32, device=q.device)
    lse_batch = lse_head = 0
    if lse is not None:
        if lse.dtype != torch.float32 or lse.shape != (W, H, Sq) or lse.stride(2) != 1:
            raise ValueError("lse must be fp32 [W, H, Sq] with unit inner stride")
        lse_batch, lse_head = lse.stride(0), lse.stride(1)
    for name, t in (("q", q), ("k", k), ("v", v), ("out", out)):
        if t.stride(3) != 1:
            raise ValueError(f"{name} must have a contiguous D dimension")
    layout = BatchedLayout(q.stride(0), q.stride(1), q.stride(2), k.stride(0), k.stride(1), k.stride(2),
                           v.stride(0), v.stride(1), v.stride(2), out.stride(0), out.stride(1), out.stride(2),
                           lse_batch, lse_head)
    if stream is None:
        stream = torch.cuda.current_stream(q.device).cuda_stream
    rc = lib().attn_fwd_batched(q.data_ptr(), k.data_ptr(), v.data_ptr(), W, Sq, Sk, H, D, ctypes.byref(layout),
                                float(softmax_scale), CAUSAL if causal else 0, out.data_ptr(),
                                lse.data_ptr() if lse is not None else None, stream)
    _check(rc)
    return out, lse


# ---- backward -----------------------------------------------------------------------

def bwd_grid_plan(cu_q, cu_k, num_heads: int, head_dim: int):
    """(preprocessing, dK/dV, dQ workgroups, dK/dV + dQ launches) for host cu arrays."""
    cq, B = _cu_array(cu_q)
    ck, Bk = _cu_array(cu_k)
    if Bk != B:
        raise ValueError("cu_q and cu_k differ in length")
    out = [ctypes.c_int64() for _ in range(4)]
    _check(lib().attn_varlen_bwd_grid_plan(cq, ck, B, num_heads, head_dim, *(ctypes.byref(x) for x in out)))
    return tuple(x.value for x in out)


def validate_bwd(ptrs, cu_q, cu_k, num_heads, head_dim, max_q, max_k, layout: BwdLayout, scale: float,
                 flags: int = 0) -> int:
    """Return code of the backward's host-side argument check (no HIP call).
    ptrs: (q, k, v, out, dout, lse, delta, dq, dk, dv) addresses or None."""
    q, k, v, o, g, lse, delta, dq, dk, dv = ptrs
    cq, B = _cu_array(cu_q)
    ck, Bk = _cu_array(cu_k)
    if Bk != B:
        raise ValueError("cu_q and cu_k differ in length")
    return lib().attn_varlen_bwd_validate(q, k, v, o, g, lse, cq, ck, B, num_heads, head_dim, max_q, max_k,
                                          ctypes.byref(layout), scale, flags, delta, dq, dk, dv)


def _fp32_rows(t, name, H, total_q):
    import torch

    if t.dtype != torch.float32 or t.dim() != 2 or t.shape[0] != H or t.stride(1) != 1 or t.shape[1] < total_q \
            or not t.is_cuda:
        raise ValueError(f"{name} must be an fp32 device tensor [H, >= total_q] with unit inner stride")
    return t.stride(0)


def bwd_preprocess(out, dout, delta=None, stream=None):
    """D[h, i] = sum_d out[i,h,d] * dout[i,h,d] (fp32 [H, total_q]) for bf16
    [total_q, H, D] device tensors with any row/head strides."""
    import torch

    if out.dtype != torch.bfloat16 or dout.dtype != torch.bfloat16 or out.shape != dout.shape or out.dim() != 3:
        raise ValueError("out and dout must be bf16 [total_q, H, D] of one shape")
    if out.stride(2) != 1 or dout.stride(2) != 1:
        raise ValueError("out and dout must have a contiguous D dimension")
    total_q, H, D = out.shape
    if delta is None:
        delta = torch.empty((H, total_q), dtype=torch.float32, device=out.device)
    dh = _fp32_rows(delta, "delta", H, total_q)
    if stream is None:
        stream = torch.cuda.current_stream(out.device).cuda_stream
    _check(lib().attn_varlen_bwd_preprocess(out.data_ptr(), dout.data_ptr(), total_q, H, D, out.stride(0),
                                            out.stride(1), dout.stride(0), dout.stride(1), delta.data_ptr(), dh,
                                            stream))
    return delta


def attn_varlen_bwd(q, k, v, out, dout, lse, cu_seqlens_q, cu_seqlens_k, max_seqlen_q: int, max_seqlen_k: int,
                    softmax_scale: float | None = None, causal: bool = False, dq=None, dk=None, dv=None,
                    delta=None, cu_seqlens_q_host=None, cu_seqlens_k_host=None, stream=None):
    """Varlen attention backward on torch's current stream.

    q, out, dout: [total_q, H, D]; k, v: [total_k, H, D] bf16 device tensors
    (any token and head strides, contiguous D); lse: the forward's fp32
    [H, >= total_q]. dq/dk/dv (bf16, q's / k's shape) and the fp32 workspace
    delta [H, >= total_q] are allocated when not given. With host copies of
    cu_seqlens the synchronisation-free entry point is used.
    Returns (dq, dk, dv, delta).
    """
    import torch

    for name, t in (("q", q), ("k", k), ("v", v), ("out", out), ("dout", dout)):
        if t.dtype != torch.bfloat16 or not t.is_cuda or t.dim() != 3 or t.stride(2) != 1:
            raise ValueError(f"{name} must be a bf16 device tensor [tokens, H, D] with contiguous D")
    total_q, H, D = q.shape
    if k.shape[1:] != (H, D) or v.shape != k.shape or out.shape != q.shape or dout.shape != q.shape:
        raise ValueError("k, v must be [total_k, H, D]; out and dout q's shape")
    if softmax_scale is None:
        softmax_scale = 1.0 / math.sqrt(D)
    dq = torch.empty_like(q, memory_format=torch.contiguous_format) if dq is None else dq
    dk = torch.empty_like(k, memory_format=torch.contiguous_format) if dk is None else dk
    dv = torch.empty_like(v, memory_format=torch.contiguous_format) if dv is None else dv
    for name, t, ref in (("dq", dq, q), ("dk", dk, k), ("dv", dv, v)):
        if t.dtype != torch.bfloat16 or t.shape != ref.shape or t.stride(2) != 1 or not t.is_cuda:
            raise ValueError(f"{name} must be bf16 with {('q', 'k', 'v')[('dq', 'dk', 'dv').index(name)]}'s shape")
    if delta is None:
        delta = torch.empty((H, total_q), dtype=torch.float32, device=q.device)
    lh = _fp32_rows(lse, "lse", H, total_q)
    dh = _fp32_rows(delta, "delta", H, total_q)
    layout = BwdLayout(q.stride(0), q.stride(1), k.stride(0), k.stride(1), v.stride(0), v.stride(1),
                       out.stride(0), out.stride(1), dout.stride(0), dout.stride(1), dq.stride(0), dq.stride(1),
                       dk.stride(0), dk.stride(1), dv.stride(0), dv.stride(1), lh, dh, total_q, k.shape[0])
    if stream is None:
        stream = torch.cuda.current_stream(q.device).cuda_stream
    ptrs = (q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(), dout.data_ptr(), lse.data_ptr())
    tail = (ctypes.byref(layout), float(softmax_scale), CAUSAL if causal else 0, delta.data_ptr(),
            dq.data_ptr(), dk.data_ptr(), dv.data_ptr(), stream)
    L = lib()
    if cu_seqlens_q_host is not None or cu_seqlens_k_host is not None:
        cq, B = _cu_array(cu_seqlens_q_host)
        ck, Bk = _cu_array(cu_seqlens_k_host)
        if B != Bk:
            raise ValueError("cu_seqlens_q and cu_seqlens_k differ in length")
        rc = L.attn_varlen_bwd_hostcu(*ptrs, cq, ck, B, H, D, int(max_seqlen_q), int(max_seqlen_k), *tail)
    else:
        for name, cu in (("cu_seqlens_q", cu_seqlens_q), ("cu_seqlens_k", cu_seqlens_k)):
            if cu.dtype != torch.int32 or not cu.is_cuda or cu.dim() != 1 or not cu.is_contiguous():
                raise ValueError(f"{name} must be a contiguous int32 device tensor")
        B = cu_seqlens_q.numel() - 1
        if cu_seqlens_k.numel() != B + 1:
            raise ValueError("cu_seqlens_q and cu_seqlens_k differ in length")
        rc = L.attn_varlen_bwd(*ptrs, cu_seqlens_q.data_ptr(), cu_seqlens_k.data_ptr(), B, H, D,
                               int(max_seqlen_q), int(max_seqlen_k), *tail)
    _check(rc)
    return dq, dk, dv, delta
