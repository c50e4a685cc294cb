"""Python binding of libpkv.so, the MI355X paged-KV split-KV decode attention
library.  Argument marshalling only: every step of the computation runs in
the library's HIP kernels; PyTorch supplies device memory and streams.

The C entry points are declared in include/pkv.h; the functions here carry
the same names without the ``pkv_`` prefix.  Loading fails loudly when the
library has not been built (``python -m paged_kv_split_amd.build``); there is
no fallback path.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libpkv.so")

PKV_OK = 0
PKV_ERR_NULL = 1
PKV_ERR_SHAPE = 2
PKV_ERR_UNSUPPORTED = 3
PKV_ERR_WORKSPACE = 4
PKV_ERR_ALIGN = 5
PKV_ERR_LAUNCH = 6
PKV_ERR_DEVICE = 7
PKV_ERR_SCRATCH = 8
PKV_MAX_SPLITS = 256
PKV_COUNTER_BYTES = 16384
PKV_MAX_FUSED_UNITS = PKV_COUNTER_BYTES // 4
PKV_KV_BLHD = 1
PKV_KV_BHLD = 2
PKV_MAX_CONTIGUOUS_KEYS = 1 << 30
PKV_CAUSAL_LAST = -2
PKV_KERNEL_VECTOR = 0
PKV_KERNEL_MATRIX = 1
PKV_KERNEL_SHARED_TILE = 2
PKV_KERNEL_PREFILL = 3
KERNEL_NAMES = {PKV_KERNEL_VECTOR: "split_decode_valu", PKV_KERNEL_MATRIX: "split_decode_mfma",
                PKV_KERNEL_SHARED_TILE: "split_decode_group", PKV_KERNEL_PREFILL: "split_prefill_mfma"}
PKV_NOALLOC_SCRATCH_BYTES = 64 << 20
KV_LAYOUTS = {"blhd": PKV_KV_BLHD, "bhld": PKV_KV_BHLD}

EXPORTED = ("pkv_num_splits", "pkv_plan", "pkv_plan_varlen", "pkv_workspace_bytes", "pkv_workspace_clear", "pkv_paged_decode",
            "pkv_paged_decode_noalloc", "pkv_paged_decode_varlen", "pkv_contiguous_decode", "pkv_paged_decode_partials", "pkv_combine", "pkv_device_cus",
            "pkv_status_string")


class PkvError(RuntimeError):
    def __init__(self, status: int, where: str):
        super().__init__(f"{where}: {status_string(status)} (status {status})")
        self.status = status


class Problem(ctypes.Structure):
    """Mirror of ``pkv_problem`` (include/pkv.h)."""
    _fields_ = [
        ("batch", ctypes.c_int32),
        ("q_len", ctypes.c_int32),
        ("num_q_heads", ctypes.c_int32),
        ("num_kv_heads", ctypes.c_int32),
        ("head_dim", ctypes.c_int32),
        ("page_size", ctypes.c_int32),
        ("num_pages", ctypes.c_int32),
        ("max_pages_per_seq", ctypes.c_int32),
        ("max_kv_len", ctypes.c_int32),
        ("scale", ctypes.c_float),
        ("causal_offset", ctypes.c_int32),
        ("num_splits", ctypes.c_int32),
        ("mask_stride_b", ctypes.c_int64),
        ("mask_stride_q", ctypes.c_int64),
        ("heads_per_block", ctypes.c_int32),
    ]


class PlanInfo(ctypes.Structure):
    """Mirror of ``pkv_plan_info`` (include/pkv.h)."""
    _fields_ = [
        ("splits", ctypes.c_int32),
        ("heads_per_block", ctypes.c_int32),
        ("rows_per_block", ctypes.c_int32),
        ("matrix_core", ctypes.c_int32),
        ("units", ctypes.c_int64),
        ("workgroups", ctypes.c_int64),
        ("merge_in_kernel", ctypes.c_int32),
        ("kernels", ctypes.c_int32),
        ("kernel", ctypes.c_int32),
        ("paired_heads", ctypes.c_int32),
    ]


_lib = None


def lib() -> ctypes.CDLL:
    """The loaded libpkv.so (raises if it is not built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError(f"{LIB_PATH} is missing: build it with `python -m paged_kv_split_amd.build`")
        L = ctypes.CDLL(LIB_PATH)
        P = ctypes.c_void_p
        PP = ctypes.POINTER(Problem)
        L.pkv_num_splits.argtypes = [PP, ctypes.c_int, ctypes.POINTER(ctypes.c_int)]
        L.pkv_plan.argtypes = [PP, ctypes.c_int, ctypes.POINTER(PlanInfo)]
        L.pkv_plan_varlen.argtypes = [PP, ctypes.c_int64, ctypes.c_int, ctypes.POINTER(PlanInfo)]
        L.pkv_workspace_bytes.argtypes = [PP, ctypes.c_int, ctypes.POINTER(ctypes.c_size_t),
                                          ctypes.POINTER(ctypes.c_size_t)]
        L.pkv_workspace_clear.argtypes = [P, ctypes.c_size_t, P]
        L.pkv_paged_decode.argtypes = [PP, P, P, P, P, P, P, P, P, ctypes.c_size_t, P,
                                       ctypes.c_size_t, P, P, P]
        L.pkv_paged_decode_partials.argtypes = [PP, P, P, P, P, P, P, P, P, ctypes.c_size_t, P,
                                                ctypes.c_size_t, P]
        L.pkv_paged_decode_noalloc.argtypes = [PP, P, P, P, P, P, P, P, P, P, P]
        L.pkv_paged_decode_varlen.argtypes = [PP, P, ctypes.c_int64, P, P, P, P, P, P, P, P,
                                              ctypes.c_size_t, P, ctypes.c_size_t, P, P, P]
        L.pkv_contiguous_decode.argtypes = [PP, ctypes.c_int, ctypes.c_int64, P, P, P, P, P, P, P,
                                            ctypes.c_size_t, P, ctypes.c_size_t, P, P, P]
        L.pkv_combine.argtypes = [ctypes.c_int64, ctypes.c_int, ctypes.c_int, P, P, P, P, P]
        L.pkv_device_cus.argtypes = [ctypes.POINTER(ctypes.c_int)]
        L.pkv_status_string.argtypes = [ctypes.c_int]
        L.pkv_status_string.restype = ctypes.c_char_p
        for name in ("pkv_num_splits", "pkv_plan", "pkv_plan_varlen", "pkv_workspace_bytes", "pkv_workspace_clear", "pkv_paged_decode",
                     "pkv_paged_decode_noalloc", "pkv_paged_decode_varlen", "pkv_contiguous_decode",
                     "pkv_paged_decode_partials", "pkv_combine", "pkv_device_cus"):
            getattr(L, name).restype = ctypes.c_int
        _lib = L
    return _lib


def status_string(status: int) -> str:
    return lib().pkv_status_string(int(status)).decode()


def _check(status: int, where: str) -> None:
    if status != PKV_OK:
        raise PkvError(status, where)


def make_problem(*, batch: int, q_len: int, num_q_heads: int, num_kv_heads: int, head_dim: int,
                 page_size: int, num_pages: int, max_pages_per_seq: int, max_kv_len: int = 0,
                 scale: float = 1.0, causal_offset: int = -1, num_splits: int = 0,
                 mask_stride_b: int = 0, mask_stride_q: int = 0, heads_per_block: int = 0) -> Problem:
    return Problem(batch, q_len, num_q_heads, num_kv_heads, head_dim, page_size, num_pages,
                   max_pages_per_seq, max_kv_len, scale, causal_offset, num_splits,
                   mask_stride_b, mask_stride_q, heads_per_block)


def device_cus() -> int:
    n = ctypes.c_int(0)
    _check(lib().pkv_device_cus(ctypes.byref(n)), "pkv_device_cus")
    return n.value


def num_splits(problem: Problem, num_cus: int = 0) -> int:
    s = ctypes.c_int(0)
    _check(lib().pkv_num_splits(ctypes.byref(problem), int(num_cus), ctypes.byref(s)), "pkv_num_splits")
    return s.value


def plan(problem: Problem, num_cus: int = 0) -> PlanInfo:
    """pkv_plan: the launch plan pkv_paged_decode follows (splits, kv heads
    per workgroup, kernel, units, merge path, launches per call)."""
    info = PlanInfo()
    _check(lib().pkv_plan(ctypes.byref(problem), int(num_cus), ctypes.byref(info)), "pkv_plan")
    return info


def plan_varlen(problem: Problem, total_tokens: int, num_cus: int = 0) -> PlanInfo:
    """pkv_plan_varlen: the launch plan of a varlen call over total_tokens tokens."""
    info = PlanInfo()
    _check(lib().pkv_plan_varlen(ctypes.byref(problem), int(total_tokens), num_cus, ctypes.byref(info)),
           "pkv_plan_varlen")
    return info


def workspace_bytes(problem: Problem, splits: int) -> tuple[int, int]:
    o = ctypes.c_size_t(0)
    ml = ctypes.c_size_t(0)
    _check(lib().pkv_workspace_bytes(ctypes.byref(problem), int(splits), ctypes.byref(o), ctypes.byref(ml)),
           "pkv_workspace_bytes")
    return o.value, ml.value


def workspace_clear_raw(ptr: int, nbytes: int, stream: int) -> int:
    """pkv_workspace_clear on a raw address; returns the status code."""
    return lib().pkv_workspace_clear(ptr or None, int(nbytes), stream or None)


def workspace_clear(t, stream=None) -> None:
    """Zero a workspace tensor with the library's fill kernel."""
    _check(workspace_clear_raw(_ptr(t), t.numel() * t.element_size(), _stream_handle(stream)),
           "pkv_workspace_clear")


def alloc_workspace(problem: Problem, splits: int, device):
    """(o_part, ml_part) fp32 device tensors for pkv_paged_decode with
    ``splits`` splits, ml_part zeroed (its counter head must start at zero);
    (None, None) for one split."""
    import torch
    if splits <= 1:
        return None, None
    ob, mb = workspace_bytes(problem, splits)
    return (torch.empty(ob // 4, dtype=torch.float32, device=device),
            torch.zeros(mb // 4, dtype=torch.float32, device=device))


def paged_decode_raw(problem: Problem, q: int, k_cache: int, v_cache: int, block_table: int,
                     kv_lens: int, causal_offsets: int, mask: int, o_part: int, o_part_bytes: int,
                     ml_part: int, ml_part_bytes: int, out_bf16: int, out_f32: int, stream: int) -> int:
    """pkv_paged_decode on raw addresses (0 = NULL); returns the status code."""
    return lib().pkv_paged_decode(ctypes.byref(problem), q or None, k_cache or None, v_cache or None,
                                  block_table or None, kv_lens or None, causal_offsets or None,
                                  mask or None, o_part or None, o_part_bytes, ml_part or None,
                                  ml_part_bytes, out_bf16 or None, out_f32 or None, stream or None)


def paged_decode_noalloc_raw(problem: Problem, q: int, k_cache: int, v_cache: int, block_table: int,
                             kv_lens: int, causal_offsets: int, mask: int, out_bf16: int, out_f32: int,
                             stream: int) -> int:
    """pkv_paged_decode_noalloc on raw addresses (0 = NULL); returns the status code."""
    return lib().pkv_paged_decode_noalloc(ctypes.byref(problem), q or None, k_cache or None, v_cache or None,
                                          block_table or None, kv_lens or None, causal_offsets or None,
                                          mask or None, out_bf16 or None, out_f32 or None, stream or None)


def paged_decode_varlen_raw(problem: Problem, cu_q_lens: int, total_tokens: int, q: int, k_cache: int,
                            v_cache: int, block_table: int, kv_lens: int, causal_offsets: int, mask: int,
                            o_part: int, o_part_bytes: int, ml_part: int, ml_part_bytes: int, out_bf16: int,
                            out_f32: int, stream: int) -> int:
    """pkv_paged_decode_varlen on raw addresses (0 = NULL); returns the status code."""
    return lib().pkv_paged_decode_varlen(ctypes.byref(problem), cu_q_lens or None, int(total_tokens), q or None,
                                         k_cache or None, v_cache or None, block_table or None, kv_lens or None,
                                         causal_offsets or None, mask or None, o_part or None, o_part_bytes,
                                         ml_part or None, ml_part_bytes, out_bf16 or None, out_f32 or None,
                                         stream or None)


def contiguous_decode_raw(problem: Problem, kv_layout: int, kv_capacity: int, q: int, k_cache: int, v_cache: int,
                          kv_lens: int, causal_offsets: int, mask: int, o_part: int, o_part_bytes: int,
                          ml_part: int, ml_part_bytes: int, out_bf16: int, out_f32: int, stream: int) -> int:
    """pkv_contiguous_decode on raw addresses (0 = NULL); returns the status code."""
    return lib().pkv_contiguous_decode(ctypes.byref(problem), int(kv_layout), int(kv_capacity), q or None,
                                       k_cache or None, v_cache or None, kv_lens or None, causal_offsets or None,
                                       mask or None, o_part or None, o_part_bytes, ml_part or None,
                                       ml_part_bytes, out_bf16 or None, out_f32 or None, stream or None)


def paged_decode_partials_raw(problem: Problem, q: int, k_cache: int, v_cache: int, block_table: int,
                              kv_lens: int, causal_offsets: int, mask: int, o_part: int,
                              o_part_bytes: int, ml_part: int, ml_part_bytes: int, stream: int) -> int:
    """pkv_paged_decode_partials on raw addresses (0 = NULL); returns the status code."""
    return lib().pkv_paged_decode_partials(ctypes.byref(problem), q or None, k_cache or None,
                                           v_cache or None, block_table or None, kv_lens or None,
                                           causal_offsets or None, mask or None, o_part or None,
                                           o_part_bytes, ml_part or None, ml_part_bytes, stream or None)


def combine_raw(rows: int, splits: int, head_dim: int, o_part: int, ml_part: int, out_bf16: int,
                out_f32: int, stream: int) -> int:
    """pkv_combine on raw addresses (0 = NULL); returns the status code."""
    return lib().pkv_combine(int(rows), int(splits), int(head_dim), o_part or None, ml_part or None,
                             out_bf16 or None, out_f32 or None, stream or None)


# ---- torch-facing helpers (device memory and streams only) ----------------

def _ptr(t) -> int:
    return 0 if t is None else int(t.data_ptr())


def _stream_handle(stream) -> int:
    import torch
    s = stream if stream is not None else torch.cuda.current_stream()
    return int(s.cuda_stream)


def _call_stream(stream):
    """The torch stream a call runs on: ``stream``, else the current one.
    Outputs and workspace that a wrapper allocates are allocated with this
    stream current, so torch's caching allocator ties them to it (their memory
    is not handed to other streams while the call's kernels may still use
    it) and the zero fill of a new workspace is queued on it, ahead of the
    call."""
    import torch
    return stream if stream is not None else torch.cuda.current_stream()


def _require(t, name, dtype, ndim=None):
    import torch
    if t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if not t.is_cuda:
        raise TypeError(f"{name} must be a device tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if ndim is not None and t.dim() != ndim:
        raise ValueError(f"{name} must have {ndim} dims, got {t.dim()}")


def problem_for(q, k_cache, block_table, *, scale: float, causal_offset: int = -1, mask=None,
                num_splits: int = 0, max_kv_len: int = 0) -> Problem:
    B, q_len, Hq, D = q.shape
    num_pages, P, Hkv, D2 = k_cache.shape
    if D2 != D:
        raise ValueError("q and k_cache head dims differ")
    msb = msq = 0
    if mask is not None:
        if mask.dim() == 2:
            msb = mask.stride(0)
        elif mask.dim() == 3:
            msb, msq = mask.stride(0), mask.stride(1)
        else:
            raise ValueError("mask must be [B, kv] or [B, q_len, kv]")
    return make_problem(batch=B, q_len=q_len, num_q_heads=Hq, num_kv_heads=Hkv, head_dim=D,
                        page_size=P, num_pages=num_pages, max_pages_per_seq=block_table.shape[1],
                        max_kv_len=max_kv_len, scale=scale, causal_offset=causal_offset,
                        num_splits=num_splits, mask_stride_b=msb, mask_stride_q=msq)


def paged_decode(q, k_cache, v_cache, block_table, kv_lens, *, scale: float,
                 causal_offset: int = -1, causal_offsets=None, mask=None, num_splits: int = 0,
                 max_kv_len: int = 0, out=None, out_f32=None, o_part=None, ml_part=None,
                 stream=None, problem: Optional[Problem] = None):
    """Paged decode on torch device tensors.  Returns ``out`` (bf16).

    q bf16 [B, q_len, Hq, D]; k_cache, v_cache bf16 [num_pages, page_size,
    Hkv, D]; block_table int32 [B, max_pages]; kv_lens int32 [B];
    causal_offsets optional int32 [B]; mask optional fp32 [B, kv] or
    [B, q_len, kv] (last dim contiguous).  ``out``/``out_f32``/``o_part``/
    ``ml_part`` may be passed preallocated (required for graph capture; see
    ``alloc_workspace``: ml_part's counter head must be zero before its first
    use, and the library leaves it zero); missing ones are allocated here,
    outside the library call.
    """
    import torch
    _require(q, "q", torch.bfloat16, 4)
    _require(k_cache, "k_cache", torch.bfloat16, 4)
    _require(v_cache, "v_cache", torch.bfloat16, 4)
    _require(block_table, "block_table", torch.int32, 2)
    _require(kv_lens, "kv_lens", torch.int32, 1)
    if k_cache.shape != v_cache.shape:
        raise ValueError("k_cache and v_cache shapes differ")
    if causal_offsets is not None:
        _require(causal_offsets, "causal_offsets", torch.int32, 1)
    if mask is not None:
        if mask.dtype != torch.float32 or not mask.is_cuda or mask.stride(-1) != 1:
            raise ValueError("mask must be a device float32 tensor with a contiguous last dim")
    p = problem if problem is not None else problem_for(q, k_cache, block_table, scale=scale,
                                                         causal_offset=causal_offset, mask=mask,
                                                         num_splits=num_splits, max_kv_len=max_kv_len)
    S = num_splits_for(p)
    s = _call_stream(stream)
    with torch.cuda.stream(s):
        if out is None:
            out = torch.empty(q.shape, dtype=torch.bfloat16, device=q.device)
        if S > 1 and (o_part is None or ml_part is None):
            o_part, ml_part = alloc_workspace(p, S, q.device)
    st = paged_decode_raw(p, _ptr(q), _ptr(k_cache), _ptr(v_cache), _ptr(block_table), _ptr(kv_lens),
                          _ptr(causal_offsets), _ptr(mask), _ptr(o_part),
                          0 if o_part is None else o_part.numel() * o_part.element_size(),
                          _ptr(ml_part), 0 if ml_part is None else ml_part.numel() * ml_part.element_size(),
                          _ptr(out), _ptr(out_f32), int(s.cuda_stream))
    _check(st, "pkv_paged_decode")
    return out


def paged_decode_varlen(q, k_cache, v_cache, block_table, kv_lens, cu_q_lens, *, max_q_len: int,
                        scale: float, causal_offset: int = PKV_CAUSAL_LAST, causal_offsets=None, mask=None,
                        num_splits: int = 0, max_kv_len: int = 0, heads_per_block: int = 0, out=None,
                        out_f32=None, o_part=None, ml_part=None, stream=None):
    """Paged decode over sequences with different query-token counts.
    Returns ``out`` (bf16 [T, Hq, D]).

    q bf16 [T, Hq, D], the tokens of sequence b at rows cu_q_lens[b] ..
    cu_q_lens[b+1] - 1; cu_q_lens int32 [B + 1] on the device with
    cu_q_lens[B] = T; max_q_len bounds every sequence's token count (the
    launch is sized for it); causal_offset defaults to PKV_CAUSAL_LAST (each
    sequence's tokens are its last keys); mask optional fp32 [B, kv] or
    [B, max_q_len, kv].  Other arguments as for ``paged_decode``.
    """
    import torch
    _require(q, "q", torch.bfloat16, 3)
    _require(k_cache, "k_cache", torch.bfloat16, 4)
    _require(v_cache, "v_cache", torch.bfloat16, 4)
    _require(block_table, "block_table", torch.int32, 2)
    _require(kv_lens, "kv_lens", torch.int32, 1)
    _require(cu_q_lens, "cu_q_lens", torch.int32, 1)
    if k_cache.shape != v_cache.shape:
        raise ValueError("k_cache and v_cache shapes differ")
    B = kv_lens.shape[0]
    if cu_q_lens.shape[0] != B + 1:
        raise ValueError("cu_q_lens must have batch + 1 entries")
    if causal_offsets is not None:
        _require(causal_offsets, "causal_offsets", torch.int32, 1)
    msb = msq = 0
    if mask is not None:
        if mask.dtype != torch.float32 or not mask.is_cuda or mask.stride(-1) != 1:
            raise ValueError("mask must be a device float32 tensor with a contiguous last dim")
        msb = mask.stride(0)
        msq = mask.stride(1) if mask.dim() == 3 else 0
    T, Hq, D = q.shape
    num_pages, P, Hkv, _ = k_cache.shape
    p = make_problem(batch=B, q_len=max_q_len, num_q_heads=Hq, num_kv_heads=Hkv, head_dim=D, page_size=P,
                     num_pages=num_pages, max_pages_per_seq=block_table.shape[1], max_kv_len=max_kv_len,
                     scale=scale, causal_offset=causal_offset, num_splits=num_splits, mask_stride_b=msb,
                     mask_stride_q=msq, heads_per_block=heads_per_block)
    S = num_splits if num_splits > 0 else plan_varlen(p, T).splits
    s = _call_stream(stream)
    with torch.cuda.stream(s):
        if out is None:
            out = torch.empty(q.shape, dtype=torch.bfloat16, device=q.device)
        if S > 1 and (o_part is None or ml_part is None):
            o_part, ml_part = alloc_workspace(p, S, q.device)
    st = paged_decode_varlen_raw(p, _ptr(cu_q_lens), T, _ptr(q), _ptr(k_cache), _ptr(v_cache), _ptr(block_table),
                                 _ptr(kv_lens), _ptr(causal_offsets), _ptr(mask), _ptr(o_part),
                                 0 if o_part is None else o_part.numel() * o_part.element_size(), _ptr(ml_part),
                                 0 if ml_part is None else ml_part.numel() * ml_part.element_size(), _ptr(out),
                                 _ptr(out_f32), int(s.cuda_stream))
    _check(st, "pkv_paged_decode_varlen")
    return out


def contiguous_problem(*, batch: int, q_len: int, num_q_heads: int, num_kv_heads: int, head_dim: int,
                       kv_capacity: int, max_kv_len: int = 0, scale: float = 1.0, causal_offset: int = -1,
                       num_splits: int = 0, mask_stride_b: int = 0, mask_stride_q: int = 0,
                       heads_per_block: int = 0) -> Problem:
    """The problem pkv_contiguous_decode plans with (its paged fields describe
    one page of kv_capacity keys per sequence), so that ``plan``,
    ``num_splits`` and ``workspace_bytes`` report what a contiguous call does."""
    return make_problem(batch=batch, q_len=q_len, num_q_heads=num_q_heads, num_kv_heads=num_kv_heads,
                        head_dim=head_dim, page_size=1, num_pages=0, max_pages_per_seq=kv_capacity,
                        max_kv_len=max_kv_len if max_kv_len > 0 else kv_capacity, scale=scale,
                        causal_offset=causal_offset, num_splits=num_splits, mask_stride_b=mask_stride_b,
                        mask_stride_q=mask_stride_q, heads_per_block=heads_per_block)


def contiguous_decode(q, k_cache, v_cache, kv_lens, *, layout: str = "blhd", scale: float,
                      causal_offset: int = -1, causal_offsets=None, mask=None, num_splits: int = 0,
                      max_kv_len: int = 0, heads_per_block: int = 0, out=None, out_f32=None, o_part=None,
                      ml_part=None, stream=None):
    """Decode over contiguous K/V on torch device tensors.  Returns ``out`` (bf16).

    layout "blhd": k_cache, v_cache bf16 [B, kv_capacity, Hkv, D]; "bhld":
    [B, Hkv, kv_capacity, D].  Other arguments as for ``paged_decode``.
    """
    import torch
    _require(q, "q", torch.bfloat16, 4)
    _require(k_cache, "k_cache", torch.bfloat16, 4)
    _require(v_cache, "v_cache", torch.bfloat16, 4)
    _require(kv_lens, "kv_lens", torch.int32, 1)
    if layout not in KV_LAYOUTS:
        raise ValueError(f"layout must be one of {sorted(KV_LAYOUTS)}")
    if k_cache.shape != v_cache.shape:
        raise ValueError("k_cache and v_cache shapes differ")
    B, q_len, Hq, D = q.shape
    if layout == "blhd":
        Bk, cap, Hkv, Dk = k_cache.shape
    else:
        Bk, Hkv, cap, Dk = k_cache.shape
    if Bk != B or Dk != D:
        raise ValueError("k_cache does not match q in batch or head dim")
    if causal_offsets is not None:
        _require(causal_offsets, "causal_offsets", torch.int32, 1)
    msb = msq = 0
    if mask is not None:
        if mask.dtype != torch.float32 or not mask.is_cuda or mask.stride(-1) != 1:
            raise ValueError("mask must be a device float32 tensor with a contiguous last dim")
        msb = mask.stride(0)
        msq = mask.stride(1) if mask.dim() == 3 else 0
    p = contiguous_problem(batch=B, q_len=q_len, num_q_heads=Hq, num_kv_heads=Hkv, head_dim=D, kv_capacity=cap,
                           max_kv_len=max_kv_len, scale=scale, causal_offset=causal_offset, num_splits=num_splits,
                           mask_stride_b=msb, mask_stride_q=msq, heads_per_block=heads_per_block)
    S = num_splits_for(p)
    s = _call_stream(stream)
    with torch.cuda.stream(s):
        if out is None:
            out = torch.empty(q.shape, dtype=torch.bfloat16, device=q.device)
        if S > 1 and (o_part is None or ml_part is None):
            o_part, ml_part = alloc_workspace(p, S, q.device)
    st = contiguous_decode_raw(p, KV_LAYOUTS[layout], cap, _ptr(q), _ptr(k_cache), _ptr(v_cache), _ptr(kv_lens),
                               _ptr(causal_offsets), _ptr(mask), _ptr(o_part),
                               0 if o_part is None else o_part.numel() * o_part.element_size(),
                               _ptr(ml_part), 0 if ml_part is None else ml_part.numel() * ml_part.element_size(),
                               _ptr(out), _ptr(out_f32), int(s.cuda_stream))
    _check(st, "pkv_contiguous_decode")
    return out


def paged_decode_partials(q, k_cache, v_cache, block_table, kv_lens, *, o_part, ml_part,
                          problem: Problem, causal_offsets=None, mask=None, stream=None):
    """Split step only: writes o_part [B, q_len, Hq, S, D] and ml_part
    [B, q_len, Hq, S, 2] (fp32, preallocated) for the problem's split count."""
    st = paged_decode_partials_raw(problem, _ptr(q), _ptr(k_cache), _ptr(v_cache), _ptr(block_table),
                                   _ptr(kv_lens), _ptr(causal_offsets), _ptr(mask), _ptr(o_part),
                                   o_part.numel() * o_part.element_size(), _ptr(ml_part),
                                   ml_part.numel() * ml_part.element_size(), _stream_handle(stream))
    _check(st, "pkv_paged_decode_partials")


def partials_bytes(problem: Problem, splits: int) -> tuple[int, int]:
    """o_part / ml_part bytes pkv_paged_decode_partials needs (any split count)."""
    rows = problem.batch * problem.q_len * problem.num_q_heads
    return rows * splits * problem.head_dim * 4, rows * splits * 8


def merges_in_kernel(problem: Problem, splits: int, num_cus: int = 0) -> bool:
    """Whether pkv_paged_decode with ``splits`` splits merges them inside the
    split kernel rather than launching the combine kernel (pkv_plan)."""
    p = Problem.from_buffer_copy(problem)
    p.num_splits = splits
    return bool(plan(p, num_cus).merge_in_kernel)


def kernel_family(problem: Problem) -> str:
    """Which split kernel serves the problem (pkv_plan)."""
    return KERNEL_NAMES[plan(problem).kernel]


def num_splits_for(problem: Problem) -> int:
    """Split count the library will use (forced, or the heuristic on this device)."""
    if problem.num_splits > 0:
        return problem.num_splits
    return num_splits(problem, 0)


def combine(o_part, ml_part, *, rows: int, splits: int, head_dim: int, out=None, out_f32=None,
            stream=None):
    """pkv_combine on torch tensors: o_part fp32 [rows, S, D], ml_part fp32 [rows, S, 2]."""
    import torch
    _require(o_part, "o_part", torch.float32)
    _require(ml_part, "ml_part", torch.float32)
    s = _call_stream(stream)
    if out is None:
        with torch.cuda.stream(s):
            out = torch.empty((rows, head_dim), dtype=torch.bfloat16, device=o_part.device)
    _check(combine_raw(rows, splits, head_dim, _ptr(o_part), _ptr(ml_part), _ptr(out), _ptr(out_f32),
                       int(s.cuda_stream)), "pkv_combine")
    return out
