"""ctypes binding of libpagedattn.so (the C ABI declared in include/pagedattn.h).

Argument marshalling only: every step of the computation runs in the HIP
kernels behind the C ABI.  Tensors are passed as raw device pointers; torch is
used for device memory and the current stream.  A missing library is an
error, never a fallback.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional

LIB_NAME = "libpagedattn.so"
LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), LIB_NAME)

PA_OK = 0
PA_ERR_INVALID_ARG = 1
PA_ERR_UNSUPPORTED = 2
PA_ERR_WORKSPACE_TOO_SMALL = 3
PA_ERR_HIP = 4

DTYPE_BF16 = 0
DTYPE_F32 = 1
DTYPE_I8 = 2
DTYPE_FP8_E4M3 = 3

SCALE_PER_TENSOR = 0
SCALE_PER_HEAD = 1
SCALE_PER_CHANNEL = 2

FLAG_DEFER_MERGE = 1
FLAG_FUSED_MERGE = 2
FLAG_BALANCED_SPLIT = 4
FLAG_PERSISTENT = 8

GATHER_ROWS = 0       # one key row at a time
GATHER_DECODE = 1     # the decode kernel's register tile loader
GATHER_DMA_4W = 2     # the LDS-DMA tile loader, 4 waves
GATHER_DMA_3W = 3     # the LDS-DMA tile loader, 3 waves
GATHER_DMA_MLA32 = 4  # the LDS-DMA tile loader as the e4m3fn MLA kernel drives it (32-key tiles)

#: Size of the static scratch behind paged_attn_decode_scratch (PA_DECODE_SCRATCH_BYTES).
DECODE_SCRATCH_BYTES = 32 << 20

#: Every entry point include/pagedattn.h declares.
EXPORTS = (
    "paged_attn_workspace_size",
    "paged_attn_append",
    "paged_attn_decode",
    "paged_attn_decode_tree",
    "paged_attn_decode_scratch",
    "paged_kv_write",
    "split_kv_merge",
    "pa_gather_debug",
    "pa_kv_read_probe",
    "pa_status_string",
    "pa_last_error",
)


class PaProblem(ctypes.Structure):
    """Mirror of ``pa_problem``."""
    _fields_ = [
        ("batch", ctypes.c_int32),
        ("num_q_heads", ctypes.c_int32),
        ("num_kv_heads", ctypes.c_int32),
        ("head_dim_qk", ctypes.c_int32),
        ("head_dim_v", ctypes.c_int32),
        ("page_size", ctypes.c_int32),
        ("num_pages", ctypes.c_int32),
        ("max_pages_per_seq", ctypes.c_int32),
        ("max_q_len", ctypes.c_int32),
        ("max_kv_len", ctypes.c_int32),
        ("q_row_stride", ctypes.c_int64),
        ("k_stride_page", ctypes.c_int64),
        ("k_stride_head", ctypes.c_int64),
        ("k_stride_token", ctypes.c_int64),
        ("v_stride_page", ctypes.c_int64),
        ("v_stride_head", ctypes.c_int64),
        ("v_stride_token", ctypes.c_int64),
        ("q_dtype", ctypes.c_int32),
        ("kv_dtype", ctypes.c_int32),
        ("scale_mode", ctypes.c_int32),
        ("causal", ctypes.c_int32),
        ("sm_scale", ctypes.c_float),
        ("chunk_size", ctypes.c_int32),
        ("flags", ctypes.c_int32),
        ("decode_waves", ctypes.c_int32),
        ("group_order", ctypes.c_int32),
        ("merge_in_kernel", ctypes.c_int32),
    ]

#: Schedule-override fields of ``pa_problem`` (0 = the library's choice).
SCHEDULE_FIELDS = ("decode_waves", "group_order", "merge_in_kernel")


class PagedAttnError(RuntimeError):
    def __init__(self, status: int, name: str, detail: str):
        super().__init__(f"{name} ({status}): {detail}")
        self.status = status
        self.name = name
        self.detail = detail


_lib = None

_P = ctypes.c_void_p
_I32 = ctypes.c_int32


def lib() -> ctypes.CDLL:
    """Load libpagedattn.so from the package directory (raises if absent)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(
            f"{LIB_PATH} is missing: build it with `python -m paged_kv_attention_gather_amd.build`")
    L = ctypes.CDLL(LIB_PATH)
    L.paged_attn_workspace_size.argtypes = [ctypes.POINTER(PaProblem), _I32]
    L.paged_attn_workspace_size.restype = ctypes.c_size_t
    L.paged_attn_append.argtypes = [ctypes.POINTER(PaProblem), _I32, _P, _P, _P, _P, _P, _P, _P, _P,
                                    _P, _P, _P, ctypes.c_size_t, _P]
    L.paged_attn_append.restype = _I32
    L.paged_attn_decode.argtypes = [ctypes.POINTER(PaProblem), _I32, _P, _P, _P, _P, _P, _P, _P,
                                    _P, _P, _P, ctypes.c_size_t, _P]
    L.paged_attn_decode.restype = _I32
    L.paged_attn_decode_scratch.argtypes = [ctypes.POINTER(PaProblem), _I32, _P, _P, _P, _P, _P, _P, _P,
                                            _P, _P, _P]
    L.paged_attn_decode_scratch.restype = _I32
    L.paged_attn_decode_tree.argtypes = [ctypes.POINTER(PaProblem), _I32, _P, _P, _P, _P, _P, _P, _P,
                                         _P, _I32, _P, _P, _P, ctypes.c_size_t, _P]
    L.paged_attn_decode_tree.restype = _I32
    L.paged_kv_write.argtypes = [ctypes.POINTER(PaProblem), _I32, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P]
    L.paged_kv_write.restype = _I32
    L.split_kv_merge.argtypes = [_P, _P, _P, _P, _I32, _I32, _I32, _I32, _I32, _I32, _I32, _I32,
                                 _P, _P, _P]
    L.split_kv_merge.restype = _I32
    L.pa_gather_debug.argtypes = [ctypes.POINTER(PaProblem), _I32, _P, _P, _P, _P, _P, _I32, _P, _P, _P]
    L.pa_kv_read_probe.argtypes = [ctypes.POINTER(PaProblem), _I32, _P, _P, _P, _P, _P, _P]
    L.pa_kv_read_probe.restype = _I32
    L.pa_gather_debug.restype = _I32
    L.pa_status_string.argtypes = [_I32]
    L.pa_status_string.restype = ctypes.c_char_p
    L.pa_last_error.argtypes = []
    L.pa_last_error.restype = ctypes.c_char_p
    _lib = L
    return L


def _check(status: int) -> None:
    if status != PA_OK:
        L = lib()
        raise PagedAttnError(status, L.pa_status_string(status).decode(), L.pa_last_error().decode())


def _ptr(x) -> Optional[int]:
    if x is None:
        return None
    if isinstance(x, int):
        return x
    return x.data_ptr()


def _nbytes(x) -> int:
    if x is None:
        return 0
    if isinstance(x, int):
        raise TypeError("pass workspace_bytes explicitly with a raw pointer")
    return x.numel() * x.element_size()


def _stream(stream) -> Optional[int]:
    if stream is None:
        import torch
        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, int):
        return stream
    return stream.cuda_stream


def make_problem(**fields) -> PaProblem:
    """Build a PaProblem from keyword fields (every field but ``flags`` and the
    schedule overrides, which default to 0, is required)."""
    fields.setdefault("flags", 0)
    for f in SCHEDULE_FIELDS:
        fields.setdefault(f, 0)
    names = [f for f, _ in PaProblem._fields_]
    missing = [n for n in names if n not in fields]
    extra = [k for k in fields if k not in names]
    if missing or extra:
        raise TypeError(f"missing fields {missing}, unknown fields {extra}")
    return PaProblem(**fields)


def workspace_size(prob: PaProblem, total_q: int) -> int:
    n = lib().paged_attn_workspace_size(ctypes.byref(prob), int(total_q))
    if n == ctypes.c_size_t(-1).value:
        raise PagedAttnError(PA_ERR_INVALID_ARG, "PA_ERR_INVALID_ARG", lib().pa_last_error().decode())
    return int(n)


def paged_attn_append(prob, total_q, q, k_cache, v_cache, k_scale, v_scale, cu_seqlens_q,
                      seq_lens_kv, block_table, out, lse=None, workspace=None,
                      workspace_bytes=None, stream=None) -> None:
    ws_bytes = _nbytes(workspace) if workspace_bytes is None else int(workspace_bytes)
    _check(lib().paged_attn_append(
        ctypes.byref(prob), int(total_q), _ptr(q), _ptr(k_cache), _ptr(v_cache), _ptr(k_scale),
        _ptr(v_scale), _ptr(cu_seqlens_q), _ptr(seq_lens_kv), _ptr(block_table), _ptr(out),
        _ptr(lse), _ptr(workspace), ws_bytes, _stream(stream)))


def paged_attn_decode(prob, q_len, q, k_cache, v_cache, k_scale, v_scale, seq_lens_kv,
                      block_table, out, lse=None, workspace=None, workspace_bytes=None,
                      stream=None) -> None:
    ws_bytes = _nbytes(workspace) if workspace_bytes is None else int(workspace_bytes)
    _check(lib().paged_attn_decode(
        ctypes.byref(prob), int(q_len), _ptr(q), _ptr(k_cache), _ptr(v_cache), _ptr(k_scale),
        _ptr(v_scale), _ptr(seq_lens_kv), _ptr(block_table), _ptr(out), _ptr(lse),
        _ptr(workspace), ws_bytes, _stream(stream)))


def paged_attn_decode_scratch(prob, q_len, q, k_cache, v_cache, k_scale, v_scale, seq_lens_kv,
                              block_table, out, lse=None, stream=None) -> None:
    _check(lib().paged_attn_decode_scratch(
        ctypes.byref(prob), int(q_len), _ptr(q), _ptr(k_cache), _ptr(v_cache), _ptr(k_scale),
        _ptr(v_scale), _ptr(seq_lens_kv), _ptr(block_table), _ptr(out), _ptr(lse), _stream(stream)))


def paged_attn_decode_tree(prob, q_len, q, k_cache, v_cache, k_scale, v_scale, seq_lens_kv,
                           block_table, tree_mask, tree_mask_len, out, lse=None, workspace=None,
                           workspace_bytes=None, stream=None) -> None:
    ws_bytes = _nbytes(workspace) if workspace_bytes is None else int(workspace_bytes)
    _check(lib().paged_attn_decode_tree(
        ctypes.byref(prob), int(q_len), _ptr(q), _ptr(k_cache), _ptr(v_cache), _ptr(k_scale),
        _ptr(v_scale), _ptr(seq_lens_kv), _ptr(block_table), _ptr(tree_mask), int(tree_mask_len),
        _ptr(out), _ptr(lse), _ptr(workspace), ws_bytes, _stream(stream)))


def paged_kv_write(prob, total_new, k_new, v_new, cu_seqlens_new, seq_lens_kv, block_table, k_scale,
                   v_scale, k_cache, v_cache, stream=None) -> None:
    _check(lib().paged_kv_write(
        ctypes.byref(prob), int(total_new), _ptr(k_new), _ptr(v_new), _ptr(cu_seqlens_new), _ptr(seq_lens_kv),
        _ptr(block_table), _ptr(k_scale), _ptr(v_scale), _ptr(k_cache), _ptr(v_cache), _stream(stream)))


def split_kv_merge(partial_o, partial_lse, cu_seqlens_q, seq_lens_kv, q_len_uniform, batch,
                   total_q, max_q_len, num_q_heads, head_dim_v, chunk_size, max_chunks, out,
                   lse=None, stream=None) -> None:
    _check(lib().split_kv_merge(
        _ptr(partial_o), _ptr(partial_lse), _ptr(cu_seqlens_q), _ptr(seq_lens_kv),
        int(q_len_uniform), int(batch), int(total_q), int(max_q_len), int(num_q_heads),
        int(head_dim_v), int(chunk_size), int(max_chunks), _ptr(out), _ptr(lse), _stream(stream)))


def pa_gather_debug(prob, k_cache, block_table, seq_lens_kv, q_lens, t_max, dst, stream=None,
                    loader=0, v_cache=None, v_dst=None) -> None:
    _check(lib().pa_gather_debug(
        ctypes.byref(prob), int(loader), _ptr(k_cache), _ptr(v_cache), _ptr(block_table), _ptr(seq_lens_kv),
        _ptr(q_lens), int(t_max), _ptr(dst), _ptr(v_dst), _stream(stream)))


def pa_kv_read_probe(prob, q_len, k_cache, v_cache, seq_lens_kv, block_table, sink, stream=None) -> None:
    _check(lib().pa_kv_read_probe(
        ctypes.byref(prob), int(q_len), _ptr(k_cache), _ptr(v_cache), _ptr(seq_lens_kv), _ptr(block_table),
        _ptr(sink), _stream(stream)))
