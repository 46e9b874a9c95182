"""Device-side marshalling of one paged-attention problem.

``DeviceProblem`` takes any object with the workload attributes (batch,
heads, dims, page size, q / k_cache / v_cache / scales / lengths / block
table as NumPy arrays, and the dtype / scale-mode / causal / sm_scale /
chunk_size / decode_q_len / shared_kv settings), copies the arrays to the GPU
with torch, describes them with a ``PaProblem`` and calls the C ABI.  It
computes nothing itself.
"""
from __future__ import annotations

import numpy as np

from . import _lib as L

_Q_DTYPES = {"bf16": L.DTYPE_BF16, "f32": L.DTYPE_F32}
_KV_DTYPES = {"i8": L.DTYPE_I8, "fp8_e4m3": L.DTYPE_FP8_E4M3}
_SCALE_MODES = {"tensor": L.SCALE_PER_TENSOR, "head": L.SCALE_PER_HEAD, "channel": L.SCALE_PER_CHANNEL}


def problem_for(w, chunk_size=None, q_row_stride=None, flags=0) -> L.PaProblem:
    """The pa_problem of a workload stored as contiguous
    [num_pages, H_kv, P, D] caches and [total_q, H_q, D_qk] queries."""
    H, P = w.num_kv_heads, w.page_size
    kD = w.k_cache.shape[-1]
    vD = kD if w.shared_kv else w.v_cache.shape[-1]
    return L.make_problem(
        batch=w.batch, num_q_heads=w.num_q_heads, num_kv_heads=H, head_dim_qk=w.head_dim_qk,
        head_dim_v=w.head_dim_v, page_size=P, num_pages=w.num_pages,
        max_pages_per_seq=int(w.block_table.shape[1]), max_q_len=int(w.q_lens.max()) if w.batch else 0,
        max_kv_len=int(w.seq_lens_kv.max()) if w.batch else 0,
        q_row_stride=int(q_row_stride if q_row_stride is not None else w.num_q_heads * w.head_dim_qk),
        k_stride_page=H * P * kD, k_stride_head=P * kD, k_stride_token=kD,
        v_stride_page=H * P * vD, v_stride_head=P * vD, v_stride_token=vD,
        q_dtype=_Q_DTYPES[w.q_dtype], kv_dtype=_KV_DTYPES[w.kv_dtype],
        scale_mode=_SCALE_MODES[w.scale_mode], causal=int(bool(w.causal)),
        sm_scale=float(w.sm_scale), chunk_size=int(w.chunk_size if chunk_size is None else chunk_size),
        flags=int(flags))


class DeviceProblem:
    """Device tensors of a workload plus its outputs and workspace."""

    def __init__(self, w, device="cuda", chunk_size=None, decode=None, defer_merge=False, fused_merge=False,
                 balanced=False, schedule=None, persistent=False):
        import torch
        self.torch = torch
        self.w = w
        dev = torch.device(device)
        self.decode = (w.decode_q_len is not None) if decode is None else decode
        if w.q_dtype == "bf16":
            self.q = torch.from_numpy(np.ascontiguousarray(w.q).view(np.int16)).view(torch.bfloat16).to(dev)
        else:
            self.q = torch.from_numpy(np.ascontiguousarray(w.q, dtype=np.float32)).to(dev)
        self.k_cache = torch.from_numpy(np.ascontiguousarray(w.k_cache)).to(dev)
        self.v_cache = self.k_cache if w.shared_kv else torch.from_numpy(np.ascontiguousarray(w.v_cache)).to(dev)
        self.k_scale = torch.from_numpy(np.ascontiguousarray(w.k_scale, dtype=np.float32)).to(dev)
        self.v_scale = torch.from_numpy(np.ascontiguousarray(w.v_scale, dtype=np.float32)).to(dev)
        self.seq_lens_kv = torch.from_numpy(np.ascontiguousarray(w.seq_lens_kv, dtype=np.int32)).to(dev)
        self.q_lens = torch.from_numpy(np.ascontiguousarray(w.q_lens, dtype=np.int32)).to(dev)
        self.cu_seqlens_q = torch.from_numpy(np.ascontiguousarray(w.cu_seqlens_q, dtype=np.int32)).to(dev)
        self.block_table = torch.from_numpy(np.ascontiguousarray(w.block_table, dtype=np.int32)).to(dev)
        tm = getattr(w, "tree_mask", None)
        self.tree_mask = None if tm is None else torch.from_numpy(np.ascontiguousarray(tm, dtype=np.uint8)).to(dev)
        flags = ((L.FLAG_DEFER_MERGE if defer_merge else 0) | (L.FLAG_FUSED_MERGE if fused_merge else 0) |
                 (L.FLAG_BALANCED_SPLIT if balanced else 0) | (L.FLAG_PERSISTENT if persistent else 0))
        self.prob = problem_for(w, chunk_size=chunk_size, flags=flags)
        for k, v in (schedule or {}).items():   # pa_problem schedule overrides
            if k not in L.SCHEDULE_FIELDS:
                raise KeyError(k)
            setattr(self.prob, k, int(v))
        self.total_q = int(w.total_q)
        self.out = torch.empty((self.total_q, w.num_q_heads, w.head_dim_v), dtype=torch.bfloat16, device=dev)
        self.lse = torch.empty((self.total_q, w.num_q_heads), dtype=torch.float32, device=dev)
        ws = L.workspace_size(self.prob, self.total_q)
        # the in-kernel merge's counters must start at zero (each call leaves them zero)
        alloc = torch.zeros if fused_merge or persistent else torch.empty
        self.workspace = alloc(max(ws, 256), dtype=torch.uint8, device=dev) if ws else None
        self.workspace_bytes = ws

    def run(self, stream=None) -> None:
        """Enqueue one attention call (plus the split-KV merge when chunked)."""
        if self.tree_mask is not None:
            L.paged_attn_decode_tree(self.prob, int(self.w.decode_q_len), self.q, self.k_cache, self.v_cache,
                                     self.k_scale, self.v_scale, self.seq_lens_kv, self.block_table,
                                     self.tree_mask, int(self.tree_mask.shape[1]), self.out, self.lse,
                                     self.workspace, self.workspace_bytes, stream)
        elif self.decode:
            L.paged_attn_decode(self.prob, int(self.w.decode_q_len), self.q, self.k_cache, self.v_cache,
                                self.k_scale, self.v_scale, self.seq_lens_kv, self.block_table, self.out,
                                self.lse, self.workspace, self.workspace_bytes, stream)
        else:
            L.paged_attn_append(self.prob, self.total_q, self.q, self.k_cache, self.v_cache,
                                self.k_scale, self.v_scale, self.cu_seqlens_q, self.seq_lens_kv,
                                self.block_table, self.out, self.lse, self.workspace,
                                self.workspace_bytes, stream)

    def merge(self, stream=None) -> None:
        """Enqueue split_kv_merge over this problem's workspace (the second half
        of a call made with defer_merge=True; a no-op without split-KV)."""
        C = int(self.prob.chunk_size)
        if C <= 0:
            return
        w = self.w
        mc = max(1, -(-(int(self.prob.max_kv_len) + int(self.prob.max_q_len)) // C))
        po_bytes = self.total_q * mc * w.num_q_heads * w.head_dim_v * 4
        base = self.workspace.data_ptr()
        L.split_kv_merge(base, base + (po_bytes + 255) // 256 * 256,
                         None if self.decode else self.cu_seqlens_q, self.seq_lens_kv,
                         int(w.decode_q_len) if self.decode else 0, w.batch, self.total_q,
                         int(self.prob.max_q_len), w.num_q_heads, w.head_dim_v, C, mc, self.out, self.lse,
                         stream)

    def outputs(self):
        """(out as float64 NumPy, lse as float64 NumPy) after synchronizing."""
        self.torch.cuda.synchronize()
        return (self.out.float().cpu().numpy().astype(np.float64),
                self.lse.cpu().numpy().astype(np.float64))
