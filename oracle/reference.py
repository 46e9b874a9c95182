"""fp64 oracle: dequantize, gather pages, exact masked softmax attention,
split-KV partials and their log-sum-exp merge.

Notation: request b has n_b appended tokens (its q_len) and L_b cached tokens
(``seq_lens_kv[b]``); it attends over T_b = L_b + n_b keys, the appended
tokens' K/V being already in the cache (FastDeploy append_attention_c8_impl.cuh,
multi_query_append_attention_c8_kernel: ``kv_len = seq_lens_kv + q_len`` and the
K/V tiles are read from the cache only).  Query head h uses KV head
g = floor(h / G), G = H_q / H_kv (same kernel: ``q_head_idx = kv_head_idx *
GROUP_SIZE`` and the packed row -> head mapping of its output write).

This module is test infrastructure; see the package docstring.
"""
from __future__ import annotations

import math
from typing import Dict, Iterable, Optional, Tuple

import numpy as np



# ---------------------------------------------------------------- decoding ---

def bf16_bits_to_f64(bits: np.ndarray) -> np.ndarray:
    """Exact value of bf16 numbers given as uint16 bit patterns: a bf16 is
    the upper half of an IEEE binary32."""
    b = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16
    return b.view(np.float32).astype(np.float64)


def int8_decode(raw: np.ndarray) -> np.ndarray:
    """Cache byte -> value for the int8 cache: two's-complement signed byte.
    (The c8 kernel stores the cache as ``uint8_t`` and leaves the decode to a
    helper not printed on the page; the workloads state int8 values in
    [-127, 127], so the byte is read as a signed integer.)"""
    return np.asarray(raw, dtype=np.uint8).view(np.int8).astype(np.float64)


def e4m3fn_decode(raw: np.ndarray) -> np.ndarray:
    """Cache byte -> value for fp8 E4M3 in the OCP "fn" flavour (1 sign, 4
    exponent bits with bias 7, 3 mantissa bits, subnormals at exponent 0, no
    infinities, S.1111.111 is NaN, largest finite 448).  XQA's mla_sm120.cu
    scales by 1/kE4M3_MAX; the workloads fix that maximum at 448, which is
    this format, not the 240-max FNUZ variant."""
    r = np.asarray(raw, dtype=np.uint8).astype(np.int64)
    sign = np.where(r >> 7, -1.0, 1.0)
    exp = (r >> 3) & 0xF
    man = (r & 0x7).astype(np.float64)
    normal = (1.0 + man / 8.0) * np.ldexp(1.0, (exp - 7).astype(np.int32))
    subnormal = (man / 8.0) * math.ldexp(1.0, -6)
    val = np.where(exp == 0, subnormal, normal) * sign
    return np.where((exp == 0xF) & ((r & 0x7) == 0x7), np.nan, val)


def _decode(raw: np.ndarray, kv_dtype: str) -> np.ndarray:
    if kv_dtype == "i8":
        return int8_decode(raw)
    if kv_dtype == "fp8_e4m3":
        return e4m3fn_decode(raw)
    raise ValueError(kv_dtype)


def _scale_vector(scale: np.ndarray, mode: str, g: int, dim: int) -> np.ndarray:
    """Dequant multiplier for KV head g over ``dim`` channels.  Granularity is
    per tensor, per KV head ``[H_kv]`` or per channel ``[H_kv, D]`` (the c8
    kernel loads either one scale per KV head or one per (head, channel) and
    multiplies; XQA applies one ``kvCacheScale`` to every element)."""
    s = np.asarray(scale, dtype=np.float32).astype(np.float64)
    if mode == "tensor":
        return np.full(dim, s.reshape(-1)[0])
    if mode == "head":
        return np.full(dim, s.reshape(-1)[g])
    if mode == "channel":
        return s.reshape(-1, s.shape[-1])[g, :dim].copy()
    raise ValueError(mode)


# ------------------------------------------------------------------ gather ---

def gather_rows(cache: np.ndarray, table_row: np.ndarray, g: int, T: int,
                page_size: int, dim: int) -> np.ndarray:
    """Raw bytes of keys 0..T-1 of one request and KV head g.

    Key j lives in physical page ``table_row[j // P]`` at slot ``j % P``; its
    channels are the first ``dim`` bytes of that row (FlashInfer persistent.cuh,
    prefetch_offest: page/entry divmod of the packed position and
    ``indices[page] * stride_page + entry * stride_n + head * stride_h``; XQA
    mla_sm120.cu, KVTilePartLoader::loadPages: ``kvCachePageList[req][page]``).
    Table entries at or beyond ceil(T / P) are never read."""
    out = np.empty((T, dim), dtype=np.uint8)
    for j in range(T):
        page = int(table_row[j // page_size])
        out[j] = cache[page, g, j % page_size, :dim]
    return out


def gather_bytes(w) -> np.ndarray:
    """Byte-exact reference for the debug page gather: ``[B, H_kv, T_max,
    D_qk]`` uint8 with K rows of each request in key order, zero past T_b."""
    T = w.kv_tokens()
    T_max = int(T.max()) if w.batch else 0
    out = np.zeros((w.batch, w.num_kv_heads, T_max, w.head_dim_qk), dtype=np.uint8)
    for b in range(w.batch):
        for g in range(w.num_kv_heads):
            out[b, g, :T[b]] = gather_rows(w.k_cache, w.block_table[b], g, int(T[b]),
                                           w.page_size, w.head_dim_qk)
    return out


def dequant_rows(raw: np.ndarray, kv_dtype: str, scale: np.ndarray, mode: str,
                 g: int) -> np.ndarray:
    """fp64 values of gathered rows: decode(byte) * scale."""
    return _decode(raw, kv_dtype) * _scale_vector(scale, mode, g, raw.shape[1])[None, :]


# ------------------------------------------------------------------- masks ---

def visible_keys(L: int, n: int, t: int, causal: bool) -> int:
    """Number of keys (a prefix 0..k-1) visible to appended token t of a
    request with L cached and n appended tokens.  Causal masking is aligned
    bottom-right: token t sits at absolute position L + t and sees keys
    j <= L + t (the c8 kernel bounds its causal loop by ``kv_len - q_len +``
    the tile's last token; XQA's multi-token decode uses ``seqLen -
    (inputSeqLen - 1) + tokenIdx`` keys).  Without causality every token sees
    all T = L + n keys."""
    return (L + t + 1) if causal else (L + n)


def visible_set(L: int, n: int, t: int, causal: bool, tree_row: Optional[np.ndarray] = None) -> np.ndarray:
    """Boolean visibility of the T = L + n keys for appended token t.

    Without a tree mask this is the prefix of ``visible_keys``.  With one (the
    c8 decode kernel's optional ``attn_mask``, a ``[bsz, max_q, max_q]`` bool
    tensor for tree-structured speculative drafts, passed to its mask step
    with the request's ``batch_id * attn_mask_len * attn_mask_len`` offset),
    the L cached keys stay visible and appended key L + s is visible to token
    t exactly when ``tree_row[s]`` (the mask's row t) is nonzero; the mask
    takes the place of the causal rule inside the appended block."""
    vis = np.zeros(L + n, dtype=bool)
    if tree_row is None:
        vis[:visible_keys(L, n, t, causal)] = True
    else:
        vis[:L] = True
        vis[L:] = np.asarray(tree_row[:n]) != 0
    return vis


# --------------------------------------------------------------- attention ---

def query_heads_of(g: int, G: int):
    """Query heads served by KV head g: the G consecutive heads g*G .. g*G+G-1
    (GQA grouping as in the c8 kernel's ``q_head_idx = kv_head_idx *
    GROUP_SIZE``)."""
    return range(g * G, g * G + G)


def _q_values(w, rows: np.ndarray) -> np.ndarray:
    if w.q_dtype == "bf16":
        return bf16_bits_to_f64(w.q[rows])
    return np.asarray(w.q[rows], dtype=np.float32).astype(np.float64)


def _softmax_lse(z: np.ndarray) -> Tuple[np.ndarray, float]:
    """Probabilities and natural log-sum-exp of one row of logits, computed
    with max subtraction."""
    m = float(np.max(z))
    e = np.exp(z - m)
    s = float(np.sum(e))
    return e / s, m + math.log(s)


def request_attention(w, b: int, key_lo: int = 0, key_hi: Optional[int] = None):
    """Exact attention of request b over keys [key_lo, key_hi) intersected
    with each token's visible prefix.

    Returns ``(O, lse)`` with O ``[n_b, H_q, D_v]`` and lse ``[n_b, H_q]`` in
    fp64; lse is ``ln sum_j exp(z_j)`` of the scaled logits
    ``z_j = sm_scale * q . K_hat[j]``.  A (token, head) whose visible key set
    is empty in the range gets O = 0 and lse = -inf (an empty split-KV chunk
    contributes nothing to the merge)."""
    n = int(w.q_lens[b])
    L = int(w.seq_lens_kv[b])
    T = L + n
    key_hi = T if key_hi is None else min(key_hi, T)
    G = w.num_q_heads // w.num_kv_heads
    O = np.zeros((n, w.num_q_heads, w.head_dim_v))
    lse = np.full((n, w.num_q_heads), -np.inf)
    if n == 0:
        return O, lse
    q0 = int(w.cu_seqlens_q[b])
    q = _q_values(w, np.arange(q0, q0 + n))                        # [n, H_q, D_qk]
    vcache = w.k_cache if w.shared_kv else w.v_cache
    tree = getattr(w, "tree_mask", None)
    vis = [visible_set(L, n, t, w.causal, None if tree is None else tree[b, t]) for t in range(n)]
    for g in range(w.num_kv_heads):
        k_raw = gather_rows(w.k_cache, w.block_table[b], g, T, w.page_size, w.head_dim_qk)
        v_raw = gather_rows(vcache, w.block_table[b], g, T, w.page_size, w.head_dim_v)
        K = dequant_rows(k_raw, w.kv_dtype, w.k_scale, w.scale_mode, g)   # [T, D_qk]
        V = dequant_rows(v_raw, w.kv_dtype, w.v_scale, w.scale_mode, g)   # [T, D_v]
        for h in query_heads_of(g, G):
            z_all = w.sm_scale * (q[:, h, :] @ K.T)                       # [n, T]
            for t in range(n):
                sel = np.nonzero(vis[t][key_lo:key_hi])[0] + key_lo
                if sel.size == 0:
                    continue
                p, l = _softmax_lse(z_all[t, sel])
                O[t, h] = p @ V[sel]
                lse[t, h] = l
    return O, lse


def attention(w, requests: Optional[Iterable[int]] = None):
    """Unsplit attention for every (or the listed) request.  Returns
    ``(O [total_q, H_q, D_v], lse [total_q, H_q])``; rows of requests not
    listed are NaN."""
    O = np.full((w.total_q, w.num_q_heads, w.head_dim_v), np.nan)
    lse = np.full((w.total_q, w.num_q_heads), np.nan)
    reqs = range(w.batch) if requests is None else requests
    for b in reqs:
        q0, q1 = int(w.cu_seqlens_q[b]), int(w.cu_seqlens_q[b + 1])
        if q1 > q0:
            O[q0:q1], lse[q0:q1] = request_attention(w, b)
    return O, lse


# ------------------------------------------------------------------ split ---

def chunk_partials(w, b: int, chunk_size: int) -> Tuple[np.ndarray, np.ndarray]:
    """Split-KV partials of request b: chunk c covers keys
    [c*C, min((c+1)*C, T_b)) for c < ceil(T_b / C) (c8 kernel: ``chunk_start =
    chunk_idx * chunk_size``, ``chunk_end = min(kv_len, chunk_start +
    chunk_size)``, chunks past ``div_up(kv_len, chunk_size)`` exit).  Each
    partial is normalized within its chunk with its own natural lse (the
    normalized-O-plus-LSE form FlashInfer's persistent reduction consumes).
    Returns O_c ``[n_b, C_b, H_q, D_v]`` and lse_c ``[n_b, C_b, H_q]``."""
    n = int(w.q_lens[b])
    T = int(w.seq_lens_kv[b]) + n
    C_b = -(-T // chunk_size)
    Oc = np.zeros((n, C_b, w.num_q_heads, w.head_dim_v))
    lc = np.full((n, C_b, w.num_q_heads), -np.inf)
    for c in range(C_b):
        Oc[:, c], lc[:, c] = request_attention(w, b, c * chunk_size, (c + 1) * chunk_size)
    return Oc, lc


def merge_partials(Oc: np.ndarray, lc: np.ndarray) -> Tuple[np.ndarray, np.ndarray]:
    """Log-sum-exp merge over the chunk axis (axis 1) of normalized partials:
    M = max_c lse_c, w_c = exp(lse_c - M), O = sum_c w_c O_c / sum_c w_c,
    lse = M + ln sum_c w_c.  Chunks with lse_c = -inf carry weight 0
    (FlashInfer persistent.cuh, BlockBatchReductionPersistent via
    ``state_t::merge``; XQA mla_sm120.cu, mergePartialOutputs rescales each
    sub-sequence by the exponential of its max difference)."""
    M = np.max(lc, axis=1)                                   # [n, H]
    Ms = np.where(np.isfinite(M), M, 0.0)
    wgt = np.where(np.isfinite(lc), np.exp(lc - Ms[:, None, :]), 0.0)
    den = wgt.sum(axis=1)
    O = (wgt[..., None] * Oc).sum(axis=1) / den[..., None]
    lse = Ms + np.log(den)
    return O, lse


def attention_split(w, chunk_size: int, requests: Optional[Iterable[int]] = None):
    """Attention computed chunk by chunk and merged; equal to ``attention``
    up to rounding (pinned by the split-merge tests)."""
    O = np.full((w.total_q, w.num_q_heads, w.head_dim_v), np.nan)
    lse = np.full((w.total_q, w.num_q_heads), np.nan)
    reqs = range(w.batch) if requests is None else requests
    for b in reqs:
        q0, q1 = int(w.cu_seqlens_q[b]), int(w.cu_seqlens_q[b + 1])
        if q1 > q0:
            Oc, lc = chunk_partials(w, b, chunk_size)
            O[q0:q1], lse[q0:q1] = merge_partials(Oc, lc)
    return O, lse

