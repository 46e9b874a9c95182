"""Seeded synthetic workloads shaped like the five paged-KV attention cases.

Every array is drawn from ``numpy.random.Generator(PCG64(seed))`` in a fixed
order (lengths, block-table permutation, Q, K pages, V pages, scales), so a
seed reproduces the same bytes on any machine.  Queries are rounded to bf16
(or kept fp32) with torch's round-to-nearest-even conversion; fp8 cache bytes
are produced with torch's float32 -> float8_e4m3fn conversion.  Nothing here
dequantizes, gathers or attends: that is the oracle's and the kernels' job.

Layouts (all C-contiguous):
  q            [total_q, H_q, D_qk]      bf16 bits as uint16, or float32
  k_cache      [num_pages, H_kv, P, D_qk] raw bytes (uint8)
  v_cache      [num_pages, H_kv, P, D_v]  raw bytes, or None when V is the
                                          first D_v bytes of each K row (MLA)
  block_table  [B, max_pages_per_seq]     int32, unused entries are -1
  seq_lens_kv  [B]  cached tokens per request (the appended tokens are extra)
  cu_seqlens_q [B+1] prefix sums of the per-request q_len
"""
from __future__ import annotations

import dataclasses
import math
from typing import Optional, Sequence

import numpy as np

try:  # torch provides the bf16 / e4m3fn rounding used to store inputs
    import torch
except Exception:  # pragma: no cover - torch is part of the image
    torch = None


@dataclasses.dataclass
class Workload:
    name: str
    seed: int
    batch: int
    num_q_heads: int
    num_kv_heads: int
    head_dim_qk: int
    head_dim_v: int
    page_size: int
    num_pages: int
    q_dtype: str          # "bf16" | "f32"
    kv_dtype: str         # "i8" | "fp8_e4m3"
    scale_mode: str       # "tensor" | "head" | "channel"
    causal: bool
    sm_scale: float
    chunk_size: int       # 0: no split-KV
    decode_q_len: Optional[int]  # uniform q_len (decode entry point) or None (append)
    shared_kv: bool       # V row = first D_v bytes of the K row
    q_lens: np.ndarray
    seq_lens_kv: np.ndarray
    cu_seqlens_q: np.ndarray
    block_table: np.ndarray
    q: np.ndarray
    k_cache: np.ndarray
    v_cache: Optional[np.ndarray]
    k_scale: np.ndarray
    v_scale: np.ndarray
    # [B, mask_len, mask_len] uint8 draft-tree visibility (row t, column s), or None
    tree_mask: Optional[np.ndarray] = None

    @property
    def group(self) -> int:
        return self.num_q_heads // self.num_kv_heads

    @property
    def total_q(self) -> int:
        return int(self.cu_seqlens_q[-1])

    @property
    def max_q_len(self) -> int:
        return int(self.q_lens.max()) if self.batch else 0

    @property
    def max_kv_len(self) -> int:
        return int(self.seq_lens_kv.max()) if self.batch else 0

    @property
    def max_pages_per_seq(self) -> int:
        return int(self.block_table.shape[1])

    @property
    def v_cache_or_k(self) -> np.ndarray:
        return self.k_cache if self.shared_kv else self.v_cache

    def kv_tokens(self) -> np.ndarray:
        """Keys attended per request, T_b = L_b + n_b."""
        return self.seq_lens_kv.astype(np.int64) + self.q_lens.astype(np.int64)


def _rng(seed: int) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(seed))


def _to_bf16_bits(x: np.ndarray) -> np.ndarray:
    t = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).to(torch.bfloat16)
    return t.view(torch.int16).numpy().view(np.uint16).copy()


def _to_e4m3_bytes(x: np.ndarray) -> np.ndarray:
    t = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).to(torch.float8_e4m3fn)
    return t.view(torch.uint8).numpy().copy()


def make_workload(
    *,
    name: str,
    seed: int,
    q_lens: Sequence[int],
    seq_lens_kv: Sequence[int],
    num_q_heads: int,
    num_kv_heads: int,
    head_dim_qk: int,
    head_dim_v: int,
    page_size: int,
    q_dtype: str,
    kv_dtype: str,
    scale_mode: str,
    causal: bool,
    sm_scale: float,
    chunk_size: int,
    decode: bool,
    shared_kv: bool = False,
    num_pages: Optional[int] = None,
    scale_range=(0.002, 0.03),
    extra_table_cols: int = 0,
    poison_tail: bool = False,
    q_outliers: Optional[tuple] = None,
    tree: bool = False,
    tree_mask_len: Optional[int] = None,
    rng: Optional[np.random.Generator] = None,
) -> Workload:
    """Draw one workload.  ``q_lens``/``seq_lens_kv`` are given explicitly; the
    remaining arrays are drawn from ``rng`` (or a fresh generator on ``seed``).

    ``poison_tail`` fills the unused slots of each request's last page with
    0x7F bytes (NaN in e4m3fn, 127 in int8) so a kernel that lets keys beyond
    the sequence leak into the result is caught.

    ``tree`` draws a random draft tree per request (draft 0 is the root, the
    parent of draft s >= 1 is uniform over drafts 0..s-1) and stores its
    ancestor-or-self matrix as ``tree_mask`` [B, mask_len, mask_len] uint8
    (mask_len = ``tree_mask_len`` or the largest q_len; unused entries 0xAA),
    drawn after every other array so the rest of the workload is unchanged.

    ``q_outliers = (channels, factor)`` multiplies those query channels by
    ``factor`` before rounding (outlier channels, as language-model queries
    have), so each query row spans a wide dynamic range.
    """
    rng = rng if rng is not None else _rng(seed)
    q_lens = np.asarray(q_lens, dtype=np.int32)
    seq_lens_kv = np.asarray(seq_lens_kv, dtype=np.int32)
    B = int(q_lens.shape[0])
    assert seq_lens_kv.shape == (B,)
    if decode:
        assert B == 0 or np.all(q_lens == q_lens[0]), "decode needs a uniform q_len"
    P = page_size
    T = seq_lens_kv.astype(np.int64) + q_lens.astype(np.int64)
    pages_per_req = (T + P - 1) // P
    total_pages_used = int(pages_per_req.sum())
    if num_pages is None:
        num_pages = max(16, total_pages_used)
    assert num_pages >= total_pages_used, "pool too small"
    width = max(1, int(pages_per_req.max()) if B else 1) + extra_table_cols

    perm = rng.permutation(num_pages).astype(np.int32)
    block_table = np.full((B, width), -1, dtype=np.int32)
    used = perm[:total_pages_used]
    off = 0
    for b in range(B):
        n = int(pages_per_req[b])
        block_table[b, :n] = used[off:off + n]
        off += n

    cu = np.zeros(B + 1, dtype=np.int32)
    cu[1:] = np.cumsum(q_lens)
    total_q = int(cu[-1])

    qf = rng.standard_normal((total_q, num_q_heads, head_dim_qk), dtype=np.float32)
    if q_outliers is not None:
        chans, factor = q_outliers
        qf[:, :, list(chans)] *= np.float32(factor)
    q = _to_bf16_bits(qf) if q_dtype == "bf16" else qf

    H = num_kv_heads
    k_cache = np.zeros((num_pages, H, P, head_dim_qk), dtype=np.uint8)
    v_cache = None if shared_kv else np.zeros((num_pages, H, P, head_dim_v), dtype=np.uint8)
    if kv_dtype == "i8":
        kd = rng.integers(-127, 128, size=(total_pages_used, H, P, head_dim_qk), dtype=np.int8)
        k_cache[used] = kd.view(np.uint8)
        if not shared_kv:
            vd = rng.integers(-127, 128, size=(total_pages_used, H, P, head_dim_v), dtype=np.int8)
            v_cache[used] = vd.view(np.uint8)
        tensor_scale_k = tensor_scale_v = None
    elif kv_dtype == "fp8_e4m3":
        # x ~ N(0,1); per-tensor scale s = max|x| / 448; stored = e4m3fn(x / s).
        xk = rng.standard_normal((total_pages_used, H, P, head_dim_qk), dtype=np.float32)
        sk = float(np.abs(xk).max()) / 448.0 if xk.size else 1.0
        k_cache[used] = _to_e4m3_bytes(xk / np.float32(sk))
        del xk
        tensor_scale_k = sk
        if shared_kv:
            tensor_scale_v = sk
        else:
            xv = rng.standard_normal((total_pages_used, H, P, head_dim_v), dtype=np.float32)
            sv = float(np.abs(xv).max()) / 448.0 if xv.size else 1.0
            v_cache[used] = _to_e4m3_bytes(xv / np.float32(sv))
            tensor_scale_v = sv
    else:
        raise ValueError(kv_dtype)

    lo, hi = scale_range
    if scale_mode == "tensor":
        if tensor_scale_k is None:
            tensor_scale_k = float(rng.uniform(lo, hi))
            tensor_scale_v = float(rng.uniform(lo, hi))
        k_scale = np.array([tensor_scale_k], dtype=np.float32)
        v_scale = np.array([tensor_scale_v], dtype=np.float32)
    elif scale_mode == "head":
        k_scale = rng.uniform(lo, hi, size=H).astype(np.float32)
        v_scale = rng.uniform(lo, hi, size=H).astype(np.float32)
    elif scale_mode == "channel":
        k_scale = rng.uniform(lo, hi, size=(H, head_dim_qk)).astype(np.float32)
        v_scale = rng.uniform(lo, hi, size=(H, head_dim_v)).astype(np.float32)
    else:
        raise ValueError(scale_mode)

    if poison_tail:
        for b in range(B):
            n = int(pages_per_req[b])
            if n == 0:
                continue
            last = int(block_table[b, n - 1])
            first_unused = int(T[b] - (n - 1) * P)
            if first_unused < P:
                k_cache[last, :, first_unused:, :] = 0x7F
                if not shared_kv:
                    v_cache[last, :, first_unused:, :] = 0x7F

    tree_mask = None
    if tree:
        ml = int(tree_mask_len) if tree_mask_len is not None else int(q_lens.max()) if B else 1
        tree_mask = np.full((B, ml, ml), 0xAA, dtype=np.uint8)
        for b in range(B):
            n = int(q_lens[b])
            anc = np.zeros((n, n), dtype=np.uint8)
            for t in range(n):
                anc[t, t] = 1
                if t > 0:
                    parent = int(rng.integers(0, t))
                    anc[t, :t] = anc[parent, :t]
            tree_mask[b, :n, :n] = anc

    return Workload(
        name=name, seed=seed, batch=B, num_q_heads=num_q_heads, num_kv_heads=num_kv_heads,
        head_dim_qk=head_dim_qk, head_dim_v=head_dim_v, page_size=P, num_pages=num_pages,
        q_dtype=q_dtype, kv_dtype=kv_dtype, scale_mode=scale_mode, causal=causal,
        sm_scale=float(sm_scale), chunk_size=int(chunk_size),
        decode_q_len=int(q_lens[0]) if (decode and B) else (1 if decode else None),
        shared_kv=shared_kv, q_lens=q_lens, seq_lens_kv=seq_lens_kv, cu_seqlens_q=cu,
        block_table=block_table, q=q, k_cache=k_cache, v_cache=v_cache,
        k_scale=k_scale, v_scale=v_scale, tree_mask=tree_mask,
    )


# --------------------------------------------------------------------------
# The five workloads.  Length draws come first from the config's generator.
# --------------------------------------------------------------------------

def _cfg1(seed=101):
    # Tiny append: B=2, GQA 4 (4 q heads / 1 kv head), D=64, P=16, cached {37, 50},
    # appended {3, 1}, fp32 Q, int8 KV with per-head scales in [0.005, 0.02],
    # 16-page permuted pool, causal, no split.
    return make_workload(
        name="tiny_append", seed=seed, q_lens=[3, 1], seq_lens_kv=[37, 50],
        num_q_heads=4, num_kv_heads=1, head_dim_qk=64, head_dim_v=64, page_size=16,
        q_dtype="f32", kv_dtype="i8", scale_mode="head", causal=True,
        sm_scale=1.0 / 8.0, chunk_size=0, decode=False, num_pages=16,
        scale_range=(0.005, 0.02))


def _cfg2(seed=102, batch=64, lo=512, hi=4096):
    rng = _rng(seed)
    L = rng.integers(lo, hi + 1, size=batch).astype(np.int32)
    return make_workload(
        name="decode_int8", seed=seed, q_lens=[1] * batch, seq_lens_kv=L,
        num_q_heads=32, num_kv_heads=8, head_dim_qk=128, head_dim_v=128, page_size=64,
        q_dtype="bf16", kv_dtype="i8", scale_mode="channel", causal=True,
        sm_scale=1.0 / math.sqrt(128), chunk_size=512, decode=True, num_pages=16384,
        rng=rng)


def _cfg3(seed=103, batch=8):
    rng = _rng(seed)
    n = rng.integers(256, 1024 + 1, size=batch).astype(np.int32)
    L = rng.integers(0, 2048 + 1, size=batch).astype(np.int32)
    return make_workload(
        name="append_prefill", seed=seed, q_lens=n, seq_lens_kv=L,
        num_q_heads=32, num_kv_heads=8, head_dim_qk=128, head_dim_v=128, page_size=64,
        q_dtype="bf16", kv_dtype="i8", scale_mode="head", causal=True,
        sm_scale=1.0 / math.sqrt(128), chunk_size=0, decode=False, num_pages=1024,
        rng=rng)


def _cfg4(seed=104, batch=128, tree=False):
    rng = _rng(seed)
    L = np.exp(rng.normal(math.log(2048.0), 1.0, size=batch))
    L = np.clip(np.rint(L), 128, 32768).astype(np.int32)
    pages = int(((L.astype(np.int64) + 5 + 63) // 64).sum())
    return make_workload(
        name="spec_decode", seed=seed, q_lens=[5] * batch, seq_lens_kv=L,
        num_q_heads=64, num_kv_heads=8, head_dim_qk=128, head_dim_v=128, page_size=64,
        q_dtype="bf16", kv_dtype="i8", scale_mode="channel", causal=True,
        sm_scale=1.0 / math.sqrt(128), chunk_size=1024, decode=True,
        num_pages=max(16384, 2 * pages), tree=tree, rng=rng)


def _cfg5(seed=105, batch=32, chunk_size=3072):
    rng = _rng(seed)
    L = rng.integers(4096, 16384 + 1, size=batch).astype(np.int32)
    return make_workload(
        name="mla_decode", seed=seed, q_lens=[1] * batch, seq_lens_kv=L,
        num_q_heads=128, num_kv_heads=1, head_dim_qk=576, head_dim_v=512, page_size=64,
        q_dtype="bf16", kv_dtype="fp8_e4m3", scale_mode="tensor", causal=True,
        sm_scale=1.0 / math.sqrt(576), chunk_size=chunk_size, decode=True, shared_kv=True,
        num_pages=16384, rng=rng)


CONFIGS = {1: _cfg1, 2: _cfg2, 3: _cfg3, 4: _cfg4, 5: _cfg5}


def config_workload(idx: int, **kw) -> Workload:
    """Full-size workload ``idx`` (1..5) with its default seed (100 + idx)."""
    return CONFIGS[idx](**kw)


def small_variant(idx: int, seed: Optional[int] = None, poison_tail: bool = False) -> Workload:
    """A reduced version of workload ``idx`` that keeps its heads, dims, page
    size, dtypes and scale mode, with hand-picked lengths that cross several
    64-key tiles, several chunks and leave ragged tails (including 1-key and
    page-aligned cases)."""
    seed = 200 + idx if seed is None else seed
    if idx == 1:
        w = _cfg1(seed)
        if poison_tail:
            w = make_workload(
                name="tiny_append_small", seed=seed, q_lens=[3, 1], seq_lens_kv=[37, 50],
                num_q_heads=4, num_kv_heads=1, head_dim_qk=64, head_dim_v=64, page_size=16,
                q_dtype="f32", kv_dtype="i8", scale_mode="head", causal=True,
                sm_scale=1.0 / 8.0, chunk_size=0, decode=False, num_pages=16,
                scale_range=(0.005, 0.02), poison_tail=True)
        return w
    if idx == 2:
        return make_workload(
            name="decode_int8_small", seed=seed, q_lens=[1] * 6,
            seq_lens_kv=[0, 62, 63, 600, 1023, 1500],
            num_q_heads=32, num_kv_heads=8, head_dim_qk=128, head_dim_v=128, page_size=64,
            q_dtype="bf16", kv_dtype="i8", scale_mode="channel", causal=True,
            sm_scale=1.0 / math.sqrt(128), chunk_size=512, decode=True, num_pages=96,
            poison_tail=poison_tail)
    if idx == 3:
        return make_workload(
            name="append_prefill_small", seed=seed, q_lens=[1, 37, 130, 64],
            seq_lens_kv=[0, 65, 200, 3],
            num_q_heads=32, num_kv_heads=8, head_dim_qk=128, head_dim_v=128, page_size=64,
            q_dtype="bf16", kv_dtype="i8", scale_mode="head", causal=True,
            sm_scale=1.0 / math.sqrt(128), chunk_size=0, decode=False, num_pages=64,
            poison_tail=poison_tail)
    if idx == 4:
        return make_workload(
            name="spec_decode_small", seed=seed, q_lens=[5] * 4,
            seq_lens_kv=[128, 700, 1019, 2100],
            num_q_heads=64, num_kv_heads=8, head_dim_qk=128, head_dim_v=128, page_size=64,
            q_dtype="bf16", kv_dtype="i8", scale_mode="channel", causal=True,
            sm_scale=1.0 / math.sqrt(128), chunk_size=1024, decode=True, num_pages=128,
            poison_tail=poison_tail)
    if idx == 5:
        return make_workload(
            name="mla_decode_small", seed=seed, q_lens=[1] * 3, seq_lens_kv=[1, 700, 1500],
            num_q_heads=128, num_kv_heads=1, head_dim_qk=576, head_dim_v=512, page_size=64,
            q_dtype="bf16", kv_dtype="fp8_e4m3", scale_mode="tensor", causal=True,
            sm_scale=1.0 / math.sqrt(576), chunk_size=512, decode=True, shared_kv=True,
            num_pages=64, poison_tail=poison_tail)
    raise ValueError(idx)


def kv_write_inputs(w: Workload, seed: Optional[int] = None, spread: float = 1.3, in_dtype: str = "bf16"):
    """New K/V rows for the cache append write of workload ``w``: one row per
    appended token (``w.q_lens`` per request, ``[total_q, H_kv, D]``), values
    N(0, 1) scaled so that value / scale spans about +-(spread x the code
    range) (127 for int8, 448 for e4m3fn), so that some codes saturate.
    Returns ``(k_vals, v_vals, k_in, v_in)``: binary32 values and the stored
    input arrays (bf16 bit patterns as uint16, or float32); ``v_*`` are None
    for the shared MLA layout."""
    rng = _rng(w.seed + 7919 if seed is None else seed)
    top = 127.0 if w.kv_dtype == "i8" else 448.0
    H = w.num_kv_heads

    def draw(D, scale):
        s = np.asarray(scale, dtype=np.float32)
        mag = float(np.median(s)) * top * spread / 3.0
        x = (rng.standard_normal((w.total_q, H, D), dtype=np.float32) * np.float32(mag)).astype(np.float32)
        if in_dtype == "bf16":
            bits = _to_bf16_bits(x)
            return (bits.astype(np.uint32) << 16).view(np.float32), bits
        return x, x

    k_vals, k_in = draw(w.head_dim_qk, w.k_scale)
    if w.shared_kv:
        return k_vals, None, k_in, None
    v_vals, v_in = draw(w.head_dim_v, w.v_scale)
    return k_vals, v_vals, k_in, v_in
