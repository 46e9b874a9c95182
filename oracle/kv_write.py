"""fp32-decided oracle of the KV-cache append write: quantize the new tokens'
K/V rows and scatter them into their pages.

This module is test infrastructure (see the package docstring).

The pages state only the read side: FastDeploy append_attention_c8_impl.cuh
(multi_query_append_attention_c8_kernel) attends over ``kv_len = seq_lens_kv +
q_len`` keys and reads the appended tokens' K/V from the cache, so a write step
must already have put token t of request b at cache position L_b + t; the
cache holds int8 or e4m3fn bytes whose value is byte * scale (per tensor, per
KV head or per (head, channel)).  The write side is therefore the inverse of
that dequantization, read plainly:

  int8:    code = clamp(round_half_even(x / s), -127, 127)
  e4m3fn:  code = the e4m3fn number nearest to x / s (ties to an even
           mantissa), saturating to +-448 (the format has no infinity)

with x / s computed as one IEEE binary32 division, because a quantized code is
an integer decided by floating point and both sides must decide it in the
same precision (the kernels divide in fp32).
"""
from __future__ import annotations

import math

import numpy as np


def fp32_ratio(x: np.ndarray, s: np.ndarray) -> np.ndarray:
    """x / s as a correctly rounded binary32 division (NumPy float32 '/')."""
    return np.asarray(x, dtype=np.float32) / np.asarray(s, dtype=np.float32)


def int8_quantize(x: np.ndarray, s: np.ndarray) -> np.ndarray:
    """int8 codes (as uint8 bytes) of x / s: round half to even, clamp to
    [-127, 127] (the symmetric range of the cache values)."""
    r = fp32_ratio(x, s).astype(np.float64)
    q = np.clip(np.rint(r), -127, 127).astype(np.int8)
    return q.view(np.uint8)


def e4m3fn_encode(v: np.ndarray) -> np.ndarray:
    """e4m3fn byte of each binary32 value, from the format's definition: sign
    bit, 4 exponent bits with bias 7, 3 mantissa bits; exponent field 0 holds
    the subnormals m * 2^-9; the largest finite value is 1.75 * 2^8 = 448 and
    S.1111.111 is NaN.  Rounds to nearest, ties to an even mantissa; finite
    values beyond 448 saturate to 448; NaN gives 0x7F."""
    v = np.asarray(v, dtype=np.float32)
    out = np.empty(v.shape, dtype=np.uint8)
    flat_in = v.reshape(-1)
    flat_out = out.reshape(-1)
    for i, x32 in enumerate(flat_in):
        x = float(x32)
        if math.isnan(x):
            flat_out[i] = 0x7F
            continue
        sign = 0x80 if math.copysign(1.0, x) < 0 else 0
        a = abs(x)
        if a >= 448.0:
            flat_out[i] = sign | 0x7E
            continue
        if a < 2.0 ** -6:
            # subnormal grid 2^-9; 8 units is the smallest normal, code 0x08
            q = int(np.rint(a * 2.0 ** 9))
            flat_out[i] = sign | q
            continue
        e = math.floor(math.log2(a))
        if 2.0 ** e > a:          # guard the log2 of values just below a power of two
            e -= 1
        elif 2.0 ** (e + 1) <= a:
            e += 1
        mant = int(np.rint((a / 2.0 ** e - 1.0) * 8.0))
        if mant == 8:
            e, mant = e + 1, 0
        code = ((e + 7) << 3) | mant
        flat_out[i] = sign | min(code, 0x7E)
    return out


def quantize(x: np.ndarray, s: np.ndarray, kv_dtype: str) -> np.ndarray:
    if kv_dtype == "i8":
        return int8_quantize(x, s)
    if kv_dtype == "fp8_e4m3":
        return e4m3fn_encode(fp32_ratio(x, s))
    raise ValueError(kv_dtype)


def scale_table(scale: np.ndarray, mode: str, H: int, D: int) -> np.ndarray:
    """The binary32 divisor of every (KV head, channel): one per tensor, one
    per head ``[H]`` or one per (head, channel) ``[H, D]``."""
    s = np.asarray(scale, dtype=np.float32)
    if mode == "tensor":
        return np.full((H, D), s.reshape(-1)[0], dtype=np.float32)
    if mode == "head":
        return np.repeat(s.reshape(-1)[:H, None], D, axis=1)
    if mode == "channel":
        return s.reshape(H, -1)[:, :D].copy()
    raise ValueError(mode)


def kv_write(cache: np.ndarray, new_rows: np.ndarray, scale: np.ndarray, mode: str, kv_dtype: str,
             block_table: np.ndarray, seq_lens_kv: np.ndarray, cu_seqlens_new: np.ndarray,
             page_size: int) -> np.ndarray:
    """A copy of ``cache`` ``[pages, H, P, row_bytes]`` with the new rows
    written: row r = cu[b] + t of ``new_rows`` ``[total_new, H, D]`` (binary32
    values) goes, quantized, to position L_b + t of request b, i.e. page
    ``block_table[b][(L_b + t) // P]``, slot ``(L_b + t) % P``, bytes 0..D-1
    of the row.  Nothing else changes."""
    out = cache.copy()
    H, D = new_rows.shape[1], new_rows.shape[2]
    div = scale_table(scale, mode, H, D)
    for b in range(len(seq_lens_kv)):
        L = int(seq_lens_kv[b])
        r0, r1 = int(cu_seqlens_new[b]), int(cu_seqlens_new[b + 1])
        codes = quantize(new_rows[r0:r1], np.broadcast_to(div, (r1 - r0, H, D)), kv_dtype)
        for t in range(r1 - r0):
            pos = L + t
            page = int(block_table[b][pos // page_size])
            out[page, :, pos % page_size, :D] = codes[t]
    return out
