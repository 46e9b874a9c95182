"""Pins for the cache append write in oracle.kv_write: hand-computed codes,
the e4m3fn table and torch's conversion, brute-force nearest codes, and a
hand-placed scatter.  Planted mistakes at the end must fail these pins."""
import math

import numpy as np
import pytest
import torch

import oracle
import oracle.kv_write as kw
from oracle.reference import e4m3fn_decode


# ------------------------------------------------------------------ int8 ---

# (x, s, code): ties go to the even integer, the range is [-127, 127]
INT8_HAND = [(2.5, 1.0, 2), (3.5, 1.0, 4), (-2.5, 1.0, -2), (-3.5, 1.0, -4), (1.25, 0.5, 2),
             (1.75, 0.5, 4), (0.0, 0.7, 0), (1.0, 3.0, 0), (2.0, 3.0, 1), (127.4, 1.0, 127),
             (127.5, 1.0, 127), (1000.0, 1.0, 127), (-1000.0, 1.0, -127), (-127.6, 1.0, -127),
             (0.049, 0.1, 0), (0.051, 0.1, 1), (-6.0, 0.25, -24), (float("inf"), 1.0, 127)]


def test_int8_hand_codes():
    x = np.array([h[0] for h in INT8_HAND], np.float32)
    s = np.array([h[1] for h in INT8_HAND], np.float32)
    got = kw.int8_quantize(x, s).view(np.int8)
    assert got.tolist() == [h[2] for h in INT8_HAND]


def test_int8_nearest_code_property():
    rng = np.random.default_rng(3)
    s = rng.uniform(0.002, 0.03, 4000).astype(np.float32)
    x = (rng.standard_normal(4000) * 1.2).astype(np.float32)
    q = kw.int8_quantize(x, s).view(np.int8).astype(np.float64)
    r = (x.astype(np.float64) / s.astype(np.float64))
    inside = np.abs(r) < 126.9
    # inside the range the code is the nearest integer to the exact ratio
    # (the binary32 ratio is within 2^-24 relative of it, far from a tie here)
    assert np.all(np.abs(q[inside] - r[inside]) <= 0.5 + 1e-5)
    assert np.all(q[~inside] == np.sign(r[~inside]) * 127)


# Codes decided by the binary32 quotient, where exact division would decide
# otherwise: x / s rounds (once, in binary32) onto a tie k + 0.5 that the exact
# quotient misses by a few parts in 1e8, so the tie rule picks the even
# integer while the exact value's nearest integer is the other one.  Values
# are binary32 numbers written as hex floats; the test first checks the premise
# (binary32 quotient on the tie, exact quotient off it) with exact fractions.
INT8_FP32_TIES = [  # (x, s, binary32 quotient, code, exact quotient's nearest integer)
    (float.fromhex("0x1.963824p-5"), float.fromhex("0x1.44f9b6p-6"), 2.5, 2, 3),
    (float.fromhex("-0x1.86e436p-3"), float.fromhex("0x1.42ccfap-9"), -77.5, -78, -77),
    (float.fromhex("0x1.e95dbap-1"), float.fromhex("0x1.1a2834p-6"), 55.5, 56, 55),
]


def _premise(x, s, q32):
    from fractions import Fraction
    xs, ss = np.float32(x), np.float32(s)
    assert float(xs) == x and float(ss) == s, "pin values must be binary32 numbers"
    assert float(xs / ss) == q32, "binary32 quotient is not the stated value"
    exact = Fraction(x) / Fraction(s)
    assert exact != Fraction(q32), "exact quotient must miss the tie"
    return exact


def test_int8_code_follows_the_binary32_quotient():
    for x, s, q32, code, exact_code in INT8_FP32_TIES:
        exact = _premise(x, s, q32)
        assert round(exact) == exact_code          # Fraction rounding: nearest integer
        got = int(kw.int8_quantize(np.array([x], np.float32), np.array([s], np.float32)).view(np.int8)[0])
        assert got == code, (x, s, got, code)


# ---------------------------------------------------------------- e4m3fn ---

def test_e4m3_roundtrip_of_every_finite_code():
    codes = np.array([c for c in range(256) if c not in (0x7F, 0xFF)], np.uint8)
    vals = e4m3fn_decode(codes).astype(np.float32)
    assert np.array_equal(kw.e4m3fn_encode(vals), codes)


def test_e4m3_hand_values():
    # 1.0625 lies halfway between 1.0 (0x38) and 1.125 (0x39): even mantissa 0x38;
    # 1.1875 halfway between 1.125 and 1.25 (0x3A): even is 0x3A; 2^-10 is half
    # the smallest subnormal 2^-9: ties to 0; 448 is 0x7E, 460 and 1e9 saturate
    vals = np.array([1.0625, 1.1875, 2.0 ** -10, 3 * 2.0 ** -10, 448.0, 460.0, 1e9, -1e9, -0.0, 0.0,
                     2.0 ** -6, 240.0, 0.1], np.float32)
    want = [0x38, 0x3A, 0x00, 0x02, 0x7E, 0x7E, 0x7E, 0xFE, 0x80, 0x00, 0x08, 0x77, 0x1D]
    assert kw.e4m3fn_encode(vals).tolist() == want


def test_e4m3_is_the_nearest_code_brute_force():
    codes = np.array([c for c in range(256) if c not in (0x7F, 0xFF)], np.int64)
    table = e4m3fn_decode(codes.astype(np.uint8))
    rng = np.random.default_rng(5)
    x = np.concatenate([rng.standard_normal(3000) * 40, rng.standard_normal(1000) * 2.0 ** -7,
                        rng.uniform(400, 448, 200)]).astype(np.float32)
    got = kw.e4m3fn_encode(x)
    for xi, gi in zip(x.astype(np.float64), got):
        d = np.abs(table - xi)
        best = codes[d == d.min()]
        if len(best) > 1:   # a tie: the even mantissa, same sign as x
            best = best[(best & 1) == 0]
            best = best[(best >> 7) == (1 if math.copysign(1, xi) < 0 else 0)] if len(best) > 1 else best
        assert gi in best, (xi, gi, best)


def test_e4m3_agrees_with_torch_in_range():
    x = (np.random.default_rng(9).standard_normal(20000) * 80).astype(np.float32)
    x = x[np.abs(x) < 448]
    t = torch.from_numpy(x).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(kw.e4m3fn_encode(x), t)


# The same for e4m3fn: the binary32 quotient lands on the midpoint of two
# e4m3fn neighbours (54 between 52 = 0x65 and 56 = 0x66; 50 between 48 = 0x64
# and 52 = 0x65), the tie goes to the even mantissa, while the exact quotient
# lies just on the other side of the midpoint.
E4M3_FP32_TIES = [  # (x, s, binary32 quotient, code, exact quotient's nearest code)
    (float.fromhex("0x1.15ac06p-1"), float.fromhex("0x1.4917bcp-7"), 54.0, 0x66, 0x65),
    (float.fromhex("0x1.3176fap+0"), float.fromhex("0x1.86feb0p-6"), 50.0, 0x64, 0x65),
]


def test_e4m3_code_follows_the_binary32_quotient():
    for x, s, q32, code, exact_code in E4M3_FP32_TIES:
        exact = _premise(x, s, q32)
        lo, hi = sorted((e4m3fn_decode(np.array([code], np.uint8))[0], e4m3fn_decode(np.array([exact_code], np.uint8))[0]))
        assert (lo + hi) / 2 == q32                # the quotient is their midpoint
        got = int(kw.quantize(np.array([x], np.float32), np.array([s], np.float32), "fp8_e4m3")[0])
        assert got == code, (x, s, hex(got), hex(code))


# --------------------------------------------------------------- scatter ---

def test_scatter_to_hand_placed_slots():
    """P = 4, request 0 has L = 5 cached keys and 3 new ones: positions 5, 6, 7
    are slots 1, 2, 3 of its second page (physical page 2); request 1 has L = 3
    and 2 new ones: positions 3 (slot 3 of page 6) and 4 (slot 0 of page 1)."""
    H, D, P = 2, 4, 4
    cache = np.random.default_rng(1).integers(0, 256, (8, H, P, 8), dtype=np.uint8)
    table = np.array([[5, 2, 7], [6, 1, -1]], np.int32)
    lens = np.array([5, 3], np.int32)
    cu = np.array([0, 3, 5], np.int32)
    rows = np.arange(5 * H * D, dtype=np.float32).reshape(5, H, D) - 17.0
    out = kw.kv_write(cache, rows, np.array([1.0], np.float32), "tensor", "i8", table, lens, cu, P)
    want = cache.copy()
    places = [(2, 1), (2, 2), (2, 3), (6, 3), (1, 0)]
    for r, (page, slot) in enumerate(places):
        for h in range(H):
            want[page, h, slot, :D] = rows[r, h].astype(np.int8).view(np.uint8)
    assert np.array_equal(out, want)


def test_per_head_scales_hand_codes():
    """Two KV heads with scales 0.5 and 0.25 (PER_HEAD): the same row values
    give different codes per head.  Head 0: [1, -0.75, 0.25, 63] / 0.5 =
    [2, -1.5, 0.5, 126] -> [2, -2, 0, 126] (ties to even); head 1:
    [1, -0.75, 0.25, 63] / 0.25 = [4, -3, 1, 252] -> [4, -3, 1, 127] (clamped).
    One token at position 2 of a request (P = 4, page 3)."""
    H, D, P = 2, 4, 4
    cache = np.zeros((4, H, P, D), np.uint8)
    row = np.array([[1.0, -0.75, 0.25, 63.0]] * H, np.float32)[None]
    out = kw.kv_write(cache, row, np.array([0.5, 0.25], np.float32), "head", "i8",
                      np.array([[3]], np.int32), np.array([2], np.int32), np.array([0, 1], np.int32), P)
    assert out[3, 0, 2].view(np.int8).tolist() == [2, -2, 0, 126]
    assert out[3, 1, 2].view(np.int8).tolist() == [4, -3, 1, 127]
    assert np.count_nonzero(out) == np.count_nonzero(out[3, :, 2])


def test_per_channel_scales_hand_codes():
    """PER_CHANNEL scales [H, D]: channel d of head g divides by s[g, d].
    Head 0 scales [1, 0.5, 0.25, 2], head 1 [0.1, 4, 1, 0.5] (binary32) on the
    row [1.5, 1.5, 1.5, 1.5]: head 0 -> [2, 3, 6, 1] (1.5 and 0.75 round to
    even / nearest), head 1 -> [15, 0, 2, 3] (1.5 / 0.1 = 15.0000002 in
    binary32, 0.375 -> 0, 1.5 -> 2)."""
    H, D, P = 2, 4, 4
    cache = np.zeros((2, H, P, D), np.uint8)
    sc = np.array([[1.0, 0.5, 0.25, 2.0], [0.1, 4.0, 1.0, 0.5]], np.float32)
    row = np.full((1, H, D), 1.5, np.float32)
    out = kw.kv_write(cache, row, sc, "channel", "i8", np.array([[1]], np.int32), np.array([0], np.int32),
                      np.array([0, 1], np.int32), P)
    assert out[1, 0, 0].view(np.int8).tolist() == [2, 3, 6, 1]
    assert out[1, 1, 0].view(np.int8).tolist() == [15, 0, 2, 3]


def test_written_rows_decode_back_within_half_a_step():
    from workloads import make_workload, kv_write_inputs
    w = make_workload(name="kvw", seed=4, q_lens=[3, 9], seq_lens_kv=[14, 0], num_q_heads=4, num_kv_heads=2,
                      head_dim_qk=16, head_dim_v=16, page_size=16, q_dtype="bf16", kv_dtype="i8",
                      scale_mode="channel", causal=True, sm_scale=0.25, chunk_size=0, decode=False)
    kv, _, _, _ = kv_write_inputs(w, spread=0.8)
    out = kw.kv_write(w.k_cache, kv, w.k_scale, "channel", "i8", w.block_table, w.seq_lens_kv,
                      w.cu_seqlens_q, w.page_size)
    for b in range(w.batch):
        L, n = int(w.seq_lens_kv[b]), int(w.q_lens[b])
        for g in range(w.num_kv_heads):
            rows = oracle.gather_rows(out, w.block_table[b], g, L + n, w.page_size, 16)[L:]
            vals = oracle.dequant_rows(rows, "i8", w.k_scale, "channel", g)
            x = kv[w.cu_seqlens_q[b]:w.cu_seqlens_q[b + 1], g].astype(np.float64)
            sc = w.k_scale[g].astype(np.float64)
            inside = np.abs(x) <= 127 * sc   # saturated codes are checked by the hand pins
            assert inside.mean() > 0.5
            assert np.all((np.abs(vals - x) <= 0.5 * sc * (1 + 1e-6))[inside])
            assert np.all((np.abs(vals) == 127 * sc)[~inside])


# --------------------------------------------------------- planted bugs ---

def _fails(fn):
    try:
        fn()
    except AssertionError:
        return True
    return False


def test_planted_truncation_is_caught(monkeypatch):
    monkeypatch.setattr(kw, "int8_quantize", lambda x, s: np.clip(np.trunc(kw.fp32_ratio(x, s)), -127, 127)
                        .astype(np.int8).view(np.uint8))
    assert _fails(test_int8_hand_codes)


def test_planted_ties_away_from_zero_is_caught(monkeypatch):
    def away(x, s):
        r = kw.fp32_ratio(x, s).astype(np.float64)
        return np.clip(np.sign(r) * np.floor(np.abs(r) + 0.5), -127, 127).astype(np.int8).view(np.uint8)
    monkeypatch.setattr(kw, "int8_quantize", away)
    assert _fails(test_int8_hand_codes)


def test_planted_unsaturated_e4m3_is_caught(monkeypatch):
    real = kw.e4m3fn_encode
    monkeypatch.setattr(kw, "e4m3fn_encode",
                        lambda v: np.where(np.abs(np.asarray(v, np.float32)) > 448, np.uint8(0x7F), real(v)))
    assert _fails(test_e4m3_hand_values)


def test_planted_off_by_one_slot_is_caught(monkeypatch):
    real = kw.kv_write
    def shifted(cache, rows, scale, mode, kv_dtype, table, lens, cu, P):
        return real(cache, rows, scale, mode, kv_dtype, table, np.asarray(lens) + 1, cu, P)
    monkeypatch.setattr(kw, "kv_write", shifted)
    assert _fails(test_scatter_to_hand_placed_slots)


def test_planted_fp64_ratio_is_caught(monkeypatch):
    """Dividing in fp64 instead of binary32 changes the int8 codes of the tie
    pins.  (The e4m3fn encoder takes binary32 input by definition, so there an
    fp64 quotient is rounded to the binary32 one before encoding.)"""
    monkeypatch.setattr(kw, "fp32_ratio", lambda x, s: np.asarray(x, np.float32).astype(np.float64) /
                        np.asarray(s, np.float32).astype(np.float64))
    assert _fails(test_int8_code_follows_the_binary32_quotient)


def test_planted_first_scale_for_every_head_is_caught(monkeypatch):
    real = kw.scale_table
    def first_only(scale, mode, H, D):
        t = real(scale, mode, H, D)
        return np.broadcast_to(t[:1], t.shape).copy()
    monkeypatch.setattr(kw, "scale_table", first_only)
    assert _fails(test_per_head_scales_hand_codes)
    assert _fails(test_per_channel_scales_hand_codes)


def test_planted_per_channel_transposed_is_caught(monkeypatch):
    real = kw.scale_table
    def transposed(scale, mode, H, D):
        t = real(scale, mode, H, D)
        return t[:, ::-1].copy() if mode == "channel" else t
    monkeypatch.setattr(kw, "scale_table", transposed)
    assert _fails(test_per_channel_scales_hand_codes)
