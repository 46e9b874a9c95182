"""Every compiled attention specialization, reached at least once through the
C ABI and compared with the oracle.

The library compiles one kernel per (head dims, cache dtype, query split,
row class, waves per unit, draft tree).  The query is split into f16 hi + lo
parts when it carries per-channel K scales or is fp32; the row class is set
by the packed rows of a (request, KV head): up to 16 or 32 rows run in the
register-staged decode kernel (its keys split over 1, 2 or 4 waves), 33..48
and 49..64 rows in the 16-row shared-tile kernel with 3 or 4 waves, more in
the 128-row append kernel (f16 tiles at head dim 128).  The cases below pick
each combination with small ragged requests that cross chunks and pages.
"""
import math
import zlib

import numpy as np
import pytest

import oracle
from gpu_util import announce, compare, need_gpu
from workloads import make_workload

pytestmark = pytest.mark.gpu

# row class -> (entry point, query lengths); G = 4 (8 query heads, 2 KV heads)
ROW_CLASSES = {
    "decode_rows8": (True, [2, 2, 2]),        # 8 packed rows: decode kernel, one 16-row tile
    "decode_rows24": (True, [6, 6, 6]),       # 24 rows: decode kernel, two 16-row tiles
    "tile_rows40": (True, [10, 10, 10]),      # 40 rows: shared-tile kernel, 3 waves
    "tile_rows56": (True, [14, 14, 14]),      # 56 rows: shared-tile kernel, 4 waves
    "append_rows160": (False, [40, 7, 23]),   # 160 rows: the 128-row append kernel
}
# query dtype / K scale mode -> hi + lo query split or not
QUERY_SCALE = {
    "bf16_head": ("bf16", "head"),        # one f16 part (exact)
    "f32_head": ("f32", "head"),          # hi + lo: fp32 query
    "bf16_channel": ("bf16", "channel"),  # hi + lo: per-channel K scales folded in
}


def _case(name, D, kv, qs, decode, q_lens, seq_lens, chunk, page, **kw):
    q_dtype, scale_mode = QUERY_SCALE[qs]
    return make_workload(
        name=name, seed=zlib.crc32(name.encode()) % 100000, q_lens=q_lens, seq_lens_kv=seq_lens,
        num_q_heads=kw.pop("num_q_heads", 8), num_kv_heads=kw.pop("num_kv_heads", 2), head_dim_qk=D,
        head_dim_v=kw.pop("head_dim_v", D), page_size=page, q_dtype=q_dtype, kv_dtype=kv, scale_mode=scale_mode,
        causal=True, sm_scale=1 / math.sqrt(D), chunk_size=chunk, decode=decode,
        # keep |V| < 4 (the range where a bf16 output can meet max-abs 1e-2)
        scale_range=(0.0005, 0.008) if kv == "fp8_e4m3" else (0.002, 0.03), **kw)


def _check(w, what, **run_kw):
    from paged_kv_attention_gather_amd.harness import DeviceProblem
    dp = DeviceProblem(w, **run_kw)
    dp.run()
    out, lse = dp.outputs()
    O_ref, lse_ref = oracle.attention(w)
    compare(out, lse, O_ref, lse_ref, what=what)


CASES = []
for D in (64, 128):
    for kv in ("i8", "fp8_e4m3"):
        for qs in QUERY_SCALE:
            for rc in ROW_CLASSES:
                waves = (1, 2, 4) if rc.startswith("decode") else (0,)
                for ks in waves:
                    CASES.append((D, kv, qs, rc, ks))


@pytest.mark.parametrize("D,kv,qs,rc,ks", CASES, ids=[f"d{c[0]}-{c[1]}-{c[2]}-{c[3]}-w{c[4]}" for c in CASES])
def test_every_specialization(D, kv, qs, rc, ks):
    need_gpu()
    decode, q_lens = ROW_CLASSES[rc]
    name = f"var_d{D}_{kv}_{qs}_{rc}_w{ks}"
    page = 16 if (len(name) % 2) else 64          # both address paths, spread over the cases
    seq = [3, 150, 700] if decode else [0, 300, 65]
    chunk = 256 if decode else (128 if D == 64 else 0)
    w = _case(name, D, kv, qs, decode, q_lens, seq, chunk, page)
    announce(f"specialization {name} page={page} chunk={chunk}")
    _check(w, name, schedule={"decode_waves": ks} if ks else None)


MLA_CASES = [(kv, qs) for kv in ("fp8_e4m3", "i8") for qs in QUERY_SCALE]


@pytest.mark.parametrize("kv,qs", MLA_CASES, ids=[f"{k}-{q}" for k, q in MLA_CASES])
def test_every_mla_specialization(kv, qs):
    need_gpu()
    name = f"var_mla_{kv}_{qs}"
    w = _case(name, 576, kv, qs, True, [2, 2], [63, 900], 256, 64, num_q_heads=16, num_kv_heads=1,
              head_dim_v=512, shared_kv=True)
    announce(f"specialization {name}")
    _check(w, name)


TREE_CASES = [(D, kv, hilo, rc) for D in (64, 128) for kv in ("i8", "fp8_e4m3") for hilo in (False, True)
              for rc in ("decode_rows8", "decode_rows24", "tile_rows40", "tile_rows56")]


@pytest.mark.parametrize("D,kv,hilo,rc", TREE_CASES, ids=[f"d{c[0]}-{c[1]}-hilo{int(c[2])}-{c[3]}" for c in TREE_CASES])
def test_every_tree_specialization(D, kv, hilo, rc):
    need_gpu()
    _, q_lens = ROW_CLASSES[rc]
    name = f"var_tree_d{D}_{kv}_{int(hilo)}_{rc}"
    qs = ("f32_head" if D == 64 else "bf16_channel") if hilo else "bf16_head"
    w = _case(name, D, kv, qs, True, q_lens, [5, 130, 640], 128, 64, tree=True)
    announce(f"specialization {name}")
    _check(w, name)
