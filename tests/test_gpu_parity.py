"""GPU parity: the HIP path through the C ABI against the fp64 oracle.

Every output element is compared, for the small workloads and for the
full-size workloads in the launch configuration bench.py times (the oracle
runs those in several CPU processes, one share of the requests each).
"""
import math
import zlib

import numpy as np
import pytest

import oracle
from gpu_util import announce, compare, need_gpu, oracle_every_request, token_rows
from workloads import config_workload, make_workload, small_variant

pytestmark = pytest.mark.gpu


def _run(w, **kw):
    from paged_kv_attention_gather_amd.harness import DeviceProblem
    dp = DeviceProblem(w, **kw)
    dp.run()
    return dp, dp.outputs()


# ------------------------------------------------------------ page gather --
#
# Byte-exact gathers through each loader the attention kernels run: one key
# row at a time, the decode kernel's register tile loader, and the LDS-DMA
# tile loader with 4 or 3 waves (also for the shared 576-byte latent rows, in
# 64-key tiles and in the e4m3fn MLA kernel's 32-key tiles), over the
# workloads' chunked units (tiles that end a chunk or a sequence, one-page
# fast path and page sizes below 64).

LOADERS = {"rows": 0, "decode": 1, "dma4": 2, "dma3": 3, "mla32": 4}


def _loaders_for(w):
    if w.shared_kv:
        return ["rows", "dma4", "mla32"]
    return ["rows", "decode", "dma4", "dma3"]


def _gather(w, loader, reqs=None):
    torch = need_gpu()
    import paged_kv_attention_gather_amd as P
    from paged_kv_attention_gather_amd.harness import DeviceProblem
    dp = DeviceProblem(w)
    T = w.kv_tokens()
    t_max = int(T.max())
    kd = torch.zeros((w.batch, w.num_kv_heads, t_max, w.head_dim_qk), dtype=torch.uint8, device="cuda")
    vd = None if w.shared_kv else torch.zeros((w.batch, w.num_kv_heads, t_max, w.head_dim_v), dtype=torch.uint8,
                                              device="cuda")
    P.pa_gather_debug(dp.prob, dp.k_cache, dp.block_table, dp.seq_lens_kv, dp.q_lens, t_max, kd,
                      loader=LOADERS[loader], v_cache=None if w.shared_kv else dp.v_cache, v_dst=vd)
    torch.cuda.synchronize()
    return kd.cpu().numpy(), None if vd is None else vd.cpu().numpy()


@pytest.mark.parametrize("idx", [1, 2, 3, 4, 5])
def test_gather_bit_exact_small(idx):
    need_gpu()
    w = small_variant(idx)
    for loader in _loaders_for(w):
        announce(f"gather small_variant({idx}) {w.name} loader={loader}")
        k, v = _gather(w, loader)
        assert np.array_equal(k, oracle.gather_bytes(w)), loader
        if v is not None:
            vw = type(w)(**{**w.__dict__, "k_cache": w.v_cache, "head_dim_qk": w.head_dim_v})
            assert np.array_equal(v, oracle.gather_bytes(vw)), loader


@pytest.mark.parametrize("idx", [2, 4, 5])
def test_gather_bit_exact_full(idx):
    need_gpu()
    w = config_workload(idx)
    T = w.kv_tokens()
    for loader in _loaders_for(w):
        announce(f"gather config_workload({idx}) {w.name} loader={loader}")
        k, v = _gather(w, loader)
        for b in range(w.batch):
            for g in range(w.num_kv_heads):
                ref = oracle.gather_rows(w.k_cache, w.block_table[b], g, int(T[b]), w.page_size, w.head_dim_qk)
                assert np.array_equal(k[b, g, :T[b]], ref), (loader, b, g)
                if v is not None:
                    ref = oracle.gather_rows(w.v_cache, w.block_table[b], g, int(T[b]), w.page_size, w.head_dim_v)
                    assert np.array_equal(v[b, g, :T[b]], ref), (loader, "V", b, g)


def test_read_probe_reads_every_tile():
    """The read probe's per-unit xor equals the xor of the unit's K and V
    bytes as 16-byte words, where the last tile's rows past the unit's end
    repeat its last key (the loader clamps them)."""
    torch = need_gpu()
    import paged_kv_attention_gather_amd as P
    from paged_kv_attention_gather_amd.harness import DeviceProblem
    w = small_variant(2)
    announce("read probe small_variant(2)")
    dp = DeviceProblem(w)
    C = w.chunk_size
    T = w.kv_tokens()
    mc = max(1, -(-(int(w.seq_lens_kv.max()) + int(w.decode_q_len)) // C))
    sink = torch.zeros(mc * w.batch * w.num_kv_heads, dtype=torch.int32, device="cuda")
    P.pa_kv_read_probe(dp.prob, int(w.decode_q_len), dp.k_cache, dp.v_cache, dp.seq_lens_kv, dp.block_table, sink)
    torch.cuda.synchronize()
    got = sink.cpu().numpy().view(np.uint32)
    for b in range(w.batch):
        for g in range(w.num_kv_heads):
            k = oracle.gather_rows(w.k_cache, w.block_table[b], g, int(T[b]), w.page_size, w.head_dim_qk)
            v = oracle.gather_rows(w.v_cache, w.block_table[b], g, int(T[b]), w.page_size, w.head_dim_v)
            for c in range(mc):
                lo, hi = c * C, min(int(T[b]), (c + 1) * C)
                want = 0
                if lo < hi:
                    n_pad = -(-(hi - lo) // 64) * 64 - (hi - lo)
                    rows = np.concatenate([k[lo:hi], v[lo:hi]] + ([np.repeat(k[hi - 1:hi], n_pad, 0),
                                                                   np.repeat(v[hi - 1:hi], n_pad, 0)] if n_pad else []))
                    want = int(np.bitwise_xor.reduce(rows.reshape(-1).view(np.uint32)))
                assert got[c * w.batch * w.num_kv_heads + b * w.num_kv_heads + g] == want, (b, g, c)


# --------------------------------------------------- attention, small sizes --

@pytest.mark.parametrize("idx", [1, 2, 3, 4, 5])
def test_small_variant_parity(idx):
    need_gpu()
    w = small_variant(idx)
    announce(f"attention small_variant({idx}) {w.name} chunk={w.chunk_size}")
    _, (out, lse) = _run(w)
    O_ref, lse_ref = oracle.attention(w)
    compare(out, lse, O_ref, lse_ref, what=w.name)


@pytest.mark.parametrize("idx", [1, 2, 3, 4, 5])
def test_poisoned_tail_is_never_read(idx):
    need_gpu()
    w = small_variant(idx, poison_tail=True)
    announce(f"attention poisoned tail small_variant({idx})")
    _, (out, lse) = _run(w)
    O_ref, lse_ref = oracle.attention(w)
    compare(out, lse, O_ref, lse_ref, what=w.name + "+poison")


def test_config1_tiny_append_full():
    need_gpu()
    w = config_workload(1)
    announce("attention config_workload(1) tiny append")
    _, (out, lse) = _run(w)
    O_ref, lse_ref = oracle.attention(w)
    compare(out, lse, O_ref, lse_ref, what=w.name)


def test_repeat_runs_are_bitwise_identical():
    torch = need_gpu()
    w = small_variant(4)
    announce("determinism small_variant(4)")
    from paged_kv_attention_gather_amd.harness import DeviceProblem
    dp = DeviceProblem(w)
    dp.run()
    a = dp.outputs()
    dp.out.zero_()
    dp.run()
    b = dp.outputs()
    assert np.array_equal(a[0], b[0]) and np.array_equal(a[1], b[1])


# ------------------------------------------------------------- edge cases --

def _edge(name, **kw):
    base = dict(name=name, seed=zlib.crc32(name.encode()) % 10000, num_q_heads=8, num_kv_heads=2, head_dim_qk=128,
                head_dim_v=128, page_size=64, q_dtype="bf16", kv_dtype="i8", scale_mode="channel",
                causal=True, sm_scale=1 / math.sqrt(128), chunk_size=0, decode=False)
    base.update(kw)
    return make_workload(**base)


EDGE_CASES = {
    "append_zero_len_request": dict(q_lens=[5, 0, 70, 1], seq_lens_kv=[10, 33, 0, 129]),
    "append_noncausal": dict(q_lens=[7, 90], seq_lens_kv=[100, 3], causal=False),
    "append_chunked": dict(q_lens=[100, 37], seq_lens_kv=[300, 500], chunk_size=128),
    "append_chunk_equals_page": dict(q_lens=[3, 80], seq_lens_kv=[200, 40], chunk_size=64),
    "append_chunk_beyond_T": dict(q_lens=[4, 9], seq_lens_kv=[20, 70], chunk_size=4096),
    "append_g1": dict(num_q_heads=4, num_kv_heads=4, q_lens=[33, 6], seq_lens_kv=[65, 190]),
    "append_page16_head_scale": dict(page_size=16, scale_mode="head", q_lens=[20, 3], seq_lens_kv=[47, 100]),
    # per-channel scales sized so |V| <= 448 * 0.008 < 4, the range where a bf16
    # output can meet max-abs 1e-2 (half an ulp of bf16 at 4 is 7.8e-3)
    "append_fp8_channel": dict(kv_dtype="fp8_e4m3", q_lens=[12, 80], seq_lens_kv=[64, 250],
                               scale_range=(0.0005, 0.008)),
    "append_f32_query": dict(q_dtype="f32", q_lens=[2, 19], seq_lens_kv=[31, 64]),
    "decode_q8_g8": dict(num_q_heads=16, num_kv_heads=2, q_lens=[8, 8, 8], seq_lens_kv=[0, 500, 1300],
                         decode=True, chunk_size=512),
    "decode_page16_chunk64": dict(page_size=16, q_lens=[1, 1], seq_lens_kv=[77, 3], decode=True, chunk_size=64),
    "decode_page256": dict(page_size=256, q_lens=[3, 3], seq_lens_kv=[700, 1], decode=True, chunk_size=256),
    "decode_d64_fp8_tensor": dict(head_dim_qk=64, head_dim_v=64, kv_dtype="fp8_e4m3", scale_mode="tensor",
                                  q_lens=[2, 2, 2], seq_lens_kv=[5, 140, 700], decode=True, chunk_size=256),
    "decode_noncausal_drafts": dict(q_lens=[4, 4], seq_lens_kv=[60, 300], decode=True, causal=False,
                                    chunk_size=128),
    # query rows whose channels 3 and 77 are 256x the rest: the int8 paths
    # quantise each query row relative to its maximum, so small channels must
    # survive next to a large one (one row per decode unit, 40 packed rows,
    # and the append kernel)
    "decode_query_outliers_head": dict(scale_mode="head", q_lens=[1, 1, 1], seq_lens_kv=[5, 300, 1200],
                                       decode=True, chunk_size=256, q_outliers=((3, 77), 256.0)),
    "spec40_query_outliers_channel": dict(num_q_heads=16, q_lens=[5, 5], seq_lens_kv=[40, 700], decode=True,
                                          chunk_size=256, q_outliers=((3, 77), 256.0)),
    "append_query_outliers_channel": dict(q_lens=[40, 7], seq_lens_kv=[100, 5], q_outliers=((3, 77), 256.0)),
    # the limits of the ABI: decode q_len 64 (256 packed rows, the append-shaped
    # kernel through the decode entry), page size 1024 (a 64-key tile inside
    # one page, 16 tiles per page), and the tree's 64-draft bitmask
    "decode_q64_g4_max_rows": dict(q_lens=[64, 64], seq_lens_kv=[3, 400], decode=True, chunk_size=256),
    "append_page1024": dict(page_size=1024, q_lens=[70, 5], seq_lens_kv=[1500, 1019]),
    "decode_page1024_chunked": dict(page_size=1024, q_lens=[2, 2, 2], seq_lens_kv=[2047, 1, 1100],
                                    decode=True, chunk_size=512),
    "mla_int8_g16_q2": dict(num_q_heads=16, num_kv_heads=1, head_dim_qk=576, head_dim_v=512,
                            shared_kv=True, scale_mode="tensor", q_lens=[2, 2], seq_lens_kv=[63, 900],
                            decode=True, chunk_size=256),
}


@pytest.mark.parametrize("case", sorted(EDGE_CASES))
def test_edge_case_parity(case):
    need_gpu()
    w = _edge(case, **EDGE_CASES[case])
    announce(f"edge case {case}")
    _, (out, lse) = _run(w)
    O_ref, lse_ref = oracle.attention(w)
    n = int(w.q_lens.sum())
    compare(out[:n], lse[:n], O_ref[:n], lse_ref[:n], what=case)


# Outlier-channel queries are where logit rounding is largest relative to the
# logits, so these cases also run under several seeds: a numerics margin must
# hold for every draw, not one.  Per-head and per-channel K scales, int8 and
# fp8 caches, each kernel family (decode unit, 40-row shared tile, append tile,
# int8 and e4m3fn MLA-shaped rows).
OUTLIER_CASES = {
    "decode_query_outliers_head": EDGE_CASES["decode_query_outliers_head"],
    "spec40_query_outliers_channel": EDGE_CASES["spec40_query_outliers_channel"],
    "append_query_outliers_channel": EDGE_CASES["append_query_outliers_channel"],
    "append_query_outliers_head": dict(scale_mode="head", q_lens=[40, 7], seq_lens_kv=[100, 5],
                                       q_outliers=((3, 77), 256.0)),
    "append_fp8_query_outliers": dict(kv_dtype="fp8_e4m3", q_lens=[33, 80], seq_lens_kv=[64, 250],
                                      scale_range=(0.0005, 0.008), q_outliers=((5, 100), 64.0)),
    "mla_int8_query_outliers": dict(num_q_heads=16, num_kv_heads=1, head_dim_qk=576, head_dim_v=512,
                                    shared_kv=True, scale_mode="tensor", q_lens=[2, 2], seq_lens_kv=[63, 900],
                                    decode=True, chunk_size=256, q_outliers=((3, 530), 64.0)),
    # e4m3fn MLA: the query goes to the fp8 MFMA in two digits (bf16, per-tensor
    # scale) or three (per-channel scales folded in)
    "mla_fp8_query_outliers": dict(num_q_heads=16, num_kv_heads=1, head_dim_qk=576, head_dim_v=512,
                                   shared_kv=True, kv_dtype="fp8_e4m3", scale_mode="tensor",
                                   scale_range=(0.0005, 0.008), q_lens=[2, 2], seq_lens_kv=[63, 900],
                                   decode=True, chunk_size=256, q_outliers=((3, 530), 64.0)),
    "mla_fp8_query_outliers_channel": dict(num_q_heads=16, num_kv_heads=1, head_dim_qk=576, head_dim_v=512,
                                           shared_kv=True, kv_dtype="fp8_e4m3", scale_mode="channel",
                                           scale_range=(0.0005, 0.008), q_lens=[2, 2], seq_lens_kv=[63, 900],
                                           decode=True, chunk_size=256, q_outliers=((3, 530), 64.0)),
}


# QK^T of the e4m3fn MLA kernel runs on the fp8 MFMA, whose accumulation was
# measured to keep ~11 bits below the largest product of an instruction
# (error 2^-11.3 of it; the f16 MFMA on the same values: 2e-7).  With two
# query channels 64x the rest, that product is the outlier's, and the LSE
# error reaches ~1.3e-2 at sm_scale 1/sqrt(128), over the 1e-3 bound; the
# seeded workloads' N(0, 1) queries stay near 2e-4.  Kept as strict expected
# failures so that a change in either direction shows.
FP8_MFMA_ACCUMULATION = pytest.mark.xfail(
    strict=True, reason="fp8 MFMA accumulation (~2^-11 of the largest product) with 64x outlier query channels")
OUTLIER_PARAMS = [pytest.param(c, marks=FP8_MFMA_ACCUMULATION) if c.startswith("mla_fp8") else c
                  for c in sorted(OUTLIER_CASES)]


@pytest.mark.parametrize("seed", [11, 2024, 7777])
@pytest.mark.parametrize("case", OUTLIER_PARAMS)
def test_query_outliers_seeds(case, seed):
    need_gpu()
    kw = dict(OUTLIER_CASES[case])
    kw["seed"] = seed
    w = _edge(case, **kw)
    announce(f"outlier case {case} seed={seed}")
    _, (out, lse) = _run(w)
    O_ref, lse_ref = oracle.attention(w)
    n = int(w.q_lens.sum())
    compare(out[:n], lse[:n], O_ref[:n], lse_ref[:n], what=f"{case} seed={seed}")


# Shared-tile and MLA workgroups find their (request, head, chunk) either from
# the grid slot directly or, for grids about one round deep, by numbering only
# the groups that hold work; both numberings are forced here on cases with
# empty requests, chunked keys and several row tiles.
GROUP_NUMBERING_CASES = ["append_zero_len_request", "append_chunked", "spec40_query_outliers_channel",
                         "mla_int8_g16_q2"]


@pytest.mark.parametrize("order", [1, 2])
@pytest.mark.parametrize("case", GROUP_NUMBERING_CASES)
def test_group_numbering_parity(case, order):
    need_gpu()
    w = _edge(case, **EDGE_CASES[case])
    announce(f"edge case {case} group_order={order}")
    _, (out, lse) = _run(w, schedule={"group_order": order})
    O_ref, lse_ref = oracle.attention(w)
    n = int(w.q_lens.sum())
    compare(out[:n], lse[:n], O_ref[:n], lse_ref[:n], what=f"{case} group_order={order}")


# Draft trees (paged_attn_decode_tree): every tree kernel (decode kernel with
# 1 or 2 row tiles, shared-tile kernel with 3 or 4 waves), drafts that straddle
# chunk and page boundaries, fp8 and fp32 queries, a mask wider than q_len
# whose unused entries are nonzero, and a poisoned page tail.
TREE_CASES = {
    "tree_q4_g4_nt1": dict(q_lens=[4, 4, 4], seq_lens_kv=[0, 70, 600], decode=True, chunk_size=256,
                           tree=True, tree_mask_len=6),
    "tree_q4_g8_nt2_chunk64": dict(num_q_heads=16, q_lens=[4, 4], seq_lens_kv=[62, 300], decode=True,
                                   chunk_size=64, tree=True),
    "tree_q5_g8_nw3": dict(num_q_heads=16, q_lens=[5, 5], seq_lens_kv=[40, 700], decode=True, chunk_size=256,
                           tree=True, tree_mask_len=8),
    "tree_q8_g8_nw4_nochunk": dict(num_q_heads=16, q_lens=[8, 8], seq_lens_kv=[1, 190], decode=True,
                                   chunk_size=0, tree=True),
    "tree_d64_fp8_tensor": dict(head_dim_qk=64, head_dim_v=64, kv_dtype="fp8_e4m3", scale_mode="tensor",
                                q_lens=[3, 3, 3], seq_lens_kv=[5, 140, 700], decode=True, chunk_size=256,
                                tree=True),
    "tree_q64_g1_full_mask": dict(num_q_heads=2, num_kv_heads=2, q_lens=[64, 64], seq_lens_kv=[0, 333],
                                  decode=True, chunk_size=128, tree=True),
    "tree_f32_query_page16": dict(q_dtype="f32", page_size=16, q_lens=[6, 6], seq_lens_kv=[13, 77],
                                  decode=True, chunk_size=64, tree=True),
}


@pytest.mark.parametrize("case", sorted(TREE_CASES))
def test_tree_decode_parity(case):
    need_gpu()
    w = _edge(case, **TREE_CASES[case])
    announce(f"tree decode {case}")
    _, (out, lse) = _run(w)
    O_ref, lse_ref = oracle.attention(w)
    n = int(w.q_lens.sum())
    compare(out[:n], lse[:n], O_ref[:n], lse_ref[:n], what=case)


def test_tree_decode_poisoned_tail():
    need_gpu()
    w = _edge("tree_poison", num_q_heads=16, q_lens=[5, 5], seq_lens_kv=[59, 123], decode=True,
              chunk_size=128, tree=True, poison_tail=True)
    announce("tree decode poisoned tail")
    _, (out, lse) = _run(w)
    O_ref, lse_ref = oracle.attention(w)
    compare(out, lse, O_ref, lse_ref, what="tree+poison")


def test_tree_decode_full_spec_workload():
    need_gpu()
    w = config_workload(4, tree=True)
    announce("tree decode on the full spec-decode workload (every request)")
    _, (out, lse) = _run(w)
    O_ref, lse_ref = oracle_every_request(4, tree=True)
    compare(out, lse, O_ref, lse_ref, what="spec_decode+tree, every request")


# Decode units whose key range is split across 2 or 4 waves of a workgroup
# (states merged in LDS), forced through the tuning override; a request with
# fewer tiles than waves leaves some waves empty (pa_problem.decode_waves).
SPLIT_WAVE_CASES = {
    "g4_q1_chunk512": dict(num_q_heads=8, num_kv_heads=2, q_lens=[1, 1, 1], seq_lens_kv=[1000, 64, 2],
                           decode=True, chunk_size=512),
    "g8_q3_nochunk": dict(num_q_heads=16, num_kv_heads=2, q_lens=[3, 3], seq_lens_kv=[900, 130],
                          decode=True, chunk_size=0),
    "d64_fp8_chunk256": dict(head_dim_qk=64, head_dim_v=64, kv_dtype="fp8_e4m3", scale_mode="tensor",
                             q_lens=[2, 2], seq_lens_kv=[700, 40], decode=True, chunk_size=256),
}


@pytest.mark.parametrize("waves", [2, 4])
@pytest.mark.parametrize("case", sorted(SPLIT_WAVE_CASES))
def test_decode_split_waves_parity(case, waves):
    need_gpu()
    w = _edge("split_" + case, **SPLIT_WAVE_CASES[case])
    announce(f"decode split waves={waves} {case}")
    _, (out, lse) = _run(w, schedule={"decode_waves": waves})
    O_ref, lse_ref = oracle.attention(w)
    n = int(w.q_lens.sum())
    compare(out[:n], lse[:n], O_ref[:n], lse_ref[:n], what=f"{case} waves={waves}")


# ------------------------------------------------------------------ merge --

@pytest.mark.parametrize("case", ["decode_q8_g8", "append_chunked", "mla_int8_g16_q2"])
def test_deferred_merge_matches_single_call(case):
    """PA_FLAG_DEFER_MERGE + an explicit split_kv_merge gives the bits of the
    single call (same kernels, same order of operations)."""
    need_gpu()
    from paged_kv_attention_gather_amd.harness import DeviceProblem
    w = _edge(case, **EDGE_CASES[case])
    announce(f"deferred merge {case}")
    a = DeviceProblem(w)
    a.run()
    ref = a.outputs()
    d = DeviceProblem(w, defer_merge=True)
    d.out.zero_()
    d.run()
    d.merge()
    got = d.outputs()
    n = int(w.q_lens.sum())
    assert np.array_equal(ref[0][:n], got[0][:n]) and np.array_equal(ref[1][:n], got[1][:n])

def test_split_kv_merge_against_oracle_partials():
    torch = need_gpu()
    import paged_kv_attention_gather_amd as P
    w = _edge("merge", q_lens=[3, 1, 6], seq_lens_kv=[700, 64, 1500], chunk_size=256)
    announce("split_kv_merge alone")
    C = w.chunk_size
    T = w.kv_tokens()
    mc = int(math.ceil((int(w.seq_lens_kv.max()) + int(w.q_lens.max())) / C))
    po = np.zeros((w.total_q, mc, w.num_q_heads, w.head_dim_v), np.float32)
    pl = np.full((w.total_q, mc, w.num_q_heads), -np.inf, np.float32)
    for b in range(w.batch):
        Oc, lc = oracle.chunk_partials(w, b, C)
        q0, q1 = int(w.cu_seqlens_q[b]), int(w.cu_seqlens_q[b + 1])
        po[q0:q1, :Oc.shape[1]] = Oc
        pl[q0:q1, :lc.shape[1]] = lc
    dev = torch.device("cuda")
    out = torch.zeros((w.total_q, w.num_q_heads, w.head_dim_v), dtype=torch.bfloat16, device=dev)
    lse = torch.zeros((w.total_q, w.num_q_heads), dtype=torch.float32, device=dev)
    P.split_kv_merge(torch.from_numpy(po).to(dev), torch.from_numpy(pl).to(dev),
                     torch.from_numpy(w.cu_seqlens_q).to(dev), torch.from_numpy(w.seq_lens_kv).to(dev),
                     0, w.batch, w.total_q, int(w.q_lens.max()), w.num_q_heads, w.head_dim_v, C, mc,
                     out, lse)
    torch.cuda.synchronize()
    O_ref, lse_ref = oracle.attention(w)
    rows = token_rows(w, [b for b in range(w.batch) if -(-int(T[b]) // C) > 1])
    compare(out.float().cpu().numpy().astype(np.float64), lse.cpu().numpy().astype(np.float64),
            O_ref, lse_ref, rows=rows, what="merge")


# ------------------------------------------------------ in-kernel merge --
#
# PA_FLAG_FUSED_MERGE: the last workgroup of each (request, KV head, row tile)
# merges the chunk partials inside the decode kernel with the same merge
# arithmetic as split_kv_merge, so the outputs must equal the two-launch
# call's bit for bit.  The library merges in-kernel only where a row tile's
# merge is one short pass (decode with a few packed rows);
# pa_problem.merge_in_kernel = 1 forces it for every decode-kernel case (1 and 2 row
# tiles, units split over 2 or 4 waves, empty chunks past the causal bound,
# page size 16, fp8, a draft tree).  The wider kernels (16-row shared tiles,
# append, MLA) enqueue split_kv_merge under the flag, which these cases check
# too.  Each case runs twice on one workspace (the counters must be back at
# zero after a call), then a workspace is reused with other lengths.
FUSED_CASES = {
    "decode_g4_chunk64": dict(q_lens=[1, 1, 1, 1], seq_lens_kv=[0, 63, 700, 2000], decode=True, chunk_size=64),
    "decode_nt2_q8_g4": dict(q_lens=[8, 8, 8], seq_lens_kv=[5, 500, 1300], decode=True, chunk_size=256),
    "decode_page16_chunk64": EDGE_CASES["decode_page16_chunk64"],
    "decode_d64_fp8_tensor": EDGE_CASES["decode_d64_fp8_tensor"],
    "spec40_query_outliers_channel": EDGE_CASES["spec40_query_outliers_channel"],
    "decode_q8_g8": EDGE_CASES["decode_q8_g8"],
    "append_chunked": EDGE_CASES["append_chunked"],
    "append_zero_len_chunked": dict(q_lens=[5, 0, 150, 1], seq_lens_kv=[10, 33, 0, 1290], chunk_size=128),
    "mla_int8_g16_q2": EDGE_CASES["mla_int8_g16_q2"],
    "tree_q5_g8_nw3": TREE_CASES["tree_q5_g8_nw3"],
    "tree_q4_g4_nt1": TREE_CASES["tree_q4_g4_nt1"],
}


def _counter_words(prob):
    """int32 merge counters at the start of a fused-merge workspace:
    [B, H_kv, ceil(max_q_len * G / 16)]."""
    G = prob.num_q_heads // prob.num_kv_heads
    return prob.batch * prob.num_kv_heads * max(1, -(-(prob.max_q_len * G) // 16))


def _fused_vs_launch(w, what, schedule=None):
    from paged_kv_attention_gather_amd.harness import DeviceProblem
    ref_dp, ref = _run(w, schedule={k: v for k, v in (schedule or {}).items() if k != "merge_in_kernel"})
    f = DeviceProblem(w, fused_merge=True, schedule=schedule)
    n = int(w.q_lens.sum())
    for call in range(2):
        f.out.zero_()
        f.lse.zero_()
        f.run()
        got = f.outputs()
        assert np.array_equal(ref[0][:n], got[0][:n]), f"{what}: call {call}: O differs from the merge launch"
        assert np.array_equal(ref[1][:n], got[1][:n]), f"{what}: call {call}: lse differs from the merge launch"
        cnt = f.workspace[:4 * _counter_words(f.prob)].view(f.torch.int32)
        assert int(cnt.abs().sum().item()) == 0, f"{what}: merge counters not reset after call {call}"
    return f, got


@pytest.mark.parametrize("case", sorted(FUSED_CASES))
def test_fused_merge_matches_merge_launch(case):
    need_gpu()
    w = _edge(case, **FUSED_CASES[case])
    announce(f"fused merge {case}")
    _, (out, lse) = _fused_vs_launch(w, case, schedule={"merge_in_kernel": 1})
    O_ref, lse_ref = oracle.attention(w)
    n = int(w.q_lens.sum())
    compare(out[:n], lse[:n], O_ref[:n], lse_ref[:n], what=f"{case} fused")


@pytest.mark.parametrize("waves", [2, 4])
def test_fused_merge_split_waves(waves):
    need_gpu()
    case = "g4_q1_chunk512"
    w = _edge("split_" + case, **SPLIT_WAVE_CASES[case])
    announce(f"fused merge, decode units over {waves} waves")
    _fused_vs_launch(w, f"{case} waves={waves}", schedule={"decode_waves": waves, "merge_in_kernel": 1})


@pytest.mark.parametrize("force", [1, 0])
def test_fused_merge_workspace_reuse_shorter_lengths(force):
    """A workspace zeroed once serves later calls of the same batch size, head
    counts and max_q_len with other lengths (fewer chunks, fewer tokens, new
    partial values: a merge that read stale partials would fail here).  With
    the automatic choice these single-token decode rows merge in-kernel."""
    need_gpu()
    sched = {"merge_in_kernel": force}
    from paged_kv_attention_gather_amd.harness import DeviceProblem
    big = _edge("reuse_big", q_lens=[1, 1, 1], seq_lens_kv=[900, 2000, 300], decode=True, chunk_size=128)
    small = _edge("reuse_small", q_lens=[1, 1, 1], seq_lens_kv=[100, 0, 700], decode=True, chunk_size=128)
    announce("fused merge workspace reuse")
    a = DeviceProblem(big, fused_merge=True, schedule=sched)
    a.run()
    a.outputs()
    b = DeviceProblem(small, fused_merge=True, schedule=sched)
    for k in ("max_q_len", "max_kv_len"):
        setattr(b.prob, k, getattr(a.prob, k))
    from paged_kv_attention_gather_amd import _lib as L
    assert L.workspace_size(b.prob, b.total_q) <= a.workspace_bytes
    b.workspace, b.workspace_bytes = a.workspace, a.workspace_bytes
    b.run()
    out, lse = b.outputs()
    O_ref, lse_ref = oracle.attention(small)
    n = int(small.q_lens.sum())
    compare(out[:n], lse[:n], O_ref[:n], lse_ref[:n], what="shorter lengths on a reused workspace")


# ------------------------------------------------------- balanced split --
#
# PA_FLAG_BALANCED_SPLIT: the MLA kernel cuts each request's keys into items
# whose length (at least chunk_size) is chosen on the device from all the
# lengths; every cut merges to the same exact attention, so the outputs are
# checked against the oracle.  The small MLA case runs at the split's floor,
# the full-size MLA workload with the device's one-round target; the other
# kernels keep fixed chunks under the flag, which the remaining cases check.
BALANCED_CASES = {
    "spec40_query_outliers_channel": EDGE_CASES["spec40_query_outliers_channel"],
    "decode_q8_g8": EDGE_CASES["decode_q8_g8"],
    "append_chunked": EDGE_CASES["append_chunked"],
    "append_zero_len_chunked": FUSED_CASES["append_zero_len_chunked"],
    "mla_int8_g16_q2": EDGE_CASES["mla_int8_g16_q2"],
    "tree_q5_g8_nw3": TREE_CASES["tree_q5_g8_nw3"],
}


@pytest.mark.parametrize("fused", [False, True])
@pytest.mark.parametrize("case", sorted(BALANCED_CASES))
def test_balanced_split_parity(case, fused):
    need_gpu()
    w = _edge(case, **BALANCED_CASES[case])
    announce(f"balanced split {case} fused={fused}")
    dp, (out, lse) = _run(w, balanced=True, fused_merge=fused, schedule={"merge_in_kernel": 1} if fused else None)
    O_ref, lse_ref = oracle.attention(w)
    n = int(w.q_lens.sum())
    compare(out[:n], lse[:n], O_ref[:n], lse_ref[:n], what=f"{case} balanced fused={fused}")
    if fused:
        dp.out.zero_()
        dp.run()
        again = dp.outputs()
        assert np.array_equal(out, again[0]) and np.array_equal(lse, again[1]), "second call differs"


@pytest.mark.parametrize("idx", [4, 5])
def test_balanced_split_full_config(idx):
    need_gpu()
    w = config_workload(idx)
    announce(f"balanced split config_workload({idx}) {w.name} (every request)")
    chunk = 1024 if idx == 5 else None   # MLA: the item floor below the 3072 fixed chunk
    _, (out, lse) = _run(w, balanced=True, chunk_size=chunk)
    O_ref, lse_ref = oracle_every_request(idx)
    compare(out, lse, O_ref, lse_ref, what=f"{w.name} balanced, every request")


# ---------------------------------------------------- persistent decode --
#
# PA_FLAG_PERSISTENT: one launch of resident-capacity waves, each taking an
# equal share of all (request, KV head) tiles (at least chunk_size keys), the
# pieces' partials merged by the wave that finishes each range last.  Any cut
# merges to the same exact attention, so the outputs are checked against the
# oracle; each case runs twice on one workspace (the counters must be back at
# zero) and the second call must give the same bits.
PERSISTENT_CASES = {
    "decode_g4_chunk64": FUSED_CASES["decode_g4_chunk64"],
    "decode_nt2_q8_g4": FUSED_CASES["decode_nt2_q8_g4"],
    "decode_page16_chunk64": EDGE_CASES["decode_page16_chunk64"],
    "decode_d64_fp8_tensor": EDGE_CASES["decode_d64_fp8_tensor"],
    "decode_q8_g8": dict(num_q_heads=8, num_kv_heads=2, q_lens=[8, 8, 8], seq_lens_kv=[0, 500, 1300], decode=True,
                         chunk_size=128),
    "decode_noncausal_drafts": EDGE_CASES["decode_noncausal_drafts"],
    "decode_f32_query_head": dict(q_dtype="f32", scale_mode="head", q_lens=[2, 2, 2, 2], seq_lens_kv=[1, 64, 65, 900],
                                  decode=True, chunk_size=64),
    "decode_many_requests": dict(q_lens=[1] * 70, seq_lens_kv=[(37 * i) % 700 for i in range(70)], decode=True,
                                 chunk_size=64),
}


@pytest.mark.parametrize("case", sorted(PERSISTENT_CASES))
def test_persistent_decode_parity(case):
    need_gpu()
    w = _edge(case, **PERSISTENT_CASES[case])
    announce(f"persistent decode {case}")
    dp, (out, lse) = _run(w, persistent=True)
    O_ref, lse_ref = oracle.attention(w)
    n = int(w.q_lens.sum())
    compare(out[:n], lse[:n], O_ref[:n], lse_ref[:n], what=f"{case} persistent")
    cnt = dp.workspace[:4 * _counter_words(dp.prob)].view(dp.torch.int32)
    assert int(cnt.abs().sum().item()) == 0, "merge counters not reset"
    dp.out.zero_()
    dp.run()
    again = dp.outputs()
    assert np.array_equal(out, again[0]) and np.array_equal(lse, again[1]), "second call differs"


def test_persistent_decode_full_workload():
    need_gpu()
    w = config_workload(2)
    announce("persistent decode on the full decode workload (every request)")
    _, (out, lse) = _run(w, persistent=True)
    O_ref, lse_ref = oracle_every_request(2)
    compare(out, lse, O_ref, lse_ref, what="decode_int8 persistent, every request")


# ----------------------------------------------------- full-size workloads --

@pytest.mark.parametrize("idx", [2, 3, 4, 5])
def test_full_config_parity(idx):
    need_gpu()
    w = config_workload(idx)
    announce(f"attention config_workload({idx}) {w.name} (every request)")
    _, (out, lse) = _run(w)   # the kernels and merge bench.py times
    assert np.isfinite(out).all() and np.isfinite(lse).all(), "non-finite output rows"
    if w.chunk_size > 0:
        # the one-launch form (PA_FLAG_FUSED_MERGE, bench.py --merge fused)
        # must give the two-launch call's bits over every row
        _, (fo, fl) = _run(w, fused_merge=True)
        assert np.array_equal(out, fo) and np.array_equal(lse, fl), "in-kernel merge differs"
    O_ref, lse_ref = oracle_every_request(idx)
    compare(out, lse, O_ref, lse_ref, what=f"{w.name}, every request")
