"""Property tests of the fp64 oracle over random tiny shapes (hypothesis).

Each property holds for exact paged attention whatever the shape, lengths,
mask, cache format or scale granularity, so a mistake in the oracle's paging,
masking or merge fails on some draw:

* page relabelling: applying one permutation of the physical pages to the
  cache and to the block table together leaves every output bit unchanged
  (the table is only a map from logical to physical pages);
* any partition: the log-sum-exp merge of the partials over any cut of a
  request's keys into contiguous ranges equals the unsplit result;
* convexity: each output channel lies within the range of that channel over
  the row's visible values (softmax weights are non-negative and sum to 1),
  and the natural lse is finite exactly when the row sees a key.
"""
import dataclasses
import math

import numpy as np
import pytest
from hypothesis import HealthCheck, given, settings
from hypothesis import strategies as st

import oracle.reference as oa
from workloads import make_workload

SETTINGS = settings(max_examples=40, deadline=None, suppress_health_check=[HealthCheck.too_slow])


@st.composite
def tiny_workloads(draw):
    B = draw(st.integers(1, 3))
    H_kv = draw(st.integers(1, 2))
    G = draw(st.integers(1, 3))
    D = draw(st.sampled_from([4, 8]))
    P = draw(st.sampled_from([2, 4, 8]))
    q_lens = draw(st.lists(st.integers(0, 4), min_size=B, max_size=B))
    seq_lens = draw(st.lists(st.integers(0, 20), min_size=B, max_size=B))
    kv_dtype = draw(st.sampled_from(["i8", "fp8_e4m3"]))
    scale_mode = draw(st.sampled_from(["tensor", "head", "channel"]))
    return make_workload(
        name="prop", seed=draw(st.integers(0, 2**31 - 1)), q_lens=q_lens, seq_lens_kv=seq_lens,
        num_q_heads=H_kv * G, num_kv_heads=H_kv, head_dim_qk=D, head_dim_v=D, page_size=P,
        q_dtype=draw(st.sampled_from(["bf16", "f32"])), kv_dtype=kv_dtype, scale_mode=scale_mode,
        causal=draw(st.booleans()), sm_scale=1.0 / math.sqrt(D), chunk_size=0, decode=False,
        extra_table_cols=draw(st.integers(0, 2)))


def relabel_pages(w, perm):
    """The same workload with physical page p stored at perm[p]."""
    k = np.empty_like(w.k_cache)
    k[perm] = w.k_cache
    v = None
    if w.v_cache is not None:
        v = np.empty_like(w.v_cache)
        v[perm] = w.v_cache
    table = np.where(w.block_table >= 0, perm[np.maximum(w.block_table, 0)], w.block_table)
    return dataclasses.replace(w, k_cache=k, v_cache=v, block_table=table.astype(w.block_table.dtype))


def check_relabel_invariance(w, perm):
    O, lse = oa.attention(w)
    O2, lse2 = oa.attention(relabel_pages(w, perm))
    assert np.array_equal(O, O2, equal_nan=True) and np.array_equal(lse, lse2, equal_nan=True)


def check_any_partition(w, rng):
    for b in range(w.batch):
        n = int(w.q_lens[b])
        T = int(w.seq_lens_kv[b]) + n
        if n == 0 or T == 0:
            continue
        O, lse = oa.request_attention(w, b, 0, T)
        k = int(rng.integers(1, T + 1))
        inner = sorted(rng.choice(np.arange(1, T), size=min(k - 1, T - 1), replace=False).tolist()) if T > 1 else []
        cuts = [0] + inner + [T]
        Oc = np.zeros((n, len(cuts) - 1, w.num_q_heads, w.head_dim_v))
        lc = np.full((n, len(cuts) - 1, w.num_q_heads), -np.inf)
        for i in range(len(cuts) - 1):
            Oc[:, i], lc[:, i] = oa.request_attention(w, b, cuts[i], cuts[i + 1])
        O2, lse2 = oa.merge_partials(Oc, lc)
        seen = np.isfinite(lse)
        np.testing.assert_allclose(O2[seen], O[seen], rtol=0, atol=1e-12)
        np.testing.assert_allclose(lse2[seen], lse[seen], rtol=0, atol=1e-12)
        assert np.array_equal(np.isfinite(lse2), seen)


def check_convexity(w):
    O, lse = oa.attention(w)
    G = w.num_q_heads // w.num_kv_heads
    for b in range(w.batch):
        n, L = int(w.q_lens[b]), int(w.seq_lens_kv[b])
        T = L + n
        q0 = int(w.cu_seqlens_q[b])
        for g in range(w.num_kv_heads):
            raw = oa.gather_rows(w.v_cache if w.v_cache is not None else w.k_cache, w.block_table[b], g, T,
                                 w.page_size, w.head_dim_v)
            V = oa.dequant_rows(raw, w.kv_dtype, w.v_scale, w.scale_mode, g)
            for t in range(n):
                vis = oa.visible_set(L, n, t, w.causal)   # boolean over the T keys
                for h in oa.query_heads_of(g, G):
                    row, l = O[q0 + t, h], lse[q0 + t, h]
                    if not vis.any():
                        assert not np.isfinite(l)
                        continue
                    assert np.isfinite(l)
                    lo, hi = V[vis].min(axis=0), V[vis].max(axis=0)
                    slack = 1e-12 * (1.0 + np.abs(V[vis]).max())
                    assert np.all(row >= lo - slack) and np.all(row <= hi + slack)


@SETTINGS
@given(w=tiny_workloads(), data=st.data())
def test_property_page_relabelling_changes_nothing(w, data):
    perm = np.asarray(data.draw(st.permutations(range(w.k_cache.shape[0]))), dtype=np.int64)
    check_relabel_invariance(w, perm)


@SETTINGS
@given(w=tiny_workloads(), seed=st.integers(0, 2**31 - 1))
def test_property_merge_over_any_partition(w, seed):
    check_any_partition(w, np.random.default_rng(seed))


@SETTINGS
@given(w=tiny_workloads())
def test_property_outputs_are_convex_combinations(w):
    check_convexity(w)


# A planted mistake in the oracle must make a property fail: reading logical
# page j // P as the physical page (ignoring the table) breaks relabelling.
def test_planted_table_ignored_is_caught(monkeypatch):
    w = make_workload(name="planted", seed=3, q_lens=[2, 3], seq_lens_kv=[9, 5], num_q_heads=2, num_kv_heads=1,
                      head_dim_qk=4, head_dim_v=4, page_size=4, q_dtype="f32", kv_dtype="i8",
                      scale_mode="head", causal=True, sm_scale=0.5, chunk_size=0, decode=False, num_pages=12)
    perm = np.random.default_rng(1).permutation(w.k_cache.shape[0])
    check_relabel_invariance(w, perm)   # holds for the real oracle

    def no_table(cache, table_row, g, T, page_size, dim):
        out = np.empty((T, dim), dtype=np.uint8)
        for j in range(T):
            out[j] = cache[j // page_size, g, j % page_size, :dim]
        return out
    monkeypatch.setattr(oa, "gather_rows", no_table)
    with pytest.raises(AssertionError):
        check_relabel_invariance(w, perm)
