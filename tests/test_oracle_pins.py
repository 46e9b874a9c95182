"""Pins for the fp64 oracle: each test checks it against something other than
itself (a library routine, brute force, a closed form or an invariant), and
the mutation tests at the end show that planted mistakes in the oracle make
these pins fail."""
import dataclasses
import math

import numpy as np
import pytest
import torch

import oracle
import oracle.reference as oa
from workloads import make_workload, small_variant


def tiny(seed=7, q_lens=(3, 2), seq_lens_kv=(9, 14), H_q=4, H_kv=2, D=8, Dv=8, P=4,
         kv_dtype="i8", scale_mode="channel", causal=True, sm_scale=None, q_dtype="bf16",
         num_pages=None, shared_kv=False, **kw):
    return make_workload(
        name="tiny", seed=seed, q_lens=list(q_lens), seq_lens_kv=list(seq_lens_kv),
        num_q_heads=H_q, num_kv_heads=H_kv, head_dim_qk=D, head_dim_v=Dv, page_size=P,
        q_dtype=q_dtype, kv_dtype=kv_dtype, scale_mode=scale_mode, causal=causal,
        sm_scale=(1.0 / math.sqrt(D)) if sm_scale is None else sm_scale, chunk_size=0,
        decode=False, num_pages=num_pages, shared_kv=shared_kv, **kw)


def _dense_kv_identity_layout(w):
    """Rewrite ``w`` so request b's pages are the consecutive physical pages
    b*npp .. b*npp+npp-1 (identity table).  The dense K/V of request b is then
    a plain reshape of a pool slice, independent of the j // P indexing."""
    npp = w.block_table.shape[1]
    pool_k = np.zeros((w.batch * npp,) + w.k_cache.shape[1:], np.uint8)
    pool_v = None if w.shared_kv else np.zeros((w.batch * npp,) + w.v_cache.shape[1:], np.uint8)
    table = np.full_like(w.block_table, -1)
    for b in range(w.batch):
        for i in range(npp):
            src = w.block_table[b, i]
            if src < 0:
                continue
            pool_k[b * npp + i] = w.k_cache[src]
            if pool_v is not None:
                pool_v[b * npp + i] = w.v_cache[src]
            table[b, i] = b * npp + i
    return dataclasses.replace(w, k_cache=pool_k, v_cache=pool_v, block_table=table,
                               num_pages=w.batch * npp)


def _torch_dequant(raw_u8, kv_dtype, scale, mode, g):
    t = torch.from_numpy(np.ascontiguousarray(raw_u8))
    if kv_dtype == "i8":
        vals = t.view(torch.int8).to(torch.float64)
    else:
        vals = t.view(torch.float8_e4m3fn).to(torch.float64)
    s = torch.from_numpy(np.asarray(scale, np.float32)).to(torch.float64)
    if mode == "tensor":
        return vals * s.reshape(-1)[0]
    if mode == "head":
        return vals * s.reshape(-1)[g]
    return vals * s.reshape(-1, s.shape[-1])[g, : vals.shape[-1]]


def _q_f64(w):
    if w.q_dtype == "bf16":
        return torch.from_numpy(w.q.view(np.int16)).view(torch.bfloat16).to(torch.float64)
    return torch.from_numpy(w.q).to(torch.float64)


def _sdpa_reference(w):
    """Attention with torch's scaled_dot_product_attention (float64, boolean
    mask) over K/V obtained by reshaping identity-layout pages."""
    npp = w.block_table.shape[1]
    P = w.page_size
    Q = _q_f64(w)
    G = w.group
    O = torch.zeros(w.total_q, w.num_q_heads, w.head_dim_v, dtype=torch.float64)
    LSE = torch.zeros(w.total_q, w.num_q_heads, dtype=torch.float64)
    vcache = w.k_cache if w.shared_kv else w.v_cache
    for b in range(w.batch):
        n, L = int(w.q_lens[b]), int(w.seq_lens_kv[b])
        T = n + L
        q0 = int(w.cu_seqlens_q[b])
        for g in range(w.num_kv_heads):
            kraw = w.k_cache[b * npp:(b + 1) * npp, g].reshape(npp * P, -1)[:T, : w.head_dim_qk]
            vraw = vcache[b * npp:(b + 1) * npp, g].reshape(npp * P, -1)[:T, : w.head_dim_v]
            K = _torch_dequant(kraw, w.kv_dtype, w.k_scale, w.scale_mode, g)
            V = _torch_dequant(vraw, w.kv_dtype, w.v_scale, w.scale_mode, g)
            rows = torch.arange(n)[:, None]
            cols = torch.arange(T)[None, :]
            mask = (cols <= L + rows) if w.causal else torch.ones(n, T, dtype=torch.bool)
            for h in range(g * G, (g + 1) * G):
                q = Q[q0:q0 + n, h]
                o = torch.nn.functional.scaled_dot_product_attention(
                    q[None, None], K[None, None], V[None, None], attn_mask=mask[None, None],
                    scale=w.sm_scale)[0, 0]
                z = (q @ K.T) * w.sm_scale
                z = torch.where(mask, z, torch.tensor(-math.inf, dtype=torch.float64))
                O[q0:q0 + n, h] = o
                LSE[q0:q0 + n, h] = torch.logsumexp(z, dim=1)
    return O.numpy(), LSE.numpy()


# ---------------------------------------------------------------- P-1 ---

@pytest.mark.parametrize("kv_dtype,mode", [("i8", "channel"), ("i8", "head"), ("fp8_e4m3", "tensor")])
@pytest.mark.parametrize("causal", [True, False])
def test_p1_dense_equivalence_against_torch_sdpa(kv_dtype, mode, causal):
    w = _dense_kv_identity_layout(
        tiny(kv_dtype=kv_dtype, scale_mode=mode, causal=causal, q_lens=(3, 1, 4), seq_lens_kv=(9, 0, 21)))
    O, lse = oracle.attention(w)
    O_ref, lse_ref = _sdpa_reference(w)
    np.testing.assert_allclose(O, O_ref, rtol=0, atol=1e-12)
    np.testing.assert_allclose(lse, lse_ref, rtol=0, atol=1e-12)


def test_p1_mla_shared_row_against_torch_sdpa():
    w = _dense_kv_identity_layout(
        tiny(kv_dtype="fp8_e4m3", scale_mode="tensor", D=12, Dv=8, H_q=4, H_kv=1, shared_kv=True))
    O, lse = oracle.attention(w)
    O_ref, lse_ref = _sdpa_reference(w)
    np.testing.assert_allclose(O, O_ref, rtol=0, atol=1e-12)
    np.testing.assert_allclose(lse, lse_ref, rtol=0, atol=1e-12)


# ---------------------------------------------------------------- P-2 ---

def _brute_force(w):
    """Pure-Python loops with math.fsum, straight from the definition."""
    def dq(byte, s):
        v = byte - 256 if byte >= 128 else byte
        return v * s
    def scale_at(arr, g, d):
        a = np.asarray(arr, np.float32).astype(float)
        if w.scale_mode == "tensor":
            return float(a.reshape(-1)[0])
        if w.scale_mode == "head":
            return float(a.reshape(-1)[g])
        return float(a[g, d])
    Q = _q_f64(w).numpy()
    G = w.group
    out = np.zeros((w.total_q, w.num_q_heads, w.head_dim_v))
    lse = np.zeros((w.total_q, w.num_q_heads))
    for b in range(w.batch):
        n, L = int(w.q_lens[b]), int(w.seq_lens_kv[b])
        for t in range(n):
            row = int(w.cu_seqlens_q[b]) + t
            for h in range(w.num_q_heads):
                g = h // G
                keys = range(L + t + 1) if w.causal else range(L + n)
                z = []
                for j in keys:
                    page = int(w.block_table[b][j // w.page_size])
                    slot = j % w.page_size
                    terms = [Q[row, h, d] * dq(int(w.k_cache[page, g, slot, d]), scale_at(w.k_scale, g, d))
                             for d in range(w.head_dim_qk)]
                    z.append(w.sm_scale * math.fsum(terms))
                m = max(z)
                e = [math.exp(x - m) for x in z]
                s = math.fsum(e)
                lse[row, h] = m + math.log(s)
                for d in range(w.head_dim_v):
                    acc = []
                    for jj, j in enumerate(keys):
                        page = int(w.block_table[b][j // w.page_size])
                        slot = j % w.page_size
                        acc.append(e[jj] / s * dq(int(w.v_cache[page, g, slot, d]), scale_at(w.v_scale, g, d)))
                    out[row, h, d] = math.fsum(acc)
    return out, lse


@pytest.mark.parametrize("mode", ["channel", "head", "tensor"])
def test_p2_brute_force_small(mode):
    w = tiny(seed=11, scale_mode=mode, q_lens=(2, 3), seq_lens_kv=(5, 11), D=6, Dv=5, P=4)
    O, lse = oracle.attention(w)
    Ob, lb = _brute_force(w)
    np.testing.assert_allclose(O, Ob, rtol=0, atol=1e-12)
    np.testing.assert_allclose(lse, lb, rtol=0, atol=1e-12)


# ---------------------------------------------------------------- P-3 ---

def test_p3_block_table_permutation_invariance_is_bitwise():
    w = tiny(seed=3, q_lens=(2, 3, 1), seq_lens_kv=(13, 6, 25), num_pages=40)
    O, lse = oracle.attention(w)
    rng = np.random.default_rng(99)
    perm = rng.permutation(w.num_pages)          # new physical slot of old page p = perm[p]
    k2 = np.empty_like(w.k_cache); k2[perm] = w.k_cache
    v2 = np.empty_like(w.v_cache); v2[perm] = w.v_cache
    t2 = np.where(w.block_table >= 0, perm[np.maximum(w.block_table, 0)], -1).astype(np.int32)
    w2 = dataclasses.replace(w, k_cache=k2, v_cache=v2, block_table=t2)
    O2, lse2 = oracle.attention(w2)
    assert np.array_equal(O, O2) and np.array_equal(lse, lse2)


# ---------------------------------------------------------------- P-4 ---

@pytest.mark.parametrize("kv_dtype,mode", [("i8", "channel"), ("fp8_e4m3", "tensor")])
def test_p4_single_key(kv_dtype, mode):
    w = tiny(seed=5, q_lens=(1,), seq_lens_kv=(0,), kv_dtype=kv_dtype, scale_mode=mode)
    O, lse = oracle.attention(w)
    page = int(w.block_table[0, 0])
    for h in range(w.num_q_heads):
        g = h // w.group
        k = _torch_dequant(w.k_cache[page, g, 0:1, :], kv_dtype, w.k_scale, mode, g).numpy()[0]
        v = _torch_dequant(w.v_cache[page, g, 0:1, :], kv_dtype, w.v_scale, mode, g).numpy()[0]
        q = _q_f64(w).numpy()[0, h]
        assert np.array_equal(O[0, h], v)
        assert lse[0, h] == w.sm_scale * float(q @ k)


# ---------------------------------------------------------------- P-5 ---

def test_p5_softmax_rows_sum_to_one():
    rng = np.random.default_rng(0)
    for n in (1, 2, 17, 300):
        z = rng.normal(0, 30, size=n)
        p, lse = oa._softmax_lse(z)
        assert abs(p.sum() - 1.0) <= 1e-14
        assert abs(lse - np.log(np.exp(z - z.max()).sum()) - z.max()) <= 1e-12


# ---------------------------------------------------------------- P-6 ---

@pytest.mark.parametrize("C", [1, 4, 8, 7, 40, 1000])
def test_p6_split_merge_equals_unsplit(C):
    w = tiny(seed=9, q_lens=(3, 1, 5), seq_lens_kv=(33, 0, 14), P=4)
    O, lse = oracle.attention(w)
    O2, lse2 = oracle.attention_split(w, C)
    np.testing.assert_allclose(O2, O, rtol=0, atol=1e-12)
    np.testing.assert_allclose(lse2, lse, rtol=0, atol=1e-12)


def _merge_over_cuts(w, b, cuts):
    """Partials of request b over the key ranges [cuts[i], cuts[i+1]), merged."""
    n = int(w.q_lens[b])
    k = len(cuts) - 1
    Oc = np.zeros((n, k, w.num_q_heads, w.head_dim_v))
    lc = np.full((n, k, w.num_q_heads), -np.inf)
    for i in range(k):
        Oc[:, i], lc[:, i] = oa.request_attention(w, b, cuts[i], cuts[i + 1])
    return oa.merge_partials(Oc, lc)


def test_p6_merge_over_any_partition_equals_unsplit():
    """The LSE merge is exact for any cut of the keys into contiguous ranges,
    not only for fixed-size chunks: ranges of one key, ranges that straddle
    pages, ranges past every visible key (lse = -inf), and the equal-tile items
    of a device-planned split (request cut into ceil(tiles / lt) items of
    ceil(tiles / items) 4-key tiles)."""
    w = tiny(seed=13, q_lens=(3, 1, 5), seq_lens_kv=(33, 0, 14), P=4)
    rng = np.random.default_rng(5)
    for b in range(w.batch):
        T = int(w.seq_lens_kv[b]) + int(w.q_lens[b])
        O, lse = oa.request_attention(w, b, 0, T)
        partitions = [list(range(T + 1)),                                  # one key each
                      [0] + sorted(rng.choice(np.arange(1, T), size=min(3, T - 1), replace=False).tolist()) + [T]
                      if T > 1 else [0, T]]
        tiles = -(-T // 4)
        for lt in (1, 2, 3):
            items = -(-tiles // lt)
            per = -(-tiles // items) * 4
            partitions.append([min(T, i * per) for i in range(items)] + [T])
        for cuts in partitions:
            O2, lse2 = _merge_over_cuts(w, b, cuts)
            np.testing.assert_allclose(O2, O, rtol=0, atol=1e-12)
            np.testing.assert_allclose(lse2, lse, rtol=0, atol=1e-12)


def test_p6_empty_chunks_have_minus_inf_lse():
    # token 0 of a request with L=2, n=6 sees keys 0..2; chunk [4, 8) is invisible to it
    w = tiny(seed=4, q_lens=(6,), seq_lens_kv=(2,), P=4)
    Oc, lc = oracle.chunk_partials(w, 0, 4)
    assert np.all(np.isneginf(lc[0, 1])) and np.all(Oc[0, 1] == 0)
    assert np.all(np.isfinite(lc[3, 1]))


# ---------------------------------------------------------------- P-7 ---

@pytest.mark.parametrize("causal", [True, False])
def test_p7_zero_query_closed_form(causal):
    w = tiny(seed=21, q_lens=(4, 1, 3), seq_lens_kv=(7, 0, 12), q_dtype="f32", causal=causal)
    w = dataclasses.replace(w, q=np.zeros_like(w.q))
    O, lse = oracle.attention(w)
    for b in range(w.batch):
        n, L = int(w.q_lens[b]), int(w.seq_lens_kv[b])
        for t in range(n):
            row = int(w.cu_seqlens_q[b]) + t
            cnt = (L + t + 1) if causal else (L + n)
            for h in range(w.num_q_heads):
                g = h // w.group
                assert abs(lse[row, h] - math.log(cnt)) <= 1e-14
                vals = []
                for j in range(cnt):
                    page = int(w.block_table[b, j // w.page_size])
                    vals.append(_torch_dequant(w.v_cache[page, g, j % w.page_size][None], "i8",
                                               w.v_scale, w.scale_mode, g).numpy()[0])
                np.testing.assert_allclose(O[row, h], np.mean(vals, axis=0), rtol=0, atol=1e-13)


# ---------------------------------------------------------------- P-8 ---

def test_p8_gqa_equals_replicated_heads():
    w = tiny(seed=31, H_q=6, H_kv=2, q_lens=(2, 3), seq_lens_kv=(10, 5))
    O, lse = oracle.attention(w)
    G = w.group
    rep = lambda a: np.repeat(a, G, axis=1)
    w1 = dataclasses.replace(
        w, num_kv_heads=w.num_q_heads, k_cache=rep(w.k_cache), v_cache=rep(w.v_cache),
        k_scale=np.repeat(w.k_scale, G, axis=0), v_scale=np.repeat(w.v_scale, G, axis=0))
    O1, lse1 = oracle.attention(w1)
    np.testing.assert_allclose(O1, O, rtol=0, atol=1e-13)
    np.testing.assert_allclose(lse1, lse, rtol=0, atol=1e-13)


# ---------------------------------------------------------------- P-9 ---

def test_p9_scale_algebra():
    w = tiny(seed=41, scale_mode="head")
    O, lse = oracle.attention(w)
    # per-channel with equal columns == per-head
    wc = dataclasses.replace(
        w, scale_mode="channel",
        k_scale=np.repeat(w.k_scale[:, None], w.head_dim_qk, axis=1),
        v_scale=np.repeat(w.v_scale[:, None], w.head_dim_v, axis=1))
    Oc, lsec = oracle.attention(wc)
    np.testing.assert_allclose(Oc, O, rtol=0, atol=1e-13)
    np.testing.assert_allclose(lsec, lse, rtol=0, atol=1e-13)
    # V scale x alpha => O x alpha, lse unchanged
    wv = dataclasses.replace(w, v_scale=(w.v_scale * np.float32(4.0)).astype(np.float32))
    Ov, lsev = oracle.attention(wv)
    np.testing.assert_allclose(Ov, 4.0 * O, rtol=1e-13, atol=1e-13)
    np.testing.assert_allclose(lsev, lse, rtol=0, atol=1e-13)
    # K scale x alpha with sm_scale / alpha => same logits
    wk = dataclasses.replace(w, k_scale=(w.k_scale * np.float32(8.0)).astype(np.float32),
                             sm_scale=w.sm_scale / 8.0)
    Ok, lsek = oracle.attention(wk)
    np.testing.assert_allclose(Ok, O, rtol=0, atol=1e-13)
    np.testing.assert_allclose(lsek, lse, rtol=0, atol=1e-13)


# ---------------------------------------------------------------- P-10 ---

def test_p10_e4m3fn_table_against_torch():
    raw = np.arange(256, dtype=np.uint8)
    ours = oracle.e4m3fn_decode(raw)
    lib = torch.from_numpy(raw).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    nan = np.isnan(lib)
    assert np.array_equal(np.isnan(ours), nan)
    assert set(np.nonzero(nan)[0].tolist()) == {0x7F, 0xFF}
    assert np.array_equal(ours[~nan], lib[~nan])
    assert np.nanmax(ours) == 448.0 and ours[0x08] == 2.0 ** -6 and ours[0x01] == 2.0 ** -9


def test_int8_decode_is_twos_complement():
    raw = np.array([0x00, 0x01, 0x7F, 0x80, 0x81, 0xFF], dtype=np.uint8)
    assert oracle.int8_decode(raw).tolist() == [0, 1, 127, -128, -127, -1]


def test_bf16_decode_against_torch():
    rng = np.random.default_rng(1)
    bits = rng.integers(0, 1 << 16, size=5000, dtype=np.uint16)
    bits = bits[((bits >> 7) & 0xFF) != 0xFF]            # drop inf/nan patterns
    lib = torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).to(torch.float64).numpy()
    assert np.array_equal(oracle.bf16_bits_to_f64(bits), lib)


# ---------------------------------------------------------------- P-11 ---

def test_p11_uniform_v_returns_v():
    w = tiny(seed=51, scale_mode="channel")
    v = w.v_cache.copy()
    v[:] = v[0, :, 0:1, :]                       # every row of every page equal per head
    w = dataclasses.replace(w, v_cache=v)
    O, _ = oracle.attention(w)
    for h in range(w.num_q_heads):
        g = h // w.group
        expect = _torch_dequant(v[0, g, 0:1], "i8", w.v_scale, "channel", g).numpy()[0]
        np.testing.assert_allclose(O[:, h], np.broadcast_to(expect, O[:, h].shape), rtol=0, atol=1e-14)


# ------------------------------------------------------ gather reference ---

def test_gather_bytes_matches_identity_layout_reshape():
    w = tiny(seed=61, q_lens=(2, 1), seq_lens_kv=(17, 6), num_pages=30)
    ref = oracle.gather_bytes(w)
    wd = _dense_kv_identity_layout(w)
    npp = w.block_table.shape[1]
    for b in range(w.batch):
        T = int(w.seq_lens_kv[b] + w.q_lens[b])
        for g in range(w.num_kv_heads):
            dense = wd.k_cache[b * npp:(b + 1) * npp, g].reshape(-1, w.head_dim_qk)[:T]
            assert np.array_equal(ref[b, g, :T], dense)
            assert not ref[b, g, T:].any()


def test_small_variants_are_finite():
    for i in range(1, 6):
        w = small_variant(i)
        O, lse = oracle.attention(w)
        assert np.isfinite(O).all() and np.isfinite(lse).all()


# ------------------------------------------------------ draft-tree mask ---
# The c8 decode kernel's optional attn_mask [bsz, max_q, max_q]: cached keys
# stay visible, appended key L + s is visible to token t iff mask[b, t, s].

def _with_tree(w, rows_of_b, mask_len=None):
    ml = mask_len or max(len(r) for r in rows_of_b)
    tm = np.full((w.batch, ml, ml), 0xAA, np.uint8)
    for b, rows in enumerate(rows_of_b):
        n = len(rows)
        tm[b, :n, :n] = np.asarray(rows, np.uint8)
    return dataclasses.replace(w, tree_mask=tm)


def test_tree_causal_triangle_equals_causal():
    w = tiny(seed=41, q_lens=(4, 3), seq_lens_kv=(6, 11))
    tri = [np.tril(np.ones((n, n), np.uint8)) for n in (4, 3)]
    wt = _with_tree(w, tri, mask_len=6)
    O, lse = oracle.attention(w)
    Ot, lset = oracle.attention(wt)
    assert np.array_equal(O, Ot) and np.array_equal(lse, lset)


# Drafts 0..4 with parents 1 -> 0, 2 -> 0, 3 -> 1, 4 -> 2; each token sees its
# ancestors and itself (written out by hand, not derived from the parents).
HAND_TREE = [[1, 0, 0, 0, 0],
             [1, 1, 0, 0, 0],
             [1, 0, 1, 0, 0],
             [1, 1, 0, 1, 0],
             [1, 0, 1, 0, 1]]
HAND_VISIBLE_DRAFTS = [{0}, {0, 1}, {0, 2}, {0, 1, 3}, {0, 2, 4}]


def test_tree_zero_query_closed_form():
    """Zero queries give uniform weights, and V row j = 100 * e_j (through the
    page table) makes O[t] the indicator of the visible keys / their count."""
    L, n = 2, 5
    w = tiny(seed=43, q_lens=(n,), seq_lens_kv=(L,), H_q=2, H_kv=1, D=8, Dv=8, scale_mode="head",
             q_dtype="f32")
    v = np.zeros_like(w.v_cache)
    for j in range(L + n):
        v[int(w.block_table[0, j // w.page_size]), 0, j % w.page_size, j] = 100
    w = dataclasses.replace(w, q=np.zeros_like(w.q), v_cache=v,
                            v_scale=np.ones_like(w.v_scale))
    w = _with_tree(w, [HAND_TREE], mask_len=7)
    O, lse = oracle.attention(w)
    for t in range(n):
        keys = set(range(L)) | {L + s for s in HAND_VISIBLE_DRAFTS[t]}
        want = np.array([100.0 / len(keys) if j in keys else 0.0 for j in range(8)])
        for h in range(2):
            np.testing.assert_allclose(O[t, h], want, rtol=0, atol=1e-13)
            assert abs(lse[t, h] - math.log(len(keys))) <= 1e-14


def test_tree_against_torch_sdpa():
    w = _dense_kv_identity_layout(tiny(seed=45, q_lens=(5, 4), seq_lens_kv=(7, 0), tree=True, tree_mask_len=6))
    O, lse = oracle.attention(w)
    npp, P, G = w.block_table.shape[1], w.page_size, w.group
    Q = _q_f64(w)
    for b in range(w.batch):
        n, L = int(w.q_lens[b]), int(w.seq_lens_kv[b])
        q0 = int(w.cu_seqlens_q[b])
        mask = torch.ones(n, L + n, dtype=torch.bool)
        mask[:, L:] = torch.from_numpy(w.tree_mask[b, :n, :n] != 0)
        for g in range(w.num_kv_heads):
            kraw = w.k_cache[b * npp:(b + 1) * npp, g].reshape(npp * P, -1)[:L + n]
            vraw = w.v_cache[b * npp:(b + 1) * npp, g].reshape(npp * P, -1)[:L + n]
            K = _torch_dequant(kraw, w.kv_dtype, w.k_scale, w.scale_mode, g)
            V = _torch_dequant(vraw, w.kv_dtype, w.v_scale, w.scale_mode, g)
            for h in range(g * G, (g + 1) * G):
                q = Q[q0:q0 + n, h]
                o = torch.nn.functional.scaled_dot_product_attention(
                    q[None, None], K[None, None], V[None, None], attn_mask=mask[None, None], scale=w.sm_scale)[0, 0]
                z = torch.where(mask, (q @ K.T) * w.sm_scale, torch.tensor(-math.inf, dtype=torch.float64))
                np.testing.assert_allclose(O[q0:q0 + n, h], o.numpy(), rtol=0, atol=1e-12)
                np.testing.assert_allclose(lse[q0:q0 + n, h], torch.logsumexp(z, 1).numpy(), rtol=0, atol=1e-12)


def test_tree_split_merge_equals_unsplit():
    w = tiny(seed=47, q_lens=(6, 3), seq_lens_kv=(13, 2), tree=True, tree_mask_len=8)
    O, lse = oracle.attention(w)
    for C in (4, 8):
        Os, lses = oracle.attention_split(w, C)
        np.testing.assert_allclose(Os, O, rtol=0, atol=1e-12)
        np.testing.assert_allclose(lses, lse, rtol=0, atol=1e-12)


# --------------------------------------------------------- planted bugs ---
# Each planted mistake in the oracle must make at least one pin fail.

def _fails(fn):
    try:
        fn()
    except AssertionError:
        return True
    return False


def test_planted_causal_off_by_one_is_caught(monkeypatch):
    monkeypatch.setattr(oa, "visible_keys", lambda L, n, t, c: (L + t) if c else (L + n))
    assert _fails(lambda: test_p7_zero_query_closed_form(True))


def test_planted_top_left_causal_is_caught(monkeypatch):
    monkeypatch.setattr(oa, "visible_keys", lambda L, n, t, c: (t + 1) if c else (L + n))
    assert _fails(lambda: test_p7_zero_query_closed_form(True))
    assert _fails(lambda: test_p1_dense_equivalence_against_torch_sdpa("i8", "channel", True))


def test_planted_unsigned_int8_is_caught(monkeypatch):
    monkeypatch.setattr(oa, "int8_decode", lambda raw: np.asarray(raw, np.uint8).astype(np.float64))
    assert _fails(lambda: test_p1_dense_equivalence_against_torch_sdpa("i8", "channel", True))


def test_planted_e4m3_bias_is_caught(monkeypatch):
    real = oa.e4m3fn_decode
    monkeypatch.setattr(oa, "e4m3fn_decode", lambda raw: real(raw) * 0.5)
    monkeypatch.setattr(oracle, "e4m3fn_decode", oa.e4m3fn_decode)
    assert _fails(test_p10_e4m3fn_table_against_torch)


def test_planted_interleaved_gqa_is_caught(monkeypatch):
    monkeypatch.setattr(oa, "query_heads_of", lambda g, G: range(g, g + 2 * G, 2) if G > 1 else range(g, g + 1))
    assert _fails(test_p8_gqa_equals_replicated_heads)


def test_planted_wrong_page_slot_is_caught(monkeypatch):
    def bad_gather(cache, table_row, g, T, P, dim):
        out = np.empty((T, dim), np.uint8)
        for j in range(T):
            out[j] = cache[int(table_row[j // P]), g, (j + 1) % P, :dim]
        return out
    monkeypatch.setattr(oa, "gather_rows", bad_gather)
    assert _fails(lambda: test_p1_dense_equivalence_against_torch_sdpa("i8", "channel", True))


def test_planted_transposed_channel_scale_is_caught(monkeypatch):
    real = oa._scale_vector
    def bad(scale, mode, g, dim):
        v = real(scale, mode, g, dim)
        return v[::-1].copy() if mode == "channel" else v
    monkeypatch.setattr(oa, "_scale_vector", bad)
    assert _fails(lambda: test_p2_brute_force_small("channel"))


def test_planted_unweighted_merge_is_caught(monkeypatch):
    def bad_merge(Oc, lc):
        fin = np.isfinite(lc)
        O = (Oc * fin[..., None]).sum(axis=1) / np.maximum(fin.sum(axis=1), 1)[..., None]
        return O, np.max(lc, axis=1)
    monkeypatch.setattr(oa, "merge_partials", bad_merge)
    assert _fails(lambda: test_p6_split_merge_equals_unsplit(4))
    assert _fails(test_p6_merge_over_any_partition_equals_unsplit)


def test_planted_transposed_tree_mask_is_caught(monkeypatch):
    # reads column t of the hand tree where row t belongs
    real = oa.visible_set
    full = np.asarray(HAND_TREE, np.uint8)
    monkeypatch.setattr(oa, "visible_set", lambda L, n, t, causal, tree_row=None:
                        real(L, n, t, causal, None if tree_row is None else full[:, t]))
    assert _fails(test_tree_zero_query_closed_form)


def test_planted_tree_mask_ignored_is_caught(monkeypatch):
    real = oa.visible_set
    monkeypatch.setattr(oa, "visible_set", lambda L, n, t, causal, tree_row=None: real(L, n, t, causal, None))
    assert _fails(test_tree_zero_query_closed_form)
    assert _fails(test_tree_against_torch_sdpa)
