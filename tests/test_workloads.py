"""Seeded generators: determinism and the shapes/structure each workload states."""
import numpy as np
import pytest

from workloads import config_workload, small_variant


def test_same_seed_same_bytes():
    a, b = small_variant(4), small_variant(4)
    for f in ("q", "k_cache", "v_cache", "k_scale", "v_scale", "block_table", "seq_lens_kv"):
        assert np.array_equal(getattr(a, f), getattr(b, f)), f


def test_tiny_append_matches_its_statement():
    w = config_workload(1)
    assert w.seq_lens_kv.tolist() == [37, 50] and w.q_lens.tolist() == [3, 1]
    assert w.q.dtype == np.float32 and w.q.shape == (4, 4, 64)
    assert w.k_cache.shape == (16, 1, 16, 64) and w.num_pages == 16
    assert w.block_table.shape == (2, 4)
    used = w.block_table[w.block_table >= 0]
    assert len(set(used.tolist())) == 7                    # 3 + 4 distinct pages
    assert np.all((w.k_scale >= 0.005) & (w.k_scale <= 0.02))
    kv = w.k_cache.view(np.int8)
    assert kv.min() >= -127 and kv.max() <= 127


@pytest.mark.slow
def test_mla_workload_scale_and_shared_row():
    w = config_workload(5)
    assert w.shared_kv and w.v_cache is None and w.head_dim_v == 512
    assert w.k_scale.shape == (1,) and w.k_scale[0] == w.v_scale[0]
    assert np.all((w.seq_lens_kv >= 4096) & (w.seq_lens_kv <= 16384))
    # the largest stored magnitude is exactly the e4m3fn maximum 448 (0x7E / 0xFE)
    assert np.any((w.k_cache & 0x7F) == 0x7E)
    assert not np.any((w.k_cache & 0x7F) == 0x7F)


def test_unused_table_entries_are_minus_one():
    w = small_variant(2)
    T = w.kv_tokens()
    for b in range(w.batch):
        n = int((T[b] + w.page_size - 1) // w.page_size)
        assert np.all(w.block_table[b, :n] >= 0) and np.all(w.block_table[b, n:] == -1)
