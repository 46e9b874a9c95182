"""GPU parity of the cache append write (paged_kv_write through the C ABI):
the whole K and V caches after the write are compared byte for byte with the
oracle's (written slots and untouched ones alike)."""
import math
import zlib

import numpy as np
import pytest

import oracle
from gpu_util import announce, need_gpu
from workloads import config_workload, kv_write_inputs, make_workload

pytestmark = pytest.mark.gpu


def _wl(name, **kw):
    base = dict(name=name, seed=zlib.crc32(name.encode()) % 10000, num_q_heads=8, num_kv_heads=2, head_dim_qk=128,
                head_dim_v=128, page_size=64, q_dtype="bf16", kv_dtype="i8", scale_mode="channel",
                causal=True, sm_scale=0.1, chunk_size=0, decode=False)
    base.update(kw)
    return make_workload(**base)


def _run_write(w, k_in, v_in):
    torch = need_gpu()
    import paged_kv_attention_gather_amd as P
    from paged_kv_attention_gather_amd.harness import problem_for
    dev = "cuda"
    t = lambda a, dt=None: torch.from_numpy(np.ascontiguousarray(a if dt is None else a.astype(dt))).to(dev)
    if w.q_dtype == "bf16":
        kn = torch.from_numpy(np.ascontiguousarray(k_in).view(np.int16)).to(dev)
        vn = None if v_in is None else torch.from_numpy(np.ascontiguousarray(v_in).view(np.int16)).to(dev)
    else:
        kn, vn = t(k_in, np.float32), (None if v_in is None else t(v_in, np.float32))
    kc = t(w.k_cache)
    vc = kc if w.shared_kv else t(w.v_cache)
    prob = problem_for(w)
    P.paged_kv_write(prob, int(w.total_q), kn, vn, t(w.cu_seqlens_q, np.int32), t(w.seq_lens_kv, np.int32),
                     t(w.block_table, np.int32), t(w.k_scale, np.float32), t(w.v_scale, np.float32), kc,
                     None if w.shared_kv else vc)
    torch.cuda.synchronize()
    return kc.cpu().numpy(), (None if w.shared_kv else vc.cpu().numpy())


def _check(w, spread=1.3, in_dtype=None, values=None):
    in_dtype = in_dtype or w.q_dtype
    if values is None:
        k_vals, v_vals, k_in, v_in = kv_write_inputs(w, spread=spread, in_dtype=in_dtype)
    else:
        k_vals, v_vals = values
        k_in, v_in = k_vals, v_vals
    kc, vc = _run_write(w, k_in, v_in)
    ref_k = oracle.kv_write.kv_write(w.k_cache, k_vals, w.k_scale, w.scale_mode, w.kv_dtype, w.block_table,
                                     w.seq_lens_kv, w.cu_seqlens_q, w.page_size)
    bad = np.argwhere(kc != ref_k)
    assert bad.size == 0, f"K cache differs at {len(bad)} bytes, first {bad[:4].tolist()}"
    if not w.shared_kv:
        ref_v = oracle.kv_write.kv_write(w.v_cache, v_vals, w.v_scale, w.scale_mode, w.kv_dtype, w.block_table,
                                         w.seq_lens_kv, w.cu_seqlens_q, w.page_size)
        bad = np.argwhere(vc != ref_v)
        assert bad.size == 0, f"V cache differs at {len(bad)} bytes, first {bad[:4].tolist()}"
    # the write really changed the appended slots (the inputs are not the old bytes)
    assert not np.array_equal(kc, w.k_cache) or int(w.q_lens.sum()) == 0


KV_WRITE_CASES = {
    "i8_channel_bf16_ragged": dict(q_lens=[5, 0, 70, 1], seq_lens_kv=[10, 33, 0, 129]),
    "i8_head_f32_d64_page16": dict(head_dim_qk=64, head_dim_v=64, page_size=16, scale_mode="head",
                                   q_dtype="f32", q_lens=[17, 3], seq_lens_kv=[15, 48]),
    "i8_tensor_page1024": dict(page_size=1024, scale_mode="tensor", q_lens=[40, 9], seq_lens_kv=[1000, 2047]),
    "fp8_channel_d64": dict(head_dim_qk=64, head_dim_v=64, kv_dtype="fp8_e4m3", q_lens=[6, 33],
                            seq_lens_kv=[60, 1], scale_range=(0.0005, 0.008)),
    "fp8_tensor_mla_shared": dict(num_q_heads=16, num_kv_heads=1, head_dim_qk=576, head_dim_v=512,
                                  shared_kv=True, kv_dtype="fp8_e4m3", scale_mode="tensor", q_lens=[2, 3],
                                  seq_lens_kv=[63, 900]),
    "i8_mla_shared_channel_f32": dict(num_q_heads=16, num_kv_heads=1, head_dim_qk=576, head_dim_v=512,
                                      shared_kv=True, scale_mode="channel", q_dtype="f32", q_lens=[1, 4],
                                      seq_lens_kv=[0, 70]),
}


@pytest.mark.parametrize("case", sorted(KV_WRITE_CASES))
def test_kv_write_bit_exact(case):
    need_gpu()
    w = _wl(case, **KV_WRITE_CASES[case])
    announce(f"kv write {case}")
    _check(w)


def test_kv_write_ties_round_to_even():
    """fp32 inputs at exact half-integer multiples of power-of-two scales:
    every ratio is a tie, which must go to the even code."""
    need_gpu()
    w = _wl("ties", scale_mode="head", q_dtype="f32", q_lens=[9, 4], seq_lens_kv=[3, 70])
    w.k_scale[:] = np.array([0.25, 0.5], np.float32)
    w.v_scale[:] = np.array([2.0, 0.125], np.float32)
    rng = np.random.default_rng(17)
    def ties(scale):
        k = rng.integers(-140, 140, size=(w.total_q, 2, 128)).astype(np.float32) + np.float32(0.5)
        return (k * scale[None, :, None]).astype(np.float32)
    kv, vv = ties(w.k_scale), ties(w.v_scale)
    announce("kv write ties")
    _check(w, values=(kv, vv))
    codes = oracle.kv_write.int8_quantize(kv[0, 0, :4], np.float32(0.25)).view(np.int8)
    assert np.all(codes % 2 == 0) or np.all(np.abs(codes) == 127)


@pytest.mark.parametrize("idx", [3, 5])
def test_kv_write_full_workload(idx):
    """The appended tokens of the append-prefill workload (int8 per head,
    ~5k tokens x 8 heads) and of the MLA workload (fp8, shared rows)."""
    need_gpu()
    w = config_workload(idx)
    announce(f"kv write config_workload({idx}) {w.name}")
    _check(w, spread=1.2)
