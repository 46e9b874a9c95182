"""paged_attn_decode_scratch (the allocation-free decode entry point) against
paged_attn_decode with a caller workspace: same inputs, same outputs, over two
calls in a row on the shared static scratch, the second with a smaller
problem (fewer requests, shorter lengths, fewer chunks), with and without the
in-kernel merge, and against the oracle."""
import numpy as np
import pytest

import oracle
from gpu_util import announce, compare, need_gpu
from workloads import config_workload, small_variant

pytestmark = pytest.mark.gpu


def _scratch_call(dp):
    from paged_kv_attention_gather_amd import _lib as L
    dp.out.zero_()
    dp.lse.zero_()
    L.paged_attn_decode_scratch(dp.prob, int(dp.w.decode_q_len), dp.q, dp.k_cache, dp.v_cache, dp.k_scale,
                                dp.v_scale, dp.seq_lens_kv, dp.block_table, dp.out, dp.lse)
    return dp.outputs()


def _workspace_call(dp):
    dp.out.zero_()
    dp.lse.zero_()
    dp.run()
    return dp.outputs()


@pytest.mark.parametrize("fused", [False, True])
def test_scratch_decode_matches_workspace_decode(fused):
    need_gpu()
    from paged_kv_attention_gather_amd.harness import DeviceProblem
    big = config_workload(2)        # 64 requests, chunk 512, ~9.4 MB of partials
    small = small_variant(2)        # a few requests with short, ragged lengths
    for w in (big, small):
        announce(f"scratch decode {w.name} fused={fused}")
        dp = DeviceProblem(w, fused_merge=fused)
        ref = _workspace_call(dp)
        got = _scratch_call(dp)
        assert np.array_equal(ref[0], got[0]) and np.array_equal(ref[1], got[1]), f"{w.name}: differs"
        if w is small:
            O_ref, lse_ref = oracle.attention(w)
            compare(got[0], got[1], O_ref, lse_ref, what=f"{w.name} scratch fused={fused}")
