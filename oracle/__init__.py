"""CPU oracle for paged-KV append/decode attention (test infrastructure).

This package is test infrastructure only.  It is a plain, slow, fp64 NumPy
statement of what the GPU path computes, written from the pages' description
of the method:

  * FastDeploy ``append_attention_c8_impl.cuh`` (multi-query c8 append
    attention over a paged int8/fp8 cache),
  * FlashInfer ``include/flashinfer/attention/persistent.cuh`` (paged KV
    address generation, partial LSE and the split-KV state reduction),
  * FlashInfer/XQA ``csrc/xqa/mla_sm120.cu`` (MLA decode over a shared
    576/512 latent row, page-list loading and the multi-block merge).

Only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may import it.  The product library never calls into it, and it
shares no code, tables or helpers with the HIP kernels.

``oracle.kv_write`` holds the cache append write (quantize the new tokens and
scatter them into their pages).

Every function is pinned by tests under ``tests/test_oracle_*.py`` against
closed forms, invariants, brute force and independent library routines; no
function here is "parity unpinned".
"""
from .reference import (  # noqa: F401
    bf16_bits_to_f64,
    int8_decode,
    e4m3fn_decode,
    dequant_rows,
    gather_rows,
    visible_keys,
    visible_set,
    request_attention,
    attention,
    chunk_partials,
    merge_partials,
    attention_split,
    gather_bytes,
)
from . import kv_write  # noqa: F401,E402
