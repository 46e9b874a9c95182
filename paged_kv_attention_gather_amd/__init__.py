"""MI355X (gfx950) paged-KV append/decode attention.

The computation lives in libpagedattn.so (hand-written HIP kernels behind the
C ABI of include/pagedattn.h); this package holds its ctypes binding, a
device-marshalling helper and the build script.
"""
from ._lib import (  # noqa: F401
    EXPORTS,
    LIB_PATH,
    PaProblem,
    PagedAttnError,
    lib,
    make_problem,
    paged_attn_append,
    paged_attn_decode,
    paged_attn_decode_scratch,
    paged_attn_decode_tree,
    paged_kv_write,
    pa_gather_debug,
    pa_kv_read_probe,
    split_kv_merge,
    workspace_size,
)
