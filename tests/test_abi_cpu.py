"""CPU checks of the C ABI: the library loads, exports every declared entry
point, and rejects invalid arguments before touching the GPU (no compute call
is made here)."""
import ctypes
import os
import re

import pytest

import paged_kv_attention_gather_amd as P
from paged_kv_attention_gather_amd import _lib as L

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "pagedattn.h")

FAKE = 0x100000  # aligned, never dereferenced: every call below fails validation first


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(L.LIB_PATH):
        from paged_kv_attention_gather_amd import build
        build.build()
    return P.lib()


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:const\s+)?[a-z_0-9]+\s*\*?\s*([a-z_0-9]+)\s*\(", text, flags=re.M)))


def test_header_declares_the_binding_exports():
    assert declared_functions() == sorted(L.EXPORTS)


def test_library_exports_every_declared_symbol(lib):
    for name in declared_functions():
        assert hasattr(lib, name), name
        assert ctypes.cast(getattr(lib, name), ctypes.c_void_p).value


def test_status_strings(lib):
    names = {0: "PA_OK", 1: "PA_ERR_INVALID_ARG", 2: "PA_ERR_UNSUPPORTED",
             3: "PA_ERR_WORKSPACE_TOO_SMALL", 4: "PA_ERR_HIP"}
    for code, name in names.items():
        assert lib.pa_status_string(code).decode() == name


def base_problem(**over):
    f = dict(batch=2, num_q_heads=8, num_kv_heads=2, head_dim_qk=128, head_dim_v=128, page_size=64,
             num_pages=64, max_pages_per_seq=16, max_q_len=4, max_kv_len=900, q_row_stride=8 * 128,
             k_stride_page=2 * 64 * 128, k_stride_head=64 * 128, k_stride_token=128,
             v_stride_page=2 * 64 * 128, v_stride_head=64 * 128, v_stride_token=128,
             q_dtype=L.DTYPE_BF16, kv_dtype=L.DTYPE_I8, scale_mode=L.SCALE_PER_CHANNEL, causal=1,
             sm_scale=0.088, chunk_size=256)
    f.update(over)
    return P.make_problem(**f)


def test_problem_struct_matches_header():
    """The binding's PaProblem mirrors the header field for field (same order)."""
    text = re.sub(r"/\*.*?\*/", "", open(HEADER).read(), flags=re.S)
    body = re.search(r"typedef struct pa_problem \{(.*?)\} pa_problem;", text, flags=re.S).group(1)
    names = re.findall(r"([a-z_0-9]+)\s*[,;]", body)
    assert names == [f for f, _ in L.PaProblem._fields_]


def test_flag_values_match_header():
    """The binding's PA_FLAG_* values are the header's."""
    text = re.sub(r"/\*.*?\*/", "", open(HEADER).read(), flags=re.S)
    flags = dict((k, int(v)) for k, v in re.findall(r"PA_FLAG_([A-Z_]+)\s*=\s*(\d+)", text))
    assert flags == {"DEFER_MERGE": L.FLAG_DEFER_MERGE, "FUSED_MERGE": L.FLAG_FUSED_MERGE,
                     "BALANCED_SPLIT": L.FLAG_BALANCED_SPLIT, "PERSISTENT": L.FLAG_PERSISTENT}


def test_workspace_size_formula(lib):
    prob = base_problem()
    total_q = 8
    mc = -(-(900 + 4) // 256)
    po = total_q * mc * 8 * 128 * 4
    expect = (po + 255) // 256 * 256 + total_q * mc * 8 * 4
    assert P.workspace_size(prob, total_q) == expect
    assert P.workspace_size(base_problem(chunk_size=0), total_q) == 0


def test_workspace_size_with_fused_merge_counters(lib):
    """PA_FLAG_FUSED_MERGE puts int32 counters [B, H_kv, ceil(max_q_len * G / 16)]
    first and the partials at the next 256-byte boundary; without split-KV
    nothing is needed."""
    prob = base_problem()
    total_q = 8
    plain = P.workspace_size(prob, total_q)
    fused = base_problem(flags=L.FLAG_FUSED_MERGE)
    G = fused.num_q_heads // fused.num_kv_heads
    groups = -(-(fused.max_q_len * G) // 16)
    counters = fused.batch * fused.num_kv_heads * groups * 4
    assert P.workspace_size(fused, total_q) == (counters + 255) // 256 * 256 + plain
    assert P.workspace_size(base_problem(chunk_size=0, flags=L.FLAG_FUSED_MERGE), total_q) == 0
    assert P.workspace_size(base_problem(flags=L.FLAG_DEFER_MERGE), total_q) == plain
    # the balanced split adds 256 bytes of plan in front of everything else
    both = base_problem(flags=L.FLAG_FUSED_MERGE | L.FLAG_BALANCED_SPLIT)
    assert P.workspace_size(both, total_q) == 256 + (counters + 255) // 256 * 256 + plain
    assert P.workspace_size(base_problem(flags=L.FLAG_BALANCED_SPLIT), total_q) == 256 + plain
    # the persistent split: the counters and one partial slot more per (token, head)
    mc = -(-(900 + 4) // 256) + 1
    po = total_q * mc * 8 * 128 * 4
    pers = (counters + 255) // 256 * 256 + (po + 255) // 256 * 256 + total_q * mc * 8 * 4
    assert P.workspace_size(base_problem(flags=L.FLAG_PERSISTENT), total_q) == pers


def _decode(prob, q_len=1, workspace=None, ws_bytes=0, **ptrs):
    p = dict(q=FAKE, k=FAKE, v=FAKE, ks=FAKE, vs=FAKE, lens=FAKE, table=FAKE, out=FAKE, lse=None)
    p.update(ptrs)
    return L.lib().paged_attn_decode(ctypes.byref(prob), q_len, p["q"], p["k"], p["v"], p["ks"], p["vs"],
                                     p["lens"], p["table"], p["out"], p["lse"], workspace, ws_bytes, None)


def _append(prob, total_q=8, workspace=None, ws_bytes=0, **ptrs):
    p = dict(q=FAKE, k=FAKE, v=FAKE, ks=FAKE, vs=FAKE, cu=FAKE, lens=FAKE, table=FAKE, out=FAKE, lse=None)
    p.update(ptrs)
    return L.lib().paged_attn_append(ctypes.byref(prob), total_q, p["q"], p["k"], p["v"], p["ks"], p["vs"],
                                     p["cu"], p["lens"], p["table"], p["out"], p["lse"], workspace, ws_bytes,
                                     None)


@pytest.mark.parametrize("over,status", [
    (dict(num_kv_heads=3), L.PA_ERR_INVALID_ARG),                 # H_q % H_kv != 0
    (dict(num_q_heads=0), L.PA_ERR_INVALID_ARG),
    (dict(head_dim_qk=96, head_dim_v=96), L.PA_ERR_UNSUPPORTED),
    (dict(page_size=48), L.PA_ERR_UNSUPPORTED),                   # not a power of two
    (dict(page_size=8), L.PA_ERR_UNSUPPORTED),                    # below 16
    (dict(chunk_size=100), L.PA_ERR_UNSUPPORTED),                 # not a multiple of 64
    (dict(q_dtype=7), L.PA_ERR_UNSUPPORTED),
    (dict(kv_dtype=L.DTYPE_BF16), L.PA_ERR_UNSUPPORTED),
    (dict(scale_mode=5), L.PA_ERR_INVALID_ARG),
    (dict(sm_scale=0.0), L.PA_ERR_INVALID_ARG),
    (dict(sm_scale=float("nan")), L.PA_ERR_INVALID_ARG),
    (dict(causal=2), L.PA_ERR_INVALID_ARG),
    (dict(q_row_stride=100), L.PA_ERR_INVALID_ARG),               # < H_q * D and misaligned
    (dict(k_stride_token=120), L.PA_ERR_INVALID_ARG),             # not 16-byte multiple
    (dict(batch=-1), L.PA_ERR_INVALID_ARG),
    (dict(batch=70000), L.PA_ERR_UNSUPPORTED),
    (dict(flags=16), L.PA_ERR_INVALID_ARG),                       # unknown flag bit
    (dict(flags=9), L.PA_ERR_INVALID_ARG),                        # persistent with a deferred merge
    (dict(flags=12), L.PA_ERR_INVALID_ARG),                       # persistent with the balanced split
    (dict(flags=3), L.PA_ERR_INVALID_ARG),                        # deferred and fused merge together
    (dict(flags=5), L.PA_ERR_INVALID_ARG),                        # deferred merge of a balanced split
    (dict(decode_waves=3), L.PA_ERR_INVALID_ARG),                 # schedule overrides: 0 or a listed value
    (dict(group_order=3), L.PA_ERR_INVALID_ARG),
    (dict(merge_in_kernel=-1), L.PA_ERR_INVALID_ARG),
])
def test_invalid_problems_are_rejected(lib, over, status):
    assert _decode(base_problem(**over)) == status
    assert lib.pa_last_error().decode()


def test_null_and_misaligned_pointers(lib):
    prob = base_problem(chunk_size=0)
    assert _decode(prob, q=None) == L.PA_ERR_INVALID_ARG
    assert _decode(prob, out=FAKE + 2) == L.PA_ERR_INVALID_ARG
    assert _append(prob, cu=None) == L.PA_ERR_INVALID_ARG
    assert lib.paged_attn_decode(None, 1, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, None, None, 0,
                                 None) == L.PA_ERR_INVALID_ARG


def test_decode_q_len_bounds(lib):
    assert _decode(base_problem(max_q_len=80), q_len=65) == L.PA_ERR_INVALID_ARG
    assert _decode(base_problem(), q_len=0) == L.PA_ERR_INVALID_ARG
    assert _decode(base_problem(max_q_len=1), q_len=2) == L.PA_ERR_INVALID_ARG


def test_workspace_too_small(lib):
    prob = base_problem()
    need = P.workspace_size(prob, 2)
    assert _decode(prob, q_len=1) == L.PA_ERR_WORKSPACE_TOO_SMALL
    assert _decode(prob, q_len=1, workspace=FAKE, ws_bytes=need - 1) == L.PA_ERR_WORKSPACE_TOO_SMALL


def test_mla_layout_requires_shared_rows(lib):
    prob = base_problem(head_dim_qk=576, head_dim_v=512, num_q_heads=16, num_kv_heads=1,
                        q_row_stride=16 * 576, k_stride_page=64 * 576, k_stride_head=64 * 576,
                        k_stride_token=576, v_stride_page=64 * 576, v_stride_head=64 * 576,
                        v_stride_token=576, chunk_size=0)
    assert _decode(prob, v=FAKE + 4096) == L.PA_ERR_UNSUPPORTED


def _tree(prob, q_len=1, mask=FAKE, mask_len=4, **ptrs):
    p = dict(q=FAKE, k=FAKE, v=FAKE, ks=FAKE, vs=FAKE, lens=FAKE, table=FAKE, out=FAKE, lse=None)
    p.update(ptrs)
    return L.lib().paged_attn_decode_tree(ctypes.byref(prob) if prob is not None else None, q_len, p["q"],
                                          p["k"], p["v"], p["ks"], p["vs"], p["lens"], p["table"], mask,
                                          mask_len, p["out"], p["lse"], None, 0, None)


def test_tree_decode_validation(lib):
    prob = base_problem(chunk_size=0, max_q_len=16)
    assert _tree(None) == L.PA_ERR_INVALID_ARG
    assert _tree(prob, q_len=4, mask=None) == L.PA_ERR_INVALID_ARG
    assert _tree(prob, q_len=4, mask_len=3) == L.PA_ERR_INVALID_ARG        # shorter than q_len
    assert _tree(prob, q_len=4, mask_len=65) == L.PA_ERR_INVALID_ARG       # beyond the 64-draft bitmask
    assert _tree(prob, q_len=17, mask_len=17) == L.PA_ERR_INVALID_ARG      # q_len > max_q_len


def test_tree_decode_row_limit_and_mla(lib):
    # G = 8: 9 drafts are 72 packed rows, more than the tree kernels hold
    prob = base_problem(num_q_heads=16, num_kv_heads=2, q_row_stride=16 * 128, chunk_size=0, max_q_len=16)
    assert _tree(prob, q_len=9, mask_len=9) == L.PA_ERR_UNSUPPORTED
    assert "64" in lib.pa_last_error().decode()
    mla = base_problem(head_dim_qk=576, head_dim_v=512, num_q_heads=16, num_kv_heads=1,
                       q_row_stride=16 * 576, k_stride_page=64 * 576, k_stride_head=64 * 576,
                       k_stride_token=576, v_stride_page=64 * 576, v_stride_head=64 * 576,
                       v_stride_token=576, chunk_size=0)
    assert _tree(mla, q_len=2, mask_len=2) == L.PA_ERR_UNSUPPORTED


def _kvw(prob, total_new=4, **ptrs):
    p = dict(k=FAKE, v=FAKE, cu=FAKE, lens=FAKE, table=FAKE, ks=FAKE, vs=FAKE, kc=FAKE, vc=FAKE)
    p.update(ptrs)
    return L.lib().paged_kv_write(ctypes.byref(prob) if prob is not None else None, total_new, p["k"], p["v"],
                                  p["cu"], p["lens"], p["table"], p["ks"], p["vs"], p["kc"], p["vc"], None)


def test_kv_write_validation(lib):
    prob = base_problem(chunk_size=0)
    assert _kvw(None) == L.PA_ERR_INVALID_ARG
    assert _kvw(prob, total_new=-1) == L.PA_ERR_INVALID_ARG
    assert _kvw(prob, k=None) == L.PA_ERR_INVALID_ARG
    assert _kvw(prob, v=None) == L.PA_ERR_INVALID_ARG
    assert _kvw(prob, cu=None) == L.PA_ERR_INVALID_ARG
    assert _kvw(prob, k=FAKE + 8) == L.PA_ERR_INVALID_ARG            # misaligned rows
    assert _kvw(base_problem(chunk_size=0, q_dtype=7)) == L.PA_ERR_UNSUPPORTED
    assert _kvw(base_problem(chunk_size=0, kv_dtype=L.DTYPE_BF16)) == L.PA_ERR_UNSUPPORTED
    assert _kvw(base_problem(chunk_size=0, page_size=48)) == L.PA_ERR_UNSUPPORTED
    mla = base_problem(head_dim_qk=576, head_dim_v=512, num_q_heads=16, num_kv_heads=1,
                       q_row_stride=16 * 576, k_stride_page=64 * 576, k_stride_head=64 * 576,
                       k_stride_token=576, v_stride_page=64 * 576, v_stride_head=64 * 576,
                       v_stride_token=576, chunk_size=0)
    assert _kvw(mla) == L.PA_ERR_INVALID_ARG                          # v_new must be NULL there
    assert _kvw(base_problem(batch=0)) == L.PA_OK
    assert _kvw(prob, total_new=0) == L.PA_OK


def test_empty_batch_is_a_no_op(lib):
    assert _decode(base_problem(batch=0)) == L.PA_OK
    assert _append(base_problem(batch=0), total_q=0) == L.PA_OK


def test_merge_validation(lib):
    m = lib.split_kv_merge
    assert m(FAKE, FAKE, None, FAKE, 0, 2, 2, 1, 8, 128, 256, 4, FAKE, None, None) == L.PA_ERR_INVALID_ARG
    assert m(FAKE, FAKE, None, FAKE, 1, 2, 2, 1, 8, 96, 256, 4, FAKE, None, None) == L.PA_ERR_UNSUPPORTED
    assert m(FAKE, FAKE, None, FAKE, 1, 2, 2, 1, 8, 128, 0, 4, FAKE, None, None) == L.PA_ERR_INVALID_ARG
    assert m(FAKE, FAKE, None, FAKE, 1, 0, 0, 1, 8, 128, 256, 4, FAKE, None, None) == L.PA_OK


def test_gather_validation(lib):
    prob = base_problem()
    g = lib.pa_gather_debug
    P_ = ctypes.byref(prob)
    assert g(P_, 0, FAKE, FAKE, FAKE, FAKE, FAKE, -1, FAKE, None, None) == L.PA_ERR_INVALID_ARG
    assert g(P_, 0, None, FAKE, FAKE, FAKE, FAKE, 64, FAKE, None, None) == L.PA_ERR_INVALID_ARG
    assert g(P_, 0, FAKE, FAKE, FAKE, FAKE, FAKE, 16 * 64 + 1, FAKE, None, None) == L.PA_ERR_INVALID_ARG
    assert g(P_, 5, FAKE, FAKE, FAKE, FAKE, FAKE, 64, FAKE, None, None) == L.PA_ERR_INVALID_ARG   # loader
    assert g(P_, -1, FAKE, FAKE, FAKE, FAKE, FAKE, 64, FAKE, None, None) == L.PA_ERR_INVALID_ARG
    assert g(P_, 0, FAKE, None, FAKE, FAKE, FAKE, 64, FAKE, FAKE, None) == L.PA_ERR_INVALID_ARG   # V dst, no V
    mla = base_problem(num_q_heads=16, num_kv_heads=1, head_dim_qk=576, head_dim_v=512, q_row_stride=16 * 576,
                       k_stride_page=64 * 576, k_stride_head=64 * 576, k_stride_token=576,
                       v_stride_page=64 * 576, v_stride_head=64 * 576, v_stride_token=576)
    assert g(ctypes.byref(mla), 2, FAKE, FAKE, FAKE, FAKE, FAKE, 64, FAKE, FAKE, None) == L.PA_ERR_INVALID_ARG


def test_read_probe_validation(lib):
    r = lib.pa_kv_read_probe
    assert r(ctypes.byref(base_problem()), 0, FAKE, FAKE, FAKE, FAKE, FAKE, None) == L.PA_ERR_INVALID_ARG
    assert r(ctypes.byref(base_problem()), 1, FAKE, None, FAKE, FAKE, FAKE, None) == L.PA_ERR_INVALID_ARG
    mla = base_problem(num_q_heads=16, num_kv_heads=1, head_dim_qk=576, head_dim_v=512)
    assert r(ctypes.byref(mla), 1, FAKE, FAKE, FAKE, FAKE, FAKE, None) == L.PA_ERR_UNSUPPORTED
    assert r(ctypes.byref(base_problem(batch=0)), 1, FAKE, FAKE, FAKE, FAKE, FAKE, None) == L.PA_OK


def test_missing_library_fails_loudly(monkeypatch, tmp_path):
    monkeypatch.setattr(L, "_lib", None)
    monkeypatch.setattr(L, "LIB_PATH", str(tmp_path / "absent.so"))
    with pytest.raises(RuntimeError, match="missing"):
        L.lib()


def test_bench_refuses_more_than_one_gpu():
    """bench.py measures one GPU: --gpus N > 1 exits with status 2 and says why
    (before touching a device)."""
    import subprocess
    import sys
    root = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    r = subprocess.run([sys.executable, os.path.join(root, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120, cwd=root)
    assert r.returncode == 2
    assert "one GPU" in r.stderr and not r.stdout.strip()


def _decode_scratch(prob, q_len=1, **ptrs):
    p = dict(q=FAKE, k=FAKE, v=FAKE, ks=FAKE, vs=FAKE, lens=FAKE, table=FAKE, out=FAKE, lse=None)
    p.update(ptrs)
    return L.lib().paged_attn_decode_scratch(ctypes.byref(prob), q_len, p["q"], p["k"], p["v"], p["ks"],
                                             p["vs"], p["lens"], p["table"], p["out"], p["lse"], None)


def test_decode_scratch_validation(lib):
    """The allocation-free decode entry point rejects, before touching the GPU,
    a problem whose split-KV workspace exceeds its static scratch, a deferred
    merge (its partials are unreachable) and the usual invalid problems."""
    assert L.DECODE_SCRATCH_BYTES == 32 << 20
    header = open(HEADER).read()
    assert "#define PA_DECODE_SCRATCH_BYTES ((size_t)32 << 20)" in header
    # 64 requests x 32 heads x 128 dims x 9 chunks of fp32 partials: ~9.4 MB, fits;
    # the same with 64-key chunks over 65536 cached keys does not
    fits = base_problem(batch=64, num_q_heads=32, num_kv_heads=8, max_q_len=1, max_kv_len=4096,
                        q_row_stride=32 * 128, chunk_size=512)
    assert P.workspace_size(fits, 64) <= L.DECODE_SCRATCH_BYTES
    big = base_problem(batch=64, num_q_heads=32, num_kv_heads=8, max_q_len=1, max_kv_len=65536,
                       q_row_stride=32 * 128, chunk_size=64, max_pages_per_seq=1025)
    assert P.workspace_size(big, 64) > L.DECODE_SCRATCH_BYTES
    assert _decode_scratch(big) == L.PA_ERR_WORKSPACE_TOO_SMALL
    assert "static scratch" in lib.pa_last_error().decode()
    assert _decode_scratch(base_problem(flags=L.FLAG_DEFER_MERGE)) == L.PA_ERR_INVALID_ARG
    assert _decode_scratch(base_problem(num_kv_heads=3)) == L.PA_ERR_INVALID_ARG
    assert _decode_scratch(base_problem(), q_len=0) == L.PA_ERR_INVALID_ARG
    assert _decode_scratch(base_problem(batch=0)) == L.PA_OK     # nothing to do, nothing touched
