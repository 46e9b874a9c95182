"""Helpers for the GPU parity tests: tolerance checks against the oracle."""
import sys

import numpy as np
import pytest

# Tolerances of the method's statement: bf16 output within max-abs 1e-2 and
# relative RMS 5e-3 of the exact result, per-row natural LSE within 1e-3.
MAX_ABS = 1e-2
REL_RMS = 5e-3
LSE_ABS = 1e-3


def need_gpu():
    torch = pytest.importorskip("torch")
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import paged_kv_attention_gather_amd as P
    P.lib()  # a GPU run without the built library must fail, not skip
    return torch


def announce(msg):
    print(f"[gpu] {msg}", flush=True)
    sys.stdout.flush()


def compare(out, lse, O_ref, lse_ref, rows=None, what=""):
    """Assert the tolerance bar over the selected token rows (all by default)."""
    if rows is not None:
        out, lse, O_ref, lse_ref = out[rows], lse[rows], O_ref[rows], lse_ref[rows]
    assert np.isfinite(out).all(), f"{what}: non-finite output"
    err = np.abs(out - O_ref)
    max_abs = float(err.max()) if err.size else 0.0
    den = float(np.sqrt(np.sum(O_ref ** 2)))
    rel_rms = float(np.sqrt(np.sum(err ** 2)) / den) if den > 0 else 0.0
    lse_err = float(np.abs(lse - lse_ref).max()) if lse.size else 0.0
    print(f"  {what}: max_abs={max_abs:.3e} rel_rms={rel_rms:.3e} lse_abs={lse_err:.3e}", flush=True)
    assert max_abs <= MAX_ABS, f"{what}: max-abs {max_abs} > {MAX_ABS}"
    assert rel_rms <= REL_RMS, f"{what}: rel-RMS {rel_rms} > {REL_RMS}"
    assert lse_err <= LSE_ABS, f"{what}: lse {lse_err} > {LSE_ABS}"
    return max_abs, rel_rms, lse_err


def token_rows(w, requests):
    rows = []
    for b in requests:
        rows.extend(range(int(w.cu_seqlens_q[b]), int(w.cu_seqlens_q[b + 1])))
    return np.array(rows, dtype=np.int64)


# --------------------------------------------------- oracle over every request --

def _oracle_requests(idx, kw, reqs):
    """Worker: the oracle on the listed requests of config_workload(idx, **kw)
    (regenerated from its seed in this process)."""
    import oracle
    from workloads import config_workload
    w = config_workload(idx, **kw)
    O, lse = oracle.attention(w, requests=reqs)
    rows = token_rows(w, reqs)
    return rows, O[rows], lse[rows]


_ORACLE_CACHE = {}


def oracle_every_request(idx, workers=8, **kw):
    """Oracle outputs of every request of a full-size workload, computed in
    `workers` CPU processes (spawned fresh: they never touch the GPU), each
    regenerating the seeded workload and taking every `workers`-th request.
    Cached per (workload, options) for the session."""
    key = (idx, tuple(sorted(kw.items())))
    if key in _ORACLE_CACHE:
        return _ORACLE_CACHE[key]
    import concurrent.futures as cf
    import multiprocessing as mp
    import os
    from workloads import config_workload
    w = config_workload(idx, **kw)
    parts = [list(range(i, w.batch, workers)) for i in range(min(workers, w.batch))]
    O = np.full((w.total_q, w.num_q_heads, w.head_dim_v), np.nan)
    lse = np.full((w.total_q, w.num_q_heads), np.nan)
    saved = {k: os.environ.get(k) for k in ("OMP_NUM_THREADS", "OPENBLAS_NUM_THREADS", "MKL_NUM_THREADS")}
    for k in saved:
        os.environ[k] = "2"
    try:
        with cf.ProcessPoolExecutor(max_workers=len(parts), mp_context=mp.get_context("spawn")) as ex:
            for rows, o, l in ex.map(_oracle_requests, [idx] * len(parts), [kw] * len(parts), parts):
                O[rows], lse[rows] = o, l
    finally:
        for k, v in saved.items():
            if v is None:
                os.environ.pop(k, None)
            else:
                os.environ[k] = v
    assert np.isfinite(O).all() and np.isfinite(lse).all(), "oracle left rows unset"
    _ORACLE_CACHE[key] = (O, lse)
    return O, lse
