#!/usr/bin/env python3
"""Benchmark of the paged-KV attention hot path on one MI355X.

A step is one call of the C ABI (attention kernel + split-KV merge) over one
batch of the synthetic workload, inputs resident in HBM.  Before every timed
step the L2 and the 256 MB last-level cache are flushed (outside the events)
by READING a 1 GiB buffer, so the KV bytes really come from HBM and no dirty
flush data is left to be written back while the step runs (a write-based
flush costs a read kernel about a third of its bandwidth).  The default
workload is the int8 decode case (B=64, q_len 1, 32/8 heads, D=128, page 64, KV lens U[512, 4096],
per-channel scales, chunk 512): the one the decode KV-bandwidth metric is
quoted on.  --config 1..5 selects another workload.

Prints ONE JSON line with the headline metric, the roofline of the attention
kernel and the oracle's throughput on a bounded sample of the same workload
(cpu_baseline).  A split-KV step makes the ABI call with PA_FLAG_DEFER_MERGE
and then runs split_kv_merge.  The steps are timed twice with HIP events on
the launch stream: once with one event pair around the whole step (nothing
recorded between the two launches: ms_per_step and value), once more with an
event between them as well (roofline.kernel_ms, the attention kernel alone,
and merge_ms).  roofline.frac is the attention kernel's (algorithmic bytes
or flops over its event time); roofline.step_frac is the whole step's
(attention + merge).  For the decode workloads the line also carries the
read probe (pa_kv_read_probe: the same tiles through the same loader with no
arithmetic), the read bandwidth this access pattern allows.  The default run
also times the append, spec-decode and MLA workloads ("configs", fewer steps,
same flush and events).  --merge fused makes one call with
PA_FLAG_FUSED_MERGE instead (where the library merges inside the attention
kernel, the step is one launch; it measured slower on these workloads, so it
is not the default).  The roofline's "traffic" (HBM bytes per launch of the
attention kernel) comes from the FETCH_SIZE / WRITE_SIZE counter summary
committed in profiles/, and is null when that summary was taken on other
kernel sources.
"""
import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0       # MI355X HBM3E, GB/s
MFMA_F16_PEAK_TFS = 2516.6  # dense f16/bf16 MFMA: 256 CU x 2.4 GHz x 4096 flop/clk

WORKLOAD_TEXT = {
    1: "tiny_append: B=2 H_q=4 H_kv=1 D=64 P=16 L={37,50} n={3,1} fp32 Q int8 per-head causal",
    2: "decode_int8: B=64 q_len=1 H_q=32 H_kv=8 D=128 P=64 L~U[512,4096] int8 per-channel chunk=512",
    3: "append_prefill: B=8 n~U[256,1024] L~U[0,2048] H_q=32 H_kv=8 D=128 P=64 int8 per-head causal",
    4: "spec_decode: B=128 q_len=5 H_q=64 H_kv=8 D=128 P=64 L~lognormal(2048,1)[128,32768] int8 per-channel chunk=1024",
    5: "mla_decode: B=32 q_len=1 H_q=128 H_kv=1 D_qk=576 D_v=512 P=64 L~U[4096,16384] fp8 per-tensor chunk=3072",
}


def work_figures(w):
    """Algorithmic work of one call: KV bytes, total bytes, useful flops."""
    T = w.kv_tokens().astype(np.int64)
    H, Dq, Dv = w.num_kv_heads, w.head_dim_qk, w.head_dim_v
    row_bytes = Dq if w.shared_kv else Dq + Dv
    kv = int((T * H * row_bytes).sum())
    q_bytes = w.q.nbytes
    out_bytes = w.total_q * w.num_q_heads * (Dv * 2 + 4)
    table = int(((T + w.page_size - 1) // w.page_size).sum()) * 4
    scales = w.k_scale.nbytes + w.v_scale.nbytes
    total = kv + q_bytes + out_bytes + table + scales
    if getattr(w, "tree_mask", None) is not None:
        total += int((w.q_lens.astype(np.int64) ** 2).sum())   # the mask entries that are read
    vis = 0
    for b in range(w.batch):
        n, L = int(w.q_lens[b]), int(w.seq_lens_kv[b])
        if w.causal:
            vis += n * L + n * (n + 1) // 2
        else:
            vis += n * (L + n)
    flops = vis * w.num_q_heads * 2 * (Dq + Dv)
    return kv, total, flops


def cpu_baseline(idx, budget_s=15.0):
    """Time the fp64 oracle (as it stands) on a bounded sample of requests."""
    import oracle
    from workloads import config_workload
    try:
        from threadpoolctl import threadpool_info
        threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:
        threads = 1
    w = config_workload(idx)
    T = w.kv_tokens().astype(np.int64)
    order = np.random.default_rng(7).permutation(w.batch)
    done, t0 = [], time.perf_counter()
    for b in order:
        oracle.attention(w, requests=[int(b)])
        done.append(int(b))
        if time.perf_counter() - t0 > budget_s:
            break
    dt = time.perf_counter() - t0
    row_bytes = w.head_dim_qk if w.shared_kv else w.head_dim_qk + w.head_dim_v
    kv = int((T[done] * w.num_kv_heads * row_bytes).sum())
    vis = sum(int(w.q_lens[b]) * int(w.seq_lens_kv[b]) + int(w.q_lens[b]) * (int(w.q_lens[b]) + 1) // 2
              for b in done)
    flops = vis * w.num_q_heads * 2 * (w.head_dim_qk + w.head_dim_v)
    if idx in (1, 3):
        val, unit = flops / dt / 1e12, "TFLOP/s"
    else:
        val, unit = kv / dt / 1e9, "GB/s"
    return {"value": round(val, 6), "unit": unit, "cores": int(threads), "kind": "oracle",
            "sample": f"{len(done)} of {w.batch} requests of {w.name} ({dt:.1f} s, fp64 NumPy, "
                      f"host cores visible: {len(os.sched_getaffinity(0))})"}


def kernel_name(dp):
    """Name of the attention kernel the library launches for this problem."""
    w = dp.w
    if w.shared_kv:
        return "paged_mla_pc_kernel" if w.kv_dtype == "fp8_e4m3" else "paged_mla_i8_kernel"
    rows = (int(w.decode_q_len) if dp.decode else int(w.q_lens.max())) * (w.num_q_heads // w.num_kv_heads)
    return "paged_decode_kernel" if rows <= 32 else "paged_attn_kernel"


def compute_dtype(dp):
    """MFMA operand types: int8 caches through the decode kernel, the 16-row
    shared-tile variants or the MLA kernel take S = K Q^T on the int8 MFMA (f16
    for PV); e4m3fn MLA caches take it on the fp8 MFMA with the query in fp8
    digits ("fp8x2": two digits, bf16 query; "fp8x3": three); every other path
    multiplies f16 (cache values converted exactly)."""
    w = dp.w
    if w.shared_kv:
        if w.kv_dtype == "i8":
            return "i8/f16"
        two = w.q_dtype == "bf16" and w.scale_mode != "channel"
        return ("fp8x2" if two else "fp8x3") + "/f16"
    rows = (int(w.decode_q_len) if dp.decode else int(w.q_lens.max())) * (w.num_q_heads // w.num_kv_heads)
    if w.kv_dtype == "i8" and not w.shared_kv and rows <= 64:
        return "i8/f16"
    return "f16"


def hbm_traffic(config, chunk, merge, balanced=False):
    """HBM bytes per launch of the attention kernel from the committed counter
    summary, or (None, reason) when it does not cover these kernel sources."""
    from paged_kv_attention_gather_amd import build
    path = os.path.join(ROOT, "profiles", "hbm_traffic_counters.md")
    if not os.path.exists(path):
        return None, "no counter summary"
    text = open(path).read()
    start = text.find("```json")
    if start < 0:
        return None, "no counter table"
    data = json.loads(text[start + 7:text.index("```", start + 7)])
    digest = build.source_digest()
    if data.get("source_digest") != digest:
        return None, f"counters taken on sources {data.get('source_digest')}, kernel now {digest}"
    row = data.get("configs", {}).get(str(config))
    if (not row or row.get("chunk_size") != chunk or (chunk > 0 and row.get("merge", "separate") != merge)
            or bool(row.get("balanced", False)) != balanced):
        return None, "no counters for this workload"
    fetch = row["fetch_kib_per_dispatch"] * 1024 * data["fetch_factor"]
    write = row["write_kib_per_dispatch"] * 1024 * data["write_factor"]
    return int(round(fetch + write)), "profiles/hbm_traffic_counters.md"


def bench_kv_write(args):
    """One JSON line for paged_kv_write: quantize + scatter the appended tokens
    of workload ``args.config`` (bf16 rows in, int8/fp8 bytes out)."""
    import torch
    import paged_kv_attention_gather_amd as P
    from paged_kv_attention_gather_amd.harness import problem_for
    from workloads import config_workload, kv_write_inputs
    w = config_workload(args.config)
    _, _, k_in, v_in = kv_write_inputs(w, spread=1.2, in_dtype="bf16")
    dev = "cuda"
    t = lambda a, dt: torch.from_numpy(np.ascontiguousarray(a.astype(dt))).to(dev)
    kn = torch.from_numpy(np.ascontiguousarray(k_in).view(np.int16)).to(dev)
    vn = None if v_in is None else torch.from_numpy(np.ascontiguousarray(v_in).view(np.int16)).to(dev)
    kc = torch.from_numpy(np.ascontiguousarray(w.k_cache)).to(dev)
    vc = None if w.shared_kv else torch.from_numpy(np.ascontiguousarray(w.v_cache)).to(dev)
    from paged_kv_attention_gather_amd import _lib as L
    prob = problem_for(w)
    prob.q_dtype = L.DTYPE_BF16   # the new rows are bf16
    args_dev = (t(w.cu_seqlens_q, np.int32), t(w.seq_lens_kv, np.int32), t(w.block_table, np.int32),
                t(w.k_scale, np.float32), t(w.v_scale, np.float32))
    elems = int(w.total_q) * w.num_kv_heads * (w.head_dim_qk + (0 if w.shared_kv else w.head_dim_v))
    nbytes = elems * 3 + int(w.batch) * 4 * 2   # bf16 in, one byte out, lengths
    stream = torch.cuda.current_stream()
    flush = torch.ones(1 << 28, dtype=torch.int32, device=dev)

    def call():
        P.paged_kv_write(prob, int(w.total_q), kn, vn, args_dev[0], args_dev[1], args_dev[2], args_dev[3],
                         args_dev[4], kc, vc)

    for _ in range(args.warmup):
        flush.max()
        call()
    torch.cuda.synchronize()
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(2)] for _ in range(args.steps)]
    for i in range(args.steps):
        flush.max()
        ev[i][0].record(stream)
        call()
        ev[i][1].record(stream)
    torch.cuda.synchronize()
    ms = float(np.mean([e[0].elapsed_time(e[1]) for e in ev]))
    gbs = nbytes / (ms * 1e-3) / 1e9
    line = {"metric": "kv cache append write: HBM GB/s (bf16 rows in, quantized bytes scattered to pages)",
            "value": round(gbs, 2), "unit": "GB/s", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
            "ms_per_step": round(ms, 5), "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
            "dtype": w.kv_dtype, "data": "synthetic",
            "config": {"workload": WORKLOAD_TEXT[args.config] + " (its appended tokens)",
                       "tokens": int(w.total_q), "elements": elems, "bytes": nbytes},
            "roofline": {"bound": "hbm", "achieved": round(gbs, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                         "frac": round(gbs / HBM_PEAK_GBS, 4), "traffic": None,
                         "traffic_source": "no counters taken for the write kernel",
                         "kernel": "kv_write_kernel", "kernel_ms": round(ms, 5)}}
    print(json.dumps(line), flush=True)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--config", type=int, default=2, choices=[1, 2, 3, 4, 5])
    ap.add_argument("--chunk", type=int, default=None, help="override chunk_size")
    ap.add_argument("--no-flush", action="store_true", help="skip the per-step cache flush")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-budget", type=float, default=15.0)
    ap.add_argument("--kv-write", action="store_true",
                    help="time the cache append write (paged_kv_write) of the workload's appended "
                         "tokens instead of attention")
    ap.add_argument("--tree", action="store_true",
                    help="spec-decode workload (config 4) with a random draft tree per request, "
                         "through paged_attn_decode_tree")
    ap.add_argument("--merge", choices=["fused", "separate"], default="separate",
                    help="split-KV merge as split_kv_merge after the attention kernel (timed on its own, "
                         "the default) or through PA_FLAG_FUSED_MERGE")
    ap.add_argument("--balanced", action="store_true",
                    help="PA_FLAG_BALANCED_SPLIT: KV items sized on the device to fill one round "
                         "(chunk_size, or --chunk, is then the shortest item)")
    ap.add_argument("--persistent", action="store_true",
                    help="PA_FLAG_PERSISTENT: the decode kernel as one persistent launch with equal per-wave "
                         "shares (chunk_size is the shortest share) and the merge inside")
    ap.add_argument("--no-extra-configs", action="store_true",
                    help="with the default workload, skip timing the append, spec-decode and MLA workloads")
    ap.add_argument("--no-probe", action="store_true", help="skip the read probe of the decode workloads")
    ap.add_argument("--copy-probe-mib", type=int, default=0,
                    help="only run a plain device copy of this many MiB (counter calibration)")
    args = ap.parse_args()

    if args.copy_probe_mib:
        import torch
        n = args.copy_probe_mib << 20
        src = torch.ones(n, dtype=torch.uint8, device="cuda")
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_probe_bytes": n, "launches": 3}))
        return

    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus > 1 or world > 1:
        print("bench.py runs on one GPU: the paged attention path has no multi-GPU leg (sharding by request "
              "or by KV head needs no communication between GPUs).",
              file=sys.stderr)
        sys.exit(2)

    import torch
    from workloads import config_workload

    if args.kv_write:
        bench_kv_write(args)
        return
    if args.tree and args.config != 4:
        print("--tree applies to the spec-decode workload (--config 4)", file=sys.stderr)
        sys.exit(2)
    print(f"[bench] generating workload {args.config}", file=sys.stderr, flush=True)
    w = config_workload(args.config, tree=True) if args.tree else config_workload(args.config)
    fused = args.merge == "fused"
    if args.balanced and not fused:
        # a balanced split's chunks are not split_kv_merge's: the call merges
        # itself, so the step is timed whole (attention kernel + merge)
        print("[bench] --balanced: the merge runs inside the ABI call", file=sys.stderr, flush=True)
    flush = torch.ones(1 << 28, dtype=torch.int32, device="cuda")  # 1 GiB, read before every timed step
    m = measure(w, args.config, flush, args.steps, args.warmup, chunk=args.chunk, fused=fused,
                balanced=args.balanced, no_flush=args.no_flush, persistent=args.persistent)
    dp, chunk = m["dp"], m["chunk"]
    kv_bytes, alg_bytes, flops = work_figures(w)
    ms, attn_ms = m["step_ms"], m["attn_ms"]

    if args.config in (1, 3):
        value, unit = flops / (ms * 1e-3) / 1e12, "TFLOP/s"
    else:
        value, unit = kv_bytes / (ms * 1e-3) / 1e9, "GB/s"
    roof = roofline(args.config, w, attn_ms, ms)
    traffic, note = ((None, "no counters for the draft-tree kernels") if args.tree
                     else hbm_traffic(args.config, chunk, args.merge, args.balanced))
    roof["traffic"] = traffic
    if traffic is not None:
        roof["traffic_over_alg_bytes"] = round(traffic / alg_bytes, 4)
    roof["traffic_source"] = note
    roof["kernel"] = kernel_name(dp)
    roof["kernel_ms"] = round(attn_ms, 5)
    roof["kernel_min_ms"] = round(m["attn_min_ms"], 5)
    roof["merge_ms"] = round(m["merge_ms"], 5)
    roof["merge"] = (("in-kernel (PA_FLAG_FUSED_MERGE)" if fused else
                      "in-kernel, last wave of each (request, head) (PA_FLAG_PERSISTENT)" if args.persistent else
                      "split_kv_merge launch" + (" inside the call (kernel_ms includes it)" if args.balanced else ""))
                     if chunk > 0 else "none")
    roof["split"] = ("PA_FLAG_BALANCED_SPLIT requested (applied by the MLA kernel; the others keep fixed chunks)"
                     if args.balanced and chunk > 0 else
                     "persistent: equal per-wave tile shares of at least chunk_size keys" if args.persistent and chunk > 0
                     else "fixed chunks")
    roof["alg_bytes_per_launch"] = alg_bytes
    roof["flops_per_launch"] = flops
    if not args.no_probe and args.config in (2, 4) and not args.tree:
        pr = read_probe(dp, flush, args.steps, args.warmup, args.no_flush)
        roof["probe_gbs"] = round(kv_bytes / (pr * 1e-3) / 1e9, 1)
        roof["probe_ms"] = round(pr, 5)
        roof["probe_frac"] = round(roof["probe_gbs"] / HBM_PEAK_GBS, 4)
        roof["kernel_over_probe"] = round(pr / attn_ms, 4)
        roof["probe"] = ("pa_kv_read_probe: the decode kernel's tile loader over the same units and KV bytes, "
                         "no arithmetic (read ceiling of this access pattern)")

    line = {
        "metric": "decode: KV GB/s & %HBM peak; append: attention TFLOP/s & %MFMA peak",
        "value": round(value, 3), "unit": unit, "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(ms, 5), "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": compute_dtype(dp),
        "data": "synthetic",
        "config": {"workload": WORKLOAD_TEXT[args.config] + (" + random draft tree" if args.tree else ""),
                   "global_batch": int(w.batch),
                   "kv_dtype": w.kv_dtype, "chunk_size": int(chunk), "cache_flush": not args.no_flush,
                   "kv_bytes": kv_bytes, "alg_bytes": alg_bytes, "flops": flops,
                   "min_ms": round(m["step_min_ms"], 5),
                   "wall_ms_per_step_incl_flush": round(m["wall_ms"], 4)},
        "roofline": roof,
    }
    del m, dp
    if not args.no_extra_configs and args.config == 2 and not args.tree and not fused and not args.balanced \
            and not args.persistent and args.chunk is None:
        line["configs"] = other_configs(flush, args)
    if not args.no_cpu_baseline:
        print("[bench] cpu baseline (oracle)", file=sys.stderr, flush=True)
        line["cpu_baseline"] = cpu_baseline(args.config, args.cpu_budget)
    print(json.dumps(line), flush=True)


def measure(w, config, flush, steps, warmup, chunk=None, fused=False, balanced=False, no_flush=False,
            persistent=False):
    """Time `steps` calls of the workload after `warmup` untimed ones, twice on
    the launch stream (torch's current stream, which the binding passes to the
    library).  The step pass brackets each call with one event pair, [flush]
    e0 attention [merge] e2, so nothing is recorded between the two launches
    (an event there costs 2-5 us on this stack).  The breakdown pass records
    e0 attention e1 [merge e2] for the kernel and merge times."""
    import torch
    from paged_kv_attention_gather_amd.harness import DeviceProblem
    one_call = fused or balanced or persistent   # the call merges by itself
    dp = DeviceProblem(w, chunk_size=chunk, defer_merge=not one_call, fused_merge=fused, balanced=balanced,
                       persistent=persistent)
    chunk = dp.prob.chunk_size
    stream = torch.cuda.current_stream()
    separate = not one_call and chunk > 0   # a merge launched here, timed apart
    print(f"[bench] {w.name}: warmup {warmup}", file=sys.stderr, flush=True)
    for _ in range(warmup):
        if not no_flush:
            flush.max()   # read-only pass over 1 GiB
        dp.run()
        if separate:
            dp.merge()
    torch.cuda.synchronize()

    def timed(breakdown):
        ev = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(steps)]
        for i in range(steps):
            if not no_flush:
                flush.max()
            ev[i][0].record(stream)
            dp.run()
            if breakdown:
                ev[i][1].record(stream)
            if separate:
                dp.merge()
            if separate or not breakdown:
                ev[i][2].record(stream)
        torch.cuda.synchronize()
        return ev

    t_wall0 = time.perf_counter()
    ev = timed(False)
    t_wall = time.perf_counter() - t_wall0
    step = [e[0].elapsed_time(e[2]) for e in ev]
    ev = timed(True)
    attn = [e[0].elapsed_time(e[1]) for e in ev]
    merge = [e[1].elapsed_time(e[2]) for e in ev] if separate else [0.0]
    print(f"[bench] {w.name}: step {np.mean(step) * 1e3:.1f} us, attention {np.mean(attn) * 1e3:.1f} us",
          file=sys.stderr, flush=True)
    return {"dp": dp, "chunk": int(chunk), "step_ms": float(np.mean(step)), "step_min_ms": float(np.min(step)),
            "attn_ms": float(np.mean(attn)), "attn_min_ms": float(np.min(attn)), "merge_ms": float(np.mean(merge)),
            "wall_ms": t_wall / steps * 1e3}


def roofline(config, w, attn_ms, step_ms):
    """Roofline of the dominant (attention) kernel: algorithmic bytes (decode)
    or flops (append, MLA) per launch over its event time; the same over the
    whole step (attention + split-KV merge) as step_achieved / step_frac."""
    _, alg_bytes, flops = work_figures(w)
    if config in (3, 5):
        a, st = flops / (attn_ms * 1e-3) / 1e12, flops / (step_ms * 1e-3) / 1e12
        r = {"bound": "mfma", "achieved": round(a, 3), "peak": MFMA_F16_PEAK_TFS, "unit": "TFLOP/s",
             "frac": round(a / MFMA_F16_PEAK_TFS, 4), "step_achieved": round(st, 3),
             "step_frac": round(st / MFMA_F16_PEAK_TFS, 4)}
        if config == 5 and w.kv_dtype == "fp8_e4m3":
            # QK^T runs on the fp8 MFMA (5.0 PFLOP/s dense) once per query digit
            r["peak_basis"] = ("QK^T: fp8 MFMA over 2 query digits = 2.5 PFLOP/s per algorithmic flop; "
                               "PV: f16 MFMA 2.5 PFLOP/s")
        return r
    a, st = alg_bytes / (attn_ms * 1e-3) / 1e9, alg_bytes / (step_ms * 1e-3) / 1e9
    return {"bound": "hbm", "achieved": round(a, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
            "frac": round(a / HBM_PEAK_GBS, 4), "step_achieved": round(st, 1), "step_frac": round(st / HBM_PEAK_GBS, 4)}


def read_probe(dp, flush, steps, warmup, no_flush=False):
    """Mean event time (ms) of pa_kv_read_probe over the problem's units,
    flushed like the attention steps."""
    import torch
    import paged_kv_attention_gather_amd as P
    w = dp.w
    C = int(dp.prob.chunk_size)
    mc = max(1, -(-(int(dp.prob.max_kv_len) + int(dp.prob.max_q_len)) // C)) if C > 0 else 1
    sink = torch.zeros(mc * w.batch * w.num_kv_heads, dtype=torch.int32, device="cuda")
    stream = torch.cuda.current_stream()

    def call():
        P.pa_kv_read_probe(dp.prob, int(w.decode_q_len), dp.k_cache, dp.v_cache, dp.seq_lens_kv, dp.block_table,
                           sink)

    for _ in range(warmup):
        if not no_flush:
            flush.max()
        call()
    torch.cuda.synchronize()
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(2)] for _ in range(steps)]
    for i in range(steps):
        if not no_flush:
            flush.max()
        ev[i][0].record(stream)
        call()
        ev[i][1].record(stream)
    torch.cuda.synchronize()
    return float(np.mean([e[0].elapsed_time(e[1]) for e in ev]))


def other_configs(flush, args):
    """The append, spec-decode and MLA workloads measured in the same run with
    the same flush and events (fewer steps): kernel and step times, roofline
    fractions, and the HBM traffic ratio where committed counters cover the
    kernel sources."""
    import torch
    from workloads import config_workload
    out = {}
    for idx in (3, 4, 5):
        print(f"[bench] generating workload {idx}", file=sys.stderr, flush=True)
        w = config_workload(idx)
        m = measure(w, idx, flush, max(5, args.steps // 2), max(2, args.warmup), no_flush=args.no_flush)
        kv_bytes, alg_bytes, flops = work_figures(w)
        r = roofline(idx, w, m["attn_ms"], m["step_ms"])
        row = {"workload": WORKLOAD_TEXT[idx], "kernel": kernel_name(m["dp"]), "dtype": compute_dtype(m["dp"]),
               "chunk_size": m["chunk"], "kernel_ms": round(m["attn_ms"], 5), "merge_ms": round(m["merge_ms"], 5),
               "step_ms": round(m["step_ms"], 5), "kv_gbs": round(kv_bytes / (m["step_ms"] * 1e-3) / 1e9, 1),
               "flops": flops, "alg_bytes": alg_bytes, "roofline": r}
        if idx in (3, 5):
            row["tflops"] = round(flops / (m["step_ms"] * 1e-3) / 1e12, 3)
        traffic, note = hbm_traffic(idx, m["chunk"], "separate")
        row["traffic_over_alg_bytes"] = round(traffic / alg_bytes, 4) if traffic else None
        row["traffic_source"] = note
        if idx == 4 and not args.no_probe:
            pr = read_probe(m["dp"], flush, max(5, args.steps // 2), 2, args.no_flush)
            row["probe_gbs"] = round(kv_bytes / (pr * 1e-3) / 1e9, 1)
        out[str(idx)] = row
        del m
        torch.cuda.synchronize()
        torch.cuda.empty_cache()
    return out


if __name__ == "__main__":
    main()
