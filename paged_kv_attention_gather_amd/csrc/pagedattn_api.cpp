// C-ABI front end of libpagedattn.so: argument validation, specialization
// choice, grid and workspace sizing, then launches on the caller's stream.
// Every check runs before the first launch, so a failing call enqueues nothing.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <atomic>
#include <cmath>
#include <cstdarg>
#include <cstdint>
#include <cstdio>
#include <string>

#include "pa_internal.h"
#include "pagedattn.h"

namespace {

thread_local std::string g_last_error;

int32_t fail(int32_t status, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof(buf), fmt, ap);
  va_end(ap);
  g_last_error = buf;
  return status;
}

int32_t ok() {
  g_last_error.clear();
  return PA_OK;
}

int log2_exact(int64_t x) {
  if (x <= 0 || (x & (x - 1)) != 0) return -1;
  int s = 0;
  while ((int64_t(1) << s) < x) ++s;
  return s;
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }

constexpr int kTileKeys = 64;

// Shape checks shared by the workspace query and the attention calls.
int32_t check_problem(const pa_problem* p) {
  if (!p) return fail(PA_ERR_INVALID_ARG, "problem is NULL");
  if (p->batch < 0) return fail(PA_ERR_INVALID_ARG, "batch %d < 0", p->batch);
  if (p->batch > 65535) return fail(PA_ERR_UNSUPPORTED, "batch %d > 65535", p->batch);
  if (p->num_q_heads <= 0 || p->num_kv_heads <= 0)
    return fail(PA_ERR_INVALID_ARG, "head counts must be positive (H_q=%d, H_kv=%d)",
                p->num_q_heads, p->num_kv_heads);
  if (p->num_q_heads % p->num_kv_heads != 0)
    return fail(PA_ERR_INVALID_ARG, "H_q=%d is not a multiple of H_kv=%d", p->num_q_heads,
                p->num_kv_heads);
  if (p->num_kv_heads > 65535) return fail(PA_ERR_UNSUPPORTED, "H_kv %d > 65535", p->num_kv_heads);
  const bool dims_ok = (p->head_dim_qk == 64 && p->head_dim_v == 64) ||
                       (p->head_dim_qk == 128 && p->head_dim_v == 128) ||
                       (p->head_dim_qk == 576 && p->head_dim_v == 512);
  if (p->head_dim_qk <= 0 || p->head_dim_v <= 0)
    return fail(PA_ERR_INVALID_ARG, "head dims must be positive");
  if (!dims_ok)
    return fail(PA_ERR_UNSUPPORTED, "head dims (%d, %d) not compiled; supported: (64,64), (128,128), (576,512)",
                p->head_dim_qk, p->head_dim_v);
  if (log2_exact(p->page_size) < 0 || p->page_size < 16 || p->page_size > 1024)
    return fail(PA_ERR_UNSUPPORTED, "page_size %d must be a power of two in [16, 1024]", p->page_size);
  if (p->flags & ~(PA_FLAG_DEFER_MERGE | PA_FLAG_FUSED_MERGE | PA_FLAG_BALANCED_SPLIT | PA_FLAG_PERSISTENT))
    return fail(PA_ERR_INVALID_ARG, "unknown flag bits 0x%x", p->flags);
  if ((p->flags & PA_FLAG_PERSISTENT) && (p->flags & (PA_FLAG_DEFER_MERGE | PA_FLAG_BALANCED_SPLIT)))
    return fail(PA_ERR_INVALID_ARG,
                "PA_FLAG_PERSISTENT merges in the launch and plans its own split: not with PA_FLAG_DEFER_MERGE or "
                "PA_FLAG_BALANCED_SPLIT");
  if ((p->flags & PA_FLAG_DEFER_MERGE) && (p->flags & PA_FLAG_BALANCED_SPLIT))
    return fail(PA_ERR_INVALID_ARG,
                "PA_FLAG_BALANCED_SPLIT cuts chunks split_kv_merge cannot derive: not with PA_FLAG_DEFER_MERGE");
  if ((p->flags & PA_FLAG_DEFER_MERGE) && (p->flags & PA_FLAG_FUSED_MERGE))
    return fail(PA_ERR_INVALID_ARG, "PA_FLAG_DEFER_MERGE and PA_FLAG_FUSED_MERGE exclude each other");
  if (p->num_pages <= 0 || p->max_pages_per_seq <= 0)
    return fail(PA_ERR_INVALID_ARG, "num_pages and max_pages_per_seq must be positive");
  if (p->max_q_len < 0 || p->max_kv_len < 0)
    return fail(PA_ERR_INVALID_ARG, "max_q_len / max_kv_len must be >= 0");
  if (p->chunk_size < 0 || p->chunk_size % kTileKeys != 0)
    return fail(PA_ERR_UNSUPPORTED, "chunk_size %d must be 0 or a positive multiple of %d",
                p->chunk_size, kTileKeys);
  if (p->decode_waves != 0 && p->decode_waves != 1 && p->decode_waves != 2 && p->decode_waves != 4)
    return fail(PA_ERR_INVALID_ARG, "decode_waves %d: 0 (automatic), 1, 2 or 4", p->decode_waves);
  if (p->group_order < 0 || p->group_order > 2)
    return fail(PA_ERR_INVALID_ARG, "group_order %d: 0 (automatic), 1 or 2", p->group_order);
  if (p->merge_in_kernel < 0 || p->merge_in_kernel > 2)
    return fail(PA_ERR_INVALID_ARG, "merge_in_kernel %d: 0 (automatic), 1 or 2", p->merge_in_kernel);
  return PA_OK;
}

// Compute units of a device, asked once per device and kept (0: unknown).
int device_cus(int dev) {
  constexpr int kMaxDevices = 64;
  static std::atomic<int> cache[kMaxDevices];
  if (dev < 0 || dev >= kMaxDevices) return 0;
  int v = cache[dev].load(std::memory_order_relaxed);
  if (v == 0) {
    if (hipDeviceGetAttribute(&v, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || v <= 0) return 0;
    cache[dev].store(v, std::memory_order_relaxed);
  }
  return v;
}

// Resident workgroups of the whole device for the kernel `cfg` selects (0: unknown).
int64_t device_capacity(const pa::AttnConfig& cfg) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return 0;
  const int per_cu = pa::resident_per_cu(cfg, dev);
  const int cus = device_cus(dev);
  return (int64_t)per_cu * cus;
}

int64_t max_chunks_of(const pa_problem* p) {
  if (p->chunk_size <= 0) return 1;
  const int64_t c = std::max<int64_t>(1, ceil_div((int64_t)p->max_kv_len + p->max_q_len, p->chunk_size));
  // the persistent split cuts a range into at most one piece more than
  // fixed chunks would (its shares are at least chunk_size keys long)
  return (p->flags & PA_FLAG_PERSISTENT) ? c + 1 : c;
}

// Waves that split one unit's key range in the register-staged decode kernel.
// Units are (request, KV head, row tile, chunk).  Each wave of a unit pays
// the unit's start-up latency (lengths, page ids, first tile), so a unit is
// split only when the units cannot fill the 2048 (NT = 1) or 1024 (NT = 2)
// resident waves, and while every wave keeps at least four tiles.
// pa_problem.decode_waves (1, 2 or 4) fixes the choice instead.
int decode_split_waves(const pa_problem* p, int nt) {
  if (p->decode_waves != 0) return p->decode_waves;
  const int64_t keys = p->chunk_size > 0 ? p->chunk_size : (int64_t)p->max_kv_len + p->max_q_len;
  const int64_t tiles = ceil_div(keys, 64);
  const int64_t units = (int64_t)p->batch * p->num_kv_heads * max_chunks_of(p);
  const int64_t slots = nt == 1 ? 2048 : 1024;
  int ks = 1;
  while (ks < 4 && tiles >= 8 * ks && units * ks * 2 <= slots) ks *= 2;
  return ks;
}

// 16-row groups of one (request, KV head): the stride of the merge counters.
int64_t count_stride_of(const pa_problem* p) {
  return std::max<int64_t>(1, ceil_div((int64_t)p->max_q_len * (p->num_q_heads / p->num_kv_heads), 16));
}

// PA_FLAG_BALANCED_SPLIT reserves 256 bytes first (the chosen item length,
// read by the merge).  With PA_FLAG_FUSED_MERGE the merge counters come next,
// so their place and size depend only on batch, the head counts, max_q_len and
// the flags (not on total_q): a workspace zeroed once stays valid for every
// call with those.
struct WorkspaceLayout {
  size_t plan_bytes, count_offset, count_bytes, part_o_offset, part_o_bytes, part_lse_offset, part_lse_bytes,
      total;
};

WorkspaceLayout workspace_layout(const pa_problem* p, int64_t total_q) {
  WorkspaceLayout w{0, 0, 0, 0, 0, 0, 0, 0};
  if (p->chunk_size <= 0) return w;
  const int64_t mc = max_chunks_of(p);
  if (p->flags & PA_FLAG_BALANCED_SPLIT) w.plan_bytes = 256;
  w.count_offset = w.plan_bytes;
  if (p->flags & (PA_FLAG_FUSED_MERGE | PA_FLAG_PERSISTENT))
    w.count_bytes = (size_t)p->batch * p->num_kv_heads * count_stride_of(p) * sizeof(int32_t);
  w.part_o_offset = (w.count_offset + w.count_bytes + 255) & ~size_t(255);
  w.part_o_bytes = (size_t)total_q * mc * p->num_q_heads * p->head_dim_v * sizeof(float);
  w.part_lse_offset = (w.part_o_offset + w.part_o_bytes + 255) & ~size_t(255);
  w.part_lse_bytes = (size_t)total_q * mc * p->num_q_heads * sizeof(float);
  w.total = w.part_lse_offset + w.part_lse_bytes;
  return w;
}

// Draft trees (tree_mask != null, decode only) are checked by the caller.
int32_t attention_common(const pa_problem* p, bool decode, int32_t q_len, int64_t total_q,
                         const void* q, const void* k_cache, const void* v_cache,
                         const float* k_scale, const float* v_scale, const int32_t* cu_seqlens_q,
                         const int32_t* seq_lens_kv, const int32_t* block_table, void* out,
                         float* lse, void* workspace, size_t workspace_bytes, void* stream,
                         const uint8_t* tree_mask = nullptr, int32_t tree_mask_len = 0,
                         bool clear_counters = false) {
  int32_t st = check_problem(p);
  if (st != PA_OK) return st;
  if (decode) {
    if (q_len < 1 || q_len > 64) return fail(PA_ERR_INVALID_ARG, "decode q_len %d not in [1, 64]", q_len);
    if (p->max_q_len < q_len)
      return fail(PA_ERR_INVALID_ARG, "max_q_len %d < q_len %d", p->max_q_len, q_len);
  } else {
    if (total_q < 0) return fail(PA_ERR_INVALID_ARG, "total_q %lld < 0", (long long)total_q);
    if (p->batch > 0 && !cu_seqlens_q) return fail(PA_ERR_INVALID_ARG, "cu_seqlens_q is NULL");
  }
  if (p->batch == 0 || total_q == 0 || p->max_q_len == 0) return ok();  // nothing to compute
  if (!q || !k_cache || !v_cache || !k_scale || !v_scale || !seq_lens_kv || !block_table || !out)
    return fail(PA_ERR_INVALID_ARG, "a required device pointer is NULL");
  if (p->q_dtype != PA_DTYPE_BF16 && p->q_dtype != PA_DTYPE_F32)
    return fail(PA_ERR_UNSUPPORTED, "q_dtype %d: only BF16 and F32 queries", p->q_dtype);
  if (p->kv_dtype != PA_DTYPE_I8 && p->kv_dtype != PA_DTYPE_FP8_E4M3)
    return fail(PA_ERR_UNSUPPORTED, "kv_dtype %d: only I8 and FP8_E4M3 caches", p->kv_dtype);
  if (p->scale_mode < PA_SCALE_PER_TENSOR || p->scale_mode > PA_SCALE_PER_CHANNEL)
    return fail(PA_ERR_INVALID_ARG, "scale_mode %d", p->scale_mode);
  if (p->causal != 0 && p->causal != 1) return fail(PA_ERR_INVALID_ARG, "causal must be 0 or 1");
  if (!(p->sm_scale > 0.f) || !std::isfinite(p->sm_scale))
    return fail(PA_ERR_INVALID_ARG, "sm_scale must be finite and > 0");
  const int esize = p->q_dtype == PA_DTYPE_F32 ? 4 : 2;
  if (p->q_row_stride < (int64_t)p->num_q_heads * p->head_dim_qk)
    return fail(PA_ERR_INVALID_ARG, "q_row_stride %lld < H_q * D_qk", (long long)p->q_row_stride);
  if ((p->q_row_stride * esize) % 16 != 0 || !aligned16(q))
    return fail(PA_ERR_INVALID_ARG, "q and its row stride must be 16-byte aligned");
  const int64_t ks[3] = {p->k_stride_page, p->k_stride_head, p->k_stride_token};
  const int64_t vs[3] = {p->v_stride_page, p->v_stride_head, p->v_stride_token};
  for (int i = 0; i < 3; ++i) {
    if (ks[i] <= 0 || vs[i] <= 0) return fail(PA_ERR_INVALID_ARG, "cache strides must be positive");
    if (ks[i] % 16 != 0 || vs[i] % 16 != 0)
      return fail(PA_ERR_INVALID_ARG, "cache strides must be multiples of 16 bytes");
  }
  if (p->k_stride_token < p->head_dim_qk || p->v_stride_token < p->head_dim_v)
    return fail(PA_ERR_INVALID_ARG, "token stride shorter than the head dim");
  if (!aligned16(k_cache) || !aligned16(v_cache) || !aligned16(out))
    return fail(PA_ERR_INVALID_ARG, "k_cache, v_cache and out must be 16-byte aligned");
  const bool shared = p->head_dim_qk == 576;
  if (shared) {
    if (v_cache != k_cache || p->v_stride_page != p->k_stride_page ||
        p->v_stride_head != p->k_stride_head || p->v_stride_token != p->k_stride_token)
      return fail(PA_ERR_UNSUPPORTED,
                  "head dims (576, 512) need the shared latent layout: v_cache == k_cache, same strides");
  }
  const int64_t G = p->num_q_heads / p->num_kv_heads;
  const int64_t rows_max = (int64_t)(decode ? q_len : p->max_q_len) * G;
  if (tree_mask) {
    if (shared) return fail(PA_ERR_UNSUPPORTED, "draft-tree masks are not supported with the MLA layout");
    if (rows_max > 64)
      return fail(PA_ERR_UNSUPPORTED, "draft-tree masks need q_len * G <= 64 packed rows (got %lld)",
                  (long long)rows_max);
  }

  // The persistent decode kernel (PA_FLAG_PERSISTENT): decode problems of at
  // most 32 packed rows (one wave holds all of a request-head's rows).
  const bool persistent = (p->flags & PA_FLAG_PERSISTENT) && p->chunk_size > 0 && decode && !tree_mask &&
                          !shared && rows_max <= 32;
  pa::AttnConfig cfg{};
  cfg.tree = tree_mask != nullptr;
  cfg.dqk = p->head_dim_qk;
  cfg.dv = p->head_dim_v;
  cfg.fp8 = p->kv_dtype == PA_DTYPE_FP8_E4M3;
  cfg.shared_kv = shared;
  cfg.hilo = p->scale_mode == PA_SCALE_PER_CHANNEL || p->q_dtype == PA_DTYPE_F32;
  if (shared) {
    cfg.nt = 1;
    cfg.nw = 4;
    cfg.nstage = 1;  // MLA kernels: 64 rows per workgroup
  } else if (rows_max <= 32) {
    // register-staged decode kernel
    cfg.nt = (int)ceil_div(rows_max, 16);
    cfg.nw = cfg.tree ? 1 : decode_split_waves(p, cfg.nt);
    cfg.nstage = 0;
  } else if (rows_max <= 64) {
    // shared-tile kernel, 16 rows per wave, 3 or 4 waves sharing LDS-DMA tiles
    cfg.nt = 1;
    cfg.nw = (int)ceil_div(rows_max, 16);
    cfg.nstage = 2;
  } else {
    cfg.nt = 2;
    cfg.nw = 4;
    cfg.f16_tiles = cfg.dqk == 128;
    cfg.nstage = cfg.f16_tiles ? 3 : 2;
  }
  if (persistent) {
    cfg.nw = 1;
    cfg.nstage = 4;
  }
  if (!pa::attention_supported(cfg))
    return fail(PA_ERR_UNSUPPORTED, "no compiled kernel for this configuration");
  if (persistent &&
      ceil_div((int64_t)p->max_kv_len + p->max_q_len, kTileKeys) * p->num_kv_heads * p->batch > 0x7fffffffLL)
    return fail(PA_ERR_UNSUPPORTED, "PA_FLAG_PERSISTENT: more than 2^31 - 1 tiles in the call");
  const int64_t rows_per_wg = 16LL * cfg.nt * (cfg.nstage == 0 || cfg.nstage == 4 ? 1 : cfg.nw);  // decode: nw splits keys
  const int64_t row_tiles = ceil_div(rows_max, rows_per_wg);
  const int64_t max_chunks = max_chunks_of(p);
  if (row_tiles > 65535 || max_chunks > 65535 ||
      (int64_t)p->batch * p->num_kv_heads * row_tiles * max_chunks > 0x7ffffff0LL)
    return fail(PA_ERR_UNSUPPORTED, "grid too large (%lld row tiles, %lld chunks, %lld request-heads)",
                (long long)row_tiles, (long long)max_chunks,
                (long long)p->batch * p->num_kv_heads);

  const WorkspaceLayout wl = workspace_layout(p, total_q);
  if (wl.total > 0) {
    if (!workspace) return fail(PA_ERR_WORKSPACE_TOO_SMALL, "split-KV needs a workspace of %zu bytes", wl.total);
    if (workspace_bytes < wl.total)
      return fail(PA_ERR_WORKSPACE_TOO_SMALL, "workspace %zu bytes < %zu needed", workspace_bytes, wl.total);
    if (!aligned16(workspace)) return fail(PA_ERR_INVALID_ARG, "workspace must be 16-byte aligned");
  }

  pa::AttnParams ap{};
  ap.q = q;
  ap.k_cache = static_cast<const uint8_t*>(k_cache);
  ap.v_cache = static_cast<const uint8_t*>(v_cache);
  ap.k_scale = k_scale;
  ap.v_scale = v_scale;
  ap.cu_seqlens_q = decode ? nullptr : cu_seqlens_q;
  ap.seq_lens_kv = seq_lens_kv;
  ap.block_table = block_table;
  ap.tree_mask = tree_mask;
  ap.tree_mask_len = tree_mask_len;
  ap.out = static_cast<uint16_t*>(out);
  ap.lse = lse;
  ap.part_o = wl.total ? reinterpret_cast<float*>(static_cast<char*>(workspace) + wl.part_o_offset) : nullptr;
  ap.part_lse = wl.total ? reinterpret_cast<float*>(static_cast<char*>(workspace) + wl.part_lse_offset) : nullptr;
  // In-kernel merge (PA_FLAG_FUSED_MERGE) where the workgroup that finishes a
  // row tile last covers the tile's merge in one pass of two four-channel
  // slots per thread (a few rows, as in decode).  A wider tile (the 16-row
  // shared-tile and MLA kernels: 40 to 128 rows of 128 to 512 channels) would
  // be merged by that one workgroup, round trip after round trip, while
  // split_kv_merge spreads the same work over the chip: measured 364 vs 265 us
  // on the spec-decode workload and 272 vs 199 us on MLA.  Those paths
  // enqueue split_kv_merge as without the flag (same results).
  // pa_problem.merge_in_kernel (1 = always, 2 = never) fixes the choice within
  // the decode kernel, the one that compiles the merge tail (in the
  // shared-tile and MLA kernels it cost SGPR spills in the main loop, and
  // the host never picks the in-kernel merge for their wide tiles).
  bool fused = wl.count_bytes > 0 && !persistent;
  if (fused) {
    const int64_t unit_rows = std::min<int64_t>(rows_max, 16LL * cfg.nt * (cfg.nstage == 0 ? 1 : cfg.nw));
    const int64_t merge_threads = 64LL * (cfg.nstage == 0 ? 1 : cfg.nw);   // decode: wave 0 merges
    fused = unit_rows * (p->head_dim_v / 4) <= 2 * merge_threads;
    if (p->merge_in_kernel != 0) fused = p->merge_in_kernel == 1;
    fused = fused && cfg.nstage == 0;
  }
  ap.merge_count = fused || persistent ? reinterpret_cast<int32_t*>(static_cast<char*>(workspace) + wl.count_offset)
                                       : nullptr;
  ap.count_stride = (int32_t)count_stride_of(p);
  ap.q_row_stride = p->q_row_stride;
  ap.k_stride_page = p->k_stride_page;
  ap.k_stride_head = p->k_stride_head;
  ap.k_stride_token = p->k_stride_token;
  ap.v_stride_page = p->v_stride_page;
  ap.v_stride_head = p->v_stride_head;
  ap.v_stride_token = p->v_stride_token;
  ap.num_q_heads = p->num_q_heads;
  ap.num_kv_heads = p->num_kv_heads;
  ap.group = (int32_t)G;
  ap.page_shift = log2_exact(p->page_size);
  ap.max_pages_per_seq = p->max_pages_per_seq;
  ap.q_len_uniform = decode ? q_len : 0;
  ap.chunk_size = p->chunk_size;
  ap.max_chunks = (int32_t)max_chunks;
  ap.row_tiles = (int32_t)row_tiles;
  ap.q_is_f32 = p->q_dtype == PA_DTYPE_F32;
  ap.scale_mode = p->scale_mode;
  ap.causal = p->causal;
  ap.qk_mult = p->sm_scale * 1.4426950408889634f;

  hipStream_t s = static_cast<hipStream_t>(stream);
  // The single-wave decode kernel runs chunk-major (empty chunks of short
  // requests dispatch last); the shared-tile kernel keeps one request-head's
  // row tiles adjacent.
  const bool decode_kernel = cfg.nstage == 0;
  // shared-tile kernels: ceil(groups / 8) rounds of 8 groups x row_tiles workgroups
  const int64_t groups = (int64_t)p->batch * p->num_kv_heads * max_chunks;
  ap.batch = p->batch;
  dim3 grid = decode_kernel
                  ? dim3((unsigned)(p->batch * p->num_kv_heads), (unsigned)row_tiles, (unsigned)max_chunks)
                  : dim3((unsigned)(ceil_div(groups, 8) * 8 * row_tiles), 1, 1);
  // Number only the groups with work when the whole grid is at most two rounds
  // of resident workgroups (then an XCD that drew more workgroups than it has
  // CUs would run a second, mostly idle round); deeper grids balance by dispatch.
  // pa_problem.group_order (1 = grid slots, 2 = compact) fixes the choice.
  // The device's capacity is asked once per device and kernel, then cached.
  const int64_t capacity = decode_kernel && !persistent ? 0 : device_capacity(cfg);
  if (persistent) {
    // one wave per workgroup, exactly the resident capacity
    if (capacity <= 0 || capacity > 0x7fffffffLL)
      return fail(PA_ERR_HIP, "PA_FLAG_PERSISTENT: the device's resident capacity could not be determined");
    grid = dim3((unsigned)capacity, 1, 1);
  }
  ap.compact_groups = 0;
  if (p->group_order != 0) {
    ap.compact_groups = p->group_order == 2;
  } else if (!decode_kernel) {
    ap.compact_groups = capacity > 0 && (int64_t)grid.x <= 2LL * capacity;
  }
  // Balanced split (PA_FLAG_BALANCED_SPLIT) in the MLA kernel, of which one
  // workgroup fits a CU: a round is coarse there, so items sized on the
  // device to fill one round replace fixed chunks whose ragged last chunks
  // leave CUs idle, and numbering only groups with work puts that round on
  // the XCDs.  On the MLA workload this makes the time independent of the
  // chunk floor (about 195 us for floors of 1024 to 3072 keys; fixed chunks
  // of 1024 keys take 313 us).  The other kernels keep fixed chunks: the
  // dispatcher balances their many short units (one round of long items
  // measured 2x slower on the spec-decode workload, 540 vs 271 us), and an
  // unchunked append is faster than either split (187 us; balanced 219 us,
  // fixed 1024-key chunks 246 us).
  if ((p->flags & PA_FLAG_BALANCED_SPLIT) && p->chunk_size > 0 && cfg.nstage == 1 && capacity > 0) {
    ap.balanced = 1;
    ap.group_cap = (int32_t)std::max<int64_t>(1, capacity / row_tiles);
    ap.plan_out = static_cast<int32_t*>(workspace);
    if (p->group_order == 0) ap.compact_groups = 1;
  }
  if (clear_counters && wl.count_bytes > 0) {
    // a workspace shared across calls (the static scratch): the merge
    // counters must start at zero whatever the last call left there
    hipError_t ez = pa::launch_zero_words(reinterpret_cast<int32_t*>(static_cast<char*>(workspace) + wl.count_offset),
                                          (int64_t)(wl.count_bytes / sizeof(int32_t)), s);
    if (ez != hipSuccess) return fail(PA_ERR_HIP, "counter clear launch failed: %s", hipGetErrorString(ez));
  }
  hipError_t e = pa::launch_attention(cfg, ap, grid, s);
  if (e != hipSuccess) return fail(PA_ERR_HIP, "attention launch failed: %s", hipGetErrorString(e));
  if (p->chunk_size > 0 && !(p->flags & PA_FLAG_DEFER_MERGE) && !fused && !persistent) {
    pa::MergeParams mp{};
    mp.part_o = ap.part_o;
    mp.part_lse = ap.part_lse;
    mp.cu_seqlens_q = ap.cu_seqlens_q;
    mp.seq_lens_kv = seq_lens_kv;
    mp.out = ap.out;
    mp.lse = lse;
    mp.q_len_uniform = ap.q_len_uniform;
    mp.num_q_heads = p->num_q_heads;
    mp.chunk_size = p->chunk_size;
    mp.max_chunks = ap.max_chunks;
    mp.item_tiles = ap.balanced ? ap.plan_out : nullptr;
    e = pa::launch_merge(p->head_dim_v, mp, p->batch, p->max_q_len, s);
    if (e != hipSuccess) return fail(PA_ERR_HIP, "merge launch failed: %s", hipGetErrorString(e));
  }
  return ok();
}

}  // namespace

extern "C" {

size_t paged_attn_workspace_size(const pa_problem* prob, int32_t total_q) {
  if (check_problem(prob) != PA_OK || total_q < 0) return (size_t)-1;
  return workspace_layout(prob, total_q).total;
}

int32_t paged_attn_append(const pa_problem* prob, int32_t total_q, const void* q,
                          const void* k_cache, const void* v_cache, const float* k_scale,
                          const float* v_scale, const int32_t* cu_seqlens_q,
                          const int32_t* seq_lens_kv, const int32_t* block_table, void* out,
                          float* lse, void* workspace, size_t workspace_bytes, void* stream) {
  return attention_common(prob, false, 0, total_q, q, k_cache, v_cache, k_scale, v_scale,
                          cu_seqlens_q, seq_lens_kv, block_table, out, lse, workspace,
                          workspace_bytes, stream);
}

int32_t paged_attn_decode(const pa_problem* prob, int32_t q_len, const void* q,
                          const void* k_cache, const void* v_cache, const float* k_scale,
                          const float* v_scale, const int32_t* seq_lens_kv,
                          const int32_t* block_table, void* out, float* lse, void* workspace,
                          size_t workspace_bytes, void* stream) {
  if (!prob) return fail(PA_ERR_INVALID_ARG, "problem is NULL");
  const int64_t total_q = (int64_t)prob->batch * q_len;
  return attention_common(prob, true, q_len, total_q, q, k_cache, v_cache, k_scale, v_scale,
                          nullptr, seq_lens_kv, block_table, out, lse, workspace, workspace_bytes,
                          stream);
}

int32_t paged_attn_decode_scratch(const pa_problem* prob, int32_t q_len, const void* q,
                                  const void* k_cache, const void* v_cache, const float* k_scale,
                                  const float* v_scale, const int32_t* seq_lens_kv,
                                  const int32_t* block_table, void* out, float* lse, void* stream) {
  int32_t st = check_problem(prob);
  if (st != PA_OK) return st;
  if (prob->flags & PA_FLAG_DEFER_MERGE)
    return fail(PA_ERR_INVALID_ARG, "PA_FLAG_DEFER_MERGE: the static scratch's partials are not reachable by the caller");
  if (q_len < 1 || q_len > 64) return fail(PA_ERR_INVALID_ARG, "decode q_len %d not in [1, 64]", q_len);
  const int64_t total_q = (int64_t)prob->batch * q_len;
  const size_t need = workspace_layout(prob, total_q).total;
  if (need > PA_DECODE_SCRATCH_BYTES)
    return fail(PA_ERR_WORKSPACE_TOO_SMALL, "this problem needs %zu bytes of split-KV workspace; the static scratch holds %zu",
                need, (size_t)PA_DECODE_SCRATCH_BYTES);
  void* ws = nullptr;
  if (need > 0) {
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e == hipSuccess) ws = pa::decode_scratch(dev, &e);
    if (!ws) return fail(PA_ERR_HIP, "static scratch lookup failed: %s", hipGetErrorString(e));
  }
  return attention_common(prob, true, q_len, total_q, q, k_cache, v_cache, k_scale, v_scale, nullptr,
                          seq_lens_kv, block_table, out, lse, ws, ws ? (size_t)PA_DECODE_SCRATCH_BYTES : 0, stream,
                          nullptr, 0, /*clear_counters=*/true);
}

int32_t paged_attn_decode_tree(const pa_problem* prob, int32_t q_len, const void* q,
                               const void* k_cache, const void* v_cache, const float* k_scale,
                               const float* v_scale, const int32_t* seq_lens_kv,
                               const int32_t* block_table, const uint8_t* tree_mask,
                               int32_t tree_mask_len, void* out, float* lse, void* workspace,
                               size_t workspace_bytes, void* stream) {
  if (!prob) return fail(PA_ERR_INVALID_ARG, "problem is NULL");
  if (!tree_mask) return fail(PA_ERR_INVALID_ARG, "tree_mask is NULL");
  if (tree_mask_len < q_len || tree_mask_len > 64)
    return fail(PA_ERR_INVALID_ARG, "tree_mask_len %d must lie in [q_len = %d, 64]", tree_mask_len, q_len);
  const int64_t total_q = (int64_t)prob->batch * q_len;
  return attention_common(prob, true, q_len, total_q, q, k_cache, v_cache, k_scale, v_scale,
                          nullptr, seq_lens_kv, block_table, out, lse, workspace, workspace_bytes,
                          stream, tree_mask, tree_mask_len);
}

int32_t split_kv_merge(const float* partial_o, const float* partial_lse,
                       const int32_t* cu_seqlens_q, const int32_t* seq_lens_kv,
                       int32_t q_len_uniform, int32_t batch, int32_t total_q, int32_t max_q_len,
                       int32_t num_q_heads, int32_t head_dim_v, int32_t chunk_size,
                       int32_t max_chunks, void* out, float* lse, void* stream) {
  if (batch < 0 || batch > 65535 || total_q < 0 || max_q_len < 0 || num_q_heads <= 0)
    return fail(PA_ERR_INVALID_ARG, "bad sizes (batch=%d total_q=%d max_q_len=%d H_q=%d)", batch,
                total_q, max_q_len, num_q_heads);
  if (head_dim_v != 64 && head_dim_v != 128 && head_dim_v != 256 && head_dim_v != 512 &&
      head_dim_v != 1024)
    return fail(PA_ERR_UNSUPPORTED, "head_dim_v %d not in {64, 128, 256, 512, 1024}", head_dim_v);
  if (chunk_size <= 0 || max_chunks <= 0)
    return fail(PA_ERR_INVALID_ARG, "chunk_size and max_chunks must be positive");
  if (!cu_seqlens_q && q_len_uniform <= 0)
    return fail(PA_ERR_INVALID_ARG, "need cu_seqlens_q or q_len_uniform > 0");
  if (!cu_seqlens_q && q_len_uniform > max_q_len)
    return fail(PA_ERR_INVALID_ARG, "q_len_uniform %d > max_q_len %d", q_len_uniform, max_q_len);
  if (batch == 0 || total_q == 0 || max_q_len == 0) return ok();
  if (!partial_o || !partial_lse || !seq_lens_kv || !out)
    return fail(PA_ERR_INVALID_ARG, "a required device pointer is NULL");
  if (!aligned16(partial_o) || !aligned16(out))
    return fail(PA_ERR_INVALID_ARG, "partial_o and out must be 16-byte aligned");
  pa::MergeParams mp{};
  mp.part_o = partial_o;
  mp.part_lse = partial_lse;
  mp.cu_seqlens_q = cu_seqlens_q;
  mp.seq_lens_kv = seq_lens_kv;
  mp.out = static_cast<uint16_t*>(out);
  mp.lse = lse;
  mp.q_len_uniform = cu_seqlens_q ? 0 : q_len_uniform;
  mp.num_q_heads = num_q_heads;
  mp.chunk_size = chunk_size;
  mp.max_chunks = max_chunks;
  hipError_t e = pa::launch_merge(head_dim_v, mp, batch, max_q_len, static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return fail(PA_ERR_HIP, "merge launch failed: %s", hipGetErrorString(e));
  return ok();
}

int32_t pa_gather_debug(const pa_problem* prob, int32_t loader, const void* k_cache, const void* v_cache,
                        const int32_t* block_table, const int32_t* seq_lens_kv, const int32_t* q_lens,
                        int32_t t_max, uint8_t* k_dst, uint8_t* v_dst, void* stream) {
  int32_t st = check_problem(prob);
  if (st != PA_OK) return st;
  if (loader < PA_GATHER_ROWS || loader > PA_GATHER_DMA_MLA32)
    return fail(PA_ERR_INVALID_ARG, "loader %d: PA_GATHER_ROWS, _DECODE, _DMA_4W, _DMA_3W or _DMA_MLA32", loader);
  if (t_max < 0) return fail(PA_ERR_INVALID_ARG, "t_max %d < 0", t_max);
  if ((int64_t)t_max > (int64_t)prob->max_pages_per_seq * prob->page_size)
    return fail(PA_ERR_INVALID_ARG, "t_max %d exceeds the block table capacity", t_max);
  if (prob->batch == 0 || t_max == 0) return ok();
  if (!k_cache || !block_table || !seq_lens_kv || !q_lens || !k_dst || (v_dst && !v_cache))
    return fail(PA_ERR_INVALID_ARG, "a required device pointer is NULL");
  const int64_t ks[3] = {prob->k_stride_page, prob->k_stride_head, prob->k_stride_token};
  const int64_t vs[3] = {prob->v_stride_page, prob->v_stride_head, prob->v_stride_token};
  for (int i = 0; i < 3; ++i)
    if (ks[i] <= 0 || ks[i] % 16 || (v_dst && (vs[i] <= 0 || vs[i] % 16)))
      return fail(PA_ERR_INVALID_ARG, "cache strides must be positive multiples of 16 bytes");
  if (!aligned16(k_cache) || !aligned16(k_dst) || (v_dst && (!aligned16(v_cache) || !aligned16(v_dst))))
    return fail(PA_ERR_INVALID_ARG, "caches and destinations must be 16-byte aligned");
  const bool shared = prob->head_dim_qk == 576;
  if (shared && v_dst) return fail(PA_ERR_INVALID_ARG, "the shared latent layout has no separate V rows: v_dst must be NULL");
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (loader == PA_GATHER_ROWS) {
    pa::GatherParams gp{};
    gp.block_table = block_table;
    gp.seq_lens_kv = seq_lens_kv;
    gp.q_lens = q_lens;
    gp.page_shift = log2_exact(prob->page_size);
    gp.max_pages_per_seq = prob->max_pages_per_seq;
    gp.num_kv_heads = prob->num_kv_heads;
    gp.t_max = t_max;
    for (int pass = 0; pass < (v_dst ? 2 : 1); ++pass) {
      gp.k_cache = static_cast<const uint8_t*>(pass ? v_cache : k_cache);
      gp.dst = pass ? v_dst : k_dst;
      gp.k_stride_page = pass ? prob->v_stride_page : prob->k_stride_page;
      gp.k_stride_head = pass ? prob->v_stride_head : prob->k_stride_head;
      gp.k_stride_token = pass ? prob->v_stride_token : prob->k_stride_token;
      gp.head_dim = pass ? prob->head_dim_v : prob->head_dim_qk;
      hipError_t e = pa::launch_gather(gp, prob->batch, s);
      if (e != hipSuccess) return fail(PA_ERR_HIP, "gather launch failed: %s", hipGetErrorString(e));
    }
    return ok();
  }
  pa::TileWalkParams w{};
  w.a.k_cache = static_cast<const uint8_t*>(k_cache);
  w.a.v_cache = static_cast<const uint8_t*>(v_cache ? v_cache : k_cache);
  w.a.seq_lens_kv = seq_lens_kv;
  w.a.block_table = block_table;
  w.a.k_stride_page = prob->k_stride_page;
  w.a.k_stride_head = prob->k_stride_head;
  w.a.k_stride_token = prob->k_stride_token;
  w.a.v_stride_page = v_cache ? prob->v_stride_page : prob->k_stride_page;
  w.a.v_stride_head = v_cache ? prob->v_stride_head : prob->k_stride_head;
  w.a.v_stride_token = v_cache ? prob->v_stride_token : prob->k_stride_token;
  w.a.num_kv_heads = prob->num_kv_heads;
  w.a.page_shift = log2_exact(prob->page_size);
  w.a.max_pages_per_seq = prob->max_pages_per_seq;
  w.q_lens = q_lens;
  w.k_dst = k_dst;
  w.v_dst = v_dst;
  w.t_max = t_max;
  const int64_t whole = ceil_div((int64_t)t_max, kTileKeys) * kTileKeys;
  w.chunk = (int32_t)(prob->chunk_size > 0 ? prob->chunk_size : whole);
  const int64_t chunks = ceil_div((int64_t)t_max, w.chunk);
  if (chunks > 65535 || (int64_t)prob->batch * prob->num_kv_heads > 0x7fffffffLL)
    return fail(PA_ERR_UNSUPPORTED, "grid too large");
  hipError_t e = pa::launch_tile_gather(loader, prob->head_dim_qk, prob->head_dim_v, shared, w, prob->batch,
                                        prob->num_kv_heads, (int)chunks, s);
  if (e == hipErrorInvalidValue)
    return fail(PA_ERR_UNSUPPORTED, "loader %d has no instance for head dims (%d, %d)", loader, prob->head_dim_qk,
                prob->head_dim_v);
  if (e != hipSuccess) return fail(PA_ERR_HIP, "gather launch failed: %s", hipGetErrorString(e));
  return ok();
}

int32_t pa_kv_read_probe(const pa_problem* prob, int32_t q_len, const void* k_cache, const void* v_cache,
                         const int32_t* seq_lens_kv, const int32_t* block_table, uint32_t* sink,
                         void* stream) {
  int32_t st = check_problem(prob);
  if (st != PA_OK) return st;
  if (q_len < 1 || q_len > 64) return fail(PA_ERR_INVALID_ARG, "decode q_len %d not in [1, 64]", q_len);
  if (prob->max_q_len < q_len) return fail(PA_ERR_INVALID_ARG, "max_q_len %d < q_len %d", prob->max_q_len, q_len);
  if (prob->head_dim_qk != prob->head_dim_v || (prob->head_dim_qk != 64 && prob->head_dim_qk != 128))
    return fail(PA_ERR_UNSUPPORTED, "the read probe follows the decode kernel: head dims 64 or 128");
  if (prob->batch == 0) return ok();
  if (!k_cache || !v_cache || !seq_lens_kv || !block_table || !sink)
    return fail(PA_ERR_INVALID_ARG, "a required device pointer is NULL");
  if (!aligned16(k_cache) || !aligned16(v_cache))
    return fail(PA_ERR_INVALID_ARG, "caches must be 16-byte aligned");
  const int64_t ks[3] = {prob->k_stride_page, prob->k_stride_head, prob->k_stride_token};
  const int64_t vs[3] = {prob->v_stride_page, prob->v_stride_head, prob->v_stride_token};
  for (int i = 0; i < 3; ++i)
    if (ks[i] <= 0 || ks[i] % 16 || vs[i] <= 0 || vs[i] % 16)
      return fail(PA_ERR_INVALID_ARG, "cache strides must be positive multiples of 16 bytes");
  pa::TileWalkParams w{};
  w.a.k_cache = static_cast<const uint8_t*>(k_cache);
  w.a.v_cache = static_cast<const uint8_t*>(v_cache);
  w.a.seq_lens_kv = seq_lens_kv;
  w.a.block_table = block_table;
  w.a.k_stride_page = prob->k_stride_page;
  w.a.k_stride_head = prob->k_stride_head;
  w.a.k_stride_token = prob->k_stride_token;
  w.a.v_stride_page = prob->v_stride_page;
  w.a.v_stride_head = prob->v_stride_head;
  w.a.v_stride_token = prob->v_stride_token;
  w.a.num_kv_heads = prob->num_kv_heads;
  w.a.page_shift = log2_exact(prob->page_size);
  w.a.max_pages_per_seq = prob->max_pages_per_seq;
  w.a.q_len_uniform = q_len;
  w.sink = sink;
  const int64_t keys = (int64_t)prob->max_kv_len + q_len;
  w.chunk = (int32_t)(prob->chunk_size > 0 ? prob->chunk_size : ceil_div(keys, kTileKeys) * kTileKeys);
  const int64_t chunks = max_chunks_of(prob);
  if (chunks > 65535 || (int64_t)prob->batch * prob->num_kv_heads > 0x7fffffffLL)
    return fail(PA_ERR_UNSUPPORTED, "grid too large");
  hipError_t e = pa::launch_read_probe(prob->head_dim_qk, w, prob->batch, prob->num_kv_heads, (int)chunks,
                                       static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return fail(PA_ERR_HIP, "probe launch failed: %s", hipGetErrorString(e));
  return ok();
}

int32_t paged_kv_write(const pa_problem* prob, int32_t total_new, const void* k_new, const void* v_new,
                       const int32_t* cu_seqlens_new, const int32_t* seq_lens_kv,
                       const int32_t* block_table, const float* k_scale, const float* v_scale,
                       void* k_cache, void* v_cache, void* stream) {
  int32_t st = check_problem(prob);
  if (st != PA_OK) return st;
  if (total_new < 0) return fail(PA_ERR_INVALID_ARG, "total_new %d < 0", total_new);
  if (prob->batch == 0 || total_new == 0 || prob->max_q_len == 0) return ok();
  const bool shared = prob->head_dim_qk == 576;
  if (!k_new || !cu_seqlens_new || !seq_lens_kv || !block_table || !k_scale || !k_cache)
    return fail(PA_ERR_INVALID_ARG, "a required device pointer is NULL");
  if (shared) {
    if (v_new) return fail(PA_ERR_INVALID_ARG, "the shared latent layout writes K rows only: v_new must be NULL");
  } else if (!v_new || !v_scale || !v_cache) {
    return fail(PA_ERR_INVALID_ARG, "v_new, v_scale and v_cache are required");
  }
  if (prob->q_dtype != PA_DTYPE_BF16 && prob->q_dtype != PA_DTYPE_F32)
    return fail(PA_ERR_UNSUPPORTED, "q_dtype %d: new rows must be BF16 or F32", prob->q_dtype);
  if (prob->kv_dtype != PA_DTYPE_I8 && prob->kv_dtype != PA_DTYPE_FP8_E4M3)
    return fail(PA_ERR_UNSUPPORTED, "kv_dtype %d: only I8 and FP8_E4M3 caches", prob->kv_dtype);
  if (prob->scale_mode < PA_SCALE_PER_TENSOR || prob->scale_mode > PA_SCALE_PER_CHANNEL)
    return fail(PA_ERR_INVALID_ARG, "scale_mode %d", prob->scale_mode);
  if (!aligned16(k_new) || (v_new && !aligned16(v_new)) || !aligned16(k_cache) || (!shared && !aligned16(v_cache)))
    return fail(PA_ERR_INVALID_ARG, "k_new, v_new and the caches must be 16-byte aligned");
  const int64_t ks[3] = {prob->k_stride_page, prob->k_stride_head, prob->k_stride_token};
  const int64_t vs[3] = {prob->v_stride_page, prob->v_stride_head, prob->v_stride_token};
  for (int i = 0; i < 3; ++i)
    if (ks[i] <= 0 || ks[i] % 16 || (!shared && (vs[i] <= 0 || vs[i] % 16)))
      return fail(PA_ERR_INVALID_ARG, "cache strides must be positive multiples of 16 bytes");
  if (prob->k_stride_token < prob->head_dim_qk || (!shared && prob->v_stride_token < prob->head_dim_v))
    return fail(PA_ERR_INVALID_ARG, "token stride shorter than the head dim");

  pa::KvWriteParams kp{};
  kp.k_new = k_new;
  kp.v_new = shared ? nullptr : v_new;
  kp.cu_seqlens_new = cu_seqlens_new;
  kp.seq_lens_kv = seq_lens_kv;
  kp.block_table = block_table;
  kp.k_scale = k_scale;
  kp.v_scale = shared ? k_scale : v_scale;
  kp.k_cache = static_cast<uint8_t*>(k_cache);
  kp.v_cache = shared ? nullptr : static_cast<uint8_t*>(v_cache);
  kp.k_stride_page = prob->k_stride_page;
  kp.k_stride_head = prob->k_stride_head;
  kp.k_stride_token = prob->k_stride_token;
  kp.v_stride_page = prob->v_stride_page;
  kp.v_stride_head = prob->v_stride_head;
  kp.v_stride_token = prob->v_stride_token;
  kp.num_kv_heads = prob->num_kv_heads;
  kp.dk = prob->head_dim_qk;
  kp.dv = shared ? 0 : prob->head_dim_v;
  kp.page_shift = log2_exact(prob->page_size);
  kp.max_pages_per_seq = prob->max_pages_per_seq;
  kp.scale_mode = prob->scale_mode;
  // about one eight-channel item per thread, so every load of the launch is
  // in flight at once (four items per thread in sequence ran at 1.4 TB/s)
  const int per_tok = prob->num_kv_heads * (kp.dk + kp.dv) / 8;
  kp.tokens_per_block = std::max(1, 256 / std::max(1, per_tok));
  if ((int64_t)ceil_div(prob->max_q_len, kp.tokens_per_block) > 0x7fffffffLL)
    return fail(PA_ERR_UNSUPPORTED, "grid too large");
  hipError_t e = pa::launch_kv_write(kp, prob->kv_dtype == PA_DTYPE_FP8_E4M3, prob->q_dtype == PA_DTYPE_F32,
                                     prob->batch, prob->max_q_len, static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return fail(PA_ERR_HIP, "cache write launch failed: %s", hipGetErrorString(e));
  return ok();
}

const char* pa_status_string(int32_t status) {
  switch (status) {
    case PA_OK: return "PA_OK";
    case PA_ERR_INVALID_ARG: return "PA_ERR_INVALID_ARG";
    case PA_ERR_UNSUPPORTED: return "PA_ERR_UNSUPPORTED";
    case PA_ERR_WORKSPACE_TOO_SMALL: return "PA_ERR_WORKSPACE_TOO_SMALL";
    case PA_ERR_HIP: return "PA_ERR_HIP";
    default: return "PA_ERR_UNKNOWN";
  }
}

const char* pa_last_error(void) { return g_last_error.c_str(); }

}  // extern "C"
