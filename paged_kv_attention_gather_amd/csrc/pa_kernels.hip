// gfx950 (CDNA4) kernels for paged-KV append/decode attention.
//
// Work unit: (request b, KV head g, tile of GQA-packed query rows, KV chunk).
// Packed row r of a request is token r / G of head g*G + r % G (FastDeploy
// append_attention_c8_impl.cuh packs GROUP_SIZE heads per KV head the same way
// in its output write).  Each workgroup has NW waves; wave w owns 16*NT rows.
// KV is walked in 64-key tiles that all waves share:
//
//   HBM --(global_load_lds_dwordx4, 16 B per lane, page-table addressed)--> LDS
//   raw int8/fp8 rows, XOR-swizzled in 16-byte chunks so that the MFMA operand
//   reads below are free of bank conflicts.
//
//   S^T = K Q^T   v_mfma_f32_16x16x32_f16; A = K rows read with ds_read_b128 and
//                 converted to f16 in registers; B = Q^T held in registers with
//                 every scale and log2(e) folded in.
//   online softmax in the exp2 domain (XQA mla_sm120.cu folds qScale, the KV
//                 scale and log2e into one logit multiplier and uses exp2).
//   O^T += V^T P^T  A = V^T fetched with ds_read_b64_tr_b8 (the gfx950 LDS
//                 transpose read) straight from the token-major V rows, then
//                 converted; B = P^T, taken from the S^T accumulators without
//                 any data movement because the key order of each lane group
//                 is chosen to match the accumulator layout.
//
// int8 -> f16 and e4m3fn -> f16 are exact, so the MFMA sees the cache values
// exactly; all scales are applied in fp32 outside the MFMA (per-channel K
// scales multiply Q, V scales multiply the final O).
#include <hip/hip_runtime.h>

#include <algorithm>
#include <atomic>
#include <mutex>

#include "pa_internal.h"

namespace pa {
namespace {

typedef _Float16 half8_t __attribute__((ext_vector_type(8)));
typedef _Float16 half2_t __attribute__((ext_vector_type(2)));
typedef float float4_t __attribute__((ext_vector_type(4)));
typedef int int2_t __attribute__((ext_vector_type(2)));
typedef uint32_t uint4_t __attribute__((ext_vector_type(4)));
typedef _Float16 half4_t __attribute__((ext_vector_type(4)));
typedef short short4_t __attribute__((ext_vector_type(4)));
typedef int int4_t __attribute__((ext_vector_type(4)));

constexpr int TK = 64;  // keys per KV tile
constexpr float LAZY_LOG2 = 8.f;  // softmax reference-max slack (log2 units)
constexpr float LN2F = 0.6931471805599453f;

// ------------------------------------------------------------ small helpers --

__device__ __forceinline__ uint16_t f32_to_bf16(float x) {
  uint32_t u = __builtin_bit_cast(uint32_t, x);
  if ((u & 0x7fffffffu) > 0x7f800000u) return (uint16_t)((u >> 16) | 0x40u);  // quiet NaN
  u += 0x7fffu + ((u >> 16) & 1u);                                              // round to nearest even
  return (uint16_t)(u >> 16);
}

__device__ __forceinline__ float bf16_to_f32(uint16_t h) {
  return __builtin_bit_cast(float, (uint32_t)h << 16);
}

// Four int8 cache bytes -> four exact f16 values.  Each byte x becomes the f16
// 1024 + (x + 128) by pairing (x ^ 0x80) with the exponent byte 0x64, then
// 1152 is subtracted (exact in f16).
__device__ __forceinline__ void i8x4_to_f16(uint32_t w, half2_t& lo, half2_t& hi) {
  const uint32_t u = w ^ 0x80808080u;
  const uint32_t a = __builtin_amdgcn_perm(0x64646464u, u, 0x04010400u);
  const uint32_t b = __builtin_amdgcn_perm(0x64646464u, u, 0x04030402u);
  const half2_t bias = {(_Float16)1152.0f, (_Float16)1152.0f};
  lo = __builtin_bit_cast(half2_t, a) - bias;
  hi = __builtin_bit_cast(half2_t, b) - bias;
}

// Four e4m3fn bytes -> four exact f16 values (gfx950 OCP fp8 conversion).
__device__ __forceinline__ void e4m3x4_to_f16(uint32_t w, half2_t& lo, half2_t& hi) {
  lo = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(w, 1.0f, false);
  hi = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(w, 1.0f, true);
}

// Four int8 cache bytes -> four f16 values 1152 + x (exact): (x ^ 0x80) = x + 128
// paired with the exponent byte 0x64 reads as 1024 + (x + 128).  The constant
// offset is removed exactly after the MFMA (a per-row logit bias for K, a
// per-channel shift of the normalized output for V).
__device__ __forceinline__ void i8x4_to_f16_off(uint32_t w, uint32_t& lo, uint32_t& hi) {
  const uint32_t u = w ^ 0x80808080u;
  lo = __builtin_amdgcn_perm(0x64646464u, u, 0x04010400u);
  hi = __builtin_amdgcn_perm(0x64646464u, u, 0x04030402u);
}

// Eight cache bytes -> eight f16 MFMA operand values: e4m3fn exactly, or int8
// as 1152 + x.  Only V operands take the offset form: on K it would add
// 1152 * sum(q) to every logit, and the fp32 accumulator of S would round at
// that magnitude instead of the logit's (K uses bytes8_to_f16).
template <bool FP8>
__device__ __forceinline__ half8_t bytes8_to_op(uint32_t w0, uint32_t w1) {
  if constexpr (FP8) {
    half2_t a, b, c, d;
    e4m3x4_to_f16(w0, a, b);
    e4m3x4_to_f16(w1, c, d);
    half8_t r;
    r[0] = a[0]; r[1] = a[1]; r[2] = b[0]; r[3] = b[1];
    r[4] = c[0]; r[5] = c[1]; r[6] = d[0]; r[7] = d[1];
    return r;
  } else {
    uint32_t a, b, c, d;
    i8x4_to_f16_off(w0, a, b);
    i8x4_to_f16_off(w1, c, d);
    const uint4_t u = {a, b, c, d};
    return __builtin_bit_cast(half8_t, u);
  }
}

template <bool FP8>
__device__ __forceinline__ half8_t bytes8_to_f16(uint32_t w0, uint32_t w1) {
  half2_t a, b, c, d;
  if constexpr (FP8) {
    e4m3x4_to_f16(w0, a, b);
    e4m3x4_to_f16(w1, c, d);
  } else {
    i8x4_to_f16(w0, a, b);
    i8x4_to_f16(w1, c, d);
  }
  half8_t r;
  r[0] = a[0]; r[1] = a[1]; r[2] = b[0]; r[3] = b[1];
  r[4] = c[0]; r[5] = c[1]; r[6] = d[0]; r[7] = d[1];
  return r;
}

// 16-byte-chunk XOR swizzle of a 64-row LDS tile with ROWB bytes per row.
// For ROWB = 128 two rows span the 64 banks; keys k and k' that one 16-lane
// MFMA operand read touches at the same chunk land on distinct bank groups.
// For ROWB = 64 or 576 (576 = 4 mod 16 bank groups) four rows interleave and
// only the low two chunk bits are permuted.  The map is an involution.
template <int ROWB>
__device__ __forceinline__ int swz(int chunk, int row) {
  if constexpr (ROWB == 128) {
    return chunk ^ (((row >> 1) & 7) ^ ((row >> 2) & 4));
  } else {
    const int qd = row >> 2;
    return chunk ^ ((qd ^ ((qd >> 2) << 1)) & 3);
  }
}

// XOR swizzle of the 16-byte chunks of an f16 key row of 256 or 1024 bytes
// (a whole number of 64-bank rows): the 16 keys of an MFMA operand read land
// on 16 distinct bank groups, and the 8 keys that a 16-bit transposed read
// pairs up land on 8 distinct 32-byte groups.  Only the low four chunk bits
// change.
__device__ __forceinline__ int kf_swz(int chunk, int key) {
  return chunk ^ (((key & 7) << 1) | ((key >> 3) & 1));
}

// Page-table address function shared by the attention loads and the debug
// gather: key -> (physical page, slot) -> row address (FlashInfer
// persistent.cuh prefetch_offest; XQA KVTilePartLoader::loadPages).
__device__ __forceinline__ int page_of(const int32_t* table_row, int key, int page_shift) {
  return table_row[key >> page_shift];
}
__device__ __forceinline__ const uint8_t* paged_row(const uint8_t* cache, int page, int key,
                                                    int page_shift, int g, int64_t s_page,
                                                    int64_t s_head, int64_t s_tok) {
  const int slot = key & ((1 << page_shift) - 1);
  return cache + (int64_t)page * s_page + (int64_t)g * s_head + (int64_t)slot * s_tok;
}

// Physical page of `key` among the (at most four) pages pp0..pp3 of a 64-key
// tile whose first page index is pg0.  Plain value selects: no indexing.
__device__ __forceinline__ int pick_page(int key, int page_shift, int pg0, int pp0, int pp1,
                                         int pp2, int pp3) {
  const int j = (key >> page_shift) - pg0;
  int r = pp0;
  r = j == 1 ? pp1 : r;
  r = j == 2 ? pp2 : r;
  r = j == 3 ? pp3 : r;
  return r;
}

// 64 lanes x 16 bytes from global memory straight into LDS: lane l's bytes land
// at lds_base + 16*l.  lds_base goes through M0 (saved and restored here, the
// compiler treats M0 as reserved).
__device__ __forceinline__ void dma16(const void* gsrc, uint32_t lds_base) {
  uint32_t saved;
  asm volatile(
      "s_mov_b32 %0, m0\n\ts_mov_b32 m0, %2\n\ts_nop 0\n\t"
      "global_load_lds_dwordx4 %1, off\n\ts_mov_b32 m0, %0"
      : "=&s"(saved)
      : "v"(gsrc), "s"(__builtin_amdgcn_readfirstlane(lds_base))
      : "memory");
}

// Same with a wave-uniform 64-bit base in SGPRs and a 32-bit per-lane offset.
__device__ __forceinline__ void dma16_s(uint32_t voff, const void* sbase, uint32_t lds_base) {
  uint32_t saved;
  asm volatile(
      "s_mov_b32 %0, m0\n\ts_mov_b32 m0, %3\n\ts_nop 0\n\t"
      "global_load_lds_dwordx4 %1, %2\n\ts_mov_b32 m0, %0"
      : "=&s"(saved)
      : "v"(voff), "s"(sbase), "s"(__builtin_amdgcn_readfirstlane(lds_base))
      : "memory");
}

// A global load whose completion wait is part of the same asm block, so the
// compiler does not add a vmcnt(0) wait at some later join point.
__device__ __forceinline__ int load_i32_sync(const int32_t* ptr) {
  int v;
  asm volatile("global_load_dword %0, %1, off\n\ts_waitcnt vmcnt(0)" : "=v"(v) : "v"(ptr) : "memory");
  return v;
}

// 16 bytes of KV cache, loaded with the non-temporal hint: each cache byte is
// read once per call, and streaming loads measured 5.8 against 5.35 TB/s on
// the decode workload's random 8 KB page slices.
__device__ __forceinline__ uint4_t stream_load16(const uint8_t* p) {
  return __builtin_nontemporal_load((const uint4_t*)p);
}

template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  asm volatile("s_waitcnt vmcnt(%0)" :: "n"(N) : "memory");
}

// Split-KV partial stores.  With the in-kernel merge (coherent = true) a
// workgroup on another XCD reads them in the same kernel, and the XCDs' L2
// caches are not coherent with each other: the stores are agent-scope relaxed
// atomics (global_store sc1, written through to device scope), which the
// merging workgroup reads with agent-scope atomic loads.  This keeps the whole
// L2 out of it: a release fence at agent scope writes back every dirty line of
// the XCD's L2 (buffer_wbl2) and measured 2.4x the decode kernel's time when
// every unit paid it.  Otherwise plain vector stores.
__device__ __forceinline__ void store_partial(float* dst, float v, bool coherent) {
  if (coherent) __hip_atomic_store(dst, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  else *dst = v;
}

__device__ __forceinline__ void store_partial4(float* dst, const float4_t& v, bool coherent) {
  if (coherent) {
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const float x = v[e];
      __hip_atomic_store(dst + e, x, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
  } else {
    *(float4_t*)dst = v;
  }
}

__device__ __forceinline__ float load_partial(const float* src) {
  return __hip_atomic_load(src, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

__device__ __forceinline__ uint32_t lds_addr(const void* p) {
  return (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) void*)p;
}

// Max / sum over the four 16-lane groups (lanes l, l^16, l^32, l^48) with the
// gfx950 lane-swap VALU ops instead of LDS permutes.  With both operands equal,
// v_permlane16_swap returns, in every lane l, the pair {v[l], v[l ^ 16]} (one
// in each result), and v_permlane32_swap the pair {v[l], v[l ^ 32]}; max and
// + are symmetric, so no lane select is needed and every lane of a row gets
// the same bits.
__device__ __forceinline__ float xor16_max(float v) {
  const uint32_t b = __builtin_bit_cast(uint32_t, v);
  const auto r = __builtin_amdgcn_permlane16_swap(b, b, false, false);
  const uint32_t r0 = r[0], r1 = r[1];
  return fmaxf(__builtin_bit_cast(float, r0), __builtin_bit_cast(float, r1));
}
__device__ __forceinline__ float xor32_max(float v) {
  const uint32_t b = __builtin_bit_cast(uint32_t, v);
  const auto r = __builtin_amdgcn_permlane32_swap(b, b, false, false);
  const uint32_t r0 = r[0], r1 = r[1];
  return fmaxf(__builtin_bit_cast(float, r0), __builtin_bit_cast(float, r1));
}
__device__ __forceinline__ float xor16_sum(float v) {
  const uint32_t b = __builtin_bit_cast(uint32_t, v);
  const auto r = __builtin_amdgcn_permlane16_swap(b, b, false, false);
  const uint32_t r0 = r[0], r1 = r[1];
  return __builtin_bit_cast(float, r0) + __builtin_bit_cast(float, r1);
}
__device__ __forceinline__ float xor32_sum(float v) {
  const uint32_t b = __builtin_bit_cast(uint32_t, v);
  const auto r = __builtin_amdgcn_permlane32_swap(b, b, false, false);
  const uint32_t r0 = r[0], r1 = r[1];
  return __builtin_bit_cast(float, r0) + __builtin_bit_cast(float, r1);
}
__device__ __forceinline__ float row_max4(float v) { return xor32_max(xor16_max(v)); }
__device__ __forceinline__ float row_sum4(float v) { return xor32_sum(xor16_sum(v)); }

}  // namespace

// ------------------------------------------------------ shared kernel parts --
//
// A work unit is (request b, KV head g, tile of GQA-packed query rows, KV
// chunk c).  Both attention kernels below share its geometry, the query
// prologue, the online softmax, the PV step and the epilogue; they differ in
// how KV tiles travel from HBM (LDS DMA shared by several waves, or register
// staging in a single wave).

struct Unit {
  int n, tok0, G, rows_total, row0, L, T;
  int c, kv_lo, kv_hi, n_chunks, key_end, mask_from, n_tiles;
  bool split;
};

// Items of the balanced split: request b's T keys are ceil(T / 64) tiles, cut
// into k = ceil(tiles / lt) items of equal tile count (the last one shorter by
// less than one item), where lt is the item length chosen for the whole call.
__device__ __forceinline__ int balanced_items(int T, int lt, int max_chunks) {
  const int tiles = (T + TK - 1) / TK;
  return min((tiles + lt - 1) / lt, max_chunks);
}

// Fills `u` for row tile rt and chunk c of request b; false when the unit is empty.
// tok0, n: the request's first query token and query length; L: its cached keys.
// lt > 0: chunk c is item c of the balanced split with items of <= lt tiles;
// lt = 0: chunk c is keys [c * chunk_size, (c + 1) * chunk_size).
template <int ROWS>
__device__ __forceinline__ bool unit_setup_from(const AttnParams& p, int rt, int c, int tok0, int n, int L,
                                                Unit& u, int lt = 0) {
  u.tok0 = tok0;
  u.n = n;
  u.G = p.group;
  u.rows_total = u.n * u.G;
  u.row0 = rt * ROWS;
  if (u.row0 >= u.rows_total) return false;
  u.L = L;
  u.T = u.L + u.n;
  u.c = c;
  u.kv_lo = 0;
  u.kv_hi = u.T;
  u.n_chunks = 1;
  if (p.chunk_size > 0 && lt > 0) {
    u.n_chunks = balanced_items(u.T, lt, p.max_chunks);
    if (c >= u.n_chunks) return false;
    const int len = ((u.T + TK - 1) / TK + u.n_chunks - 1) / u.n_chunks * TK;   // keys per item
    u.kv_lo = c * len;
    u.kv_hi = min(u.T, u.kv_lo + len);
  } else if (p.chunk_size > 0) {
    u.n_chunks = (u.T + p.chunk_size - 1) / p.chunk_size;
    if (c >= u.n_chunks) return false;
    u.kv_lo = c * p.chunk_size;
    u.kv_hi = min(u.T, u.kv_lo + p.chunk_size);
  } else if (c > 0) {
    return false;
  }
  u.split = u.n_chunks > 1;
  const int last_tok = (min(u.rows_total, u.row0 + ROWS) - 1) / u.G;
  const int first_tok = u.row0 / u.G;
  // Bottom-right causal: token t sees keys j <= L + t.  A draft-tree mask
  // decides every appended key instead (cached keys stay visible).
  const bool causal_rule = p.causal && !p.tree_mask;
  u.key_end = causal_rule ? min(u.kv_hi, u.L + last_tok + 1) : u.kv_hi;
  u.mask_from = p.tree_mask ? min(u.kv_hi, u.L)
                            : (p.causal ? min(u.kv_hi, u.L + first_tok + 1) : u.kv_hi);  // keys >= this need masks
  u.n_tiles = u.key_end > u.kv_lo ? (u.key_end - u.kv_lo + TK - 1) / TK : 0;
  return true;
}

template <int ROWS>
__device__ __forceinline__ bool unit_setup(const AttnParams& p, int b, int rt, int c, Unit& u) {
  const int tok0 = p.cu_seqlens_q ? p.cu_seqlens_q[b] : b * p.q_len_uniform;
  const int n = p.cu_seqlens_q ? p.cu_seqlens_q[b + 1] - tok0 : p.q_len_uniform;
  return unit_setup_from<ROWS>(p, rt, c, tok0, n, p.seq_lens_kv[b], u);
}

// Unit of a workgroup of the shared-tile kernels.  Workgroup L runs on XCD
// L % 8 (round-robin dispatch).  A group is the row tiles of one (request, KV
// head, chunk): they read the same KV tiles, so they are kept on one XCD (one
// L2), in consecutive dispatch slots there, and groups are dealt round-robin
// over the XCDs in (request, head, chunk) order.  Later (longer, causal) row
// tiles go first.
//
// Group numbering: when the grid is many rounds of resident workgroups deep,
// group r is slot r of the (request, head, chunk) grid, empty or not (empty
// ones exit at once and the dispatcher balances the rest).  When the grid is
// about one round deep (compact_groups), only the groups that hold work are
// numbered, so every XCD gets the same number of them (+-1) however the
// request lengths are spread, and no XCD is left with more workgroups than
// CUs.  False for the padding past the last group and for empty row tiles;
// otherwise `u` is set.
// Item length of the balanced split (after the work-list planner of
// FlashInfer persistent.cuh, which cuts each request's KV into chunks so that
// the CTAs get equal work, there on the host): the smallest lt >= chunk_size /
// 64 tiles for which the groups H_kv * sum_b ceil(tiles_b / lt) fit p.group_cap
// (one round of resident workgroups), by binary search over lt; the longest
// request's tile count when no lt fits.  Every wave of every workgroup computes
// the same value from the lengths.
__device__ __forceinline__ int balanced_item_tiles(const AttnParams& p, int lane) {
  auto tiles_of = [&](int bb) {
    if (bb >= p.batch) return 0;
    const int n = p.cu_seqlens_q ? p.cu_seqlens_q[bb + 1] - p.cu_seqlens_q[bb] : p.q_len_uniform;
    return n > 0 ? (p.seq_lens_kv[bb] + n + TK - 1) / TK : 0;   // requests without queries: no items
  };
  const int t0 = tiles_of(lane);   // the first 64 requests stay in a register
  // wave reductions, returned as scalars (the same in every lane), so the
  // search and every address derived from lt stay uniform
  auto wave_sum = [](int v) {
#pragma unroll
    for (int d = 1; d < 64; d <<= 1) v += __shfl_xor(v, d, 64);
    return __builtin_amdgcn_readfirstlane(v);
  };
  auto wave_max = [](int v) {
#pragma unroll
    for (int d = 1; d < 64; d <<= 1) v = max(v, __shfl_xor(v, d, 64));
    return __builtin_amdgcn_readfirstlane(v);
  };
  int tmax = t0;
  for (int b0 = 64; b0 < p.batch; b0 += 64) tmax = max(tmax, tiles_of(b0 + lane));
  tmax = wave_max(tmax);
  auto groups = [&](int lt) {
    int s = (t0 + lt - 1) / lt;
    for (int b0 = 64; b0 < p.batch; b0 += 64) s += (tiles_of(b0 + lane) + lt - 1) / lt;
    return wave_sum(s) * p.num_kv_heads;
  };
  int lo = max(1, p.chunk_size / TK), hi = max(lo, tmax);
  while (lo < hi) {
    const int mid = (lo + hi) >> 1;
    if (groups(mid) <= p.group_cap) hi = mid;
    else lo = mid + 1;
  }
  return lo;
}

// BAL: the balanced split's planner is compiled in (a variant of the MLA
// kernel of its own: in the kernels' main loops it cost SGPR spills).
template <int ROWS, bool BAL = false>
__device__ __forceinline__ bool shared_tile_unit(const AttnParams& p, int& b, int& g, Unit& u) {
  const int L = (int)blockIdx.x;
  const int lane = (int)threadIdx.x & 63;
  const int slot = L >> 3;
  const int rt = p.row_tiles - 1 - slot % p.row_tiles;
  int r = (slot / p.row_tiles) * 8 + (L & 7);   // group index
  int lt = 0;
  if constexpr (BAL) {
    if (p.balanced) lt = balanced_item_tiles(p, lane);
    if (p.balanced && p.plan_out && L == 0 && threadIdx.x == 0) *p.plan_out = lt;   // for the merge
  }
  if (!p.compact_groups) {
    const int c = r % p.max_chunks;
    r /= p.max_chunks;
    g = r % p.num_kv_heads;
    b = r / p.num_kv_heads;
    if (b >= p.batch) return false;
    const int tok0 = p.cu_seqlens_q ? p.cu_seqlens_q[b] : b * p.q_len_uniform;
    const int n = p.cu_seqlens_q ? p.cu_seqlens_q[b + 1] - tok0 : p.q_len_uniform;
    return unit_setup_from<ROWS>(p, rt, c, tok0, n, p.seq_lens_kv[b], u, lt);
  }
  // lane l looks at request b0 + l: first token, query length, cached keys
  auto fetch = [&](int b0, int& tok0, int& n, int& kl) {
    const int bb = min(b0 + lane, p.batch - 1);
    tok0 = p.cu_seqlens_q ? p.cu_seqlens_q[bb] : bb * p.q_len_uniform;
    n = p.cu_seqlens_q ? p.cu_seqlens_q[bb + 1] : tok0 + p.q_len_uniform;
    kl = p.seq_lens_kv[bb];
  };
  int tok0, n, kl;
  fetch(0, tok0, n, kl);
  int base = 0;
  for (int b0 = 0; b0 < p.batch; b0 += 64) {
    int tok0_nx = 0, n_nx = 0, kl_nx = 0;
    if (b0 + 64 < p.batch) fetch(b0 + 64, tok0_nx, n_nx, kl_nx);   // next batch in flight
    n -= tok0;
    int cnt = 0;   // groups of request b0 + lane: KV heads x chunks with work
    if (b0 + lane < p.batch && n > 0)
      cnt = p.num_kv_heads * (p.chunk_size <= 0 ? 1
                              : lt > 0      ? balanced_items(kl + n, lt, p.max_chunks)
                                            : min((kl + n + p.chunk_size - 1) / p.chunk_size, p.max_chunks));
    int incl = cnt;   // inclusive prefix sum over the 64 lanes
#pragma unroll
    for (int d = 1; d < 64; d <<= 1) {
      const int t = __shfl_up(incl, d, 64);
      if (lane >= d) incl += t;
    }
    const int total = __builtin_amdgcn_readlane(incl, 63);
    if (r < base + total) {
      const uint64_t hit = __ballot(base + incl > r);
      const int lb = (int)__builtin_ctzll(hit);
      const int start = base + __builtin_amdgcn_readlane(incl - cnt, lb);
      const int nch = __builtin_amdgcn_readlane(cnt, lb) / p.num_kv_heads;
      b = b0 + lb;
      r -= start;
      g = r / nch;
      const int c = r - g * nch;
      return unit_setup_from<ROWS>(p, rt, c, __builtin_amdgcn_readlane(tok0, lb), __builtin_amdgcn_readlane(n, lb),
                                   __builtin_amdgcn_readlane(kl, lb), u, lt);
    }
    base += total;
    tok0 = tok0_nx;
    n = n_nx;
    kl = kl_nx;
  }
  return false;
}

// Query rows of one wave as the B operand of S^T = K Q^T.
// k-step 2s covers dims 64s + 16*grp + [0,8), k-step 2s+1 dims 64s + 16*grp + [8,16).
// A row is multiplied by a power of two 2^k that puts its largest element in
// [2^14, 2^15), so f16 keeps full relative precision.  Per-channel K scales and
// sm_scale*log2(e) are folded into Q in that case (then hi + lo parts keep the
// products exact to ~2^-22); otherwise they multiply S^T in fp32 (row_mult).
// kbias is the log2-domain logit offset that the int8 operand offset adds.
template <int DQK, int NT, bool HILO>
struct QRows {
  static constexpr int KPAIRS = DQK / 64;
  half8_t hi[NT][2 * KPAIRS];
  half8_t lo[HILO ? NT : 1][HILO ? 2 * KPAIRS : 1];
  float row_mult[NT];
  float kbias[NT];
  int tok[NT], head[NT];
  bool ok[NT];
};

template <int DQK, int NT, bool HILO>
__device__ __forceinline__ void load_query(const AttnParams& p, const Unit& u, int g, int row_base,
                                           int lane, float kv_off, QRows<DQK, NT, HILO>& q) {
  constexpr int KPAIRS = DQK / 64;
  const int l16 = lane & 15, grp = lane >> 4;
  const int mode = p.scale_mode;
  const bool fold_channel = mode == PA_SCALE_PER_CHANNEL;
  const float k_uniform = fold_channel ? 1.f : p.k_scale[mode == PA_SCALE_PER_HEAD ? g : 0];
  // Short heads keep the row and its per-channel scales in registers (one pass
  // over global memory); long ones re-read the row after finding its maximum.
  constexpr bool ONE_PASS = KPAIRS <= 2;
  float ksc[ONE_PASS ? KPAIRS : 1][16];
  if constexpr (ONE_PASS) {
    if (fold_channel) {
#pragma unroll
      for (int sp = 0; sp < KPAIRS; ++sp) {
        const float4_t* sc = (const float4_t*)(p.k_scale + (int64_t)g * DQK + 64 * sp + 16 * grp);
#pragma unroll
        for (int v = 0; v < 4; ++v) {
          const float4_t f = sc[v];
#pragma unroll
          for (int e = 0; e < 4; ++e) ksc[sp][4 * v + e] = p.qk_mult * f[e];
        }
      }
    }
  }
  auto load_q16 = [&](int64_t qoff, int sp, float* x) {
    const int d0 = 64 * sp + 16 * grp;
    if (p.q_is_f32) {
      const float4_t* src = (const float4_t*)((const float*)p.q + qoff + d0);
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        const float4_t f = src[v];
        x[4 * v] = f[0]; x[4 * v + 1] = f[1]; x[4 * v + 2] = f[2]; x[4 * v + 3] = f[3];
      }
    } else {
      const uint4_t* src = (const uint4_t*)((const uint16_t*)p.q + qoff + d0);
#pragma unroll
      for (int v = 0; v < 2; ++v) {
        const uint4_t w = src[v];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          x[8 * v + 2 * e] = bf16_to_f32((uint16_t)(w[e] & 0xffffu));
          x[8 * v + 2 * e + 1] = bf16_to_f32((uint16_t)(w[e] >> 16));
        }
      }
    }
    if (fold_channel) {
      if constexpr (ONE_PASS) {
#pragma unroll
        for (int e = 0; e < 16; ++e) x[e] *= ksc[sp][e];
      } else {
        const float4_t* sc = (const float4_t*)(p.k_scale + (int64_t)g * DQK + d0);
#pragma unroll
        for (int v = 0; v < 4; ++v) {
          const float4_t f = sc[v];
#pragma unroll
          for (int e = 0; e < 4; ++e) x[4 * v + e] *= p.qk_mult * f[e];
        }
      }
    }
  };
#pragma unroll
  for (int nt = 0; nt < NT; ++nt) {
    const int r = row_base + nt * 16 + l16;
    q.ok[nt] = r < u.rows_total;
    const int t = q.ok[nt] ? r / u.G : 0;
    q.tok[nt] = t;
    q.head[nt] = g * u.G + (q.ok[nt] ? r % u.G : 0);
    const int64_t qoff = (int64_t)(u.tok0 + t) * p.q_row_stride + (int64_t)q.head[nt] * DQK;
    float xq[ONE_PASS ? KPAIRS : 1][16];
    float amax = 0.f;
#pragma unroll
    for (int sp = 0; sp < KPAIRS; ++sp) {
      float x[16];
      if (q.ok[nt]) {
        load_q16(qoff, sp, x);
      } else {
#pragma unroll
        for (int e = 0; e < 16; ++e) x[e] = 0.f;
      }
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        amax = fmaxf(amax, fabsf(x[e]));
        if constexpr (ONE_PASS) xq[sp][e] = x[e];
      }
    }
    amax = row_max4(amax);
    int ex = 0;
    if (amax > 0.f) (void)frexpf(amax, &ex);     // amax < 2^ex
    const int k2 = min(max(15 - ex, -120), 120);
    const float up = ldexpf(1.f, k2);
    q.row_mult[nt] = ldexpf(1.f, -k2) * (fold_channel ? 1.f : p.qk_mult * k_uniform);
    float qsum = 0.f;
#pragma unroll
    for (int sp = 0; sp < KPAIRS; ++sp) {
      float x[16];
      if constexpr (ONE_PASS) {
#pragma unroll
        for (int e = 0; e < 16; ++e) x[e] = xq[sp][e];
      } else if (q.ok[nt]) {
        load_q16(qoff, sp, x);
      } else {
#pragma unroll
        for (int e = 0; e < 16; ++e) x[e] = 0.f;
      }
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        const float v = x[e] * up;
        const _Float16 h = (_Float16)v;
        q.hi[nt][2 * sp + e / 8][e % 8] = h;
        qsum += (float)h;
        if constexpr (HILO) {
          const _Float16 l = (_Float16)(v - (float)h);
          q.lo[nt][2 * sp + e / 8][e % 8] = l;
          qsum += (float)l;
        }
      }
    }
    q.kbias[nt] = kv_off * row_sum4(qsum) * q.row_mult[nt];
  }
}

// Split form of load_query for short heads (D <= 128), used where the first KV
// tile should be in flight while the query is processed: query_fetch issues
// every query and scale load, then the caller issues its tile loads, and
// query_finish does the arithmetic once the query bytes are in.  Loads of one
// wave complete in order, so the query is waited for without waiting for the
// tile.  The fetch is branch-free (rows past the unit re-read the unit's first
// row, bf16 rows re-read their first 32 bytes where fp32 rows read 64, scale
// loads that the mode does not use re-read the query) so that the compiler's
// wait counts stay exact.  The result equals load_query's.
template <int DQK, int NT>
struct QRaw {
  static constexpr int KPAIRS = DQK / 64;
  uint4_t x[NT][KPAIRS][4];   // 16 bf16 (first two vectors) or 16 fp32 per (row, pair)
  float4_t ksc[KPAIRS][4];    // per-channel K scales of this lane's 16 dims per pair
  float k_uniform;            // per-tensor or per-head K scale
};

template <int DQK, int NT>
__device__ __forceinline__ void query_fetch(const AttnParams& p, const Unit& u, int g, int row_base,
                                            int lane, QRaw<DQK, NT>& raw) {
  constexpr int KPAIRS = DQK / 64;
  static_assert(KPAIRS <= 2, "query_fetch holds the whole row in registers");
  const int l16 = lane & 15, grp = lane >> 4;
  const int mode = p.scale_mode;
  const bool f32 = p.q_is_f32;
  const int esize = f32 ? 4 : 2;
  const uint8_t* qrow[NT];
#pragma unroll
  for (int nt = 0; nt < NT; ++nt) {
    const int r0 = row_base + nt * 16 + l16;
    const int r = r0 < u.rows_total ? r0 : u.row0;
    const int64_t qoff = (int64_t)(u.tok0 + r / u.G) * p.q_row_stride + (int64_t)(g * u.G + r % u.G) * DQK;
    qrow[nt] = (const uint8_t*)p.q + qoff * esize;
  }
#pragma unroll
  for (int sp = 0; sp < KPAIRS; ++sp) {
    const uint8_t* sc = mode == PA_SCALE_PER_CHANNEL
                            ? (const uint8_t*)(p.k_scale + (int64_t)g * DQK + 64 * sp + 16 * grp)
                            : qrow[0];
#pragma unroll
    for (int v = 0; v < 4; ++v) raw.ksc[sp][v] = *(const float4_t*)(sc + 16 * v);
  }
  raw.k_uniform = p.k_scale[mode == PA_SCALE_PER_HEAD ? g : 0];
#pragma unroll
  for (int nt = 0; nt < NT; ++nt)
#pragma unroll
    for (int sp = 0; sp < KPAIRS; ++sp) {
      const uint8_t* src = qrow[nt] + (64 * sp + 16 * grp) * esize;
#pragma unroll
      for (int v = 0; v < 4; ++v) raw.x[nt][sp][v] = *(const uint4_t*)(src + 16 * (f32 ? v : (v & 1)));
    }
}

template <int DQK, int NT, bool HILO>
__device__ __forceinline__ void query_finish(const AttnParams& p, const Unit& u, int g, int row_base,
                                             int lane, float kv_off, const QRaw<DQK, NT>& raw,
                                             QRows<DQK, NT, HILO>& q) {
  constexpr int KPAIRS = DQK / 64;
  const int l16 = lane & 15;
  const int mode = p.scale_mode;
  const bool fold_channel = mode == PA_SCALE_PER_CHANNEL;
  const float k_uniform = fold_channel ? 1.f : raw.k_uniform;
#pragma unroll
  for (int nt = 0; nt < NT; ++nt) {
    const int r = row_base + nt * 16 + l16;
    q.ok[nt] = r < u.rows_total;
    const int t = q.ok[nt] ? r / u.G : 0;
    q.tok[nt] = t;
    q.head[nt] = g * u.G + (q.ok[nt] ? r % u.G : 0);
    float xq[KPAIRS][16];
    float amax = 0.f;
#pragma unroll
    for (int sp = 0; sp < KPAIRS; ++sp) {
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        float x;
        if (p.q_is_f32) {
          // (the element goes through a scalar: bit-casting a vector element
          // in place made this compiler read lane 0 of the vector)
          const uint32_t bits = raw.x[nt][sp][e / 4][e % 4];
          x = __builtin_bit_cast(float, bits);
        } else {
          const uint32_t w = raw.x[nt][sp][e / 8][(e % 8) / 2];
          x = bf16_to_f32((uint16_t)((e & 1) ? (w >> 16) : (w & 0xffffu)));
        }
        if (fold_channel) x *= p.qk_mult * raw.ksc[sp][e / 4][e % 4];
        x = q.ok[nt] ? x : 0.f;
        xq[sp][e] = x;
        amax = fmaxf(amax, fabsf(x));
      }
    }
    amax = row_max4(amax);
    int ex = 0;
    if (amax > 0.f) (void)frexpf(amax, &ex);     // amax < 2^ex
    const int k2 = min(max(15 - ex, -120), 120);
    const float up = ldexpf(1.f, k2);
    q.row_mult[nt] = ldexpf(1.f, -k2) * (fold_channel ? 1.f : p.qk_mult * k_uniform);
    float qsum = 0.f;
#pragma unroll
    for (int sp = 0; sp < KPAIRS; ++sp)
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        const float v = xq[sp][e] * up;
        const _Float16 h = (_Float16)v;
        q.hi[nt][2 * sp + e / 8][e % 8] = h;
        qsum += (float)h;
        if constexpr (HILO) {
          const _Float16 l = (_Float16)(v - (float)h);
          q.lo[nt][2 * sp + e / 8][e % 8] = l;
          qsum += (float)l;
        }
      }
    q.kbias[nt] = kv_off * row_sum4(qsum) * q.row_mult[nt];
  }
}

// Query rows for S^T = K Q^T on the int8 MFMA (v_mfma_i32_16x16x64_i8), used
// with int8 caches: K bytes go to the MFMA as they are, and each query row,
// scaled by QI8_MAX / max|row| and rounded to an integer q, is split into three
// balanced base-256 digits q = 65536 qh + 256 qm + ql, each in [-128, 127].
// S = 65536 (K . qh) + 256 (K . qm) + K . ql with every product exact in int32;
// the rounding of q, 2^-23 of the row maximum per element, is the only error,
// so rows with outlier channels keep their small elements (two digits, 2^-15,
// were not enough for rows whose maximum is 16x their typical element).  Lane
// l holds, per 64-dim step s, the digits of dims 64s + 16*grp + [0, 16) of row
// l16, the same dims its K operand holds.
constexpr float QI8_MAX = 8355000.f;   // |q| <= 127 * 65536 + 32767: top digit stays in int8

template <int DQK, int NT>
struct QRowsI8 {
  static constexpr int KSTEPS = DQK / 64;
  int4_t qd[KSTEPS][3][NT];   // step, digit (high, middle, low), row tile
  float row_mult[NT];
  float kbias[NT];   // 0: no operand offset on K
  int tok[NT], head[NT];
  bool ok[NT];
};

// Digits of one row from its 16 * KSTEPS lane values (already scaled by the
// per-channel K scales and sm_scale * log2(e) when those are folded).
template <int DQK, int NT>
__device__ __forceinline__ void query_digits(float (&xq)[DQK / 64][16], int nt, float mult_rest,
                                             QRowsI8<DQK, NT>& q) {
  constexpr int KSTEPS = DQK / 64;
  float amax = 0.f;
#pragma unroll
  for (int sp = 0; sp < KSTEPS; ++sp)
#pragma unroll
    for (int e = 0; e < 16; ++e) amax = fmaxf(amax, fabsf(xq[sp][e]));
  amax = row_max4(amax);
  const bool nz = amax > 1e-30f;
  const float up = nz ? QI8_MAX / amax : 0.f;
  q.row_mult[nt] = nz ? (amax / QI8_MAX) * mult_rest : 0.f;
  q.kbias[nt] = 0.f;
#pragma unroll
  for (int sp = 0; sp < KSTEPS; ++sp) {
    uint32_t w[3][4] = {};
#pragma unroll
    for (int e = 0; e < 16; ++e) {
      const int v = min(max((int)rintf(xq[sp][e] * up), -8355000), 8355000);
      const int d0 = ((v + 128) & 255) - 128;        // low digit
      const int v1 = (v - d0) >> 8;
      const int d1 = ((v1 + 128) & 255) - 128;       // middle digit
      const int d2 = (v1 - d1) >> 8;                 // high digit, |d2| <= 128 * (8355000 / 2^23)
      w[0][e / 4] |= ((uint32_t)d2 & 0xffu) << (8 * (e % 4));
      w[1][e / 4] |= ((uint32_t)d1 & 0xffu) << (8 * (e % 4));
      w[2][e / 4] |= ((uint32_t)d0 & 0xffu) << (8 * (e % 4));
    }
#pragma unroll
    for (int k = 0; k < 3; ++k) q.qd[sp][k][nt] = int4_t{(int)w[k][0], (int)w[k][1], (int)w[k][2], (int)w[k][3]};
  }
}

// QRowsI8 of one 16-row tile for long heads (the MLA kernel's 576 dims): the
// row is read twice (maximum, then digits), lane l taking dims 64 s + 16
// (l / 16) + [0, 16) of row l % 16, with per-channel K scales and sm_scale *
// log2(e) folded in when K is per channel.
template <int DQK>
__device__ __forceinline__ void load_query_i8(const AttnParams& p, const Unit& u, int g, int row_base, int lane,
                                              QRowsI8<DQK, 1>& q) {
  constexpr int KSTEPS = DQK / 64;
  const int l16 = lane & 15, grp = lane >> 4;
  const int mode = p.scale_mode;
  const bool fold_channel = mode == PA_SCALE_PER_CHANNEL;
  const float k_uniform = fold_channel ? 1.f : p.k_scale[mode == PA_SCALE_PER_HEAD ? g : 0];
  const int r = row_base + l16;
  q.ok[0] = r < u.rows_total;
  const int t = q.ok[0] ? r / u.G : 0;
  q.tok[0] = t;
  q.head[0] = g * u.G + (q.ok[0] ? r % u.G : 0);
  const int64_t qoff = (int64_t)(u.tok0 + t) * p.q_row_stride + (int64_t)q.head[0] * DQK;
  float xq[KSTEPS][16];
#pragma unroll
  for (int sp = 0; sp < KSTEPS; ++sp) {
    const int d0 = 64 * sp + 16 * grp;
#pragma unroll
    for (int e = 0; e < 16; ++e) xq[sp][e] = 0.f;
    if (q.ok[0]) {
      if (p.q_is_f32) {
        const float4_t* src = (const float4_t*)((const float*)p.q + qoff + d0);
#pragma unroll
        for (int v = 0; v < 4; ++v) {
          const float4_t f = src[v];
#pragma unroll
          for (int e = 0; e < 4; ++e) xq[sp][4 * v + e] = f[e];
        }
      } else {
        const uint4_t* src = (const uint4_t*)((const uint16_t*)p.q + qoff + d0);
#pragma unroll
        for (int v = 0; v < 2; ++v) {
          const uint4_t w = src[v];
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            xq[sp][8 * v + 2 * e] = bf16_to_f32((uint16_t)(w[e] & 0xffffu));
            xq[sp][8 * v + 2 * e + 1] = bf16_to_f32((uint16_t)(w[e] >> 16));
          }
        }
      }
      if (fold_channel) {
        const float4_t* sc = (const float4_t*)(p.k_scale + (int64_t)g * DQK + d0);
#pragma unroll
        for (int v = 0; v < 4; ++v) {
          const float4_t f = sc[v];
#pragma unroll
          for (int e = 0; e < 4; ++e) xq[sp][4 * v + e] *= p.qk_mult * f[e];
        }
      }
    }
  }
  query_digits<DQK, 1>(xq, 0, fold_channel ? 1.f : p.qk_mult * k_uniform, q);
}

// query_finish for the int8 MFMA (see QRowsI8).
template <int DQK, int NT>
__device__ __forceinline__ void query_finish_i8(const AttnParams& p, const Unit& u, int g, int row_base,
                                                int lane, const QRaw<DQK, NT>& raw, QRowsI8<DQK, NT>& q) {
  constexpr int KPAIRS = DQK / 64;
  const int l16 = lane & 15;
  const int mode = p.scale_mode;
  const bool fold_channel = mode == PA_SCALE_PER_CHANNEL;
  const float k_uniform = fold_channel ? 1.f : raw.k_uniform;
#pragma unroll
  for (int nt = 0; nt < NT; ++nt) {
    const int r = row_base + nt * 16 + l16;
    q.ok[nt] = r < u.rows_total;
    q.tok[nt] = q.ok[nt] ? r / u.G : 0;
    q.head[nt] = g * u.G + (q.ok[nt] ? r % u.G : 0);
    float xq[KPAIRS][16];
#pragma unroll
    for (int sp = 0; sp < KPAIRS; ++sp)
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        float x;
        if (p.q_is_f32) {
          const uint32_t bits = raw.x[nt][sp][e / 4][e % 4];
          x = __builtin_bit_cast(float, bits);
        } else {
          const uint32_t w = raw.x[nt][sp][e / 8][(e % 8) / 2];
          x = bf16_to_f32((uint16_t)((e & 1) ? (w >> 16) : (w & 0xffffu)));
        }
        if (fold_channel) x *= p.qk_mult * raw.ksc[sp][e / 4][e % 4];
        xq[sp][e] = q.ok[nt] ? x : 0.f;
      }
    query_digits<DQK, NT>(xq, nt, fold_channel ? 1.f : p.qk_mult * k_uniform, q);
  }
}

// Query rows for S^T = K Q^T on the fp8 MFMA (v_mfma_scale_f32_16x16x128_
// f8f6f4), used with e4m3fn caches: the K bytes go to the MFMA as they are
// (block scale 1), and the query is split into ND e4m3fn digits q = d_0 + ...
// + d_{ND-1}, each the nearest e4m3fn value to what the earlier digits left.
// The instruction scales each 32-deep K block of each row by a power of two
// (E8M0).  Its K order: lane group g (lanes 16g..16g+15) holds K indices
// 16g + [0, 16) in bytes 0..15 and 64 + 16g + [0, 16) in bytes 16..31, so
// block b (K indices 32b..32b+31) is one 16-byte half (the first for b < 2)
// of lane groups 2 (b % 2) and 2 (b % 2) + 1, and its scale is read from lane
// group b (measured on the GPU; an unscaled product cannot tell, since A and B
// share the order).  Every block of the query is scaled so that its largest
// element lies in (224, 448], the top of e4m3fn's range, and the MFMA scales
// it back.  A bf16 value (8 significant bits) is then two 4-bit digits
// exactly unless its second digit falls below e4m3fn's subnormal step, i.e.
// for elements under ~2^-9 of their block's maximum (an error of at most
// 2^-18 of that maximum each); fp32 queries and per-channel folded scales take
// three digits.  Scaling per block rather than per row keeps a few large
// channels from pushing the rest of the row into that range (rows with two
// channels 64x the rest: LSE error 3.1e-3 with one scale per row, 9.3e-5 per
// block, in a CPU model of the split).  Lane l holds, per 128-dim step s,
// bytes for dims 128 s + 32 (l / 16) + [0, 32) of row l % 16 (the same
// permutation for K and Q), zero past the head dim, and in sc[s] the E8M0
// exponent of block l / 16 of its row.
typedef int v8i_t __attribute__((ext_vector_type(8)));

template <int DQK, int ND>
struct QRowsF8 {
  static constexpr int STEPS = (DQK + 127) / 128;
  v8i_t qd[ND][STEPS];
  int sc[STEPS];      // E8M0 block scale (2^(sc - 127)) of this lane's block per step
  float row_mult[1];
  float kbias[1];   // 0: K operands are exact
  int tok[1], head[1];
  bool ok[1];
};

template <int DQK, int ND>
__device__ __forceinline__ void load_query_f8(const AttnParams& p, const Unit& u, int g, int row_base, int lane,
                                              QRowsF8<DQK, ND>& q) {
  constexpr int STEPS = QRowsF8<DQK, ND>::STEPS;
  const int l16 = lane & 15, grp = lane >> 4;
  const int mode = p.scale_mode;
  const bool fold_channel = mode == PA_SCALE_PER_CHANNEL;
  const float k_uniform = fold_channel ? 1.f : p.k_scale[mode == PA_SCALE_PER_HEAD ? g : 0];
  const int r = row_base + l16;
  q.ok[0] = r < u.rows_total;
  const int t = q.ok[0] ? r / u.G : 0;
  q.tok[0] = t;
  q.head[0] = g * u.G + (q.ok[0] ? r % u.G : 0);
  const int64_t qoff = (int64_t)(u.tok0 + t) * p.q_row_stride + (int64_t)q.head[0] * DQK;
  // 8 elements from dim d0 = 128 s + 32 grp + 8 j8 (step s, lane group grp)
  auto load8 = [&](int d0, float* x) {
    if (!q.ok[0] || d0 >= DQK) {
#pragma unroll
      for (int e = 0; e < 8; ++e) x[e] = 0.f;
      return;
    }
    if (p.q_is_f32) {
      const float4_t* src = (const float4_t*)((const float*)p.q + qoff + d0);
      const float4_t a = src[0], b = src[1];
#pragma unroll
      for (int e = 0; e < 4; ++e) { x[e] = a[e]; x[4 + e] = b[e]; }
    } else {
      const uint4_t w = *(const uint4_t*)((const uint16_t*)p.q + qoff + d0);
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        x[2 * e] = bf16_to_f32((uint16_t)(w[e] & 0xffffu));
        x[2 * e + 1] = bf16_to_f32((uint16_t)(w[e] >> 16));
      }
    }
    if (fold_channel) {
      const float4_t* sc = (const float4_t*)(p.k_scale + (int64_t)g * DQK + d0);
      const float4_t a = sc[0], b = sc[1];
#pragma unroll
      for (int e = 0; e < 4; ++e) { x[e] *= p.qk_mult * a[e]; x[4 + e] *= p.qk_mult * b[e]; }
    }
  };
  q.row_mult[0] = fold_channel ? 1.f : p.qk_mult * k_uniform;
  // 2^k2 puts amax = m 2^ex (m in [0.5, 1)) into (224, 448]
  auto block_k2 = [](float amax) {
    int ex = 0;
    const float m = amax > 0.f ? frexpf(amax, &ex) : 1.f;
    return min(max((m > 0.875f ? 8 : 9) - ex, -120), 120);
  };
#pragma unroll
  for (int st = 0; st < STEPS; ++st) {
    float x[32];   // dims 128 st + 32 grp + [0, 32)
#pragma unroll
    for (int j8 = 0; j8 < 4; ++j8) load8(128 * st + 32 * grp + 8 * j8, x + 8 * j8);
    float a_lo = 0.f, a_hi = 0.f;
#pragma unroll
    for (int e = 0; e < 16; ++e) {
      a_lo = fmaxf(a_lo, fabsf(x[e]));
      a_hi = fmaxf(a_hi, fabsf(x[16 + e]));
    }
    // block maxima: this lane pair's two blocks (xor 16), the other pair's (xor 32)
    const float p_lo = xor16_max(a_lo), p_hi = xor16_max(a_hi);
    const float o_lo = __shfl_xor(p_lo, 32, 64), o_hi = __shfl_xor(p_hi, 32, 64);
    const int k_lo = block_k2(p_lo), k_hi = block_k2(p_hi);
    // block grp's maximum: groups 0, 1 hold blocks 0 (lo) and 2 (hi), groups 2, 3 blocks 1 and 3
    const float bmax = grp == 0 ? p_lo : grp == 1 ? o_lo : grp == 2 ? o_hi : p_hi;
    q.sc[st] = 127 - block_k2(bmax);
    const float up_lo = ldexpf(1.f, k_lo), up_hi = ldexpf(1.f, k_hi);
#pragma unroll
    for (int j8 = 0; j8 < 4; ++j8) {
      const float up = j8 < 2 ? up_lo : up_hi;
      uint32_t w[ND][2] = {};
#pragma unroll
      for (int e = 0; e < 8; e += 2) {
        float r0 = x[8 * j8 + e] * up, r1 = x[8 * j8 + e + 1] * up;
#pragma unroll
        for (int d = 0; d < ND; ++d) {
          // two e4m3fn (OCP) codes in one 16-bit half, and their exact values
          typedef short short2_t __attribute__((ext_vector_type(2)));
          const short2_t zero2 = {0, 0};
          const uint32_t pk =
              __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_fp8_f32(zero2, r0, r1, 1.0f, false)) &
              0xffffu;
          const auto back = __builtin_amdgcn_cvt_scalef32_pk_f32_fp8((int)pk, 1.0f, false);
          r0 -= back[0];
          r1 -= back[1];
          w[d][(e / 2) >> 1] |= pk << (16 * ((e / 2) & 1));
        }
      }
#pragma unroll
      for (int d = 0; d < ND; ++d) {
        q.qd[d][st][2 * j8] = (int)w[d][0];
        q.qd[d][st][2 * j8 + 1] = (int)w[d][1];
      }
    }
    __builtin_amdgcn_sched_barrier(0);   // one step's 32 elements live at a time
  }
}

// S^T += K Q^T over one 64-dim step on the int8 MFMA: `a` holds the lane's 16
// K bytes; the three digit products accumulate apart (combined by s_from_i8).
template <int NT>
__device__ __forceinline__ void qk_i8_step(const int4_t& a, const int4_t (&qd)[3][NT], int4_t (&acc)[3][NT]) {
#pragma unroll
  for (int k = 0; k < 3; ++k)
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) acc[k][nt] = __builtin_amdgcn_mfma_i32_16x16x64_i8(a, qd[k][nt], acc[k][nt], 0, 0, 0);
}

// 65536 h + 256 m + l: (h << 8) + m is exact in int32 (|K . qh| < 2^21), the
// last step runs in fp32 (relative rounding 2^-24).
__device__ __forceinline__ float4_t s_from_i8(const int4_t& h, const int4_t& m, const int4_t& l) {
  float4_t r;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int hi = h[i], mi = m[i], lo = l[i];
    const int t = (int)(((uint32_t)hi << 8) + (uint32_t)mi);
    r[i] = fmaf((float)t, 256.f, (float)lo);
  }
  return r;
}

// Online-softmax state of one wave: O^T accumulators (lane holds dims
// 16*md + 4*grp + i of row l16), running max (log2 units) and denominator.
template <int NT, int MD>
struct SoftmaxState {
  float4_t o[MD > 0 ? MD : 1][NT];   // MD == 0: no O here (the caller keeps it elsewhere)
  float m[NT], l[NT];
};

template <int NT, int MD>
__device__ __forceinline__ void softmax_init(SoftmaxState<NT, MD>& st) {
#pragma unroll
  for (int nt = 0; nt < NT; ++nt) {
    st.m[nt] = -INFINITY;
    st.l[nt] = 0.f;
#pragma unroll
    for (int md = 0; md < MD; ++md) st.o[md][nt] = float4_t{0.f, 0.f, 0.f, 0.f};
  }
}

// Draft-tree visibility of the rows of one wave (row_base + 16 nt + lane % 16),
// written to `rows_lds` (two words per row: bits 0..31 and 32..63): bit s is
// set when appended key L + s is visible to the row's token, i.e.
// tree_mask[b][t][s] != 0 with s < n.  The four lanes of a row read 16
// entries each and combine them with two xor shuffles; lane group 0 stores.
// Rows past the last token read token n - 1 (their results are never
// written).  The words live in LDS, not registers, because only the tiles
// that reach the appended keys read them.  The same wave reads them back, so
// LDS ordering within the wave is all the synchronisation needed.
template <int NT>
__device__ __forceinline__ void load_tree_bits(const AttnParams& p, int b, const Unit& u, int row_base, int lane,
                                               uint32_t* rows_lds) {
  const int l16 = lane & 15, grp = lane >> 4;
  const int ml = p.tree_mask_len;
#pragma unroll
  for (int nt = 0; nt < NT; ++nt) {
    const int r = row_base + nt * 16 + l16;
    const int t = min(r / u.G, u.n - 1);
    const uint8_t* row = p.tree_mask + ((int64_t)b * ml + t) * ml;
    uint32_t bits = 0;
#pragma unroll
    for (int e = 0; e < 16; ++e) {
      const int sidx = 16 * grp + e;
      const uint8_t v = row[min(sidx, u.n - 1)];
      bits |= (uint32_t)(sidx < u.n && v != 0) << e;
    }
    uint32_t w = bits << (16 * (grp & 1));
    w |= (uint32_t)__shfl_xor((int)w, 16, 64);
    const uint32_t other = (uint32_t)__shfl_xor((int)w, 32, 64);
    if (grp == 0) {
      rows_lds[2 * (nt * 16 + l16)] = w;
      rows_lds[2 * (nt * 16 + l16) + 1] = other;
    }
  }
}

// Masks one 64-key tile of S^T, updates the running max/denominator, rescales
// O when a row maximum grows, and returns P^T (f16) in the B-operand layout of
// the PV MFMA: pb[ks][nt] holds keys {32ks + 4grp + i, 32ks + 16 + 4grp + i}.
template <int NT, int MD, typename QT, bool TREE = false>
__device__ __forceinline__ void softmax_tile(const AttnParams& p, const Unit& u, int kbase, int grp,
                                             const QT& q, float4_t (&s)[4][NT],
                                             SoftmaxState<NT, MD>& st, half8_t (&pb)[2][NT],
                                             const uint32_t* tree_rows = nullptr) {
  const bool need_mask = kbase + TK > u.mask_from;
  const half2_t ones2 = {(_Float16)1.0f, (_Float16)1.0f};
  float alpha[NT];
#pragma unroll
  for (int nt = 0; nt < NT; ++nt) {
    if (need_mask) {
      if constexpr (TREE) {
        // Visibility of keys kbase + j, j < 64, as one 64-bit word: the cached
        // keys below min(kv_hi, L), the appended keys whose draft bit is set,
        // nothing at or past kv_hi.  Lane group grp tests bits 16 mt + 4 grp + i.
        const int r16 = (int)threadIdx.x & 15;
        const uint64_t drafts = ((uint64_t)tree_rows[2 * (nt * 16 + r16) + 1] << 32) | tree_rows[2 * (nt * 16 + r16)];
        const int dl = u.L - kbase;   // key kbase + j is draft j - dl
        const uint64_t vis_d = dl >= 0 ? (dl < 64 ? drafts << dl : 0ull) : (-dl < 64 ? drafts >> (-dl) : 0ull);
        const int nc = min(max(min(u.kv_hi, u.L) - kbase, 0), 64);
        const int ne = min(max(u.kv_hi - kbase, 0), 64);
        const uint64_t below_c = nc >= 64 ? ~0ull : ((1ull << nc) - 1);
        const uint64_t below_e = ne >= 64 ? ~0ull : ((1ull << ne) - 1);
        const uint64_t vis = ((below_c | vis_d) & below_e) >> (4 * grp);
#pragma unroll
        for (int mt = 0; mt < 4; ++mt)
#pragma unroll
          for (int i = 0; i < 4; ++i)
            if (!((vis >> (mt * 16 + i)) & 1ull)) s[mt][nt][i] = -INFINITY;
      } else {
        const int lim = p.causal ? min(u.kv_hi, u.L + q.tok[nt] + 1) : u.kv_hi;
#pragma unroll
        for (int mt = 0; mt < 4; ++mt)
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const int key = kbase + mt * 16 + grp * 4 + i;
            if (key >= lim) s[mt][nt][i] = -INFINITY;
          }
      }
    }
    float mx = -INFINITY;
#pragma unroll
    for (int mt = 0; mt < 4; ++mt)
#pragma unroll
      for (int i = 0; i < 4; ++i) mx = fmaxf(mx, s[mt][nt][i]);
    mx = row_max4(mx) * q.row_mult[nt] - q.kbias[nt];
    // Lazy rescaling: the reference maximum only moves when the row maximum
    // exceeds it by more than 2^LAZY_LOG2; weights then stay <= 256 (exact
    // enough in f16 and fp32) and O is rescaled rarely.  lse = m + log2(l)
    // holds for any reference m.
    const float m_new = mx > st.m[nt] + LAZY_LOG2 ? mx : st.m[nt];
    const float m_use = m_new == -INFINITY ? 0.f : m_new;
    alpha[nt] = __builtin_amdgcn_exp2f(st.m[nt] - m_use);
    st.m[nt] = m_new;
    const float nb = -(q.kbias[nt] + m_use);
#pragma unroll
    for (int ks = 0; ks < 2; ++ks)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        pb[ks][nt][i] = (_Float16)__builtin_amdgcn_exp2f(fmaf(s[2 * ks][nt][i], q.row_mult[nt], nb));
        pb[ks][nt][4 + i] = (_Float16)__builtin_amdgcn_exp2f(fmaf(s[2 * ks + 1][nt][i], q.row_mult[nt], nb));
      }
    // Row sum of the f16 weights the MFMA actually sees.  (The pairs are built
    // from vector elements: bit-casting uint4 lanes to half2 here made this
    // compiler reuse one register for all four dot products.)
    float ls = 0.f;
#pragma unroll
    for (int ks = 0; ks < 2; ++ks)
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const half2_t pr = {pb[ks][nt][2 * e], pb[ks][nt][2 * e + 1]};
        ls = __builtin_amdgcn_fdot2(pr, ones2, ls, false);
      }
    st.l[nt] = st.l[nt] * alpha[nt] + ls;
  }
  if constexpr (MD > 0) {
    bool grew = false;
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) grew |= alpha[nt] != 1.f;
    if (__builtin_amdgcn_ballot_w64(grew) != 0) {
#pragma unroll
      for (int nt = 0; nt < NT; ++nt)
#pragma unroll
        for (int md = 0; md < MD; ++md) st.o[md][nt] *= alpha[nt];
    }
  }
}

// O^T += V^T P^T for one 64-key tile whose V rows sit in LDS (VROW bytes per
// row, XOR-swizzled chunks).  tr8 read: lanes 2j, 2j+1 of a 16-lane group give
// the two 8-byte halves of key row kappa(grp, j); lane i then holds
// V[kappa(grp, j)][16*md + i], j = 0..7.
template <bool FP8, int NT, int MD, int VROW>
__device__ __forceinline__ void pv_tile(const uint8_t* vs, int lane, const half8_t (&pb)[2][NT],
                                        SoftmaxState<NT, MD>& st) {
  const int l16 = lane & 15, grp = lane >> 4;
  const int jr = l16 >> 1;
  const int hlf = lane & 1;
#pragma unroll
  for (int ks = 0; ks < 2; ++ks) {
    const int vrow = 32 * ks + (jr < 4 ? 4 * grp + jr : 16 + 4 * grp + (jr - 4));
#pragma unroll
    for (int md = 0; md < MD; ++md) {
      const uint8_t* addr = vs + vrow * VROW + swz<VROW>(md, vrow) * 16 + hlf * 8;
      const int2_t raw = __builtin_amdgcn_ds_read_tr8_b64_v2i32(
          (__attribute__((address_space(3))) int2_t*)(addr));
      const half8_t a = bytes8_to_op<FP8>((uint32_t)raw[0], (uint32_t)raw[1]);
#pragma unroll
      for (int nt = 0; nt < NT; ++nt)
        st.o[md][nt] = __builtin_amdgcn_mfma_f32_16x16x32_f16(a, pb[ks][nt], st.o[md][nt], 0, 0, 0);
    }
  }
}

// Normalize, remove the int8 operand offset, apply V scales and write the final
// bf16 row + natural lse, or the chunk's fp32 partial + lse.
template <int DV, int NT, typename QT>
__device__ __forceinline__ void write_rows(const AttnParams& p, const Unit& u, int g, int c, int lane,
                                           float kv_off, const QT& q,
                                           const SoftmaxState<NT, DV / 16>& st,
                                           const float4_t (&vsc)[DV / 16]) {
  constexpr int MD = DV / 16;
  const int grp = lane >> 4;
  const int H_q = p.num_q_heads;
#pragma unroll
  for (int nt = 0; nt < NT; ++nt) {
    const float lt = row_sum4(st.l[nt]);
    const int tok = u.tok0 + q.tok[nt];
    const int h = q.head[nt];
    const float inv = lt > 0.f ? 1.f / lt : 0.f;
    const float off = lt > 0.f ? kv_off : 0.f;
    const float lse_nat = lt > 0.f ? (st.m[nt] + __log2f(lt)) * LN2F : -INFINITY;
    if (!q.ok[nt]) continue;
    float* prow = u.split ? p.part_o + (((int64_t)tok * p.max_chunks + c) * H_q + h) * DV : nullptr;
    uint16_t* orow = p.out + ((int64_t)tok * H_q + h) * DV;
#pragma unroll
    for (int md = 0; md < MD; ++md) {
      const int d = md * 16 + grp * 4;
      float4_t v;
#pragma unroll
      for (int i = 0; i < 4; ++i) v[i] = fmaf(st.o[md][nt][i], inv, -off) * vsc[md][i];
      if (u.split) {
        store_partial4(prow + d, v, p.merge_count != nullptr);
      } else {
        const uint32_t w0 = (uint32_t)f32_to_bf16(v[0]) | ((uint32_t)f32_to_bf16(v[1]) << 16);
        const uint32_t w1 = (uint32_t)f32_to_bf16(v[2]) | ((uint32_t)f32_to_bf16(v[3]) << 16);
        *(int2_t*)(orow + d) = int2_t{(int)w0, (int)w1};
      }
    }
    if (grp == 0) {
      if (u.split)
        store_partial(p.part_lse + ((int64_t)tok * p.max_chunks + c) * H_q + h, lse_nat, p.merge_count != nullptr);
      else if (p.lse) p.lse[(int64_t)tok * H_q + h] = lse_nat;
    }
  }
}

// Per-channel V scales of this lane's output dims (16*md + 4*grp + i).
template <int DV>
__device__ __forceinline__ void load_v_scales(const AttnParams& p, int g, int lane, float4_t (&vsc)[DV / 16]) {
  constexpr int MD = DV / 16;
  const int grp = lane >> 4;
  const int mode = p.scale_mode;
  if (mode == PA_SCALE_PER_CHANNEL) {
#pragma unroll
    for (int md = 0; md < MD; ++md)
      vsc[md] = *(const float4_t*)(p.v_scale + (int64_t)g * DV + md * 16 + grp * 4);
  } else {
    const float v = p.v_scale[mode == PA_SCALE_PER_HEAD ? g : 0];
#pragma unroll
    for (int md = 0; md < MD; ++md) vsc[md] = float4_t{v, v, v, v};
  }
}

// ------------------------------------------------------ split-KV merge math --
//
// Log-sum-exp merge of one (token, head) row's chunk partials, four channels
// per thread, in chunk order with a running maximum: M = max_c lse_c,
// w_c = e^(lse_c - M), O = sum_c w_c O_c / sum_c w_c, lse = M + ln sum_c w_c.
// A chunk with lse = -inf (no visible key) weighs 0; a row whose chunks are
// all -inf gives O = 0, lse = -inf.  split_merge_kernel and the in-kernel
// merge (merge_if_last) share it, so both produce the same bits.
struct RowMerge {
  float M = -INFINITY, den = 0.f;
  float4_t acc = {0.f, 0.f, 0.f, 0.f};
  __device__ __forceinline__ void add(bool use, float l, const float4_t& o) {
    use = use && l != -INFINITY;
    const float m_new = use ? fmaxf(M, l) : M;
    const float sc = m_new == M ? 1.f : __expf(M - m_new);   // M = -inf gives 0
    const float w = use ? __expf(l - m_new) : 0.f;
    den = den * sc + w;
#pragma unroll
    for (int e = 0; e < 4; ++e) acc[e] = acc[e] * sc + (use ? w * o[e] : 0.f);
    M = m_new;
  }
  // four bf16 channels to dst; the natural lse to *lse_dst unless it is null
  __device__ __forceinline__ void store(uint16_t* dst, float* lse_dst) const {
    const float inv = den > 0.f ? 1.f / den : 0.f;
    const uint32_t w0 = (uint32_t)f32_to_bf16(acc[0] * inv) | ((uint32_t)f32_to_bf16(acc[1] * inv) << 16);
    const uint32_t w1 = (uint32_t)f32_to_bf16(acc[2] * inv) | ((uint32_t)f32_to_bf16(acc[3] * inv) << 16);
    *(int2_t*)dst = int2_t{(int)w0, (int)w1};
    if (lse_dst) *lse_dst = den > 0.f ? M + __logf(den) : -INFINITY;
  }
};

// In-kernel merge of the split-KV partials (PA_FLAG_FUSED_MERGE), after the
// semaphore pattern of XQA mla_sm120.cu (mergePartialOutputs: the last CTA of
// a sequence merges, then resets the semaphore).  Every unit of a (request,
// KV head, row tile) stores its chunk's partial rows, then adds one to
// merge_count[b][g][row0 / 16]; the unit that brings the count to the
// request's chunk count merges the partials of those rows and sets the
// counter back to 0 for the next call.  The units run on different XCDs,
// whose L2 caches are not coherent with each other, so the partials travel
// as agent-scope atomics (store_partial / load_partial: each access is
// coherent at device scope by itself), and the order is kept by waiting for
// the wave's stores to be acknowledged (vmcnt 0; stores count there on this
// ISA) before the counter's atomic add, whose result the merging unit waits
// for before its first load.  Called by the decode kernel's wave that writes
// the unit's rows (ROWS packed rows from u.row0), after its partial stores; the
// wider shared-tile and MLA tiles merge in split_merge_kernel instead (merged
// here by one workgroup they measured slower, and the tail cost their main
// loops SGPR spills).
template <int DV, int ROWS>
__device__ __forceinline__ void merge_if_last(const AttnParams& p, const Unit& u, int b, int g, int lane) {
  if (!p.merge_count || !u.split) return;
  wait_vmcnt<0>();   // this wave's partial stores are visible at device scope
  int32_t* cnt = p.merge_count + ((int64_t)b * p.num_kv_heads + g) * p.count_stride + (u.row0 >> 4);
  int old = 0;
  if (lane == 0) old = __hip_atomic_fetch_add(cnt, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  const bool last = __builtin_amdgcn_readfirstlane(old) == u.n_chunks - 1;
  if (!last) return;
  // Reader side: an agent-scope acquire orders the partial loads below after
  // the counter's read-modify-write in the memory model (one unit per row tile
  // pays for it).  The writer side has no release fence: at agent scope it
  // would write back the XCD's whole L2 in every unit; the partials are
  // agent-scope atomic stores instead, each coherent by itself, and the
  // vmcnt(0) wait above makes them complete before the counter's atomic issues.
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
  if (lane == 0) __hip_atomic_store(cnt, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  constexpr int QPR = DV / 4;   // four-channel slots per row
  // chunk slots loaded per round trip: the agent-scope loads are single
  // dwords, so eight slots in flight (40 loads) raised the register count of
  // the narrow kernels that compile this tail
  constexpr int MB = 4;
  // row slots per thread whose loads travel together: one, since this tail is
  // compiled into every attention kernel and its loads in flight set the
  // kernel's register count (two measured no faster on decode and cost the
  // 64-dim kernels a wave per SIMD)
  constexpr int SPT = 1;
  const int rows = min(u.rows_total, u.row0 + ROWS) - u.row0;
  const int64_t H = p.num_q_heads;
  const int nc = u.n_chunks;
  for (int base = lane; base < rows * QPR; base += SPT * 64) {
    bool ok[SPT];
    int64_t tok[SPT];
    int h[SPT], q4[SPT];
    RowMerge m[SPT];
#pragma unroll
    for (int t = 0; t < SPT; ++t) {
      const int idx = base + t * 64;
      ok[t] = idx < rows * QPR;
      const int r = u.row0 + (ok[t] ? idx / QPR : 0);
      q4[t] = idx % QPR;
      tok[t] = u.tok0 + r / u.G;
      h[t] = g * u.G + r % u.G;
    }
    for (int c0 = 0; c0 < nc; c0 += MB) {
      float lc[SPT][MB];
      float4_t v[SPT][MB];
#pragma unroll
      for (int t = 0; t < SPT; ++t)
#pragma unroll
        for (int k = 0; k < MB; ++k) {
          lc[t][k] = -INFINITY;
          v[t][k] = float4_t{0.f, 0.f, 0.f, 0.f};
          if (ok[t] && c0 + k < nc) {
            const int64_t slot = tok[t] * p.max_chunks + c0 + k;
            lc[t][k] = load_partial(p.part_lse + slot * H + h[t]);
            const float* src = p.part_o + (slot * H + h[t]) * DV + q4[t] * 4;
#pragma unroll
            for (int e = 0; e < 4; ++e) v[t][k][e] = load_partial(src + e);
          }
        }
#pragma unroll
      for (int t = 0; t < SPT; ++t)
#pragma unroll
        for (int k = 0; k < MB; ++k) m[t].add(c0 + k < nc, lc[t][k], v[t][k]);
    }
#pragma unroll
    for (int t = 0; t < SPT; ++t)
      if (ok[t])
        m[t].store(p.out + (tok[t] * H + h[t]) * DV + q4[t] * 4,
                   (p.lse && q4[t] == 0) ? p.lse + tok[t] * H + h[t] : nullptr);
  }
}

// DmaTileLoader: the shared-tile and MLA kernels' loader.  A 64-key tile
// (K rows of KROW bytes, then V rows of VROW bytes unless V is the prefix of
// the K row) travels by LDS DMA (global_load_lds_dwordx4, 16 bytes per lane)
// into one LDS stage, its 16-byte chunks XOR-swizzled per row (swz).  The NW
// waves of a workgroup split the tile's 1 KB blocks: block j*NW + wave of K,
// then of V.  Page ids, the one-page fast path and the clamped general path
// are as in RegTileLoader.
// HOLD: keep each DMA's per-lane source offset in a register (else recompute
// it at every issue, for kernels short of registers).
template <int KROW, int VROW, int NW, bool SHARED, bool HOLD = true, int TKEYS = TK>
struct DmaTileLoader {
  static_assert(TKEYS == 32 || TKEYS == 64, "32- or 64-key tiles");
  static constexpr int KTILE = TKEYS * KROW;
  static constexpr int VTILE = SHARED ? 0 : TKEYS * VROW;
  static constexpr int STAGE = KTILE + VTILE;
  static constexpr int KCH = KTILE / 16;                 // 16-byte chunks per K tile
  static constexpr int VCH = VTILE / 16;
  static constexpr int KCPR = KROW / 16;                 // chunks per K row
  static constexpr int VCPR = VROW / 16;
  static constexpr int K_DMA = (KCH + 64 * NW - 1) / (64 * NW);   // DMA instructions per wave (at most)
  static constexpr int V_DMA = (VCH + 64 * NW - 1) / (64 * NW);
  const int32_t* table_row;
  int g, wave, kv_lo, key_end, last_page, page_shift;
  int pw_base, pw_val;
  bool one_page, fast_addr;
  uint32_t smem_base;
  uint32_t koff[HOLD ? K_DMA : 1], voff[HOLD && V_DMA > 0 ? V_DMA : 1];
  int64_t ks_tok, vs_tok;

  __device__ __forceinline__ uint32_t k_offset(int j) const {
    if constexpr (HOLD) return koff[j];
    const int ch = (j * NW + wave) * 64 + (int)(threadIdx.x & 63);
    const int row = ch / KCPR;
    return (uint32_t)(row * ks_tok + swz<KROW>(ch % KCPR, row) * 16);
  }
  __device__ __forceinline__ uint32_t v_offset(int j) const {
    if constexpr (HOLD) return voff[j];
    const int ch = (j * NW + wave) * 64 + (int)(threadIdx.x & 63);
    const int row = ch / VCPR;
    return (uint32_t)(row * vs_tok + swz<VROW>(ch % VCPR, row) * 16);
  }

  __device__ __forceinline__ void init(const AttnParams& p, int b, int g_, int wave_, int kv_lo_, int key_end_,
                                       int n_tiles, int lane, uint32_t smem_base_) {
    table_row = p.block_table + (int64_t)b * p.max_pages_per_seq;
    g = g_;
    wave = wave_;
    kv_lo = kv_lo_;
    key_end = key_end_;
    page_shift = p.page_shift;
    last_page = n_tiles > 0 ? (key_end - 1) >> page_shift : 0;   // never read past it
    pw_base = -(1 << 30);
    pw_val = 0;
    one_page = page_shift >= (TKEYS == 64 ? 6 : 5);   // tiles start at multiples of TKEYS
    fast_addr = one_page && (int64_t)TKEYS * p.k_stride_token < (1LL << 30) &&
                (SHARED || (int64_t)TKEYS * p.v_stride_token < (1LL << 30));
    smem_base = smem_base_;
    ks_tok = p.k_stride_token;
    vs_tok = p.v_stride_token;
    if constexpr (HOLD) {
#pragma unroll
      for (int j = 0; j < K_DMA; ++j) {
        const int ch = (j * NW + wave) * 64 + lane;
        const int row = ch / KCPR;
        koff[j] = (uint32_t)(row * p.k_stride_token + swz<KROW>(ch % KCPR, row) * 16);
      }
#pragma unroll
      for (int j = 0; j < V_DMA; ++j) {
        const int ch = (j * NW + wave) * 64 + lane;
        const int row = ch / VCPR;
        voff[j] = (uint32_t)(row * p.v_stride_token + swz<VROW>(ch % VCPR, row) * 16);
      }
    }
  }

  // Issues this wave's share of tile `tile` into LDS stage `stage`.
  __device__ __forceinline__ void issue(const AttnParams& p, int tile, int stage) {
    const int kbase = kv_lo + tile * TKEYS;
    const int pg0 = kbase >> page_shift;
    const int pg_last = min(pg0 + 3, last_page);
    if (pg0 < pw_base || pg_last > pw_base + 63) {
      // Refill the window (drains the DMA queue; once per 64 pages).
      pw_base = pg0;
      pw_val = load_i32_sync(table_row + min(pg0 + (int)(threadIdx.x & 63), last_page));
    }
    const int pp0 = __builtin_amdgcn_readlane(pw_val, pg0 - pw_base);
    const uint32_t kdst = smem_base + stage * STAGE;
    const uint32_t vdst = kdst + KTILE;
    if (fast_addr && kbase + TKEYS <= key_end) {
      const uint8_t* kb = paged_row(p.k_cache, pp0, kbase, page_shift, g, p.k_stride_page, p.k_stride_head,
                                    p.k_stride_token);
#pragma unroll
      for (int j = 0; j < K_DMA; ++j)
        if ((j * NW + wave) * 64 < KCH) dma16_s(k_offset(j), kb, kdst + (j * NW + wave) * 1024);
      if constexpr (!SHARED) {
        const uint8_t* vb = paged_row(p.v_cache, pp0, kbase, page_shift, g, p.v_stride_page, p.v_stride_head,
                                      p.v_stride_token);
#pragma unroll
        for (int j = 0; j < V_DMA; ++j)
          if ((j * NW + wave) * 64 < VCH) dma16_s(v_offset(j), vb, vdst + (j * NW + wave) * 1024);
      }
      return;
    }
    // general path: up to four pages per tile (page_size >= 16), clamped rows
    int pp1 = pp0, pp2 = pp0, pp3 = pp0;
    if (!one_page) {
      pp1 = __builtin_amdgcn_readlane(pw_val, min(pg0 + 1, pg_last) - pw_base);
      pp2 = __builtin_amdgcn_readlane(pw_val, min(pg0 + 2, pg_last) - pw_base);
      pp3 = __builtin_amdgcn_readlane(pw_val, pg_last - pw_base);
    }
    const int lane = threadIdx.x & 63;
#pragma unroll
    for (int j = 0; j < K_DMA; ++j) {
      const int blk = j * NW + wave;
      if (blk * 64 < KCH) {
        const int ch = blk * 64 + lane;
        const int row = ch / KCPR;
        const int key = min(kbase + row, key_end - 1);
        const uint8_t* src = paged_row(p.k_cache, pick_page(key, page_shift, pg0, pp0, pp1, pp2, pp3), key,
                                       page_shift, g, p.k_stride_page, p.k_stride_head, p.k_stride_token) +
                             swz<KROW>(ch % KCPR, row) * 16;
        dma16(src, kdst + blk * 1024);
      }
    }
    if constexpr (!SHARED) {
#pragma unroll
      for (int j = 0; j < V_DMA; ++j) {
        const int blk = j * NW + wave;
        if (blk * 64 < VCH) {
          const int ch = blk * 64 + lane;
          const int row = ch / VCPR;
          const int key = min(kbase + row, key_end - 1);
          const uint8_t* src = paged_row(p.v_cache, pick_page(key, page_shift, pg0, pp0, pp1, pp2, pp3), key,
                                         page_shift, g, p.v_stride_page, p.v_stride_head, p.v_stride_token) +
                               swz<VROW>(ch % VCPR, row) * 16;
          dma16(src, vdst + blk * 1024);
        }
      }
    }
  }
};

// ----------------------------------------------- shared-tile attention kernel --
//
// Template parameters: head dims, cache format, NT 16-row MFMA tiles per wave,
// NW waves per workgroup (they split the rows and share every KV tile), SHARED
// (V = prefix of the K row), HILO (Q is split into f16 hi + lo parts because
// its values carry per-channel scales or come from fp32; a bf16 query with
// per-head or per-tensor scales is exact in f16 and needs one part), NSTAGE
// (KV tiles staged in LDS; NSTAGE - 1 tiles are in flight while one is used).
//
// KV tiles travel by LDS DMA (global_load_lds_dwordx4, 16 B per lane), issued
// with inline assembly and tracked with explicit s_waitcnt vmcnt(N): the
// compiler would otherwise drain every outstanding DMA before each LDS access.
// No other vector-memory instruction is issued inside the main loop except the
// rare refill of the page-id window, which waits for itself.

// CONV: the workgroup converts each raw K/V tile to f16 tiles in LDS once
// (each wave a quarter) and the waves read MFMA operands from those, instead of
// every wave converting the whole raw tile for its own rows (D = 128 only).
template <int DQK, int DV, bool FP8, int NT, int NW, bool SHARED, bool HILO, int NSTAGE, bool CONV, bool TREE>
__global__ __launch_bounds__(64 * NW, NT == 1 ? 3 : (NW == 4 ? 2 : 1)) void paged_attn_kernel(AttnParams p) {
  constexpr int ROWS_W = 16 * NT;
  constexpr int ROWS = ROWS_W * NW;
  constexpr int KROW = DQK;                       // bytes per K row in LDS
  constexpr int VROW = SHARED ? DQK : DV;         // bytes per V row in LDS
  constexpr int KTILE = TK * KROW;
  constexpr int VTILE = SHARED ? 0 : TK * VROW;
  constexpr int STAGE = KTILE + VTILE;
  constexpr int KCH = KTILE / 16;                 // 16-byte chunks per K tile
  constexpr int VCH = VTILE / 16;
  constexpr int KCPR = KROW / 16;                 // chunks per K row
  constexpr int VCPR = VROW / 16;
  constexpr int KPAIRS = DQK / 64;                // pairs of 32-wide k-steps
  constexpr int MD = DV / 16;                     // 16-dim output tiles
  constexpr int K_DMA = (KCH + 64 * NW - 1) / (64 * NW);
  constexpr int V_DMA = (VCH + 64 * NW - 1) / (64 * NW);
  constexpr int DMA_PER_TILE = K_DMA + V_DMA;     // exact for NW == 1
  // int8 V operands reach the MFMA as 1152 + x (see i8x4_to_f16_off); K
  // operands are exact (bytes8_to_f16), so the query carries no logit bias
  constexpr float KV_OFF = FP8 ? 0.f : 1152.f;
  static_assert(DQK % 64 == 0 && DV % 16 == 0, "head dims");
  static_assert(KCH % 64 == 0 && VCH % 64 == 0, "tile chunks");
  static_assert(NSTAGE == 2 || NW == 1 || (KCH % (64 * NW) == 0 && VCH % (64 * NW) == 0),
                "deep multi-wave pipelines need equal per-wave DMA counts");
  static_assert(DMA_PER_TILE * (NSTAGE - 2) <= 63, "vmcnt range");
  static_assert(!CONV || (DQK == 128 && DV == 128 && !SHARED && (TK * 16) % (64 * NW) == 0),
                "f16 tiles: 256-byte rows, separate K and V");
  constexpr int FROW = 2 * DQK;                   // f16 row bytes (CONV)
  // int8 caches: S^T on the int8 MFMA (QRowsI8), except with f16 tiles, where
  // converting K once per workgroup costs less than turning int32 S into fp32
  // in every wave
  constexpr bool I8QK = !FP8 && DQK <= 128 && !CONV;
  constexpr int VF16 = I8QK ? 0 : TK * FROW;      // offset of the f16 V tile (after f16 K)

  __shared__ __attribute__((aligned(1024))) uint8_t smem[NSTAGE * STAGE];
  __shared__ __attribute__((aligned(1024))) uint8_t f16t[CONV ? VF16 + TK * FROW : 16];

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int l16 = lane & 15;
  const int grp = lane >> 4;
  // grid = (row tiles * chunks, H_kv, B): the row tiles of one request and head
  // are dispatched next to each other (they read the same KV), longest first
  int b, g;
  Unit u;
  if (!shared_tile_unit<ROWS>(p, b, g, u)) return;
  const int key_end = u.key_end, kv_lo = u.kv_lo, n_tiles = u.n_tiles;

  // ---- KV tile loader ----
  DmaTileLoader<KROW, VROW, NW, SHARED> ld;
  ld.init(p, b, g, wave, kv_lo, key_end, n_tiles, lane, lds_addr(smem));
  auto issue_tile = [&](int tile, int stage) { ld.issue(p, tile, stage); };

  // First tiles go out before the query prologue so both latencies overlap.
#pragma unroll
  for (int st = 0; st < NSTAGE - 1; ++st)
    if (st < n_tiles) issue_tile(st, st);

  using QT = typename std::conditional<I8QK, QRowsI8<DQK, NT>, QRows<DQK, NT, HILO>>::type;
  QT q;
  if constexpr (I8QK) {
    QRaw<DQK, NT> qraw;
    query_fetch<DQK, NT>(p, u, g, u.row0 + wave * ROWS_W, lane, qraw);
    query_finish_i8<DQK, NT>(p, u, g, u.row0 + wave * ROWS_W, lane, qraw, q);
  } else {
    load_query<DQK, NT, HILO>(p, u, g, u.row0 + wave * ROWS_W, lane, 0.f, q);
  }
  __shared__ uint32_t tree_lds[TREE ? NW * NT * 32 : 1];
  uint32_t* const tb = tree_lds + (TREE ? wave * NT * 32 : 0);
  if constexpr (TREE) load_tree_bits<NT>(p, b, u, u.row0 + wave * ROWS_W, lane, tb);
  SoftmaxState<NT, MD> st;
  softmax_init(st);

  for (int it = 0; it < n_tiles; ++it) {
    const int stage = it % NSTAGE;
    // tile `it` has landed once at most (tiles issued after it) * DMA_PER_TILE DMAs remain
    if constexpr (NSTAGE == 2) {
      wait_vmcnt<0>();
    } else {
      const int ahead = min(NSTAGE - 2, n_tiles - 1 - it);
      if (ahead <= 0) wait_vmcnt<0>();
      else if (ahead == 1) wait_vmcnt<DMA_PER_TILE>();
      else if (ahead == 2) wait_vmcnt<(NSTAGE >= 4 ? 2 : 1) * DMA_PER_TILE>();
      else wait_vmcnt<(NSTAGE >= 5 ? 3 : 1) * DMA_PER_TILE>();
    }
    if constexpr (NW > 1) __syncthreads();
    if (it + NSTAGE - 1 < n_tiles) issue_tile(it + NSTAGE - 1, (it + NSTAGE - 1) % NSTAGE);
    const uint8_t* ks = smem + stage * STAGE;
    const uint8_t* vs = SHARED ? ks : ks + KTILE;
    const int kbase = kv_lo + it * TK;

    if constexpr (CONV) {
      // raw rows -> f16 rows (V always; K only when S^T is not on the int8 MFMA);
      // thread item: one 8-byte half-chunk of a 128-byte row, a wave's lanes
      // covering 4 consecutive keys
      constexpr int ITEMS = TK * 16 / (64 * NW);   // per thread and matrix
      constexpr int NM = I8QK ? 1 : 2;              // matrices converted: V (and K)
      int2_t raw[NM][ITEMS];
#pragma unroll
      for (int i = 0; i < ITEMS; ++i) {
        const int item = (i * NW + wave) * 64 + lane;
        const int key = item >> 4, hc = item & 15;
        const int src = key * KROW + swz<KROW>(hc >> 1, key) * 16 + (hc & 1) * 8;
        raw[0][i] = *(const int2_t*)(vs + src);
        if constexpr (NM == 2) raw[1][i] = *(const int2_t*)(ks + src);
      }
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int i = 0; i < ITEMS; ++i) {
        const int item = (i * NW + wave) * 64 + lane;
        const int key = item >> 4, hc = item & 15;
        const int dst = key * FROW + kf_swz(hc, key) * 16;
        *(half8_t*)(f16t + VF16 + dst) = bytes8_to_op<FP8>((uint32_t)raw[0][i][0], (uint32_t)raw[0][i][1]);
        if constexpr (NM == 2)
          *(half8_t*)(f16t + dst) = bytes8_to_f16<FP8>((uint32_t)raw[1][i][0], (uint32_t)raw[1][i][1]);
      }
      __syncthreads();   // f16 tiles complete (the next B0 orders their reuse)

      float4_t s[4][NT];
      {
#pragma unroll
      for (int mt = 0; mt < 4; ++mt)
#pragma unroll
        for (int nt = 0; nt < NT; ++nt) s[mt][nt] = float4_t{0.f, 0.f, 0.f, 0.f};
      half8_t ka[KPAIRS][4][2];
#pragma unroll
      for (int sp = 0; sp < KPAIRS; ++sp)
#pragma unroll
        for (int mt = 0; mt < 4; ++mt)
#pragma unroll
          for (int h = 0; h < 2; ++h) {
            const int key = mt * 16 + l16;
            ka[sp][mt][h] = *(const half8_t*)(f16t + key * FROW + kf_swz(8 * sp + 2 * grp + h, key) * 16);
          }
      // QK, softmax and PV at raised wave priority: the other workgroup on the
      // CU, if it is converting its tile or waiting at a barrier, yields the
      // issue slots (measured 174 -> 163 us on the append workload; priority
      // around the MFMA loops alone gave nothing)
      __builtin_amdgcn_s_setprio(1);
#pragma unroll
      for (int sp = 0; sp < KPAIRS; ++sp)
#pragma unroll
        for (int h = 0; h < 2; ++h)
#pragma unroll
          for (int mt = 0; mt < 4; ++mt)
#pragma unroll
            for (int nt = 0; nt < NT; ++nt) {
              s[mt][nt] = __builtin_amdgcn_mfma_f32_16x16x32_f16(ka[sp][mt][h], q.hi[nt][2 * sp + h], s[mt][nt], 0, 0, 0);
              if constexpr (HILO)
                s[mt][nt] = __builtin_amdgcn_mfma_f32_16x16x32_f16(ka[sp][mt][h], q.lo[nt][2 * sp + h], s[mt][nt], 0, 0, 0);
            }
      }
      half8_t pb[2][NT];
      softmax_tile<NT, MD, QT, TREE>(p, u, kbase, grp, q, s, st, pb, tb);
      // O^T += V^T P^T, V^T by the 16-bit transposed read of the f16 V tile
      const int tr_j = l16 >> 2, tr_q = l16 & 3;
#pragma unroll
      for (int ks2 = 0; ks2 < 2; ++ks2) {
        half8_t va[MD];
#pragma unroll
        for (int md = 0; md < MD; ++md) {
          const int kA = 32 * ks2 + 4 * grp + tr_j;
          const int kB = kA + 16;
          const int fch = 2 * md + (tr_q >> 1);
          const uint8_t* vt = f16t + VF16;
          const short4_t ra = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
              (__attribute__((address_space(3))) short4_t*)(vt + kA * FROW + kf_swz(fch, kA) * 16 + (tr_q & 1) * 8));
          const short4_t rb = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
              (__attribute__((address_space(3))) short4_t*)(vt + kB * FROW + kf_swz(fch, kB) * 16 + (tr_q & 1) * 8));
          va[md] = __builtin_shufflevector(__builtin_bit_cast(half4_t, ra), __builtin_bit_cast(half4_t, rb),
                                           0, 1, 2, 3, 4, 5, 6, 7);
        }
#pragma unroll
        for (int md = 0; md < MD; ++md)
#pragma unroll
          for (int nt = 0; nt < NT; ++nt)
            st.o[md][nt] = __builtin_amdgcn_mfma_f32_16x16x32_f16(va[md], pb[ks2][nt], st.o[md][nt], 0, 0, 0);
      }
      __builtin_amdgcn_s_setprio(0);
      continue;
    }

    // ---- S^T = K Q^T: 4 x NT independent accumulator chains ----
    float4_t s[4][NT];
    if constexpr (I8QK) {
      int4_t acc[4][3][NT];
#pragma unroll
      for (int mt = 0; mt < 4; ++mt)
#pragma unroll
        for (int k = 0; k < 3; ++k)
#pragma unroll
          for (int nt = 0; nt < NT; ++nt) acc[mt][k][nt] = int4_t{0, 0, 0, 0};
#pragma unroll
      for (int sp = 0; sp < KPAIRS; ++sp) {
        int4_t raw[4];
#pragma unroll
        for (int mt = 0; mt < 4; ++mt) {
          const int row = mt * 16 + l16;
          raw[mt] = *(const int4_t*)(ks + row * KROW + swz<KROW>(4 * sp + grp, row) * 16);
        }
#pragma unroll
        for (int mt = 0; mt < 4; ++mt) qk_i8_step<NT>(raw[mt], q.qd[sp], acc[mt]);
      }
#pragma unroll
      for (int mt = 0; mt < 4; ++mt)
#pragma unroll
        for (int nt = 0; nt < NT; ++nt) s[mt][nt] = s_from_i8(acc[mt][0][nt], acc[mt][1][nt], acc[mt][2][nt]);
    } else {
#pragma unroll
    for (int mt = 0; mt < 4; ++mt)
#pragma unroll
      for (int nt = 0; nt < NT; ++nt) s[mt][nt] = float4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int sp = 0; sp < KPAIRS; ++sp) {
      uint4_t raw[4];
#pragma unroll
      for (int mt = 0; mt < 4; ++mt) {
        const int row = mt * 16 + l16;
        raw[mt] = *(const uint4_t*)(ks + row * KROW + swz<KROW>(4 * sp + grp, row) * 16);
      }
#pragma unroll
      for (int hk = 0; hk < 2; ++hk) {
        half8_t a[4];
#pragma unroll
        for (int mt = 0; mt < 4; ++mt) a[mt] = bytes8_to_f16<FP8>(raw[mt][2 * hk], raw[mt][2 * hk + 1]);
#pragma unroll
        for (int mt = 0; mt < 4; ++mt)
#pragma unroll
          for (int nt = 0; nt < NT; ++nt)
            s[mt][nt] = __builtin_amdgcn_mfma_f32_16x16x32_f16(a[mt], q.hi[nt][2 * sp + hk], s[mt][nt], 0, 0, 0);
        if constexpr (HILO) {
#pragma unroll
          for (int mt = 0; mt < 4; ++mt)
#pragma unroll
            for (int nt = 0; nt < NT; ++nt)
              s[mt][nt] = __builtin_amdgcn_mfma_f32_16x16x32_f16(a[mt], q.lo[nt][2 * sp + hk], s[mt][nt], 0, 0, 0);
        }
      }
    }

    }

    half8_t pb[2][NT];
    softmax_tile<NT, MD, QT, TREE>(p, u, kbase, grp, q, s, st, pb, tb);
    pv_tile<FP8, NT, MD, VROW>(vs, lane, pb, st);
  }

  float4_t vsc[MD];
  load_v_scales<DV>(p, g, lane, vsc);
  write_rows<DV, NT>(p, u, g, u.c, lane, KV_OFF, q, st, vsc);

}

// ------------------------------------------------------------ tile loaders --
//
// The page-table-driven KV loads of the attention kernels, as reusable parts:
// the attention kernels, the debug gather (pa_gather_debug) and the read probe
// (pa_kv_read_probe) all run these same functions, so the byte-exact gather
// test covers the address code the kernels execute.
//
// RegTileLoader: the decode kernel's loader.  A 64-key tile of one KV head
// arrives in registers by row-coalesced 16-byte loads (lane l reads row
// RPL*j + l / CPR, chunk l % CPR), with the non-temporal hint.  Page ids come
// from a 64-entry register window (lane l holds the page of page index
// pw_base + l), refilled with a load that waits for itself.  With pages of at
// least 64 keys a full tile lies in one page: its base is computed once and
// every lane adds a fixed offset (the fast path); otherwise, and for the
// tile that ends the range, each row goes through paged_row with its key
// clamped to the range's last key, so no byte past it is read.  Table entries
// past the last key's page are never read.
template <int D>
struct RegTileLoader {
  static constexpr int CPR = D / 16;     // 16-byte chunks per row
  static constexpr int RPL = 64 / CPR;   // rows per 1 KB wave load
  static constexpr int NLD = TK / RPL;   // loads per tile (K or V)
  const int32_t* table_row;
  int g, kv_lo, key_end, last_page, page_shift;
  int pw_base, pw_val;
  int ld_row, ld_chunk;
  int64_t k_lane, v_lane;
  bool one_page;

  __device__ __forceinline__ void init(const AttnParams& p, int b, int g_, int kv_lo_, int key_end_, int n_tiles,
                                       int lane) {
    table_row = p.block_table + (int64_t)b * p.max_pages_per_seq;
    g = g_;
    kv_lo = kv_lo_;
    key_end = key_end_;
    page_shift = p.page_shift;
    last_page = n_tiles > 0 ? (key_end - 1) >> page_shift : 0;   // never read past it
    pw_base = kv_lo >> page_shift;
    pw_val = table_row[min(pw_base + lane, last_page)];
    one_page = page_shift >= 6;
    ld_row = lane / CPR;
    ld_chunk = lane % CPR;
    k_lane = (int64_t)ld_row * p.k_stride_token + 16 * ld_chunk;
    v_lane = (int64_t)ld_row * p.v_stride_token + 16 * ld_chunk;
  }

  // Tile `tile` of the range into kr / vr (rows RPL*j + ld_row, chunk ld_chunk).
  __device__ __forceinline__ void load(const AttnParams& p, int tile, uint4_t (&kr)[NLD], uint4_t (&vr)[NLD]) {
    const int kbase = kv_lo + tile * TK;
    const int pg0 = kbase >> page_shift;
    const int pg_last = min(pg0 + 3, last_page);
    if (pg0 < pw_base || pg_last > pw_base + 63) {
      pw_base = pg0;
      pw_val = load_i32_sync(table_row + min(pg0 + (int)(threadIdx.x & 63), last_page));  // waits here, not at a join
    }
    const int pp0 = __builtin_amdgcn_readlane(pw_val, pg0 - pw_base);
    if (one_page && kbase + TK <= key_end) {
      const uint8_t* kb = paged_row(p.k_cache, pp0, kbase, page_shift, g, p.k_stride_page, p.k_stride_head,
                                    p.k_stride_token);
      const uint8_t* vb = paged_row(p.v_cache, pp0, kbase, page_shift, g, p.v_stride_page, p.v_stride_head,
                                    p.v_stride_token);
#pragma unroll
      for (int j = 0; j < NLD; ++j) {
        kr[j] = stream_load16(kb + (int64_t)(RPL * j) * p.k_stride_token + k_lane);
        vr[j] = stream_load16(vb + (int64_t)(RPL * j) * p.v_stride_token + v_lane);
      }
    } else {
      int pp1 = pp0, pp2 = pp0, pp3 = pp0;
      if (!one_page) {
        pp1 = __builtin_amdgcn_readlane(pw_val, min(pg0 + 1, pg_last) - pw_base);
        pp2 = __builtin_amdgcn_readlane(pw_val, min(pg0 + 2, pg_last) - pw_base);
        pp3 = __builtin_amdgcn_readlane(pw_val, pg_last - pw_base);
      }
#pragma unroll
      for (int j = 0; j < NLD; ++j) {
        const int key = min(kbase + RPL * j + ld_row, key_end - 1);
        const int page = pick_page(key, page_shift, pg0, pp0, pp1, pp2, pp3);
        kr[j] = stream_load16(paged_row(p.k_cache, page, key, page_shift, g, p.k_stride_page,
                                        p.k_stride_head, p.k_stride_token) + 16 * ld_chunk);
        vr[j] = stream_load16(paged_row(p.v_cache, page, key, page_shift, g, p.v_stride_page,
                                        p.v_stride_head, p.v_stride_token) + 16 * ld_chunk);
      }
    }
  }
};

// -------------------------------------------------------- decode attention --
//
// KS waves per unit: wave w takes tiles w, w + KS, ... of the unit's key range
// and the waves merge their softmax states through LDS at the end, so a unit
// of n tiles finishes in about n / KS tile times (short units fill the tail of
// the dispatch).  KV tiles are staged in registers with plain, row-coalesced
// global loads (the compiler tracks their completion).  At the top of each
// iteration the arrived tile is written to the wave's LDS tile and the same
// registers immediately take the next tile, so every load has a whole
// iteration to arrive while the register file, not LDS, holds the bytes in
// flight.  K is then read back in the MFMA A-operand layout, V transposed.

// LDS of one decode workgroup (KS waves).
template <int D, int NT, int KS, bool TREE>
struct DecodeLds {
  __attribute__((aligned(1024))) uint8_t kv[KS][2][TK * D];   // per wave: K tile, V tile
  float vscale[D];
  float mrg_m[KS][16 * NT], mrg_l[KS][16 * NT];
  uint32_t tree[TREE ? NT * 32 : 1];   // tree kernels run one wave per unit
};

// One decode unit u of (request b, KV head g), computed by the KS waves of the
// workgroup (wave wv takes tiles wv, wv + KS, ...), written as final rows or
// as the chunk's partial (merged in-kernel by the unit that finishes the row
// tile last when p.merge_count is set).
template <int D, bool FP8, int NT, bool HILO, int KS, bool TREE>
__device__ __forceinline__ void decode_unit(const AttnParams& p, int b, int g, const Unit& u, int lane, int wv,
                                            DecodeLds<D, NT, KS, TREE>& sm) {
  constexpr int KPAIRS = D / 64;
  constexpr int MD = D / 16;
  constexpr int RPL = RegTileLoader<D>::RPL;   // rows per 1 KB wave load
  constexpr int NLD = RegTileLoader<D>::NLD;   // loads per tile (K or V)
  constexpr float KV_OFF = FP8 ? 0.f : 1152.f;
  auto& kvlds = sm.kv;
  float* const vscale_lds = sm.vscale;
  auto& mrg_m = sm.mrg_m;
  auto& mrg_l = sm.mrg_l;
  uint8_t* const ktile = kvlds[wv][0];
  uint8_t* const vtile = kvlds[wv][1];
  const int l16 = lane & 15;
  const int grp = lane >> 4;
  const int c = u.c;
  const int kv_lo = u.kv_lo, n_tiles = u.n_tiles;
  RegTileLoader<D> ld;
  ld.init(p, b, g, kv_lo, u.key_end, n_tiles, lane);
  uint4_t kr[RegTileLoader<D>::NLD];   // K row RPL*j + ld_row, chunk ld_chunk
  uint4_t vr[RegTileLoader<D>::NLD];   // V rows, same places
  const int ld_row = ld.ld_row, ld_chunk = ld.ld_chunk;
  auto load_tile = [&](int tile) { ld.load(p, tile, kr, vr); };

  SoftmaxState<NT, MD> st;
  softmax_init(st);
  // int8 caches use the int8 MFMA for S^T (QRowsI8); fp8 caches the f16 one
  using QT = typename std::conditional<FP8, QRows<D, NT, HILO>, QRowsI8<D, NT>>::type;
  if (n_tiles == 0) {
    // No visible key in this unit: (0, -inf) rows, written by wave 0.
    if (wv > 0) return;
    QT q;
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) {
      const int r = u.row0 + nt * 16 + l16;
      q.ok[nt] = r < u.rows_total;
      q.tok[nt] = q.ok[nt] ? r / u.G : 0;
      q.head[nt] = g * u.G + (q.ok[nt] ? r % u.G : 0);
    }
    float4_t vsc[MD];
#pragma unroll
    for (int md = 0; md < MD; ++md) vsc[md] = float4_t{0.f, 0.f, 0.f, 0.f};
    write_rows<D, NT>(p, u, g, c, lane, KV_OFF, q, st, vsc);
    merge_if_last<D, 16 * NT>(p, u, b, g, lane);
    return;
  }

  // Query (and its scales) first: it arrives before the first tile, so it is
  // processed while that tile is still in flight.  Every wave loads a valid
  // first tile (a surplus wave of a short unit loads the last one and skips
  // it), so no path skips the load and the wait counts stay exact.
  QRaw<D, NT> qraw;
  query_fetch<D, NT>(p, u, g, u.row0, lane, qraw);
  const bool fold_channel = p.scale_mode == PA_SCALE_PER_CHANNEL;
  float vs_lane[D / 64];   // per-channel V scales (other modes re-read the first one)
#pragma unroll
  for (int i = 0; i < D / 64; ++i) vs_lane[i] = p.v_scale[fold_channel ? (int64_t)g * D + lane + 64 * i : 0];
  uint32_t* const tb = sm.tree;
  if constexpr (TREE) load_tree_bits<NT>(p, b, u, u.row0, lane, tb);
  load_tile(min(wv, n_tiles - 1));
  QT q;
  if constexpr (FP8) query_finish<D, NT, HILO>(p, u, g, u.row0, lane, KV_OFF, qraw, q);
  else query_finish_i8<D, NT>(p, u, g, u.row0, lane, qraw, q);

  for (int it = wv; it < n_tiles; it += KS) {
    const int kbase = kv_lo + it * TK;
    // tile `it` -> LDS (swizzled rows); its registers take tile it + 1
#pragma unroll
    for (int j = 0; j < NLD; ++j) {
      const int row = RPL * j + ld_row;
      *(uint4_t*)(ktile + row * D + swz<D>(ld_chunk, row) * 16) = kr[j];
      *(uint4_t*)(vtile + row * D + swz<D>(ld_chunk, row) * 16) = vr[j];
    }
    if (it + KS < n_tiles) load_tile(it + KS);

    // ---- S^T = K Q^T: 4 x NT independent accumulator chains ----
    float4_t s[4][NT];
    if constexpr (!FP8) {
      int4_t acc[4][3][NT];
#pragma unroll
      for (int mt = 0; mt < 4; ++mt)
#pragma unroll
        for (int k = 0; k < 3; ++k)
#pragma unroll
          for (int nt = 0; nt < NT; ++nt) acc[mt][k][nt] = int4_t{0, 0, 0, 0};
#pragma unroll
      for (int sp = 0; sp < KPAIRS; ++sp) {
        int4_t raw[4];
#pragma unroll
        for (int mt = 0; mt < 4; ++mt) {
          const int row = mt * 16 + l16;
          raw[mt] = *(const int4_t*)(ktile + row * D + swz<D>(4 * sp + grp, row) * 16);
        }
#pragma unroll
        for (int mt = 0; mt < 4; ++mt) qk_i8_step<NT>(raw[mt], q.qd[sp], acc[mt]);
      }
#pragma unroll
      for (int mt = 0; mt < 4; ++mt)
#pragma unroll
        for (int nt = 0; nt < NT; ++nt) s[mt][nt] = s_from_i8(acc[mt][0][nt], acc[mt][1][nt], acc[mt][2][nt]);
    } else {
#pragma unroll
    for (int mt = 0; mt < 4; ++mt)
#pragma unroll
      for (int nt = 0; nt < NT; ++nt) s[mt][nt] = float4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int sp = 0; sp < KPAIRS; ++sp) {
      uint4_t raw[4];
#pragma unroll
      for (int mt = 0; mt < 4; ++mt) {
        const int row = mt * 16 + l16;
        raw[mt] = *(const uint4_t*)(ktile + row * D + swz<D>(4 * sp + grp, row) * 16);
      }
#pragma unroll
      for (int hk = 0; hk < 2; ++hk) {
        half8_t a[4];
#pragma unroll
        for (int mt = 0; mt < 4; ++mt) a[mt] = bytes8_to_f16<FP8>(raw[mt][2 * hk], raw[mt][2 * hk + 1]);
#pragma unroll
        for (int mt = 0; mt < 4; ++mt)
#pragma unroll
          for (int nt = 0; nt < NT; ++nt)
            s[mt][nt] = __builtin_amdgcn_mfma_f32_16x16x32_f16(a[mt], q.hi[nt][2 * sp + hk], s[mt][nt], 0, 0, 0);
        if constexpr (HILO) {
#pragma unroll
          for (int mt = 0; mt < 4; ++mt)
#pragma unroll
            for (int nt = 0; nt < NT; ++nt)
              s[mt][nt] = __builtin_amdgcn_mfma_f32_16x16x32_f16(a[mt], q.lo[nt][2 * sp + hk], s[mt][nt], 0, 0, 0);
        }
      }
    }

    }

    half8_t pb[2][NT];
    softmax_tile<NT, MD, QT, TREE>(p, u, kbase, grp, q, s, st, pb, tb);
    pv_tile<FP8, NT, MD, D>(vtile, lane, pb, st);
  }

  if (fold_channel && wv == 0) {
#pragma unroll
    for (int i = 0; i < D / 64; ++i) vscale_lds[lane + 64 * i] = vs_lane[i];
  }

  if constexpr (KS > 1) {
    // Merge the KS partial states of the unit: common reference max M per row,
    // each wave's (O, l) weighted by 2^(m_w - M); wave 0 sums and writes.
    float lt[NT];
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) {
      lt[nt] = row_sum4(st.l[nt]);
      if (grp == 0) {
        mrg_m[wv][nt * 16 + l16] = st.m[nt];
        mrg_l[wv][nt * 16 + l16] = lt[nt];
      }
    }
    __syncthreads();  // also: every wave is done with its K/V tiles
    float f[NT];
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) {
      float mm = -INFINITY;
#pragma unroll
      for (int w = 0; w < KS; ++w) mm = fmaxf(mm, mrg_m[w][nt * 16 + l16]);
      float lsum = 0.f;
#pragma unroll
      for (int w = 0; w < KS; ++w) {
        const float mw = mrg_m[w][nt * 16 + l16];
        lsum += mw == -INFINITY ? 0.f : mrg_l[w][nt * 16 + l16] * __builtin_amdgcn_exp2f(mw - mm);
      }
      f[nt] = st.m[nt] == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(st.m[nt] - mm);
      st.m[nt] = mm;
      st.l[nt] = grp == 0 ? lsum : 0.f;   // write_rows sums the four lane groups
    }
    // O of wave w > 0 -> its own K/V tile area (lane-major float4s)
    float4_t* obuf = (float4_t*)kvlds[wv][0];
    if (wv > 0) {
#pragma unroll
      for (int md = 0; md < MD; ++md)
#pragma unroll
        for (int nt = 0; nt < NT; ++nt) obuf[(md * NT + nt) * 64 + lane] = st.o[md][nt] * f[nt];
    }
    __syncthreads();
    if (wv > 0) return;
#pragma unroll
    for (int md = 0; md < MD; ++md)
#pragma unroll
      for (int nt = 0; nt < NT; ++nt) {
        float4_t acc = st.o[md][nt] * f[nt];
#pragma unroll
        for (int w = 1; w < KS; ++w) acc += ((const float4_t*)kvlds[w][0])[(md * NT + nt) * 64 + lane];
        st.o[md][nt] = acc;
      }
  }

  float4_t vsc[MD];
  if (fold_channel) {
#pragma unroll
    for (int md = 0; md < MD; ++md) vsc[md] = *(const float4_t*)(vscale_lds + md * 16 + grp * 4);
  } else {
    load_v_scales<D>(p, g, lane, vsc);
  }
  write_rows<D, NT>(p, u, g, c, lane, KV_OFF, q, st, vsc);
  merge_if_last<D, 16 * NT>(p, u, b, g, lane);   // wave 0 alone is left when KS > 1
}

template <int D, bool FP8, int NT, bool HILO, int KS, bool TREE>
__global__ __launch_bounds__(64 * KS, NT == 1 ? 2 : 1) void paged_decode_kernel(AttnParams p) {
  __shared__ DecodeLds<D, NT, KS, TREE> sm;
  const int lane = threadIdx.x & 63;
  const int wv = KS > 1 ? __builtin_amdgcn_readfirstlane((int)threadIdx.x >> 6) : 0;
  // grid = (B * H_kv, row tiles, chunks): chunk-major, so the empty units of
  // short requests (chunks past their length) are dispatched last
  const int b = (int)blockIdx.x / p.num_kv_heads;
  const int g = (int)blockIdx.x % p.num_kv_heads;
  const int rt = p.row_tiles - 1 - (int)blockIdx.y;  // long (late-token) row tiles first
  const int c = (int)blockIdx.z;
  Unit u;
  if (!unit_setup<16 * NT>(p, b, rt, c, u)) return;
  decode_unit<D, FP8, NT, HILO, KS, TREE>(p, b, g, u, lane, wv, sm);
}

// ------------------------------------------------ persistent decode (F-3) --
//
// After FlashInfer persistent.cuh (BlockBatchPagedAttentionPersistent walks a
// per-CTA work list of (request, head, KV range) items; the partial states of
// each row are then reduced): a grid of exactly the resident wave capacity,
// each workgroup one wave, walks an equal share of all KV tiles.  The
// (request b, KV head g) segments are laid end to end in 64-key tiles:
// segment (b, g) is tiles [S_b + g t_b, S_b + (g + 1) t_b) with t_b =
// ceil(T_b / 64) and S_b = H_kv sum_{b' < b} t_b'.  Of the N tiles, wave w
// takes [start(w), start(w + 1)) with start(w) = floor(w N / W); W = the
// smaller of the grid and N / floor (floor = chunk_size / 64 tiles, the
// shortest share), so the starts strictly increase.  A wave's share is cut
// at segment ends into pieces; piece k of segment s is its k-th piece in tile
// order, k = #{w : a_s < start(w) <= x} for a piece starting at tile x of a
// segment starting at a_s, and segment s has 1 + #{w : a_s < start(w) <= e_s
// - 1} pieces.  The planner runs in every wave from the lengths (no host
// plan, no device-to-host copy); each piece is a decode unit whose partial
// goes to slot k, and the wave finishing a segment's last piece merges it
// (the in-kernel merge), so the call is one launch with no grid barrier.
struct PersistentPlan {
  int n;   // tiles of all segments (< 2^31, checked by the host)
  int w;   // waves that take a share (<= gridDim.x, <= n)
  __device__ __forceinline__ int start(int v) const { return (int)((int64_t)v * n / w); }
  // waves whose start is at or before tile x (0 <= x < n)
  __device__ __forceinline__ int count(int x) const {
    return (int)min((int64_t)w, (((int64_t)x + 1) * w + n - 1) / n);
  }
};

// The wave's walk through its share, kept in LDS between pieces (the decode
// unit's body needs every register): the request block b0 .. b0 + 63 (lane l:
// tiles t of request b0 + l and the inclusive prefix of H_kv * t over the
// block, `base` = the tiles before b0), the next tile x and the share's end.
struct PersistentLds {
  int t[64], incl[64];
  int b0, base, x, x_end;
};

// Loads the request block starting at b0 (lane-parallel prefix sum).
__device__ __forceinline__ int seg_block(const AttnParams& p, int b0, int lane, int& t, int& incl) {
  const int bb = b0 + lane;
  const int n = p.q_len_uniform;
  t = bb < p.batch && n > 0 ? (p.seq_lens_kv[bb] + n + TK - 1) / TK : 0;
  incl = t * p.num_kv_heads;
#pragma unroll
  for (int d = 1; d < 64; d <<= 1) {
    const int v = __shfl_up(incl, d, 64);
    if (lane >= d) incl += v;
  }
  return __builtin_amdgcn_readlane(incl, 63);   // the block's tiles
}

template <int D, bool FP8, int NT, bool HILO>
__global__ __launch_bounds__(64, NT == 1 ? 2 : 1) void paged_decode_persistent_kernel(AttnParams p) {
  __shared__ DecodeLds<D, NT, 1, false> sm;
  __shared__ PersistentLds pl;
  const int lane = threadIdx.x & 63;
  const int H = p.num_kv_heads;
  // total tiles (every wave computes the same sum)
  int n_all = 0;
  for (int b0 = 0; b0 < p.batch; b0 += 64) {
    int t, incl;
    n_all += seg_block(p, b0, lane, t, incl);
  }
  const int floor_tiles = max(1, p.chunk_size / TK);
  PersistentPlan plan;
  plan.n = n_all;
  plan.w = min((int)gridDim.x, max(1, n_all / floor_tiles));
  const int me = (int)blockIdx.x;
  if (me >= plan.w || n_all == 0) return;
  {
    // the request block holding the share's first tile
    const int x0 = plan.start(me);
    int base = 0, b0 = 0, t = 0, incl = 0;
    for (;; b0 += 64) {
      const int tot = seg_block(p, b0, lane, t, incl);
      if (x0 < base + tot || b0 + 64 >= p.batch) break;
      base += tot;
    }
    pl.t[lane] = t;
    pl.incl[lane] = incl;
    if (lane == 0) {
      pl.b0 = b0;
      pl.base = base;
      pl.x = x0;
      pl.x_end = plan.start(me + 1);
    }
  }
  for (;;) {
    // the state comes back from LDS after every piece (nothing kept live
    // across the unit's body)
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    asm volatile("" ::: "memory");
    const int x = pl.x, x_end = pl.x_end;
    if (x >= x_end) break;
    const int base = pl.base;
    const uint64_t hit = __ballot(base + pl.incl[lane] > x);
    if (hit == 0) {   // past this block: the next one
      int t, incl;
      const int tot = __builtin_amdgcn_readlane(pl.incl[lane], 63);
      seg_block(p, pl.b0 + 64, lane, t, incl);
      pl.t[lane] = t;
      pl.incl[lane] = incl;
      if (lane == 0) {
        pl.b0 += 64;
        pl.base = base + tot;
      }
      continue;
    }
    const int lb = (int)__builtin_ctzll(hit);
    const int b = pl.b0 + lb;
    const int t_b = __builtin_amdgcn_readlane(pl.t[lane], lb);
    const int s_b = base + __builtin_amdgcn_readlane(pl.incl[lane], lb) - t_b * H;
    const int g = (x - s_b) / t_b;
    const int a = s_b + g * t_b;   // the segment is tiles [a, a + t_b)
    const int piece_end = min(a + t_b, x_end);
    if (lane == 0) pl.x = piece_end;
    Unit u;
    u.n = p.q_len_uniform;
    u.tok0 = b * u.n;
    u.G = p.group;
    u.rows_total = u.n * u.G;
    u.row0 = 0;
    u.L = p.seq_lens_kv[b];
    u.T = u.L + u.n;
    u.c = plan.count(x) - plan.count(a);
    u.n_chunks = 1 + plan.count(a + t_b - 1) - plan.count(a);
    u.split = u.n_chunks > 1;
    u.kv_lo = (x - a) * TK;
    u.kv_hi = min(u.T, (piece_end - a) * TK);
    u.key_end = p.causal ? min(u.kv_hi, u.L + u.n) : u.kv_hi;   // the last token sees every key
    u.mask_from = p.causal ? min(u.kv_hi, u.L + 1) : u.kv_hi;
    u.n_tiles = u.key_end > u.kv_lo ? (u.key_end - u.kv_lo + TK - 1) / TK : 0;
    decode_unit<D, FP8, NT, HILO, 1, false>(p, b, g, u, lane, 0, sm);
  }
}

// ------------------------------------------------------- MLA latent decode --
//
// Shared 576/512 latent rows (V = first 512 bytes of each K row), one KV head,
// 64 packed query rows (64 of the request's query heads) per workgroup, one
// workgroup per CU.  Raw K tiles arrive by LDS DMA and are never converted as
// a whole: S^T = K Q^T takes the K bytes on the fp8 or int8 MFMA as they are
// (the query in fp8 or int8 digits), and PV converts the V^T operands in
// registers after the 8-bit LDS transpose read.

constexpr int MLA_WAVES = 4;  // waves of the four-wave MLA kernel

// MLA, int8 caches: four waves.  The raw 64 x 576 tile arrives by LDS DMA
// into a three-stage ring (two tiles ahead).  Phase A (wave w, rows
// 16w..16w+15) feeds the raw K bytes to the int8 MFMA as they are, against
// three int8 digits of the query (QRowsI8: fp32 queries and per-channel K
// scales need nothing more).  The softmax writes P^T and the per-row rescale
// factors to LDS.  Phase B (wave w, output dims 128w..128w+127 of all 64 rows)
// reads V^T from the same raw rows with the 8-bit LDS transpose read and
// converts it in registers (int8 V as the offset value 1152 + x, removed in
// the epilogue).  Two barriers per tile: the tile has landed for every wave
// (and the stage two tiles back is free again), then P^T is complete.
template <bool BAL>
__global__ __launch_bounds__(MLA_WAVES * 64, 1) void paged_mla_i8_kernel(AttnParams p) {
  constexpr int DQK = 576, DV = 512, NW = MLA_WAVES;
  constexpr int ROWS = 16 * NW;                   // 64 packed rows per workgroup
  constexpr int NTB = ROWS / 16;                  // row tiles in phase B
  constexpr int MDW = DV / 16 / NW;               // output-dim tiles per wave (8)
  constexpr int KROW = DQK;
  constexpr int KTILE = TK * KROW;                // 36 KB raw tile
  constexpr int NSTAGE = 3;
  constexpr int SP = DQK / 64;                    // 64-dim steps of S^T (9)
  constexpr float KV_OFF = 1152.f;                // int8 V operands carry 1152 + x
  using LD = DmaTileLoader<KROW, KROW, NW, true>;
  static_assert(LD::KCH % (64 * NW) == 0, "every wave issues the same number of DMA blocks");
  constexpr int DMA_W = LD::K_DMA;                // per wave per tile

  __shared__ __attribute__((aligned(1024))) uint8_t kst[NSTAGE * KTILE];   // raw tiles
  __shared__ __attribute__((aligned(16))) half8_t pt_lds[NTB * 2 * 64];    // P^T operands
  __shared__ float alpha_lds[ROWS];
  __shared__ float lrow_lds[ROWS];

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane((int)threadIdx.x >> 6);
  const int l16 = lane & 15;
  const int grp = lane >> 4;
  int b, g;
  Unit u;
  if (!shared_tile_unit<ROWS, BAL>(p, b, g, u)) return;   // a chunk's row tiles share an XCD
  const int kv_lo = u.kv_lo, n_tiles = u.n_tiles;
  LD ld;
  ld.init(p, b, g, wave, kv_lo, u.key_end, n_tiles, lane, lds_addr(kst));
#pragma unroll
  for (int st = 0; st < NSTAGE - 1; ++st)
    if (st < n_tiles) ld.issue(p, st, st);

  // S^T on the int8 MFMA: K bytes go to the MFMA as they are stored
  QRowsI8<DQK, 1> q;
  load_query_i8<DQK>(p, u, g, u.row0 + wave * 16, lane, q);
  SoftmaxState<1, 0> sa;   // phase-A row state (m, l); O lives in phase B
  softmax_init(sa);
  float4_t o[MDW][NTB];    // dims 16*(MDW*wave + md) + 4*grp + i, row 16*nt + l16
#pragma unroll
  for (int md = 0; md < MDW; ++md)
#pragma unroll
    for (int nt = 0; nt < NTB; ++nt) o[md][nt] = float4_t{0.f, 0.f, 0.f, 0.f};

  // phase A: lane reads key mt*16 + l16, chunk 4*sp + grp (dims 64sp + 16grp .. +16)
  int ka_off[4][2];   // row offset and swizzle term per key tile (swz<576> depends on key % 32)
#pragma unroll
  for (int mt = 0; mt < 4; ++mt) {
    const int key = mt * 16 + l16;
    ka_off[mt][0] = key * KROW;
    ka_off[mt][1] = key;
  }
  // phase B: the tr8 read of V^T (see pv_tile): lanes 2j, 2j+1 of a 16-lane
  // group read the halves of key row kappa(grp, j)
  const int jr = l16 >> 1, hlf = lane & 1;

  for (int it = 0; it < n_tiles; ++it) {
    const int stage = it % NSTAGE;
    // this wave's DMA of tile it + 1 may stay in flight
    if (it + 1 < n_tiles) wait_vmcnt<DMA_W>();
    else wait_vmcnt<0>();
    __syncthreads();   // X: tile it landed; every wave is done with phase B of it - 1
    if (it + NSTAGE - 1 < n_tiles) ld.issue(p, it + NSTAGE - 1, (it + NSTAGE - 1) % NSTAGE);
    const uint8_t* ks = kst + stage * KTILE;
    const int kbase = kv_lo + it * TK;

    // ---- phase A: S^T = K Q^T for this wave's rows, K bytes straight to the MFMA ----
    float4_t s[4][1];
    {
    constexpr int KSTEPS = DQK / 64;
    int4_t acc[4][3][1];
#pragma unroll
    for (int mt = 0; mt < 4; ++mt)
#pragma unroll
      for (int d = 0; d < 3; ++d) acc[mt][d][0] = int4_t{0, 0, 0, 0};
    int4_t raw[4];
#pragma unroll
    for (int mt = 0; mt < 4; ++mt) {
      const int key = mt * 16 + l16;
      raw[mt] = *(const int4_t*)(ks + key * KROW + swz<KROW>(grp, key) * 16);
    }
#pragma unroll
    for (int sp = 0; sp < KSTEPS; ++sp) {
#pragma unroll
      for (int mt = 0; mt < 4; ++mt) {
        qk_i8_step<1>(raw[mt], q.qd[sp], acc[mt]);
        if (sp + 1 < KSTEPS) {
          const int key = mt * 16 + l16;
          raw[mt] = *(const int4_t*)(ks + key * KROW + swz<KROW>(4 * (sp + 1) + grp, key) * 16);
        }
      }
    }
    // (as for fp8: per key tile, its 3 digit MFMAs, then its next read)
    __builtin_amdgcn_sched_group_barrier(0x100, 4, 0);
#pragma unroll
    for (int i = 0; i < 4 * (KSTEPS - 1); ++i) {
      __builtin_amdgcn_sched_group_barrier(0x008, 3, 0);
      __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
    }
    __builtin_amdgcn_sched_group_barrier(0x008, 12, 0);
#pragma unroll
    for (int mt = 0; mt < 4; ++mt) s[mt][0] = s_from_i8(acc[mt][0][0], acc[mt][1][0], acc[mt][2][0]);
    }
    {
      half8_t pb[2][1];
      const float m_before = sa.m[0];
      softmax_tile<1, 0>(p, u, kbase, grp, q, s, sa, pb);
      const float m_use = sa.m[0] == -INFINITY ? 0.f : sa.m[0];
      if (grp == 0) alpha_lds[wave * 16 + l16] = __builtin_amdgcn_exp2f(m_before - m_use);
      pt_lds[(wave * 2 + 0) * 64 + lane] = pb[0][0];
      pt_lds[(wave * 2 + 1) * 64 + lane] = pb[1][0];
    }
    __syncthreads();   // Y: P^T and factors ready

    // ---- phase B: O^T[128 dims of this wave][all rows] += V^T P^T ----
    {
      float al[NTB];
      bool grew = false;
#pragma unroll
      for (int nt = 0; nt < NTB; ++nt) {
        al[nt] = alpha_lds[nt * 16 + l16];
        grew |= al[nt] != 1.f;
      }
      if (__builtin_amdgcn_ballot_w64(grew) != 0) {
#pragma unroll
        for (int md = 0; md < MDW; ++md)
#pragma unroll
          for (int nt = 0; nt < NTB; ++nt) o[md][nt] *= al[nt];
      }
    }
#pragma unroll
    for (int ks2 = 0; ks2 < 2; ++ks2) {
      const int vrow = 32 * ks2 + (jr < 4 ? 4 * grp + jr : 16 + 4 * grp + (jr - 4));
      half8_t pbn[NTB];
#pragma unroll
      for (int nt = 0; nt < NTB; ++nt) pbn[nt] = pt_lds[(nt * 2 + ks2) * 64 + lane];
      int2_t vraw[MDW];
#pragma unroll
      for (int md = 0; md < MDW; ++md) {
        const int chunk = wave * MDW + md;
        vraw[md] = __builtin_amdgcn_ds_read_tr8_b64_v2i32((__attribute__((address_space(3))) int2_t*)(
            ks + vrow * KROW + swz<KROW>(chunk, vrow) * 16 + hlf * 8));
      }
#pragma unroll
      for (int md = 0; md < MDW; ++md) {
        const half8_t a = bytes8_to_op<false>((uint32_t)vraw[md][0], (uint32_t)vraw[md][1]);
#pragma unroll
        for (int nt = 0; nt < NTB; ++nt)
          o[md][nt] = __builtin_amdgcn_mfma_f32_16x16x32_f16(a, pbn[nt], o[md][nt], 0, 0, 0);
      }
    }
  }

  // ---- epilogue: row sums and lse from the owner waves, outputs per dim slice ----
  const int H_q = p.num_q_heads;
  {
    const float lt = row_sum4(sa.l[0]);
    const float lse_nat = lt > 0.f ? (sa.m[0] + __log2f(lt)) * LN2F : -INFINITY;
    if (grp == 0) lrow_lds[wave * 16 + l16] = lt;
    if (grp == 0 && q.ok[0]) {
      const int tok = u.tok0 + q.tok[0];
      if (u.split) p.part_lse[((int64_t)tok * p.max_chunks + u.c) * H_q + q.head[0]] = lse_nat;
      else if (p.lse) p.lse[(int64_t)tok * H_q + q.head[0]] = lse_nat;
    }
  }
  __syncthreads();
  const int mode = p.scale_mode;
  float4_t vsc[MDW];
  if (mode == PA_SCALE_PER_CHANNEL) {
#pragma unroll
    for (int md = 0; md < MDW; ++md)
      vsc[md] = *(const float4_t*)(p.v_scale + (int64_t)g * DV + (wave * MDW + md) * 16 + grp * 4);
  } else {
    const float v = p.v_scale[mode == PA_SCALE_PER_HEAD ? g : 0];
#pragma unroll
    for (int md = 0; md < MDW; ++md) vsc[md] = float4_t{v, v, v, v};
  }
#pragma unroll
  for (int nt = 0; nt < NTB; ++nt) {
    const int r = u.row0 + nt * 16 + l16;
    if (r >= u.rows_total) continue;
    const float lt = lrow_lds[nt * 16 + l16];
    const float inv = lt > 0.f ? 1.f / lt : 0.f;
    const float off = lt > 0.f ? KV_OFF : 0.f;
    const int tok = u.tok0 + r / u.G;
    const int h = g * u.G + r % u.G;
    float* prow = u.split ? p.part_o + (((int64_t)tok * p.max_chunks + u.c) * H_q + h) * DV : nullptr;
    uint16_t* orow = p.out + ((int64_t)tok * H_q + h) * DV;
#pragma unroll
    for (int md = 0; md < MDW; ++md) {
      const int d = (wave * MDW + md) * 16 + grp * 4;
      float4_t v;
#pragma unroll
      for (int i = 0; i < 4; ++i) v[i] = fmaf(o[md][nt][i], inv, -off) * vsc[md][i];
      if (u.split) {
        *(float4_t*)(prow + d) = v;
      } else {
        const uint32_t w0 = (uint32_t)f32_to_bf16(v[0]) | ((uint32_t)f32_to_bf16(v[1]) << 16);
        const uint32_t w1 = (uint32_t)f32_to_bf16(v[2]) | ((uint32_t)f32_to_bf16(v[3]) << 16);
        *(int2_t*)(orow + d) = int2_t{(int)w0, (int)w1};
      }
    }
  }
}

// MLA, producer/consumer form (e4m3fn caches; the query in two fp8 digits, or
// three when it is fp32 or carries per-channel K scales: HILO).  Eight waves,
// 64 rows, 32-key tiles, one barrier per tile.  Waves 0..3 (producers) own
// row tile w: they compute S^T for the tile's 32 keys on the fp8 MFMA (query
// in two fp8 digits), run the online softmax and write P^T and the rows'
// rescale factors to LDS.  Waves 4..7 (consumers) issue the tile DMA and wait
// for it, own output dims 128 (w - 4) .. +127 of all 64 rows and accumulate
// O^T += V^T P^T for the tile the producers finished in the previous
// iteration.  Each SIMD holds one producer and one consumer, so the MFMAs of
// one overlap the other's LDS reads, conversions and softmax instead of every
// wave passing through the same phases between barriers.  The DMA sits with
// the consumers because an issue that stalls on a full load path would hold
// back the producers' dependent QK^T chain; the consumers' 32 accumulators
// are independent (measured 129-133 against 134-135 us on the MLA workload).
// Iteration j: producers handle tile j (j < n), consumers tile j - 1 (j > 0).
// The barrier that opens iteration j says: tile j has landed, P^T of tile
// j - 1 is written, and the consumers are done with tile j - 2, whose stage
// then takes the DMA of tile j + NSTAGE - 2.
constexpr int MLAPC_WAVES = 8;
constexpr int MLAPC_TK = 32;       // keys per tile
constexpr int MLAPC_NSTAGE = 8;    // producer's tile, consumer's tile, 6 in flight

// s_waitcnt vmcnt(n) for a wave-uniform n in [0, 31] (n > 31 waits for all).
__device__ __forceinline__ void wait_vmcnt_dyn(int n) {
#define PA_WAIT_CASE(N) \
  case N:               \
    wait_vmcnt<N>();    \
    break;
  switch (n) {
    PA_WAIT_CASE(1) PA_WAIT_CASE(2) PA_WAIT_CASE(3) PA_WAIT_CASE(4) PA_WAIT_CASE(5) PA_WAIT_CASE(6)
    PA_WAIT_CASE(7) PA_WAIT_CASE(8) PA_WAIT_CASE(9) PA_WAIT_CASE(10) PA_WAIT_CASE(11) PA_WAIT_CASE(12)
    PA_WAIT_CASE(13) PA_WAIT_CASE(14) PA_WAIT_CASE(15) PA_WAIT_CASE(16) PA_WAIT_CASE(17) PA_WAIT_CASE(18)
    PA_WAIT_CASE(19) PA_WAIT_CASE(20) PA_WAIT_CASE(21) PA_WAIT_CASE(22) PA_WAIT_CASE(23) PA_WAIT_CASE(24)
    PA_WAIT_CASE(25) PA_WAIT_CASE(26) PA_WAIT_CASE(27) PA_WAIT_CASE(28) PA_WAIT_CASE(29) PA_WAIT_CASE(30)
    PA_WAIT_CASE(31)
    default: wait_vmcnt<0>(); break;
  }
#undef PA_WAIT_CASE
}

template <bool BAL, bool HILO>
__global__ __launch_bounds__(MLAPC_WAVES * 64, 1) void paged_mla_pc_kernel(AttnParams p) {
  constexpr int DQK = 576, DV = 512;
  constexpr int ROWS = 64, NTB = ROWS / 16;      // packed rows, row tiles
  constexpr int MDC = DV / 16 / 4;                // output-dim tiles per consumer (8)
  constexpr int KROW = DQK;
  constexpr int T32 = MLAPC_TK;
  constexpr int KTILE = T32 * KROW;               // 18 KB raw tile
  constexpr int NSTAGE = MLAPC_NSTAGE;
  constexpr int ND = HILO ? 3 : 2;                // fp8 digits of the query
  constexpr int STEPS = QRowsF8<DQK, ND>::STEPS;  // 128-dim steps of S^T (5)
  using LD = DmaTileLoader<KROW, KROW, 4, true, true, T32>;
  static_assert(LD::K_DMA == 5 && LD::KCH == 18 * 64, "consumers 0, 1 issue 5 blocks per tile, 2, 3 issue 4");
  static_assert((NSTAGE - 3) * 5 <= 31, "wait_vmcnt_dyn covers the tiles in flight");

  __shared__ __attribute__((aligned(1024))) uint8_t kst[NSTAGE * KTILE];   // raw tiles
  __shared__ __attribute__((aligned(16))) half8_t pt_lds[2][NTB * 64];     // P^T operands per row tile
  __shared__ float alpha_lds[2][ROWS];
  __shared__ float lrow_lds[ROWS];

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane((int)threadIdx.x >> 6);
  const int l16 = lane & 15;
  const int grp = lane >> 4;
  int b, g;
  Unit u;
  if (!shared_tile_unit<ROWS, BAL>(p, b, g, u)) return;
  const int kv_lo = u.kv_lo;
  const int n = u.key_end > kv_lo ? (u.key_end - kv_lo + T32 - 1) / T32 : 0;
  const int H_q = p.num_q_heads;

  if (wave < 4) {
    // ------------------------------------------------------------ producer --
    const int rt = wave;
    QRowsF8<DQK, ND> q;
    load_query_f8<DQK, ND>(p, u, g, u.row0 + rt * 16, lane, q);
    float m = -INFINITY, l = 0.f;
    const half2_t ones2 = {(_Float16)1.0f, (_Float16)1.0f};
    for (int j = 0; j <= n; ++j) {
      __syncthreads();
      if (j == n) break;
      const uint8_t* ks = kst + (j % NSTAGE) * KTILE;

      float4_t s[2];
      s[0] = s[1] = float4_t{0.f, 0.f, 0.f, 0.f};
      auto read_k = [&](int st, int jb) {
        const int key = jb * 16 + l16;
        const bool live = st * 128 + 32 * grp < DQK;
        const int c0 = min(8 * st + 2 * grp, DQK / 16 - 2);
        const uint4_t a = *(const uint4_t*)(ks + key * KROW + swz<KROW>(c0, key) * 16);
        const uint4_t c = *(const uint4_t*)(ks + key * KROW + swz<KROW>(c0 + 1, key) * 16);
        v8i_t r;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          r[e] = live ? (int)a[e] : 0;
          r[4 + e] = live ? (int)c[e] : 0;
        }
        return r;
      };
      v8i_t kr[2];
      kr[0] = read_k(0, 0);
      kr[1] = read_k(0, 1);
#pragma unroll
      for (int st = 0; st < STEPS; ++st) {
#pragma unroll
        for (int jb = 0; jb < 2; ++jb) {
#pragma unroll
          for (int d = 0; d < ND; ++d)
            s[jb] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(kr[jb], q.qd[d][st], s[jb], 0, 0, 0, 127, 0,
                                                                  q.sc[st]);
          if (st + 1 < STEPS) kr[jb] = read_k(st + 1, jb);
        }
        // this step's MFMAs interleaved with the next step's operand reads
        if (st == 0) __builtin_amdgcn_sched_group_barrier(0x100, 4, 0);
        if (st + 1 < STEPS) {
#pragma unroll
          for (int i2 = 0; i2 < 2; ++i2) {
            __builtin_amdgcn_sched_group_barrier(0x008, ND, 0);
            __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
          }
        } else {
          __builtin_amdgcn_sched_group_barrier(0x008, 2 * ND, 0);
        }
        // the accumulators pass through an empty asm here, so each step's
        // MFMAs stay in their step (otherwise they sink to the softmax)
        asm volatile("" : "+v"(s[0]), "+v"(s[1]));
      }

      // online softmax of this tile's 32 keys (key of s[jb][i]: kbase + 16 jb + 4 grp + i)
      const int kbase = kv_lo + j * T32;
      if (kbase + T32 > u.mask_from) {
        const int lim = p.causal ? min(u.kv_hi, u.L + q.tok[0] + 1) : u.kv_hi;
#pragma unroll
        for (int jb = 0; jb < 2; ++jb)
#pragma unroll
          for (int i = 0; i < 4; ++i)
            if (kbase + 16 * jb + 4 * grp + i >= lim) s[jb][i] = -INFINITY;
      }
      float mx = -INFINITY;
#pragma unroll
      for (int jb = 0; jb < 2; ++jb)
#pragma unroll
        for (int i = 0; i < 4; ++i) mx = fmaxf(mx, s[jb][i]);
      mx = row_max4(mx) * q.row_mult[0];
      const float m_new = mx > m + LAZY_LOG2 ? mx : m;
      const float m_use = m_new == -INFINITY ? 0.f : m_new;
      const float alpha = __builtin_amdgcn_exp2f(m - m_use);
      m = m_new;
      half8_t pb;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        pb[i] = (_Float16)__builtin_amdgcn_exp2f(fmaf(s[0][i], q.row_mult[0], -m_use));
        pb[4 + i] = (_Float16)__builtin_amdgcn_exp2f(fmaf(s[1][i], q.row_mult[0], -m_use));
      }
      float ls = 0.f;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const half2_t pr = {pb[2 * e], pb[2 * e + 1]};
        ls = __builtin_amdgcn_fdot2(pr, ones2, ls, false);
      }
      l = l * alpha + ls;
      if (grp == 0) alpha_lds[j & 1][rt * 16 + l16] = alpha;
      pt_lds[j & 1][rt * 64 + lane] = pb;
    }
    // row sums over the four lane groups; lse
    const float lt = row_sum4(l);
    if (grp == 0) lrow_lds[rt * 16 + l16] = lt;
    const float lse_nat = lt > 0.f ? (m + __log2f(lt)) * LN2F : -INFINITY;
    if (grp == 0 && q.ok[0]) {
      const int tok = u.tok0 + q.tok[0];
      if (u.split) p.part_lse[((int64_t)tok * p.max_chunks + u.c) * H_q + q.head[0]] = lse_nat;
      else if (p.lse) p.lse[(int64_t)tok * H_q + q.head[0]] = lse_nat;
    }
    __syncthreads();   // row sums
  } else {
    // ------------------------------------------------------------ consumer --
    const int cw = wave - 4;
    float4_t o[MDC][NTB];    // dims 16 (MDC cw + md) + 4 grp + i, row 16 nt + l16
#pragma unroll
    for (int md = 0; md < MDC; ++md)
#pragma unroll
      for (int nt = 0; nt < NTB; ++nt) o[md][nt] = float4_t{0.f, 0.f, 0.f, 0.f};
    const int jr = l16 >> 1, hlf = lane & 1;
    // V^T operand rows in the key order of the P^T operand: lane group grp holds
    // keys 4 grp .. 4 grp + 3 and 16 + 4 grp .. 16 + 4 grp + 3
    const int vrow = jr < 4 ? 4 * grp + jr : 16 + 4 * grp + (jr - 4);
    LD ld;
    ld.init(p, b, g, cw, kv_lo, u.key_end, n, lane, lds_addr(kst));
#pragma unroll
    for (int st = 0; st < NSTAGE - 2; ++st)
      if (st < n) ld.issue(p, st, st);
    const int per_tile = cw < 2 ? 5 : 4;          // this wave's DMA blocks per tile
    for (int j = 0; j <= n; ++j) {
      if (j < n) wait_vmcnt_dyn(min(n - 1 - j, NSTAGE - 3) * per_tile);   // tile j landed
      __syncthreads();
      if (j + NSTAGE - 2 < n) ld.issue(p, j + NSTAGE - 2, (j + NSTAGE - 2) % NSTAGE);
      if (j == 0) continue;
      const int t = j - 1, buf = t & 1;
      const uint8_t* vs = kst + (t % NSTAGE) * KTILE;
      {
        float al[NTB];
        bool grew = false;
#pragma unroll
        for (int nt = 0; nt < NTB; ++nt) {
          al[nt] = alpha_lds[buf][nt * 16 + l16];
          grew |= al[nt] != 1.f;
        }
        if (__builtin_amdgcn_ballot_w64(grew) != 0) {
#pragma unroll
          for (int md = 0; md < MDC; ++md)
#pragma unroll
            for (int nt = 0; nt < NTB; ++nt) o[md][nt] *= al[nt];
        }
      }
      half8_t pbn[NTB];
#pragma unroll
      for (int nt = 0; nt < NTB; ++nt) pbn[nt] = pt_lds[buf][nt * 64 + lane];
#pragma unroll
      for (int md = 0; md < MDC; ++md) {
        const int chunk = cw * MDC + md;
        const int2_t vraw = __builtin_amdgcn_ds_read_tr8_b64_v2i32(
            (__attribute__((address_space(3))) int2_t*)(vs + vrow * KROW + swz<KROW>(chunk, vrow) * 16 + hlf * 8));
        const half8_t a = bytes8_to_op<true>((uint32_t)vraw[0], (uint32_t)vraw[1]);
#pragma unroll
        for (int nt = 0; nt < NTB; ++nt)
          o[md][nt] = __builtin_amdgcn_mfma_f32_16x16x32_f16(a, pbn[nt], o[md][nt], 0, 0, 0);
      }
    }
    __syncthreads();   // row sums
    const int mode = p.scale_mode;
    float4_t vsc[MDC];   // V scales of this wave's dims
    if (mode == PA_SCALE_PER_CHANNEL) {
#pragma unroll
      for (int md = 0; md < MDC; ++md)
        vsc[md] = *(const float4_t*)(p.v_scale + (int64_t)g * DV + (cw * MDC + md) * 16 + grp * 4);
    } else {
      const float v = p.v_scale[mode == PA_SCALE_PER_HEAD ? g : 0];
#pragma unroll
      for (int md = 0; md < MDC; ++md) vsc[md] = float4_t{v, v, v, v};
    }
#pragma unroll
    for (int nt = 0; nt < NTB; ++nt) {
      const int r = u.row0 + nt * 16 + l16;
      if (r >= u.rows_total) continue;
      const float lt = lrow_lds[nt * 16 + l16];
      const float inv = lt > 0.f ? 1.f / lt : 0.f;
      const int tok = u.tok0 + r / u.G;
      const int h = g * u.G + r % u.G;
      float* prow = u.split ? p.part_o + (((int64_t)tok * p.max_chunks + u.c) * H_q + h) * DV : nullptr;
      uint16_t* orow = p.out + ((int64_t)tok * H_q + h) * DV;
#pragma unroll
      for (int md = 0; md < MDC; ++md) {
        const int d = (cw * MDC + md) * 16 + grp * 4;
        float4_t v;
#pragma unroll
        for (int i = 0; i < 4; ++i) v[i] = o[md][nt][i] * inv * vsc[md][i];
        if (u.split) {
          *(float4_t*)(prow + d) = v;
        } else {
          const uint32_t w0 = (uint32_t)f32_to_bf16(v[0]) | ((uint32_t)f32_to_bf16(v[1]) << 16);
          const uint32_t w1 = (uint32_t)f32_to_bf16(v[2]) | ((uint32_t)f32_to_bf16(v[3]) << 16);
          *(int2_t*)(orow + d) = int2_t{(int)w0, (int)w1};
        }
      }
    }
  }
}

// ------------------------------------------------------------------- merge --
// One group of DV/4 lanes per (token, head) row; each lane owns 4 channels.
template <int DV>
__global__ __launch_bounds__(256) void split_merge_kernel(MergeParams p) {
  constexpr int LPR = DV / 4;
  constexpr int RPB = 256 / LPR;
  constexpr int MB = 8;   // chunk slots loaded per round trip
  const int b = blockIdx.y;
  int n, tok0;
  if (p.cu_seqlens_q) {
    tok0 = p.cu_seqlens_q[b];
    n = p.cu_seqlens_q[b + 1] - tok0;
  } else {
    n = p.q_len_uniform;
    tok0 = b * n;
  }
  const int kv_cached = p.seq_lens_kv[b];
  const int pair = blockIdx.x * RPB + (int)threadIdx.x / LPR;
  if (pair >= n * p.num_q_heads) return;
  const int t = pair / p.num_q_heads;
  const int h = pair % p.num_q_heads;
  const int lane = threadIdx.x % LPR;
  const int64_t tok = tok0 + t;
  const int64_t H = p.num_q_heads;
  const float* lrow = p.part_lse + tok * p.max_chunks * H + h;
  const float* orow = p.part_o + (tok * p.max_chunks * H + h) * DV + lane * 4;
  // One pass with a running maximum.  Slots 0 and 1, which every merged row
  // has, are loaded before the chunk count is known (with the length's load);
  // later slots go out MB at a time, only those below the count.  So a row
  // with 2 chunks costs one memory round trip and one with up to 2 + MB two,
  // and single-chunk rows (written by the attention kernel, left alone here)
  // read only two slots.  Loaded slots past the count are dropped by selects.
  RowMerge m;
  const int64_t c1 = min(1, p.max_chunks - 1);
  const float l0 = lrow[0], l1 = lrow[c1 * H];
  const float4_t o0 = *(const float4_t*)orow;
  const float4_t o1 = *(const float4_t*)(orow + c1 * H * DV);
  const int T = kv_cached + n;
  const int nc = p.item_tiles ? balanced_items(T, *p.item_tiles, p.max_chunks)
                              : min((T + p.chunk_size - 1) / p.chunk_size, p.max_chunks);
  m.add(nc > 0, l0, o0);
  m.add(nc > 1, l1, o1);
  for (int c0 = 2; c0 < nc; c0 += MB) {
    float lc[MB];
    float4_t v[MB];
#pragma unroll
    for (int k = 0; k < MB; ++k) {
      lc[k] = -INFINITY;
      v[k] = float4_t{0.f, 0.f, 0.f, 0.f};
      if (c0 + k < nc) {
        lc[k] = lrow[(int64_t)(c0 + k) * H];
        v[k] = *(const float4_t*)(orow + (int64_t)(c0 + k) * H * DV);
      }
    }
#pragma unroll
    for (int k = 0; k < MB; ++k) m.add(c0 + k < nc, lc[k], v[k]);
  }
  if (nc <= 1) return;
  m.store(p.out + (tok * H + h) * DV + lane * 4, (p.lse && lane == 0) ? p.lse + tok * H + h : nullptr);
}

// ------------------------------------------------------------ debug gather --
// grid (ceil(t_max / 4), H_kv, B), 64 threads: 16 lanes per key row, 4 rows.
__global__ __launch_bounds__(64) void gather_kernel(GatherParams p) {
  const int b = blockIdx.z, g = blockIdx.y;
  const int key = blockIdx.x * 4 + (threadIdx.x >> 4);
  const int T = p.seq_lens_kv[b] + p.q_lens[b];
  if (key >= T) return;
  const int32_t* table_row = p.block_table + (int64_t)b * p.max_pages_per_seq;
  const int page = page_of(table_row, key, p.page_shift);
  const uint8_t* src = paged_row(p.k_cache, page, key, p.page_shift, g, p.k_stride_page,
                                 p.k_stride_head, p.k_stride_token);
  uint8_t* dst = p.dst + (((int64_t)b * p.num_kv_heads + g) * p.t_max + key) * p.head_dim;
  for (int d = (threadIdx.x & 15) * 16; d < p.head_dim; d += 256)
    *(uint4_t*)(dst + d) = *(const uint4_t*)(src + d);
}

// ------------------------------------------- tile-loader gather and probe --
// Unit (b, g, c) of a tile walk: keys [kv_lo, key_end); false when empty.
__device__ __forceinline__ bool walk_unit(const TileWalkParams& w, int& b, int& g, int& kv_lo, int& key_end) {
  b = (int)blockIdx.x / w.a.num_kv_heads;
  g = (int)blockIdx.x % w.a.num_kv_heads;
  const int n = w.q_lens ? w.q_lens[b] : w.a.q_len_uniform;
  const int T = w.a.seq_lens_kv[b] + n;
  kv_lo = (int)blockIdx.z * w.chunk;
  key_end = min(T, kv_lo + w.chunk);
  return kv_lo < key_end;
}

// The decode kernel's loader, tile by tile, rows written to the gather
// destinations in key order.
template <int D>
__global__ __launch_bounds__(64) void gather_reg_kernel(TileWalkParams w) {
  using LD = RegTileLoader<D>;
  int b, g, kv_lo, key_end;
  if (!walk_unit(w, b, g, kv_lo, key_end)) return;
  const int lane = threadIdx.x & 63;
  const int n_tiles = (key_end - kv_lo + TK - 1) / TK;
  LD ld;
  ld.init(w.a, b, g, kv_lo, key_end, n_tiles, lane);
  uint4_t kr[LD::NLD], vr[LD::NLD];
  const int64_t bg = (int64_t)b * w.a.num_kv_heads + g;
  for (int it = 0; it < n_tiles; ++it) {
    ld.load(w.a, it, kr, vr);
#pragma unroll
    for (int j = 0; j < LD::NLD; ++j) {
      const int key = kv_lo + it * TK + LD::RPL * j + ld.ld_row;
      if (key < key_end) {
        const int64_t row = bg * w.t_max + key;
        if (w.k_dst) *(uint4_t*)(w.k_dst + row * D + 16 * ld.ld_chunk) = kr[j];
        if (w.v_dst) *(uint4_t*)(w.v_dst + row * D + 16 * ld.ld_chunk) = vr[j];
      }
    }
  }
}

// The shared-tile / MLA kernels' loader: each tile lands in one LDS stage by
// DMA (NW waves), then is copied out unswizzled.
template <int KROW, int VROW, int NW, bool SHARED, int TKEYS = TK>
__global__ __launch_bounds__(64 * NW) void gather_dma_kernel(TileWalkParams w) {
  using LD = DmaTileLoader<KROW, VROW, NW, SHARED, true, TKEYS>;
  __shared__ __attribute__((aligned(1024))) uint8_t stage[LD::STAGE];
  int b, g, kv_lo, key_end;
  if (!walk_unit(w, b, g, kv_lo, key_end)) return;
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane((int)threadIdx.x >> 6);
  const int n_tiles = (key_end - kv_lo + TKEYS - 1) / TKEYS;
  LD ld;
  ld.init(w.a, b, g, wave, kv_lo, key_end, n_tiles, lane, lds_addr(stage));
  const int64_t bg = (int64_t)b * w.a.num_kv_heads + g;
  for (int it = 0; it < n_tiles; ++it) {
    ld.issue(w.a, it, 0);
    wait_vmcnt<0>();
    __syncthreads();
    for (int ch = threadIdx.x; ch < LD::KCH + LD::VCH; ch += 64 * NW) {
      const bool is_k = ch < LD::KCH;
      const int c2 = is_k ? ch : ch - LD::KCH;
      const int cpr = is_k ? LD::KCPR : LD::VCPR;
      const int row = c2 / cpr, pos = c2 % cpr;
      const int key = kv_lo + it * TKEYS + row;
      if (key >= key_end) continue;
      const int off = is_k ? row * KROW + swz<KROW>(pos, row) * 16 : LD::KTILE + row * VROW + swz<VROW>(pos, row) * 16;
      const uint4_t v = *(const uint4_t*)(stage + off);
      const int64_t r = bg * w.t_max + key;
      if (is_k && w.k_dst) *(uint4_t*)(w.k_dst + r * KROW + pos * 16) = v;
      if (!is_k && w.v_dst) *(uint4_t*)(w.v_dst + r * VROW + pos * 16) = v;
    }
    __syncthreads();
  }
}

// Read probe: the decode kernel's loads and nothing else.  One tile stays in
// flight while the previous one is folded into an xor (as the kernel keeps
// one in flight while it computes).
template <int D>
__global__ __launch_bounds__(64) void read_probe_kernel(TileWalkParams w) {
  using LD = RegTileLoader<D>;
  int b, g, kv_lo, key_end;
  if (!walk_unit(w, b, g, kv_lo, key_end)) return;
  const int lane = threadIdx.x & 63;
  const int n_tiles = (key_end - kv_lo + TK - 1) / TK;
  LD ld;
  ld.init(w.a, b, g, kv_lo, key_end, n_tiles, lane);
  uint4_t kr[LD::NLD], vr[LD::NLD];
  uint4_t acc = {0u, 0u, 0u, 0u};
  ld.load(w.a, 0, kr, vr);
  for (int it = 0; it < n_tiles; ++it) {
    uint4_t x = {0u, 0u, 0u, 0u};
#pragma unroll
    for (int j = 0; j < LD::NLD; ++j) x ^= kr[j] ^ vr[j];
    if (it + 1 < n_tiles) ld.load(w.a, it + 1, kr, vr);
    acc ^= x;
  }
  uint32_t v = acc[0] ^ acc[1] ^ acc[2] ^ acc[3];
#pragma unroll
  for (int d = 1; d < 64; d <<= 1) v ^= (uint32_t)__shfl_xor((int)v, d, 64);
  if (lane == 0) w.sink[(int64_t)blockIdx.z * gridDim.x + blockIdx.x] = v;
}

// ------------------------------------------------------------------ launch --

namespace {
template <int DQK, int DV, bool FP8, int NT, int NW, bool SHARED, bool HILO, int NSTAGE, bool CONV, bool TREE>
hipError_t launch_one(const AttnParams& p, dim3 grid, hipStream_t stream) {
  hipLaunchKernelGGL((paged_attn_kernel<DQK, DV, FP8, NT, NW, SHARED, HILO, NSTAGE, CONV, TREE>), grid,
                     dim3(64 * NW), 0, stream, p);
  return hipGetLastError();
}

template <bool FP8, bool HILO>
hipError_t launch_mla(const AttnParams& p, dim3 grid, hipStream_t stream) {
  // the balanced split's planner is a variant of its own (it costs the main
  // loop SGPR spills)
  if constexpr (FP8) {   // e4m3fn keys: producer/consumer kernel
    if (p.balanced)
      hipLaunchKernelGGL((paged_mla_pc_kernel<true, HILO>), grid, dim3(MLAPC_WAVES * 64), 0, stream, p);
    else
      hipLaunchKernelGGL((paged_mla_pc_kernel<false, HILO>), grid, dim3(MLAPC_WAVES * 64), 0, stream, p);
  } else if (p.balanced) {   // int8 keys (the query's dtype and scales change nothing there)
    hipLaunchKernelGGL((paged_mla_i8_kernel<true>), grid, dim3(MLA_WAVES * 64), 0, stream, p);
  } else {
    hipLaunchKernelGGL((paged_mla_i8_kernel<false>), grid, dim3(MLA_WAVES * 64), 0, stream, p);
  }
  return hipGetLastError();
}

template <int D, bool FP8, int NT, bool HILO, int KS, bool TREE>
hipError_t launch_decode(const AttnParams& p, dim3 grid, hipStream_t stream) {
  hipLaunchKernelGGL((paged_decode_kernel<D, FP8, NT, HILO, KS, TREE>), grid, dim3(64 * KS), 0, stream, p);
  return hipGetLastError();
}

using LaunchFn = hipError_t (*)(const AttnParams&, dim3, hipStream_t);
using OccFn = int (*)();

// Workgroups of one kernel that fit on a CU at once (0 if the query fails).
template <typename K>
int occupancy_of(K kernel, int threads) {
  int n = 0;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, kernel, threads, 0) != hipSuccess) return 0;
  return n;
}
template <int DQK, int DV, bool FP8, int NT, int NW, bool SHARED, bool HILO, int NSTAGE, bool CONV, bool TREE>
int occ_one() {
  return occupancy_of(paged_attn_kernel<DQK, DV, FP8, NT, NW, SHARED, HILO, NSTAGE, CONV, TREE>, 64 * NW);
}
template <bool FP8, bool HILO>
int occ_mla() {
  if constexpr (FP8) return occupancy_of(paged_mla_pc_kernel<false, HILO>, MLAPC_WAVES * 64);
  return occupancy_of(paged_mla_i8_kernel<false>, MLA_WAVES * 64);
}
template <int D, bool FP8, int NT, bool HILO, int KS, bool TREE>
int occ_decode() {
  return occupancy_of(paged_decode_kernel<D, FP8, NT, HILO, KS, TREE>, 64 * KS);
}

template <int D, bool FP8, int NT, bool HILO>
hipError_t launch_persistent_one(const AttnParams& p, dim3 grid, hipStream_t stream) {
  hipLaunchKernelGGL((paged_decode_persistent_kernel<D, FP8, NT, HILO>), grid, dim3(64), 0, stream, p);
  return hipGetLastError();
}
template <int D, bool FP8, int NT, bool HILO>
int occ_persistent() {
  return occupancy_of(paged_decode_persistent_kernel<D, FP8, NT, HILO>, 64);
}

struct Entry {
  AttnConfig cfg;
  LaunchFn fn;
  OccFn occ;
};

// nstage == 0 marks the register-staged single-wave decode kernel.
#define PA_ENTRY_T(DQK, DV, FP8, NT, NW, SH, HL, NS, TR)                                      \
  Entry{AttnConfig{DQK, DV, FP8, SH, NT, NW, HL, NS, false, TR},                                \
        &launch_one<DQK, DV, FP8, NT, NW, SH, HL, NS, false, TR>,                               \
        &occ_one<DQK, DV, FP8, NT, NW, SH, HL, NS, false, TR>}
#define PA_ENTRY(DQK, DV, FP8, NT, NW, SH, HL, NS) PA_ENTRY_T(DQK, DV, FP8, NT, NW, SH, HL, NS, false)
#define PA_CONV(D, FP8, HL)                                                                     \
  Entry{AttnConfig{D, D, FP8, false, 2, 4, HL, 3, true, false},                                 \
        &launch_one<D, D, FP8, 2, 4, false, HL, 3, true, false>, &occ_one<D, D, FP8, 2, 4, false, HL, 3, true, false>}
// (for it, nw counts the waves that split one unit's key range)
#define PA_DEC_T(D, FP8, NT, HL, KS, TR)                                                        \
  Entry{AttnConfig{D, D, FP8, false, NT, KS, HL, 0, false, TR}, &launch_decode<D, FP8, NT, HL, KS, TR>, \
        &occ_decode<D, FP8, NT, HL, KS, TR>}
#define PA_DEC(D, FP8, NT, HL, KS) PA_DEC_T(D, FP8, NT, HL, KS, false)
// the persistent decode kernel (one wave per workgroup) is marked nstage == 4
#define PA_PERSIST(D, FP8, NT, HL)                                                              \
  Entry{AttnConfig{D, D, FP8, false, NT, 1, HL, 4, false, false}, &launch_persistent_one<D, FP8, NT, HL>, \
        &occ_persistent<D, FP8, NT, HL>}
#define PA_PERSIST_SET(D)                                                                        \
  PA_PERSIST(D, false, 1, false), PA_PERSIST(D, false, 1, true), PA_PERSIST(D, true, 1, false),     \
      PA_PERSIST(D, true, 1, true), PA_PERSIST(D, false, 2, false), PA_PERSIST(D, false, 2, true),  \
      PA_PERSIST(D, true, 2, false), PA_PERSIST(D, true, 2, true)
// the MLA kernel (4 waves and 64 rows) is marked nstage == 1
#define PA_MLA(FP8, HL) \
  Entry{AttnConfig{576, 512, FP8, true, 1, MLA_WAVES, HL, 1, false, false}, &launch_mla<FP8, HL>, &occ_mla<FP8, HL>}

#define PA_SET(D, FP8, HL)                                                                       \
  PA_DEC(D, FP8, 1, HL, 1), PA_DEC(D, FP8, 1, HL, 2), PA_DEC(D, FP8, 1, HL, 4),                    \
      PA_DEC(D, FP8, 2, HL, 1), PA_DEC(D, FP8, 2, HL, 2), PA_DEC(D, FP8, 2, HL, 4),                 \
      PA_ENTRY(D, D, FP8, 1, 3, false, HL, 2), PA_ENTRY(D, D, FP8, 1, 4, false, HL, 2)
// more than 64 rows: 2 x 4 waves on raw tiles (D = 64; D = 128 takes the f16-tile kernel)
#define PA_WIDE(D, FP8, HL) PA_ENTRY(D, D, FP8, 2, 4, false, HL, 2)
// draft-tree variants: up to 64 packed rows, one wave per decode unit
#define PA_TREE_SET(D, FP8, HL)                                                                  \
  PA_DEC_T(D, FP8, 1, HL, 1, true), PA_DEC_T(D, FP8, 2, HL, 1, true),                              \
      PA_ENTRY_T(D, D, FP8, 1, 3, false, HL, 2, true), PA_ENTRY_T(D, D, FP8, 1, 4, false, HL, 2, true)

const Entry kTable[] = {
    PA_SET(64, false, false),   PA_SET(64, false, true),
    PA_SET(64, true, false),    PA_SET(64, true, true),
    PA_WIDE(64, false, false),  PA_WIDE(64, false, true),
    PA_WIDE(64, true, false),   PA_WIDE(64, true, true),
    PA_SET(128, false, false), PA_SET(128, false, true),
    PA_SET(128, true, false),  PA_SET(128, true, true),
    PA_MLA(true, false), PA_MLA(true, true), PA_MLA(false, false), PA_MLA(false, true),
    PA_CONV(128, false, false), PA_CONV(128, false, true), PA_CONV(128, true, false), PA_CONV(128, true, true),
    PA_TREE_SET(64, false, false),  PA_TREE_SET(64, false, true),
    PA_TREE_SET(64, true, false),   PA_TREE_SET(64, true, true),
    PA_TREE_SET(128, false, false), PA_TREE_SET(128, false, true),
    PA_TREE_SET(128, true, false),  PA_TREE_SET(128, true, true),
    PA_PERSIST_SET(64), PA_PERSIST_SET(128),
};

const Entry* find_entry(const AttnConfig& c) {
  for (const Entry& e : kTable)
    if (e.cfg.dqk == c.dqk && e.cfg.dv == c.dv && e.cfg.fp8 == c.fp8 &&
        e.cfg.shared_kv == c.shared_kv && e.cfg.nt == c.nt && e.cfg.nw == c.nw &&
        e.cfg.hilo == c.hilo && e.cfg.nstage == c.nstage && e.cfg.f16_tiles == c.f16_tiles &&
        e.cfg.tree == c.tree)
      return &e;
  return nullptr;
}
}  // namespace

bool attention_supported(const AttnConfig& cfg) { return find_entry(cfg) != nullptr; }

hipError_t launch_attention(const AttnConfig& cfg, const AttnParams& p, dim3 grid,
                            hipStream_t stream) {
  const Entry* e = find_entry(cfg);
  if (!e) return hipErrorInvalidValue;
  return e->fn(p, grid, stream);
}

int resident_per_cu(const AttnConfig& cfg, int dev) {
  constexpr int kMaxDevices = 64;
  constexpr int kEntries = sizeof(kTable) / sizeof(kTable[0]);
  static std::atomic<int> cache[kMaxDevices][kEntries];   // value + 1; 0 = not asked yet
  const Entry* e = find_entry(cfg);
  if (!e) return 0;
  if (dev < 0 || dev >= kMaxDevices) return e->occ();
  std::atomic<int>& slot = cache[dev][e - kTable];
  int v = slot.load(std::memory_order_relaxed);
  if (v == 0) {
    v = e->occ() + 1;   // the occupancy query runs on the current device
    slot.store(v, std::memory_order_relaxed);
  }
  return v - 1;
}

hipError_t launch_merge(int dv, const MergeParams& p, int batch, int max_q_len,
                        hipStream_t stream) {
  const int rows = max_q_len * p.num_q_heads;
  switch (dv) {
#define PA_MERGE_CASE(D)                                                                     \
  case D: {                                                                                  \
    constexpr int RPB = 256 / (D / 4);                                                       \
    dim3 grid((rows + RPB - 1) / RPB, batch);                                                \
    hipLaunchKernelGGL(split_merge_kernel<D>, grid, dim3(256), 0, stream, p);                \
    return hipGetLastError();                                                                \
  }
    PA_MERGE_CASE(64)
    PA_MERGE_CASE(128)
    PA_MERGE_CASE(256)
    PA_MERGE_CASE(512)
    PA_MERGE_CASE(1024)
#undef PA_MERGE_CASE
    default:
      return hipErrorInvalidValue;
  }
}

// ---------------------------------------------------------- decode scratch --
// The workspace of paged_attn_decode_scratch: one static array per device,
// held until the process ends.  In host code `scratch` names a host-side
// stand-in, not device memory, so its device address is looked up once per
// device (hipGetSymbolAddress with that device current) and only that address
// is ever handed to kernels.
namespace {
static __device__ __align__(256) uint8_t scratch[PA_DECODE_SCRATCH_BYTES];

__global__ __launch_bounds__(256) void zero_words_kernel(int32_t* p, int64_t n) {
  for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < n; i += (int64_t)gridDim.x * 256) p[i] = 0;
}
}  // namespace

void* decode_scratch(int dev, hipError_t* err) {
  constexpr int kMaxDevices = 64;
  static std::mutex mu;
  static void* addr[kMaxDevices] = {};
  *err = hipSuccess;
  if (dev < 0 || dev >= kMaxDevices) {
    *err = hipErrorInvalidDevice;
    return nullptr;
  }
  std::lock_guard<std::mutex> lock(mu);
  if (!addr[dev]) {
    void* ptr = nullptr;
    const hipError_t e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    if (e != hipSuccess || !ptr) {
      *err = e != hipSuccess ? e : hipErrorInvalidSymbol;
      return nullptr;
    }
    addr[dev] = ptr;
  }
  return addr[dev];
}

hipError_t launch_zero_words(int32_t* p, int64_t n, hipStream_t stream) {
  if (n <= 0) return hipSuccess;
  const int64_t blocks = std::min<int64_t>((n + 255) / 256, 1024);
  hipLaunchKernelGGL(zero_words_kernel, dim3((unsigned)blocks), dim3(256), 0, stream, p, n);
  return hipGetLastError();
}

hipError_t launch_tile_gather(int loader, int dqk, int dv, bool shared_kv, const TileWalkParams& p, int batch,
                              int num_kv_heads, int max_chunks, hipStream_t stream) {
  const dim3 grid((unsigned)(batch * num_kv_heads), 1, (unsigned)max_chunks);
#define PA_TG(KERNEL, THREADS)                                                  \
  do {                                                                          \
    hipLaunchKernelGGL(KERNEL, grid, dim3(THREADS), 0, stream, p);              \
    return hipGetLastError();                                                   \
  } while (0)
  if (loader == 1 && !shared_kv && dqk == dv) {
    if (dqk == 64) PA_TG((gather_reg_kernel<64>), 64);
    if (dqk == 128) PA_TG((gather_reg_kernel<128>), 64);
  }
  if ((loader == 2 || loader == 3) && !shared_kv && dqk == dv) {
    if (dqk == 64 && loader == 2) PA_TG((gather_dma_kernel<64, 64, 4, false>), 256);
    if (dqk == 64 && loader == 3) PA_TG((gather_dma_kernel<64, 64, 3, false>), 192);
    if (dqk == 128 && loader == 2) PA_TG((gather_dma_kernel<128, 128, 4, false>), 256);
    if (dqk == 128 && loader == 3) PA_TG((gather_dma_kernel<128, 128, 3, false>), 192);
  }
  if (loader == 2 && shared_kv && dqk == 576) PA_TG((gather_dma_kernel<576, 576, MLA_WAVES, true>), 64 * MLA_WAVES);
  if (loader == 4 && shared_kv && dqk == 576) PA_TG((gather_dma_kernel<576, 576, 4, true, 32>), 256);
#undef PA_TG
  return hipErrorInvalidValue;
}

hipError_t launch_read_probe(int d, const TileWalkParams& p, int batch, int num_kv_heads, int max_chunks,
                             hipStream_t stream) {
  const dim3 grid((unsigned)(batch * num_kv_heads), 1, (unsigned)max_chunks);
  if (d == 64) hipLaunchKernelGGL(read_probe_kernel<64>, grid, dim3(64), 0, stream, p);
  else if (d == 128) hipLaunchKernelGGL(read_probe_kernel<128>, grid, dim3(64), 0, stream, p);
  else return hipErrorInvalidValue;
  return hipGetLastError();
}

hipError_t launch_gather(const GatherParams& p, int batch, hipStream_t stream) {
  dim3 grid((p.t_max + 3) / 4, p.num_kv_heads, batch);
  hipLaunchKernelGGL(gather_kernel, grid, dim3(64), 0, stream, p);
  return hipGetLastError();
}

}  // namespace pa
