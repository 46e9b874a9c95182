// Internal launch parameters shared by the C-ABI front end (pagedattn_api.cpp)
// and the gfx950 kernels (pa_kernels.hip).  Not part of the public ABI.
#pragma once

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h>

#include "pagedattn.h"

namespace pa {

// One launch of the paged attention kernel.  A work unit is (request b, KV
// head g, packed-row tile, KV chunk); the decode kernel's grid is
// (B * H_kv, row_tiles, chunk_slots), the shared-tile kernel's
// (row_tiles * chunk_slots, H_kv, B).
struct AttnParams {
  const void* q;
  const uint8_t* k_cache;
  const uint8_t* v_cache;
  const float* k_scale;
  const float* v_scale;
  const int32_t* cu_seqlens_q;  // null: uniform q_len_uniform tokens per request
  const int32_t* seq_lens_kv;
  const int32_t* block_table;
  const uint8_t* tree_mask;     // [B, tree_mask_len, tree_mask_len] draft visibility, or null
  uint16_t* out;                // bf16 [total_q, H_q, D_v]
  float* lse;                   // [total_q, H_q] or null
  float* part_o;                // [total_q, max_chunks, H_q, D_v] (split only)
  float* part_lse;              // [total_q, max_chunks, H_q]
  int32_t* merge_count;         // in-kernel merge counters [B, H_kv, count_stride], or null
  int64_t q_row_stride;         // elements
  int64_t k_stride_page, k_stride_head, k_stride_token;
  int64_t v_stride_page, v_stride_head, v_stride_token;
  int32_t num_q_heads;
  int32_t num_kv_heads;
  int32_t group;                // G = H_q / H_kv
  int32_t page_shift;           // log2(page_size)
  int32_t max_pages_per_seq;
  int32_t q_len_uniform;
  int32_t chunk_size;           // 0 = no split
  int32_t max_chunks;           // chunk slots in the grid / partial buffers
  int32_t row_tiles;
  int32_t batch;
  int32_t compact_groups;       // shared-tile kernels: number only the groups that hold work
  int32_t q_is_f32;
  int32_t scale_mode;
  int32_t causal;
  int32_t tree_mask_len;
  int32_t count_stride;         // 16-row groups per (request, KV head) in merge_count
  int32_t balanced;             // balanced split: item length chosen from the lengths (shared-tile kernels)
  int32_t group_cap;            // balanced split: (request, KV head, item) groups that fit one round
  int32_t* plan_out;            // balanced split: the chosen item length (tiles) for the merge, or null
  float qk_mult;                // sm_scale * log2(e)
};

struct MergeParams {
  const float* part_o;
  const float* part_lse;
  const int32_t* cu_seqlens_q;
  const int32_t* seq_lens_kv;
  uint16_t* out;
  float* lse;
  int32_t q_len_uniform;
  int32_t num_q_heads;
  int32_t chunk_size;
  int32_t max_chunks;
  const int32_t* item_tiles;    // balanced split: item length in 64-key tiles (device), or null
};

struct GatherParams {
  const uint8_t* k_cache;
  const int32_t* block_table;
  const int32_t* seq_lens_kv;
  const int32_t* q_lens;
  uint8_t* dst;
  int64_t k_stride_page, k_stride_head, k_stride_token;
  int32_t num_kv_heads;
  int32_t head_dim;
  int32_t page_shift;
  int32_t max_pages_per_seq;
  int32_t t_max;
};

// The debug gather through an attention kernel's tile loader, and the read
// probe: units (request, KV head, chunk) over keys [c * chunk, min(T_b,
// (c + 1) * chunk)) with T_b = seq_lens_kv[b] + q_lens[b] (q_len_uniform when
// q_lens is null); grid (B * H_kv, 1, C_max).
struct TileWalkParams {
  AttnParams a;                 // cache pointers, strides, block table, page shift
  const int32_t* q_lens;        // [B] or null (a.q_len_uniform)
  uint8_t* k_dst;               // gather: [B, H_kv, t_max, D_qk] or null
  uint8_t* v_dst;               // gather: [B, H_kv, t_max, D_v] or null
  uint32_t* sink;               // probe: [B * H_kv * C_max] xor of the bytes read
  int32_t t_max;
  int32_t chunk;                // keys per unit (> 0)
};

// One launch of the KV-cache append write (kv_write.hip).  Grid (token
// slices of tokens_per_block, B); dv = 0 writes K rows only (shared layout).
struct KvWriteParams {
  const void* k_new;            // [total_new, H_kv, dk] bf16 bits or fp32
  const void* v_new;            // [total_new, H_kv, dv] or null
  const int32_t* cu_seqlens_new;
  const int32_t* seq_lens_kv;
  const int32_t* block_table;
  const float* k_scale;
  const float* v_scale;
  uint8_t* k_cache;
  uint8_t* v_cache;
  int64_t k_stride_page, k_stride_head, k_stride_token;
  int64_t v_stride_page, v_stride_head, v_stride_token;
  int32_t num_kv_heads, dk, dv, page_shift, max_pages_per_seq, scale_mode, tokens_per_block;
};

// Compiled attention specializations.
struct AttnConfig {
  int dqk, dv;      // head dims
  bool fp8;         // cache bytes are e4m3fn (else int8)
  bool shared_kv;   // V = first dv bytes of the K row
  int nt;           // 16-row MFMA tiles per wave
  int nw;           // waves per workgroup (they split the rows, share KV tiles)
  bool hilo;        // Q carries per-channel scales or is fp32: f16 hi + lo parts
  int nstage;       // KV tiles staged in LDS (0: register-staged decode kernel, 1: MLA kernel,
                    // 4: persistent register-staged decode kernel)
  bool f16_tiles;   // shared-tile kernel converts each tile to f16 in LDS once
  bool tree;        // draft-tree mask over the appended keys (decode-path kernels)
};

// Workgroups of the kernel `cfg` selects that fit on one CU of device `dev` at
// once (0: unknown); asked once per (device, kernel) and cached.
int resident_per_cu(const AttnConfig& cfg, int dev);
// Returns hipSuccess, hipErrorInvalidValue when no specialization matches.
hipError_t launch_attention(const AttnConfig& cfg, const AttnParams& p, dim3 grid,
                            hipStream_t stream);
hipError_t launch_merge(int dv, const MergeParams& p, int batch, int max_q_len,
                        hipStream_t stream);
hipError_t launch_gather(const GatherParams& p, int batch, hipStream_t stream);
// Debug gather through the decode kernel's register loader (loader 1) or the
// shared-tile / MLA kernels' LDS-DMA loader with 4 or 3 waves (loader 2, 3);
// head dims as in the problem.  hipErrorInvalidValue for other geometries.
hipError_t launch_tile_gather(int loader, int dqk, int dv, bool shared_kv, const TileWalkParams& p, int batch,
                              int num_kv_heads, int max_chunks, hipStream_t stream);
// The read probe: every unit's K/V tiles through the decode kernel's loader,
// no arithmetic on them but an xor into the sink (head dims 64 or 128).
hipError_t launch_read_probe(int d, const TileWalkParams& p, int batch, int num_kv_heads, int max_chunks,
                             hipStream_t stream);
hipError_t launch_kv_write(const KvWriteParams& p, bool fp8, bool f32_in, int batch, int max_new,
                           hipStream_t stream);
bool attention_supported(const AttnConfig& cfg);
// Device address of the static decode scratch (PA_DECODE_SCRATCH_BYTES) on
// device `dev`, looked up once per device with that device current; null
// when the lookup failed (*err then holds the HIP error).
void* decode_scratch(int dev, hipError_t* err);
// Sets n int32 words at p to zero with a kernel on `stream` (no memset node,
// so the call stays safe under graph capture).
hipError_t launch_zero_words(int32_t* p, int64_t n, hipStream_t stream);

}  // namespace pa
