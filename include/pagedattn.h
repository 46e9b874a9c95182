/*
 * pagedattn.h - C ABI of the MI355X (gfx950) paged-KV append/decode attention
 * library (libpagedattn.so).
 *
 * The operation (stated in full by the pages' kernels, see each entry point):
 * for request b with n_b appended query tokens and L_b cached tokens, the
 * appended tokens attend over the T_b = L_b + n_b keys of the request, whose
 * K/V rows (the appended tokens' rows included) are already stored in a paged,
 * quantized cache.  Key j of request b lives in physical page
 * block_table[b][j / page_size], slot j % page_size.  Query head h reads KV
 * head g = h / G with G = H_q / H_kv (GQA).  Values are decode(byte) * scale
 * with int8 (two's complement) or fp8 E4M3 (OCP "fn", max 448) bytes and a
 * per-tensor, per-KV-head or per-(KV-head, channel) fp32 scale.  Logits are
 * z_j = sm_scale * q . K[j]; with causal masking, appended token t sees keys
 * j <= L_b + t (bottom-right aligned).  The outputs are
 *   out[t, h, :] = sum_j softmax(z)_j * V[j, :]      (bf16)
 *   lse[t, h]    = ln sum_j exp(z_j)                 (fp32, natural log)
 * Long contexts may be split into KV chunks of chunk_size keys; each chunk's
 * normalized partial output and natural LSE are then merged by log-sum-exp.
 *
 * Conventions shared by every entry point:
 *  - Every array argument is a DEVICE pointer owned by the caller.  The library
 *    never allocates, frees or retains a pointer after the enqueued work ends.
 *  - Work is enqueued on `stream` (a hipStream_t; NULL = the default stream).
 *    Calls are stateless and re-entrant and never synchronize the host.
 *  - All arguments are validated before anything is enqueued: a call that
 *    returns PA_ERR_INVALID_ARG, PA_ERR_UNSUPPORTED or
 *    PA_ERR_WORKSPACE_TOO_SMALL has enqueued nothing.  A kernel launch failure
 *    is reported as PA_ERR_HIP; a call that enqueues two kernels (attention,
 *    then split_kv_merge) and fails to launch the second returns PA_ERR_HIP
 *    with the first already enqueued (the outputs are then undefined).  The
 *    contents of device arrays (lengths, page ids) are the caller's contract
 *    and are not checked: page ids must be valid for every key j < T_b,
 *    entries past ceil(T_b / page_size) are never read.
 *  - pa_last_error() returns a thread-local description of the last failure.
 */
#ifndef PAGEDATTN_H_
#define PAGEDATTN_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Status codes returned by every entry point. */
enum {
  PA_OK = 0,
  PA_ERR_INVALID_ARG = 1,         /* null pointer, bad size or inconsistent shape */
  PA_ERR_UNSUPPORTED = 2,         /* valid but not compiled (head dim, dtype, ...) */
  PA_ERR_WORKSPACE_TOO_SMALL = 3, /* workspace_bytes < paged_attn_workspace_size() */
  PA_ERR_HIP = 4                  /* a HIP runtime call or launch failed */
};

/* Element types. */
enum {
  PA_DTYPE_BF16 = 0,
  PA_DTYPE_F32 = 1,
  PA_DTYPE_I8 = 2,       /* two's-complement int8 cache bytes */
  PA_DTYPE_FP8_E4M3 = 3  /* OCP E4M3 "fn" cache bytes (max 448, no inf) */
};

/* Dequant scale granularity.  PER_TENSOR: k_scale/v_scale hold 1 float;
 * PER_HEAD: [H_kv]; PER_CHANNEL: [H_kv, D] (D_qk for K, D_v for V). */
enum {
  PA_SCALE_PER_TENSOR = 0,
  PA_SCALE_PER_HEAD = 1,
  PA_SCALE_PER_CHANNEL = 2
};

/* Problem description (host struct, read during the call only).
 * Cache strides are in elements (= bytes, the cache is 1 byte per element);
 * the head dimension is contiguous.  Keys of request b come from
 *   k_cache + page * k_stride_page + g * k_stride_head + slot * k_stride_token.
 * For the MLA layout pass v_cache == k_cache with head_dim_v < head_dim_qk:
 * V is then the first head_dim_v bytes of each K row. */
typedef struct pa_problem {
  int32_t batch;              /* B, number of requests */
  int32_t num_q_heads;        /* H_q */
  int32_t num_kv_heads;       /* H_kv, divides H_q */
  int32_t head_dim_qk;        /* D_qk: 64, 128 or 576 */
  int32_t head_dim_v;         /* D_v: 64 (D_qk 64), 128 (D_qk 128) or 512 (D_qk 576, MLA) */
  int32_t page_size;          /* P: power of two, 16..1024 */
  int32_t num_pages;          /* pages in the pool (bounds the page ids) */
  int32_t max_pages_per_seq;  /* row length of block_table */
  int32_t max_q_len;          /* host upper bound of every n_b (sizes the grid) */
  int32_t max_kv_len;         /* host upper bound of every L_b (sizes the grid) */
  int64_t q_row_stride;       /* elements between consecutive query tokens */
  int64_t k_stride_page, k_stride_head, k_stride_token;
  int64_t v_stride_page, v_stride_head, v_stride_token;
  int32_t q_dtype;            /* PA_DTYPE_BF16 or PA_DTYPE_F32 */
  int32_t kv_dtype;           /* PA_DTYPE_I8 or PA_DTYPE_FP8_E4M3 */
  int32_t scale_mode;         /* PA_SCALE_* */
  int32_t causal;             /* 1: bottom-right causal mask, 0: none */
  float sm_scale;             /* softmax scale on q . k (> 0) */
  int32_t chunk_size;         /* 0: no split-KV; else a multiple of 64 keys */
  int32_t flags;              /* PA_FLAG_* bits, 0 for the default behaviour */
  /* Schedule overrides.  0 (the value for normal use) lets the library choose;
   * the other values fix one choice of how the work is laid out on the GPU,
   * for tuning and for tests that must reach every code path.  They never
   * change what is computed: outputs stay within the same rounding of the
   * exact result (decode_waves changes the order of the softmax merge, so the
   * bits may differ; the other two leave the bits unchanged).  Any other value
   * is INVALID_ARG. */
  int32_t decode_waves;       /* 1, 2 or 4: waves that split the keys of one unit of the
                                 decode kernel (<= 32 packed rows), merged in LDS */
  int32_t group_order;        /* shared-tile and MLA kernels: 1 = workgroup L takes slot L
                                 of the (request, KV head, chunk) grid, 2 = only the
                                 groups that hold work are numbered */
  int32_t merge_in_kernel;    /* with PA_FLAG_FUSED_MERGE: 1 = the decode kernel merges
                                 every row tile itself, 2 = never (split_kv_merge runs) */
} pa_problem;

/* pa_problem.flags bits.
 * PA_FLAG_DEFER_MERGE: with chunk_size > 0 the attention call writes the
 *   per-chunk partials of multi-chunk requests to the workspace (and the
 *   final rows of single-chunk requests to out / lse) but does not enqueue
 *   split_kv_merge; the caller runs split_kv_merge on that workspace later,
 *   for instance after adding partial states of its own.  Ignored when
 *   chunk_size is 0. */
/* PA_FLAG_FUSED_MERGE: with chunk_size > 0 the attention kernel merges the
 *   partials itself and no split_kv_merge is enqueued: the last workgroup to
 *   finish a (request, KV head, row tile) merges its rows, as XQA
 *   mla_sm120.cu does with its semaphores in mergePartialOutputs.  This is
 *   done in the decode kernel (at most 32 packed rows) where a row tile's
 *   merge is one short pass (q_len * G <= 4 for head dim 128); elsewhere the
 *   call enqueues split_kv_merge as without the flag, which spreads that work
 *   over the chip.  Either way the results are the same bits.  The
 *   workspace then holds int32 counters [B, H_kv, ceil(max_q_len * G / 16)]
 *   (G = H_q / H_kv) at its start (after the 256 plan bytes of
 *   PA_FLAG_BALANCED_SPLIT when that is set), and the partials follow at the
 *   next 256-byte boundary (paged_attn_workspace_size counts all of it).  The
 *   counters MUST be zero when a call starts: allocate the workspace zeroed;
 *   every completed call leaves them zero.  Their place depends only on
 *   batch, the head counts, max_q_len and the flags, so the workspace stays
 *   valid across calls while those are unchanged (re-zero it when they
 *   change).  Calls that
 *   overlap on one workspace race (as the partials already do).  Combined
 *   with PA_FLAG_DEFER_MERGE it is INVALID_ARG.  Ignored when chunk_size is
 *   0. */
/* PA_FLAG_BALANCED_SPLIT: with chunk_size > 0, the KV split is sized from the
 *   request lengths instead of cut at multiples of chunk_size, after the
 *   work-list planner of FlashInfer persistent.cuh (each request's KV is cut
 *   into chunks so that every CTA gets the same work).  On the device, the
 *   call picks one item length lt (in 64-key tiles, at least chunk_size / 64):
 *   the smallest for which the (request, KV head, item) groups
 *   H_kv * sum_b ceil(ceil(T_b / 64) / lt) fit one round of resident
 *   workgroups.  It then cuts request b into ceil(ceil(T_b / 64) / lt) items
 *   of equal tile count, so no group carries more than lt tiles while short
 *   last chunks leave CUs idle.  Applies to the MLA layout (one workgroup per
 *   CU); the other kernels keep fixed chunks (the dispatcher balances their
 *   many small resident workgroups, and an unchunked append is faster than
 *   either split).  The
 *   workspace starts with 256 bytes for the plan (paged_attn_workspace_size
 *   counts them); the partial-buffer bound stays C_max, since items are at
 *   least chunk_size keys.  Not with PA_FLAG_DEFER_MERGE (INVALID_ARG):
 *   split_kv_merge derives chunks from chunk_size.  Ignored when chunk_size
 *   is 0. */
/* PA_FLAG_PERSISTENT: with chunk_size > 0, paged_attn_decode problems of at
 *   most 32 packed rows (q_len * G) and head dims 64 or 128 run as one
 *   persistent launch, after FlashInfer persistent.cuh
 *   (BlockBatchPagedAttentionPersistent over a work list, then the reduction
 *   of each row's partial states): exactly as many one-wave workgroups as the
 *   device holds at once; the (request, KV head) key ranges are laid end to
 *   end in 64-key tiles and wave w takes the tiles [w N / W, (w + 1) N / W),
 *   with W = min(resident waves, N / (chunk_size / 64)), so no wave's share
 *   is shorter than chunk_size keys and every wave gets the same work.  The
 *   planner runs on the device from the lengths.  A share is cut at the end of
 *   each (request, head) range into pieces whose partials the wave that
 *   finishes a range's last piece merges in the same launch (as with
 *   PA_FLAG_FUSED_MERGE, whose counters it uses: the workspace must start
 *   zeroed and stays zeroed after every call).  The partial buffer holds
 *   C_max + 1 slots.  Not with PA_FLAG_DEFER_MERGE or PA_FLAG_BALANCED_SPLIT
 *   (INVALID_ARG); other problems (append, draft trees, wider rows, MLA) run
 *   as without the flag.  Ignored when chunk_size is 0. */
enum {
  PA_FLAG_DEFER_MERGE = 1,
  PA_FLAG_FUSED_MERGE = 2,
  PA_FLAG_BALANCED_SPLIT = 4,
  PA_FLAG_PERSISTENT = 8
};

/*
 * paged_attn_workspace_size - bytes of workspace the attention calls need.
 *
 * Split-KV (chunk_size > 0) keeps, for every query token and head, one
 * normalized fp32 partial output row and one natural-log fp32 partial LSE per
 * chunk: [total_q, C_max, H_q, D_v] floats followed (256-byte aligned) by
 * [total_q, C_max, H_q] floats, with C_max = ceil((max_kv_len + max_q_len) /
 * chunk_size) (one more with PA_FLAG_PERSISTENT).  PA_FLAG_BALANCED_SPLIT puts
 * 256 bytes of plan first; with PA_FLAG_FUSED_MERGE or PA_FLAG_PERSISTENT the
 * int32 merge counters [B, H_kv, ceil(max_q_len * H_q / H_kv / 16)] come next,
 * and the partials start at the next 256-byte boundary.  This is the partial-buffer layout of FastDeploy
 * append_attention_c8_impl.cuh (tmp_workspace / tmp_m / tmp_d, indexed
 * [token, chunk, head, dim]), with FlashInfer persistent.cuh's normalized
 * output + LSE pair in place of the (m, d) pair.  Returns 0 when chunk_size is
 * 0 and (size_t)-1 for an invalid problem.
 */
size_t paged_attn_workspace_size(const pa_problem* prob, int32_t total_q);

/*
 * paged_attn_append - ragged append / chunked-prefill attention.
 *
 * Follows FastDeploy append_attention_c8_impl.cuh (CascadeAppendAttentionC8Kernel
 * and multi_query_append_attention_c8_kernel): ragged queries by cu_seqlens_q,
 * kv_len = seq_lens_kv + q_len with the appended K/V read from the cache,
 * GQA-packed query rows, causal bound, KV chunks of chunk_size keys.
 *
 *  q            [total_q, H_q, D_qk] in q_dtype, token rows q_row_stride apart.
 *  k_cache      paged K bytes, v_cache paged V bytes (see pa_problem strides).
 *  k_scale      fp32 dequant scales of K, v_scale of V (see PA_SCALE_*).
 *  cu_seqlens_q int32 [B+1] prefix sums of n_b (cu_seqlens_q[0] = 0); n_b <= max_q_len.
 *  seq_lens_kv  int32 [B] cached tokens L_b <= max_kv_len.
 *  block_table  int32 [B, max_pages_per_seq] physical page ids.
 *  out          bf16 [total_q, H_q, D_v] (contiguous).
 *  lse          fp32 [total_q, H_q] natural-log LSE, or NULL.
 *  workspace    device buffer of workspace_bytes (may be NULL when
 *               paged_attn_workspace_size() is 0).
 * Requests with n_b = 0 write nothing.  With chunk_size > 0, requests that
 * span more than one chunk go through the workspace and split_kv_merge is
 * enqueued on the same stream (unless PA_FLAG_DEFER_MERGE); single-chunk
 * requests are written directly.  Unknown flag bits are INVALID_ARG.
 */
int32_t paged_attn_append(const pa_problem* prob, int32_t total_q, const void* q,
                          const void* k_cache, const void* v_cache, const float* k_scale,
                          const float* v_scale, const int32_t* cu_seqlens_q,
                          const int32_t* seq_lens_kv, const int32_t* block_table, void* out,
                          float* lse, void* workspace, size_t workspace_bytes, void* stream);

/*
 * paged_attn_decode - decode and multi-token (speculative) decode.
 *
 * Same operation with a uniform host q_len (1..64) per request: q is
 * [B * q_len, H_q, D_qk] and request b's tokens are rows b*q_len .. b*q_len +
 * q_len - 1 (FastDeploy's decoder path with speculate_max_draft_token_num
 * drafts; XQA mla_sm120.cu's inputSeqLen tokens with a per-token causal
 * length).  Causal masking among the drafts is the bottom-right rule above.
 * Arguments are as for paged_attn_append with cu_seqlens_q replaced by q_len.
 */
int32_t paged_attn_decode(const pa_problem* prob, int32_t q_len, const void* q,
                          const void* k_cache, const void* v_cache, const float* k_scale,
                          const float* v_scale, const int32_t* seq_lens_kv,
                          const int32_t* block_table, void* out, float* lse, void* workspace,
                          size_t workspace_bytes, void* stream);

/*
 * paged_attn_decode_tree - speculative decode with a draft tree.
 *
 * The decode path of FastDeploy append_attention_c8_impl.cuh takes an
 * optional attn_mask of shape [bsz, max_q, max_q] for tree-structured drafts
 * (multi_query_append_attention_c8_warp1_4_kernel hands its mask step the
 * request's slice at offset batch_id * attn_mask_len * attn_mask_len, and the
 * host reads attn_mask_len from the mask's second dimension).  Here:
 *   tree_mask      device, uint8 [B, tree_mask_len, tree_mask_len], row-major,
 *                  caller-owned, read only.  Entry [b][t][s] != 0 makes
 *                  appended key L_b + s visible to token t of request b; 0
 *                  hides it.  Only entries with t, s < q_len are read.
 *   tree_mask_len  q_len <= tree_mask_len <= 64.
 * Cached keys (j < L_b) stay visible to every token; the mask takes the place
 * of the causal rule inside the appended block, whatever prob->causal says.
 * Everything else is as for paged_attn_decode.  Supported for the int8/fp8
 * layouts with D_qk 64 or 128 and at most 64 packed rows (q_len * H_q / H_kv);
 * MLA (576/512) and wider row counts are UNSUPPORTED, a null mask or a length
 * outside [q_len, 64] is INVALID_ARG.
 */
int32_t paged_attn_decode_tree(const pa_problem* prob, int32_t q_len, const void* q,
                               const void* k_cache, const void* v_cache, const float* k_scale,
                               const float* v_scale, const int32_t* seq_lens_kv,
                               const int32_t* block_table, const uint8_t* tree_mask,
                               int32_t tree_mask_len, void* out, float* lse, void* workspace,
                               size_t workspace_bytes, void* stream);

/*
 * paged_kv_write - the cache append write: quantize the new tokens' K/V rows
 * and scatter them into their pages.
 *
 * FastDeploy append_attention_c8_impl.cuh attends over kv_len = seq_lens_kv +
 * q_len keys and reads the appended tokens' K/V from the cache; this call puts
 * them there.  Token t (0 <= t < n_b) of request b goes to position L_b + t:
 * page block_table[b][(L_b + t) / P], slot (L_b + t) % P, bytes 0..D-1 of the
 * row.  With s the scale of its (head, channel) as for dequantization (per
 * tensor, per KV head or per channel, prob->scale_mode) and r = x / s one
 * correctly rounded binary32 division:
 *   int8     code = clamp(round_half_even(r), -127, 127)
 *   e4m3fn   code = nearest e4m3fn value (ties to an even mantissa), finite
 *            values beyond 448 saturate to +-448, NaN gives 0x7F
 * (the pages fix only the read side, value = code * s; this is its inverse).
 *   prob            as for attention; q_dtype is the dtype of k_new / v_new
 *                   (BF16 or F32), max_q_len bounds every n_b (grid size).
 *   total_new       rows of k_new / v_new (= cu_seqlens_new[B]).
 *   k_new, v_new    device [total_new, H_kv, D_qk] and [total_new, H_kv, D_v],
 *                   dense, 16-byte aligned, read only.  For the shared latent
 *                   layout (D_qk 576) v_new must be NULL: the 576-byte K row
 *                   holds V in its first 512 bytes.
 *   cu_seqlens_new  device int32 [B+1] prefix sums of n_b.
 *   seq_lens_kv     device int32 [B] cached tokens L_b before this append.
 *   block_table     device int32 [B, max_pages_per_seq]; entries up to page
 *                   (L_b + n_b - 1) / P must name pages of the pool.
 *   k_scale/v_scale device fp32 scales (layout of prob->scale_mode).
 *   k_cache/v_cache device caches, written in place; nothing else changes.
 * Rows of different requests must not map to the same slot (their order is
 * unspecified).  Enqueued on `stream`; validation errors enqueue nothing.
 */
int32_t paged_kv_write(const pa_problem* prob, int32_t total_new, const void* k_new, const void* v_new,
                       const int32_t* cu_seqlens_new, const int32_t* seq_lens_kv,
                       const int32_t* block_table, const float* k_scale, const float* v_scale,
                       void* k_cache, void* v_cache, void* stream);

/*
 * paged_attn_decode_scratch - paged_attn_decode for callers that cannot
 * allocate device memory (code under HIP graph capture, tight serving loops,
 * harnesses that forbid hipMalloc).
 *
 * Same operation, arguments and results as paged_attn_decode, without the
 * workspace: the split-KV partials (and, with PA_FLAG_FUSED_MERGE, the merge
 * counters) live in a static device array of PA_DECODE_SCRATCH_BYTES that
 * the library holds on every GPU it runs on until the process ends.  The call
 * allocates nothing (no hipMalloc, no allocating library routine); on the
 * first call on a device it looks the array's address up once.
 *   - A problem whose paged_attn_workspace_size(prob, B * q_len) exceeds
 *     PA_DECODE_SCRATCH_BYTES is PA_ERR_WORKSPACE_TOO_SMALL (checked before
 *     anything else happens on the GPU).
 *   - PA_FLAG_DEFER_MERGE is INVALID_ARG: the partials are not reachable by
 *     the caller.  The merge counters of PA_FLAG_FUSED_MERGE are cleared by
 *     the call itself (a fill kernel on `stream`).
 *   - Every call on one GPU shares that GPU's array, which keeps the last
 *     call's contents: calls that overlap on one GPU (other streams, other
 *     threads, graph replays in flight together) race and must be ordered by
 *     the caller.
 */
#define PA_DECODE_SCRATCH_BYTES ((size_t)32 << 20)

int32_t paged_attn_decode_scratch(const pa_problem* prob, int32_t q_len, const void* q,
                                  const void* k_cache, const void* v_cache, const float* k_scale,
                                  const float* v_scale, const int32_t* seq_lens_kv,
                                  const int32_t* block_table, void* out, float* lse, void* stream);

/*
 * split_kv_merge - log-sum-exp merge of split-KV partials.
 *
 * For every query token t of request b and head h, with C_b = ceil((L_b + n_b)
 * / chunk_size) > 1: M = max_c lse_c, w_c = exp(lse_c - M), out = sum_c w_c O_c
 * / sum_c w_c (bf16), lse = M + ln sum_c w_c.  Chunks with lse_c = -inf carry
 * weight 0; a row whose chunks are all -inf gets out = 0, lse = -inf.  Rows
 * with C_b <= 1 are left untouched (they were written directly).  Slots c
 * with C_b <= c < max_chunks may be read (they stay inside the buffers above)
 * and their contents are ignored, whatever they hold.  Follows FlashInfer persistent.cuh (BlockBatchReductionPersistent,
 * which skips rows with 0 or 1 partials) and XQA mla_sm120.cu
 * (mergePartialOutputs); C_b is derived from the lengths as in FastDeploy's
 * merge launches.
 *
 *  partial_o    fp32 [total_q, max_chunks, H_q, D_v] normalized partial outputs.
 *  partial_lse  fp32 [total_q, max_chunks, H_q] natural-log partial LSE.
 *  cu_seqlens_q int32 [B+1], or NULL with q_len_uniform > 0 (token b*q_len + t).
 *  seq_lens_kv  int32 [B] cached tokens L_b.
 *  out          bf16 [total_q, H_q, D_v]; lse fp32 [total_q, H_q] or NULL.
 * D_v must be 64, 128, 256, 512 or 1024 (other values are UNSUPPORTED).
 */
int32_t split_kv_merge(const float* partial_o, const float* partial_lse,
                       const int32_t* cu_seqlens_q, const int32_t* seq_lens_kv,
                       int32_t q_len_uniform, int32_t batch, int32_t total_q, int32_t max_q_len,
                       int32_t num_q_heads, int32_t head_dim_v, int32_t chunk_size,
                       int32_t max_chunks, void* out, float* lse, void* stream);

/*
 * pa_gather_debug - raw-byte page gather (test aid).
 *
 * Copies the K rows (and V rows when v_dst is not NULL) of keys 0..T_b-1 of
 * every request and KV head, in key order, to k_dst [B, H_kv, t_max, D_qk]
 * and v_dst [B, H_kv, t_max, D_v] bytes (rows past T_b are left as they
 * are).  T_b = seq_lens_kv[b] + q_lens[b]; q_lens int32 [B]; t_max >= max_b T_b.
 * `loader` picks the code that computes the addresses (key j -> page
 * block_table[b][j / P], slot j % P, as in FlashInfer persistent.cuh
 * prefetch_offest and XQA KVTilePartLoader::loadPages):
 *   PA_GATHER_ROWS        one key row at a time through the kernels' page
 *                         and row address functions;
 *   PA_GATHER_DECODE      the decode kernel's register tile loader (64-key
 *                         tiles, one-page fast path, clamped last tile), over
 *                         units of prob->chunk_size keys (whole sequences when
 *                         0); head dims 64 or 128 with D_qk == D_v;
 *   PA_GATHER_DMA_4W      the shared-tile / append / MLA kernels' LDS-DMA tile
 *   PA_GATHER_DMA_3W      loader with 4 or 3 waves splitting each 64-key
 *                         tile, over the same units; head dims 64/128
 *                         (D_qk == D_v) or, with 4 waves, the shared 576/512
 *                         layout (V is then the K prefix: v_dst must be NULL);
 *   PA_GATHER_DMA_MLA32   the same loader as the e4m3fn MLA kernel drives it:
 *                         4 waves splitting 32-key tiles, shared 576/512
 *                         layout only.
 * Other combinations are UNSUPPORTED.
 */
enum {
  PA_GATHER_ROWS = 0,
  PA_GATHER_DECODE = 1,
  PA_GATHER_DMA_4W = 2,
  PA_GATHER_DMA_3W = 3,
  PA_GATHER_DMA_MLA32 = 4
};

int32_t pa_gather_debug(const pa_problem* prob, int32_t loader, const void* k_cache, const void* v_cache,
                        const int32_t* block_table, const int32_t* seq_lens_kv, const int32_t* q_lens,
                        int32_t t_max, uint8_t* k_dst, uint8_t* v_dst, void* stream);

/*
 * pa_kv_read_probe - the decode kernel's KV reads alone (measurement aid).
 *
 * Walks the units of paged_attn_decode (request, KV head, chunk of
 * prob->chunk_size keys; whole sequences when 0) with q_len tokens per
 * request and reads every K/V byte the attention kernel reads, through the
 * same tile loader, with no arithmetic on them but an xor folded into
 * sink[c * B * H_kv + b * H_kv + g] (device uint32 [C_max * B * H_kv],
 * C_max as in paged_attn_workspace_size).  Its time over the KV bytes is the
 * read bandwidth the decode access pattern allows.  Head dims 64 or 128 with
 * D_qk == D_v; other problems are UNSUPPORTED.
 */
int32_t pa_kv_read_probe(const pa_problem* prob, int32_t q_len, const void* k_cache, const void* v_cache,
                         const int32_t* seq_lens_kv, const int32_t* block_table, uint32_t* sink,
                         void* stream);

/* Human-readable name of a status code. */
const char* pa_status_string(int32_t status);

/* Thread-local description of the last failing call on this thread ("" if none). */
const char* pa_last_error(void);

#ifdef __cplusplus
}
#endif

#endif /* PAGEDATTN_H_ */
