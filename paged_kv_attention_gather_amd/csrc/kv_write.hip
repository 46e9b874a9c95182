// KV-cache append write for gfx950: quantize the new tokens' K/V rows and
// scatter them into their pages.
//
// The attention kernels read the appended tokens from the cache (FastDeploy
// append_attention_c8_impl.cuh: kv_len = seq_lens_kv + q_len, K/V tiles only
// from the cache), so token t of request b must sit at position L_b + t, in
// page block_table[b][(L_b + t) / P], slot (L_b + t) % P, as int8 or e4m3fn
// bytes whose value is byte * scale.  This kernel writes them: code =
// round-half-even(x / s) clamped to [-127, 127] for int8, the nearest e4m3fn
// (ties to even, saturating at 448) for fp8, with x / s one correctly rounded
// binary32 division.
//
// Memory-bound scatter: a workgroup takes the tokens of one request that make
// about 256 items; an item is 8 consecutive channels of one (token, head,
// matrix) row: one 16-byte (bf16) or two 16-byte (fp32) loads, one 8-byte
// store.  Wide rows (more than 256 items per token) loop.
#include <hip/hip_runtime.h>

#include "pa_internal.h"

namespace pa {
namespace {

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef int i32x2 __attribute__((ext_vector_type(2)));

__device__ __forceinline__ uint32_t code_int8(float r) {
  const float q = fminf(fmaxf(rintf(r), -127.f), 127.f);   // rintf rounds half to even
  return (uint32_t)((int)q) & 0xffu;
}

// e4m3fn from the binary32 bits: sign, then |r| >= 448 saturates to 0x7E,
// |r| < 2^-6 lands on the subnormal grid 2^-9 (8 units is the smallest
// normal, code 0x08), otherwise the 23-bit mantissa is rounded to 3 bits
// (ties to even) and a carry bumps the exponent.  NaN gives 0x7F.
__device__ __forceinline__ uint32_t code_e4m3(float r) {
  const uint32_t u = __builtin_bit_cast(uint32_t, r);
  const uint32_t sign = (u >> 24) & 0x80u;
  const float a = fabsf(r);
  if (a != a) return 0x7Fu;
  if (a >= 448.f) return sign | 0x7Eu;
  if (a < 0.015625f) return sign | (uint32_t)rintf(a * 512.f);
  const uint32_t ua = u & 0x7fffffffu;
  int e = (int)(ua >> 23) - 127;
  uint32_t m = (ua >> 20) & 7u;
  const uint32_t rem = ua & 0xfffffu;
  if (rem > 0x80000u || (rem == 0x80000u && (m & 1u))) ++m;
  if (m == 8u) {
    m = 0u;
    ++e;
  }
  const uint32_t code = ((uint32_t)(e + 7) << 3) | m;
  return sign | (code < 0x7Eu ? code : 0x7Eu);
}

template <bool FP8, bool F32IN>
__global__ __launch_bounds__(256) void kv_write_kernel(KvWriteParams p) {
  const int b = blockIdx.y;
  const int tok0 = p.cu_seqlens_new[b];
  const int n = p.cu_seqlens_new[b + 1] - tok0;
  const int t_lo = blockIdx.x * p.tokens_per_block;
  if (t_lo >= n) return;
  const int L = p.seq_lens_kv[b];
  const int nk8 = p.dk / 8, nv8 = p.dv / 8;
  const int per_head = nk8 + nv8;
  const int per_tok = p.num_kv_heads * per_head;
  const int items = min(p.tokens_per_block, n - t_lo) * per_tok;
  const int32_t* table_row = p.block_table + (int64_t)b * p.max_pages_per_seq;
  const int slot_mask = (1 << p.page_shift) - 1;
  for (int it = threadIdx.x; it < items; it += 256) {
    const int t = t_lo + it / per_tok;
    const int rem = it - (it / per_tok) * per_tok;
    const int h = rem / per_head;
    const int j = rem - h * per_head;
    const bool is_v = j >= nk8;
    const int d0 = 8 * (is_v ? j - nk8 : j);
    const int dim = is_v ? p.dv : p.dk;
    const int pos = L + t;
    const int64_t page = table_row[pos >> p.page_shift];
    const int64_t row = (int64_t)(tok0 + t) * p.num_kv_heads + h;
    float x[8];
    if constexpr (F32IN) {
      const float* src = static_cast<const float*>(is_v ? p.v_new : p.k_new) + row * dim + d0;
      const f32x4 a = *(const f32x4*)src, c = *(const f32x4*)(src + 4);
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        x[e] = a[e];
        x[4 + e] = c[e];
      }
    } else {
      const uint16_t* src = static_cast<const uint16_t*>(is_v ? p.v_new : p.k_new) + row * dim + d0;
      const u32x4 w = *(const u32x4*)src;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const uint32_t we = w[e];
        x[2 * e] = __builtin_bit_cast(float, we << 16);
        x[2 * e + 1] = __builtin_bit_cast(float, we & 0xffff0000u);
      }
    }
    const float* scale = is_v ? p.v_scale : p.k_scale;
    uint32_t lo = 0, hi = 0;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const int sidx = p.scale_mode == PA_SCALE_PER_CHANNEL ? h * dim + d0 + e
                       : (p.scale_mode == PA_SCALE_PER_HEAD ? h : 0);
      const float r = __fdiv_rn(x[e], scale[sidx]);
      const uint32_t c = FP8 ? code_e4m3(r) : code_int8(r);
      if (e < 4) lo |= c << (8 * e);
      else hi |= c << (8 * (e - 4));
    }
    uint8_t* dst = is_v ? p.v_cache + page * p.v_stride_page + (int64_t)h * p.v_stride_head +
                              (int64_t)(pos & slot_mask) * p.v_stride_token
                        : p.k_cache + page * p.k_stride_page + (int64_t)h * p.k_stride_head +
                              (int64_t)(pos & slot_mask) * p.k_stride_token;
    *(i32x2*)(dst + d0) = i32x2{(int)lo, (int)hi};
  }
}

}  // namespace

hipError_t launch_kv_write(const KvWriteParams& p, bool fp8, bool f32_in, int batch, int max_new,
                           hipStream_t stream) {
  dim3 grid((unsigned)((max_new + p.tokens_per_block - 1) / p.tokens_per_block), (unsigned)batch);
  if (fp8) {
    if (f32_in) hipLaunchKernelGGL((kv_write_kernel<true, true>), grid, dim3(256), 0, stream, p);
    else hipLaunchKernelGGL((kv_write_kernel<true, false>), grid, dim3(256), 0, stream, p);
  } else {
    if (f32_in) hipLaunchKernelGGL((kv_write_kernel<false, true>), grid, dim3(256), 0, stream, p);
    else hipLaunchKernelGGL((kv_write_kernel<false, false>), grid, dim3(256), 0, stream, p);
  }
  return hipGetLastError();
}

}  // namespace pa
