// Checking hooks: the block-table gather and the FP8, INT8 and INT4 decodes,
// run with the same device helpers (chunk_offset, k_in_chunk, v_in_chunk,
// kv8x8_to_bf16x8; chunk_offset4, k4_code, v4_code, i4x8_to_bf16x8) as the
// attention kernels.

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "device_common.h"
#include "kernel_params.h"

namespace pa {

// one thread per (sequence, kv head, token, d)
__global__ __launch_bounds__(256) void debug_gather_kernel(GatherParams p) {
  const int64_t per_seq = (int64_t)p.num_kv_heads * p.max_ctx_len * p.head_dim;
  const int64_t total = per_seq * p.num_seqs;
  for (int64_t e = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; e < total; e += (int64_t)gridDim.x * blockDim.x) {
    const int d = (int)(e % p.head_dim);
    int64_t r = e / p.head_dim;
    const int t = (int)(r % p.max_ctx_len);
    r /= p.max_ctx_len;
    const int h = (int)(r % p.num_kv_heads);
    const int b = (int)(r / p.num_kv_heads);
    const int L = p.ctx_lens[b];
    const int64_t st = ((int64_t)b * p.num_kv_heads + h) * p.max_ctx_len + t;
    if (t < L) {
      const int32_t page = p.block_table[(int64_t)b * p.bt_stride + t / kPageSize];
      const int slot = t % kPageSize;
      if (p.kv_format == kKvInt4) {
        // INT4: the 4-bit codes, one per output byte
        const uint64_t base = chunk_offset4(page, h, p.num_kv_heads, p.head_dim);
        p.k_out[e] = (uint8_t)k4_code(p.k_pages + base, slot, d);
        p.v_out[e] = (uint8_t)v4_code(p.v_pages + base, slot, d);
      } else {
        const uint64_t base = chunk_offset(page, h, p.num_kv_heads, p.head_dim);
        p.k_out[e] = p.k_pages[base + k_in_chunk(slot, d, p.head_dim)];
        p.v_out[e] = p.v_pages[base + v_in_chunk(slot, d, p.head_dim)];
      }
      if (d == 0) {
        const int64_t sidx = (int64_t)page * p.num_kv_heads + h;
        p.scale_out[st] = p.kv_scales[sidx];
        p.scale_out[(int64_t)p.num_seqs * p.num_kv_heads * p.max_ctx_len + st] = p.kv_scales[p.v_scale_offset + sidx];
        if (h == 0) p.page_out[(int64_t)b * p.max_ctx_len + t] = page;
      }
    } else {
      p.k_out[e] = 0;
      p.v_out[e] = 0;
      if (d == 0) {
        p.scale_out[st] = 0.f;
        p.scale_out[(int64_t)p.num_seqs * p.num_kv_heads * p.max_ctx_len + st] = 0.f;
        if (h == 0) p.page_out[(int64_t)b * p.max_ctx_len + t] = -1;
      }
    }
  }
}

// one thread per 8 input bytes: E4M3 codes, or INT8 with KI8
template <bool KI8>
__global__ __launch_bounds__(256) void debug_decode_kernel(const uint8_t* in, float* out, int64_t n) {
  const int64_t i0 = ((int64_t)blockIdx.x * blockDim.x + threadIdx.x) * 8;
  if (i0 >= n) return;
  uint32_t w[2] = {0u, 0u};
  for (int k = 0; k < 8 && i0 + k < n; ++k) w[k / 4] |= (uint32_t)in[i0 + k] << (8 * (k % 4));
  const bf16x8 v = kv8x8_to_bf16x8<KI8>(w[0], w[1]);
  for (int k = 0; k < 8 && i0 + k < n; ++k) out[i0 + k] = (float)v[k];
}

// one thread per 4 input bytes of INT4 codes (8 values): the kernels'
// widening to 16 times the value, then the factor 1/16 they fold into the
// page scales (exact)
__global__ __launch_bounds__(256) void debug_decode4_kernel(const uint8_t* in, float* out, int64_t n) {
  const int64_t i0 = ((int64_t)blockIdx.x * blockDim.x + threadIdx.x) * 4;
  if (i0 >= n) return;
  uint32_t w = 0u;
  for (int k = 0; k < 4 && i0 + k < n; ++k) w |= (uint32_t)in[i0 + k] << (8 * k);
  const bf16x8 v = i4x8_to_bf16x8(w);
  for (int k = 0; k < 8 && i0 + k / 2 < n; ++k) out[2 * i0 + k] = (float)v[k] * code_unit<kKvInt4>();
}

hipError_t launch_debug_gather(const GatherParams& p, hipStream_t stream) {
  const int64_t total = (int64_t)p.num_seqs * p.num_kv_heads * p.max_ctx_len * p.head_dim;
  if (total <= 0) return hipSuccess;
  int64_t blocks = (total + 255) / 256;
  if (blocks > 65536) blocks = 65536;
  hipLaunchKernelGGL(debug_gather_kernel, dim3((unsigned)blocks), dim3(256), 0, stream, p);
  return hipGetLastError();
}

hipError_t launch_debug_decode(const uint8_t* in, float* out, int64_t n, int kv_format, hipStream_t stream) {
  if (n <= 0) return hipSuccess;
  if (kv_format == kKvInt4) {
    const int64_t blocks4 = ((n + 3) / 4 + 255) / 256;
    if (blocks4 > 0x7fffffff) return hipErrorInvalidValue;
    hipLaunchKernelGGL(debug_decode4_kernel, dim3((unsigned)blocks4), dim3(256), 0, stream, in, out, n);
    return hipGetLastError();
  }
  const int64_t threads = (n + 7) / 8;
  const int64_t blocks = (threads + 255) / 256;
  if (blocks > 0x7fffffff) return hipErrorInvalidValue;
  if (kv_format == kKvInt8)
    hipLaunchKernelGGL(debug_decode_kernel<true>, dim3((unsigned)blocks), dim3(256), 0, stream, in, out, n);
  else
    hipLaunchKernelGGL(debug_decode_kernel<false>, dim3((unsigned)blocks), dim3(256), 0, stream, in, out, n);
  return hipGetLastError();
}

}  // namespace pa
