// Paged FP8 KV append for gfx950: the new tokens' K and V rows of each
// sequence are quantised into its pages through the block table, with one
// fp32 scale per (page, kv head).  INT8 pools (KI8) take the same steps
// with 127 in place of 448 and round-half-even integer codes.
//
// Follows the memory section of the Atlas engine article (ainews.cool,
// "技术深度解析": fixed-size KV blocks from a preallocated pool), its
// quantisation section (FP8 with per-group scale factors) and the paged FP8
// KV cache of the GB10 article (ainews.surl.tw).  Per touched (page, head):
//   scale = fp32(max |value| over the page's valid slots) / 448 (1 if 0),
// where cached slots count as decoded byte * old scale; every valid slot is
// encoded as the nearest E4M3 code of fp32(value / scale) (ties to even,
// saturated at 448); slots past the new length keep their bytes.
//
// One wave per (sequence, touched page, kv head, K or V).  A (page, head)
// chunk is 16 * D bytes in the pool's layout; lane l owns its 16-byte units
// (K: units D/64 * l ..; V at D = 128: the two units of one slot group and
// 16-row block, so each slot's 8 new values are one 16-byte bf16 load), and
// the wave's stores cover the chunk in whole lines.
// New rows are read before anything that waits for the block table.  A unit
// is loaded only if it holds a cached slot or an untouched slot beside a new
// one, and stored only if it holds a new slot or a cached one whose scale
// changed (re-encoding with an unchanged scale reproduces the bytes).

#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "device_common.h"
#include "kernel_params.h"

namespace pa {

namespace {

constexpr int kAppendWaves = 4;

__device__ __forceinline__ float wave_max(float x) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) x = fmaxf(x, __shfl_xor(x, off));
  return x;
}

__device__ __forceinline__ int wave_sum(int x) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) x += __shfl_xor(x, off);
  return x;
}

// N consecutive new values (N = 16, 8 or 4) of one row.
template <bool F32IN, int N>
__device__ __forceinline__ void load_row(const void* base, int64_t off, float* v) {
  if constexpr (F32IN) {
    const u32x4* src = reinterpret_cast<const u32x4*>(static_cast<const float*>(base) + off);
#pragma unroll
    for (int k = 0; k < N / 4; ++k) {
      const u32x4 w = src[k];
#pragma unroll
      for (int e = 0; e < 4; ++e) v[4 * k + e] = __uint_as_float(w[e]);
    }
  } else {
    const uint16_t* src = static_cast<const uint16_t*>(base) + off;
    if constexpr (N == 16 || N == 8) {
      const u32x4* s4 = reinterpret_cast<const u32x4*>(src);
#pragma unroll
      for (int k = 0; k < N / 8; ++k) {
        const u32x4 w = s4[k];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          v[8 * k + 2 * e] = __uint_as_float(w[e] << 16);
          v[8 * k + 2 * e + 1] = __uint_as_float(w[e] & 0xffff0000u);
        }
      }
    } else {
      const uint2 w = *reinterpret_cast<const uint2*>(src);
      v[0] = __uint_as_float(w.x << 16);
      v[1] = __uint_as_float(w.x & 0xffff0000u);
      v[2] = __uint_as_float(w.y << 16);
      v[3] = __uint_as_float(w.y & 0xffff0000u);
    }
  }
}

// Four INT8 bytes (two's complement) -> four fp32 values, exactly.
__device__ __forceinline__ f32x4 i8x4_to_f32x4(uint32_t w) {
  f32x4 r;
#pragma unroll
  for (int e = 0; e < 4; ++e) r[e] = (float)(int8_t)(uint8_t)(w >> (8 * e));
  return r;
}

// Four fp32 -> four INT8 bytes: nearest integer, ties to even, clipped to
// +-127, two's complement (a in byte 0).
__device__ __forceinline__ uint32_t f32x4_to_i8x4(float a, float b, float c, float d) {
  const float x[4] = {a, b, c, d};
  uint32_t w = 0u;
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    const float q = __builtin_fminf(__builtin_fmaxf(__builtin_rintf(x[e]), -127.f), 127.f);
    w |= ((uint32_t)(int32_t)q & 0xffu) << (8 * e);
  }
  return w;
}

template <int D, bool F32IN, bool KI8>
__global__ __launch_bounds__(64 * kAppendWaves) void kv_append_kernel(AppendParams p) {
  constexpr int U = D / 64;     // 16-byte units per lane
  constexpr int NVB = D / 16;   // V: values of d per 16-row block
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int b = blockIdx.y;
  const int job = (int)blockIdx.x * kAppendWaves + wave;
  const int per_page = 2 * p.num_kv_heads;
  const int pi_local = job / per_page;
  const int rem = job - pi_local * per_page;
  const int h = rem >> 1;
  const bool is_v = (rem & 1) != 0;
  if (pi_local >= p.max_touch) return;
  const int L = p.ctx_lens[b];
  const int Q = p.q_lens[b];
  const int n0 = L - Q;                      // keys cached before the append
  const int pi = n0 / kPageSize + pi_local;  // page index inside the sequence
  if (pi * kPageSize >= L) return;
  int row0 = 0;  // first new row of sequence b
  for (int base = 0; base < b; base += 64) {
    const int i = base + lane;
    row0 += wave_sum(i < b ? p.q_lens[i] : 0);
  }
  const int32_t page = p.block_table[(int64_t)b * p.bt_stride + pi];
  const int valid = min(kPageSize, L - pi * kPageSize);
  const int n_old = max(0, min(kPageSize, n0 - pi * kPageSize));
  float* scale_at = p.kv_scales + (is_v ? p.v_scale_offset : 0) + (int64_t)page * p.num_kv_heads + h;
  const float old_scale = n_old > 0 ? *scale_at : 0.f;
  uint8_t* chunk = (is_v ? p.v_pages : p.k_pages) + chunk_offset(page, h, p.num_kv_heads, D);
  const void* rows = is_v ? p.v_new : p.k_new;
  const int64_t row_stride = (int64_t)p.num_kv_heads * D;

  // Unit u of lane l.  K: unit j = U l + u holds slot j % 16, d = 16 (j / 16)
  // + k at byte k.  V: with D = 128 the lane takes the two units of one
  // (slot group sg, a) with i = 0, 1, so that for each of its 4 slots the 8
  // values d = 8 a .. 8 a + 7 are consecutive in the new row; byte 4 e + r of
  // unit (sg, i, a) holds d = NVB a + 4 i + e of slot 4 sg + r.
  auto unit_of = [&](int u) -> int {
    if (is_v && D == 128) return ((lane >> 4) * 2 + u) * 16 + (lane & 15);
    return U * lane + u;
  };
  auto slot_lo = [&](int j) -> int { return is_v ? 4 * (j / (D / 4)) : j % 16; };
  auto slot_of = [&](int j, int k) -> int { return is_v ? slot_lo(j) + (k & 3) : j % 16; };
  float val[U][16];  // untouched slots keep 0 here (their bytes are restored)
#pragma unroll
  for (int u = 0; u < U; ++u)
#pragma unroll
    for (int k = 0; k < 16; ++k) val[u][k] = 0.f;
  u32x4 oldw[U];
  // new rows first: their addresses do not wait for the block table
#pragma unroll
  for (int u = 0; u < U; ++u) {
    const int j = unit_of(u);
    if (!is_v) {
      const int s = j % 16;
      if (s >= n_old && s < valid) {
        const int64_t r = row0 + (pi * kPageSize + s - n0);
        load_row<F32IN, 16>(rows, r * row_stride + (int64_t)h * D + 16 * (j / 16), val[u]);
      }
    } else if (D != 128) {
      const int d0 = NVB * (j % 16) + 4 * ((j / 16) % (D / 64));
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int s = slot_lo(j) + r;
        if (s >= n_old && s < valid) {
          float nv[4];
          load_row<F32IN, 4>(rows, (row0 + (pi * kPageSize + s - n0)) * row_stride + (int64_t)h * D + d0, nv);
#pragma unroll
          for (int e = 0; e < 4; ++e) val[u][4 * e + r] = nv[e];
        }
      }
    }
  }
  if constexpr (D == 128) {
    if (is_v) {
      // both units of the lane: slots 4 sg + r, d = 8 a + 4 u + e
      const int j0 = unit_of(0);
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int s = slot_lo(j0) + r;
        if (s >= n_old && s < valid) {
          float nv[8];
          load_row<F32IN, 8>(rows, (row0 + (pi * kPageSize + s - n0)) * row_stride + (int64_t)h * D +
                                       NVB * (lane & 15), nv);
#pragma unroll
          for (int u = 0; u < 2; ++u)
#pragma unroll
            for (int e = 0; e < 4; ++e) val[u][4 * e + r] = nv[4 * u + e];
        }
      }
    }
  }
  // cached and untouched bytes: a unit is read if it holds a cached slot, or
  // an untouched slot next to a new one (its bytes are written back)
  float amax = 0.f;
#pragma unroll
  for (int u = 0; u < U; ++u) {
    const int j = unit_of(u);
    const int s_lo = slot_lo(j);
    const int s_hi = is_v ? s_lo + 3 : s_lo;
    const bool has_new = s_hi >= n_old && s_lo < valid;
    const bool need_old = s_lo < n_old || (s_hi >= valid && has_new);
    oldw[u] = need_old ? *reinterpret_cast<const u32x4*>(chunk + 16 * j) : u32x4{0u, 0u, 0u, 0u};
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const f32x4 f = KI8 ? i8x4_to_f32x4(oldw[u][q]) : fp8x4_to_f32x4(oldw[u][q]);
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int k = 4 * q + e;
        const int s = slot_of(j, k);
        if (s < n_old) val[u][k] = f[e] * old_scale;
        if (s < valid) amax = fmaxf(amax, fabsf(val[u][k]));
      }
    }
  }
  amax = wave_max(amax);
  const float scale = (amax == 0.f) ? 1.f : amax / (KI8 ? 127.f : 448.f);
  const bool changed = n_old == 0 || __float_as_uint(scale) != __float_as_uint(old_scale);
  // value / scale, correctly rounded, without a full division per value:
  // y = 1/scale is correctly rounded (one IEEE division per wave); q0 = x y
  // is within two ulps of x / scale; one fma correction makes it faithful,
  // and a second gives the correctly rounded quotient (Markstein's theorem:
  // a correctly rounded reciprocal and a faithful quotient).  The residuals
  // x - q scale are exact fmas and stay normal for scales in [2^-90, 2^90];
  // other scales take the IEEE division.
  const bool fast_div = scale >= 0x1p-90f && scale <= 0x1p90f;
  const float rcp = 1.f / scale;
  auto quot = [&](float x) -> float {
    if (!fast_div) return x / scale;
    const float q0 = x * rcp;
    const float q1 = __builtin_fmaf(__builtin_fmaf(-q0, scale, x), rcp, q0);
    const float q2 = __builtin_fmaf(__builtin_fmaf(-q1, scale, x), rcp, q1);
    // the scale is positive, so the quotient has x's sign; the corrections
    // would turn a -0 quotient into +0 (-0 + +0 is +0)
    return __builtin_copysignf(q2, x);
  };

#pragma unroll
  for (int u = 0; u < U; ++u) {
    const int j = unit_of(u);
    const int s_lo = slot_lo(j);
    const int s_hi = is_v ? s_lo + 3 : s_lo;
    const bool has_new = s_hi >= n_old && s_lo < valid;
    const bool has_old = s_lo < n_old;
    if (!(has_new || (changed && has_old))) continue;
    u32x4 w;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      float y[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) y[e] = quot(val[u][4 * q + e]);
      const uint32_t enc = KI8 ? f32x4_to_i8x4(y[0], y[1], y[2], y[3]) : f32x4_to_fp8x4(y[0], y[1], y[2], y[3]);
      // bytes of slots at or past the new length keep their old value
      uint32_t keep = 0u;
#pragma unroll
      for (int e = 0; e < 4; ++e)
        if (slot_of(j, 4 * q + e) >= valid) keep |= 0xffu << (8 * e);
      w[q] = (enc & ~keep) | (oldw[u][q] & keep);
    }
    *reinterpret_cast<u32x4*>(chunk + 16 * j) = w;
  }
  if (lane == 0) *scale_at = scale;
}

// one thread per 4 values
__global__ __launch_bounds__(256) void debug_encode_kernel(const float* in, uint8_t* out, int64_t n) {
  const int64_t i0 = ((int64_t)blockIdx.x * blockDim.x + threadIdx.x) * 4;
  if (i0 >= n) return;
  float x[4] = {0.f, 0.f, 0.f, 0.f};
  for (int k = 0; k < 4 && i0 + k < n; ++k) x[k] = in[i0 + k];
  const uint32_t w = f32x4_to_fp8x4(x[0], x[1], x[2], x[3]);
  for (int k = 0; k < 4 && i0 + k < n; ++k) out[i0 + k] = (uint8_t)(w >> (8 * k));
}

}  // namespace

template <int D>
static const void* append_kernel(bool new_f32, bool kv_int8) {
  if (kv_int8)
    return new_f32 ? reinterpret_cast<const void*>(&kv_append_kernel<D, true, true>)
                   : reinterpret_cast<const void*>(&kv_append_kernel<D, false, true>);
  return new_f32 ? reinterpret_cast<const void*>(&kv_append_kernel<D, true, false>)
                 : reinterpret_cast<const void*>(&kv_append_kernel<D, false, false>);
}

hipError_t launch_kv_append(const AppendParams& p, int head_dim, bool new_f32, bool kv_int8, hipStream_t stream,
                            hipEvent_t ev_start, hipEvent_t ev_stop) {
  const int64_t jobs = (int64_t)p.max_touch * 2 * p.num_kv_heads;
  const int64_t gx = (jobs + kAppendWaves - 1) / kAppendWaves;
  if (gx <= 0 || p.num_seqs <= 0) return hipSuccess;
  if (gx > 0x7fffffff || p.num_seqs > 65535) return hipErrorInvalidValue;
  const void* fn = head_dim == 128 ? append_kernel<128>(new_f32, kv_int8) : append_kernel<64>(new_f32, kv_int8);
  AppendParams copy = p;
  void* args[] = {&copy};
  return hipExtLaunchKernel(fn, dim3((unsigned)gx, (unsigned)p.num_seqs), dim3(64 * kAppendWaves), args, 0, stream,
                            ev_start, ev_stop, 0);
}

hipError_t launch_debug_encode(const float* in, uint8_t* out, int64_t n, hipStream_t stream) {
  if (n <= 0) return hipSuccess;
  const int64_t threads = (n + 3) / 4;
  const int64_t blocks = (threads + 255) / 256;
  if (blocks > 0x7fffffff) return hipErrorInvalidValue;
  hipLaunchKernelGGL(debug_encode_kernel, dim3((unsigned)blocks), dim3(256), 0, stream, in, out, n);
  return hipGetLastError();
}

}  // namespace pa
