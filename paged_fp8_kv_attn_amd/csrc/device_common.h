// Device helpers shared by the attention kernels and the checking hooks, so
// that the hooks exercise exactly the address arithmetic and FP8 decode the
// attention kernels run.  gfx950 only.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "kernel_params.h"

namespace pa {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

// Byte offset of the (page, kv head) chunk in k_pages / v_pages: a chunk is
// the 16 tokens x D bytes of one head inside one page.
__device__ __forceinline__ uint64_t chunk_offset(int32_t page, int head, int num_kv_heads, int head_dim) {
  return ((uint64_t)(uint32_t)page * (uint64_t)num_kv_heads + (uint64_t)head) * (uint64_t)(kPageSize * head_dim);
}

// K chunk: 16-byte blocks of d, slot-major inside a block; the byte of
// (slot, d) sits at ((d / 16) * 16 + slot) * 16 + d % 16.  Sixteen lanes
// reading one 16-byte block each for slots 0..15 cover 256 contiguous bytes.
__device__ __forceinline__ uint32_t k_in_chunk(int slot, int d, int head_dim) {
  (void)head_dim;
  return (uint32_t)((((d >> 4) * kPageSize + slot) << 4) + (d & 15));
}

// V chunk: four consecutive slots interleaved per d.  With NVB = D / 16 and
// d = NVB * a + 4 * i + e, the byte of (slot, d) sits at
// ((((slot / 4) * (D / 64) + i) * 16 + a) * 4 + e) * 4 + slot % 4: a lane's
// 16-byte load holds 4 values of d times the 4 slots of its group, and the
// 16 lanes a = 0..15 read 256 contiguous bytes.
__device__ __forceinline__ uint32_t v_in_chunk(int slot, int d, int head_dim) {
  const int nvb = head_dim >> 4;
  const int a = d / nvb;
  const int r = d - a * nvb;
  return (uint32_t)((((((slot >> 2) * (head_dim >> 6) + (r >> 2)) * 16 + a) * 4 + (r & 3)) << 2) + (slot & 3));
}

// Two FP8 E4M3 bytes of `w` (bytes 0,1 or, with HI, bytes 2,3) -> two bf16,
// exactly: every E4M3 value is a bf16 value.  gfx950's converter reads the
// OCP E4M3 encoding; the scale operand 1.0 leaves values unchanged.
template <bool HI>
__device__ __forceinline__ bf16x2 fp8x2_to_bf16x2(uint32_t w) {
  return __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w, 1.0f, HI);
}

// Eight FP8 bytes (w0 bytes 0..3, then w1 bytes 0..3) -> eight bf16 in order.
__device__ __forceinline__ bf16x8 fp8x8_to_bf16x8(uint32_t w0, uint32_t w1) {
  const bf16x2 a = fp8x2_to_bf16x2<false>(w0);
  const bf16x2 b = fp8x2_to_bf16x2<true>(w0);
  const bf16x2 c = fp8x2_to_bf16x2<false>(w1);
  const bf16x2 d = fp8x2_to_bf16x2<true>(w1);
  return bf16x8{a[0], a[1], b[0], b[1], c[0], c[1], d[0], d[1]};
}

// Four fp32 -> four OCP E4M3 bytes (a in byte 0 .. d in byte 3), round to
// nearest even.  Magnitudes above 448 are clamped first, since the converter
// gives the NaN code for values past the largest finite one; -0 keeps its
// sign.  Inputs are finite.
__device__ __forceinline__ uint32_t f32x4_to_fp8x4(float a, float b, float c, float d) {
  auto sat = [](float x) { return __builtin_fminf(__builtin_fmaxf(x, -448.f), 448.f); };
  int w = __builtin_amdgcn_cvt_pk_fp8_f32(sat(a), sat(b), 0, false);
  w = __builtin_amdgcn_cvt_pk_fp8_f32(sat(c), sat(d), w, true);
  return (uint32_t)w;
}

// Four FP8 E4M3 bytes -> four fp32 values, exactly.
__device__ __forceinline__ f32x4 fp8x4_to_f32x4(uint32_t w) {
  const f32x2 lo = __builtin_amdgcn_cvt_pk_f32_fp8((int)w, false);
  const f32x2 hi = __builtin_amdgcn_cvt_pk_f32_fp8((int)w, true);
  return f32x4{lo[0], lo[1], hi[0], hi[1]};
}

// Four INT8 bytes (two's complement) -> four bf16, exactly: each byte is
// sign-extended and converted to fp32 (one v_cvt_f32_i32 with an SDWA byte
// select each), and every integer in [-128, 127] is a bf16 value.
__device__ __forceinline__ bf16x4 i8x4_to_bf16x4(uint32_t w) {
  float f[4];
#pragma unroll
  for (int e = 0; e < 4; ++e) f[e] = (float)(int)(int8_t)(uint8_t)(w >> (8 * e));
  const bf16x2 a = __builtin_convertvector(f32x2{f[0], f[1]}, bf16x2);
  const bf16x2 b = __builtin_convertvector(f32x2{f[2], f[3]}, bf16x2);
  return bf16x4{a[0], a[1], b[0], b[1]};
}

// Eight KV bytes -> eight bf16 in order: OCP E4M3 codes, or INT8 with KI8.
template <bool KI8>
__device__ __forceinline__ bf16x8 kv8x8_to_bf16x8(uint32_t w0, uint32_t w1) {
  if constexpr (KI8) {
    const bf16x4 a = i8x4_to_bf16x4(w0);
    const bf16x4 b = i8x4_to_bf16x4(w1);
    return bf16x8{a[0], a[1], a[2], a[3], b[0], b[1], b[2], b[3]};
  } else {
    return fp8x8_to_bf16x8(w0, w1);
  }
}

// Four KV bytes -> four bf16 in order.
template <bool KI8>
__device__ __forceinline__ bf16x4 kv8x4_to_bf16x4(uint32_t w) {
  if constexpr (KI8) {
    return i8x4_to_bf16x4(w);
  } else {
    const bf16x2 a = fp8x2_to_bf16x2<false>(w);
    const bf16x2 b = fp8x2_to_bf16x2<true>(w);
    return bf16x4{a[0], a[1], b[0], b[1]};
  }
}

// ---- KV formats (kKvE4M3, kKvInt8, kKvInt4: kernel_params.h) ----------------

// Bytes of one (page, kv head) chunk: 16 slots x D codes.
template <int KF>
__host__ __device__ constexpr int chunk_bytes(int head_dim) {
  return KF == kKvInt4 ? kPageSize * head_dim / 2 : kPageSize * head_dim;
}

// Byte offset of the (page, kv head) chunk in an INT4 pool.
__device__ __forceinline__ uint64_t chunk_offset4(int32_t page, int head, int num_kv_heads, int head_dim) {
  return ((uint64_t)(uint32_t)page * (uint64_t)num_kv_heads + (uint64_t)head) * (uint64_t)(kPageSize * head_dim / 2);
}

// INT4 chunks (D = 128): lane (lq, ln)'s 16 bytes start at (16 lq + ln) * 16
// in both pools.  K: quarter lq of d of slot ln, codes d = 32 lq + u in byte
// u / 2 (u even: low nibble).  V: the four slots 4 lq .. 4 lq + 3 of each
// d = 8 ln + r in the 16-bit half r (slot 4 lq + j in nibble j).
__device__ __forceinline__ uint32_t lane_in_chunk4(int lq, int ln) { return (uint32_t)((16 * lq + ln) * 16); }

// K code (0..15) of (slot, d) in an INT4 chunk, and V code: for the gather hook.
__device__ __forceinline__ uint32_t k4_code(const uint8_t* chunk, int slot, int d) {
  const int u = d & 31;
  return (chunk[lane_in_chunk4(d >> 5, slot) + (u >> 1)] >> (4 * (u & 1))) & 0xFu;
}
__device__ __forceinline__ uint32_t v4_code(const uint8_t* chunk, int slot, int d) {
  const int a = d >> 3, r = d & 7;
  return (chunk[lane_in_chunk4(slot >> 2, a) + 2 * r + ((slot & 3) >> 1)] >> (4 * (slot & 1))) & 0xFu;
}

__device__ __forceinline__ float sext_byte(uint32_t w, int e) { return (float)(int)(int8_t)(uint8_t)(w >> (8 * e)); }

// Eight INT4 codes (w: code j in bits 4j..4j+3) -> eight bf16 holding 16
// times their values, exactly: each code is moved to the top nibble of a
// byte and sign-extended as an INT8 byte.  The caller's scales carry 1/16.
__device__ __forceinline__ bf16x8 i4x8_to_bf16x8(uint32_t w) {
  const uint32_t lo = (w << 4) & 0xF0F0F0F0u;  // codes 0, 2, 4, 6
  const uint32_t hi = w & 0xF0F0F0F0u;         // codes 1, 3, 5, 7
  bf16x8 r;
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    const bf16x2 pr = __builtin_convertvector(f32x2{sext_byte(lo, e), sext_byte(hi, e)}, bf16x2);
    r[2 * e] = pr[0];
    r[2 * e + 1] = pr[1];
  }
  return r;
}

// Four INT4 codes (h: code j in bits 4j..4j+3, j < 4) -> four bf16 of 16
// times their values, exactly.
__device__ __forceinline__ bf16x4 i4x4_to_bf16x4(uint32_t h) {
  const uint32_t lo = (h << 4) & 0xF0F0u;  // codes 0, 2
  const uint32_t hi = h & 0xF0F0u;         // codes 1, 3
  const bf16x2 a = __builtin_convertvector(f32x2{sext_byte(lo, 0), sext_byte(hi, 0)}, bf16x2);
  const bf16x2 b = __builtin_convertvector(f32x2{sext_byte(lo, 1), sext_byte(hi, 1)}, bf16x2);
  return bf16x4{a[0], a[1], b[0], b[1]};
}

// The factor the decoded values carry: INT4 codes come out 16 times larger.
template <int KF>
__host__ __device__ constexpr float code_unit() {
  return KF == kKvInt4 ? 0.0625f : 1.0f;
}

__device__ __forceinline__ float bf16_bits_to_f32(uint32_t bits16) {
  return __uint_as_float(bits16 << 16);
}

}  // namespace pa
