// Greedy acceptance of multi-token-prediction drafts for gfx950: the step
// after the verification attention.  The GB10 article (ainews.surl.tw)
// serves with MTP, K = 4 drafts, under deterministic decoding: the target's
// token at each of the K + 1 positions is the argmax of its logits row, and
// the drafts are accepted along the longest prefix that equals them.
//
// argmax_partial_kernel: workgroup (s, r) scans segment s of logits row r
// with 16-byte loads, four in flight per thread; each thread keeps, per
// element position inside a vector, the largest value and the first vector
// holding it (strict >, so the lowest index wins), then the workgroup
// reduces 64-bit keys (order-preserving bits of the value, +0 for -0, above
// the inverted index) to one key per (row, segment).
// accept_kernel: one thread per sequence combines the keys of each row's
// segments (the largest key is the largest value at the lowest index), writes
// the K + 1 target tokens and counts the leading drafts equal to them.
// Integer maxima only: the result does not depend on scheduling.

#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "device_common.h"
#include "kernel_params.h"

namespace pa {

namespace {

constexpr int kArgmaxThreads = 256;
constexpr int kArgmaxUnroll = 4;

__device__ __forceinline__ uint64_t argmax_key(float v, uint32_t idx) {
  uint32_t u = __float_as_uint(v);
  if ((u << 1) == 0u) u = 0u;  // -0 and +0 are the same value
  const uint32_t ord = (u & 0x80000000u) ? ~u : (u | 0x80000000u);
  return ((uint64_t)ord << 32) | (uint64_t)(0xffffffffu - idx);
}

__device__ __forceinline__ uint64_t max64(uint64_t a, uint64_t b) { return a > b ? a : b; }

__device__ __forceinline__ uint64_t wave_max64(uint64_t x) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) {
    const uint32_t lo = __shfl_xor((uint32_t)x, off);
    const uint32_t hi = __shfl_xor((uint32_t)(x >> 32), off);
    x = max64(x, ((uint64_t)hi << 32) | lo);
  }
  return x;
}

template <bool F32>
__global__ __launch_bounds__(kArgmaxThreads) void argmax_partial_kernel(AcceptParams p) {
  constexpr int EPV = F32 ? 4 : 8;  // values per 16-byte vector
  const int s = blockIdx.x;
  const int64_t r = blockIdx.y;
  const int64_t nvec = p.vocab / EPV;
  const int64_t per = (nvec + p.segments - 1) / p.segments;
  const int64_t vbeg = s * per;
  const int64_t vend = min(nvec, vbeg + per);
  const u32x4* row = reinterpret_cast<const u32x4*>(static_cast<const char*>(p.logits) +
                                                    r * p.vocab * (F32 ? 4 : 2));
  float best[EPV];
  int64_t bvec[EPV];
#pragma unroll
  for (int j = 0; j < EPV; ++j) {
    best[j] = -__builtin_huge_valf();
    bvec[j] = -1;
  }
  auto take = [&](const u32x4& w, int64_t v) {
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      if constexpr (F32) {
        const float x = __uint_as_float(w[q]);
        if (x > best[q]) { best[q] = x; bvec[q] = v; }
      } else {
        const float lo = __uint_as_float(w[q] << 16);
        const float hi = __uint_as_float(w[q] & 0xffff0000u);
        if (lo > best[2 * q]) { best[2 * q] = lo; bvec[2 * q] = v; }
        if (hi > best[2 * q + 1]) { best[2 * q + 1] = hi; bvec[2 * q + 1] = v; }
      }
    }
  };
  int64_t v = vbeg + threadIdx.x;
  constexpr int STEP = kArgmaxThreads * kArgmaxUnroll;
  for (; v + (kArgmaxUnroll - 1) * kArgmaxThreads < vend; v += STEP) {
    u32x4 w[kArgmaxUnroll];
#pragma unroll
    for (int k = 0; k < kArgmaxUnroll; ++k) w[k] = __builtin_nontemporal_load(row + v + k * kArgmaxThreads);
#pragma unroll
    for (int k = 0; k < kArgmaxUnroll; ++k) take(w[k], v + k * kArgmaxThreads);
  }
  for (; v < vend; v += kArgmaxThreads) take(__builtin_nontemporal_load(row + v), v);

  uint64_t key = 0;  // below every value: an empty share
#pragma unroll
  for (int j = 0; j < EPV; ++j)
    if (bvec[j] >= 0) key = max64(key, argmax_key(best[j], (uint32_t)(bvec[j] * EPV + j)));
  key = wave_max64(key);
  __shared__ uint64_t part[kArgmaxThreads / 64];
  const int wave = threadIdx.x >> 6;
  if ((threadIdx.x & 63) == 0) part[wave] = key;
  __syncthreads();
  if (threadIdx.x == 0) {
    uint64_t k = part[0];
#pragma unroll
    for (int w2 = 1; w2 < kArgmaxThreads / 64; ++w2) k = max64(k, part[w2]);
    p.partial[r * p.segments + s] = k;
  }
}

__global__ __launch_bounds__(64) void accept_kernel(AcceptParams p) {
  const int b = blockIdx.x * 64 + threadIdx.x;
  if (b >= p.num_seqs) return;
  const int K = p.num_drafts;
  int n = 0;
  bool run = true;
  for (int i = 0; i <= K; ++i) {
    const int64_t r = (int64_t)b * (K + 1) + i;
    uint64_t k = 0;
    for (int s = 0; s < p.segments; ++s) k = max64(k, p.partial[r * p.segments + s]);
    const int32_t t = (int32_t)(0xffffffffu - (uint32_t)k);
    p.target_tokens[r] = t;
    if (i < K && run) {
      if (p.drafts[(int64_t)b * K + i] == t)
        ++n;
      else
        run = false;
    }
  }
  p.num_accepted[b] = n;
}

}  // namespace

int accept_segments(int64_t rows, int64_t vocab) {
  // enough workgroups to cover the GPU a few times over, each segment at
  // least 64 KB of bf16 logits
  int64_t s = (4096 + rows - 1) / rows;
  const int64_t max_s = vocab / 32768;
  if (s > max_s) s = max_s;
  if (s < 1) s = 1;
  if (s > 1024) s = 1024;
  return (int)s;
}

hipError_t launch_mtp_accept(const AcceptParams& p, bool f32, hipStream_t stream, hipEvent_t ev_start,
                             hipEvent_t ev_stop) {
  const int64_t rows = (int64_t)p.num_seqs * (p.num_drafts + 1);
  if (rows <= 0) return hipSuccess;
  if (rows > 65535) return hipErrorInvalidValue;
  AcceptParams copy = p;
  void* args[] = {&copy};
  const void* fn = f32 ? reinterpret_cast<const void*>(&argmax_partial_kernel<true>)
                       : reinterpret_cast<const void*>(&argmax_partial_kernel<false>);
  hipError_t e = hipExtLaunchKernel(fn, dim3((unsigned)p.segments, (unsigned)rows), dim3(kArgmaxThreads), args, 0,
                                    stream, ev_start, ev_stop, 0);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(accept_kernel, dim3((unsigned)((p.num_seqs + 63) / 64)), dim3(64), 0, stream, p);
  return hipGetLastError();
}

}  // namespace pa
