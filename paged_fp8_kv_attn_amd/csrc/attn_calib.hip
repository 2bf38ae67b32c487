// Measurement hook: the streaming-read ceiling that the attention kernels'
// HBM fraction is compared against.  It reads a list of equal-sized chunks
// scattered over a large pool -- the access pattern of a paged KV cache,
// where every (page, kv head) is one contiguous chunk at a random place --
// and nothing else: no arithmetic beyond an XOR that keeps the loads live.
//
// Wave w of W streams the 1 KB lines [floor(w N / W), floor((w+1) N / W))
// of the N lines the chunks hold, in list order, with 16-byte non-temporal
// loads kept NR deep in a ring of registers.  Access 0: the 64 lanes read
// one whole 1 KB run per instruction (eight whole 128-byte lines), the
// pattern of the library's page layouts.  Access 1: each 2 KB of a chunk is
// 16 rows of 128 bytes and lane (q, r) of a wave (q = lane / 16, r = lane %
// 16) reads bytes 32 q + 16 i of row r in instruction i = 0, 1, so every
// instruction touches half of 16 lines: the pattern a [16 slots][128 d]
// page layout gives a lane that holds 32 values of d of one slot.

#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "device_common.h"
#include "kernel_params.h"

namespace pa {

namespace {

constexpr int kCalibRing = 16;     // 1 KB lines in flight per wave
constexpr int kCalibWaves = 4;     // waves per workgroup

struct CalibParams {
  const uint8_t* pool;
  const int32_t* ids;
  int64_t pool_chunks;  // ids are clamped to [0, pool_chunks): no read leaves the pool
  int64_t num_lines;    // chunks * lines_per_chunk
  int32_t lpc_log2;     // log2(chunk_bytes / 1024)
  int32_t waves;
  int32_t access;       // 0: whole lines per instruction; 1: half lines
  uint32_t* sink;       // [waves * 64]
};

__global__ __launch_bounds__(64 * kCalibWaves) void stream_read_kernel(CalibParams p) {
  const int lane = threadIdx.x & 63;
  const int w = (int)blockIdx.x * kCalibWaves + __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  if (w >= p.waves) return;
  const int64_t lo = (int64_t)w * p.num_lines / p.waves;
  const int64_t n = (int64_t)(w + 1) * p.num_lines / p.waves - lo;
  auto addr = [&](int64_t line) {
    const int64_t c = line >> p.lpc_log2;
    int64_t id = p.ids[c];
    id = id < 0 ? 0 : (id >= p.pool_chunks ? p.pool_chunks - 1 : id);
    const int64_t li = line & ((1 << p.lpc_log2) - 1);  // 1 KB line inside the chunk
    const int64_t lane_off = p.access == 0 ? lane * 16
                                           : (li & ~int64_t{1}) * 1024 + (lane & 15) * 128 + (lane >> 4) * 32 +
                                                 (li & 1) * 16 - li * 1024;
    const int64_t off = ((id << p.lpc_log2) + li) * 1024 + lane_off;
    return reinterpret_cast<const u32x4*>(p.pool + off);
  };
  u32x4 acc = {0u, 0u, 0u, 0u};
  u32x4 buf[kCalibRing];
  constexpr int R = kCalibRing;
  if (n >= R) {
#pragma unroll
    for (int j = 0; j < R; ++j) buf[j] = __builtin_nontemporal_load(addr(lo + j));
    int64_t k = 0;
    // steady state: every consumption is followed by an unconditional refill
    for (; k + 2 * R <= n; k += R) {
#pragma unroll
      for (int j = 0; j < R; ++j) {
        acc ^= buf[j];
        buf[j] = __builtin_nontemporal_load(addr(lo + k + j + R));
      }
    }
#pragma unroll
    for (int j = 0; j < R; ++j) {
      acc ^= buf[j];
      if (k + j + R < n) buf[j] = __builtin_nontemporal_load(addr(lo + k + j + R));
    }
#pragma unroll
    for (int j = 0; j < R; ++j)
      if (k + R + j < n) acc ^= buf[j];
  } else {
    for (int64_t k = 0; k < n; ++k) acc ^= __builtin_nontemporal_load(addr(lo + k));
  }
  p.sink[(int64_t)w * 64 + lane] = acc[0] ^ acc[1] ^ acc[2] ^ acc[3];
}

}  // namespace

hipError_t launch_stream_read(const uint8_t* pool, int64_t pool_bytes, const int32_t* ids, int64_t num_chunks,
                              int32_t chunk_bytes, int32_t waves, int32_t access, uint32_t* sink, hipStream_t stream,
                              hipEvent_t ev_start, hipEvent_t ev_stop) {
  int lpc_log2 = 0;
  while ((1024 << lpc_log2) < chunk_bytes) ++lpc_log2;
  CalibParams p{};
  p.pool = pool;
  p.ids = ids;
  p.pool_chunks = pool_bytes / chunk_bytes;
  p.num_lines = num_chunks << lpc_log2;
  p.lpc_log2 = lpc_log2;
  p.waves = waves;
  p.access = access;
  p.sink = sink;
  const int grid = (waves + kCalibWaves - 1) / kCalibWaves;
  void* args[] = {&p};
  if (ev_start)
    return hipExtLaunchKernel(reinterpret_cast<const void*>(&stream_read_kernel), dim3(grid),
                              dim3(64 * kCalibWaves), args, 0, stream, ev_start, ev_stop, 0);
  return hipLaunchKernel(reinterpret_cast<const void*>(&stream_read_kernel), dim3(grid), dim3(64 * kCalibWaves),
                         args, 0, stream);
}

}  // namespace pa
