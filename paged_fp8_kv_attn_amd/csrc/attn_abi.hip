// Host side of the C ABI (include/pagedattn.h): descriptor validation, the
// plan's tile/split choice and one-time workspace allocation, and the
// stream-ordered forward.
//
// The plan object follows the memory section of the Atlas engine article
// (ainews.cool, "技术深度解析"): everything the forward needs is allocated
// once up front, and the forward itself allocates nothing and never
// synchronises the host.  Tile and split sizes are chosen from the static
// shape once, the "block sizes adapted to sequence length and GPU" of its
// attention section, here for gfx950 only.

#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <cstdint>
#include <cstring>
#include <mutex>
#include <new>

#include "../../include/pagedattn.h"
#include "kernel_params.h"

struct attn_plan_s {
  attn_plan_desc_t desc;
  pa::Variant variant;
  int device;
  int group;
  int cols_per_block;
  int col_blocks;
  int num_segments;  // (sequence, kv head, column block) units
  int grid;          // attention workgroups
  int max_units;     // waves (packed) or workgroups sharing the key chunks
  int unit_min_chunks;  // chunks per unit at least (within [1, max_units] units)
  int start_cost;       // chunks a segment's start counts for in the balanced split
  bool whole_ok;        // the tile kernel may give each unit one segment whole
  int piece_chunks;     // > 0: every segment cut into fixed pieces of this many chunks
  int piece_log2;       // log2(piece_chunks), a power of two
  uint64_t* timeline;   // null, or the caller's timeline rows
  int wallclock_khz;    // rate of the timeline's counter
  int occupancy;     // resident attention workgroups per compute unit
  int num_cus;
  float sm_scale;
  void* workspace;
  size_t workspace_bytes;
  size_t ws_o_bytes, ws_ml_bytes, ws_r0_bytes;  // byte sizes of the workspace's parts
  float* part_o;
  float* part_ml;
  int32_t* seq_row0;
  int2* seg_merge;
  int merge_grid;
  int merge_cols;  // query columns per merge workgroup
  hipEvent_t ev_start;  // optional: recorded around the attention kernel
  hipEvent_t ev_stop;
  hipEvent_t mev_start;  // optional: recorded around the merge kernel
  hipEvent_t mev_stop;
};

namespace {

thread_local int g_last_hip_error = 0;

attn_status_t hip_fail(hipError_t e) {
  g_last_hip_error = static_cast<int>(e);
  return ATTN_ERR_HIP;
}

bool aligned(const void* p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) & (a - 1)) == 0; }

int ceil_div(int64_t a, int64_t b) { return static_cast<int>((a + b - 1) / b); }

size_t round_up256(size_t x) { return (x + 255) & ~static_cast<size_t>(255); }

constexpr int kChunkTokens = 32;  // keys per chunk (two pages)
constexpr int kMinChunksPerGroup = 16;  // a workgroup's share is at least 4 chunks per wave
constexpr int kMinChunksPerWave = 8;    // a wave's share in the packed layout
// A shared-KV workgroup's share: at least 16 chunks (128 KB of K+V at
// D = 128).  Wide column blocks write large partials (columns x D fp32) at
// each piece boundary, but with fewer, longer units too few waves share a
// compute unit to hide the latency of each chunk's load-convert-compute
// chain (measured on MI355X: 16 beats 32 by 15-20% on MTP verification
// and MQA decode, 8 gains nothing more).
#ifndef TILE_MIN_CHUNKS
#define TILE_MIN_CHUNKS 16
#endif
constexpr int kMinChunksPerTile = TILE_MIN_CHUNKS;
constexpr int kStartCostPacked = 1;  // chunks a segment start counts for (see choose_plan)
constexpr int kStartCostTile = 3;

attn_status_t validate_desc(const attn_plan_desc_t& d) {
  for (int r : d.reserved)
    if (r != 0) return ATTN_ERR_INVALID_ARGUMENT;
  if (d.num_seqs < 1 || d.num_kv_heads < 1 || d.num_q_heads < 1) return ATTN_ERR_INVALID_ARGUMENT;
  if (d.num_q_heads % d.num_kv_heads != 0) return ATTN_ERR_INVALID_ARGUMENT;
  if (d.num_pages < 1 || d.max_q_len < 1 || d.max_ctx_len < d.max_q_len) return ATTN_ERR_INVALID_ARGUMENT;
  if (d.page_size < 1 || d.head_dim < 1) return ATTN_ERR_INVALID_ARGUMENT;
  if (d.max_pages_per_seq < 1) return ATTN_ERR_INVALID_ARGUMENT;
  if (d.q_dtype != ATTN_DTYPE_F32 && d.q_dtype != ATTN_DTYPE_BF16) return ATTN_ERR_INVALID_ARGUMENT;
  if (d.out_dtype != ATTN_DTYPE_F32 && d.out_dtype != ATTN_DTYPE_BF16) return ATTN_ERR_INVALID_ARGUMENT;
  if (!(d.sm_scale >= 0.f) || !std::isfinite(d.sm_scale)) return ATTN_ERR_INVALID_ARGUMENT;
  if (d.num_kv_splits < 0) return ATTN_ERR_INVALID_ARGUMENT;
  if (d.kv_piece_len < 0 || d.kv_piece_len % kChunkTokens != 0) return ATTN_ERR_INVALID_ARGUMENT;
  const int piece_chunks = d.kv_piece_len / kChunkTokens;
  if ((piece_chunks & (piece_chunks - 1)) != 0) return ATTN_ERR_INVALID_ARGUMENT;  // a power of two
  if (d.kv_piece_len > 0 && d.num_kv_splits > 0) return ATTN_ERR_INVALID_ARGUMENT;
  if (d.kv_format != ATTN_KV_E4M3 && d.kv_format != ATTN_KV_INT8 && d.kv_format != ATTN_KV_INT4)
    return ATTN_ERR_INVALID_ARGUMENT;
  if (d.kv_format != ATTN_KV_E4M3 && (d.q_dtype != ATTN_DTYPE_BF16 || d.out_dtype != ATTN_DTYPE_BF16))
    return ATTN_ERR_UNSUPPORTED;
  if (d.kv_format == ATTN_KV_INT4 && d.head_dim != 128) return ATTN_ERR_UNSUPPORTED;
  if (d.page_size != pa::kPageSize) return ATTN_ERR_UNSUPPORTED;
  if (d.head_dim != 64 && d.head_dim != 128) return ATTN_ERR_UNSUPPORTED;
  if (static_cast<int64_t>(d.max_pages_per_seq) * d.page_size < d.max_ctx_len) return ATTN_ERR_INVALID_ARGUMENT;
  return ATTN_OK;
}

// The plan's choices for desc on `device` -- column tiles, kernel variant,
// units, grid, merge shape and the workspace size -- with no allocation and
// no device work; p->workspace and the pointers into it stay null.
attn_status_t choose_plan(const attn_plan_desc_t& d, int device, attn_plan_s* p) {
  p->desc = d;
  p->device = device;
  p->group = d.num_q_heads / d.num_kv_heads;
  p->sm_scale = d.sm_scale > 0.f ? d.sm_scale : 1.0f / std::sqrt(static_cast<float>(d.head_dim));

  // Query columns of one (sequence, kv head): G heads x up to max_q_len tokens.
  const int64_t cols = static_cast<int64_t>(p->group) * d.max_q_len;
  pa::Variant v{};
  v.head_dim = d.head_dim;
  v.q_f32 = d.q_dtype == ATTN_DTYPE_F32;
  v.out_f32 = d.out_dtype == ATTN_DTYPE_F32;
  v.kv_format = d.kv_format;
  if (cols <= 4) {  // four pages per score tile
    v.col_tiles = 1;
    v.packed = true;
    v.packed_ring = 2;  // one wave per SIMD, two groups in flight; see below
    p->cols_per_block = static_cast<int>(cols);
  } else if (cols <= 8) {  // hi parts of P in columns 0..7, lo parts in 8..15
    v.col_tiles = 1;
    v.dup_lo = true;
    p->cols_per_block = static_cast<int>(cols);
  } else if (cols <= 16) {
    v.col_tiles = 1;
    p->cols_per_block = 16;
  } else if (cols <= 32) {  // two waves share each KV chunk, one tile each
    v.tile_waves = 2;
    v.col_tiles = 1;
    p->cols_per_block = 32;
  } else if (cols <= 64) {  // four waves, one tile each
    v.tile_waves = 4;
    v.col_tiles = 1;
    p->cols_per_block = 64;
  } else if (d.head_dim == 128) {
    // eight waves, two tiles each: 256-column blocks.  Against 128-column
    // blocks of four waves this halves how often each key is read (measured
    // on the 8 x 512 prefill chunk: half the L2 fetch, same time) and each
    // thread holds one 1 KB load per chunk instead of two.
    v.tile_waves = 8;
    v.col_tiles = 2;
    p->cols_per_block = 256;
  } else {  // four waves, two tiles each: 128-column blocks
    v.tile_waves = 4;
    v.col_tiles = 2;
    p->cols_per_block = 128;
  }
  p->col_blocks = ceil_div(cols, p->cols_per_block);
  p->variant = v;

  p->workspace = nullptr;
  p->workspace_bytes = 0;
  p->part_o = nullptr;
  p->part_ml = nullptr;
  p->seq_row0 = nullptr;
  p->seg_merge = nullptr;
  p->ev_start = nullptr;
  p->ev_stop = nullptr;
  p->mev_start = nullptr;
  p->mev_stop = nullptr;
  const int64_t segments = static_cast<int64_t>(d.num_seqs) * d.num_kv_heads * p->col_blocks;
  if (segments > 0x3fffffffLL || segments * p->cols_per_block > 0x3fffffffLL) return ATTN_ERR_UNSUPPORTED;
  p->num_segments = static_cast<int>(segments);

  // Workgroups of the attention kernel: by default as many as the GPU keeps
  // resident at once (every one then streams an equal share of the chunks in
  // a single round), and no more than one per kMinChunksPerGroup chunks of
  // the largest lengths, so that small problems are not split at all.
  hipError_t e = hipDeviceGetAttribute(&p->num_cus, hipDeviceAttributeMultiprocessorCount, device);
  if (e == hipSuccess) e = pa::stream_attention_occupancy(v, &p->occupancy);
  if (e == hipSuccess && v.packed && d.num_kv_splits > 0) {
    // Packed decode with two groups in flight holds one wave per SIMD; when a
    // forced split count asks for more units than that resident at once,
    // one group per wave at two waves per SIMD runs them in a single round.
    const int64_t resident = static_cast<int64_t>(p->num_cus) * std::max(p->occupancy, 1) * pa::kPackedWaves;
    const int64_t forced = static_cast<int64_t>(d.num_seqs) * d.num_kv_heads * d.num_kv_splits;
    if (forced > resident) {
      v.packed_ring = 1;
      p->variant = v;
      e = pa::stream_attention_occupancy(v, &p->occupancy);
    }
  }
  if (e != hipSuccess) return hip_fail(e);
  if (p->occupancy < 1) p->occupancy = 1;
  // Units sharing the chunks: waves for the packed decode layout (each wave
  // streams its own range), workgroups otherwise.  By default as many as
  // the GPU keeps resident at once, so that every unit streams an equal
  // share in a single round; the kernel uses one per unit_min_chunks chunks
  // of the actual lengths, at most that many.
  const int64_t seg_max_chunks = ceil_div(d.max_ctx_len, kChunkTokens);
  const int64_t max_chunks = segments * seg_max_chunks;
  // Fixed pieces: the positions the units share are pieces, at most
  // ceil(chunks / piece) per segment.
  p->piece_chunks = d.kv_piece_len / kChunkTokens;
  p->piece_log2 = 0;
  while ((1 << p->piece_log2) < p->piece_chunks) ++p->piece_log2;
  const int64_t seg_max_pieces = p->piece_chunks > 0 ? ceil_div(seg_max_chunks, p->piece_chunks) : 0;
  const int64_t max_positions = p->piece_chunks > 0 ? segments * seg_max_pieces : max_chunks;
  const int64_t wpg = pa::waves_per_group(v);
  const int64_t unit_waves = v.packed ? 1 : wpg;
  int64_t units;
  if (d.num_kv_splits > 0) {
    // forced: segments * n units, cut no finer than one chunk each
    units = segments * d.num_kv_splits;
    p->unit_min_chunks = 1;
  } else {
    units = static_cast<int64_t>(p->num_cus) * p->occupancy * wpg / unit_waves;
    p->unit_min_chunks = p->piece_chunks > 0 ? 1
                         : v.packed          ? kMinChunksPerWave
                         : v.tile_waves > 0  ? kMinChunksPerTile
                                             : kMinChunksPerGroup;
  }
  units = std::min<int64_t>(units, std::max<int64_t>(1, max_positions / p->unit_min_chunks));
  units = std::max<int64_t>(units, 1);
  if (units > 0x3fffffffLL) return ATTN_ERR_UNSUPPORTED;
  p->max_units = static_cast<int>(units);
  // A unit that begins a segment inside its range restarts its load
  // pipeline (block-table batch, then the first KV chunks; in the tile
  // kernels also the LDS staging): on the batch-32 decode shape, splits in
  // which a quarter of the waves do so ran 31.6-32.3 us against 30.0-30.2 us
  // for the same bytes with none.  The balanced split counts each segment
  // start as chunks, so those units stream that much less: one for the
  // packed decode (3 and 5 measured no better), three for the tile kernels,
  // whose restart also refills the ring and LDS staging (the prefill chunk
  // 420 us with 3 or 4 against 432 us with 2; MQA and MTP unchanged).  A
  // forced split count keeps its exact cut: n equal pieces of every segment.
  p->start_cost = d.num_kv_splits != 0 || p->piece_chunks > 0 ? 0 : (v.packed ? kStartCostPacked : kStartCostTile);
  // Where the segments are about as many as the units and of similar
  // lengths, the shared-KV tile kernel gives each unit one segment whole
  // (it decides from the lengths of each forward): the MTP verification
  // shape (1024 segments of 4-36 chunks) then ran 54.9-55.3 us per step
  // against 58.8-59.0 us for the balanced split (kernel 50.3-50.4 against
  // 48.6-49.0 us; the merge finds nothing to do).  Not with a forced split
  // count; with fixed pieces only where every segment is one piece (the
  // kernel checks).
  p->whole_ok = d.num_kv_splits == 0 && v.tile_waves > 0;
  p->timeline = nullptr;
  p->wallclock_khz = 0;
  if (hipDeviceGetAttribute(&p->wallclock_khz, hipDeviceAttributeWallClockRate, device) != hipSuccess)
    p->wallclock_khz = 0;
  p->grid = static_cast<int>(ceil_div(units * unit_waves, wpg));
  // merge: one workgroup per segment (and slice of its columns); segments
  // with many pieces on average get fewer columns per workgroup.  Fixed
  // pieces take the widest slices whatever the batch, so that the order in
  // which a segment's pieces are combined depends on their count alone.
  if (p->piece_chunks > 0) {
    p->merge_grid = seg_max_pieces > 1 ? p->num_segments : 0;
    p->merge_cols = pa::merge_cols_for(v, p->cols_per_block, 1);
  } else {
    p->merge_grid = units > 1 ? p->num_segments : 0;
    p->merge_cols = pa::merge_cols_for(v, p->cols_per_block, (units + segments - 1) / segments);
  }

  // Workspace: partial slots (segments + units of them, one per (segment,
  // unit) pair that can occur; with fixed pieces one per piece), each
  // sequence's first query row, and each segment's partial slots.
  const size_t slots = p->piece_chunks > 0 ? static_cast<size_t>(max_positions)
                                           : static_cast<size_t>(segments) + static_cast<size_t>(units);
  if (slots > 0x3fffffffULL) return ATTN_ERR_UNSUPPORTED;
  p->ws_o_bytes = round_up256(slots * p->cols_per_block * d.head_dim * sizeof(float));
  p->ws_ml_bytes = round_up256(slots * p->cols_per_block * 2 * sizeof(float));
  p->ws_r0_bytes = round_up256(static_cast<size_t>(d.num_seqs) * sizeof(int32_t));
  const size_t job_bytes = round_up256(static_cast<size_t>(segments) * 2 * sizeof(int32_t));
  p->workspace_bytes = p->ws_o_bytes + p->ws_ml_bytes + p->ws_r0_bytes + job_bytes;
  return ATTN_OK;
}

// Point the plan's partial buffers into `base` (workspace_bytes of device
// memory, 256-byte aligned).
void place_workspace(attn_plan_s* p, void* base) {
  char* ws = static_cast<char*>(base);
  p->workspace = base;
  p->part_o = reinterpret_cast<float*>(ws);
  ws += p->ws_o_bytes;
  p->part_ml = reinterpret_cast<float*>(ws);
  ws += p->ws_ml_bytes;
  p->seq_row0 = reinterpret_cast<int32_t*>(ws);
  ws += p->ws_r0_bytes;
  p->seg_merge = reinterpret_cast<int2*>(ws);
}

attn_status_t check_forward_args(const void* q, const uint8_t* k_pages, const uint8_t* v_pages,
                                 const float* kv_scales, const int32_t* block_table, const int32_t* ctx_lens,
                                 const int32_t* q_lens, const void* out) {
  if (!q || !k_pages || !v_pages || !kv_scales || !block_table || !ctx_lens || !q_lens || !out)
    return ATTN_ERR_INVALID_ARGUMENT;
  if (!aligned(q, 16) || !aligned(k_pages, 16) || !aligned(v_pages, 16) || !aligned(out, 16) ||
      !aligned(kv_scales, 4) || !aligned(block_table, 4) || !aligned(ctx_lens, 4) || !aligned(q_lens, 4))
    return ATTN_ERR_INVALID_ARGUMENT;
  return ATTN_OK;
}

// Enqueue the attention kernel, and the merge kernel when keys were split,
// of a plan whose workspace pointers are placed.
attn_status_t enqueue_forward(const attn_plan_s* plan, const void* q, const uint8_t* k_pages,
                              const uint8_t* v_pages, const float* kv_scales, const int32_t* block_table,
                              const int32_t* ctx_lens, const int32_t* q_lens, void* out, hipStream_t stream) {
  const attn_plan_desc_t& d = plan->desc;
  pa::StreamParams sp{};
  sp.q = q;
  sp.k_pages = k_pages;
  sp.v_pages = v_pages;
  sp.kv_scales = kv_scales;
  sp.block_table = block_table;
  sp.ctx_lens = ctx_lens;
  sp.q_lens = q_lens;
  sp.out = out;
  sp.part_o = plan->part_o;
  sp.part_ml = plan->part_ml;
  sp.num_seqs = d.num_seqs;
  sp.num_q_heads = d.num_q_heads;
  sp.num_kv_heads = d.num_kv_heads;
  sp.group = plan->group;
  sp.bt_stride = d.max_pages_per_seq;
  sp.max_q_len = d.max_q_len;
  sp.cols_per_block = plan->cols_per_block;
  sp.col_blocks = plan->col_blocks;
  sp.merge_cols = plan->merge_cols;
  sp.unit_min_chunks = plan->unit_min_chunks;
  sp.max_units = plan->max_units;
  sp.start_cost = plan->start_cost;
  sp.whole_ok = plan->whole_ok ? 1 : 0;
  sp.piece_chunks = plan->piece_chunks;
  sp.piece_log2 = plan->piece_log2;
  sp.timeline = reinterpret_cast<unsigned long long*>(plan->timeline);
  sp.seq_row0 = plan->seq_row0;
  sp.seg_merge = plan->seg_merge;
  sp.v_scale_offset = static_cast<int64_t>(d.num_pages) * d.num_kv_heads;
  sp.qk_scale_log2 = plan->sm_scale * 1.4426950408889634f;

  hipError_t e = pa::launch_stream_attention(plan->variant, sp, plan->grid, stream, plan->ev_start, plan->ev_stop);
  if (e == hipSuccess && plan->merge_grid > 0) {
    e = pa::launch_split_merge(plan->variant, sp, plan->merge_grid, stream, plan->mev_start, plan->mev_stop);
  } else if (e == hipSuccess && plan->mev_start) {
    // no merge launched: both events mark the same point of the stream
    e = hipEventRecord(plan->mev_start, stream);
    if (e == hipSuccess) e = hipEventRecord(plan->mev_stop, stream);
  }
  return e == hipSuccess ? ATTN_OK : hip_fail(e);
}

// ---- the allocation-free forward's scratch ---------------------------------
// Device memory that attn_paged_forward_static uses in place of a plan's
// workspace: one file-scope array per GPU, held until the process ends.  In
// host code the array's name is only a stand-in for the symbol: its device
// address comes from hipGetSymbolAddress, taken once per device with that
// device current, and only that address is passed to kernels.
constexpr size_t kStaticScratchBytes = size_t{32} << 20;
__device__ __align__(256) uint8_t scratch[kStaticScratchBytes];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

// The scratch address on `device` (current), looked up on the first call.
attn_status_t static_scratch(int device, void** ptr) {
  if (device < 0 || device >= kMaxDevices) return ATTN_ERR_UNSUPPORTED;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[device]) {
    void* a = nullptr;
    const hipError_t e = hipGetSymbolAddress(&a, HIP_SYMBOL(scratch));
    if (e != hipSuccess || !a) return hip_fail(e != hipSuccess ? e : hipErrorInvalidSymbol);
    g_scratch_ptr[device] = a;
  }
  *ptr = g_scratch_ptr[device];
  return ATTN_OK;
}

}  // namespace

extern "C" {

const char* attn_status_string(attn_status_t s) {
  switch (s) {
    case ATTN_OK: return "ATTN_OK: success";
    case ATTN_ERR_INVALID_ARGUMENT: return "ATTN_ERR_INVALID_ARGUMENT: null/misaligned pointer or inconsistent descriptor";
    case ATTN_ERR_UNSUPPORTED: return "ATTN_ERR_UNSUPPORTED: request outside what this library implements";
    case ATTN_ERR_OUT_OF_MEMORY: return "ATTN_ERR_OUT_OF_MEMORY: workspace allocation failed";
    case ATTN_ERR_HIP: return "ATTN_ERR_HIP: a HIP runtime call failed (see attn_last_hip_error)";
  }
  return "unknown attn_status_t";
}

int attn_last_hip_error(void) { return g_last_hip_error; }

attn_status_t attn_plan_create(const attn_plan_desc_t* desc, attn_plan_t* out_plan) {
  if (!desc || !out_plan) return ATTN_ERR_INVALID_ARGUMENT;
  *out_plan = nullptr;
  const attn_status_t st = validate_desc(*desc);
  if (st != ATTN_OK) return st;
  int device = 0;
  if (hipGetDevice(&device) != hipSuccess) return hip_fail(hipGetLastError());

  attn_plan_s* p = new (std::nothrow) attn_plan_s();
  if (!p) return ATTN_ERR_OUT_OF_MEMORY;
  const attn_status_t cs = choose_plan(*desc, device, p);
  if (cs != ATTN_OK) {
    delete p;
    return cs;
  }
  // the workspace, allocated once
  void* ws = nullptr;
  const hipError_t e = hipMalloc(&ws, p->workspace_bytes);
  if (e != hipSuccess) {
    (void)hipGetLastError();
    delete p;
    return e == hipErrorOutOfMemory ? ATTN_ERR_OUT_OF_MEMORY : hip_fail(e);
  }
  place_workspace(p, ws);
  *out_plan = p;
  return ATTN_OK;
}

attn_status_t attn_plan_destroy(attn_plan_t plan) {
  if (!plan) return ATTN_OK;
  attn_status_t st = ATTN_OK;
  if (plan->workspace) {
    const hipError_t e = hipFree(plan->workspace);
    if (e != hipSuccess) st = hip_fail(e);
  }
  delete plan;
  return st;
}

attn_status_t attn_plan_get_info(attn_plan_t plan, attn_plan_info_t* info) {
  if (!plan || !info) return ATTN_ERR_INVALID_ARGUMENT;
  info->col_tiles = plan->variant.col_tiles;
  info->dup_lo_columns = plan->variant.dup_lo ? 1 : 0;
  info->cols_per_block = plan->cols_per_block;
  info->col_blocks = plan->col_blocks;
  info->waves_per_group = pa::waves_per_group(plan->variant);
  info->num_segments = plan->num_segments;
  info->grid_size = plan->grid;
  info->merge_grid_size = plan->merge_grid;
  info->work_units = plan->max_units;
  info->packed = plan->variant.packed ? plan->variant.packed_ring : 0;
  info->shared_kv = plan->variant.tile_waves > 0 ? 1 : 0;
  info->resident_groups_per_cu = plan->occupancy;
  info->compute_units = plan->num_cus;
  info->workspace_bytes = plan->workspace_bytes;
  info->wallclock_khz = plan->wallclock_khz;
  return ATTN_OK;
}

static_assert(pa::kTimelineSlots == ATTN_TIMELINE_WORDS, "timeline row length");

attn_status_t attn_plan_set_timeline(attn_plan_t plan, uint64_t* rows, size_t num_rows) {
  if (!plan) return ATTN_ERR_INVALID_ARGUMENT;
  if (rows) {
    if (!pa::timeline_supported(plan->variant)) return ATTN_ERR_UNSUPPORTED;
    const size_t need = static_cast<size_t>(plan->grid) * pa::waves_per_group(plan->variant);
    if (num_rows < need || !aligned(rows, 8)) return ATTN_ERR_INVALID_ARGUMENT;
  }
  plan->timeline = rows;
  return ATTN_OK;
}

attn_status_t attn_plan_set_kernel_events(attn_plan_t plan, hipEvent_t attention_start, hipEvent_t attention_stop) {
  if (!plan) return ATTN_ERR_INVALID_ARGUMENT;
  if ((attention_start == nullptr) != (attention_stop == nullptr)) return ATTN_ERR_INVALID_ARGUMENT;
  plan->ev_start = attention_start;
  plan->ev_stop = attention_stop;
  return ATTN_OK;
}

attn_status_t attn_plan_set_merge_events(attn_plan_t plan, hipEvent_t merge_start, hipEvent_t merge_stop) {
  if (!plan) return ATTN_ERR_INVALID_ARGUMENT;
  if ((merge_start == nullptr) != (merge_stop == nullptr)) return ATTN_ERR_INVALID_ARGUMENT;
  plan->mev_start = merge_start;
  plan->mev_stop = merge_stop;
  return ATTN_OK;
}

static attn_status_t check_device(const attn_plan_s* plan) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess) return hip_fail(hipGetLastError());
  return dev == plan->device ? ATTN_OK : ATTN_ERR_INVALID_ARGUMENT;
}

attn_status_t attn_paged_forward(attn_plan_t plan, const void* q, const uint8_t* k_pages, const uint8_t* v_pages,
                                 const float* kv_scales, const int32_t* block_table, const int32_t* ctx_lens,
                                 const int32_t* q_lens, void* out, hipStream_t stream) {
  if (!plan) return ATTN_ERR_INVALID_ARGUMENT;
  const attn_status_t ast = check_forward_args(q, k_pages, v_pages, kv_scales, block_table, ctx_lens, q_lens, out);
  if (ast != ATTN_OK) return ast;
  const attn_status_t dst = check_device(plan);
  if (dst != ATTN_OK) return dst;
  return enqueue_forward(plan, q, k_pages, v_pages, kv_scales, block_table, ctx_lens, q_lens, out, stream);
}

attn_status_t attn_paged_forward_static(const attn_plan_desc_t* desc, const void* q, const uint8_t* k_pages,
                                        const uint8_t* v_pages, const float* kv_scales, const int32_t* block_table,
                                        const int32_t* ctx_lens, const int32_t* q_lens, void* out,
                                        hipStream_t stream) {
  if (!desc) return ATTN_ERR_INVALID_ARGUMENT;
  const attn_status_t vst = validate_desc(*desc);
  if (vst != ATTN_OK) return vst;
  const attn_status_t ast = check_forward_args(q, k_pages, v_pages, kv_scales, block_table, ctx_lens, q_lens, out);
  if (ast != ATTN_OK) return ast;
  int device = 0;
  if (hipGetDevice(&device) != hipSuccess) return hip_fail(hipGetLastError());
  void* ws = nullptr;
  const attn_status_t sst = static_scratch(device, &ws);
  if (sst != ATTN_OK) return sst;
  // the same choices as attn_plan_create, in a plan on the stack
  attn_plan_s plan;
  const attn_status_t cst = choose_plan(*desc, device, &plan);
  if (cst != ATTN_OK) return cst;
  if (plan.workspace_bytes > kStaticScratchBytes) return ATTN_ERR_UNSUPPORTED;
  place_workspace(&plan, ws);
  return enqueue_forward(&plan, q, k_pages, v_pages, kv_scales, block_table, ctx_lens, q_lens, out, stream);
}

size_t attn_static_scratch_bytes(void) { return kStaticScratchBytes; }

attn_status_t attn_debug_gather(attn_plan_t plan, const uint8_t* k_pages, const uint8_t* v_pages,
                                const float* kv_scales, const int32_t* block_table, const int32_t* ctx_lens,
                                uint8_t* k_out, uint8_t* v_out, float* scale_out, int32_t* page_out,
                                hipStream_t stream) {
  if (!plan || !k_pages || !v_pages || !kv_scales || !block_table || !ctx_lens || !k_out || !v_out ||
      !scale_out || !page_out)
    return ATTN_ERR_INVALID_ARGUMENT;
  if (!aligned(kv_scales, 4) || !aligned(block_table, 4) || !aligned(ctx_lens, 4) || !aligned(scale_out, 4) ||
      !aligned(page_out, 4))
    return ATTN_ERR_INVALID_ARGUMENT;
  const attn_status_t dst = check_device(plan);
  if (dst != ATTN_OK) return dst;
  const attn_plan_desc_t& d = plan->desc;
  pa::GatherParams gp{};
  gp.k_pages = k_pages;
  gp.v_pages = v_pages;
  gp.kv_scales = kv_scales;
  gp.block_table = block_table;
  gp.ctx_lens = ctx_lens;
  gp.k_out = k_out;
  gp.v_out = v_out;
  gp.scale_out = scale_out;
  gp.page_out = page_out;
  gp.num_seqs = d.num_seqs;
  gp.num_kv_heads = d.num_kv_heads;
  gp.head_dim = d.head_dim;
  gp.bt_stride = d.max_pages_per_seq;
  gp.max_ctx_len = d.max_ctx_len;
  gp.v_scale_offset = static_cast<int64_t>(d.num_pages) * d.num_kv_heads;
  gp.kv_format = d.kv_format;
  const hipError_t e = pa::launch_debug_gather(gp, stream);
  return e == hipSuccess ? ATTN_OK : hip_fail(e);
}

attn_status_t attn_kv_append(attn_plan_t plan, const void* k_new, const void* v_new, attn_dtype_t new_dtype,
                             uint8_t* k_pages, uint8_t* v_pages, float* kv_scales, const int32_t* block_table,
                             const int32_t* ctx_lens, const int32_t* q_lens, hipStream_t stream) {
  if (!plan || !k_new || !v_new || !k_pages || !v_pages || !kv_scales || !block_table || !ctx_lens || !q_lens)
    return ATTN_ERR_INVALID_ARGUMENT;
  if (new_dtype != ATTN_DTYPE_F32 && new_dtype != ATTN_DTYPE_BF16) return ATTN_ERR_INVALID_ARGUMENT;
  if (!aligned(k_new, 16) || !aligned(v_new, 16) || !aligned(k_pages, 16) || !aligned(v_pages, 16) ||
      !aligned(kv_scales, 4) || !aligned(block_table, 4) || !aligned(ctx_lens, 4) || !aligned(q_lens, 4))
    return ATTN_ERR_INVALID_ARGUMENT;
  const attn_status_t dst = check_device(plan);
  if (dst != ATTN_OK) return dst;
  const attn_plan_desc_t& d = plan->desc;
  if (d.kv_format == ATTN_KV_INT4) return ATTN_ERR_UNSUPPORTED;
  pa::AppendParams ap{};
  ap.k_new = k_new;
  ap.v_new = v_new;
  ap.k_pages = k_pages;
  ap.v_pages = v_pages;
  ap.kv_scales = kv_scales;
  ap.block_table = block_table;
  ap.ctx_lens = ctx_lens;
  ap.q_lens = q_lens;
  ap.num_seqs = d.num_seqs;
  ap.num_kv_heads = d.num_kv_heads;
  ap.bt_stride = d.max_pages_per_seq;
  // Q new keys starting anywhere in a page span at most ceil(Q/16) + 1 pages
  ap.max_touch = std::min<int>(ceil_div(d.max_q_len, pa::kPageSize) + 1, d.max_pages_per_seq);
  ap.v_scale_offset = static_cast<int64_t>(d.num_pages) * d.num_kv_heads;
  const hipError_t e = pa::launch_kv_append(ap, d.head_dim, new_dtype == ATTN_DTYPE_F32,
                                            d.kv_format == ATTN_KV_INT8, stream, plan->ev_start, plan->ev_stop);
  return e == hipSuccess ? ATTN_OK : hip_fail(e);
}

size_t attn_mtp_accept_workspace_size(int32_t num_seqs, int32_t num_drafts, int32_t vocab) {
  if (num_seqs < 1 || num_drafts < 0 || vocab < 8) return 0;
  const int64_t rows = static_cast<int64_t>(num_seqs) * (num_drafts + 1);
  return static_cast<size_t>(rows) * pa::accept_segments(rows, vocab) * sizeof(uint64_t);
}

attn_status_t attn_mtp_accept(const void* logits, attn_dtype_t logits_dtype, const int32_t* draft_tokens,
                              int32_t num_seqs, int32_t num_drafts, int32_t vocab, int32_t* target_tokens,
                              int32_t* num_accepted, void* workspace, size_t workspace_bytes,
                              hipEvent_t kernel_start, hipEvent_t kernel_stop, hipStream_t stream) {
  if (!logits || !target_tokens || !num_accepted || !workspace) return ATTN_ERR_INVALID_ARGUMENT;
  if (num_drafts > 0 && !draft_tokens) return ATTN_ERR_INVALID_ARGUMENT;
  if (logits_dtype != ATTN_DTYPE_F32 && logits_dtype != ATTN_DTYPE_BF16) return ATTN_ERR_INVALID_ARGUMENT;
  if (num_seqs < 1 || num_drafts < 0 || vocab < 8 || vocab % 8 != 0) return ATTN_ERR_INVALID_ARGUMENT;
  if ((kernel_start == nullptr) != (kernel_stop == nullptr)) return ATTN_ERR_INVALID_ARGUMENT;
  const int64_t rows = static_cast<int64_t>(num_seqs) * (num_drafts + 1);
  if (rows > 65535) return ATTN_ERR_UNSUPPORTED;
  if (!aligned(logits, 16) || !aligned(workspace, 8) || !aligned(target_tokens, 4) || !aligned(num_accepted, 4) ||
      (draft_tokens && !aligned(draft_tokens, 4)))
    return ATTN_ERR_INVALID_ARGUMENT;
  if (workspace_bytes < attn_mtp_accept_workspace_size(num_seqs, num_drafts, vocab)) return ATTN_ERR_INVALID_ARGUMENT;
  pa::AcceptParams ap{};
  ap.logits = logits;
  ap.drafts = draft_tokens;
  ap.target_tokens = target_tokens;
  ap.num_accepted = num_accepted;
  ap.partial = static_cast<uint64_t*>(workspace);
  ap.num_seqs = num_seqs;
  ap.num_drafts = num_drafts;
  ap.vocab = vocab;
  ap.segments = pa::accept_segments(rows, vocab);
  const hipError_t e = pa::launch_mtp_accept(ap, logits_dtype == ATTN_DTYPE_F32, stream, kernel_start, kernel_stop);
  return e == hipSuccess ? ATTN_OK : hip_fail(e);
}

attn_status_t attn_calib_stream_read(const uint8_t* pool, int64_t pool_bytes, const int32_t* chunk_ids,
                                     int64_t num_chunks, int32_t chunk_bytes, int32_t waves, int32_t access,
                                     uint32_t* sink, hipEvent_t kernel_start, hipEvent_t kernel_stop,
                                     hipStream_t stream) {
  if (!pool || !chunk_ids || !sink) return ATTN_ERR_INVALID_ARGUMENT;
  if (chunk_bytes < 1024 || chunk_bytes > (1 << 24) || (chunk_bytes & (chunk_bytes - 1)) != 0)
    return ATTN_ERR_INVALID_ARGUMENT;
  if (pool_bytes < chunk_bytes || num_chunks < 1 || num_chunks > (int64_t{1} << 40) / chunk_bytes)
    return ATTN_ERR_INVALID_ARGUMENT;
  if (waves < 1 || waves > (1 << 20)) return ATTN_ERR_INVALID_ARGUMENT;
  if (access != 0 && (access != 1 || chunk_bytes < 2048)) return ATTN_ERR_INVALID_ARGUMENT;
  if ((kernel_start == nullptr) != (kernel_stop == nullptr)) return ATTN_ERR_INVALID_ARGUMENT;
  if (!aligned(pool, 16) || !aligned(chunk_ids, 4) || !aligned(sink, 4)) return ATTN_ERR_INVALID_ARGUMENT;
  const hipError_t e = pa::launch_stream_read(pool, pool_bytes, chunk_ids, num_chunks, chunk_bytes, waves, access,
                                              sink, stream, kernel_start, kernel_stop);
  return e == hipSuccess ? ATTN_OK : hip_fail(e);
}

attn_status_t attn_debug_encode_fp8(const float* in, uint8_t* out, int64_t n, hipStream_t stream) {
  if (n < 0) return ATTN_ERR_INVALID_ARGUMENT;
  if (n == 0) return ATTN_OK;
  if (!in || !out || !aligned(in, 4)) return ATTN_ERR_INVALID_ARGUMENT;
  const hipError_t e = pa::launch_debug_encode(in, out, n, stream);
  return e == hipSuccess ? ATTN_OK : hip_fail(e);
}

attn_status_t attn_debug_decode_fp8(const uint8_t* in, float* out, int64_t n, hipStream_t stream) {
  if (n < 0) return ATTN_ERR_INVALID_ARGUMENT;
  if (n == 0) return ATTN_OK;
  if (!in || !out || !aligned(out, 4)) return ATTN_ERR_INVALID_ARGUMENT;
  const hipError_t e = pa::launch_debug_decode(in, out, n, pa::kKvE4M3, stream);
  return e == hipSuccess ? ATTN_OK : hip_fail(e);
}

attn_status_t attn_debug_decode_int8(const uint8_t* in, float* out, int64_t n, hipStream_t stream) {
  if (n < 0) return ATTN_ERR_INVALID_ARGUMENT;
  if (n == 0) return ATTN_OK;
  if (!in || !out || !aligned(out, 4)) return ATTN_ERR_INVALID_ARGUMENT;
  const hipError_t e = pa::launch_debug_decode(in, out, n, pa::kKvInt8, stream);
  return e == hipSuccess ? ATTN_OK : hip_fail(e);
}

attn_status_t attn_debug_decode_int4(const uint8_t* in, float* out, int64_t n, hipStream_t stream) {
  if (n < 0) return ATTN_ERR_INVALID_ARGUMENT;
  if (n == 0) return ATTN_OK;
  if (!in || !out || !aligned(out, 4)) return ATTN_ERR_INVALID_ARGUMENT;
  const hipError_t e = pa::launch_debug_decode(in, out, n, pa::kKvInt4, stream);
  return e == hipSuccess ? ATTN_OK : hip_fail(e);
}

}  // extern "C"
