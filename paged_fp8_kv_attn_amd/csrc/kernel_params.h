// Parameter blocks passed by value from the host launcher to the kernels,
// and the launcher entry points (defined next to their kernels).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace pa {

constexpr int kPageSize = 16;  // tokens per page
constexpr int kTimelineSlots = 64;  // event words per wave in a timeline row

// KV formats: OCP E4M3 bytes; INT8 bytes; INT4, two 4-bit two's-complement
// codes per byte (low nibble first), head_dim 128 only.
constexpr int kKvE4M3 = 0;
constexpr int kKvInt8 = 1;
constexpr int kKvInt4 = 2;

struct StreamParams {
  const void* q;               // [sum Q][Hq][D] bf16 or fp32
  const uint8_t* k_pages;      // [P][Hkv][D/16][16][16]
  const uint8_t* v_pages;      // [P][Hkv][4][D/64][16][4][4]
  const float* kv_scales;      // [2][P][Hkv]
  const int32_t* block_table;  // [B][bt_stride]
  const int32_t* ctx_lens;     // [B]
  const int32_t* q_lens;       // [B]
  void* out;                   // [sum Q][Hq][D] bf16 or fp32
  float* part_o;               // [slots][cols_per_block][D] unnormalised partial outputs
  float* part_ml;              // [slots][cols_per_block][2] running max (log2 units), sum
  int32_t* seq_row0;           // [B] first query row of each sequence
  int2* seg_merge;             // [segments] written by the unit holding a segment's first
                               // chunk: (first partial slot, pieces; 1 = written whole)
  int32_t num_seqs;
  int32_t num_q_heads;
  int32_t num_kv_heads;
  int32_t group;               // Hq / Hkv
  int32_t bt_stride;           // max_pages_per_seq
  int32_t max_q_len;
  int32_t cols_per_block;      // query columns (new token x head of a group) per workgroup
  int32_t col_blocks;          // column blocks of one (sequence, kv head)
  int32_t merge_cols;          // query columns per merge workgroup
  int32_t unit_min_chunks;     // units in use: total chunks / this, within [1, max_units]
  int32_t max_units;           // units sharing the chunks at most (waves or workgroups)
  int32_t start_cost;          // chunks a segment's start counts for in the balanced split
  int32_t whole_ok;            // the tile kernel may give each unit one segment whole
  int32_t piece_chunks;        // > 0: fixed pieces of this many chunks (a power of two); counts are pieces
  int32_t piece_log2;          // log2(piece_chunks)
  unsigned long long* timeline;  // null, or [waves][64] event words (measurement)
  int64_t v_scale_offset;      // P * Hkv: start of the V scales in kv_scales
  float qk_scale_log2;         // sm_scale * log2(e)
};

struct Variant {
  int head_dim;     // 64 or 128
  bool packed;      // at most 4 query columns: four pages share a score tile
  int packed_ring;  // packed: groups of four pages in flight per wave (1 or 2)
  int tile_waves;   // > 0: waves sharing each KV chunk through LDS, col_tiles each
  int col_tiles;    // 16-column MFMA tiles per wave (1, or 2 with tile_waves)
  bool dup_lo;      // low halves of P in spare columns (col_tiles == 1, <= 8 columns)
  bool q_f32;
  bool out_f32;
  int kv_format;    // 0: OCP E4M3 bytes; 1: INT8 bytes; 2: INT4, two codes per byte
};

constexpr int kWavesPerGroup = 4;
#ifndef PACKED_GROUP_WAVES
#define PACKED_GROUP_WAVES 4
#endif
// Waves per workgroup of the packed decode kernel (each wave streams its own
// chunk range, so the workgroup is only a unit of dispatch).
constexpr int kPackedWaves = PACKED_GROUP_WAVES;

inline int waves_per_group(const Variant& v) {
  return v.packed ? kPackedWaves : v.tile_waves > 0 ? v.tile_waves : kWavesPerGroup;
}

// Attention kernel: the units of `grid` workgroups (waves when packed) share
// the key chunks of all segments equally.  Partial slots needed: segments +
// max_units.  With ev_start/ev_stop non-null they record the kernel's own
// start and end.
hipError_t launch_stream_attention(const Variant& v, const StreamParams& p, int grid, hipStream_t stream,
                                   hipEvent_t ev_start = nullptr, hipEvent_t ev_stop = nullptr);
// Resident workgroups per compute unit for the variant's attention kernel.
hipError_t stream_attention_occupancy(const Variant& v, int* blocks_per_cu);
bool timeline_supported(const Variant& v);  // kernels that record a timeline exist for v
// Merge kernel: `grid` = segments workgroups along x, merge_grid_y along y.
hipError_t launch_split_merge(const Variant& v, const StreamParams& p, int grid, hipStream_t stream,
                              hipEvent_t ev_start = nullptr, hipEvent_t ev_stop = nullptr);
int merge_cols_for(const Variant& v, int cols_per_block, int64_t expected_parts);
int merge_grid_y(int cols_per_block, int merge_cols);

struct GatherParams {
  const uint8_t* k_pages;
  const uint8_t* v_pages;
  const float* kv_scales;
  const int32_t* block_table;
  const int32_t* ctx_lens;
  uint8_t* k_out;
  uint8_t* v_out;
  float* scale_out;
  int32_t* page_out;
  int32_t num_seqs;
  int32_t num_kv_heads;
  int32_t head_dim;
  int32_t bt_stride;
  int32_t max_ctx_len;
  int64_t v_scale_offset;
  int32_t kv_format;           // 2: INT4 pools (two codes per byte); otherwise one byte per value
};

// Paged FP8 KV append: the q_lens[b] new rows of each sequence become keys
// ctx_lens[b] - q_lens[b] .. ctx_lens[b] - 1 of its pages.
struct AppendParams {
  const void* k_new;           // [sum Q][Hkv][D] bf16 or fp32
  const void* v_new;
  uint8_t* k_pages;            // [P][Hkv][D/16][16][16]
  uint8_t* v_pages;            // [P][Hkv][4][D/64][16][4][4]
  float* kv_scales;            // [2][P][Hkv]
  const int32_t* block_table;  // [B][bt_stride]
  const int32_t* ctx_lens;     // [B] after the append
  const int32_t* q_lens;       // [B] rows appended
  int32_t num_seqs;
  int32_t num_kv_heads;
  int32_t bt_stride;
  int32_t max_touch;           // pages one sequence's append touches at most
  int64_t v_scale_offset;      // P * Hkv
};

hipError_t launch_kv_append(const AppendParams& p, int head_dim, bool new_f32, bool kv_int8, hipStream_t stream,
                            hipEvent_t ev_start = nullptr, hipEvent_t ev_stop = nullptr);
hipError_t launch_debug_encode(const float* in, uint8_t* out, int64_t n, hipStream_t stream);

// Greedy MTP acceptance: K + 1 logits rows per sequence.
struct AcceptParams {
  const void* logits;          // [B][K+1][V] bf16 or fp32
  const int32_t* drafts;       // [B][K]
  int32_t* target_tokens;      // [B][K+1]
  int32_t* num_accepted;       // [B]
  uint64_t* partial;           // [B (K+1)][segments] workspace
  int32_t num_seqs;
  int32_t num_drafts;
  int64_t vocab;               // a multiple of 8
  int32_t segments;            // workgroups per row
};

int accept_segments(int64_t rows, int64_t vocab);
hipError_t launch_mtp_accept(const AcceptParams& p, bool f32, hipStream_t stream, hipEvent_t ev_start = nullptr,
                             hipEvent_t ev_stop = nullptr);

hipError_t launch_debug_gather(const GatherParams& p, hipStream_t stream);
// Streaming-read calibration: `waves` waves read the chunk_bytes-sized chunks
// ids[0..num_chunks) of pool (ids clamped to the pool) and write one XOR word
// per lane to sink[waves * 64].  chunk_bytes: a power of two >= 1024 (>= 2048
// with access 1: half lines of 16 rows of 128 bytes per instruction).
hipError_t launch_stream_read(const uint8_t* pool, int64_t pool_bytes, const int32_t* ids, int64_t num_chunks,
                              int32_t chunk_bytes, int32_t waves, int32_t access, uint32_t* sink, hipStream_t stream,
                              hipEvent_t ev_start, hipEvent_t ev_stop);
// kv_format 0/1: one E4M3/INT8 byte per value (n values); 2: n bytes of two
// INT4 codes each (2n values, low nibble first).
hipError_t launch_debug_decode(const uint8_t* in, float* out, int64_t n, int kv_format, hipStream_t stream);

}  // namespace pa
