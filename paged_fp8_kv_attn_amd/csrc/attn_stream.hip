// Paged FP8-KV attention for gfx950: the keys of every (sequence, kv head,
// block of query columns) are cut into 32-key chunks, the chunks of all of
// them are laid end to end, and each work unit streams an equal contiguous
// range of that list.
//
// Follows the attention section of the Atlas engine article (ainews.cool,
// "技术深度解析": a FlashAttention-2 variant with dedicated MQA/GQA kernels and
// tiling adapted to sequence length and GPU), its quantisation section (FP8
// with per-group scales folded into the kernel) and the paged FP8 KV cache of
// the GB10 article (ainews.surl.tw).
//
// Shape of the work.  The G = Hq/Hkv query heads of a kv head, times the Q_b
// new tokens of a sequence, form G*Q_b "query columns" that all read the same
// keys.  A segment is one (sequence, kv head, block of columns) with its
// keys; it owns n = ceil(kv_end / 32) chunks.  Segments are ordered
// (sequence, kv head, column block) and unit w of W takes global chunks
// [floor(w T / W), floor((w+1) T / W)) of the T in total, so every unit does
// the same amount of streaming whatever the length mix.  A segment that lies
// inside one unit's range is written to `out` directly; otherwise each unit
// writes an unnormalised partial into slot (segment + w), unique because
// ranges and segments are both ordered, and the merge kernel combines them by
// log-sum-exp.  Three kernel families share this schedule:
//   * packed decode (at most 4 columns): each wave is a unit; four pages share
//     one 16x16 score tile (run_piece_packed);
//   * one 16-column tile (5..16 columns): the workgroup is the unit, its
//     waves take the chunks of a piece in turn and merge through LDS
//     (run_piece);
//   * shared KV (more than 16 columns): the workgroup is the unit, its waves
//     split the columns and share each chunk, converted to bf16 once, through
//     LDS (run_piece_tile).
//
// Per chunk, in each wave (lane = 16*lq + ln):
//   * K: lane reads the bytes of token slot ln at d in [lq*D/4, (lq+1)*D/4)
//     of both pages as 16-byte loads; in the (page, head) layout each load
//     instruction of the wave reads whole 128-byte lines (1 KB per load);
//   * S^T = K * Q^T with v_mfma_f32_16x16x32_bf16: A = K (rows = 16 keys of
//     a page, exact FP8->bf16), B = Q^T (columns = query columns).  The
//     d-order inside the contraction is permuted identically on both sides;
//   * online softmax in log2 units with the page's K scale and sm_scale
//     folded into one multiply; row max over the 4 lanes of a column by
//     permlane16/32 swaps;
//   * P~ = p * (page's V scale) split into bf16 hi + lo parts (the pair is
//     exact to ~2^-17 relative), so PV adds no rounding beyond fp32;
//   * O^T += V^T * P~^T: A = V^T (rows = d, k = the 32 keys), B = P~^T taken
//     straight from the S^T accumulator layout.  The 4-token interleave of
//     the V page layout gives each lane its operand in 16-byte loads that,
//     across the wave, read whole lines.

#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "device_common.h"
#include "kernel_params.h"

// Eight-wave workgroups (two waves per SIMD from one workgroup, meeting at
// the same barrier every chunk) run the ping-pong schedule.
#ifndef TILE_PINGPONG
#define TILE_PINGPONG 1
#endif
// Which waves lead: the first half (waves w and w + 4 share a SIMD when the
// dispatcher places wave w on SIMD w % 4), or the even ones.
#ifndef TILE_PP_PARITY
#define TILE_PP_PARITY 0
#endif
// Wave priority in the tile kernel: 1 raises it while a wave issues its
// matrix products, 2 while it runs the softmax, 0 leaves it.
#ifndef TILE_SETPRIO
#define TILE_SETPRIO 1
#endif

namespace pa {

namespace {

template <int D>
struct Geo {
  static constexpr int NSLAB = D / 32;  // MFMA K=32 steps along d
  static constexpr int DQ = D / 4;      // K bytes per lane per page
  static constexpr int NKV = DQ / 16;   // 16-byte K loads per lane per page
  static constexpr int NVB = D / 16;    // V dwords per lane per page = 16-row blocks of d
  static constexpr int NVV = NVB / 4;   // 16-byte V loads per lane per page
};

// Loads of one page's K and V per lane: 16-byte loads; INT4 chunks are half
// as large, one load each.
template <int D, int KF>
struct KvLoads {
  static constexpr int NK = KF == kKvInt4 ? 1 : Geo<D>::NKV;
  static constexpr int NV = KF == kKvInt4 ? 1 : Geo<D>::NVV;
  static_assert(KF != kKvInt4 || D == 128, "INT4 pools are laid out for head_dim 128");
};

// Byte offset of a (page, kv head) chunk in the pool of format KF.
template <int D, int KF>
__device__ __forceinline__ uint64_t chunk_base(int32_t page, int head, int num_kv_heads) {
  if constexpr (KF == kKvInt4) return chunk_offset4(page, head, num_kv_heads, D);
  return chunk_offset(page, head, num_kv_heads, D);
}

// Lane (lq, ln)'s byte offset of K load i / V load i inside a chunk.
template <int D, int KF>
__device__ __forceinline__ uint32_t k_lane_off(int lq, int ln, int i) {
  if constexpr (KF == kKvInt4) return lane_in_chunk4(lq, ln);
  return k_in_chunk(ln, lq * Geo<D>::DQ + 16 * i, D);
}
template <int D, int KF>
__device__ __forceinline__ uint32_t v_lane_off(int lq, int ln, int i) {
  if constexpr (KF == kKvInt4) return lane_in_chunk4(lq, ln);
  return v_in_chunk(4 * lq, Geo<D>::NVB * ln + 4 * i, D);
}

// K operand of slab s (8 values of d in the contraction order of the Q
// operand) from a lane's K loads of one page.
template <int D, int KF>
__device__ __forceinline__ bf16x8 k_slab(const u32x4 (&kl)[KvLoads<D, KF>::NK], int s) {
  if constexpr (KF == kKvInt4) {
    return i4x8_to_bf16x8(kl[0][s]);
  } else {
    const u32x4 w = kl[(2 * s) / 4];
    return kv8x8_to_bf16x8<KF == kKvInt8>(w[(2 * s) % 4], w[(2 * s) % 4 + 1]);
  }
}

// The four slots of d-block cblk in a lane's V loads of one page: four
// bytes, or four 4-bit codes (the low 16 bits) for INT4.
template <int D, int KF>
__device__ __forceinline__ uint32_t v_word(const u32x4 (&vl)[KvLoads<D, KF>::NV], int cblk) {
  if constexpr (KF == kKvInt4) return (vl[0][cblk >> 1] >> (16 * (cblk & 1))) & 0xFFFFu;
  return vl[cblk / 4][cblk % 4];
}

// Bits of slot j (< 4) in a four-slot word.
template <int KF>
__device__ __forceinline__ uint32_t slot_bits(int j) {
  return KF == kKvInt4 ? (0xFu << (4 * j)) : (0xFFu << (8 * j));
}

// Four-slot words -> bf16: one page (4 values) or two pages (8 values).
template <int KF>
__device__ __forceinline__ bf16x4 v4_to_bf16(uint32_t w) {
  if constexpr (KF == kKvInt4) return i4x4_to_bf16x4(w);
  return kv8x4_to_bf16x4<KF == kKvInt8>(w);
}
template <int KF>
__device__ __forceinline__ bf16x8 v8_to_bf16(uint32_t w0, uint32_t w1) {
  if constexpr (KF == kKvInt4) {
    const bf16x4 a = i4x4_to_bf16x4(w0), b = i4x4_to_bf16x4(w1);
    return bf16x8{a[0], a[1], a[2], a[3], b[0], b[1], b[2], b[3]};
  }
  return kv8x8_to_bf16x8<KF == kKvInt8>(w0, w1);
}

constexpr float kNegInf = -__builtin_huge_valf();
constexpr int kChunk = 32;  // keys per chunk (two pages)

__device__ __forceinline__ float max_over_lq(float x) {
  // maximum over the four lanes ln, ln+16, ln+32, ln+48
  auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  x = fmaxf(__uint_as_float(a[0]), __uint_as_float(a[1]));
  auto c = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(c[0]), __uint_as_float(c[1]));
}

__device__ __forceinline__ float sum_over_lq(float x) {
  // one of the two swapped copies is the lane's own value, the other the
  // partner's: their sum is the pair sum in every lane
  auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  x = __uint_as_float(a[0]) + __uint_as_float(a[1]);
  auto c = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(c[0]) + __uint_as_float(c[1]);
}

__device__ __forceinline__ uint32_t pack_bf16(float a, float b) {
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2{a, b}, bf16x2));
}

// bf16 pair (lo half = first) -> the two fp32 values
__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

__device__ __forceinline__ void split_q_f32(const float* x, bf16x8& p1, bf16x8& p2, bf16x8& p3) {
  // x = p1 + p2 + p3 exactly (8 + 8 + 8 significant bits)
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    const __bf16 a = (__bf16)x[j];
    const float r1 = x[j] - (float)a;
    const __bf16 b = (__bf16)r1;
    const float r2 = r1 - (float)b;
    p1[j] = a;
    p2[j] = b;
    p3[j] = (__bf16)r2;
  }
}

// ---- schedule ------------------------------------------------------------

// Chunks of segment (sequence with L keys and Q new tokens, column block cb):
// the keys visible to at least one of its columns, in 32-key chunks.
__device__ __forceinline__ int seg_chunks(int L, int Q, int G, int cpb, int cb) {
  const int ncols = G * Q;
  const int col0 = cb * cpb;
  if (col0 >= ncols) return 0;
  const int i_hi = (min(col0 + cpb, ncols) - 1) / G;
  return (L - Q + i_hi + 1 + kChunk - 1) / kChunk;
}

// What a segment counts for in the balanced split: its chunks, plus
// p.start_cost for its start, and nothing without chunks.  Position v of a
// segment's count is its chunk v - start_cost (none for v < start_cost).
// With fixed pieces (p.piece_chunks = C > 0, a power of two) a segment
// counts its pieces, position v being its chunks [vC, min((v+1)C, chunks)).
__device__ __forceinline__ int sched_chunks(const StreamParams& p, int L, int Q, int cb) {
  const int n = seg_chunks(L, Q, p.group, p.cols_per_block, cb);
  if (p.piece_chunks > 0) return (n + p.piece_chunks - 1) >> p.piece_log2;
  return n > 0 ? n + p.start_cost : 0;
}

// Count of one kv head of a sequence in the balanced split: all of its
// column blocks.
__device__ __forceinline__ int head_chunks(const StreamParams& p, int L, int Q) {
  if (p.col_blocks == 1) return sched_chunks(p, L, Q, 0);
  int s = 0;
  for (int cb = 0; cb < p.col_blocks; ++cb) s += sched_chunks(p, L, Q, cb);
  return s;
}

// ---- wave-wide scans without LDS -------------------------------------------
// Within each row of 16 lanes a Hillis-Steele scan by DPP row shifts (lanes
// shifted in from outside the row read 0), then the totals of the rows
// before are added from scalar reads of lanes 15, 31 and 47.  (Shuffles
// through ds_bpermute put a round trip through LDS on every step of the
// schedule at the kernels' start.)
template <int CTRL>
__device__ __forceinline__ int64_t dpp_row_shr64(int64_t x) {
  const int lo = __builtin_amdgcn_update_dpp(0, (int)(uint32_t)(uint64_t)x, CTRL, 0xf, 0xf, true);
  const int hi = __builtin_amdgcn_update_dpp(0, (int)((uint64_t)x >> 32), CTRL, 0xf, 0xf, true);
  return (int64_t)(((uint64_t)(uint32_t)hi << 32) | (uint32_t)lo);
}

__device__ __forceinline__ int64_t readlane64(int64_t x, int l) {
  const uint32_t lo = __builtin_amdgcn_readlane((int)(uint32_t)(uint64_t)x, l);
  const uint32_t hi = __builtin_amdgcn_readlane((int)((uint64_t)x >> 32), l);
  return (int64_t)(((uint64_t)hi << 32) | lo);
}

__device__ __forceinline__ int64_t wave_incl_scan64(int64_t x, int lane) {
  x += dpp_row_shr64<0x111>(x);  // row_shr:1
  x += dpp_row_shr64<0x112>(x);  // row_shr:2
  x += dpp_row_shr64<0x114>(x);  // row_shr:4
  x += dpp_row_shr64<0x118>(x);  // row_shr:8
  const int64_t r0 = readlane64(x, 15), r1 = readlane64(x, 31), r2 = readlane64(x, 47);
  const int row = lane >> 4;
  return x + (row >= 1 ? r0 : 0) + (row >= 2 ? r1 : 0) + (row >= 3 ? r2 : 0);
}

__device__ __forceinline__ int64_t wave_sum64(int64_t x) {
  return readlane64(wave_incl_scan64(x, __lane_id()), 63);
}

// Maximum of non-negative values over the wave (lanes shifted in read 0).
__device__ __forceinline__ int wave_max_nonneg(int x) {
  x = max(x, __builtin_amdgcn_update_dpp(0, x, 0x111, 0xf, 0xf, true));
  x = max(x, __builtin_amdgcn_update_dpp(0, x, 0x112, 0xf, 0xf, true));
  x = max(x, __builtin_amdgcn_update_dpp(0, x, 0x114, 0xf, 0xf, true));
  x = max(x, __builtin_amdgcn_update_dpp(0, x, 0x118, 0xf, 0xf, true));
  return max(max(__builtin_amdgcn_readlane(x, 15), __builtin_amdgcn_readlane(x, 31)),
             max(__builtin_amdgcn_readlane(x, 47), __builtin_amdgcn_readlane(x, 63)));
}

// Lengths of sequence b and its chunk count over all kv heads (zeros for
// b >= B).  Lane i of a wave holds sequence base + i.
struct SeqLens {
  int L, Q;
  int64_t nb;
};

__device__ __forceinline__ SeqLens load_seq(const StreamParams& p, int b) {
  SeqLens c{0, 0, 0};
  if (b < p.num_seqs) {
    c.L = p.ctx_lens[b];
    c.Q = p.q_lens[b];
    c.nb = (int64_t)p.num_kv_heads * head_chunks(p, c.L, c.Q);
  }
  return c;
}

// Where sequence b starts: its first global chunk and first query row.
struct SeqStart {
  int b;
  int64_t chunk0;
  int row0;
  int L, Q;
};

// Total chunks over all sequences (wave-uniform); `c0` and `c1` hold
// sequences 0 .. 63 and 64 .. 127 (loaded together at the kernel's start).
__device__ __forceinline__ int64_t total_chunks(const StreamParams& p, int lane, const SeqLens& c0, const SeqLens& c1) {
  int64_t total = wave_sum64(c0.nb) + wave_sum64(c1.nb);
  for (int base = 128; base < p.num_seqs; base += 64) total += wave_sum64(load_seq(p, base + lane).nb);
  return total;
}

// The sequence whose chunks contain global chunk `pos` (< total).
__device__ __forceinline__ SeqStart locate_seq(const StreamParams& p, int64_t pos, int lane, const SeqLens& c0,
                                                const SeqLens& c1) {
  int64_t carry = 0;
  int rows = 0;
  for (int base = 0; base < p.num_seqs; base += 64) {
    const SeqLens c = (base == 0) ? c0 : (base == 64) ? c1 : load_seq(p, base + lane);
    const int64_t incl = wave_incl_scan64(c.nb, lane);
    const int qincl = (int)wave_incl_scan64(c.Q, lane);
    const int64_t start = carry + incl - c.nb;
    const uint64_t hit = __builtin_amdgcn_ballot_w64(c.nb > 0 && start <= pos && pos < start + c.nb);
    if (hit) {
      const int src = __builtin_ctzll(hit);
      SeqStart s;
      s.b = base + src;
      s.chunk0 = readlane64(start, src);
      s.row0 = rows + __builtin_amdgcn_readlane(qincl - c.Q, src);
      s.L = __builtin_amdgcn_readlane(c.L, src);
      s.Q = __builtin_amdgcn_readlane(c.Q, src);
      return s;
    }
    carry += readlane64(incl, 63);
    rows += __builtin_amdgcn_readlane(qincl, 63);
  }
  SeqStart s{p.num_seqs, carry, rows, 0, 0};  // not reached for pos < total
  return s;
}

// Workgroup 0 records the first query row of every sequence for the merge
// kernel, which runs after this kernel on the same stream.
__device__ __forceinline__ void write_seq_meta(const StreamParams& p, int lane) {
  int rows = 0;
  for (int base = 0; base < p.num_seqs; base += 64) {
    const int b = base + lane;
    const int qb = (b < p.num_seqs) ? p.q_lens[b] : 0;
    const int qincl = (int)wave_incl_scan64(qb, lane);
    if (b < p.num_seqs) p.seq_row0[b] = rows + qincl - qb;
    rows += __builtin_amdgcn_readlane(qincl, 63);
  }
}

// Units that share the chunks (waves when packed, workgroups otherwise):
// one per unit_min_chunks chunks, at least one and at most max_units, so
// small problems are not cut into pieces that cost more to merge than to
// stream, and no unit's range is empty.
__device__ __forceinline__ int work_units(const StreamParams& p, int64_t T) {
  const int64_t want = T / p.unit_min_chunks;
  return (int)(want < 1 ? 1 : (want < p.max_units ? want : p.max_units));
}

// First unit whose range holds global chunk g: ranges start at
// floor(w T / W), so it is the largest w with w T < (g + 1) W.
__device__ __forceinline__ int wg_of_chunk(int64_t g, int64_t T, int W) {
  return (int)(((g + 1) * (int64_t)W + T - 1) / T) - 1;
}

// ---- ring of register buffers ---------------------------------------------
// Units k < nk of a wave go through NRING buffers: unit k lives in buffer
// k % NRING and the buffer is refilled with unit k + NRING right after unit k
// is consumed.  In the steady state every consumption is followed by a refill
// unconditionally, so the compiler knows exactly how many loads were issued
// after each buffer's and waits for that buffer alone (a conditional refill
// would make it wait for every outstanding load).  issue(k, slot) and
// step(k, slot) take the buffer index as a compile-time constant after
// unrolling.
template <int NRING, class Issue, class Step>
__device__ __forceinline__ void ring_loop(int nk, Issue&& issue, Step&& step) {
  if (nk >= NRING) {
#pragma unroll
    for (int j = 0; j < NRING; ++j) issue(j, j);
    int k = 0;
    for (; k + 2 * NRING <= nk; k += NRING) {
#pragma unroll
      for (int j = 0; j < NRING; ++j) {
        step(k + j, j);
        issue(k + j + NRING, j);
      }
    }
    // NRING <= nk - k < 2 * NRING units remain
#pragma unroll
    for (int j = 0; j < NRING; ++j) {
      step(k + j, j);
      if (k + j + NRING < nk) issue(k + j + NRING, j);
    }
#pragma unroll
    for (int j = 0; j < NRING; ++j)
      if (k + NRING + j < nk) step(k + NRING + j, j);
  } else {
#pragma unroll
    for (int j = 0; j < NRING; ++j)
      if (j < nk) issue(j, j);
#pragma unroll
    for (int j = 0; j < NRING; ++j)
      if (j < nk) step(j, j);
  }
}

// A block-table batch (page ids and page scales, one gather per 16-32
// chunks) is waited for where it is loaded.  Its registers are read at
// every refill; were the batch still pending there on some path, the
// compiler, which cannot tell that path is rare, would make every refill
// wait until only the newest chunk's loads are in flight, emptying the
// ring.  Reading the registers in an empty asm completes the loads once
// per batch instead.
__device__ __forceinline__ void settle_batch(int32_t bt, float sk, float sv) {
  __asm__ volatile("" : : "v"(bt), "v"(sk), "v"(sv));
}

// ---- one piece of a segment ----------------------------------------------

struct PieceDesc {
  int b, h, cb;
  int L, Q, row0;
  int c_begin, c_end;  // chunk range of the piece inside its segment
  bool whole;          // the piece is the whole segment
  int slot;            // partial slot when not whole
};

// Measurement: the kernels instantiated with ON record, for every wave, events
// in its own row of kTimelineSlots words of p.timeline (row = workgroup x
// waves per workgroup + wave), each (s_memrealtime << 4) | type, in order:
// kTlEntry, kTlLengths (the lengths read and summed), kTlScheduled (its
// unit's range known), then per piece
// kTlPieceStart, kTlStep per chunk (per group of chunks in the packed
// decode), kTlPieceEnd; the row's last word holds kTlWaveEnd.  Events past
// the row's first kTimelineSlots - 1 words are dropped.  Lane 0 writes;
// the count is the same in every lane.  The kernels without ON (the ones
// forwards use unless a timeline is set) contain none of it: a run-time
// check per chunk step measured 1-4% slower.
enum : unsigned {
  kTlEntry = 1, kTlScheduled = 2, kTlPieceStart = 3, kTlStep = 4, kTlPieceEnd = 5, kTlLengths = 6, kTlWaveEnd = 7
};
// An event's word is stored at the next event (or the wave's end): the
// counter read then has had a whole step to return, and the wave does not
// wait for it (and, with it, for its outstanding LDS accesses) where it is
// taken.
template <bool ON>
struct Timeline {
  unsigned long long* row;
  int n;
  unsigned long long pending;
  __device__ __forceinline__ void rec(unsigned type, int lane) {
    if constexpr (ON) {
      if (n < kTimelineSlots - 1) {
        const unsigned long long t = __builtin_amdgcn_s_memrealtime();
        if (n > 0 && lane == 0) row[n - 1] = pending;
        pending = (t << 4) | type;
        ++n;
      }
    }
  }
  __device__ __forceinline__ void end(int lane) {
    if constexpr (ON) {
      if (n > 0 && lane == 0) row[n - 1] = pending;
      const unsigned long long t = __builtin_amdgcn_s_memrealtime();
      if (lane == 0) row[kTimelineSlots - 1] = (t << 4) | kTlWaveEnd;
    }
  }
};

template <bool ON>
__device__ __forceinline__ Timeline<ON> timeline_for(const StreamParams& p, int wave) {
  Timeline<ON> tl;
  tl.row = ON ? p.timeline + ((size_t)blockIdx.x * (blockDim.x / 64) + wave) * kTimelineSlots : nullptr;
  tl.n = 0;
  tl.pending = 0;
  return tl;
}

template <int D, int NCT, bool DUPLO, bool QF32, bool OUTF32, int NBUF, int KF, class TLT>
__device__ __forceinline__ void run_piece(const StreamParams& p, const PieceDesc& pc, int lane, int wave, TLT& tl) {
  tl.rec(kTlPieceStart, lane);
  using GD = Geo<D>;
  using KL = KvLoads<D, KF>;
  constexpr int NW = kWavesPerGroup;
  constexpr int NP = QF32 ? 3 : 1;
  const int lq = lane >> 4;
  const int ln = lane & 15;
  const int h = pc.h;
  const int L = pc.L;
  const int Qb = pc.Q;
  const int G = p.group;
  const int ncols = G * Qb;
  const int col0 = pc.cb * p.cols_per_block;
  const int cols_here = min(p.cols_per_block, ncols - col0);
  const int i_lo = col0 / G;
  const int first_masked_key = L - Qb + i_lo + 1;  // keys >= this are hidden from some column
  const int npages = (L + kPageSize - 1) / kPageSize;

  // ---- this lane's query columns and Q operand ----------------------------
  int lim[NCT];  // last visible key of the lane's column (-1: unused column)
  int qrow[NCT], qhead[NCT];
  bf16x8 qop[NP][NCT][GD::NSLAB];
#pragma unroll
  for (int t = 0; t < NCT; ++t) {
    const int rc = DUPLO ? (ln & 7) : (16 * t + ln);
    const bool valid = rc < cols_here;
    const int gc = col0 + (valid ? rc : 0);
    const int i = gc / G;
    const int g = gc - i * G;
    lim[t] = valid ? (L - Qb + i) : -1;
    qrow[t] = pc.row0 + i;
    qhead[t] = h * G + g;
    const size_t qoff = ((size_t)qrow[t] * p.num_q_heads + qhead[t]) * D + (size_t)lq * GD::DQ;
    if constexpr (QF32) {
      const u32x4* src = reinterpret_cast<const u32x4*>(static_cast<const float*>(p.q) + qoff);
#pragma unroll
      for (int s = 0; s < GD::NSLAB; ++s) {
        float x[8];
        if (valid) {
          const u32x4 w0 = src[2 * s], w1 = src[2 * s + 1];
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            x[j] = __uint_as_float(w0[j]);
            x[4 + j] = __uint_as_float(w1[j]);
          }
        } else {
#pragma unroll
          for (int j = 0; j < 8; ++j) x[j] = 0.f;
        }
        split_q_f32(x, qop[0][t][s], qop[1][t][s], qop[2][t][s]);
      }
    } else {
      const u32x4* src = reinterpret_cast<const u32x4*>(static_cast<const uint16_t*>(p.q) + qoff);
#pragma unroll
      for (int s = 0; s < GD::NSLAB; ++s) {
        const u32x4 w = valid ? src[s] : u32x4{0u, 0u, 0u, 0u};
        qop[0][t][s] = __builtin_bit_cast(bf16x8, w);
      }
    }
  }
  const bool lo_lane = DUPLO && (ln >= 8);

  // ---- accumulators -------------------------------------------------------
  f32x4 o[NCT][GD::NVB];
  float m[NCT], l[NCT];
#pragma unroll
  for (int t = 0; t < NCT; ++t) {
    m[t] = kNegInf;
    l[t] = 0.f;
#pragma unroll
    for (int c = 0; c < GD::NVB; ++c) o[t][c] = f32x4{0.f, 0.f, 0.f, 0.f};
  }

  const int32_t* bt = p.block_table + (size_t)pc.b * p.bt_stride;
  // load i of a lane reads 16 bytes: K block d = lq*DQ + 16i of slot ln; V
  // values d = NVB*ln + 4i .. +3 of the slots 4lq..4lq+3
  uint32_t koff[KL::NK], voff[KL::NV];
#pragma unroll
  for (int i = 0; i < KL::NK; ++i) koff[i] = k_lane_off<D, KF>(lq, ln, i);
#pragma unroll
  for (int i = 0; i < KL::NV; ++i) voff[i] = v_lane_off<D, KF>(lq, ln, i);
  const uint8_t* kpool = p.k_pages;
  const uint8_t* vpool = p.v_pages;

  // ---- chunk loop --------------------------------------------------------
  // This wave's chunks are c_k = c_begin + wave + k * NW, k < nk.  The block
  // table entries and the K/V page scales of 32 chunks at a time are fetched
  // by one gather (lane j: chunk k0 + j/2, page j%2) and read with readlane,
  // so the loop never waits on a scalar memory load.  K/V bytes go into a
  // ring of NBUF register buffers: a buffer is refilled with chunk k + NBUF
  // as soon as chunk k has been consumed, so NBUF chunks are in flight while
  // one is computed.  A buffer's page scales are latched when it is filled.
  const int c_begin = pc.c_begin;
  const int nk = (c_begin + wave < pc.c_end) ? (pc.c_end - c_begin - wave + NW - 1) / NW : 0;
  int32_t bt_v = 0;
  float sk_v = 0.f, sv_v = 0.f;
  auto load_batch = [&](int k0) {
    const int k = k0 + (lane >> 1);
    int32_t ph = 0;
    float a = 0.f, bsc = 0.f;
    if (k < nk) {
      const int c = c_begin + wave + k * NW;
      const int pg = min(2 * c + (lane & 1), npages - 1);  // a missing second page repeats the first
      ph = bt[pg];
      const int64_t sidx = (int64_t)ph * p.num_kv_heads + h;
      a = p.kv_scales[sidx] * code_unit<KF>();
      bsc = p.kv_scales[p.v_scale_offset + sidx] * code_unit<KF>();
    }
    bt_v = ph;
    sk_v = a;
    sv_v = bsc;
    settle_batch(bt_v, sk_v, sv_v);
  };
  u32x4 kbuf[NBUF][2][KL::NK], vbuf[NBUF][2][KL::NV];
  float skb[NBUF][2], svb[NBUF][2];
  // fill ring slot j with chunk k (k < nk); a new batch of block-table
  // entries is fetched when k starts one (every chunk before k has already
  // been issued and has its scales latched)
  auto issue = [&](int k, int j) {
    u32x4 (&kb)[2][KL::NK] = kbuf[j];
    u32x4 (&vb)[2][KL::NV] = vbuf[j];
    float (&skj)[2] = skb[j];
    float (&svj)[2] = svb[j];
    if ((k & 31) == 0) load_batch(k);
    const int slot = 2 * (k & 31);
#pragma unroll
    for (int pg = 0; pg < 2; ++pg) {
      const int32_t ph = __builtin_amdgcn_readlane(bt_v, slot + pg);
      const uint64_t base = chunk_base<D, KF>(ph, h, p.num_kv_heads);
#pragma unroll
      for (int i = 0; i < KL::NK; ++i)
        kb[pg][i] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(kpool + base + koff[i]));
#pragma unroll
      for (int i = 0; i < KL::NV; ++i)
        vb[pg][i] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(vpool + base + voff[i]));
    }
    // the scales are read after the KV loads are issued: waiting for them
    // (they were fetched before) leaves the KV loads in flight
#pragma unroll
    for (int pg = 0; pg < 2; ++pg) {
      skj[pg] = __uint_as_float(__builtin_amdgcn_readlane(__float_as_uint(sk_v), slot + pg));
      svj[pg] = __uint_as_float(__builtin_amdgcn_readlane(__float_as_uint(sv_v), slot + pg));
    }
  };

  // compute chunk k from its ring slot
  auto step = [&](int k, int j) {
    tl.rec(kTlStep, lane);
    const u32x4 (&kc)[2][KL::NK] = kbuf[j];
    const u32x4 (&vc)[2][KL::NV] = vbuf[j];
    const float (&skc)[2] = skb[j];
    const float (&svc)[2] = svb[j];
    const int c = c_begin + wave + k * NW;
    // S^T = K Q^T for both pages
    f32x4 sacc[2][NCT];
#pragma unroll
    for (int pg = 0; pg < 2; ++pg) {
#pragma unroll
      for (int t = 0; t < NCT; ++t) sacc[pg][t] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int s = 0; s < GD::NSLAB; ++s) {
        const bf16x8 kb = k_slab<D, KF>(kc[pg], s);
#pragma unroll
        for (int t = 0; t < NCT; ++t) {
#pragma unroll
          for (int part = 0; part < NP; ++part)
            sacc[pg][t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kb, qop[part][t][s], sacc[pg][t], 0, 0, 0);
        }
      }
    }

    // online softmax (log2 units)
    const float fk0 = p.qk_scale_log2 * skc[0];
    const float fk1 = p.qk_scale_log2 * skc[1];
    const int key0 = c * kChunk + 4 * lq;  // key of register j: key0 + j (page 0), key0 + 16 + j (page 1)
    const bool need_mask = (c * kChunk + kChunk - 1) >= first_masked_key;
    uint32_t phi[NCT][4], plo[NCT][4];
    bool rescale = false;
    float alpha[NCT];
#pragma unroll
    for (int t = 0; t < NCT; ++t) {
      float x[8];
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        x[j] = sacc[0][t][j] * fk0;
        x[4 + j] = sacc[1][t][j] * fk1;
      }
      if (need_mask) {
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          x[j] = (key0 + j <= lim[t]) ? x[j] : kNegInf;
          x[4 + j] = (key0 + 16 + j <= lim[t]) ? x[4 + j] : kNegInf;
        }
      }
      float mx = x[0];
#pragma unroll
      for (int j = 1; j < 8; ++j) mx = fmaxf(mx, x[j]);
      mx = max_over_lq(mx);
      const float mn = fmaxf(m[t], mx);
      const float base = (mn == kNegInf) ? 0.f : mn;
      alpha[t] = __builtin_amdgcn_exp2f(m[t] - base);
      rescale |= (mn > m[t]);
      m[t] = mn;
      float pr[8];
      float rs = 0.f;
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        pr[j] = __builtin_amdgcn_exp2f(x[j] - base);
        rs += pr[j];
      }
      l[t] = l[t] * alpha[t] + rs;
      // P~ = p * V scale, as bf16 hi + lo
#pragma unroll
      for (int k2 = 0; k2 < 4; ++k2) {
        const float sc = (k2 < 2) ? svc[0] : svc[1];
        const float a = pr[2 * k2] * sc;
        const float bb = pr[2 * k2 + 1] * sc;
        const uint32_t hw = pack_bf16(a, bb);
        const uint32_t lw = pack_bf16(a - bf16_lo(hw), bb - bf16_hi(hw));
        if constexpr (DUPLO) {
          phi[t][k2] = lo_lane ? lw : hw;
        } else {
          phi[t][k2] = hw;
          plo[t][k2] = lw;
        }
      }
    }
    if (__builtin_amdgcn_ballot_w64(rescale)) {
#pragma unroll
      for (int t = 0; t < NCT; ++t)
#pragma unroll
        for (int cb2 = 0; cb2 < GD::NVB; ++cb2) o[t][cb2] *= alpha[t];
    }

    // O^T += V^T P~^T
    const bool tail = (c * kChunk + kChunk) > L;
    uint32_t vmask0 = 0xffffffffu, vmask1 = 0xffffffffu;
    if (tail) {
      vmask0 = 0u;
      vmask1 = 0u;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        vmask0 |= (key0 + j < L) ? slot_bits<KF>(j) : 0u;
        vmask1 |= (key0 + 16 + j < L) ? slot_bits<KF>(j) : 0u;
      }
    }
    bf16x8 pop_hi[NCT], pop_lo[NCT];
#pragma unroll
    for (int t = 0; t < NCT; ++t) {
      pop_hi[t] = __builtin_bit_cast(bf16x8, u32x4{phi[t][0], phi[t][1], phi[t][2], phi[t][3]});
      if constexpr (!DUPLO) pop_lo[t] = __builtin_bit_cast(bf16x8, u32x4{plo[t][0], plo[t][1], plo[t][2], plo[t][3]});
    }
#pragma unroll
    for (int cblk = 0; cblk < GD::NVB; ++cblk) {
      const uint32_t w0 = v_word<D, KF>(vc[0], cblk) & vmask0;
      const uint32_t w1 = v_word<D, KF>(vc[1], cblk) & vmask1;
      const bf16x8 va = v8_to_bf16<KF>(w0, w1);
#pragma unroll
      for (int t = 0; t < NCT; ++t) {
        o[t][cblk] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(va, pop_hi[t], o[t][cblk], 0, 0, 0);
        if constexpr (!DUPLO)
          o[t][cblk] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(va, pop_lo[t], o[t][cblk], 0, 0, 0);
      }
    }
  };

  ring_loop<NBUF>(nk, issue, step);

  // ---- per-wave finish: column sums; fold spare-column low parts ----------
#pragma unroll
  for (int t = 0; t < NCT; ++t) l[t] = sum_over_lq(l[t]);
  if constexpr (DUPLO) {
#pragma unroll
    for (int cblk = 0; cblk < GD::NVB; ++cblk)
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const float other = __uint_as_float(
            __builtin_amdgcn_mov_dpp(__float_as_uint(o[0][cblk][j]), 0x128 /*row_ror:8*/, 0xf, 0xf, false));
        o[0][cblk][j] += other;
      }
  }

  // ---- merge the waves through LDS (lane-private slots) -------------------
  constexpr int NVEC = NCT * GD::NVB;  // f32x4 per lane
  __shared__ f32x4 s_o[NW / 2][NVEC][64];
  __shared__ float s_ml[NW / 2][NCT][2][64];
#pragma unroll
  for (int half = NW / 2; half >= 1; half >>= 1) {
    if (wave >= half && wave < 2 * half) {
      const int buf = wave - half;
#pragma unroll
      for (int t = 0; t < NCT; ++t) {
#pragma unroll
        for (int cblk = 0; cblk < GD::NVB; ++cblk) s_o[buf][t * GD::NVB + cblk][lane] = o[t][cblk];
        s_ml[buf][t][0][lane] = m[t];
        s_ml[buf][t][1][lane] = l[t];
      }
    }
    __syncthreads();
    if (wave < half) {
#pragma unroll
      for (int t = 0; t < NCT; ++t) {
        const float mb = s_ml[wave][t][0][lane];
        const float lb = s_ml[wave][t][1][lane];
        const float mn = fmaxf(m[t], mb);
        const float base = (mn == kNegInf) ? 0.f : mn;
        const float fa = __builtin_amdgcn_exp2f(m[t] - base);
        const float fb = __builtin_amdgcn_exp2f(mb - base);
        m[t] = mn;
        l[t] = l[t] * fa + lb * fb;
#pragma unroll
        for (int cblk = 0; cblk < GD::NVB; ++cblk)
          o[t][cblk] = o[t][cblk] * fa + s_o[wave][t * GD::NVB + cblk][lane] * fb;
      }
    }
    __syncthreads();
  }

  // ---- write: final output, or this piece's partial -----------------------
  if (wave == 0) {
#pragma unroll
    for (int t = 0; t < NCT; ++t) {
      const int rc = DUPLO ? ln : (16 * t + ln);
      if (rc >= cols_here || (DUPLO && ln >= 8)) continue;
      if (pc.whole) {
        const float inv = 1.f / l[t];
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const size_t off = ((size_t)qrow[t] * p.num_q_heads + qhead[t]) * D + (size_t)GD::NVB * (4 * lq + j);
          if constexpr (OUTF32) {
            float* dst = static_cast<float*>(p.out) + off;
#pragma unroll
            for (int c4 = 0; c4 < GD::NVB / 4; ++c4) {
              f32x4 v;
#pragma unroll
              for (int e = 0; e < 4; ++e) v[e] = o[t][4 * c4 + e][j] * inv;
              *reinterpret_cast<f32x4*>(dst + 4 * c4) = v;
            }
          } else {
            uint16_t* dst = static_cast<uint16_t*>(p.out) + off;
            uint32_t w[GD::NVB / 2];
#pragma unroll
            for (int e = 0; e < GD::NVB / 2; ++e) w[e] = pack_bf16(o[t][2 * e][j] * inv, o[t][2 * e + 1][j] * inv);
            if constexpr (GD::NVB == 8) {
              *reinterpret_cast<u32x4*>(dst) = u32x4{w[0], w[1], w[2], w[3]};
            } else {
              *reinterpret_cast<uint2*>(dst) = make_uint2(w[0], w[1]);
            }
          }
        }
      } else {
        float* po = p.part_o + ((size_t)pc.slot * p.cols_per_block + rc) * D;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          float* dst = po + GD::NVB * (4 * lq + j);
#pragma unroll
          for (int c4 = 0; c4 < GD::NVB / 4; ++c4) {
            f32x4 v;
#pragma unroll
            for (int e = 0; e < 4; ++e) v[e] = o[t][4 * c4 + e][j];
            *reinterpret_cast<f32x4*>(dst + 4 * c4) = v;
          }
        }
        if (lq == 0) {
          float* pm = p.part_ml + ((size_t)pc.slot * p.cols_per_block + rc) * 2;
          pm[0] = m[t];
          pm[1] = l[t];
        }
      }
    }
  }
  tl.rec(kTlPieceEnd, lane);
}

// ---- packed decode piece: at most 4 query columns --------------------------
// Four consecutive pages share one 16x16 score tile.  Each page has its own
// QK accumulator (K of the page as A, the query columns replicated over the
// 16 B columns), and lane (lq, ln) keeps the scores of page ln/4, keys
// 4lq..4lq+3, query column ln%4: every lane then holds four useful scores and
// the softmax runs on full registers.  The running max is lazy: it moves
// only when a new score exceeds it by more than kLazyLog2 (weights stay
// below 2^kLazyLog2, harmless in fp32 and in the bf16 hi + lo split), so the
// accumulators are almost never rescaled.  In PV each chunk (two pages) uses
// a B operand in which a lane's P sits in the half of its own page, so the
// output column ln accumulates the pages at group position ln/4; the four
// positions are summed at the end of the piece.  One wave streams the whole
// piece in groups of two chunks (four pages, 64 keys); keys at or past the
// piece's end (or L) are masked.
constexpr float kLazyLog2 = 8.f;
// Packed decode tuning, measured on MI355X: either one group of four pages
// (16 KB of K+V) in flight per wave at two waves per SIMD, or two groups at
// one wave per SIMD (the plan takes the second when its units fit on the
// GPU at once: ~3% faster on batch-32 decode).  Deeper rings overfill the
// memory queues: latency grows, bandwidth does not.

__device__ __forceinline__ float dpp_ror4(float x) {
  return __uint_as_float(__builtin_amdgcn_mov_dpp(__float_as_uint(x), 0x124 /*row_ror:4*/, 0xf, 0xf, false));
}
__device__ __forceinline__ float dpp_ror8(float x) {
  return __uint_as_float(__builtin_amdgcn_mov_dpp(__float_as_uint(x), 0x128 /*row_ror:8*/, 0xf, 0xf, false));
}

template <int D, bool QF32, bool OUTF32, int NRING, int KF, class TLT>
__device__ __forceinline__ void run_piece_packed(const StreamParams& p, const PieceDesc& pc, int lane, TLT& tl) {
  tl.rec(kTlPieceStart, lane);
  using GD = Geo<D>;
  using KL = KvLoads<D, KF>;
  constexpr int NP = QF32 ? 3 : 1;
  const int lq = lane >> 4;
  const int ln = lane & 15;
  const int pj = ln >> 2;  // group position of the page whose scores this lane keeps
  const int qc = ln & 3;   // query column of this lane
  const int h = pc.h;
  const int L = pc.L;
  const int Qb = pc.Q;
  const int G = p.group;
  const int ncols = G * Qb;
  const int col0 = pc.cb * p.cols_per_block;
  const int cols_here = min(p.cols_per_block, ncols - col0);
  const int npages = (L + kPageSize - 1) / kPageSize;
  const int kend = min(L, pc.c_end * kChunk);  // keys past this belong to another piece
  const int lim_lo = L - Qb + col0 / G;         // smallest causal limit of the block

  // ---- Q operand: B column ln is query column qc ---------------------------
  const bool qvalid = qc < cols_here;
  const int gc = col0 + (qvalid ? qc : 0);
  const int qi = gc / G;
  const int qg = gc - qi * G;
  const int lim = qvalid ? (L - Qb + qi) : -1;
  const int qrow = pc.row0 + qi;
  const int qhead = h * G + qg;
  bf16x8 qop[NP][GD::NSLAB];
  {
    const size_t qoff = ((size_t)qrow * p.num_q_heads + qhead) * D + (size_t)lq * GD::DQ;
    if constexpr (QF32) {
      const u32x4* src = reinterpret_cast<const u32x4*>(static_cast<const float*>(p.q) + qoff);
#pragma unroll
      for (int s = 0; s < GD::NSLAB; ++s) {
        float x[8];
        if (qvalid) {
          const u32x4 w0 = src[2 * s], w1 = src[2 * s + 1];
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            x[j] = __uint_as_float(w0[j]);
            x[4 + j] = __uint_as_float(w1[j]);
          }
        } else {
#pragma unroll
          for (int j = 0; j < 8; ++j) x[j] = 0.f;
        }
        split_q_f32(x, qop[0][s], qop[1][s], qop[2][s]);
      }
    } else {
      const u32x4* src = reinterpret_cast<const u32x4*>(static_cast<const uint16_t*>(p.q) + qoff);
#pragma unroll
      for (int s = 0; s < GD::NSLAB; ++s) {
        const u32x4 w = qvalid ? src[s] : u32x4{0u, 0u, 0u, 0u};
        qop[0][s] = __builtin_bit_cast(bf16x8, w);
      }
    }
  }

  f32x4 o[GD::NVB];
#pragma unroll
  for (int c = 0; c < GD::NVB; ++c) o[c] = f32x4{0.f, 0.f, 0.f, 0.f};
  float m = kNegInf;  // reference max (log2 units), the same in the 16 lanes of a query column
  float l = 0.f;      // this lane's share of the weight sum

  const int32_t* bt = p.block_table + (size_t)pc.b * p.bt_stride;
  // load i of a lane reads 16 bytes: K block d = lq*DQ + 16i of slot ln; V
  // values d = NVB*ln + 4i .. +3 of the slots 4lq..4lq+3
  uint32_t koff[KL::NK], voff[KL::NV];
#pragma unroll
  for (int i = 0; i < KL::NK; ++i) koff[i] = k_lane_off<D, KF>(lq, ln, i);
#pragma unroll
  for (int i = 0; i < KL::NV; ++i) voff[i] = v_lane_off<D, KF>(lq, ln, i);
  const uint8_t* kpool = p.k_pages;
  const uint8_t* vpool = p.v_pages;

  // The wave's groups start at chunk c_begin + 2k, k < nk (the last group of
  // an odd piece has one chunk; its second is masked by kend).
  const int c_begin = pc.c_begin;
  const int nk = (pc.c_end - c_begin + 1) / 2;

  // block-table batch: lane j holds the page of group k0 + j/4, position j%4,
  // and that page's K and V scales
  int32_t bt_v = 0;
  float sk_v = 0.f, sv_v = 0.f;
  auto load_batch = [&](int k0) {
    const int k = k0 + (lane >> 2);
    int32_t ph = 0;
    float a = 0.f, bsc = 0.f;
    if (k < nk) {
      const int c = c_begin + 2 * k;
      const int pg = min(2 * c + (lane & 3), npages - 1);  // missing pages repeat the last one
      ph = bt[pg];
      const int64_t sidx = (int64_t)ph * p.num_kv_heads + h;
      a = p.kv_scales[sidx] * code_unit<KF>();
      bsc = p.kv_scales[p.v_scale_offset + sidx] * code_unit<KF>();
    }
    bt_v = ph;
    sk_v = a;
    sv_v = bsc;
    settle_batch(bt_v, sk_v, sv_v);
  };

  u32x4 kbuf[NRING][4][KL::NK], vbuf[NRING][4][KL::NV];
  float skb[NRING], svb[NRING];  // scales of the page this lane's scores belong to
  auto issue = [&](int k, int j) {
    u32x4 (&kb)[4][KL::NK] = kbuf[j];
    u32x4 (&vb)[4][KL::NV] = vbuf[j];
    float& skl = skb[j];
    float& svl = svb[j];
    if ((k & 15) == 0) load_batch(k);
    const int e = 4 * (k & 15);
#pragma unroll
    for (int pg = 0; pg < 4; ++pg) {
      const int32_t ph = __builtin_amdgcn_readlane(bt_v, e + pg);
      const uint64_t base = chunk_base<D, KF>(ph, h, p.num_kv_heads);
#pragma unroll
      for (int i = 0; i < KL::NK; ++i)
        kb[pg][i] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(kpool + base + koff[i]));
    }
#pragma unroll
    for (int pg = 0; pg < 4; ++pg) {
      const int32_t ph = __builtin_amdgcn_readlane(bt_v, e + pg);
      const uint64_t base = chunk_base<D, KF>(ph, h, p.num_kv_heads);
#pragma unroll
      for (int i = 0; i < KL::NV; ++i)
        vb[pg][i] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(vpool + base + voff[i]));
    }
    skl = __shfl(sk_v, e + pj);
    svl = __shfl(sv_v, e + pj);
  };

  auto step = [&](int k, int j) {
    tl.rec(kTlStep, lane);
    const u32x4 (&kc)[4][KL::NK] = kbuf[j];
    const u32x4 (&vc)[4][KL::NV] = vbuf[j];
    const float skl = skb[j];
    const float svl = svb[j];
    const int c = c_begin + 2 * k;
    const int key0 = c * kChunk;  // first key of the group
    // QK: one accumulator per page; each lane keeps the tile of its page
    f32x4 sc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int pg = 0; pg < 4; ++pg) {
      f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int s = 0; s < GD::NSLAB; ++s) {
        const bf16x8 kb = k_slab<D, KF>(kc[pg], s);
#pragma unroll
        for (int part = 0; part < NP; ++part)
          acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kb, qop[part][s], acc, 0, 0, 0);
      }
      if (pj == pg) sc = acc;
    }
    const float fk = p.qk_scale_log2 * skl;
    const int kl = key0 + 16 * pj + 4 * lq;  // key of sc[0]
    float x[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) x[i] = sc[i] * fk;
    if (key0 + 2 * kChunk > kend || key0 + 2 * kChunk - 1 > lim_lo) {
#pragma unroll
      for (int i = 0; i < 4; ++i) x[i] = (kl + i <= lim && kl + i < kend) ? x[i] : kNegInf;
    }
    // the lane's max; a column's max passes m + 8 iff one of its lanes'
    // does, so the reduction over the column's 16 lanes runs only when the
    // reference moves
    float mx = fmaxf(fmaxf(x[0], x[1]), fmaxf(x[2], x[3]));
    if (__builtin_amdgcn_ballot_w64(mx > m + kLazyLog2)) {
      mx = max_over_lq(mx);
      mx = fmaxf(mx, dpp_ror4(mx));
      mx = fmaxf(mx, dpp_ror8(mx));
      const float mn = fmaxf(m, mx);
      const float alpha = __builtin_amdgcn_exp2f(m - ((mn == kNegInf) ? 0.f : mn));
#pragma unroll
      for (int cb2 = 0; cb2 < GD::NVB; ++cb2) o[cb2] *= alpha;
      l *= alpha;
      m = mn;
    }
    const float base = (m == kNegInf) ? 0.f : m;
    float pr[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      pr[i] = __builtin_amdgcn_exp2f(x[i] - base);
      l += pr[i];
    }
    // P~ = p * V scale as bf16 hi + lo
    float a[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) a[i] = pr[i] * svl;
    const uint32_t hw0 = pack_bf16(a[0], a[1]);
    const uint32_t hw1 = pack_bf16(a[2], a[3]);
    const uint32_t lw0 = pack_bf16(a[0] - bf16_lo(hw0), a[1] - bf16_hi(hw0));
    const uint32_t lw1 = pack_bf16(a[2] - bf16_lo(hw1), a[3] - bf16_hi(hw1));
    // PV, one chunk (two pages) at a time
#pragma unroll
    for (int ch = 0; ch < 2; ++ch) {
      const uint32_t mA = (pj == 2 * ch) ? 0xffffffffu : 0u;
      const uint32_t mB = (pj == 2 * ch + 1) ? 0xffffffffu : 0u;
      const bf16x8 bhi = __builtin_bit_cast(bf16x8, u32x4{hw0 & mA, hw1 & mA, hw0 & mB, hw1 & mB});
      const bf16x8 blo = __builtin_bit_cast(bf16x8, u32x4{lw0 & mA, lw1 & mA, lw0 & mB, lw1 & mB});
      const int kc0 = key0 + ch * kChunk + 4 * lq;  // key of the lane's first V byte of page 2ch
      uint32_t vm0 = 0xffffffffu, vm1 = 0xffffffffu;
      if (key0 + ch * kChunk + kChunk > L) {  // bytes of keys >= L may be anything: select them to 0
        vm0 = 0u;
        vm1 = 0u;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          vm0 |= (kc0 + j < L) ? slot_bits<KF>(j) : 0u;
          vm1 |= (kc0 + 16 + j < L) ? slot_bits<KF>(j) : 0u;
        }
      }
#pragma unroll
      for (int cblk = 0; cblk < GD::NVB; ++cblk) {
        const uint32_t w0 = v_word<D, KF>(vc[2 * ch], cblk) & vm0;
        const uint32_t w1 = v_word<D, KF>(vc[2 * ch + 1], cblk) & vm1;
        const bf16x8 va = v8_to_bf16<KF>(w0, w1);
        o[cblk] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(va, bhi, o[cblk], 0, 0, 0);
        o[cblk] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(va, blo, o[cblk], 0, 0, 0);
      }
    }
  };

  ring_loop<NRING>(nk, issue, step);

  // ---- per-wave finish: sum over lane quarters and page positions ---------
  l = sum_over_lq(l);
  l += dpp_ror4(l);
  l += dpp_ror8(l);
#pragma unroll
  for (int cblk = 0; cblk < GD::NVB; ++cblk)
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      float v = o[cblk][j];
      v += dpp_ror4(v);
      v += dpp_ror8(v);
      o[cblk][j] = v;
    }

  // ---- write: final output, or this piece's partial -----------------------
  if (pj == 0 && qc < cols_here) {
    if (pc.whole) {
      const float inv = 1.f / l;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const size_t off = ((size_t)qrow * p.num_q_heads + qhead) * D + (size_t)GD::NVB * (4 * lq + j);
        if constexpr (OUTF32) {
          float* dst = static_cast<float*>(p.out) + off;
#pragma unroll
          for (int c4 = 0; c4 < GD::NVB / 4; ++c4) {
            f32x4 v;
#pragma unroll
            for (int e = 0; e < 4; ++e) v[e] = o[4 * c4 + e][j] * inv;
            *reinterpret_cast<f32x4*>(dst + 4 * c4) = v;
          }
        } else {
          uint16_t* dst = static_cast<uint16_t*>(p.out) + off;
          uint32_t w[GD::NVB / 2];
#pragma unroll
          for (int e = 0; e < GD::NVB / 2; ++e) w[e] = pack_bf16(o[2 * e][j] * inv, o[2 * e + 1][j] * inv);
          if constexpr (GD::NVB == 8) {
            *reinterpret_cast<u32x4*>(dst) = u32x4{w[0], w[1], w[2], w[3]};
          } else {
            *reinterpret_cast<uint2*>(dst) = make_uint2(w[0], w[1]);
          }
        }
      }
    } else {
      float* po = p.part_o + ((size_t)pc.slot * p.cols_per_block + qc) * D;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        float* dst = po + GD::NVB * (4 * lq + j);
#pragma unroll
        for (int c4 = 0; c4 < GD::NVB / 4; ++c4) {
          f32x4 v;
#pragma unroll
          for (int e = 0; e < 4; ++e) v[e] = o[4 * c4 + e][j];
          *reinterpret_cast<f32x4*>(dst + 4 * c4) = v;
        }
      }
      if (lq == 0) {
        float* pm = p.part_ml + ((size_t)pc.slot * p.cols_per_block + qc) * 2;
        pm[0] = m;
        pm[1] = l;
      }
    }
  }
  tl.rec(kTlPieceEnd, lane);
}


// ---- wide column blocks: each KV chunk shared by the waves through LDS ----
// With more than 16 query columns per segment the NW waves of a workgroup
// split the columns (NT 16-column tiles each, column 16 (wave NT + t) + ln)
// and all of them walk every chunk of the piece.  The workgroup reads a
// chunk from HBM once: its 2 (NKV + NVV) full-line 1 KB loads (the loads of
// the register path) are spread over the waves, each thread converts its
// bytes to bf16 once and stores them in LDS in MFMA operand order, one
// 16-byte operand per lane and slab, so every operand read is a 16-byte LDS
// read by consecutive lanes.  Raw chunks wait in a ring of R register
// buffers; LDS holds two converted chunks, so the one barrier per chunk both
// publishes chunk k and frees the buffer of chunk k - 1 for chunk k + 1.
template <int D, int NW, int KF>
struct TileGeo {
  using GD = Geo<D>;
  using KL = KvLoads<D, KF>;
  static constexpr int NL = 2 * (KL::NK + KL::NV);     // 1 KB loads per chunk
  // loads per thread per chunk; with fewer loads than waves (INT4 in eight
  // waves) the last waves load nothing
  static constexpr int LPT = (NL + NW - 1) / NW;
  static constexpr int KSL = 2 * GD::NSLAB;             // K operands: pages x slabs
  static constexpr int SLOTS = KSL + GD::NVB;           // + V operands: 16-row blocks of d
  static_assert(NL % NW == 0 || NL < NW, "the loads of a chunk split evenly over the loading waves");
};

__device__ __forceinline__ bf16x4 fp8x4_to_bf16x4(uint32_t w) {
  const bf16x2 a = fp8x2_to_bf16x2<false>(w);
  const bf16x2 b = fp8x2_to_bf16x2<true>(w);
  return bf16x4{a[0], a[1], b[0], b[1]};
}

// Workgroup barrier ordering LDS only: global loads stay in flight.
__device__ __forceinline__ void lds_barrier() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}

// Like ring_loop, with the consumption of a buffer split from the work on
// it: consume(k, slot) empties the buffer, the buffer is refilled, then
// compute(k) runs while the refill is in flight.
template <int NRING, class Issue, class Consume, class Compute>
__device__ __forceinline__ void ring_loop_split(int nk, Issue&& issue, Consume&& consume, Compute&& compute) {
  if (nk >= NRING) {
#pragma unroll
    for (int j = 0; j < NRING; ++j) issue(j, j);
    int k = 0;
    for (; k + 2 * NRING <= nk; k += NRING) {
#pragma unroll
      for (int j = 0; j < NRING; ++j) {
        consume(k + j, j);
        issue(k + j + NRING, j);
        compute(k + j);
      }
    }
#pragma unroll
    for (int j = 0; j < NRING; ++j) {
      consume(k + j, j);
      if (k + j + NRING < nk) issue(k + j + NRING, j);
      compute(k + j);
    }
#pragma unroll
    for (int j = 0; j < NRING; ++j)
      if (k + NRING + j < nk) {
        consume(k + NRING + j, j);
        compute(k + NRING + j);
      }
  } else {
#pragma unroll
    for (int j = 0; j < NRING; ++j)
      if (j < nk) issue(j, j);
#pragma unroll
    for (int j = 0; j < NRING; ++j)
      if (j < nk) {
        consume(j, j);
        compute(j);
      }
  }
}

// Q^T as the B operand of one 16-column tile: lane (lq, ln) holds, per slab
// s, the values d = lq D/4 + 8s .. +7 of its column's query row (the
// contraction order of the K operand); fp32 Q is split into three bf16
// parts whose sum is exact.
template <int D, bool QF32>
__device__ __forceinline__ void load_q_operand(const StreamParams& p, size_t qoff, bool valid,
                                               bf16x8 (&op)[QF32 ? 3 : 1][Geo<D>::NSLAB]) {
  using GD = Geo<D>;
  if constexpr (QF32) {
    const u32x4* src = reinterpret_cast<const u32x4*>(static_cast<const float*>(p.q) + qoff);
#pragma unroll
    for (int s = 0; s < GD::NSLAB; ++s) {
      float x[8];
      if (valid) {
        const u32x4 w0 = src[2 * s], w1 = src[2 * s + 1];
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          x[j] = __uint_as_float(w0[j]);
          x[4 + j] = __uint_as_float(w1[j]);
        }
      } else {
#pragma unroll
        for (int j = 0; j < 8; ++j) x[j] = 0.f;
      }
      split_q_f32(x, op[0][s], op[1][s], op[2][s]);
    }
  } else {
    const u32x4* src = reinterpret_cast<const u32x4*>(static_cast<const uint16_t*>(p.q) + qoff);
#pragma unroll
    for (int s = 0; s < GD::NSLAB; ++s) {
      const u32x4 w = valid ? src[s] : u32x4{0u, 0u, 0u, 0u};
      op[0][s] = __builtin_bit_cast(bf16x8, w);
    }
  }
}

template <int D, int NW, int NT, bool QF32, bool OUTF32, int R, int KF, bool PP, class TLT>
__device__ __forceinline__ void run_piece_tile(const StreamParams& p, const PieceDesc& pc, int lane, int wave,
                                               TLT& tl) {
  tl.rec(kTlPieceStart, lane);
  using GD = Geo<D>;
  using TG = TileGeo<D, NW, KF>;
  using KL = KvLoads<D, KF>;
  constexpr int NP = QF32 ? 3 : 1;
  const int lq = lane >> 4;
  const int ln = lane & 15;
  const int h = pc.h;
  const int L = pc.L;
  const int Qb = pc.Q;
  const int G = p.group;
  const int ncols = G * Qb;
  const int col0 = pc.cb * p.cols_per_block;
  const int cols_here = min(p.cols_per_block, ncols - col0);
  const int first_masked_key = L - Qb + col0 / G + 1;  // keys >= this are hidden from some column
  const int npages = (L + kPageSize - 1) / kPageSize;

  // ---- this wave's query columns ------------------------------------------
  int lim[NT], qrow[NT], qhead[NT];
  bool cvalid[NT];
  bf16x8 qop[NT][NP][GD::NSLAB];
#pragma unroll
  for (int t = 0; t < NT; ++t) {
    const int rc = 16 * (wave * NT + t) + ln;
    cvalid[t] = rc < cols_here;
    const int gc = col0 + (cvalid[t] ? rc : 0);
    const int i = gc / G;
    const int g = gc - i * G;
    lim[t] = cvalid[t] ? (L - Qb + i) : -1;
    qrow[t] = pc.row0 + i;
    qhead[t] = h * G + g;
    load_q_operand<D, QF32>(p, ((size_t)qrow[t] * p.num_q_heads + qhead[t]) * D + (size_t)lq * GD::DQ, cvalid[t],
                            qop[t]);
  }

  f32x4 o[NT][GD::NVB];
  float m[NT], l[NT], base[NT];  // base: the exponent reference, m or 0 while m = -inf
#pragma unroll
  for (int t = 0; t < NT; ++t) {
    m[t] = kNegInf;
    l[t] = 0.f;
    base[t] = 0.f;
#pragma unroll
    for (int c = 0; c < GD::NVB; ++c) o[t][c] = f32x4{0.f, 0.f, 0.f, 0.f};
  }

  // ---- this thread's share of a chunk's loads -----------------------------
  // load r is slot j = r NW + wave of the chunk (j < NL): K of page j / NK,
  // 16-byte block j % NK of the lane's quarter of d, or V of page j' / NV
  // (j' = j - 2 NK), the lane's values d = NVB ln + 4 i .. +3 (i = j' % NV)
  // for the 4 keys of its quarter (INT4: all of its d-blocks, one load).
  uint32_t soff[TG::LPT];  // lane's byte offset inside the (page, head) chunk
  int ldpg[TG::LPT];
#pragma unroll
  for (int r = 0; r < TG::LPT; ++r) {
    const int j = r * NW + wave;
    if (j < 2 * KL::NK) {
      ldpg[r] = j / KL::NK;
      soff[r] = k_lane_off<D, KF>(lq, ln, j % KL::NK);
    } else {
      const int jj = j - 2 * KL::NK;
      ldpg[r] = jj / KL::NV;
      soff[r] = v_lane_off<D, KF>(lq, ln, jj % KL::NV);
    }
  }

  // Converted chunks in LDS: two buffers, or three with the ping-pong
  // schedule (the lagging half of the waves still reads chunk k - 1 after
  // the barrier that publishes chunk k).
  constexpr int NB = PP ? 3 : 2;
  __shared__ bf16x8 s_kv[NB][TG::SLOTS][64];
  // the previous piece may still read any buffer
  lds_barrier();

  const int32_t* bt = p.block_table + (size_t)pc.b * p.bt_stride;
  const int c_begin = pc.c_begin;
  const int nk = pc.c_end - c_begin;
  // block-table batch: lane j holds the page of chunk k0 + j/2, position j%2,
  // with that page's score factor (K scale times sm_scale log2 e) and log2
  // of its V scale
  int32_t bt_v = 0;
  float sk_v = 0.f, lv_v = 0.f;
  auto load_batch = [&](int k0) {
    const int k = k0 + (lane >> 1);
    int32_t ph = 0;
    float a = 0.f, bsc = 1.f;
    if (k < nk) {
      const int pg = min(2 * (c_begin + k) + (lane & 1), npages - 1);  // a missing second page repeats the first
      ph = bt[pg];
      const int64_t sidx = (int64_t)ph * p.num_kv_heads + h;
      a = p.kv_scales[sidx] * code_unit<KF>();
      bsc = p.kv_scales[p.v_scale_offset + sidx] * code_unit<KF>();
    }
    bt_v = ph;
    sk_v = a * p.qk_scale_log2;
    lv_v = __builtin_log2f(bsc);
    settle_batch(bt_v, sk_v, lv_v);
  };

  // what the softmax of a chunk needs: per page, the score factor and log2
  // of the V scale
  struct ChunkMeta {
    float fk[2], lv[2];
  };
  u32x4 raw[R][TG::LPT];
  ChunkMeta rm[R];
  auto issue = [&](int k, int j) {
    if ((k & 31) == 0) load_batch(k);
    const int e = 2 * (k & 31);
#pragma unroll
    for (int r = 0; r < TG::LPT; ++r) {
      if (TG::NL % NW != 0 && r * NW + wave >= TG::NL) continue;  // wave-uniform
      const int32_t ph = __builtin_amdgcn_readlane(bt_v, e + ldpg[r]);
      const uint8_t* pool = (r * NW + wave < 2 * KL::NK) ? p.k_pages : p.v_pages;
      raw[j][r] = __builtin_nontemporal_load(
          reinterpret_cast<const u32x4*>(pool + chunk_base<D, KF>(ph, h, p.num_kv_heads) + soff[r]));
    }
#pragma unroll
    for (int pg = 0; pg < 2; ++pg) {
      rm[j].fk[pg] = __uint_as_float(__builtin_amdgcn_readlane(__float_as_uint(sk_v), e + pg));
      rm[j].lv[pg] = __uint_as_float(__builtin_amdgcn_readlane(__float_as_uint(lv_v), e + pg));
    }
  };

  // the chunk between its consume and compute (its ring buffer is refilled
  // in between)
  ChunkMeta cm;
  auto consume = [&](int k, int j) {
    const int c = c_begin + k;
    bf16x8 (*dst)[64] = s_kv[k % NB];
#pragma unroll
    for (int r = 0; r < TG::LPT; ++r) {
      const int jj = r * NW + wave;
      if (TG::NL % NW != 0 && jj >= TG::NL) continue;  // wave-uniform
      const u32x4 w = raw[j][r];
      if (jj < 2 * KL::NK) {
        if constexpr (KF == kKvInt4) {
          // the lane's 32 codes of d: slabs 0..3 of its page
#pragma unroll
          for (int s2 = 0; s2 < GD::NSLAB; ++s2) dst[ldpg[r] * GD::NSLAB + s2][lane] = i4x8_to_bf16x8(w[s2]);
        } else {
          const int s0 = ldpg[r] * GD::NSLAB + 2 * (jj % KL::NK);
          dst[s0][lane] = kv8x8_to_bf16x8<KF == kKvInt8>(w[0], w[1]);
          dst[s0 + 1][lane] = kv8x8_to_bf16x8<KF == kKvInt8>(w[2], w[3]);
        }
      } else {
        // V codes of keys >= L may be anything (NaN codes included): zero them
        const int key0 = c * kChunk + 16 * ldpg[r] + 4 * lq;
        uint32_t vm = 0xffffffffu;
        if (c * kChunk + kChunk > L) {
          vm = 0u;
#pragma unroll
          for (int e = 0; e < 4; ++e) vm |= (key0 + e < L) ? slot_bits<KF>(e) : 0u;
        }
        if constexpr (KF == kKvInt4) {
          // four slots of every d-block of the lane's page
          const u32x4 wv[1] = {w};
#pragma unroll
          for (int cb = 0; cb < GD::NVB; ++cb)
            reinterpret_cast<bf16x4*>(&dst[TG::KSL + cb][lane])[ldpg[r]] = i4x4_to_bf16x4(v_word<D, KF>(wv, cb) & vm);
        } else {
          const int i = (jj - 2 * KL::NK) % KL::NV;
#pragma unroll
          for (int e = 0; e < 4; ++e)
            reinterpret_cast<bf16x4*>(&dst[TG::KSL + 4 * i + e][lane])[ldpg[r]] =
                kv8x4_to_bf16x4<KF == kKvInt8>(w[e] & vm);
        }
      }
    }
    cm = rm[j];
  };

  // S^T = K Q^T for both pages of chunk k
  auto qk = [&](int k, f32x4 (&sacc)[2][NT]) {
    if (TILE_SETPRIO == 1) __builtin_amdgcn_s_setprio(1);
    const bf16x8 (*kv)[64] = s_kv[k % NB];
#pragma unroll
    for (int pg = 0; pg < 2; ++pg) {
#pragma unroll
      for (int t = 0; t < NT; ++t) sacc[pg][t] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int s = 0; s < GD::NSLAB; ++s) {
        const bf16x8 kb = kv[pg * GD::NSLAB + s][lane];
#pragma unroll
        for (int t = 0; t < NT; ++t)
#pragma unroll
          for (int part = 0; part < NP; ++part)
            sacc[pg][t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kb, qop[t][part][s], sacc[pg][t], 0, 0, 0);
      }
    }
    if (TILE_SETPRIO == 1) __builtin_amdgcn_s_setprio(0);
  };

  // Online softmax of one chunk in log2 units with a lazy running max: the
  // max is taken on the raw scores of each page (the page's positive score
  // factor keeps the order), and each weight comes out of one fma and one
  // exp2 with the V scale already in it: P~ = 2^(s fk + log2 sV - base)
  // = p sV.  The row sum adds P~ / sV = P~ 2^-log2 sV per page (the same
  // rounding of log2 sV on both sides of the quotient).  P~ leaves as bf16
  // hi + lo operands.
  auto softmax = [&](int k, const ChunkMeta& ch, f32x4 (&sacc)[2][NT], bf16x8 (&pop_hi)[NT],
                     bf16x8 (&pop_lo)[NT]) {
    if (TILE_SETPRIO == 2) __builtin_amdgcn_s_setprio(1);
    const int cu = __builtin_amdgcn_readfirstlane(c_begin + k);
    const int key0 = cu * kChunk + 4 * lq;  // key of register j: key0 + j (page 0), key0 + 16 + j (page 1)
    const bool need_mask = (cu * kChunk + kChunk - 1) >= first_masked_key;
#pragma unroll
    for (int t = 0; t < NT; ++t) {
      if (need_mask) {
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          sacc[0][t][j] = (key0 + j <= lim[t]) ? sacc[0][t][j] : kNegInf;
          sacc[1][t][j] = (key0 + 16 + j <= lim[t]) ? sacc[1][t][j] : kNegInf;
        }
      }
      const float r0 = __builtin_elementwise_maximum(__builtin_elementwise_maximum(sacc[0][t][0], sacc[0][t][1]),
                                                     __builtin_elementwise_maximum(sacc[0][t][2], sacc[0][t][3]));
      const float r1 = __builtin_elementwise_maximum(__builtin_elementwise_maximum(sacc[1][t][0], sacc[1][t][1]),
                                                     __builtin_elementwise_maximum(sacc[1][t][2], sacc[1][t][3]));
      // the lane's max over its 8 keys; some column's max passes m + 8 iff
      // some lane's does, so the reduction across the column's four lanes
      // runs only when the reference moves
      float mx = __builtin_elementwise_maximum(r0 * ch.fk[0], r1 * ch.fk[1]);
      if (__builtin_amdgcn_ballot_w64(mx > m[t] + kLazyLog2)) {
        auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(mx), __float_as_uint(mx), false, false);
        mx = __builtin_elementwise_maximum(__uint_as_float(a[0]), __uint_as_float(a[1]));
        auto c2 = __builtin_amdgcn_permlane32_swap(__float_as_uint(mx), __float_as_uint(mx), false, false);
        mx = __builtin_elementwise_maximum(__uint_as_float(c2[0]), __uint_as_float(c2[1]));
        const float mn = fmaxf(m[t], mx);
        const float alpha = __builtin_amdgcn_exp2f(m[t] - ((mn == kNegInf) ? 0.f : mn));
#pragma unroll
        for (int cb2 = 0; cb2 < GD::NVB; ++cb2) o[t][cb2] *= alpha;
        l[t] *= alpha;
        m[t] = mn;
        base[t] = (mn == kNegInf) ? 0.f : mn;
      }
      const float c0 = ch.lv[0] - base[t];
      const float c1 = ch.lv[1] - base[t];
      float pw[8];
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        pw[j] = __builtin_amdgcn_exp2f(__builtin_fmaf(sacc[0][t][j], ch.fk[0], c0));
        pw[4 + j] = __builtin_amdgcn_exp2f(__builtin_fmaf(sacc[1][t][j], ch.fk[1], c1));
      }
      const float rs0 = (pw[0] + pw[1]) + (pw[2] + pw[3]);
      const float rs1 = (pw[4] + pw[5]) + (pw[6] + pw[7]);
      l[t] = __builtin_fmaf(rs1, __builtin_amdgcn_exp2f(-ch.lv[1]),
                            __builtin_fmaf(rs0, __builtin_amdgcn_exp2f(-ch.lv[0]), l[t]));
      uint32_t phi[4], plo[4];
#pragma unroll
      for (int k2 = 0; k2 < 4; ++k2) {
        phi[k2] = pack_bf16(pw[2 * k2], pw[2 * k2 + 1]);
        plo[k2] = pack_bf16(pw[2 * k2] - bf16_lo(phi[k2]), pw[2 * k2 + 1] - bf16_hi(phi[k2]));
      }
      pop_hi[t] = __builtin_bit_cast(bf16x8, u32x4{phi[0], phi[1], phi[2], phi[3]});
      pop_lo[t] = __builtin_bit_cast(bf16x8, u32x4{plo[0], plo[1], plo[2], plo[3]});
    }
    if (TILE_SETPRIO == 2) __builtin_amdgcn_s_setprio(0);
  };

  // O^T += V^T P~^T for chunk k
  auto pv = [&](int k, const bf16x8 (&pop_hi)[NT], const bf16x8 (&pop_lo)[NT]) {
    if (TILE_SETPRIO == 1) __builtin_amdgcn_s_setprio(1);
    const bf16x8 (*kv)[64] = s_kv[k % NB];
#pragma unroll
    for (int cblk = 0; cblk < GD::NVB; ++cblk) {
      const bf16x8 va = kv[TG::KSL + cblk][lane];
#pragma unroll
      for (int t = 0; t < NT; ++t) {
        o[t][cblk] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(va, pop_hi[t], o[t][cblk], 0, 0, 0);
        o[t][cblk] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(va, pop_lo[t], o[t][cblk], 0, 0, 0);
      }
    }
    if (TILE_SETPRIO == 1) __builtin_amdgcn_s_setprio(0);
  };

  // Ping-pong (PP): the waves of the first half (one per SIMD) issue their
  // matrix work first and then the softmax, the second half the other way
  // round, so that on every SIMD one wave's softmax runs beside the other's
  // MFMAs.  First half, chunk k: PV of k - 1, QK of k, softmax of k.
  // Second half: softmax and PV of k - 1, QK of k.  Both meet at the one
  // barrier per chunk; each carries its chunk k - 1 work across it.
  if constexpr (!PP) {
    auto compute = [&](int k) {
      lds_barrier();
      tl.rec(kTlStep, lane);
      f32x4 sacc[2][NT];
      bf16x8 pop_hi[NT], pop_lo[NT];
      qk(k, sacc);
      softmax(k, cm, sacc, pop_hi, pop_lo);
      pv(k, pop_hi, pop_lo);
    };
    ring_loop_split<R>(nk, issue, consume, compute);
  } else if (TILE_PP_PARITY ? (wave % 2 == 0) : (wave < NW / 2)) {
    // leading half: its P~ of chunk k - 1 crosses the barrier
    bf16x8 pop_hi[NT], pop_lo[NT];
    auto compute = [&](int k) {
      lds_barrier();
      tl.rec(kTlStep, lane);
      if (k > 0) pv(k - 1, pop_hi, pop_lo);
      f32x4 sacc[2][NT];
      qk(k, sacc);
      softmax(k, cm, sacc, pop_hi, pop_lo);
    };
    ring_loop_split<R>(nk, issue, consume, compute);
    if (nk > 0) pv(nk - 1, pop_hi, pop_lo);
  } else {
    // lagging half: its scores of chunk k - 1 cross the barrier
    f32x4 sacc[2][NT];
    ChunkMeta cm_prev;
    auto compute = [&](int k) {
      lds_barrier();
      tl.rec(kTlStep, lane);
      if (k > 0) {
        bf16x8 pop_hi[NT], pop_lo[NT];
        softmax(k - 1, cm_prev, sacc, pop_hi, pop_lo);
        pv(k - 1, pop_hi, pop_lo);
      }
      qk(k, sacc);
      cm_prev = cm;
    };
    ring_loop_split<R>(nk, issue, consume, compute);
    if (nk > 0) {
      bf16x8 pop_hi[NT], pop_lo[NT];
      softmax(nk - 1, cm_prev, sacc, pop_hi, pop_lo);
      pv(nk - 1, pop_hi, pop_lo);
    }
  }

  // ---- write: final output, or this piece's partial -----------------------
#pragma unroll
  for (int t = 0; t < NT; ++t) {
    l[t] = sum_over_lq(l[t]);
    if (!cvalid[t]) continue;
    const int rc = 16 * (wave * NT + t) + ln;
    if (pc.whole) {
      const float inv = 1.f / l[t];
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const size_t off = ((size_t)qrow[t] * p.num_q_heads + qhead[t]) * D + (size_t)GD::NVB * (4 * lq + j);
        if constexpr (OUTF32) {
          float* dst = static_cast<float*>(p.out) + off;
#pragma unroll
          for (int c4 = 0; c4 < GD::NVB / 4; ++c4) {
            f32x4 v;
#pragma unroll
            for (int e = 0; e < 4; ++e) v[e] = o[t][4 * c4 + e][j] * inv;
            *reinterpret_cast<f32x4*>(dst + 4 * c4) = v;
          }
        } else {
          uint16_t* dst = static_cast<uint16_t*>(p.out) + off;
          uint32_t w[GD::NVB / 2];
#pragma unroll
          for (int e = 0; e < GD::NVB / 2; ++e) w[e] = pack_bf16(o[t][2 * e][j] * inv, o[t][2 * e + 1][j] * inv);
          if constexpr (GD::NVB == 8) {
            *reinterpret_cast<u32x4*>(dst) = u32x4{w[0], w[1], w[2], w[3]};
          } else {
            *reinterpret_cast<uint2*>(dst) = make_uint2(w[0], w[1]);
          }
        }
      }
    } else {
      float* po = p.part_o + ((size_t)pc.slot * p.cols_per_block + rc) * D;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        float* dst = po + GD::NVB * (4 * lq + j);
#pragma unroll
        for (int c4 = 0; c4 < GD::NVB / 4; ++c4) {
          f32x4 v;
#pragma unroll
          for (int e = 0; e < 4; ++e) v[e] = o[t][4 * c4 + e][j];
          *reinterpret_cast<f32x4*>(dst + 4 * c4) = v;
        }
      }
      if (lq == 0) {
        float* pm = p.part_ml + ((size_t)pc.slot * p.cols_per_block + rc) * 2;
        pm[0] = m[t];
        pm[1] = l[t];
      }
    }
  }
  tl.rec(kTlPieceEnd, lane);
}

}  // namespace

// ---- the pieces of one unit's chunk range ---------------------------------
// Unit w of W takes global chunks [floor(w T / W), floor((w+1) T / W)) and
// runs run(piece) for the part of each segment inside that range, in order.
// `leader` is the one lane of the unit that records, for each segment whose
// first chunk lies in its range, where the segment's partials start and how
// many units hold pieces of it (1: written whole).  With fixed pieces the
// positions are pieces: each is run on its own, into the partial slot of
// its global position, so that where a segment is cut, and every value
// computed for it, depends on that segment alone.
template <class Run>
__device__ __forceinline__ void walk_pieces(const StreamParams& p, int lane, bool leader, int w, int W, int64_t T,
                                            const SeqLens& c0, const SeqLens& c1, Run&& run) {
  const int64_t lo = (int64_t)w * T / W;
  const int64_t hi = (int64_t)(w + 1) * T / W;
  if (lo >= hi) return;
  SeqStart ss = locate_seq(p, lo, lane, c0, c1);
  int b = ss.b;
  int row0 = ss.row0;
  int L = ss.L;
  int Q = ss.Q;
  const int per_head = head_chunks(p, L, Q);
  const int64_t off = lo - ss.chunk0;
  int h = (int)(off / per_head);
  int r = (int)(off - (int64_t)h * per_head);
  int cb = 0;
  int n = sched_chunks(p, L, Q, 0);
  while (r >= n) {
    r -= n;
    ++cb;
    n = sched_chunks(p, L, Q, cb);
  }
  int64_t cur = lo;
  const int C = p.piece_chunks;
  while (true) {
    const int take = C > 0 ? 1 : (int)min((int64_t)(n - r), hi - cur);
    PieceDesc pc;
    pc.b = b;
    pc.h = h;
    pc.cb = cb;
    pc.L = L;
    pc.Q = Q;
    pc.row0 = row0;
    // positions [r, r + take) of the segment's count: its chunks from
    // r - start_cost (a piece holding only the start position has none and
    // writes an empty partial: max -inf, sum 0)
    const int seg = (b * p.num_kv_heads + h) * p.col_blocks + cb;
    if (C > 0) {
      pc.c_begin = r * C;
      pc.c_end = min(r * C + C, seg_chunks(L, Q, p.group, p.cols_per_block, cb));
      pc.whole = n == 1;
      pc.slot = (int)cur;
    } else {
      pc.c_begin = max(r - p.start_cost, 0);
      pc.c_end = max(r + take - p.start_cost, 0);
      pc.whole = (r == 0) && (take == n);
      pc.slot = seg + w;
    }
    // the same in every lane: hand the piece over in scalar registers
    pc.b = __builtin_amdgcn_readfirstlane(pc.b);
    pc.h = __builtin_amdgcn_readfirstlane(pc.h);
    pc.cb = __builtin_amdgcn_readfirstlane(pc.cb);
    pc.L = __builtin_amdgcn_readfirstlane(pc.L);
    pc.Q = __builtin_amdgcn_readfirstlane(pc.Q);
    pc.row0 = __builtin_amdgcn_readfirstlane(pc.row0);
    pc.c_begin = __builtin_amdgcn_readfirstlane(pc.c_begin);
    pc.c_end = __builtin_amdgcn_readfirstlane(pc.c_end);
    pc.whole = __builtin_amdgcn_readfirstlane((int)pc.whole) != 0;
    pc.slot = __builtin_amdgcn_readfirstlane(pc.slot);
    if (r == 0 && leader) {
      if (C > 0) {
        // its n pieces are at the global positions cur .. cur + n - 1
        p.seg_merge[seg] = make_int2((int)cur, n);
      } else {
        // units w .. last hold the pieces; their partial slots are seg + w ..
        const int last = pc.whole ? w : wg_of_chunk(cur + n - 1, T, W);
        p.seg_merge[seg] = make_int2(seg + w, last - w + 1);
      }
    }
    run(pc);
    cur += take;
    if (cur >= hi) break;
    r += take;
    if (r < n) continue;  // fixed pieces: the segment's next piece
    // next non-empty segment
    r = 0;
    do {
      if (++cb == p.col_blocks) {
        cb = 0;
        if (++h == p.num_kv_heads) {
          h = 0;
          row0 += Q;
          ++b;
          L = p.ctx_lens[b];
          Q = p.q_lens[b];
        }
      }
      n = sched_chunks(p, L, Q, cb);
    } while (n == 0);
  }
}

// Whole-segment schedule of the shared-KV tile kernel.  When the segments
// are about as many as the units (at least three quarters of them, at most
// all) and none holds more than twice the mean chunks, unit w takes one
// segment whole: no partials are written and the merge has nothing to do.
// The balanced split would cut nearly every segment in two there, and the
// partial writes and their merge cost more than the longest segment's
// excess over the mean.  The longest segments (by length class) go to the
// lowest unit numbers, which the dispatcher starts first (later workgroups
// of a compute unit start and step later).  Every unit takes the same decision from the
// same lengths.  Needs at most 128 sequences (their lengths sit in the
// lanes of c0 and c1) and one column block per (sequence, kv head); unit w
// takes kv head w % Hkv of the sequence ranked w / Hkv.  Returns false for
// the balanced split; otherwise pc is unit w's piece (no chunks for w >= the
// segments), its segment's record written.
__device__ __forceinline__ bool whole_segment_piece(const StreamParams& p, int lane, bool leader, int w, int W,
                                                    const SeqLens& c0, const SeqLens& c1, PieceDesc& pc) {
  if (!p.whole_ok || p.num_seqs > 128 || p.col_blocks != 1) return false;
  const int S = p.num_seqs * p.num_kv_heads;
  if (S > W || 4 * S < 3 * W) return false;
  const int n0 = seg_chunks(c0.L, c0.Q, p.group, p.cols_per_block, 0);
  const int n1 = seg_chunks(c1.L, c1.Q, p.group, p.cols_per_block, 0);
  const int mx = wave_max_nonneg(max(n0, n1));
  const int64_t sum = wave_sum64((int64_t)n0 + n1);
  if ((int64_t)mx * p.num_seqs > 2 * sum) return false;
  // fixed pieces: only where every segment is one piece, which is then the
  // piece the walk would run, so only the order of the units changes
  if (p.piece_chunks > 0 && mx > p.piece_chunks) return false;
  pc.c_end = 0;
  if (w >= S) return true;
  // rank of each lane's two sequences (lane and 64 + lane): by class of
  // chunk count, kWholeClasses classes of equal width up to the longest,
  // longest class first, by sequence index within a class.  One ballot per
  // class and bit counts: an exact sort of the 128 counts through lane reads
  // took ~6 us here, at the start of every unit; with 8, 16 and 32 classes
  // MTP verification measured 46.6-47.1, 47.3-47.6 and 48.3-48.5 us.
  constexpr int kWholeClasses = 8;
  const int cls0 = (n0 * kWholeClasses) / (mx + 1);
  const int cls1 = (n1 * kWholeClasses) / (mx + 1);
  const bool real0 = lane < p.num_seqs;
  const bool real1 = 64 + lane < p.num_seqs;
  int rk0 = 0, rk1 = 0;
  int above = 0;  // sequences in the longer classes
  for (int c = kWholeClasses - 1; c >= 0; --c) {
    const uint64_t m0 = __builtin_amdgcn_ballot_w64(real0 && cls0 == c);
    const uint64_t m1 = __builtin_amdgcn_ballot_w64(real1 && cls1 == c);
    const int k0 = __popcll(m0);
    // members of the class in lanes below this one
    const int b0 = __builtin_amdgcn_mbcnt_hi((uint32_t)(m0 >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)m0, 0));
    const int b1 = __builtin_amdgcn_mbcnt_hi((uint32_t)(m1 >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)m1, 0));
    if (cls0 == c) rk0 = above + b0;
    if (cls1 == c) rk1 = above + k0 + b1;
    above += k0 + __popcll(m1);
  }
  const int r = w / p.num_kv_heads;
  const uint64_t hit0 = __builtin_amdgcn_ballot_w64(rk0 == r && lane < p.num_seqs);
  const uint64_t hit1 = __builtin_amdgcn_ballot_w64(rk1 == r && 64 + lane < p.num_seqs);
  const bool in0 = hit0 != 0;
  const int src = in0 ? __builtin_ctzll(hit0) : __builtin_ctzll(hit1);
  // the sequence's first query row: new tokens of the sequences before it
  const int q0 = (int)wave_incl_scan64(c0.Q, lane);
  const int q1 = (int)wave_incl_scan64(c1.Q, lane);
  pc.b = (in0 ? 0 : 64) + src;
  pc.h = w - r * p.num_kv_heads;
  pc.cb = 0;
  pc.L = __builtin_amdgcn_readlane(in0 ? c0.L : c1.L, src);
  pc.Q = __builtin_amdgcn_readlane(in0 ? c0.Q : c1.Q, src);
  pc.row0 = (in0 ? __builtin_amdgcn_readlane(q0, src)
                 : __builtin_amdgcn_readlane(q0, 63) + __builtin_amdgcn_readlane(q1, src)) - pc.Q;
  pc.c_begin = 0;
  pc.c_end = __builtin_amdgcn_readlane(in0 ? n0 : n1, src);
  pc.whole = true;
  const int seg = pc.b * p.num_kv_heads + pc.h;
  pc.slot = seg + w;
  pc.b = __builtin_amdgcn_readfirstlane(pc.b);
  pc.L = __builtin_amdgcn_readfirstlane(pc.L);
  pc.Q = __builtin_amdgcn_readfirstlane(pc.Q);
  pc.row0 = __builtin_amdgcn_readfirstlane(pc.row0);
  pc.c_end = __builtin_amdgcn_readfirstlane(pc.c_end);
  pc.slot = __builtin_amdgcn_readfirstlane(pc.slot);
  if (leader) p.seg_merge[seg] = make_int2(pc.slot, 1);
  return true;
}

// ---- attention kernels -------------------------------------------------------
// NCT = 0 is the packed decode layout (at most 4 query columns; each wave is
// a unit) with PR groups in flight per wave, NCT = 1 one 16-column tile whose
// 4 waves take the chunks of a piece in turn (the workgroup is the unit).
// Two waves per SIMD (256 registers each), one for the packed layout with
// two groups in flight.
template <int D, int NCT, bool DUPLO, bool QF32, bool OUTF32, int PR, int KF, bool TL = false>
__global__ __launch_bounds__(64 * (NCT == 0 ? kPackedWaves : kWavesPerGroup),
                             (NCT == 0 ? (PR == 1 ? 2 : 1) : 2)) void attn_stream_kernel(StreamParams p) {
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int w = (NCT == 0) ? (int)blockIdx.x * kPackedWaves + wave : (int)blockIdx.x;
  const bool leader = lane == 0 && (NCT == 0 || wave == 0);

  Timeline<TL> tl = timeline_for<TL>(p, wave);
  tl.rec(kTlEntry, lane);
  if (blockIdx.x == 0 && wave == 0) write_seq_meta(p, lane);
  const SeqLens c0 = load_seq(p, lane);
  const SeqLens c1 = load_seq(p, 64 + lane);
  const int64_t T = total_chunks(p, lane, c0, c1);
  const int W = work_units(p, T);
  tl.rec(kTlLengths, lane);
  tl.rec(kTlScheduled, lane);
  if (w < W) {
    walk_pieces(p, lane, leader, w, W, T, c0, c1, [&](const PieceDesc& pc) {
      if constexpr (NCT == 0) {
        // at most 4 query columns: four pages per score tile
        run_piece_packed<D, QF32, OUTF32, PR, KF>(p, pc, lane, tl);
      } else {
        run_piece<D, NCT, DUPLO, QF32, OUTF32, 2, KF>(p, pc, lane, wave, tl);
      }
    });
  }
  tl.end(lane);
}

// Wide column blocks: NW waves share each chunk through LDS, NT tiles each,
// two waves per SIMD.  Ring depth (raw chunks ahead of the one converted):
// three with two waves per workgroup, six with four (a few workgroups per
// compute unit must keep ~48 KB in flight each), two with two tiles per
// wave, whose accumulators take the registers.
#ifndef TILE_RING2
#define TILE_RING2 3
#endif
#ifndef TILE_RING4
#define TILE_RING4 6
#endif
#ifndef TILE_RING_WIDE
#define TILE_RING_WIDE 2
#endif
template <int NW, int NT>
struct TileCfg {
  static constexpr int R = (NT == 2) ? TILE_RING_WIDE : (NW == 2 ? TILE_RING2 : TILE_RING4);
  static constexpr int WAVES_PER_SIMD = 2;
  static constexpr bool PP = TILE_PINGPONG && NW == 8;
};

template <int D, int NW, int NT, bool QF32, bool OUTF32, int KF, bool TL = false>
__global__ __launch_bounds__(64 * NW, (TileCfg<NW, NT>::WAVES_PER_SIMD)) void attn_tile_kernel(StreamParams p) {
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int w = blockIdx.x;
  const bool leader = lane == 0 && wave == 0;

  Timeline<TL> tl = timeline_for<TL>(p, wave);
  tl.rec(kTlEntry, lane);
  if (w == 0 && wave == 0) write_seq_meta(p, lane);
  const SeqLens c0 = load_seq(p, lane);
  const SeqLens c1 = load_seq(p, 64 + lane);
  const int64_t T = total_chunks(p, lane, c0, c1);
  const int W = work_units(p, T);
  tl.rec(kTlLengths, lane);
  if (w < W) {
    PieceDesc whole;
    if (whole_segment_piece(p, lane, leader, w, W, c0, c1, whole)) {
      tl.rec(kTlScheduled, lane);
      // its own inlined copy of the piece, specialised for a whole segment
      if (whole.c_end > 0)
        run_piece_tile<D, NW, NT, QF32, OUTF32, TileCfg<NW, NT>::R, KF, TileCfg<NW, NT>::PP>(p, whole, lane, wave,
                                                                                             tl);
    } else {
      tl.rec(kTlScheduled, lane);
      walk_pieces(p, lane, leader, w, W, T, c0, c1, [&](const PieceDesc& pc) {
        run_piece_tile<D, NW, NT, QF32, OUTF32, TileCfg<NW, NT>::R, KF, TileCfg<NW, NT>::PP>(p, pc, lane, wave, tl);
      });
    }
  } else {
    tl.rec(kTlScheduled, lane);  // an empty range
  }
  tl.end(lane);
}

// ---- log-sum-exp merge of the partials of one segment ---------------------
// out = sum_k 2^(m_k - m) O_k / sum_k 2^(m_k - m) l_k,  m = max_k m_k, over
// the pieces k of a segment.  Workgroup (s, y) of 256 threads takes segment
// s and its columns [y CW, (y+1) CW), CW = merge_cols (chosen by the plan:
// few columns per workgroup when segments have many pieces, up to the NG =
// 256 / (D/4) columns its NG groups of D/4 threads cover).  With C columns
// here (rounded up to a power of two), GPC = NG / C groups share a column, each
// merging the pieces k = phase, phase + GPC, ... online (four loads in
// flight), and the groups of a column are combined through LDS in phase
// order.  The result depends only on the pieces, not on timing.  Segments
// written whole by the attention kernel, and segments without chunks in
// this forward (their entry is stale), are skipped.
constexpr int kMergeThreads = 256;

template <int D, bool OUTF32>
__global__ __launch_bounds__(kMergeThreads) void split_merge_kernel(StreamParams p) {
  constexpr int V4 = D / 4;
  constexpr int NG = kMergeThreads / V4;
  const int s = blockIdx.x;
  const int cb = s % p.col_blocks;
  const int h = (s / p.col_blocks) % p.num_kv_heads;
  const int b = s / (p.col_blocks * p.num_kv_heads);
  // independent loads, issued together
  const int L = p.ctx_lens[b];
  const int Q = p.q_lens[b];
  const int2 sj = p.seg_merge[s];
  const int rows = p.seq_row0[b];
  const int G = p.group;
  const int col0 = cb * p.cols_per_block;
  if (seg_chunks(L, Q, G, p.cols_per_block, cb) == 0) return;
  const int slot0 = sj.x;
  const int nparts = sj.y;
  if (nparts <= 1) return;  // written whole by the attention kernel
  const int cw = p.merge_cols;
  const int cy0 = blockIdx.y * cw;
  const int cols_here = min(cw, min(p.cols_per_block, G * Q - col0) - cy0);
  if (cols_here <= 0) return;
  int cpass = 1;
  while (cpass < cols_here) cpass <<= 1;
  const int gpc = NG / cpass;
  const int grp = threadIdx.x / V4;
  const int t4 = threadIdx.x - grp * V4;
  const int d4 = t4 * 4;
  const int cl = grp / gpc;
  const int phase = grp - cl * gpc;
  const int rc = cy0 + cl;  // column inside the block
  const bool active = cl < cols_here;

  float mx = kNegInf;
  float lsum = 0.f;
  f32x4 acc = {0.f, 0.f, 0.f, 0.f};
  if (active) {
    for (int k0 = phase; k0 < nparts; k0 += 4 * gpc) {
      float mkp[4], lkp[4];
      f32x4 v[4];
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int k = k0 + q * gpc;
        if (k < nparts) {
          const size_t ri = (size_t)(slot0 + k) * p.cols_per_block + rc;
          mkp[q] = p.part_ml[ri * 2];
          lkp[q] = p.part_ml[ri * 2 + 1];
          v[q] = *reinterpret_cast<const f32x4*>(p.part_o + ri * D + d4);
        } else {
          mkp[q] = kNegInf;
          lkp[q] = 0.f;
          v[q] = f32x4{0.f, 0.f, 0.f, 0.f};
        }
      }
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const float mn = fmaxf(mx, mkp[q]);
        const float base = (mn == kNegInf) ? 0.f : mn;
        const float fo = __builtin_amdgcn_exp2f(mx - base);
        const float fk = __builtin_amdgcn_exp2f(mkp[q] - base);
        lsum = lsum * fo + lkp[q] * fk;
        acc = acc * fo + v[q] * fk;
        mx = mn;
      }
    }
  }
  if (gpc > 1) {
    // combine the phases of each column in phase order
    __shared__ f32x4 s_acc[NG][V4];
    __shared__ float s_m[NG], s_l[NG];
    s_acc[grp][t4] = acc;
    if (t4 == 0) {
      s_m[grp] = mx;
      s_l[grp] = lsum;
    }
    __syncthreads();
    if (phase != 0 || !active) return;
    float m_all = kNegInf;
    for (int j = 0; j < gpc; ++j) m_all = fmaxf(m_all, s_m[grp + j]);
    const float base = (m_all == kNegInf) ? 0.f : m_all;
    lsum = 0.f;
    acc = f32x4{0.f, 0.f, 0.f, 0.f};
    for (int j = 0; j < gpc; ++j) {
      const float f = __builtin_amdgcn_exp2f(s_m[grp + j] - base);
      lsum += s_l[grp + j] * f;
      acc += s_acc[grp + j][t4] * f;
    }
  }
  if (!active) return;
  const float inv = 1.f / lsum;
  const int gc = col0 + rc;
  const int i = gc / G;
  const int gg = gc - i * G;
  const size_t off = ((size_t)(rows + i) * p.num_q_heads + h * G + gg) * D + d4;
  if constexpr (OUTF32) {
    *reinterpret_cast<f32x4*>(static_cast<float*>(p.out) + off) = acc * inv;
  } else {
    const uint32_t w0 = pack_bf16(acc[0] * inv, acc[1] * inv);
    const uint32_t w1 = pack_bf16(acc[2] * inv, acc[3] * inv);
    *reinterpret_cast<uint2*>(static_cast<uint16_t*>(p.out) + off) = make_uint2(w0, w1);
  }
}

// ---- dispatch --------------------------------------------------------------

// With tl, the kernels that record a timeline: built for E4M3 KV with bf16
// Q and output only (nullptr otherwise).
template <int D, int NCT, bool DUPLO, int PR = 1>
static const void* kernel_d(const Variant& v, bool tl) {
  if (tl) {
    if (v.kv_format != kKvE4M3 || v.q_f32 || v.out_f32) return nullptr;
    return reinterpret_cast<const void*>(&attn_stream_kernel<D, NCT, DUPLO, false, false, PR, kKvE4M3, true>);
  }
  // INT8 and INT4 KV: bf16 Q and output only (the plan rejects the rest)
  if (v.kv_format == kKvInt8)
    return reinterpret_cast<const void*>(&attn_stream_kernel<D, NCT, DUPLO, false, false, PR, kKvInt8>);
  if (v.kv_format == kKvInt4) {
    if constexpr (D == 128)
      return reinterpret_cast<const void*>(&attn_stream_kernel<D, NCT, DUPLO, false, false, PR, kKvInt4>);
    return nullptr;
  }
  if (v.q_f32 && v.out_f32)
    return reinterpret_cast<const void*>(&attn_stream_kernel<D, NCT, DUPLO, true, true, PR, kKvE4M3>);
  if (v.q_f32) return reinterpret_cast<const void*>(&attn_stream_kernel<D, NCT, DUPLO, true, false, PR, kKvE4M3>);
  if (v.out_f32) return reinterpret_cast<const void*>(&attn_stream_kernel<D, NCT, DUPLO, false, true, PR, kKvE4M3>);
  return reinterpret_cast<const void*>(&attn_stream_kernel<D, NCT, DUPLO, false, false, PR, kKvE4M3>);
}

template <int D, int NW, int NT>
static const void* tile_d(const Variant& v, bool tl) {
  if (tl) {
    if (v.kv_format != kKvE4M3 || v.q_f32 || v.out_f32) return nullptr;
    return reinterpret_cast<const void*>(&attn_tile_kernel<D, NW, NT, false, false, kKvE4M3, true>);
  }
  if (v.kv_format == kKvInt8) return reinterpret_cast<const void*>(&attn_tile_kernel<D, NW, NT, false, false, kKvInt8>);
  if (v.kv_format == kKvInt4) {
    if constexpr (D == 128) return reinterpret_cast<const void*>(&attn_tile_kernel<D, NW, NT, false, false, kKvInt4>);
    return nullptr;
  }
  if (v.q_f32 && v.out_f32) return reinterpret_cast<const void*>(&attn_tile_kernel<D, NW, NT, true, true, kKvE4M3>);
  if (v.q_f32) return reinterpret_cast<const void*>(&attn_tile_kernel<D, NW, NT, true, false, kKvE4M3>);
  if (v.out_f32) return reinterpret_cast<const void*>(&attn_tile_kernel<D, NW, NT, false, true, kKvE4M3>);
  return reinterpret_cast<const void*>(&attn_tile_kernel<D, NW, NT, false, false, kKvE4M3>);
}

template <int D>
static const void* kernel_tiles(const Variant& v, bool tl) {
  if (v.packed) return v.packed_ring == 2 ? kernel_d<D, 0, false, 2>(v, tl) : kernel_d<D, 0, false, 1>(v, tl);
  if (v.tile_waves == 2 && v.col_tiles == 1) return tile_d<D, 2, 1>(v, tl);
  if (v.tile_waves == 4 && v.col_tiles == 1) return tile_d<D, 4, 1>(v, tl);
  if (v.tile_waves == 4 && v.col_tiles == 2) return tile_d<D, 4, 2>(v, tl);
  if constexpr (D == 128) {
    if (v.tile_waves == 8 && v.col_tiles == 2) return tile_d<D, 8, 2>(v, tl);
  }
  if (v.tile_waves != 0 || v.col_tiles != 1) return nullptr;
  return v.dup_lo ? kernel_d<D, 1, true>(v, tl) : kernel_d<D, 1, false>(v, tl);
}

static const void* stream_kernel(const Variant& v, bool tl = false) {
  if (v.head_dim == 128) return kernel_tiles<128>(v, tl);
  if (v.head_dim == 64) return kernel_tiles<64>(v, tl);
  return nullptr;
}

hipError_t stream_attention_occupancy(const Variant& v, int* blocks_per_cu) {
  const void* f = stream_kernel(v);
  if (!f) return hipErrorInvalidValue;
  return hipOccupancyMaxActiveBlocksPerMultiprocessor(blocks_per_cu, f, 64 * waves_per_group(v), 0);
}

bool timeline_supported(const Variant& v) { return stream_kernel(v, true) != nullptr; }

hipError_t launch_stream_attention(const Variant& v, const StreamParams& p, int grid, hipStream_t stream,
                                   hipEvent_t ev_start, hipEvent_t ev_stop) {
  if (grid <= 0) return hipSuccess;
  const void* f = stream_kernel(v, p.timeline != nullptr);
  if (!f) return hipErrorInvalidValue;
  void* args[] = {const_cast<StreamParams*>(&p)};
  if (ev_start) {
    // the events take the timestamps of this kernel's own dispatch
    return hipExtLaunchKernel(f, dim3(grid), dim3(64 * waves_per_group(v)), args, 0, stream, ev_start, ev_stop, 0);
  }
  return hipLaunchKernel(f, dim3(grid), dim3(64 * waves_per_group(v)), args, 0, stream);
}

// Columns per merge workgroup: one for blocks of at most 4 columns (decode);
// otherwise the NG = 256 / (D/4) thread groups are spread over a column's
// pieces (expected_parts per segment) so that each group still merges two
// or more of them, and the rest of the groups take further columns.  (On
// 64-column MQA blocks with ~8 pieces, two columns per workgroup measured
// faster than one column over all eight groups or eight columns of one.)
int merge_cols_for(const Variant& v, int cols_per_block, int64_t expected_parts) {
  if (cols_per_block <= 4) return 1;
  const int ng = kMergeThreads / (v.head_dim / 4);
  int spread = 1;
  while (2 * spread < expected_parts && spread < ng) spread <<= 1;
  return ng / spread;
}

int merge_grid_y(int cols_per_block, int merge_cols) {
  return (cols_per_block + merge_cols - 1) / merge_cols;
}

hipError_t launch_split_merge(const Variant& v, const StreamParams& p, int grid, hipStream_t stream,
                              hipEvent_t ev_start, hipEvent_t ev_stop) {
  if (grid <= 0) return hipSuccess;
  const dim3 g(grid, merge_grid_y(p.cols_per_block, p.merge_cols));
  const dim3 block(kMergeThreads);
  const void* f = nullptr;
  if (v.head_dim == 128) {
    f = v.out_f32 ? reinterpret_cast<const void*>(&split_merge_kernel<128, true>)
                  : reinterpret_cast<const void*>(&split_merge_kernel<128, false>);
  } else if (v.head_dim == 64) {
    f = v.out_f32 ? reinterpret_cast<const void*>(&split_merge_kernel<64, true>)
                  : reinterpret_cast<const void*>(&split_merge_kernel<64, false>);
  } else {
    return hipErrorInvalidValue;
  }
  void* args[] = {const_cast<StreamParams*>(&p)};
  if (ev_start) return hipExtLaunchKernel(f, g, block, args, 0, stream, ev_start, ev_stop, 0);
  return hipLaunchKernel(f, g, block, args, 0, stream);
}

}  // namespace pa
