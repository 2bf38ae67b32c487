// Paged FP8-KV attention for gfx950: one workgroup per (sequence, kv head,
// block of query columns, key partition), KV streamed from HBM straight into
// MFMA operand registers.
//
// Follows the attention section of the Atlas engine article (ainews.cool,
// "技术深度解析": a FlashAttention-2 variant with dedicated MQA/GQA kernels),
// its quantisation section (FP8 with per-group scales folded into the
// kernel) and the paged FP8 KV cache of the GB10 article (ainews.surl.tw).
//
// Shape of the work.  The G = Hq/Hkv query heads of a kv head, times the Q_b
// new tokens of a sequence, form G*Q_b "query columns" that all read the same
// keys.  A workgroup owns up to 16*col_tiles of them (decode: the G heads;
// MTP verification: 5 tokens x G heads; prefill: a slice of tokens x G) and a
// partition of the keys.  Its 4 waves take 32-key chunks (two pages) in turn.
//
// Per chunk, in each wave (lane = 16*lq + ln):
//   * K: lane reads 32 (D=128) contiguous bytes of token slot ln at
//     d in [lq*D/4, (lq+1)*D/4) of both pages -- 16-byte loads, the whole
//     2 KB (page, head) chunk covered once by the wave;
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
//     the V page layout makes each lane's operand 32 contiguous bytes.
// Waves then merge their (m, l, O) through LDS; a workgroup writes the final
// output, or an unnormalised partial that a second small kernel merges by
// log-sum-exp with the other partitions of its (sequence, kv head).

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "device_common.h"
#include "kernel_params.h"

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

constexpr float kNegInf = -__builtin_huge_valf();

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

__device__ __forceinline__ int xcd_remap(int bid, int n) {
  // Workgroups are handed to the 8 XCDs round-robin; map consecutive logical
  // items onto one XCD so items sharing a kv head share that XCD's L2.
  const int per = n >> 3;
  if (bid >= (per << 3)) return bid;
  return (bid & 7) * per + (bid >> 3);
}

__device__ __forceinline__ int prefix_rows(const int32_t* q_lens, int b, int lane) {
  int acc = 0;
  for (int k = lane; k < b; k += 64) acc += q_lens[k];
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) acc += __shfl_xor(acc, off);
  return __builtin_amdgcn_readfirstlane(acc);
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

}  // namespace

// ---- log-sum-exp merge of key partitions --------------------------------
// out = sum_s 2^(m_s - m) O_s / sum_s 2^(m_s - m) l_s,  m = max_s m_s,
// over the partials of one (sequence, kv head, column block), in split order.
template <int D, bool OUTF32>
__device__ __forceinline__ void merge_partials(const StreamParams& p, size_t item0, int nsplit, int cols_here,
                                               int col0, int row0, int h) {
  constexpr int V4 = D / 4;
  const int G = p.group;
  for (int e = threadIdx.x; e < cols_here * V4; e += blockDim.x) {
    const int rc = e / V4;
    const int d4 = (e - rc * V4) * 4;
    float mx = kNegInf;
    for (int s = 0; s < nsplit; ++s) mx = fmaxf(mx, p.part_ml[((item0 + s) * p.cols_per_block + rc) * 2]);
    const float base = (mx == kNegInf) ? 0.f : mx;
    float lsum = 0.f;
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
    for (int s = 0; s < nsplit; ++s) {
      const size_t ri = (item0 + s) * p.cols_per_block + rc;
      const float w = __builtin_amdgcn_exp2f(p.part_ml[ri * 2] - base);
      lsum += w * p.part_ml[ri * 2 + 1];
      const f32x4 v = *reinterpret_cast<const f32x4*>(p.part_o + ri * D + d4);
      acc += v * w;
    }
    const float inv = 1.f / lsum;
    const int gc = col0 + rc;
    const int i = gc / G;
    const int g = gc - i * G;
    const size_t off = ((size_t)(row0 + i) * p.num_q_heads + h * G + g) * D + d4;
    if constexpr (OUTF32) {
      *reinterpret_cast<f32x4*>(static_cast<float*>(p.out) + off) = acc * inv;
    } else {
      const uint32_t w0 = pack_bf16(acc[0] * inv, acc[1] * inv);
      const uint32_t w1 = pack_bf16(acc[2] * inv, acc[3] * inv);
      *reinterpret_cast<uint2*>(static_cast<uint16_t*>(p.out) + off) = make_uint2(w0, w1);
    }
  }
}

template <int D, int NCT, bool DUPLO, bool QF32, bool OUTF32>
__global__ __launch_bounds__(64 * kWavesPerGroup) void attn_stream_kernel(StreamParams p) {
  using GD = Geo<D>;
  constexpr int NW = kWavesPerGroup;
  constexpr int NP = QF32 ? 3 : 1;
  static_assert(!DUPLO || NCT == 1, "spare-column low parts need a single tile");

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int lq = lane >> 4;
  const int ln = lane & 15;

  // ---- work item -------------------------------------------------------
  int item = xcd_remap(blockIdx.x, gridDim.x);
  const int item_id = item;
  const int split = item % p.num_splits;
  item /= p.num_splits;
  const int cb = item % p.col_blocks;
  item /= p.col_blocks;
  const int h = item % p.num_kv_heads;
  const int b = item / p.num_kv_heads;

  const int L = p.ctx_lens[b];
  const int Qb = p.q_lens[b];
  const int G = p.group;
  const int ncols = G * Qb;
  const int col0 = cb * p.cols_per_block;
  if (col0 >= ncols) return;
  const int cols_here = min(p.cols_per_block, ncols - col0);
  const int i_lo = col0 / G;
  const int i_hi = (col0 + cols_here - 1) / G;
  const int kv_end = L - Qb + i_hi + 1;  // keys seen by at least one column here
  const int nchunks = (kv_end + 31) >> 5;
  const int c_begin = split * p.chunks_per_split;
  if (c_begin >= nchunks) return;
  const int c_end = min(c_begin + p.chunks_per_split, nchunks);
  const int nsplit_here = (nchunks + p.chunks_per_split - 1) / p.chunks_per_split;
  const int row0 = (p.max_q_len == 1) ? b : prefix_rows(p.q_lens, b, lane);
  const int first_masked_key = L - Qb + i_lo + 1;  // keys >= this are hidden from some column
  const int npages = (L + kPageSize - 1) / kPageSize;

  // ---- this lane's query columns and Q operand ----------------------------
  int lim[NCT];        // last visible key of the lane's column (-1: unused column)
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
    qrow[t] = row0 + i;
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

  const int32_t* bt = p.block_table + (size_t)b * p.bt_stride;
  const uint32_t koff = k_in_chunk(ln, lq * GD::DQ, D);
  const uint32_t voff = v_in_chunk(4 * lq, GD::NVB * ln, D);
  const uint8_t* kpool = p.k_pages;
  const uint8_t* vpool = p.v_pages;

  // ---- chunk loop --------------------------------------------------------
  // This wave's chunks are c_k = c_begin + wave + k * NW, k < nk.  The block
  // table entries and the K/V page scales of the next 32 chunks are fetched
  // by one gather (lane j: chunk k0 + j/2, page j%2) and read with readlane,
  // so the loop never waits on a scalar memory load.  K/V bytes of chunk
  // k+1 are in flight while chunk k is computed.
  const int nk = (c_begin + wave < c_end) ? (c_end - c_begin - wave + NW - 1) / NW : 0;
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
      a = p.kv_scales[sidx];
      bsc = p.kv_scales[p.v_scale_offset + sidx];
    }
    bt_v = ph;
    sk_v = a;
    sv_v = bsc;
  };
  u32x4 kr[2][GD::NKV], vr[2][GD::NVV];
  auto load_kv = [&](int k) {
    const int slot = 2 * (k & 31);
#pragma unroll
    for (int pg = 0; pg < 2; ++pg) {
      const int32_t ph = __builtin_amdgcn_readlane(bt_v, slot + pg);
      const uint64_t base = chunk_offset(ph, h, p.num_kv_heads, D);
      const u32x4* kp = reinterpret_cast<const u32x4*>(kpool + base + koff);
      const u32x4* vp = reinterpret_cast<const u32x4*>(vpool + base + voff);
#pragma unroll
      for (int i = 0; i < GD::NKV; ++i) kr[pg][i] = __builtin_nontemporal_load(kp + i);
#pragma unroll
      for (int i = 0; i < GD::NVV; ++i) vr[pg][i] = __builtin_nontemporal_load(vp + i);
    }
  };

  if (nk > 0) {
    load_batch(0);
    load_kv(0);
  }
  for (int k = 0; k < nk; ++k) {
    const int c = c_begin + wave + k * NW;
    u32x4 kc[2][GD::NKV], vc[2][GD::NVV];
#pragma unroll
    for (int pg = 0; pg < 2; ++pg) {
#pragma unroll
      for (int i = 0; i < GD::NKV; ++i) kc[pg][i] = kr[pg][i];
#pragma unroll
      for (int i = 0; i < GD::NVV; ++i) vc[pg][i] = vr[pg][i];
    }
    const int slot = 2 * (k & 31);
    float skc[2], svc[2];
    skc[0] = __uint_as_float(__builtin_amdgcn_readlane(__float_as_uint(sk_v), slot));
    skc[1] = __uint_as_float(__builtin_amdgcn_readlane(__float_as_uint(sk_v), slot + 1));
    svc[0] = __uint_as_float(__builtin_amdgcn_readlane(__float_as_uint(sv_v), slot));
    svc[1] = __uint_as_float(__builtin_amdgcn_readlane(__float_as_uint(sv_v), slot + 1));
    if (k + 1 < nk) {
      if (((k + 1) & 31) == 0) load_batch(k + 1);
      load_kv(k + 1);
    }

    // S^T = K Q^T for both pages
    f32x4 sacc[2][NCT];
#pragma unroll
    for (int pg = 0; pg < 2; ++pg) {
#pragma unroll
      for (int t = 0; t < NCT; ++t) sacc[pg][t] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int s = 0; s < GD::NSLAB; ++s) {
        const u32x4 w = kc[pg][(2 * s) / 4];
        const bf16x8 kb = fp8x8_to_bf16x8(w[(2 * s) % 4], w[(2 * s) % 4 + 1]);
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
    const int key0 = c * 32 + 4 * lq;  // key of register j: key0 + j (page 0), key0 + 16 + j (page 1)
    const bool need_mask = (c * 32 + 31) >= first_masked_key;
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
      for (int k = 0; k < 4; ++k) {
        const float sc = (k < 2) ? svc[0] : svc[1];
        const float a = pr[2 * k] * sc;
        const float bb = pr[2 * k + 1] * sc;
        const uint32_t hw = pack_bf16(a, bb);
        const uint32_t lw = pack_bf16(a - bf16_lo(hw), bb - bf16_hi(hw));
        if constexpr (DUPLO) {
          phi[t][k] = lo_lane ? lw : hw;
        } else {
          phi[t][k] = hw;
          plo[t][k] = lw;
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
    const bool tail = (c * 32 + 32) > L;
    uint32_t vmask0 = 0xffffffffu, vmask1 = 0xffffffffu;
    if (tail) {
      vmask0 = 0u;
      vmask1 = 0u;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        vmask0 |= (key0 + j < L) ? (0xffu << (8 * j)) : 0u;
        vmask1 |= (key0 + 16 + j < L) ? (0xffu << (8 * j)) : 0u;
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
      const uint32_t w0 = vc[0][cblk / 4][cblk % 4] & vmask0;
      const uint32_t w1 = vc[1][cblk / 4][cblk % 4] & vmask1;
      const bf16x8 va = fp8x8_to_bf16x8(w0, w1);
#pragma unroll
      for (int t = 0; t < NCT; ++t) {
        o[t][cblk] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(va, pop_hi[t], o[t][cblk], 0, 0, 0);
        if constexpr (!DUPLO)
          o[t][cblk] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(va, pop_lo[t], o[t][cblk], 0, 0, 0);
      }
    }
  }

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
  // ---- write: final output, or a partial plus the last-arriver merge ------
  const bool final_out = (nsplit_here == 1);
  if (wave == 0) {
#pragma unroll
    for (int t = 0; t < NCT; ++t) {
      const int rc = DUPLO ? ln : (16 * t + ln);
      if (rc >= cols_here || (DUPLO && ln >= 8)) continue;
      if (final_out) {
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
        float* po = p.part_o + ((size_t)item_id * p.cols_per_block + rc) * D;
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
          float* pm = p.part_ml + ((size_t)item_id * p.cols_per_block + rc) * 2;
          pm[0] = m[t];
          pm[1] = l[t];
        }
      }
    }
  }
}

// One workgroup per (sequence, kv head, column block) whose keys were split:
// merges its partitions' partials in split order.  Launched right after the
// attention kernel on the same stream.
template <int D, bool OUTF32>
__global__ __launch_bounds__(256) void split_merge_kernel(StreamParams p) {
  int item = blockIdx.x;
  const int cb = item % p.col_blocks;
  item /= p.col_blocks;
  const int h = item % p.num_kv_heads;
  const int b = item / p.num_kv_heads;
  const int L = p.ctx_lens[b];
  const int Qb = p.q_lens[b];
  const int G = p.group;
  const int ncols = G * Qb;
  const int col0 = cb * p.cols_per_block;
  if (col0 >= ncols) return;
  const int cols_here = min(p.cols_per_block, ncols - col0);
  const int i_hi = (col0 + cols_here - 1) / G;
  const int nchunks = (L - Qb + i_hi + 1 + 31) >> 5;
  const int nsplit = (nchunks + p.chunks_per_split - 1) / p.chunks_per_split;
  if (nsplit <= 1) return;  // the attention kernel wrote this block's output itself
  const int row0 = (p.max_q_len == 1) ? b : prefix_rows(p.q_lens, b, threadIdx.x & 63);
  merge_partials<D, OUTF32>(p, (size_t)blockIdx.x * p.num_splits, nsplit, cols_here, col0, row0, h);
}


// ---- dispatch --------------------------------------------------------------

template <int D, int NCT, bool DUPLO>
static hipError_t launch_d(const Variant& v, const StreamParams& p, int grid, hipStream_t stream) {
  const dim3 block(64 * kWavesPerGroup);
  if (v.q_f32 && v.out_f32)
    hipLaunchKernelGGL((attn_stream_kernel<D, NCT, DUPLO, true, true>), dim3(grid), block, 0, stream, p);
  else if (v.q_f32)
    hipLaunchKernelGGL((attn_stream_kernel<D, NCT, DUPLO, true, false>), dim3(grid), block, 0, stream, p);
  else if (v.out_f32)
    hipLaunchKernelGGL((attn_stream_kernel<D, NCT, DUPLO, false, true>), dim3(grid), block, 0, stream, p);
  else
    hipLaunchKernelGGL((attn_stream_kernel<D, NCT, DUPLO, false, false>), dim3(grid), block, 0, stream, p);
  return hipGetLastError();
}

template <int D>
static hipError_t launch_tiles(const Variant& v, const StreamParams& p, int grid, hipStream_t stream) {
  if (v.dup_lo) return launch_d<D, 1, true>(v, p, grid, stream);
  switch (v.col_tiles) {
    case 1: return launch_d<D, 1, false>(v, p, grid, stream);
    case 2: return launch_d<D, 2, false>(v, p, grid, stream);
    case 4: return launch_d<D, 4, false>(v, p, grid, stream);
    default: return hipErrorInvalidValue;
  }
}

hipError_t launch_stream_attention(const Variant& v, const StreamParams& p, int grid, hipStream_t stream) {
  if (grid <= 0) return hipSuccess;
  if (v.head_dim == 128) return launch_tiles<128>(v, p, grid, stream);
  if (v.head_dim == 64) return launch_tiles<64>(v, p, grid, stream);
  return hipErrorInvalidValue;
}

hipError_t launch_split_merge(const Variant& v, const StreamParams& p, int grid, hipStream_t stream) {
  if (grid <= 0) return hipSuccess;
  const dim3 block(256);
  if (v.head_dim == 128) {
    if (v.out_f32) hipLaunchKernelGGL((split_merge_kernel<128, true>), dim3(grid), block, 0, stream, p);
    else hipLaunchKernelGGL((split_merge_kernel<128, false>), dim3(grid), block, 0, stream, p);
  } else if (v.head_dim == 64) {
    if (v.out_f32) hipLaunchKernelGGL((split_merge_kernel<64, true>), dim3(grid), block, 0, stream, p);
    else hipLaunchKernelGGL((split_merge_kernel<64, false>), dim3(grid), block, 0, stream, p);
  } else {
    return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace pa
