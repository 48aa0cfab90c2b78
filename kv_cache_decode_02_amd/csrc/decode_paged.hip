// Split-KV decode attention over a paged cache: partial results.
//
// What is computed (per sequence b, query head h, K/V head g = h / r):
//   z_t = scale * q . K_t,  out = sum_t softmax(z)_t V_t  over t < seq_lens[b]
// ("KV缓存原理与显存估算", 知识点二, the z / a / o equations; the single
// decode row sees every cached position, "单请求 KV Cache", 改动三).
// The positions are cut into pieces; for each (b, h, piece) a kernel here
// writes the running maximum m (log2 units), the sum l = sum 2^(z' - m) and
// the unnormalised acc = sum 2^(z' - m) V_t, with z' = z * log2(e).
// decode_merge.hip combines the pieces.
//
// Per wavefront: a unit is one KV head g and a chunk of HPW query heads of
// its group.  The 64 lanes form 8 groups of 8 lanes.  For each 16-token block
// the group k handles tokens k and k + 8; inside a group each lane owns D/8
// dimensions of the row, loaded as 16-byte (or 8-byte) vectors laid out so
// that one load instruction of the 8 lanes covers a contiguous 128 B of the
// row.  A K/V row is loaded from HBM once and used by all HPW query heads from
// registers (the GQA sharing), so the cache is read exactly once.
//   Scores: per-lane bf16 dot2 partial sums, reduced over the 8 lanes of the
//   group with DPP moves.
//   Softmax: every lane group keeps its own running max; the reference max is
//   only raised when a score exceeds it by more than kRaise (log2 units),
//   which keeps every exponential below 2^kRaise and makes rescaling of the
//   accumulators rare.  The groups are merged when a piece is written.
//   Latency: blocks stream through NBUF register buffers, so NBUF - 1 blocks
//   of loads are in flight while one is being computed.
//
// Two decompositions:
//   fixed partitions (partition_tokens > 0): one wavefront per (b, partition,
//     unit), paged_partials_kernel;
//   balanced split (automatic mode): one workgroup per compute unit, each
//     streaming an equal share of all blocks, paged_balanced_kernel.
#include <stdlib.h>
#include <string.h>

#include "kvd_device.h"
#include "kvd_internal.h"

namespace kvd {
namespace {

// Storage of the K/V cache: fp32, bf16, or one-byte codes (INT8 or FP8 E4M3)
// with per-channel K and per-token V scales.
enum Kind : int { kF32 = 0, kBF16 = 1, kI8 = 2, kF8 = 3 };

constexpr float kRaise = 8.0f;
constexpr int kMaxPartitionBlocks = 64;  // one block id per lane
constexpr int kMinPieceBlocks = kBalancedMinPieceBlocks;
// Relative share of a workgroup on an even and an odd XCD (workgroup k runs
// on XCD k mod 8), per 1000 for an odd one; each worker flavour sets its
// even share (kEvenXcdShare).  Measured on MI355X with the GQA decode batch:
// with the VALU flavour, streaming the same number of blocks takes the odd
// XCDs 6-9% longer and a sweep of the even share over 1.00 .. 1.17 gives the
// shortest kernel at 1.11 - 1.14; the MFMA flavour does best near 1.06
// (per-workgroup end times show which XCDs lag changing from run to run).
constexpr long long kOddXcdShare = 1000;
// Virtual blocks charged for each segment (sequence, unit group) a share
// starts: the restart (query and block-id loads, then the first blocks'
// loads) costs a few blocks' time.  Measured on MI355X with the GQA decode
// batch over 0 .. 6: shortest at 3 - 4 (1.3% below 1), the MHA batch
// unchanged.
#ifndef KVD_SEGMENT_COST
#define KVD_SEGMENT_COST 4
#endif
constexpr int kSegmentCost = KVD_SEGMENT_COST;

template <int KT, int D>
struct RowShape {
  static constexpr int EPW = KT == kF32 ? 1 : (KT == kBF16 ? 2 : 4);  // elements per word
  static constexpr int DPL = D / 8;         // elements of a row per lane
  static constexpr int W = DPL / EPW;       // words of a row per lane
  static constexpr int CW = W < 4 ? W : 4;  // words per vector load
  static constexpr int NCH = W / CW;        // vector loads per row per lane
  static constexpr int RW = D / EPW;        // words per row (one head)
  // Query words per lane: one-byte codes are widened to fp16 pairs, so each
  // code word meets two words of (scaled) query.
  static constexpr int QW = KT >= kI8 ? 2 * W : W;
  static_assert(W >= 1 && W % CW == 0, "unsupported head_dim");
  // Word offset, inside a row, of the lane's chunk c.
  static __device__ __forceinline__ int chunk_word(int c, int sub) { return (c * 8 + sub) * CW; }
  // Dimension of the lane's e-th element.
  static __device__ __forceinline__ int dim_of(int e, int sub) {
    const int w = e / EPW;
    return (chunk_word(w / CW, sub) + w % CW) * EPW + e % EPW;
  }
};

// Running softmax state of HPW query heads; each lane holds its D / 8
// dimensions of every accumulator.  INT8 cache: vb[h] is the sum of the
// weights that met biased V codes since the bias was last taken out of acc.
template <int HPW, int DPL>
struct HeadState {
  float m[HPW], l[HPW], vb[HPW], acc[HPW][DPL];
};

template <int HPW, int DPL>
__device__ __forceinline__ void reset_state(HeadState<HPW, DPL>& st) {
#pragma unroll
  for (int h = 0; h < HPW; ++h) {
    st.m[h] = kMinusBig;
    st.l[h] = 0.f;
    st.vb[h] = 0.f;
#pragma unroll
    for (int e = 0; e < DPL; ++e) st.acc[h][e] = 0.f;
  }
}

// INT8 codes as fp16 numbers with a bias: the signed byte c becomes the fp16
// value 1024 + (c + 128) = kI8Bias + c, exactly.  With 0x64 as the high byte
// the number lies in [1024, 2048), where fp16 steps by 1, and the low byte
// c xor 0x80 is c + 128.  A byte permute builds two of them per instruction,
// against three instructions (two conversions and a pack) for exact codes.
// The scores start from -kI8Bias times the sum of the query terms, and the
// value sums drop kI8Bias times the weights they took (HeadState::vb).
constexpr float kI8Bias = 1152.0f;
constexpr uint32_t kBiasHigh = 0x64646464u;
constexpr uint32_t kSignBits = 0x80808080u;

// Codes 2i and 2i + 1 of word w (already xor kSignBits) as a biased pair.
__device__ __forceinline__ uint32_t biased_pair(uint32_t u, int i) {
  return __builtin_amdgcn_perm(kBiasHigh, u, i == 0 ? 0x04010400u : 0x04030402u);
}
// Code i of words w0 (low half) and w1 (high half) as a biased pair: the
// permute puts the two bytes under zero high bytes, the xor flips their sign
// bits and sets the high bytes to 0x64.
__device__ __forceinline__ uint32_t biased_tokens(uint32_t w0, uint32_t w1, int i) {
  const uint32_t sel = 0x0c000c00u | static_cast<uint32_t>(4 + i) << 16 | static_cast<uint32_t>(i);
  return __builtin_amdgcn_perm(w1, w0, sel) ^ 0x64806480u;
}

// Takes the INT8 value bias out of the accumulators (kept below ~64 blocks
// of weights, so the fp32 sums keep their precision).
template <int HPW, int DPL>
__device__ __forceinline__ void unbias(HeadState<HPW, DPL>& st) {
#pragma unroll
  for (int h = 0; h < HPW; ++h) {
#pragma unroll
    for (int e = 0; e < DPL; ++e) st.acc[h][e] = fmaf(-kI8Bias, st.vb[h], st.acc[h][e]);
    st.vb[h] = 0.f;
  }
}

// The K and V rows of the lane's two token slots of one block (one-byte
// caches: codes, and the two tokens' V scales).
template <int KT, int D>
struct Frag {
  uint32_t k[2][RowShape<KT, D>::W];
  uint32_t v[2][RowShape<KT, D>::W];
  float vs[KT >= kI8 ? 2 : 1];
};

// Query slice of heads h0 .. h0 + HPW - 1 of sequence b, in the lane layout of
// the K rows.  One-byte caches: the query is bf16 and is multiplied by KV head g's
// per-channel K scales (q . (s * code) = (q * s) . code), then rounded to
// fp16 pairs that meet the widened codes in dot2 (fp16 keeps 11 bits of the
// scaled query; bf16's 8 would cost ~0.5% in the scores).
template <int KT, int D, int HPW>
__device__ __forceinline__ void load_query(const PagedLaunch& a, int lane, int b, int h0, int g,
                                           uint32_t (&qv)[HPW][RowShape<KT, D>::QW],
                                           float (&qb)[HPW]) {
  using S = RowShape<KT, D>;
  const int sub = lane & 7;
  if constexpr (KT >= kI8) {
    const uint32_t* qw = static_cast<const uint32_t*>(a.q) +
                         (static_cast<size_t>(b) * a.num_q_heads + h0) * (D / 2);
    const float* ks = a.k_scale + static_cast<size_t>(g) * D;
#pragma unroll
    for (int c = 0; c < S::NCH; ++c)
#pragma unroll
      for (int w = 0; w < S::CW; ++w) {
        const int d0 = (S::chunk_word(c, sub) + w) * 4;  // the code word's 4 dimensions
        const float4 s4 = *reinterpret_cast<const float4*>(ks + d0);
#pragma unroll
        for (int h = 0; h < HPW; ++h) {
          uint32_t q2[2];
          load_words<2>(q2, qw + h * (D / 2) + d0 / 2);
          const int k = c * S::CW + w;
          qv[h][2 * k] = pack_f16x2(bf16_lo(q2[0]) * s4.x, bf16_hi(q2[0]) * s4.y);
          qv[h][2 * k + 1] = pack_f16x2(bf16_lo(q2[1]) * s4.z, bf16_hi(q2[1]) * s4.w);
        }
      }
    // INT8: each score starts from -kI8Bias times the lane's query terms,
    // summed from the same fp16 values the products use.  (FP8 codes widen
    // exactly, with no bias.)
#pragma unroll
    for (int h = 0; h < HPW; ++h) {
      float t = 0.f;
#pragma unroll
      for (int i = 0; i < S::QW; ++i) t = dot2_f16(qv[h][i], kF16OnePair, t);
      qb[h] = KT == kI8 ? -kI8Bias * t : 0.f;
    }
  } else {
    const uint32_t* qw = static_cast<const uint32_t*>(a.q) +
                         (static_cast<size_t>(b) * a.num_q_heads + h0) * S::RW;
#pragma unroll
    for (int h = 0; h < HPW; ++h)
#pragma unroll
      for (int c = 0; c < S::NCH; ++c)
        load_words<S::CW>(&qv[h][c * S::CW], qw + h * S::RW + S::chunk_word(c, sub));
  }
}

// Issues the loads of physical block `blk` for KV head g: the lane's two token
// rows of K and V.  One buffer resource per tensor whose record count ends
// after the block's nvalid valid tokens: rows past them (the unused tail of a
// sequence's last block, contents arbitrary) and a block with nvalid == 0
// read back as zeros without touching memory.
// Token rows tok (grp + 8 tok) of KV head g from K and V arrays laid out like
// a cache block (token rows of num_kv_heads * head_dim values), nvalid rows.
template <int KT, int D>
__device__ __forceinline__ void load_rows(Frag<KT, D>& f, const uint32_t* kbase,
                                          const uint32_t* vbase, const PagedLaunch& a, int lane,
                                          int g, int nvalid, const float* sbase = nullptr) {
  using S = RowShape<KT, D>;
  const int grp = lane >> 3;
  const int sub = lane & 7;
  const size_t tok_stride = static_cast<size_t>(a.num_kv_heads) * S::RW;  // words per token
  const int bytes = nvalid * static_cast<int>(tok_stride) * 4;
  const BufRsrc rk = make_rsrc(kbase, bytes);
  const BufRsrc rv = make_rsrc(vbase, bytes);
#pragma unroll
  for (int tok = 0; tok < 2; ++tok) {
    const uint32_t off = static_cast<uint32_t>(
        ((grp + 8 * tok) * tok_stride + g * S::RW + S::chunk_word(0, sub)) * 4);
#pragma unroll
    for (int c = 0; c < S::NCH; ++c) {
      buffer_load_words<S::CW>(&f.k[tok][c * S::CW], rk, off + c * 8 * S::CW * 4);
      buffer_load_words<S::CW>(&f.v[tok][c * S::CW], rv, off + c * 8 * S::CW * 4);
    }
  }
  if constexpr (KT >= kI8) {
    // V scales [token][KV head] of the block, nvalid tokens.
    const BufRsrc rs = make_rsrc(sbase, nvalid * a.num_kv_heads * 4);
#pragma unroll
    for (int tok = 0; tok < 2; ++tok)
      f.vs[tok] = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(
          rs, static_cast<uint32_t>(((grp + 8 * tok) * a.num_kv_heads + g) * 4), 0, 0));
  }
}

template <int KT, int D>
__device__ __forceinline__ void load_block(Frag<KT, D>& f, const PagedLaunch& a, int lane, int g,
                                           int blk, int nvalid) {
  using S = RowShape<KT, D>;
  const size_t tok_stride = static_cast<size_t>(a.num_kv_heads) * S::RW;
  const size_t blk0 = static_cast<size_t>(nvalid > 0 ? blk : 0) * kBlockTokens;
  const size_t base = blk0 * tok_stride;
  load_rows<KT, D>(f, static_cast<const uint32_t*>(a.k_cache) + base,
                   static_cast<const uint32_t*>(a.v_cache) + base, a, lane, g, nvalid,
                   KT >= kI8 ? a.v_scale + blk0 * a.num_kv_heads : nullptr);
}

// One block through the online softmax of HPW heads; tokens [nskip, nvalid)
// of the block count.
template <int KT, int D, int HPW>
__device__ __forceinline__ void softmax_block(const Frag<KT, D>& f,
                                              const uint32_t (&qv)[HPW][RowShape<KT, D>::QW],
                                              const float (&qb)[HPW], int lane, int nskip,
                                              int nvalid, float sl2, HeadState<HPW, D / 8>& st) {
  using S = RowShape<KT, D>;
  constexpr int W = S::W, DPL = S::DPL;
  const int grp = lane >> 3;
  float (&m)[HPW] = st.m;
  float (&l)[HPW] = st.l;
  float (&acc)[HPW][DPL] = st.acc;
  float s[2][HPW];
  // One-byte codes as fp16 pairs, once for all heads: K as pairs of
  // neighbouring dimensions, V as (token 0, token 1) pairs of one dimension.
  // INT8: biased numbers kI8Bias + code (byte permutes).  FP8: the exact
  // E4M3 values (v_cvt_pk_f32_fp8, then a pack that is exact since every
  // E4M3 value is an fp16 number).
  uint32_t kp[KT >= kI8 ? 2 : 1][KT >= kI8 ? 2 * W : 1];
  uint32_t vp[KT >= kI8 ? DPL : 1];
  if constexpr (KT == kF8) {
#pragma unroll
    for (int tok = 0; tok < 2; ++tok)
#pragma unroll
      for (int w = 0; w < W; ++w) {
        const auto lo = __builtin_amdgcn_cvt_pk_f32_fp8(f.k[tok][w], false);
        const auto hi = __builtin_amdgcn_cvt_pk_f32_fp8(f.k[tok][w], true);
        kp[tok][2 * w] = pack_f16x2_int(lo[0], lo[1]);
        kp[tok][2 * w + 1] = pack_f16x2_int(hi[0], hi[1]);
      }
#pragma unroll
    for (int w = 0; w < W; ++w)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        // bytes (token 0 code i, token 1 code i) as the low half-word
        const uint32_t sel = 0x0c0c0000u | static_cast<uint32_t>(4 + i) << 8 | static_cast<uint32_t>(i);
        const auto t = __builtin_amdgcn_cvt_pk_f32_fp8(
            __builtin_amdgcn_perm(f.v[1][w], f.v[0][w], sel), false);
        vp[4 * w + i] = pack_f16x2_int(t[0], t[1]);
      }
  }
  if constexpr (KT == kI8) {
#pragma unroll
    for (int tok = 0; tok < 2; ++tok)
#pragma unroll
      for (int w = 0; w < W; ++w) {
        const uint32_t u = f.k[tok][w] ^ kSignBits;
        kp[tok][2 * w] = biased_pair(u, 0);
        kp[tok][2 * w + 1] = biased_pair(u, 1);
      }
#pragma unroll
    for (int w = 0; w < W; ++w)
#pragma unroll
      for (int i = 0; i < 4; ++i) vp[4 * w + i] = biased_tokens(f.v[0][w], f.v[1][w], i);
  }
#pragma unroll
  for (int tok = 0; tok < 2; ++tok) {
    const bool ok = grp + 8 * tok >= nskip && grp + 8 * tok < nvalid;
#pragma unroll
    for (int h = 0; h < HPW; ++h) {
      float part = KT == kI8 ? qb[h] : 0.f;
      if constexpr (KT >= kI8) {
#pragma unroll
        for (int i = 0; i < 2 * W; ++i) part = dot2_f16(qv[h][i], kp[tok][i], part);
      }
#pragma unroll
      for (int w = 0; w < (KT >= kI8 ? 0 : W); ++w) {
        if constexpr (KT == kBF16) {
          part = dot2_bf16(qv[h][w], f.k[tok][w], part);
        } else {
          part = fmaf(__uint_as_float(qv[h][w]), __uint_as_float(f.k[tok][w]), part);
        }
      }
      const float z = sum_over_8(part) * sl2;
      s[tok][h] = ok ? z : -INFINITY;
    }
  }
  // Rows past the valid tokens were read as zeros: weight 0 times value 0.
  const uint32_t (&vw)[2][W] = f.v;
#pragma unroll
  for (int h = 0; h < HPW; ++h) {
    const float mx = fmaxf(s[0][h], s[1][h]);
    const bool up = mx > m[h] + kRaise;
    if (__builtin_amdgcn_ballot_w64(up)) {
      const float mn = up ? mx : m[h];
      const float alpha = exp2_fast(m[h] - mn);
      l[h] *= alpha;
      st.vb[h] *= alpha;
#pragma unroll
      for (int e = 0; e < DPL; ++e) acc[h][e] *= alpha;
      m[h] = mn;
    }
    const float p0 = exp2_fast(s[0][h] - m[h]);
    const float p1 = exp2_fast(s[1][h] - m[h]);
    if constexpr (KT >= kI8) {
      // One-byte codes: the weights times the tokens' V scales meet the
      // widened codes (p * (s * code) = (p * s) * code) as fp16 pairs; the
      // sum takes the plain weights, rounded the same way.
      l[h] = dot2_f16(pack_f16x2(p0, p1), kF16OnePair, l[h]);
      const uint32_t pp = pack_f16x2(p0 * f.vs[0], p1 * f.vs[1]);
      if constexpr (KT == kI8) st.vb[h] = dot2_f16(pp, kF16OnePair, st.vb[h]);
#pragma unroll
      for (int e = 0; e < DPL; ++e) acc[h][e] = dot2_f16(pp, vp[e], acc[h][e]);
    } else {
      // fp32 weights and products.  (bf16 weights, paired for dot2, halve
      // this work but their 8-bit rounding costs up to ~2e-3 absolute on
      // outputs that cancel to near zero over a few positions.)
      l[h] += p0 + p1;
#pragma unroll
      for (int w = 0; w < W; ++w) {
        if constexpr (KT == kBF16) {
          acc[h][2 * w] = fmaf(p1, bf16_lo(vw[1][w]), fmaf(p0, bf16_lo(vw[0][w]), acc[h][2 * w]));
          acc[h][2 * w + 1] =
              fmaf(p1, bf16_hi(vw[1][w]), fmaf(p0, bf16_hi(vw[0][w]), acc[h][2 * w + 1]));
        } else {
          acc[h][w] = fmaf(p1, __uint_as_float(vw[1][w]), fmaf(p0, __uint_as_float(vw[0][w]), acc[h][w]));
        }
      }
    }
  }
}

// Combination of x over the 8 lane groups (lanes differing in bits 3..5),
// on the VALU: a row rotation by 8 pairs lanes l and l ^ 8 inside each
// 16-lane row, the permlane swaps pair rows (l ^ 16) and halves (l ^ 32).
// Every lane ends with the same value, since each step combines a lane's
// value with its partner's in an order-independent way.
__device__ __forceinline__ float groups_max(float x) {
  x = fmaxf(x, dpp_move<0x128>(x));  // row_ror:8
  auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  x = fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
  r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float groups_sum(float x) {
  x = x + dpp_move<0x128>(x);
  auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  x = __uint_as_float(r[0]) + __uint_as_float(r[1]);
  r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// Merges the 8 lane groups: afterwards every group holds the (m, l, acc) of
// all the tokens the wave has seen.
template <int HPW, int DPL>
__device__ __forceinline__ void merge_groups(HeadState<HPW, DPL>& st) {
#pragma unroll
  for (int h = 0; h < HPW; ++h) {
    const float M = groups_max(st.m[h]);
    const float f = exp2_fast(st.m[h] - M);
    st.l[h] = groups_sum(st.l[h] * f);
#pragma unroll
    for (int e = 0; e < DPL; ++e) st.acc[h][e] = groups_sum(st.acc[h][e] * f);
    st.m[h] = M;
  }
}

// Streams blocks [j_begin, j_end) of sequence b through the online softmax of
// query heads h0 .. h0 + HPW - 1, which all read KV head g; tokens before
// t_start or at or past t_end carry no weight.  Block ids are read 64 at a
// time, one per lane, and
// broadcast with readlane.  On return the lane groups are merged.
// With `fused` (the range ends at the sequence's last position t_end - 1 and
// this step's K/V rows are given): that position is taken from k_new / v_new
// instead of the cache, as the last token of the softmax, and when
// `write_new` the wave also stores KV head g's part of the rows into their
// cache slot (the append of the same step).
template <int KT, int D, int HPW, int NBUF>
__device__ __forceinline__ void attend(const PagedLaunch& a, int lane, int b, int g, int h0,
                                       int j_begin, int j_end, int t_start, int t_end,
                                       HeadState<HPW, D / 8>& st, bool fused = false,
                                       bool write_new = false) {
  uint32_t qv[HPW][RowShape<KT, D>::QW];
  float qb[HPW];
  load_query<KT, D, HPW>(a, lane, b, h0, g, qv, qb);
  reset_state(st);
  const int t_last = t_end - 1;  // the appended position when fused
  if (fused) t_end = t_last;
  const float sl2 = a.scale * kLog2e;
  const int32_t* trow = a.block_table + static_cast<size_t>(b) * a.max_blocks_per_seq;
  Frag<KT, D> buf[NBUF];

  for (int c0 = j_begin; c0 < j_end; c0 += kMaxPartitionBlocks) {
    const int nblk = min(kMaxPartitionBlocks, j_end - c0);
    const int my_id = lane < nblk ? trow[c0 + lane] : -1;
    // Block id and valid tokens of block jj of this run of ids: 0 tokens
    // past the run's last block and for a table entry outside the pool.
    auto block_of = [&](int jj, int& nvalid) __attribute__((always_inline)) {
      const int blk = __builtin_amdgcn_readlane(my_id, jj & (kWave - 1));
      const bool ok = jj < nblk && blk >= 0 && blk < a.num_blocks;
      nvalid = ok ? min(kBlockTokens, t_end - (c0 + jj) * kBlockTokens) : 0;
      return blk;
    };
    // Refills are unconditional: a block past the end gets a zero-length
    // resource, so its loads touch no memory and keep the buffers in place.
#pragma unroll
    for (int s0 = 0; s0 < NBUF; ++s0) {
      int nv;
      const int blk = block_of(s0, nv);
      load_block<KT, D>(buf[s0], a, lane, g, blk, nv);
    }
    for (int base = 0; base < nblk; base += NBUF) {
#pragma unroll
      for (int s0 = 0; s0 < NBUF; ++s0) {
        const int jj = base + s0;
        if (jj < nblk) {
          int nv;
          block_of(jj, nv);
          softmax_block<KT, D, HPW>(buf[s0], qv, qb, lane,
                                    max(0, t_start - (c0 + jj) * kBlockTokens), nv, sl2, st);
        }
        int nv;
        const int blk = block_of(jj + NBUF, nv);
        load_block<KT, D>(buf[s0], a, lane, g, blk, nv);
      }
    }
    if constexpr (KT == kI8) unbias(st);
  }
  if (KT < kI8 && fused) {
    // The new rows, as token slot 0 of lane group 0 of a one-token block.
    // (One-byte caches have no fused append: their rows must be quantised.)
    using S = RowShape<KT, D>;
    const int blk = wave_uniform(trow[t_last / kBlockTokens]);
    if (blk >= 0 && blk < a.num_blocks) {
      const size_t row_words = static_cast<size_t>(a.num_kv_heads) * S::RW;
      const size_t src = static_cast<size_t>(b) * row_words;
      Frag<KT, D> f;
      load_rows<KT, D>(f, static_cast<const uint32_t*>(a.k_new) + src,
                         static_cast<const uint32_t*>(a.v_new) + src, a, lane, g, 1);
      softmax_block<KT, D, HPW>(f, qv, qb, lane, 0, 1, sl2, st);
      if (write_new && lane < 8) {
        const size_t dst = (static_cast<size_t>(blk) * kBlockTokens + t_last % kBlockTokens) * row_words +
                           g * S::RW;
        // The fused entry point receives writable caches.
        uint32_t* kd = static_cast<uint32_t*>(const_cast<void*>(a.k_cache)) + dst;
        uint32_t* vd = static_cast<uint32_t*>(const_cast<void*>(a.v_cache)) + dst;
#pragma unroll
        for (int c = 0; c < S::NCH; ++c) {
          store_words<S::CW>(kd + S::chunk_word(c, lane), &f.k[0][c * S::CW]);
          store_words<S::CW>(vd + S::chunk_word(c, lane), &f.v[0][c * S::CW]);
        }
      }
    }
  }
  merge_groups(st);
}

// After merge_groups every lane group holds all heads: lane group h (< HPW)
// takes head h.  The values are picked with selects (an indexed access into
// the state would put it in scratch memory).
template <int DPL>
struct GroupRow {
  float m, l, v[DPL];
};

template <int HPW, int DPL>
__device__ __forceinline__ GroupRow<DPL> pick_group(const HeadState<HPW, DPL>& st, int lane) {
  const int grp = lane >> 3;
  GroupRow<DPL> r;
  r.m = st.m[0];
  r.l = st.l[0];
#pragma unroll
  for (int e = 0; e < DPL; ++e) r.v[e] = st.acc[0][e];
#pragma unroll
  for (int h = 1; h < HPW; ++h) {
    const bool mine = grp == h;
    r.m = mine ? st.m[h] : r.m;
    r.l = mine ? st.l[h] : r.l;
#pragma unroll
    for (int e = 0; e < DPL; ++e) r.v[e] = mine ? st.acc[h][e] : r.v[e];
  }
  return r;
}

// Lane group h (< HPW) writes its row to workspace slot slot0 + h * stride
// (slot = (b * H_q + head) * P + piece); all stores sit under one branch.
template <int KT, int D, int HPW>
__device__ __forceinline__ void write_partial(const PagedLaunch& a, int lane, size_t slot0,
                                              size_t stride, const GroupRow<D / 8>& r) {
  using S = RowShape<KT, D>;
  const int grp = lane >> 3;
  const int sub = lane & 7;
  if (grp < HPW) {
    const size_t slot = slot0 + grp * stride;
    float* orow = a.ws_o + slot * D;
    // Chunk c of the lane is CW * EPW consecutive dimensions from
    // (8 c + sub) CW EPW: 16-byte stores.
    constexpr int RUN = S::CW * S::EPW;
    static_assert(RUN % 4 == 0, "vector stores");
#pragma unroll
    for (int c = 0; c < S::NCH; ++c)
#pragma unroll
      for (int v = 0; v < RUN / 4; ++v) {
        const float* x = &r.v[c * RUN + 4 * v];
        *reinterpret_cast<float4*>(orow + (c * 8 + sub) * RUN + 4 * v) = make_float4(x[0], x[1], x[2], x[3]);
      }
    if (sub == 0) *reinterpret_cast<float2*>(a.ws_ml + 2 * slot) = make_float2(r.m, r.l);
  }
}

// First position a decode row of length len sees: 0, or with a sliding
// window of W positions max(0, len - W) ("KV-Cache——为什么AI回复越来越快",
// Window Attention / Sliding Window: only the most recent W tokens count).
__device__ __forceinline__ int first_visible(const PagedLaunch& a, int len) {
  return a.window > 0 ? max(0, len - a.window) : 0;
}

// Blocks of a sequence of len positions (clamped to max_seq_len) that hold
// visible positions, from block first_visible / 16 on.
__device__ __forceinline__ int visible_blocks(const PagedLaunch& a, int len) {
  if (len <= 0) return 0;
  return (len + kBlockTokens - 1) / kBlockTokens - first_visible(a, len) / kBlockTokens;
}

// ---- Workers: one unit of work (sequence, K/V head, chunk of query heads)
// streamed over a range of blocks and written as one piece ---------------------

// VALU flavour: lane groups of 8, dot2 scores, fp32 FMA values (above).
template <int KT, int D, int HPW, int NBUF>
struct ValuWorker {
  static constexpr int kLdsPerWave = 0;
  static constexpr long long kEvenXcdShare = 1120;
  static constexpr bool kPace = false;
  static __device__ __forceinline__ int heads_per_wave(int /*ratio*/) { return HPW; }
  struct Pre {};  // (this flavour issues its first requests inside attend)
  static __device__ __forceinline__ void prefetch(const PagedLaunch&, int, int, int, int, int,
                                                  Pre&) {}
  static __device__ __forceinline__ void unit(const PagedLaunch& a, int lane, unsigned char* /*lds*/,
                                              int b, int g, int h0, int j_begin, int j_end,
                                              int t_start, int t_end, bool fused, bool write_new,
                                              size_t slot0, size_t P, const Pre&, int,
                                              int* = nullptr, const int* = nullptr) {
    HeadState<HPW, D / 8> st;
    attend<KT, D, HPW, NBUF>(a, lane, b, g, h0, j_begin, j_end, t_start, t_end, st, fused,
                             write_new);
    write_partial<KT, D, HPW>(a, lane, slot0, P, pick_group(st, lane));
  }
  static __device__ __forceinline__ void empty(const PagedLaunch& a, int lane, size_t slot0,
                                               size_t P) {
    HeadState<HPW, D / 8> st;
    reset_state(st);
    write_partial<KT, D, HPW>(a, lane, slot0, P, pick_group(st, lane));
  }
};

// MFMA flavour (bf16 and one-byte caches, groups of up to 16 query heads per
// wave).  For
// one 16-token block of K/V head g and the wave's query heads:
//   scores  S^T[token][head] = K_blk[16 x D] . Q^T[D x 16]: D/32 MFMA
//           16x16x32; K rows go straight from HBM into the A operand (lane
//           (G, i) = (lane / 16, lane % 16) holds token i, dimensions
//           32 s + 8 G .. + 7 of K-step s), the queries stay in registers as
//           the B operand (head i, same dimensions; heads past the group are
//           zero), and lane (G, i) ends with head i, tokens 4 G .. 4 G + 3.
//   softmax online per head with a lazily raised reference max, which is
//           uniform over the four lanes of a head (row_max4), so that every
//           weight of a head meets the same reference in the product below.
//   values  O^T[D x 16] += V_blk^T[D x 16] . P^T[16 x 16]: D/16 column tiles,
//           MFMA 16x16x16 with each weight as a bf16 value plus its bf16
//           remainder (two MFMAs, about 16 bits of weight; the running sum
//           takes the fp32 weights).  The weights are the B operand exactly
//           as the score MFMA left them (head i, tokens 4 G .. + 3); the V
//           operand (one dimension per lane, four tokens along K) is V_blk
//           transposed: the wave writes its block of V into its own LDS
//           slice (token rows, 16-byte chunks XOR-swizzled by row so that
//           the writes and the transpose reads are free of bank conflicts)
//           and reads it back with ds_read_b64_tr_b16.  Lane (G, i) ends
//           with head i and dimensions 16 t + 4 G .. + 3 of tile t, so a
//           rescale of head i touches only its own lane's registers.
// Per block and wave this is D/32 + D/8 MFMAs and ~50 VALU instructions
// for all heads of the group, against ~300 VALU instructions per 4 heads in
// the VALU flavour.
// One-byte caches (INT8, FP8 E4M3) use fp16 MFMAs: the codes are widened in
// registers to fp16 (INT8 as kI8Bias + code by byte permutes, its offsets
// removed from the scores and the accumulators; FP8 exactly), the queries
// carry the per-channel K scales and the weights the per-token V scales, and
// the weights enter once as fp16 (as in the VALU flavour), since the codes
// themselves are coarser than that.
template <int KT, int D>
struct MShape {
  static constexpr int EB = KT == kBF16 ? 2 : 1;  // bytes per stored element
  static constexpr int KS = D / 32;               // K-steps of the scores
  static constexpr int NL = D * EB / 64;          // 16-byte loads per row per lane (each of K, V)
  static constexpr int NT = D / 16;               // 16-dimension column tiles of the output
  static constexpr int C = D / 8;                 // 16-byte chunks per LDS row (16-bit values)
  static constexpr int ROWB = 2 * D;              // LDS bytes per row (bf16 or fp16 values)
  static constexpr int GROWB = D * EB;            // cache bytes per row of one K/V head
  static_assert(NL >= 1, "head_dim too small for this element kind");
  // Chunk position of chunk c of LDS row r (XOR swizzle).
  static __device__ __forceinline__ int pos(int r, int c) { return c ^ ((r * D / 128) % C); }
  // First dimension of the 8 that lane group G supplies in K-step s: bf16
  // rows give 8 consecutive dimensions per K-step; one-byte rows give 16
  // consecutive codes per load, i.e. two K-steps.
  static __device__ __forceinline__ int kdim(int s, int G) {
    return EB == 2 ? 32 * s + 8 * G : 64 * (s >> 1) + 16 * G + 8 * (s & 1);
  }
};

template <int KT, int D>
struct MFrag {
  uint32_t k[MShape<KT, D>::NL][4];
  uint32_t v[MShape<KT, D>::NL][4];
  float vs[1];  // one-byte caches: V scale of token 4 G + lane % 4
};

// Rows of K/V head g for the lane (G, i): token i of the block, its 16-byte
// loads p covering bytes 64 p + 16 G .. + 15 of the head's row; rows at or
// past nvalid read as zeros.  One-byte caches also fetch the V scale of
// token 4 G + i % 4 (sbase: the block's [16][H_kv] scales).
template <int KT, int D>
__device__ __forceinline__ void mfma_rows(MFrag<KT, D>& f, const void* kbase, const void* vbase,
                                          const PagedLaunch& a, int lane, int g, int nvalid,
                                          const float* sbase = nullptr) {
  using S = MShape<KT, D>;
  const int tok_bytes = a.num_kv_heads * S::GROWB;
  const int bytes = nvalid * tok_bytes;
  const BufRsrc rk = make_rsrc(kbase, bytes);
  const BufRsrc rv = make_rsrc(vbase, bytes);
  const int G = lane >> 4;
  const uint32_t off = static_cast<uint32_t>((lane & 15) * tok_bytes + g * S::GROWB + 16 * G);
#pragma unroll
  for (int p = 0; p < S::NL; ++p) {
    buffer_load_words<4>(f.k[p], rk, off + 64 * p);
    buffer_load_words<4>(f.v[p], rv, off + 64 * p);
  }
  if constexpr (KT != kBF16) {
    // One load: lane (G, i) fetches the scale of token 4 G + i % 4; the
    // quad broadcasts in mfma_block hand each lane all four.
    const BufRsrc rs = make_rsrc(sbase, nvalid * a.num_kv_heads * 4);
    f.vs[0] = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(
        rs, static_cast<uint32_t>(((4 * G + (lane & 3)) * a.num_kv_heads + g) * 4), 0, 0));
  }
}

template <int KT, int D>
__device__ __forceinline__ void mfma_block_rows(MFrag<KT, D>& f, const PagedLaunch& a, int lane,
                                                int g, int blk, int nvalid) {
  using S = MShape<KT, D>;
  const size_t row0 = static_cast<size_t>(nvalid > 0 ? blk : 0) * kBlockTokens;
  const size_t bytes = row0 * a.num_kv_heads * S::GROWB;
  mfma_rows<KT, D>(f, static_cast<const unsigned char*>(a.k_cache) + bytes,
                   static_cast<const unsigned char*>(a.v_cache) + bytes, a, lane, g, nvalid,
                   KT == kBF16 ? nullptr : a.v_scale + row0 * a.num_kv_heads);
}

template <int D>
struct MState {
  f32x4_t acc[D / 16];  // O^T: head lane % 16, dims 16 t + 4 (lane / 16) + j
  float m;              // reference max of the lane's head (log2 units)
  float l;              // the lane's share of the weight sum
  float vb;             // INT8: the lane's share of the weights that met biased codes
};

typedef __attribute__((ext_vector_type(8))) _Float16 f16x8_t;
typedef __attribute__((ext_vector_type(4))) _Float16 f16x4_t;

// Sixteen one-byte codes (four words) as eight fp16 pairs of neighbouring
// codes: INT8 as biased numbers kI8Bias + code (byte permutes), FP8 as the
// exact E4M3 values.
template <int KT>
__device__ __forceinline__ void widen16(const uint32_t (&w)[4], uint32_t (&o)[8]) {
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    if constexpr (KT == kI8) {
      const uint32_t u = w[k] ^ kSignBits;
      o[2 * k] = biased_pair(u, 0);
      o[2 * k + 1] = biased_pair(u, 1);
    } else {
      const auto lo = __builtin_amdgcn_cvt_pk_f32_fp8(w[k], false);
      const auto hi = __builtin_amdgcn_cvt_pk_f32_fp8(w[k], true);
      o[2 * k] = pack_f16x2_int(lo[0], lo[1]);
      o[2 * k + 1] = pack_f16x2_int(hi[0], hi[1]);
    }
  }
}

// One block through the online softmax: tokens [nskip, nvalid) count.  `lds`
// is the wave's LDS slice (16 rows of one K/V head as 16-bit values).
// q: the B operand of the scores (bf16, or fp16 scaled queries); qb: INT8's
// score offset of the lane's head.
template <int KT, int D>
__device__ __forceinline__ void mfma_block(const MFrag<KT, D>& f, const uint32_t (&q)[D / 32][4],
                                           float qb, unsigned char* lds, int lane, int nskip,
                                           int nvalid, float sl2, MState<D>& st) {
  using S = MShape<KT, D>;
  const int G = lane >> 4, i = lane & 15;
  f32x4_t sc = {0.f, 0.f, 0.f, 0.f};
  if constexpr (KT == kBF16) {
#pragma unroll
    for (int s = 0; s < S::KS; ++s)
      sc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
          as_bf16x8(f.k[s][0], f.k[s][1], f.k[s][2], f.k[s][3]),
          as_bf16x8(q[s][0], q[s][1], q[s][2], q[s][3]), sc, 0, 0, 0);
    // V rows into the LDS slice: row i, chunk 4 s + G.
#pragma unroll
    for (int s = 0; s < S::KS; ++s)
      *reinterpret_cast<uint4*>(lds + i * S::ROWB + S::pos(i, 4 * s + G) * 16) =
          make_uint4(f.v[s][0], f.v[s][1], f.v[s][2], f.v[s][3]);
  } else {
#pragma unroll
    for (int p = 0; p < S::NL; ++p) {
      uint32_t kw[8], vw[8];
      widen16<KT>(f.k[p], kw);
      widen16<KT>(f.v[p], vw);
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const int s = 2 * p + h;
        const uint4 ka = make_uint4(kw[4 * h], kw[4 * h + 1], kw[4 * h + 2], kw[4 * h + 3]);
        const uint4 qa = make_uint4(q[s][0], q[s][1], q[s][2], q[s][3]);
        sc = __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8_t, ka),
                                                    __builtin_bit_cast(f16x8_t, qa), sc, 0, 0, 0);
        // fp16 V values: row i, chunk 8 p + 2 G + h.
        *reinterpret_cast<uint4*>(lds + i * S::ROWB + S::pos(i, 8 * p + 2 * G + h) * 16) =
            make_uint4(vw[4 * h], vw[4 * h + 1], vw[4 * h + 2], vw[4 * h + 3]);
      }
    }
  }
  float z[4];
  float mx = -INFINITY;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int t = 4 * G + j;
    z[j] = (t >= nskip && t < nvalid) ? (sc[j] + qb) * sl2 : -INFINITY;
    mx = fmaxf(mx, z[j]);
  }
  mx = row_max4(mx);
  const bool up = mx > st.m + kRaise;
  if (__builtin_amdgcn_ballot_w64(up)) {
    const float mn = up ? mx : st.m;
    const float alpha = exp2_fast(st.m - mn);
    st.l *= alpha;
    if constexpr (KT == kI8) st.vb *= alpha;
#pragma unroll
    for (int t = 0; t < S::NT; ++t)
#pragma unroll
      for (int j = 0; j < 4; ++j) st.acc[t][j] *= alpha;
    st.m = mn;
  }
  float p[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) p[j] = exp2_fast(z[j] - st.m);
  st.l += (p[0] + p[1]) + (p[2] + p[3]);
  // Transpose reads: lane (G, i) addresses row 4 G + i / 4, dimensions
  // 16 t + 4 (i % 4) .. + 3, and receives dimension 16 t + i of rows
  // 4 G .. 4 G + 3.
  const int rr = 4 * G + (i >> 2);
  unsigned char* rbase = lds + rr * S::ROWB + 8 * (i & 1);
  if constexpr (KT == kBF16) {
    const uint32_t h0 = pack_bf16x2(p[0], p[1]), h1 = pack_bf16x2(p[2], p[3]);
    const uint32_t r0 = pack_bf16x2(p[0] - bf16_lo(h0), p[1] - bf16_hi(h0));
    const uint32_t r1 = pack_bf16x2(p[2] - bf16_lo(h1), p[3] - bf16_hi(h1));
    const s16x4_t ph = __builtin_bit_cast(s16x4_t, make_uint2(h0, h1));
    const s16x4_t pr = __builtin_bit_cast(s16x4_t, make_uint2(r0, r1));
#pragma unroll
    for (int t = 0; t < S::NT; ++t) {
      const int c = 2 * t + ((i & 3) >> 1);
      const s16x4_t vt = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
          (lds_s16x4_t*)(rbase + S::pos(rr, c) * 16));
      st.acc[t] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(vt, ph, st.acc[t], 0, 0, 0);
      st.acc[t] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(vt, pr, st.acc[t], 0, 0, 0);
    }
  } else {
    // One-byte caches: the weights times the tokens' V scales meet the
    // widened codes (p * (s * code) = (p * s) * code) as fp16.
    // quad_perm broadcasts: every lane of a quad takes lane j's scale
    const float s0 = dpp_move<0x00>(f.vs[0]), s1 = dpp_move<0x55>(f.vs[0]);
    const float s2 = dpp_move<0xAA>(f.vs[0]), s3 = dpp_move<0xFF>(f.vs[0]);
    const uint32_t w0 = pack_f16x2(p[0] * s0, p[1] * s1);
    const uint32_t w1 = pack_f16x2(p[2] * s2, p[3] * s3);
    if constexpr (KT == kI8) st.vb = dot2_f16(w1, kF16OnePair, dot2_f16(w0, kF16OnePair, st.vb));
    const f16x4_t pw = __builtin_bit_cast(f16x4_t, make_uint2(w0, w1));
#pragma unroll
    for (int t = 0; t < S::NT; ++t) {
      const int c = 2 * t + ((i & 3) >> 1);
      const s16x4_t vt = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
          (lds_s16x4_t*)(rbase + S::pos(rr, c) * 16));
      st.acc[t] = __builtin_amdgcn_mfma_f32_16x16x16f16(__builtin_bit_cast(f16x4_t, vt), pw,
                                                        st.acc[t], 0, 0, 0);
    }
  }
}

// INT8: takes the value bias out of the accumulators (the weights of all 16
// tokens of a block meet every output column, so the bias of a column is
// kI8Bias times the head's whole weight sum, gathered over the four lanes).
template <int D>
__device__ __forceinline__ void mfma_unbias(MState<D>& st) {
  const float vb = row_sum4(st.vb);
#pragma unroll
  for (int t = 0; t < D / 16; ++t)
#pragma unroll
    for (int j = 0; j < 4; ++j) st.acc[t][j] = fmaf(-kI8Bias, vb, st.acc[t][j]);
  st.vb = 0.f;
}

template <int KT, int D, int NBUF>
struct MfmaWorker {
  using S = MShape<KT, D>;
  static constexpr int kLdsPerWave = 16 * S::ROWB;
  static constexpr long long kEvenXcdShare = 1060;
  // The two waves on one SIMD keep pace (see unit): by default the older
  // one takes the issue slots and finishes its share long before the other,
  // which then streams alone for the rest of the launch; with one-byte
  // caches, whose blocks are half the bytes, that half of the launch ran
  // short of loads in flight (the GQA batch over INT8 codes: 124.4 -> 119.6
  // us with pacing, HIP events; bf16 blocks: 217 -> 219 us, so not there).
  static constexpr bool kPace = KT != kBF16;
  static __device__ __forceinline__ int heads_per_wave(int ratio) { return ratio < 16 ? ratio : 16; }

  static __device__ __forceinline__ void write(const PagedLaunch& a, int lane, size_t slot0,
                                               size_t P, int nheads, const MState<D>& st) {
    const int G = lane >> 4, i = lane & 15;
    const float lsum = row_sum4(st.l);
    if (i < nheads) {
      const size_t slot = slot0 + i * P;
      float* orow = a.ws_o + slot * D + 4 * G;
#pragma unroll
      for (int t = 0; t < S::NT; ++t)
        *reinterpret_cast<float4*>(orow + 16 * t) =
            make_float4(st.acc[t][0], st.acc[t][1], st.acc[t][2], st.acc[t][3]);
      if (G == 0) *reinterpret_cast<float2*>(a.ws_ml + 2 * slot) = make_float2(st.m, lsum);
    }
  }

  static __device__ __forceinline__ void reset(MState<D>& st) {
#pragma unroll
    for (int t = 0; t < S::NT; ++t) st.acc[t] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    st.m = kMinusBig;
    st.l = 0.f;
    st.vb = 0.f;
  }

  static __device__ __forceinline__ void empty(const PagedLaunch& a, int lane, size_t slot0,
                                               size_t P) {
    MState<D> st;
    reset(st);
    const int ratio = a.num_q_heads / a.num_kv_heads;
    write(a, lane, slot0, P, heads_per_wave(ratio), st);
  }

  // The first requests of a unit, issued before anything waits on memory, so
  // that they share one round trip (and, in the kernels, the one that reads
  // the sequence length): the block ids of blocks j_pre .. j_pre + 63 of
  // sequence b (one per lane; lanes past the table row read 0) and the query
  // rows of heads h0 .. h0 + nheads - 1 in the B operand's layout (head
  // lane % 16, zeros past the wave's heads), with the K/V head's per-channel
  // K scales for one-byte caches.  The ids are requested first: waiting for
  // them does not wait for the queries.
  // Block id of block j + lane of sequence b's table row (0 past the row).
  static __device__ __forceinline__ int table_ids(const PagedLaunch& a, int b, int j, int lane) {
    const int32_t* trow = a.block_table + static_cast<size_t>(b) * a.max_blocks_per_seq;
    const int left = wave_uniform(min(max(0, a.max_blocks_per_seq - j), kWave));
    const BufRsrc rt = make_rsrc(trow + min(j, a.max_blocks_per_seq), left * 4);
    return static_cast<int>(__builtin_amdgcn_raw_buffer_load_b32(rt, 4 * lane, 0, 0));
  }
  struct Pre {
    int ids;                  // block id of block j_pre + lane
    uint32_t qw[S::KS][4];    // query words (bf16)
    float4 ks[S::KS][2];      // one-byte caches: K scales of those dimensions
  };
  static __device__ __forceinline__ void prefetch(const PagedLaunch& a, int lane, int b, int g,
                                                  int h0, int j_pre, Pre& pr) {
    const int ratio = a.num_q_heads / a.num_kv_heads;
    const int nheads = heads_per_wave(ratio);
    const int G = lane >> 4, i = lane & 15;
    pr.ids = table_ids(a, b, j_pre, lane);
    const BufRsrc rq = make_rsrc(static_cast<const uint16_t*>(a.q) +
                                     (static_cast<size_t>(b) * a.num_q_heads + h0) * D,
                                 nheads * D * 2);
#pragma unroll
    for (int s = 0; s < S::KS; ++s)
      buffer_load_words<4>(pr.qw[s], rq, static_cast<uint32_t>((i * D + S::kdim(s, G)) * 2));
    if constexpr (KT != kBF16) {
#pragma unroll
      for (int s = 0; s < S::KS; ++s) {
        const float* ks = a.k_scale + static_cast<size_t>(g) * D + S::kdim(s, G);
        pr.ks[s][0] = *reinterpret_cast<const float4*>(ks);
        pr.ks[s][1] = *reinterpret_cast<const float4*>(ks + 4);
      }
    }
  }

  // The prefetched queries as the B operand.  bf16 caches: the bf16 queries.
  // One-byte caches: q times K/V head g's per-channel K scales, rounded to
  // fp16 (q . (s * code) = (q * s) . code); INT8 also returns the score offset
  // -kI8Bias * (sum of the head's scaled query), from the same fp16 values.
  // The empty asm statements pin the arithmetic here: hoisted above the
  // first block loads, it would make them wait for the queries.
  static __device__ __forceinline__ float make_q(Pre pr, uint32_t (&q)[D / 32][4]) {
    float qs = 0.f;
#pragma unroll
    for (int s = 0; s < S::KS; ++s) {
#pragma unroll
      for (int k = 0; k < 4; ++k) asm volatile("" : "+v"(pr.qw[s][k]));
      if constexpr (KT != kBF16) {
#pragma unroll
        for (int h = 0; h < 2; ++h)
          asm volatile("" : "+v"(pr.ks[s][h].x), "+v"(pr.ks[s][h].y), "+v"(pr.ks[s][h].z),
                       "+v"(pr.ks[s][h].w));
      }
      if constexpr (KT == kBF16) {
#pragma unroll
        for (int k = 0; k < 4; ++k) q[s][k] = pr.qw[s][k];
      } else {
        const uint32_t* w = pr.qw[s];
        const float4 s0 = pr.ks[s][0], s1 = pr.ks[s][1];
        q[s][0] = pack_f16x2(bf16_lo(w[0]) * s0.x, bf16_hi(w[0]) * s0.y);
        q[s][1] = pack_f16x2(bf16_lo(w[1]) * s0.z, bf16_hi(w[1]) * s0.w);
        q[s][2] = pack_f16x2(bf16_lo(w[2]) * s1.x, bf16_hi(w[2]) * s1.y);
        q[s][3] = pack_f16x2(bf16_lo(w[3]) * s1.z, bf16_hi(w[3]) * s1.w);
#pragma unroll
        for (int k = 0; k < 4; ++k) qs = dot2_f16(q[s][k], kF16OnePair, qs);
      }
    }
    return KT == kI8 ? -kI8Bias * row_sum4(qs) : 0.f;
  }

  // Blocks [j_begin, j_end) of sequence b, K/V head g, query heads h0 ..;
  // tokens before t_start or at or past t_end carry no weight.  With
  // `fused` (bf16 caches) the range ends at position t_end - 1, which is
  // taken from k_new / v_new as a one-token block after the others, and with
  // `write_new` the wave also stores head g's part of those rows into their
  // cache slot.  `pr` holds this unit's prefetch for blocks j_pre .. +63.
  // With `pace` (this wave's count of blocks done, in LDS) and `sibling`
  // (that of the other wave on its SIMD), a wave more than one block ahead
  // of its sibling lowers its issue priority until the sibling catches up.
  static __device__ __forceinline__ void unit(const PagedLaunch& a, int lane, unsigned char* lds,
                                              int b, int g, int h0, int j_begin, int j_end,
                                              int t_start, int t_end, bool fused, bool write_new,
                                              size_t slot0, size_t P, const Pre& pr, int j_pre,
                                              int* pace = nullptr, const int* sibling = nullptr) {
    const int ratio = a.num_q_heads / a.num_kv_heads;
    const int nheads = heads_per_wave(ratio);
    const int G = lane >> 4, i = lane & 15;
    uint32_t q[S::KS][4];
    float qb = 0.f;
    MState<D> st;
    reset(st);
    const int t_last = t_end - 1;
    if (fused) t_end = t_last;
    const float sl2 = a.scale * kLog2e;
    const int32_t* trow = a.block_table + static_cast<size_t>(b) * a.max_blocks_per_seq;
    MFrag<KT, D> buf[NBUF];
    if (j_begin >= j_end) qb = make_q(pr, q);  // (no cached block: the fused row only)

    // The first chunk's ids are the prefetched ones (callers start the
    // prefetch at or before j_begin and no more than 64 blocks before the
    // chunk's end); each chunk requests the next one's ids (lane k: block
    // c0 + 64 + k) before it waits on anything, with no branch, so that no
    // wait has to cover a load that only some paths issue.
    int my_id = pr.ids, off = j_begin - j_pre;
    for (int c0 = j_begin; c0 < j_end; c0 += kMaxPartitionBlocks) {
      const int nblk = min(kMaxPartitionBlocks, j_end - c0);
      const int next_id = table_ids(a, b, c0 + kMaxPartitionBlocks, lane);
      auto block_of = [&](int jj, int& nvalid) __attribute__((always_inline)) {
        const int blk = __builtin_amdgcn_readlane(my_id, (off + jj) & (kWave - 1));
        const bool ok = jj < nblk && blk >= 0 && blk < a.num_blocks;
        nvalid = ok ? min(kBlockTokens, t_end - (c0 + jj) * kBlockTokens) : 0;
        return blk;
      };
      // (In buffer order: the scheduler would otherwise be free to issue the
      // first block's loads last, and the first wait would cover them all.)
#pragma unroll
      for (int s0 = 0; s0 < NBUF; ++s0) {
        int nv;
        const int blk = block_of(s0, nv);
        mfma_block_rows<KT, D>(buf[s0], a, lane, g, blk, nv);
        __builtin_amdgcn_sched_barrier(0);
      }
      // The queries are formed after the first block loads are on their way.
      if (c0 == j_begin) qb = make_q(pr, q);
      for (int base = 0; base < nblk; base += NBUF) {
#pragma unroll
        for (int s0 = 0; s0 < NBUF; ++s0) {
          const int jj = base + s0;
          if (jj < nblk) {
            int nv;
            block_of(jj, nv);
            mfma_block<KT, D>(buf[s0], q, qb, lds, lane,
                              max(0, t_start - (c0 + jj) * kBlockTokens), nv, sl2, st);
            if (pace) {
              const int done = *pace + 1;
              *pace = done;
              if (done > *sibling + 1)
                __builtin_amdgcn_s_setprio(0);
              else
                __builtin_amdgcn_s_setprio(2);
            }
          }
          int nv;
          const int blk = block_of(jj + NBUF, nv);
          mfma_block_rows<KT, D>(buf[s0], a, lane, g, blk, nv);
        }
      }
      if constexpr (KT == kI8) mfma_unbias(st);
      my_id = next_id;
      off = 0;
    }
    if constexpr (KT == kBF16) {
      if (fused) {
        const int blk = wave_uniform(trow[t_last / kBlockTokens]);
        if (blk >= 0 && blk < a.num_blocks) {
          const size_t row_words = static_cast<size_t>(a.num_kv_heads) * (D / 2);
          const size_t src = static_cast<size_t>(b) * row_words;
          MFrag<KT, D> f;
          mfma_rows<KT, D>(f, static_cast<const uint32_t*>(a.k_new) + src,
                           static_cast<const uint32_t*>(a.v_new) + src, a, lane, g, 1);
          mfma_block<KT, D>(f, q, qb, lds, lane, 0, 1, sl2, st);
          if (write_new && i == 0) {
            // Lanes (G, 0) hold dimensions 32 s + 8 G .. + 7 of the new rows.
            const size_t dst = (static_cast<size_t>(blk) * kBlockTokens + t_last % kBlockTokens) *
                                   row_words + g * (D / 2);
            uint32_t* kd = static_cast<uint32_t*>(const_cast<void*>(a.k_cache)) + dst;
            uint32_t* vd = static_cast<uint32_t*>(const_cast<void*>(a.v_cache)) + dst;
#pragma unroll
            for (int s = 0; s < S::KS; ++s) {
              store_words<4>(kd + (32 * s + 8 * G) / 2, f.k[s]);
              store_words<4>(vd + (32 * s + 8 * G) / 2, f.v[s]);
            }
          }
        }
      }
    }
    write(a, lane, slot0, P, nheads, st);
  }
};

// NBUF: register buffers per wave (NBUF - 1 blocks in flight during compute).
// WPE: waves per SIMD the register allocation is sized for.
//
// Fixed partitions: one wavefront per unit (b, partition, kv head g, chunk of
// HPW query heads).  WG: wavefronts per workgroup.  Consecutive units are the
// KV heads (and head chunks) of one (sequence, partition), so a workgroup's
// waves read the same blocks together: for 8 KV heads an 8-wave workgroup
// reads whole contiguous token rows of every block.
template <class W, int WPE, int WG>
__global__ __launch_bounds__(64 * WG) __attribute__((amdgpu_waves_per_eu(WPE, WPE)))
void paged_partials_kernel(PagedLaunch a) {
  __shared__ __attribute__((aligned(16))) unsigned char wave_lds[WG * W::kLdsPerWave + 16];
  const int lane = threadIdx.x & (kWave - 1);
  unsigned char* lds = wave_lds + wave_uniform(threadIdx.x >> 6) * W::kLdsPerWave;
  const int ratio = a.num_q_heads / a.num_kv_heads;
  const int hpw = W::heads_per_wave(ratio);
  const int hchunks = ratio / hpw;

  int u = wave_uniform(blockIdx.x * WG + (threadIdx.x >> 6));
  const int units = a.batch * a.num_partitions * a.num_kv_heads * hchunks;
  if (u >= units) return;
  const int hc = u % hchunks;
  u /= hchunks;
  const int g = u % a.num_kv_heads;
  u /= a.num_kv_heads;
  const int p = u % a.num_partitions;
  const int b = u / a.num_partitions;

  // The sequence length, the partition's block ids and the queries are
  // requested together (the length first), before anything waits.
  int len = a.seq_lens[b];
  const int p_begin = p * a.partition_tokens;
  const int h0 = g * ratio + hc * hpw;
  const int j_pre = p_begin / kBlockTokens;
  typename W::Pre pr;
  W::prefetch(a, lane, b, g, h0, j_pre, pr);
  // (Keeps the requests above the early exit below: sunk past it, they
  // would wait for the length.)
  asm volatile("" ::: "memory");
  len = min(len, a.max_seq_len);
  if (len <= p_begin) return;
  const int t_end = min(len, p_begin + a.partition_tokens);
  const int t_begin = max(p_begin, first_visible(a, len));
  const size_t P = a.num_partitions;
  const size_t slot0 = (static_cast<size_t>(b) * a.num_q_heads + h0) * P + p;
  if (t_begin >= t_end) {
    // Before a sliding window: an empty piece (l = 0), which the merge skips.
    W::empty(a, lane, slot0, P);
    return;
  }
  const int j0 = t_begin / kBlockTokens;
  const int nblk = (t_end + kBlockTokens - 1) / kBlockTokens - j0;

  const bool fused = a.k_new != nullptr && t_end == len;
  W::unit(a, lane, lds, b, g, h0, j0, j0 + nblk, t_begin, t_end, fused, hc == 0, slot0, P, pr,
          j_pre);
}

// Balanced split (automatic mode).  The work list is every (sequence b,
// unit group ug, block j) in that order, a unit group being WG consecutive
// units (KV head, head chunk); wave w of a workgroup does unit ug * WG + w, so
// the workgroup's waves read the same block rows together.  As many
// workgroups as are resident at once each take one contiguous share of the
// list, [bound(k), bound(k + 1)), whatever the length mix: shares are
// proportional to kEvenXcdShare / kOddXcdShare by the parity of the
// workgroup's XCD, so that all finish together; when the list is short
// (fewer than kMinPieceBlocks + 1 items per workgroup) the shares are equal,
// kMinPieceBlocks long, and the last workgroups have none.  Every share is
// at least kMinPieceBlocks items but the last.  The waves walk their share as
// segments of one (b, ug) each; at a segment's end each wave writes the
// partial result of its unit's heads as piece (k - the workgroup holding the
// segment's first item), and the workgroup of piece 0 records the number of
// pieces for the merge.  Pieces of one (b, h) never exceed ceil(blocks /
// kMinPieceBlocks) + 1.
template <class W, int WPE, int WG>
__global__ __launch_bounds__(64 * WG) __attribute__((amdgpu_waves_per_eu(WPE, WPE)))
void paged_balanced_kernel(PagedLaunch a) {
  __shared__ __attribute__((aligned(16))) unsigned char wave_lds[WG * W::kLdsPerWave + 16];
  // [batch + 1] blocks of the sequences before b, [batch + 1] count of the
  // non-empty sequences before b, then [batch] lengths clamped to
  // max_seq_len.
  extern __shared__ int blk_prefix[];
  // Blocks done by each wave (pacing of the two waves on a SIMD, wave w and
  // w ^ 4 of an eight-wave workgroup).
  __shared__ int pace[WG];
  if ((threadIdx.x & (kWave - 1)) == 0) pace[threadIdx.x >> 6] = 0;
  int* const seq_prefix = blk_prefix + a.batch + 1;
  int* const len_of = seq_prefix + a.batch + 1;
  const int lane = threadIdx.x & (kWave - 1);
  const int wave = wave_uniform(threadIdx.x >> 6);
  unsigned char* lds = wave_lds + wave * W::kLdsPerWave;
  const int ratio = a.num_q_heads / a.num_kv_heads;
  const int hpw = W::heads_per_wave(ratio);
  const int hchunks = ratio / hpw;
  const int units = a.num_kv_heads * hchunks;
  const int n_ug = (units + WG - 1) / WG;

  if (wave == 0) {
    int run = 0, run_seq = 0;
    for (int c = 0; c < a.batch; c += kWave) {
      const int len = c + lane < a.batch ? min(a.seq_lens[c + lane], a.max_seq_len) : 0;
      int x = visible_blocks(a, len);
      int y = x > 0 ? 1 : 0;
      if (c + lane < a.batch) len_of[c + lane] = len;
#pragma unroll
      for (int sh = 1; sh < kWave; sh <<= 1) {
        const int xs = __shfl_up(x, sh, kWave);
        const int ys = __shfl_up(y, sh, kWave);
        if (lane >= sh) {
          x += xs;
          y += ys;
        }
      }
      if (c + lane < a.batch) {
        blk_prefix[c + lane + 1] = run + x;
        seq_prefix[c + lane + 1] = run_seq + y;
      }
      run += __shfl(x, kWave - 1, kWave);
      run_seq += __shfl(y, kWave - 1, kWave);
    }
    if (lane == 0) {
      blk_prefix[0] = 0;
      seq_prefix[0] = 0;
    }
  }
  __syncthreads();

  // Prefix reads are wave-uniform; readfirstlane tells the compiler, which
  // would otherwise keep the segment state in VGPRs under masked branches.
  auto prefix = [&](int i) __attribute__((always_inline)) { return wave_uniform(blk_prefix[i]); };
  // Shares are cut in a virtual list where every segment (b, ug) is preceded
  // by kSegmentCost items of no work: a share that starts a new segment pays
  // for the restart of its load pipeline with fewer blocks.
  auto vprefix = [&](int i) __attribute__((always_inline)) {
    return n_ug * (prefix(i) + kSegmentCost * wave_uniform(seq_prefix[i]));
  };
  const int total = n_ug * prefix(a.batch);
  const int vtotal = vprefix(a.batch);
  const int groups = gridDim.x;
  const int wg = blockIdx.x;
  const bool weighted = vtotal >= groups * 2 * kMinPieceBlocks;
  const int per = max(kMinPieceBlocks, (vtotal + groups - 1) / groups);  // equal shares
  // Weight of the first k workgroups (even ones: indices 0, 2, 4, ...).
  auto weight = [&](int k) __attribute__((always_inline)) {
    return W::kEvenXcdShare * ((k + 1) / 2) + kOddXcdShare * (k / 2);
  };
  const long long wsum = weight(groups);
  auto bound = [&](int k) __attribute__((always_inline)) {
    return weighted ? static_cast<int>(static_cast<long long>(vtotal) * weight(k) / wsum)
                    : min(vtotal, k * per);
  };
  // Workgroup whose share holds virtual position v.
  auto owner = [&](int v) __attribute__((always_inline)) {
    if (!weighted) return v / per;
    int k = static_cast<int>(static_cast<long long>(v) * groups / vtotal);
    while (k + 1 < groups && bound(k + 1) <= v) ++k;
    while (k > 0 && bound(k) > v) --k;
    return k;
  };
  // Virtual position of block j of segment (b, ug), nb blocks per segment.
  auto vpos = [&](int b_, int ug, int nb, int j) __attribute__((always_inline)) {
    return vprefix(b_) + ug * (nb + kSegmentCost) + kSegmentCost + j;
  };
  // The first real item at or after virtual position v, and its sequence (the
  // last b whose virtual items start at or before v, never an empty one).
  auto to_real = [&](int v, int& b_out) __attribute__((always_inline)) {
    if (v >= vtotal) {
      b_out = a.batch;
      return total;
    }
    int lo = 0, hi = a.batch - 1;
    while (lo < hi) {
      const int mid = (lo + hi + 1) >> 1;
      if (vprefix(mid) <= v) lo = mid; else hi = mid - 1;
    }
    const int nb = prefix(lo + 1) - prefix(lo);
    const int off = v - vprefix(lo);
    const int ug = off / (nb + kSegmentCost);
    const int j = max(0, off - ug * (nb + kSegmentCost) - kSegmentCost);
    b_out = lo;
    return n_ug * prefix(lo) + ug * nb + j;
  };
  int b, b_end;
  int item = to_real(bound(wg), b);
  const int end = to_real(bound(wg + 1), b_end);
  if (item >= end) return;  // whole workgroup

  const size_t P = a.num_partitions;
  while (item < end) {
    const int pb = prefix(b);
    const int nb = prefix(b + 1) - pb;
    const int base = n_ug * pb;
    const int ug = (item - base) / nb;
    const int j0 = item - base - ug * nb;
    const int seg_begin = base + ug * nb;
    const int seg_end = min(end, seg_begin + nb);
    const int u = ug * WG + wave;
    if (u < units) {
      const int g = u / hchunks, hc = u % hchunks;
      const int h0 = g * ratio + hc * hpw;
      const int t_end = wave_uniform(len_of[b]);
      const int t_start = first_visible(a, t_end);
      const int js = t_start / kBlockTokens;  // the sequence's first visible block
      // The block ids from the segment's first block and the queries are
      // requested together, before anything waits on memory.
      typename W::Pre pr;
      W::prefetch(a, lane, b, g, h0, js + j0, pr);
      const bool fused = a.k_new != nullptr && seg_end == seg_begin + nb;
      const int first = owner(vpos(b, ug, nb, 0));
      const int piece = wg - first;
      const size_t row0 = static_cast<size_t>(b) * a.num_q_heads + h0;
      constexpr bool kPaced = W::kPace && WG == 8;
      W::unit(a, lane, lds, b, g, h0, js + j0, js + j0 + (seg_end - item), t_start, t_end, fused,
              hc == 0, row0 * P + piece, P, pr, js + j0, kPaced ? &pace[wave] : nullptr,
              kPaced ? &pace[wave ^ 4] : nullptr);
      if (piece == 0 && lane < hpw)
        a.counts[row0 + lane] = owner(vpos(b, ug, nb, nb - 1)) - first + 1;
    }
    item = seg_end;
    if (item == base + n_ug * nb) {
      ++b;
      while (b < a.batch && prefix(b + 1) == prefix(b)) ++b;
    }
  }
}

// Compute units of the current device (cached per device).
int device_cus() {
  static int cus[64];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
  if (cus[dev] == 0) {
    int n = 0;
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n < 1)
      n = 256;
    cus[dev] = n;
  }
  return cus[dev];
}

template <class W, int WPE, int WG>
hipError_t launch_variant(const PagedLaunch& a, int hpw, hipStream_t stream) {
  const int ratio = a.num_q_heads / a.num_kv_heads;
  const long long units = static_cast<long long>(a.batch) * a.num_partitions * a.num_kv_heads *
                          (ratio / hpw);
  const long long blocks = (units + WG - 1) / WG;
  hipLaunchKernelGGL((paged_partials_kernel<W, WPE, WG>),
                     dim3(static_cast<unsigned>(blocks)), dim3(64 * WG), 0, stream, a);
  return hipGetLastError();
}

// LDS bytes per compute unit of the current device (cached per device;
// 160 KiB on MI355X).
size_t device_lds_per_cu() {
  static size_t lds[64] = {};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 160 * 1024;
  if (lds[dev] == 0) {
    int n = 0;
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMaxSharedMemoryPerMultiprocessor, dev) !=
            hipSuccess || n < 1)
      n = 160 * 1024;
    lds[dev] = static_cast<size_t>(n);
  }
  return lds[dev];
}

// Balanced split: as many workgroups as are resident at once: 4 * WPE
// wavefronts per compute unit in workgroups of WG waves, or fewer when their
// LDS (the static wave slices, the two batch prefixes and the lengths) does
// not fit that many (large batches).
template <class W, int WPE, int WG>
hipError_t launch_balanced(const PagedLaunch& a, hipStream_t stream) {
  const size_t lds = (3 * static_cast<size_t>(a.batch) + 2) * sizeof(int);
  const size_t lds_wg = lds + WG * W::kLdsPerWave + 16;
  const int by_waves = (4 * WPE) / WG;
  const int by_lds = static_cast<int>(device_lds_per_cu() / lds_wg);
  const int groups = device_cus() * max(1, min(by_waves, by_lds));
  hipLaunchKernelGGL((paged_balanced_kernel<W, WPE, WG>),
                     dim3(static_cast<unsigned>(groups)), dim3(64 * WG), lds, stream, a);
  return hipGetLastError();
}

// Tuned on MI355X (bf16, d_head 128): one head per wave keeps 3 waves per
// SIMD; four heads per wave need ~200 VGPRs (2 waves per SIMD) and do best
// with two buffers.  With one head per wave, eight-wave workgroups read whole
// token rows of every block together.  Head chunks of one group share a
// workgroup of four waves when they fit in it: its finer grain (half the
// blocks of an eight-wave one) shortens the tail of long fixed partitions;
// larger groups take eight waves, so that a block's second and later reads
// stay in one XCD's L2.
template <int KT, int D, int HPW>
hipError_t launch_typed(const PagedLaunch& a, hipStream_t stream) {
  constexpr bool kWide = KT != kF32 || D < 128;  // register budget allows >= 2 waves
  // One-byte buffers are half the registers of bf16 ones: three fit beside
  // four heads at two waves per SIMD.
  constexpr int NBUF = (KT >= kI8 || (KT == kBF16 && HPW == 1)) ? 3 : 2;
  constexpr int WPE = (HPW == 1 && kWide) ? 3 : (kWide ? 2 : 1);
  using W = ValuWorker<KT, D, HPW, NBUF>;
  const int ratio = a.num_q_heads / a.num_kv_heads;
  if (a.counts) {
    // Whole workgroups must fill the 4 * WPE wave slots of a compute unit.
    if constexpr ((4 * WPE) % 8 == 0) return launch_balanced<W, WPE, 8>(a, stream);
    return launch_balanced<W, WPE, 4>(a, stream);
  }
  if constexpr (kWide) {
    if (HPW == 1 || ratio > 4 * HPW) return launch_variant<W, WPE, 8>(a, HPW, stream);
  }
  return launch_variant<W, WPE, 4>(a, HPW, stream);
}

// MFMA flavour: one wave per (K/V head, up to 16 query heads).
// Tuned on MI355X (bf16, head_dim 128, GQA and long-context batches): three
// register buffers (two blocks in flight) at two waves per SIMD; four
// buffers changed nothing.  Fixed partitions run in four-wave workgroups,
// whose finer grain shortened the long-context batch by 6%; the balanced
// split keeps eight waves (all K/V heads of a block in one workgroup).
#ifndef KVD_MFMA_NBUF
#define KVD_MFMA_NBUF 3
#endif
#ifndef KVD_MFMA_WPE
#define KVD_MFMA_WPE 2
#endif
#ifndef KVD_MFMA_WG_FIXED
#define KVD_MFMA_WG_FIXED 4
#endif
#ifndef KVD_MFMA_WG_BALANCED
#define KVD_MFMA_WG_BALANCED 8
#endif
#ifndef KVD_MFMA_NBUF_BYTE
#define KVD_MFMA_NBUF_BYTE 3
#endif
#ifndef KVD_MFMA_WPE_BYTE
#define KVD_MFMA_WPE_BYTE 2
#endif
constexpr int kMfmaNbuf = KVD_MFMA_NBUF;
constexpr int kMfmaWpe = KVD_MFMA_WPE;

template <int KT, int D>
hipError_t launch_mfma(const PagedLaunch& a, hipStream_t stream) {
  constexpr int NBUF = KT == kBF16 ? kMfmaNbuf : KVD_MFMA_NBUF_BYTE;
  constexpr int WPE = KT == kBF16 ? kMfmaWpe : KVD_MFMA_WPE_BYTE;
  using W = MfmaWorker<KT, D, NBUF>;
  const int ratio = a.num_q_heads / a.num_kv_heads;
  const int hpw = ratio < 16 ? ratio : 16;
  if (a.counts) {
    if constexpr ((4 * WPE) % KVD_MFMA_WG_BALANCED == 0)
      return launch_balanced<W, WPE, KVD_MFMA_WG_BALANCED>(a, stream);
    return launch_balanced<W, WPE, 4>(a, stream);
  }
  return launch_variant<W, WPE, KVD_MFMA_WG_FIXED>(a, hpw, stream);
}

// Which flavour runs: the MFMA one for bf16 caches with groups of 4 to 16
// query heads (or multiples of 16), where the VALU flavour's per-head work
// makes it ALU-bound (VALU busy 74% of the long-context kernel); groups of 1
// or 2 heads leave most of the MFMA idle, and the VALU flavour measured
// faster there (MHA batch 188 against 193-199 us).  KVD_PAGED_KERNEL=valu
// selects the VALU flavour for every group size (for comparisons).
bool mfma_enabled() {
  static int v = -1;
  if (v < 0) {
    const char* e = getenv("KVD_PAGED_KERNEL");
    v = (e && strcmp(e, "valu") == 0) ? 0 : 1;
  }
  return v == 1;
}

// Groups of more than 4 query heads are split over ratio / 4 wavefronts of the
// same workgroup; they read the same K/V rows, the second time from cache.
template <int KT, int D>
hipError_t launch_by_ratio(const PagedLaunch& a, hipStream_t stream) {
  const int ratio = a.num_q_heads / a.num_kv_heads;
  switch (ratio) {
    case 1: return launch_typed<KT, D, 1>(a, stream);
    case 2: return launch_typed<KT, D, 2>(a, stream);
    default: return launch_typed<KT, D, 4>(a, stream);  // multiples of 4
  }
}

template <int KT>
hipError_t launch_by_dim(const PagedLaunch& a, hipStream_t stream) {
  switch (a.head_dim) {
    case 32: return launch_by_ratio<KT, 32>(a, stream);
    case 64: return launch_by_ratio<KT, 64>(a, stream);
    default: return launch_by_ratio<KT, 128>(a, stream);
  }
}

}  // namespace

bool paged_supported(int head_dim, int ratio, bool /*bf16*/) {
  const bool dim_ok = head_dim == 32 || head_dim == 64 || head_dim == 128;
  const bool ratio_ok = ratio == 1 || ratio == 2 || (ratio % 4 == 0 && ratio <= 64);
  return dim_ok && ratio_ok;
}

int max_partition_blocks() { return kMaxPartitionBlocks; }

hipError_t launch_paged_partials(const PagedLaunch& a, hipStream_t stream) {
  const int ratio = a.num_q_heads / a.num_kv_heads;
  const bool mfma = mfma_enabled() && ratio >= 4 && (ratio <= 16 || ratio % 16 == 0);
  if (a.int8) {
    if (mfma && (a.head_dim == 64 || a.head_dim == 128)) {
      if (a.fp8) return a.head_dim == 64 ? launch_mfma<kF8, 64>(a, stream) : launch_mfma<kF8, 128>(a, stream);
      return a.head_dim == 64 ? launch_mfma<kI8, 64>(a, stream) : launch_mfma<kI8, 128>(a, stream);
    }
    return a.fp8 ? launch_by_dim<kF8>(a, stream) : launch_by_dim<kI8>(a, stream);
  }
  if (!a.bf16) return launch_by_dim<kF32>(a, stream);
  if (mfma) {
    switch (a.head_dim) {
      case 32: return launch_mfma<kBF16, 32>(a, stream);
      case 64: return launch_mfma<kBF16, 64>(a, stream);
      default: return launch_mfma<kBF16, 128>(a, stream);
    }
  }
  return launch_by_dim<kBF16>(a, stream);
}
}  // namespace kvd
