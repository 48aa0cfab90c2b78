// Split-KV decode attention over a paged cache: per-partition partials.
//
// What is computed (per sequence b, query head h, K/V head g = h / r):
//   z_t = scale * q . K_t,  out = sum_t softmax(z)_t V_t  over t < seq_lens[b]
// ("KV缓存原理与显存估算", 知识点二, the z / a / o equations; the single
// decode row sees every cached position, "单请求 KV Cache", 改动三).
// The positions are cut into partitions; this kernel produces, for each
// (b, h, partition), the running maximum m (log2 units), the sum
// l = sum 2^(z' - m) and the unnormalised acc = sum 2^(z' - m) V_t, with
// z' = z * log2(e).  decode_merge.hip combines the partitions.
//
// Work decomposition (one wavefront = one unit):
//   unit = (b, partition, kv head g, chunk of HPW query heads of the group)
//   The 64 lanes form 8 groups of 8 lanes.  For each 16-token block the
//   group k handles tokens k and k + 8; inside a group each lane owns D/8
//   dimensions of the row, loaded as 16-byte (or 8-byte) vectors laid out so
//   that one load instruction of the 8 lanes covers a contiguous 128 B of the
//   row.  A K/V row is loaded from HBM once and used by all HPW query heads
//   from registers (the GQA sharing), so the cache is read exactly once.
//   Scores: per-lane bf16 dot2 partial sums, reduced over the 8 lanes of the
//   group with DPP moves.
//   Softmax: every lane group keeps its own running max; the reference max
//   is only raised when a score exceeds it by more than kRaise (log2 units),
//   which keeps every exponential below 2^kRaise and makes rescaling of the
//   accumulators rare.  The groups are merged once at the end with shuffles.
//   Latency: the 16-token blocks of a partition are streamed through NBUF
//   register buffers, so NBUF - 1 blocks of loads are in flight while one is
//   being computed; the partition's block ids are read once, one per lane,
//   and broadcast with readlane.
#include "kvd_device.h"
#include "kvd_internal.h"

namespace kvd {
namespace {

constexpr float kRaise = 8.0f;
constexpr int kMaxPartitionBlocks = 64;  // one block id per lane

template <bool BF16, int D>
struct RowShape {
  static constexpr int EPW = BF16 ? 2 : 1;  // elements per 32-bit word
  static constexpr int DPL = D / 8;         // elements of a row per lane
  static constexpr int W = DPL / EPW;       // words of a row per lane
  static constexpr int CW = W < 4 ? W : 4;  // words per vector load
  static constexpr int NCH = W / CW;        // vector loads per row per lane
  static constexpr int RW = D / EPW;        // words per row (one head)
  static_assert(W >= 1 && W % CW == 0, "unsupported head_dim");
  // Word offset, inside a row, of the lane's chunk c.
  static __device__ __forceinline__ int chunk_word(int c, int sub) { return (c * 8 + sub) * CW; }
  // Dimension of the lane's e-th element.
  static __device__ __forceinline__ int dim_of(int e, int sub) {
    const int w = e / EPW;
    return (chunk_word(w / CW, sub) + w % CW) * EPW + e % EPW;
  }
};

// NBUF: register buffers per wave (NBUF - 1 blocks in flight during compute).
// WPE: waves per SIMD the register allocation is sized for.
// WG: wavefronts per workgroup.  Consecutive units are the KV heads (and head
// chunks) of one (sequence, partition), so a workgroup's waves read the same
// blocks together: for 8 KV heads an 8-wave workgroup reads whole contiguous
// token rows of every block.
// PBF16: softmax weights enter the V product as bf16 pairs (dot2, fp32
// accumulation) instead of fp32 FMAs; only for bf16 caches.
template <bool BF16, int D, int HPW, int NBUF, int WPE, int WG, bool PBF16>
__global__ __launch_bounds__(64 * WG) __attribute__((amdgpu_waves_per_eu(WPE, WPE)))
void paged_partials_kernel(PagedLaunch a) {
  static_assert(BF16 || !PBF16, "bf16 weights need a bf16 cache");
  using S = RowShape<BF16, D>;
  constexpr int W = S::W, CW = S::CW, NCH = S::NCH, RW = S::RW, DPL = S::DPL;

  const int lane = threadIdx.x & (kWave - 1);
  const int grp = lane >> 3;
  const int sub = lane & 7;
  const int ratio = a.num_q_heads / a.num_kv_heads;
  const int hchunks = ratio / HPW;

  int u = wave_uniform(blockIdx.x * WG + (threadIdx.x >> 6));
  const int units = a.batch * a.num_partitions * a.num_kv_heads * hchunks;
  if (u >= units) return;
  const int hc = u % hchunks;
  u /= hchunks;
  const int g = u % a.num_kv_heads;
  u /= a.num_kv_heads;
  const int p = u % a.num_partitions;
  const int b = u / a.num_partitions;

  int len = a.seq_lens[b];
  len = min(len, a.max_seq_len);
  len = min(len, a.max_blocks_per_seq * kBlockTokens);
  const int t_begin = p * a.partition_tokens;
  if (len <= t_begin) return;
  const int t_end = min(len, t_begin + a.partition_tokens);
  const int nblk = (t_end - t_begin + kBlockTokens - 1) / kBlockTokens;
  const int j0 = t_begin / kBlockTokens;

  const int32_t* trow = a.block_table + static_cast<size_t>(b) * a.max_blocks_per_seq + j0;
  const int my_id = lane < nblk ? trow[lane] : -1;

  const int h0 = g * ratio + hc * HPW;
  const uint32_t* qw = static_cast<const uint32_t*>(a.q) +
                       (static_cast<size_t>(b) * a.num_q_heads + h0) * RW;
  // Query slice of each head, in the same lane layout as the K rows.
  uint32_t qv[HPW][W];
#pragma unroll
  for (int h = 0; h < HPW; ++h)
#pragma unroll
    for (int c = 0; c < NCH; ++c)
      load_words<CW>(&qv[h][c * CW], qw + h * RW + S::chunk_word(c, sub));

  float m[HPW], l[HPW], acc[HPW][DPL];
#pragma unroll
  for (int h = 0; h < HPW; ++h) {
    m[h] = kMinusBig;
    l[h] = 0.f;
#pragma unroll
    for (int e = 0; e < DPL; ++e) acc[h][e] = 0.f;
  }

  const size_t tok_stride = static_cast<size_t>(a.num_kv_heads) * RW;  // words per token
  const float sl2 = a.scale * kLog2e;
  // Byte offset, inside a physical block, of the lane's chunk 0 for its two
  // token slots (tokens grp and grp + 8); the same for every block.
  uint32_t lane_off[2];
#pragma unroll
  for (int tok = 0; tok < 2; ++tok)
    lane_off[tok] = static_cast<uint32_t>(((grp + 8 * tok) * tok_stride + g * RW +
                                           S::chunk_word(0, sub)) * 4);
  const uint32_t* kcache = static_cast<const uint32_t*>(a.k_cache);
  const uint32_t* vcache = static_cast<const uint32_t*>(a.v_cache);

  struct Frag {
    uint32_t k[2][W];
    uint32_t v[2][W];
  };
  Frag buf[NBUF];

  // Tokens of block jj that hold data: 0 past the partition's last block and
  // for a table entry outside the pool.
  auto valid_tokens = [&](int jj, int& blk) __attribute__((always_inline)) {
    blk = __builtin_amdgcn_readlane(my_id, jj & (kWave - 1));
    const bool ok_blk = jj < nblk && blk >= 0 && blk < a.num_blocks;
    const int tb = t_begin + jj * kBlockTokens;
    return ok_blk ? min(kBlockTokens, t_end - tb) : 0;
  };

  // One buffer resource per block and tensor, whose record count ends after
  // the block's last valid token: rows past it read back as zeros, so the
  // unused tail of a sequence's last block (allocated, contents arbitrary)
  // and out-of-pool table entries contribute nothing.
  auto load_block = [&](Frag& f, int jj) __attribute__((always_inline)) {
    int blk;
    const int nvalid = valid_tokens(jj, blk);
    const size_t base = static_cast<size_t>(nvalid > 0 ? blk : 0) * kBlockTokens * tok_stride;
    const int bytes = nvalid * static_cast<int>(tok_stride) * 4;
    const BufRsrc rk = make_rsrc(kcache + base, bytes);
    const BufRsrc rv = make_rsrc(vcache + base, bytes);
#pragma unroll
    for (int tok = 0; tok < 2; ++tok)
#pragma unroll
      for (int c = 0; c < NCH; ++c) {
        buffer_load_words<CW>(&f.k[tok][c * CW], rk, lane_off[tok] + c * 8 * CW * 4);
        buffer_load_words<CW>(&f.v[tok][c * CW], rv, lane_off[tok] + c * 8 * CW * 4);
      }
  };

  auto compute_block = [&](const Frag& f, int jj) __attribute__((always_inline)) {
    int blk;
    const int nvalid = valid_tokens(jj, blk);
    float s[2][HPW];
#pragma unroll
    for (int tok = 0; tok < 2; ++tok) {
      const bool ok = grp + 8 * tok < nvalid;
#pragma unroll
      for (int h = 0; h < HPW; ++h) {
        float part = 0.f;
#pragma unroll
        for (int w = 0; w < W; ++w) {
          if constexpr (BF16) {
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
    // For bf16 weights: the V elements of the lane's two tokens, paired per
    // dimension (shared by all heads of the group).
    uint32_t vlo[PBF16 ? W : 1], vhi[PBF16 ? W : 1];
    if constexpr (PBF16) {
#pragma unroll
      for (int w = 0; w < W; ++w) {
        vlo[w] = pair_lo(vw[0][w], vw[1][w]);
        vhi[w] = pair_hi(vw[0][w], vw[1][w]);
      }
    }
#pragma unroll
    for (int h = 0; h < HPW; ++h) {
      const float mx = fmaxf(s[0][h], s[1][h]);
      const bool up = mx > m[h] + kRaise;
      if (__builtin_amdgcn_ballot_w64(up)) {
        const float mn = up ? mx : m[h];
        const float alpha = exp2_fast(m[h] - mn);
        l[h] *= alpha;
#pragma unroll
        for (int e = 0; e < DPL; ++e) acc[h][e] *= alpha;
        m[h] = mn;
      }
      const float p0 = exp2_fast(s[0][h] - m[h]);
      const float p1 = exp2_fast(s[1][h] - m[h]);
      if constexpr (PBF16) {
        // Weights rounded to bf16 and paired over the lane's two tokens; the
        // same rounded weights feed the sum, so the output stays an exact
        // convex combination of V rows.  Products accumulate in fp32.
        const uint32_t pp = pack_bf16x2(p0, p1);
        l[h] = dot2_bf16(pp, kBf16OnePair, l[h]);
#pragma unroll
        for (int w = 0; w < W; ++w) {
          acc[h][2 * w] = dot2_bf16(pp, vlo[w], acc[h][2 * w]);
          acc[h][2 * w + 1] = dot2_bf16(pp, vhi[w], acc[h][2 * w + 1]);
        }
      } else {
        l[h] += p0 + p1;
#pragma unroll
        for (int w = 0; w < W; ++w) {
          if constexpr (BF16) {
            acc[h][2 * w] = fmaf(p1, bf16_lo(vw[1][w]), fmaf(p0, bf16_lo(vw[0][w]), acc[h][2 * w]));
            acc[h][2 * w + 1] = fmaf(p1, bf16_hi(vw[1][w]), fmaf(p0, bf16_hi(vw[0][w]), acc[h][2 * w + 1]));
          } else {
            acc[h][w] = fmaf(p1, __uint_as_float(vw[1][w]), fmaf(p0, __uint_as_float(vw[0][w]), acc[h][w]));
          }
        }
      }
    }
  };

  // Refills are unconditional: a block past the end gets a zero-length
  // resource, so its loads touch no memory and keep the buffers in place.
#pragma unroll
  for (int s0 = 0; s0 < NBUF; ++s0) load_block(buf[s0], s0);
  for (int base = 0; base < nblk; base += NBUF) {
#pragma unroll
    for (int s0 = 0; s0 < NBUF; ++s0) {
      const int jj = base + s0;
      if (jj < nblk) compute_block(buf[s0], jj);
      load_block(buf[s0], jj + NBUF);
    }
  }

  // Merge the 8 lane groups (lanes differing in bits 3..5).
#pragma unroll
  for (int h = 0; h < HPW; ++h) {
    float M = m[h];
    M = fmaxf(M, shfl_xor_f(M, 8));
    M = fmaxf(M, shfl_xor_f(M, 16));
    M = fmaxf(M, shfl_xor_f(M, 32));
    const float f = exp2_fast(m[h] - M);
    float lt = l[h] * f;
    lt += shfl_xor_f(lt, 8);
    lt += shfl_xor_f(lt, 16);
    lt += shfl_xor_f(lt, 32);
#pragma unroll
    for (int e = 0; e < DPL; ++e) {
      float x = acc[h][e] * f;
      x += shfl_xor_f(x, 8);
      x += shfl_xor_f(x, 16);
      x += shfl_xor_f(x, 32);
      acc[h][e] = x;
    }
    m[h] = M;
    l[h] = lt;
  }

  // Group k writes query head h0 + k.
  const size_t P = a.num_partitions;
#pragma unroll
  for (int h = 0; h < HPW; ++h) {
    if (grp == h) {
      const size_t slot = (static_cast<size_t>(b) * a.num_q_heads + h0 + h) * P + p;
      float* orow = a.ws_o + slot * D;
#pragma unroll
      for (int e = 0; e < DPL; ++e) orow[S::dim_of(e, sub)] = acc[h][e];
      if (sub == 0) {
        float2 ml;
        ml.x = m[h];
        ml.y = l[h];
        reinterpret_cast<float2*>(a.ws_ml)[slot] = ml;
      }
    }
  }
}

template <bool BF16, int D, int HPW, int NBUF, int WPE, int WG, bool PBF16 = BF16>
hipError_t launch_variant(const PagedLaunch& a, hipStream_t stream) {
  const int ratio = a.num_q_heads / a.num_kv_heads;
  const long long units = static_cast<long long>(a.batch) * a.num_partitions * a.num_kv_heads *
                          (ratio / HPW);
  const long long blocks = (units + WG - 1) / WG;
  hipLaunchKernelGGL((paged_partials_kernel<BF16, D, HPW, NBUF, WPE, WG, PBF16>),
                     dim3(static_cast<unsigned>(blocks)), dim3(64 * WG), 0, stream, a);
  return hipGetLastError();
}

// Tuned on MI355X (bf16, d_head 128): one head per wave keeps 3 waves per
// SIMD; four heads per wave need ~200 VGPRs (2 waves per SIMD) and do best
// with two buffers.  Eight-wave workgroups help when a group's rows are read
// by several wavefronts (one head per wave, or head chunks of one group).
template <bool BF16, int D, int HPW>
hipError_t launch_typed(const PagedLaunch& a, hipStream_t stream) {
  constexpr bool kWide = BF16 || D < 128;  // register budget allows >= 2 waves
  constexpr int NBUF = (BF16 && HPW == 1) ? 3 : 2;
  constexpr int WPE = (HPW == 1 && kWide) ? 3 : (kWide ? 2 : 1);
  const int ratio = a.num_q_heads / a.num_kv_heads;
  if constexpr (kWide) {
    if (HPW == 1 || ratio > HPW) return launch_variant<BF16, D, HPW, NBUF, WPE, 8>(a, stream);
  }
  return launch_variant<BF16, D, HPW, NBUF, WPE, 4>(a, stream);
}

// Groups of more than 4 query heads are split over ratio / 4 wavefronts of the
// same workgroup; they read the same K/V rows, the second time from cache.
template <bool BF16, int D>
hipError_t launch_by_ratio(const PagedLaunch& a, hipStream_t stream) {
  const int ratio = a.num_q_heads / a.num_kv_heads;
  switch (ratio) {
    case 1: return launch_typed<BF16, D, 1>(a, stream);
    case 2: return launch_typed<BF16, D, 2>(a, stream);
    default: return launch_typed<BF16, D, 4>(a, stream);  // multiples of 4
  }
}

template <bool BF16>
hipError_t launch_by_dim(const PagedLaunch& a, hipStream_t stream) {
  switch (a.head_dim) {
    case 32: return launch_by_ratio<BF16, 32>(a, stream);
    case 64: return launch_by_ratio<BF16, 64>(a, stream);
    default: return launch_by_ratio<BF16, 128>(a, stream);
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
  return a.bf16 ? launch_by_dim<true>(a, stream) : launch_by_dim<false>(a, stream);
}

}  // namespace kvd
