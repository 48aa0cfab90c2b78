// Absorbed multi-head latent attention (MLA) decode: per-partition partials.
//
// The cache keeps one row per token, the latent c_t (d_c = 512) followed by
// the decoupled RoPE key (d_R = 64); with the up-projections folded into the
// query and output projections every query head arrives as one 576-wide
// vector q~ and attends over the shared rows:
//   z_t = scale * q~ . row_t,   out = sum_t softmax(z)_t c_t   (width 512)
// ("KV Cache（键值缓存）", 2.2 路线一, the MLA equations and the decoupled-RoPE
// note; 4 实现要点, MLA needs a kernel that absorbs the up-projection).
// 128 heads against one shared row is a dense contraction, so both products
// run on MFMA (bf16 operands, fp32 accumulation).
//
// Work decomposition:
//   workgroup = (sequence b, partition p, group of 64 query heads), 4 waves,
//   wave w owns 16 heads.  The partition's tokens are processed in tiles of
//   32 (two 16-token blocks).  Each tile is loaded once from HBM by the whole
//   workgroup (buffer loads through the block table, rows past the sequence
//   end read as zeros), stored token-major in LDS, and read by all 4 waves.
//   Scores:  S^T[token][head] = C_tile[32 x 576] . Q~^T[576 x 16] as
//            2 x 18 MFMA 16x16x32 per wave; Q~ stays in registers as the B
//            operand.  The result leaves every lane with one head and 8
//            tokens, exactly the A-operand shape of the second product.
//   Softmax: online per head with a lazily raised reference max (raised only
//            when a score exceeds it by more than kRaise log2 units); weights
//            are rounded to bf16 for the MFMA, and the running sum is taken
//            from the same rounded weights.
//   Output:  O[16 x 512] += P[16 x 32] . C_tile[32 x 512] as 32 MFMA
//            16x16x32; the B operand (tokens along K, one latent dimension per
//            lane) is read from the token-major tile with LDS transpose loads.
//   The partials (m, l, unnormalised O) go to the same workspace layout as
//   the paged decode and are merged by the same log-sum-exp kernel.
#include "kvd_device.h"
#include "kvd_internal.h"

namespace kvd {
namespace {

constexpr int kDc = 512;                  // latent width (value part)
constexpr int kDr = 64;                   // decoupled RoPE key width
constexpr int kW = kDc + kDr;             // cached row width
constexpr int kRowBytes = kW * 2;         // 1152
constexpr int kTile = 32;                 // tokens per tile
constexpr int kChunks = kRowBytes / 16;   // 72 16-byte chunks per row
constexpr int kLdsRow = kRowBytes + 32;   // padded LDS row (bank spread)
constexpr int kThreads = 256;
constexpr int kLoadsPerThread = kBlockTokens * kChunks / (kThreads / 2);  // 9
constexpr int kHeadsPerWave = 16;
constexpr int kHeadsPerGroup = 4 * kHeadsPerWave;
constexpr int kKSteps = kW / 32;          // 18
constexpr int kKBatch = 3;                // K-steps whose LDS reads are in flight together
constexpr int kNTiles = kDc / 16;         // 32
constexpr float kRaise = 8.0f;

static_assert(kBlockTokens * kChunks % (kThreads / 2) == 0, "tile load split");

typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8_t;
typedef __attribute__((ext_vector_type(4))) float f32x4_t;
typedef __attribute__((ext_vector_type(4))) short s16x4_t;
typedef __attribute__((address_space(3))) s16x4_t lds_s16x4_t;

__device__ __forceinline__ bf16x8_t as_bf16x8(uint32_t a, uint32_t b, uint32_t c, uint32_t d) {
  uint4 u = make_uint4(a, b, c, d);
  return __builtin_bit_cast(bf16x8_t, u);
}

__device__ __forceinline__ f32x4_t mfma16(bf16x8_t a, bf16x8_t b, f32x4_t c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

struct MlaLaunchDev {
  const uint16_t* q;        // [B, H, 576]
  const uint16_t* cache;    // [NB, 16, 576]
  const int32_t* block_table;
  const int32_t* seq_lens;
  float* ws_o;              // [B, H, P, 512]
  float* ws_ml;             // [B, H, P, 2]
  int batch, num_heads, max_blocks_per_seq, num_blocks, max_seq_len;
  int partition_tokens, num_partitions, head_groups;
  float scale;
};

__global__ __launch_bounds__(kThreads) void mla_partials_kernel(MlaLaunchDev a) {
  __shared__ __attribute__((aligned(16))) uint8_t tiles[2][kTile * kLdsRow];

  const int tid = threadIdx.x;
  const int lane = tid & (kWave - 1);
  const int wave = tid >> 6;
  const int col = lane & 15;   // MFMA column lane
  const int kb = lane >> 4;    // MFMA K-group

  int u = blockIdx.x;
  const int hg = u % a.head_groups;
  u /= a.head_groups;
  const int p = u % a.num_partitions;
  const int b = u / a.num_partitions;

  int len = a.seq_lens[b];
  len = min(len, a.max_seq_len);
  len = min(len, a.max_blocks_per_seq * kBlockTokens);
  const int t_begin = p * a.partition_tokens;
  if (len <= t_begin) return;  // whole workgroup exits together
  const int t_end = min(len, t_begin + a.partition_tokens);
  const int ntiles = (t_end - t_begin + kTile - 1) / kTile;

  const int head0 = hg * kHeadsPerGroup + wave * kHeadsPerWave;
  const bool active = head0 < a.num_heads;  // waves past the last head only help load
  const int32_t* trow = a.block_table + static_cast<size_t>(b) * a.max_blocks_per_seq;

  // Q~ as B operand: lane holds head head0 + col, K-slots 32 ks + 8 kb .. +7.
  uint32_t qf[kKSteps][4];
  {
    const int h = active ? head0 + col : 0;
    const uint32_t* qrow = reinterpret_cast<const uint32_t*>(
        a.q + (static_cast<size_t>(b) * a.num_heads + h) * kW);
#pragma unroll
    for (int ks = 0; ks < kKSteps; ++ks) load_words<4>(qf[ks], qrow + (32 * ks + 8 * kb) / 2);
  }

  f32x4_t acc[kNTiles];
#pragma unroll
  for (int nt = 0; nt < kNTiles; ++nt) acc[nt] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  float m_run = kMinusBig;  // reference max of head head0 + col (log2 units)
  float l_lane = 0.f;       // this lane's share of the weight sum
  const float sl2 = a.scale * kLog2e;

  // Tile loads: waves 0-1 fetch the tile's first 16-token block, waves 2-3
  // the second, 9 chunks of 16 B per thread (a block is 16 x 1152 contiguous
  // bytes), so every load instruction uses one wave-uniform buffer resource
  // whose byte count ends at the block's last valid row.
  const int half = wave_uniform(wave >> 1);
  const int lt = tid & 127;
  uint32_t pre[2][kLoadsPerThread][4];
  auto load_tile = [&](int ti, uint32_t (&dst)[kLoadsPerThread][4]) __attribute__((always_inline)) {
    const int t0 = t_begin + ti * kTile + half * kBlockTokens;
    int blk = -1;
    if (ti < ntiles && t0 < t_end) blk = trow[t0 / kBlockTokens];
    const bool ok = blk >= 0 && blk < a.num_blocks;
    const int nvalid = ok ? min(kBlockTokens, t_end - t0) : 0;
    const BufRsrc r = make_rsrc(a.cache + static_cast<size_t>(ok ? blk : 0) * kBlockTokens * kW,
                                nvalid * kRowBytes);
#pragma unroll
    for (int c = 0; c < kLoadsPerThread; ++c)
      buffer_load_words<4>(dst[c], r, static_cast<uint32_t>((lt + 128 * c) * 16));
  };
  auto store_tile = [&](const uint32_t (&src)[kLoadsPerThread][4], uint8_t* tile)
      __attribute__((always_inline)) {
#pragma unroll
    for (int c = 0; c < kLoadsPerThread; ++c) {
      const int qi = lt + 128 * c;
      const int row = half * kBlockTokens + qi / kChunks, ch = qi % kChunks;
      *reinterpret_cast<uint4*>(tile + row * kLdsRow + ch * 16) =
          make_uint4(src[c][0], src[c][1], src[c][2], src[c][3]);
    }
  };

  // Valid rows of each 16-token half of tile ti (0 for a table entry outside
  // the pool, whose rows were read as zeros and must not get weight).
  auto half_valid = [&](int ti, int hb) __attribute__((always_inline)) {
    const int t0 = t_begin + ti * kTile + hb * kBlockTokens;
    if (t0 >= t_end) return 0;
    const int blk = trow[t0 / kBlockTokens];
    return (blk >= 0 && blk < a.num_blocks) ? min(kBlockTokens, t_end - t0) : 0;
  };

  auto compute_tile = [&](int ti, const uint8_t* tile) __attribute__((always_inline)) {
    if (!active) return;
    const int nv0 = half_valid(ti, 0), nv1 = half_valid(ti, 1);
    // Scores S^T: lane gets head head0 + col, tokens 16 mt + 4 kb + i.  Two
    // independent accumulator chains per token half keep the MFMA pipe fed.
    f32x4_t s[2][2];
#pragma unroll
    for (int mt = 0; mt < 2; ++mt) {
      s[mt][0] = f32x4_t{0.f, 0.f, 0.f, 0.f};
      s[mt][1] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    }
    // LDS reads are issued in batches of kKBatch K-steps ahead of their
    // MFMAs so that their latency overlaps.
    const uint8_t* arow = tile + col * kLdsRow + 16 * kb;
#pragma unroll
    for (int ks0 = 0; ks0 < kKSteps; ks0 += kKBatch) {
      uint4 av[kKBatch][2];
#pragma unroll
      for (int k = 0; k < kKBatch; ++k)
#pragma unroll
        for (int mt = 0; mt < 2; ++mt)
          av[k][mt] = *reinterpret_cast<const uint4*>(arow + 16 * mt * kLdsRow + 64 * (ks0 + k));
#pragma unroll
      for (int k = 0; k < kKBatch; ++k) {
        const int ks = ks0 + k;
        const bf16x8_t bq = as_bf16x8(qf[ks][0], qf[ks][1], qf[ks][2], qf[ks][3]);
#pragma unroll
        for (int mt = 0; mt < 2; ++mt)
          s[mt][ks & 1] = mfma16(as_bf16x8(av[k][mt].x, av[k][mt].y, av[k][mt].z, av[k][mt].w),
                                 bq, s[mt][ks & 1]);
      }
    }
    float z[2][4];
    float mx = -INFINITY;
#pragma unroll
    for (int mt = 0; mt < 2; ++mt)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const bool ok = 4 * kb + i < (mt ? nv1 : nv0);
        z[mt][i] = ok ? (s[mt][0][i] + s[mt][1][i]) * sl2 : -INFINITY;
        mx = fmaxf(mx, z[mt][i]);
      }
    mx = fmaxf(mx, shfl_xor_f(mx, 16));
    mx = fmaxf(mx, shfl_xor_f(mx, 32));
    const bool up = mx > m_run + kRaise;
    if (__builtin_amdgcn_ballot_w64(up)) {
      const float mn = up ? mx : m_run;
      const float alpha = exp2_fast(m_run - mn);  // per head (col)
      l_lane *= alpha;
      // O rows are heads 4 kb + i: fetch those heads' factors.
      float al[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) al[i] = __shfl(alpha, 4 * kb + i, kWave);
#pragma unroll
      for (int nt = 0; nt < kNTiles; ++nt)
#pragma unroll
        for (int i = 0; i < 4; ++i) acc[nt][i] *= al[i];
      m_run = mn;
    }
    // Weights as the A operand: K-slot j < 4 is token 4 kb + j, j >= 4 is
    // token 16 + 4 kb + (j - 4).
    uint32_t pw[4];
#pragma unroll
    for (int mt = 0; mt < 2; ++mt) {
      const float p0 = exp2_fast(z[mt][0] - m_run), p1 = exp2_fast(z[mt][1] - m_run);
      const float p2 = exp2_fast(z[mt][2] - m_run), p3 = exp2_fast(z[mt][3] - m_run);
      pw[2 * mt] = pack_bf16x2(p0, p1);
      pw[2 * mt + 1] = pack_bf16x2(p2, p3);
      l_lane = dot2_bf16(pw[2 * mt], kBf16OnePair, l_lane);
      l_lane = dot2_bf16(pw[2 * mt + 1], kBf16OnePair, l_lane);
    }
    const bf16x8_t pa = as_bf16x8(pw[0], pw[1], pw[2], pw[3]);
    // Values: lane (col, kb) of the transpose load supplies row
    // T + col / 4 and latent columns 16 nt + 4 (col % 4) .. + 3.
    const uint8_t* vrow0 = tile + (4 * kb + (col >> 2)) * kLdsRow + 8 * (col & 3);
    const uint8_t* vrow1 = vrow0 + 16 * kLdsRow;
#pragma unroll
    for (int nt = 0; nt < kNTiles; ++nt) {
      const s16x4_t v0 = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
          (lds_s16x4_t*)(vrow0 + 32 * nt));
      const s16x4_t v1 = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
          (lds_s16x4_t*)(vrow1 + 32 * nt));
      // Whole-vector casts: K-slots 0-3 from v0, 4-7 from v1.
      const uint2 w0 = __builtin_bit_cast(uint2, v0);
      const uint2 w1 = __builtin_bit_cast(uint2, v1);
      acc[nt] = mfma16(pa, as_bf16x8(w0.x, w0.y, w1.x, w1.y), acc[nt]);
    }
  };

  // Pipeline: tile ti is computed from LDS buffer ti % 2 while tile ti + 1
  // sits in the other buffer and tiles ti + 2 and ti + 3 are in flight in the
  // two register slots (slot ti % 2 holds tile ti + 1 at the start of step
  // ti).  Only the store/refill alternates between the slots, so the compute
  // body exists once.  One barrier per tile; loads past the last tile get a
  // zero-length resource (no memory traffic).
  load_tile(0, pre[0]);
  store_tile(pre[0], tiles[0]);
  load_tile(1, pre[0]);
  load_tile(2, pre[1]);
  __syncthreads();
  for (int ti = 0; ti < ntiles; ++ti) {
    uint8_t* next = tiles[(ti + 1) & 1];
    if ((ti & 1) == 0) {
      store_tile(pre[0], next);
      load_tile(ti + 3, pre[0]);
    } else {
      store_tile(pre[1], next);
      load_tile(ti + 3, pre[1]);
    }
    compute_tile(ti, tiles[ti & 1]);
    __syncthreads();
  }

  if (!active) return;
  float lsum = l_lane;
  lsum += shfl_xor_f(lsum, 16);
  lsum += shfl_xor_f(lsum, 32);
  const size_t P = a.num_partitions;
  if (kb == 0) {
    const size_t slot = (static_cast<size_t>(b) * a.num_heads + head0 + col) * P + p;
    float2 ml;
    ml.x = m_run;
    ml.y = lsum;
    reinterpret_cast<float2*>(a.ws_ml)[slot] = ml;
  }
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const size_t slot = (static_cast<size_t>(b) * a.num_heads + head0 + 4 * kb + i) * P + p;
    float* orow = a.ws_o + slot * kDc + col;
#pragma unroll
    for (int nt = 0; nt < kNTiles; ++nt) orow[16 * nt] = acc[nt][i];
  }
}

}  // namespace

bool mla_supported(int num_heads, int d_c, int d_rope) {
  return d_c == kDc && d_rope == kDr && num_heads >= kHeadsPerWave && num_heads % kHeadsPerWave == 0;
}

hipError_t launch_mla_partials(const MlaLaunch& m, hipStream_t stream) {
  MlaLaunchDev a;
  a.q = static_cast<const uint16_t*>(m.q);
  a.cache = static_cast<const uint16_t*>(m.c_cache);
  a.block_table = m.block_table;
  a.seq_lens = m.seq_lens;
  a.ws_o = m.ws_o;
  a.ws_ml = m.ws_ml;
  a.batch = m.batch;
  a.num_heads = m.num_heads;
  a.max_blocks_per_seq = m.max_blocks_per_seq;
  a.num_blocks = m.num_blocks;
  a.max_seq_len = m.max_seq_len;
  a.partition_tokens = m.partition_tokens;
  a.num_partitions = m.num_partitions;
  a.head_groups = (m.num_heads + kHeadsPerGroup - 1) / kHeadsPerGroup;
  a.scale = m.scale;
  const long long groups = static_cast<long long>(m.batch) * m.num_partitions * a.head_groups;
  hipLaunchKernelGGL(mla_partials_kernel, dim3(static_cast<unsigned>(groups)), dim3(kThreads), 0,
                     stream, a);
  return hipGetLastError();
}

}  // namespace kvd
