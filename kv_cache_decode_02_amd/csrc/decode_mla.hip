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
//   workgroup = (sequence b, partition p, group of 64 query heads), 8 waves
//   (two per SIMD).  Waves w and w + 4 form a pair that owns 16 heads: for
//   the scores each takes one half of the 576-wide K dimension and the two
//   partial score blocks are added through LDS; for the output each takes
//   one half of the 512 latent columns.  No MFMA work is duplicated and a
//   wave needs 64 accumulator registers, not 128, which leaves room for two
//   waves per SIMD.
//   The partition's tokens are processed in tiles of 32 (two 16-token
//   blocks).  Each tile is loaded once from HBM by the whole workgroup
//   (buffer loads through the block table, rows past the sequence end read
//   as zeros), stored token-major in LDS and read by all 8 waves.  The two
//   head groups of one (sequence, partition) are launched 8 workgroups
//   apart, so they run on the same XCD and the second reads the tile from L2.
//   Scores:  S^T[token][head] = C_tile[32 x 288] . Q~^T[288 x 16] per wave
//            as 2 x 9 MFMA 16x16x32; Q~ stays in registers as the B operand.
//            Every lane ends with one head and 8 tokens.
//   Softmax: online per head with a lazily raised reference max (raised only
//            when a score exceeds it by more than kRaise log2 units); weights
//            enter the MFMA as a bf16 value plus its bf16 remainder, the
//            running sum takes them in fp32.  Both waves of a pair compute the
//            same weights from the same summed scores.
//   Output:  O^T[256 x 16] += C_tile^T[256 x 32] . P^T[32 x 16] as 2 x 16 MFMA
//            16x16x32; the A operand (one latent column per lane, tokens
//            along K) is read from the token-major tile with LDS transpose
//            loads, and each lane's accumulator column is its own head, so
//            rescaling needs no data movement between lanes.
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
constexpr int kTileBytes = kTile * kLdsRow;
constexpr int kStages = 3;                // LDS tile buffers
constexpr int kThreads = 512;             // 8 waves: 4 head blocks x 2 halves
constexpr int kHeadsPerWave = 16;
constexpr int kHeadBlocks = 4;
constexpr int kHeadsPerGroup = kHeadBlocks * kHeadsPerWave;  // 64
constexpr int kKSteps = kW / 32 / 2;      // 9 MFMA K-steps per wave (half of 576)
constexpr int kKBatch = 3;                // K-steps whose LDS reads are in flight together
constexpr int kNTiles = kDc / 2 / 16;     // 16 output tiles per wave (half of 512)
constexpr int kLoadWords = 18;            // 72 bytes per thread and tile
constexpr int kXchgFloats = kWave * 8;    // one wave's partial scores
constexpr float kRaise = 8.0f;

static_assert(kKSteps % kKBatch == 0, "batched K-steps");
// Each 16-token block (18432 bytes) is fetched by 256 threads: 4 x 16 B + 8 B.
static_assert(kBlockTokens * kRowBytes == 256 * (4 * 16 + 8), "tile load split");

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
  const uint16_t* c_new;    // fused append: [B, 576], NULL otherwise
};

__global__ __launch_bounds__(kThreads) void mla_partials_kernel(MlaLaunchDev a) {
  __shared__ __attribute__((aligned(16))) uint8_t tiles[kStages][kTileBytes];
  __shared__ __attribute__((aligned(16))) float xchg[2][kThreads / kWave][kXchgFloats];

  const int tid = threadIdx.x;
  const int lane = tid & (kWave - 1);
  const int wave = tid >> 6;
  const int col = lane & 15;   // MFMA column lane: the head
  const int kb = lane >> 4;    // MFMA K-group
  const int hb = wave & 3;     // head block of the wave
  const int kh = wave >> 2;    // K half of the scores, output half of the values

  // Launch order: the head groups of one (sequence, partition) are 8 apart,
  // so that consecutive dispatch places them on the same XCD and the second
  // reads the tiles from that XCD's L2.
  const int u = blockIdx.x;
  const int hg = (u >> 3) % a.head_groups;
  const int pp = (u / (8 * a.head_groups)) * 8 + (u & 7);
  if (pp >= a.batch * a.num_partitions) return;  // whole workgroup exits together
  const int p = pp % a.num_partitions;
  const int b = pp / a.num_partitions;

  const int len_in = a.seq_lens[b];
  int len = min(len_in, a.max_seq_len);
  len = min(len, a.max_blocks_per_seq * kBlockTokens);
  const int t_begin = p * a.partition_tokens;
  if (len <= t_begin) return;
  const int t_end = min(len, t_begin + a.partition_tokens);
  const int ntiles = (t_end - t_begin + kTile - 1) / kTile;
  // Fused append: the partition holding position len - 1 takes that row from
  // c_new (substituted when its tile is staged in LDS), and head group 0
  // writes it into the cache slot.  Not for a length outside the bounds.
  const bool fused = a.c_new != nullptr && len == len_in && t_end == len;
  const int rel_new = len - 1 - t_begin;          // the new row in the partition
  const int ti_new = fused ? rel_new / kTile : -1;  // its tile, -1 for none
  const int r_new = rel_new % kBlockTokens;        // its row in its block

  const int head0 = hg * kHeadsPerGroup + hb * kHeadsPerWave;
  const bool active = head0 < a.num_heads;  // waves past the last head only load

  // The partition's block-table entries (at most 64 blocks), one per lane,
  // read once: tile loads pick theirs with readlane, and `valid` has bit j
  // set when block j of the partition lies inside the pool.  No memory reads
  // remain in the tile loop besides the tile loads themselves.
  const int blk0 = t_begin / kBlockTokens;
  const int nblk = (t_end - t_begin + kBlockTokens - 1) / kBlockTokens;
  int entry = -1;
  if (lane < nblk) entry = a.block_table[static_cast<size_t>(b) * a.max_blocks_per_seq + blk0 + lane];
  const uint64_t valid = __builtin_amdgcn_ballot_w64(entry >= 0 && entry < a.num_blocks);

  // Q~ as B operand: lane holds head head0 + col, K-slots
  // 288 kh + 32 ks + 8 kb .. +7.
  uint32_t qf[kKSteps][4];
  {
    const int h = active ? head0 + col : 0;
    const uint32_t* qrow = reinterpret_cast<const uint32_t*>(
        a.q + (static_cast<size_t>(b) * a.num_heads + h) * kW + kh * (kW / 2));
#pragma unroll
    for (int ks = 0; ks < kKSteps; ++ks) load_words<4>(qf[ks], qrow + (32 * ks + 8 * kb) / 2);
  }

  // O^T accumulators: lane holds head head0 + col, latent columns
  // 256 kh + 16 nt + 4 kb + i.
  f32x4_t acc[kNTiles];
#pragma unroll
  for (int nt = 0; nt < kNTiles; ++nt) acc[nt] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  float m_run = kMinusBig;  // reference max of head head0 + col (log2 units)
  float l_lane = 0.f;       // this lane's share of the weight sum
  const float sl2 = a.scale * kLog2e;

  // Tile loads: waves 0-3 fetch the tile's first 16-token block, waves 4-7
  // the second (a block is 16 x 1152 contiguous bytes), each thread 4 chunks
  // of 16 B and one of 8 B, so every load instruction uses one wave-uniform
  // buffer resource whose byte count ends at the block's last valid row.
  const int half = wave_uniform(wave >> 2);
  const int lt = tid & 255;
  uint32_t pre[2][kLoadWords];

  // The new row's bytes in the lanes that load them from the cache block
  // (load_tile's split of a block): at most one 16-byte chunk (c_sel) and
  // one 8-byte piece (tail_sel) per lane.
  int c_sel = -1;
  bool tail_sel = false;
  uint4 new16 = make_uint4(0u, 0u, 0u, 0u);
  uint2 new8 = make_uint2(0u, 0u);
  if (fused && half == ((rel_new / kBlockTokens) & 1)) {
    const uint8_t* src = reinterpret_cast<const uint8_t*>(a.c_new + static_cast<size_t>(b) * kW);
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      const int qi = lt + 256 * c;
      if (qi / kChunks == r_new) {
        c_sel = c;
        new16 = *reinterpret_cast<const uint4*>(src + (qi % kChunks) * 16);
      }
    }
    const int o = 4 * 256 * 16 + 8 * lt;
    if (o / kRowBytes == r_new) {
      tail_sel = true;
      new8 = *reinterpret_cast<const uint2*>(src + o % kRowBytes);
    }
    const int jn = rel_new / kBlockTokens;  // block of the partition
    if (hg == 0 && ((valid >> jn) & 1)) {
      // The cache receives the caller's writable buffer on this path.
      uint8_t* dst = reinterpret_cast<uint8_t*>(const_cast<uint16_t*>(a.cache)) +
                     static_cast<size_t>(__builtin_amdgcn_readlane(entry, jn)) * kBlockTokens * kRowBytes;
      if (c_sel >= 0) *reinterpret_cast<uint4*>(dst + (lt + 256 * c_sel) * 16) = new16;
      if (tail_sel) *reinterpret_cast<uint2*>(dst + o) = new8;
    }
  }
  auto load_tile = [&](int ti, uint32_t (&dst)[kLoadWords]) __attribute__((always_inline)) {
    const int j = 2 * ti + half;  // block of the partition
    const int t0 = t_begin + j * kBlockTokens;
    const bool ok = j < nblk && ((valid >> j) & 1);
    const int blk = ok ? __builtin_amdgcn_readlane(entry, j) : 0;
    const int nvalid = ok ? min(kBlockTokens, t_end - t0) : 0;
    const BufRsrc r = make_rsrc(a.cache + static_cast<size_t>(blk) * kBlockTokens * kW,
                                nvalid * kRowBytes);
#pragma unroll
    for (int c = 0; c < 4; ++c)
      buffer_load_words<4>(dst + 4 * c, r, static_cast<uint32_t>((lt + 256 * c) * 16));
    buffer_load_words<2>(dst + 16, r, static_cast<uint32_t>(4 * 256 * 16 + 8 * lt));
  };
  // Tile tix goes to LDS; the tile holding the new row takes it from c_new.
  auto store_tile = [&](const uint32_t (&src)[kLoadWords], uint8_t* tile, int tix)
      __attribute__((always_inline)) {
    const bool sub = tix == ti_new;
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      const int qi = lt + 256 * c;
      const int row = half * kBlockTokens + qi / kChunks, ch = qi % kChunks;
      uint4 v = make_uint4(src[4 * c], src[4 * c + 1], src[4 * c + 2], src[4 * c + 3]);
      if (sub && c == c_sel) v = new16;
      *reinterpret_cast<uint4*>(tile + row * kLdsRow + ch * 16) = v;
    }
    const int o = 4 * 256 * 16 + 8 * lt;
    const int row = half * kBlockTokens + o / kRowBytes;
    uint2 t = make_uint2(src[16], src[17]);
    if (sub && tail_sel) t = new8;
    *reinterpret_cast<uint2*>(tile + row * kLdsRow + o % kRowBytes) = t;
  };

  // Valid rows of each 16-token half of tile ti (0 for a table entry outside
  // the pool, whose rows were read as zeros and must not get weight).
  auto half_valid = [&](int ti, int hv) __attribute__((always_inline)) {
    const int j = 2 * ti + hv;
    const bool ok = j < nblk && ((valid >> j) & 1);
    return ok ? min(kBlockTokens, t_end - t_begin - j * kBlockTokens) : 0;
  };

  // Partial scores over this wave's K half: S^T lane gets head head0 + col,
  // tokens 16 mt + 4 kb + i.  Two accumulator chains per token half.
  auto partial_scores = [&](const uint8_t* tile, float (&part)[2][4]) __attribute__((always_inline)) {
    f32x4_t s[2][2];
#pragma unroll
    for (int mt = 0; mt < 2; ++mt) {
      s[mt][0] = f32x4_t{0.f, 0.f, 0.f, 0.f};
      s[mt][1] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    }
    // LDS reads are issued in batches of kKBatch K-steps ahead of their MFMAs.
    const uint8_t* arow = tile + col * kLdsRow + 16 * kb + kh * kRowBytes / 2;
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
#pragma unroll
    for (int mt = 0; mt < 2; ++mt)
#pragma unroll
      for (int i = 0; i < 4; ++i) part[mt][i] = s[mt][0][i] + s[mt][1][i];
  };

  auto softmax_values = [&](int ti, const uint8_t* tile, const float (&full)[2][4])
      __attribute__((always_inline)) {
    const int nv0 = half_valid(ti, 0), nv1 = half_valid(ti, 1);
    float z[2][4];
    float mx = -INFINITY;
#pragma unroll
    for (int mt = 0; mt < 2; ++mt)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const bool ok = 4 * kb + i < (mt ? nv1 : nv0);
        z[mt][i] = ok ? full[mt][i] * sl2 : -INFINITY;
        mx = fmaxf(mx, z[mt][i]);
      }
    mx = row_max4(mx);
    const bool up = mx > m_run + kRaise;
    if (__builtin_amdgcn_ballot_w64(up)) {
      const float mn = up ? mx : m_run;
      const float alpha = exp2_fast(m_run - mn);  // this lane's head
      l_lane *= alpha;
#pragma unroll
      for (int nt = 0; nt < kNTiles; ++nt)
#pragma unroll
        for (int i = 0; i < 4; ++i) acc[nt][i] *= alpha;
      m_run = mn;
    }
    // Weights as the B operand: K-slot j < 4 is token 4 kb + j, j >= 4 is
    // token 16 + 4 kb + (j - 4); a bf16 high part and its bf16 remainder
    // (about 16 bits of weight: 8-bit weights move outputs that cancel over a
    // few positions by ~1e-3); the sum takes the fp32 weights.
    uint32_t pw[4], pr[4];
#pragma unroll
    for (int mt = 0; mt < 2; ++mt) {
#pragma unroll
      for (int h2 = 0; h2 < 2; ++h2) {
        const float p0 = exp2_fast(z[mt][2 * h2] - m_run);
        const float p1 = exp2_fast(z[mt][2 * h2 + 1] - m_run);
        l_lane += p0 + p1;
        const uint32_t w = pack_bf16x2(p0, p1);
        pw[2 * mt + h2] = w;
        pr[2 * mt + h2] = pack_bf16x2(p0 - bf16_lo(w), p1 - bf16_hi(w));
      }
    }
    const bf16x8_t pb = as_bf16x8(pw[0], pw[1], pw[2], pw[3]);
    const bf16x8_t prb = as_bf16x8(pr[0], pr[1], pr[2], pr[3]);
    // Values as the A operand: lane (col, kb) of the transpose load supplies
    // row T + col / 4 and latent columns 16 nt + 4 (col % 4) .. + 3, which
    // leaves the lane with tokens 4 kb .. +3 (and 16 + 4 kb .. +3) of latent
    // column 16 nt + col.
    const uint8_t* vrow0 =
        tile + (4 * kb + (col >> 2)) * kLdsRow + 8 * (col & 3) + kh * (kDc / 2) * 2;
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
      const bf16x8_t va = as_bf16x8(w0.x, w0.y, w1.x, w1.y);
      acc[nt] = mfma16(va, pb, acc[nt]);
      acc[nt] = mfma16(va, prb, acc[nt]);
    }
  };

  // Pipeline: three LDS buffers and two register slots.  Step ti computes
  // the softmax and the value product of tile ti (buffer ti % 3) and the
  // partial scores of tile ti + 1 (buffer (ti + 1) % 3), which are issued
  // first so that their MFMAs overlap the softmax; tile ti + 2 moves from
  // register slot ti % 2 into buffer (ti + 2) % 3 and slot ti % 2 starts
  // loading tile ti + 4.  The step's one barrier at its end publishes the
  // partial scores of tile ti + 1 (exchange buffer (ti + 1) % 2) and tile
  // ti + 2; before it every wave has finished step ti - 1, which makes
  // buffer (ti + 2) % 3 free.  Loads past the last tile get a zero-length
  // resource (no memory traffic) and tiles past the last are masked out.
  // Steps run in pairs, even step on slot 0 and odd step on slot 1, so the
  // order of the loads in flight is the same on every pass and each store
  // waits only for its own slot.
  auto publish = [&](int ti, const float (&part)[2][4]) __attribute__((always_inline)) {
    float4* xo = reinterpret_cast<float4*>(&xchg[ti & 1][wave][lane * 8]);
    xo[0] = make_float4(part[0][0], part[0][1], part[0][2], part[0][3]);
    xo[1] = make_float4(part[1][0], part[1][1], part[1][2], part[1][3]);
  };
  int cur = 0;  // ti % 3
  float part[2][4] = {};  // this wave's partial scores of tile ti
  auto step = [&](int ti, uint32_t (&slot)[kLoadWords]) __attribute__((always_inline)) {
    const int nx = cur == 2 ? 0 : cur + 1;   // (ti + 1) % 3
    const int nxt = cur == 0 ? 2 : cur - 1;  // (ti + 2) % 3
    if (active) {
      const float4* xp = reinterpret_cast<const float4*>(&xchg[ti & 1][wave ^ 4][lane * 8]);
      const float4 o0 = xp[0], o1 = xp[1];
      float next[2][4];
      partial_scores(tiles[nx], next);
      const float oth[2][4] = {{o0.x, o0.y, o0.z, o0.w}, {o1.x, o1.y, o1.z, o1.w}};
      // Both waves of the pair form the same sum (K half 0 first), so they
      // take identical softmax decisions.
      float full[2][4];
#pragma unroll
      for (int mt = 0; mt < 2; ++mt)
#pragma unroll
        for (int i = 0; i < 4; ++i)
          full[mt][i] = kh == 0 ? part[mt][i] + oth[mt][i] : oth[mt][i] + part[mt][i];
      softmax_values(ti, tiles[cur], full);
      publish(ti + 1, next);
#pragma unroll
      for (int mt = 0; mt < 2; ++mt)
#pragma unroll
        for (int i = 0; i < 4; ++i) part[mt][i] = next[mt][i];
    }
    store_tile(slot, tiles[nxt], ti + 2);
    load_tile(ti + 4, slot);
    __syncthreads();
    cur = nx;
  };

  load_tile(0, pre[0]);
  load_tile(1, pre[1]);
  store_tile(pre[0], tiles[0], 0);
  store_tile(pre[1], tiles[1], 1);
  load_tile(2, pre[0]);
  load_tile(3, pre[1]);
  __syncthreads();
  if (active) {
    partial_scores(tiles[0], part);
    publish(0, part);
  }
  __syncthreads();
  for (int ti = 0; ti < ntiles; ti += 2) {
    step(ti, pre[0]);
    step(ti + 1, pre[1]);
  }

  if (!active) return;
  const float lsum = row_sum4(l_lane);
  const size_t P = a.num_partitions;
  const size_t slot = (static_cast<size_t>(b) * a.num_heads + head0 + col) * P + p;
  if (kh == 0 && kb == 0) {
    float2 ml;
    ml.x = m_run;
    ml.y = lsum;
    reinterpret_cast<float2*>(a.ws_ml)[slot] = ml;
  }
  float* orow = a.ws_o + slot * kDc + kh * (kDc / 2) + 4 * kb;
#pragma unroll
  for (int nt = 0; nt < kNTiles; ++nt)
    *reinterpret_cast<float4*>(orow + 16 * nt) = make_float4(acc[nt][0], acc[nt][1], acc[nt][2], acc[nt][3]);
}

}  // namespace

bool mla_supported(int num_heads, int d_c, int d_rope) {
  return d_c == kDc && d_rope == kDr && num_heads >= kHeadsPerWave && num_heads % kHeadsPerWave == 0;
}

int mla_head_groups(int num_heads) { return (num_heads + kHeadsPerGroup - 1) / kHeadsPerGroup; }

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
  a.head_groups = mla_head_groups(m.num_heads);
  a.scale = m.scale;
  a.c_new = static_cast<const uint16_t*>(m.c_new);
  // Workgroups come in runs of 8 (sequence, partition) pairs per head group.
  const long long pairs = static_cast<long long>(m.batch) * m.num_partitions;
  const long long groups = (pairs + 7) / 8 * 8 * a.head_groups;
  hipLaunchKernelGGL(mla_partials_kernel, dim3(static_cast<unsigned>(groups)), dim3(kThreads), 0,
                     stream, a);
  return hipGetLastError();
}

}  // namespace kvd
