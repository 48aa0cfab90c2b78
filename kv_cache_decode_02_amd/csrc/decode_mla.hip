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
// run on MFMA 32x32x16 (bf16 operands, fp32 accumulation).
//
// Work decomposition:
//   workgroup = (sequence b, partition p, group of 64 query heads), 8 waves,
//   two blocks of 32 heads.  The waves specialise:
//     score waves 0-3   (head block w & 1, K half w >> 1): partial scores
//                       over their half of the 576-wide rows, Q~ held in
//                       registers; the two halves are added through LDS and
//                       both waves of a block take the same softmax
//                       decisions; each writes the weights of one 16-token
//                       half of the tile to LDS;
//     value waves 4-7   (head block w & 1, column half (w - 4) >> 1): the
//                       unnormalised output of 32 heads x 256 latent columns
//                       in registers, fed by those weights.
//   With the usual placement of wave w on SIMD w % 4 every SIMD holds one
//   score wave and one value wave, so the softmax arithmetic of the one
//   overlaps the matrix products of the other.  Every LDS fragment of the
//   tile feeds the MFMAs of 32 heads.
//   Tokens come in tiles of 32 (two 16-token blocks), loaded once per
//   workgroup through the block table (rows past the sequence end read as
//   zeros), stored token-major in LDS and shared by all 8 waves.  The two head
//   groups of one (sequence, partition) are launched 8 workgroups apart, so
//   they run on the same XCD and the second reads the tiles from L2.
//   Scores:  S^T[token][head] = C_tile[32 x 288] . Q~^T[288 x 32] per score
//            wave, 18 MFMAs; every lane ends with one head and 16 tokens.
//   Softmax: online per head with a lazily raised reference max (raised only
//            when a score exceeds it by more than kRaise log2 units); the
//            weights enter the value MFMA as a bf16 value plus its bf16
//            remainder, the running sum takes them in fp32.
//   Output:  O^T[256 x 32] += C_tile^T[256 x 32] . P^T[32 x 32] per value
//            wave, 8 column tiles x 2 token halves x 2 (value, remainder);
//            the A operand (one latent column per lane, tokens along K) is
//            read from the token-major tile with LDS transpose loads, and
//            each lane's accumulator column is its own head, so rescaling
//            needs no data movement between lanes.
//   Pipeline: step t computes the scores and weights of tile t and the value
//   product of tile t - 1, in two phases separated by barriers: (A) partial
//   scores of tile t, first value column tiles of tile t - 1, staging of tile
//   t + 1; (B) softmax of tile t, the remaining value column tiles.
//   The partials (m, l, unnormalised O) go to the same workspace layout as
//   the paged decode and are merged by the same log-sum-exp kernel.
#include <type_traits>

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
// Padded LDS row: a stride of 16 mod 256 bytes puts the 16-byte pieces of 16
// consecutive rows in distinct bank groups.
constexpr int kLdsRow = kRowBytes + 16;
constexpr int kTileBytes = kTile * kLdsRow;
constexpr int kStages = 3;                // LDS tile buffers
constexpr int kThreads = 512;             // 8 waves: 4 score + 4 value
constexpr int kBlockHeads = 32;           // heads per MFMA block
constexpr int kHeadsPerGroup = 2 * kBlockHeads;  // 64
constexpr int kKSteps = kW / 2 / 16;      // 18 score K-steps per wave (half of 576)
constexpr int kKBatch = 6;                // K-steps whose LDS reads are in flight together
constexpr int kColTiles = kDc / 2 / 32;   // 8 value column tiles per wave (half of 512)
constexpr int kColTilesA = 4;             // of which phase A runs the first kColTilesA
constexpr int kPvAhead = 3;               // value fragments whose loads run ahead
constexpr int kLoadWords = 18;            // 72 bytes per thread and tile
constexpr float kRaise = 8.0f;

static_assert(kKSteps % kKBatch == 0, "batched K-steps");
static_assert(kLdsRow % 16 == 0, "16-byte aligned rows");
// Each 16-token block (18432 bytes) is fetched by 256 threads: 4 x 16 B + 8 B.
static_assert(kBlockTokens * kRowBytes == 256 * (4 * 16 + 8), "tile load split");

typedef __attribute__((ext_vector_type(16))) float f32x16_t;

__device__ __forceinline__ f32x16_t mfma32(bf16x8_t a, bf16x8_t b, f32x16_t c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ bf16x8_t as_bf16x8(uint4 u) { return __builtin_bit_cast(bf16x8_t, u); }

// x, as a value the compiler must take to change at this point: addresses
// derived from it are formed where they are used instead of being kept in
// registers across the loop for every buffer they may point into.
__device__ __forceinline__ uint32_t opaque(uint32_t x) {
  asm volatile("" : "+v"(x));
  return x;
}

// Instruction-group ordering for the scheduler of the enclosing block
// (masks of the LLVM AMDGPU scheduling-group barrier).
constexpr int kSchedMfma = 0x008;
constexpr int kSchedDsRead = 0x100;
#define KVD_SCHED_GROUP(mask, n) __builtin_amdgcn_sched_group_barrier((mask), (n), 0)

typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));

// Maximum of x over lanes l and l ^ 32 (the swap returns the lane's own
// value and its partner's).
__device__ __forceinline__ float max_over_halves(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
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

struct MlaShared {
  uint8_t tiles[kStages][kTileBytes];
  float4 xchg[4][4][kWave];        // partial scores of each score wave
  uint4 pw[2][2][2][kWave];        // [head block][token half][value, remainder][lane]
  float alpha[2][kBlockHeads];     // rescale of the step, per head
  float lsum[2][2][kWave];         // final weight sums [head block][K half][lane]
};

__global__ __launch_bounds__(kThreads) void mla_partials_kernel(MlaLaunchDev a) {
  __shared__ __attribute__((aligned(16))) MlaShared sh;

  const int tid = threadIdx.x;
  const int lane = tid & (kWave - 1);
  const int wave = wave_uniform(tid >> 6);
  const bool score_wave = wave < 4;
  const int hb = wave & 1;          // head block
  const int hx = (wave >> 1) & 1;   // K half (score waves) or column half (value waves)
  const int r32 = lane & 31;        // MFMA column / row lane: the head, or the token
  const int g = lane >> 5;          // MFMA K group

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

  const int head0 = hg * kHeadsPerGroup + hb * kBlockHeads;
  const bool active = head0 < a.num_heads;  // blocks past the last head only load
  const int head = head0 + r32;             // this lane's head
  const bool head_ok = head < a.num_heads;

  // The partition's block-table entries (at most 64 blocks), one per lane,
  // read once: tile loads pick theirs with readlane, and `valid` has bit j
  // set when block j of the partition lies inside the pool.  No memory reads
  // remain in the tile loop besides the tile loads themselves.
  const int blk0 = t_begin / kBlockTokens;
  const int nblk = (t_end - t_begin + kBlockTokens - 1) / kBlockTokens;
  int entry = -1;
  if (lane < nblk) entry = a.block_table[static_cast<size_t>(b) * a.max_blocks_per_seq + blk0 + lane];
  const uint64_t valid = __builtin_amdgcn_ballot_w64(entry >= 0 && entry < a.num_blocks);

  // Tile loads: waves 0-3 fetch the tile's first 16-token block, waves 4-7
  // the second (a block is 16 x 1152 contiguous bytes), each thread 4 chunks
  // of 16 B and one of 8 B, so every load instruction uses one wave-uniform
  // buffer resource whose byte count ends at the block's last valid row.
  const int half = wave >> 2;
  const int lt = tid & 255;

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
  uint32_t st_off[5];  // LDS byte offsets of this thread's pieces of a tile
#pragma unroll
  for (int c = 0; c < 4; ++c) {
    const int qi = lt + 256 * c;
    st_off[c] = (half * kBlockTokens + qi / kChunks) * kLdsRow + (qi % kChunks) * 16;
  }
  {
    const int o = 4 * 256 * 16 + 8 * lt;
    st_off[4] = (half * kBlockTokens + o / kRowBytes) * kLdsRow + o % kRowBytes;
  }
  auto store_tile = [&](const uint32_t (&src)[kLoadWords], uint8_t* tile, int tix)
      __attribute__((always_inline)) {
    const bool sub = tix == ti_new;
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      uint4 v = make_uint4(src[4 * c], src[4 * c + 1], src[4 * c + 2], src[4 * c + 3]);
      if (sub && c == c_sel) v = new16;
      *reinterpret_cast<uint4*>(tile + opaque(st_off[c])) = v;
    }
    uint2 t = make_uint2(src[16], src[17]);
    if (sub && tail_sel) t = new8;
    *reinterpret_cast<uint2*>(tile + opaque(st_off[4])) = t;
  };

  // Register slots of the staging: step t stores tile t + 1 from slot
  // (t + 1) % 2 into buffer (t + 1) % 3 and starts loading tile t + 3 into
  // that slot.  Loads past the last tile get a zero-length resource (no
  // memory traffic).  Steps run in pairs (even step on slot 1, odd on slot
  // 0), so the order of the loads in flight is the same on every pass and
  // each store waits only for its own slot.
  uint32_t pre[2][kLoadWords];
  load_tile(0, pre[0]);
  load_tile(1, pre[1]);
  // Tile 0 into LDS (inside each branch, after the score waves have requested
  // their query rows, so that both loads are in flight together).
  auto first_tile = [&]() __attribute__((always_inline)) {
    store_tile(pre[0], sh.tiles[0], 0);
    load_tile(2, pre[0]);
    __syncthreads();
  };

  const int nsteps = ntiles + 1;  // the value product trails the scores by one tile
  auto stage = [&](int t, uint32_t (&slot)[kLoadWords]) __attribute__((always_inline)) {
    store_tile(slot, sh.tiles[(t + 1) % kStages], t + 1);
    load_tile(t + 3, slot);
  };

  const size_t P = a.num_partitions;
  const size_t ws_slot = (static_cast<size_t>(b) * a.num_heads + head) * P + p;

  if (score_wave) {
    // Q~ as the B operand: lane holds head `head`, K-slots
    // 288 hx + 16 ks + 8 g .. +7.  (Marked as changed after the load, so
    // that the compiler keeps it in registers rather than loading it again
    // inside the loop.)
    u32x4_t qf[kKSteps];
    {
      const u32x4_t* qrow = reinterpret_cast<const u32x4_t*>(
          a.q + (static_cast<size_t>(b) * a.num_heads + (head_ok ? head : 0)) * kW + hx * (kW / 2));
#pragma unroll
      for (int ks = 0; ks < kKSteps; ++ks) qf[ks] = head_ok ? qrow[2 * ks + g] : u32x4_t{0u, 0u, 0u, 0u};
    }
    first_tile();
#pragma unroll
    for (int ks = 0; ks < kKSteps; ++ks) asm volatile("" : "+v"(qf[ks]));
    float m_run = kMinusBig;  // reference max of this lane's head (log2 units)
    float l_half = 0.f;       // this lane's share of the weight sum
    const float sl2 = a.scale * kLog2e;
    f32x16_t s;               // this wave's partial scores of the current tile
    const uint32_t a_off = r32 * kLdsRow + hx * (kRowBytes / 2) + 16 * g;  // A operand row piece

    // Valid rows of each 16-token half of tile ti (0 for a table entry
    // outside the pool, whose rows were read as zeros and must not get weight).
    auto half_valid = [&](int ti, int hv) __attribute__((always_inline)) {
      const int j = 2 * ti + hv;
      const bool ok = j < nblk && ((valid >> j) & 1);
      return ok ? min(kBlockTokens, t_end - t_begin - j * kBlockTokens) : 0;
    };

    auto phase_a = [&](int t) __attribute__((always_inline)) {
      if (!active || t >= ntiles) return;
      // A operand: lane holds token r32 of the tile, K-slots as qf.
      const uint8_t* arow = sh.tiles[t % kStages] + opaque(a_off);
      s = f32x16_t{};
      uint4 av[kKSteps];
#pragma unroll
      for (int ks = 0; ks < kKSteps; ++ks) av[ks] = *reinterpret_cast<const uint4*>(arow + 32 * ks);
#pragma unroll
      for (int ks = 0; ks < kKSteps; ++ks)
        s = mfma32(as_bf16x8(av[ks]), __builtin_bit_cast(bf16x8_t, qf[ks]), s);
      // kKBatch reads ahead of the MFMA chain.
      KVD_SCHED_GROUP(kSchedDsRead, kKBatch);
#pragma unroll
      for (int ks = 0; ks < kKSteps - kKBatch; ++ks) {
        KVD_SCHED_GROUP(kSchedMfma, 1);
        KVD_SCHED_GROUP(kSchedDsRead, 1);
      }
      KVD_SCHED_GROUP(kSchedMfma, kKBatch);
#pragma unroll
      for (int qd = 0; qd < 4; ++qd)
        sh.xchg[wave][qd][lane] = make_float4(s[4 * qd], s[4 * qd + 1], s[4 * qd + 2], s[4 * qd + 3]);
    };

    auto phase_b = [&](int t) __attribute__((always_inline)) {
      if (!active || t >= ntiles) return;
      // Both waves of the block form the same sum (K half 0 first), so they
      // take identical softmax decisions.
      float z[16];
#pragma unroll
      for (int qd = 0; qd < 4; ++qd) {
        const float4 o = sh.xchg[wave ^ 2][qd][lane];
        const float ov[4] = {o.x, o.y, o.z, o.w};
#pragma unroll
        for (int i = 0; i < 4; ++i) z[4 * qd + i] = hx == 0 ? s[4 * qd + i] + ov[i] : ov[i] + s[4 * qd + i];
      }
      // Register r holds token 8 (r / 4) + 4 g + r % 4 of the tile.
      const int nv0 = half_valid(t, 0), nv1 = half_valid(t, 1);
      float mx = -INFINITY;
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int tok = 8 * (r / 4) + 4 * g + (r % 4);
        const bool ok = tok < 16 ? tok < nv0 : tok - 16 < nv1;
        z[r] = ok ? z[r] * sl2 : -INFINITY;
        mx = fmaxf(mx, z[r]);
      }
      mx = max_over_halves(mx);
      const bool up = mx > m_run + kRaise;
      float al = 1.f;
      if (__builtin_amdgcn_ballot_w64(up)) {
        const float mn = up ? mx : m_run;
        al = exp2_fast(m_run - mn);
        l_half *= al;
        m_run = mn;
      }
      if (hx == 0 && g == 0) sh.alpha[hb][r32] = al;
      // Weights of token half hx (registers 8 hx .. 8 hx + 7, the K-slots of
      // the value product's K-step hx): a bf16 value and its bf16 remainder
      // (about 16 bits of weight: 8-bit weights move outputs that cancel over
      // a few positions by ~1e-3); the sum takes the fp32 weights.
      // (A branch per half keeps the register indices static.)
      auto weights = [&](auto half_c) __attribute__((always_inline)) {
        constexpr int o = 8 * decltype(half_c)::value;
        uint32_t hi[4], lo[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const float p0 = exp2_fast(z[o + 2 * e] - m_run);
          const float p1 = exp2_fast(z[o + 2 * e + 1] - m_run);
          l_half += p0 + p1;
          const uint32_t w = pack_bf16x2(p0, p1);
          hi[e] = w;
          lo[e] = pack_bf16x2(p0 - bf16_lo(w), p1 - bf16_hi(w));
        }
        sh.pw[hb][hx][0][lane] = make_uint4(hi[0], hi[1], hi[2], hi[3]);
        sh.pw[hb][hx][1][lane] = make_uint4(lo[0], lo[1], lo[2], lo[3]);
      };
      if (hx) weights(std::integral_constant<int, 1>{});
      else weights(std::integral_constant<int, 0>{});
    };

    for (int t = 0; t < nsteps; t += 2) {
      phase_a(t);
      stage(t, pre[1]);
      __syncthreads();
      phase_b(t);
      __syncthreads();
      phase_a(t + 1);
      stage(t + 1, pre[0]);
      __syncthreads();
      phase_b(t + 1);
      __syncthreads();
    }
    // Weight sum of the head: both K halves, both half-waves.
    sh.lsum[hb][hx][lane] = l_half;
    __syncthreads();
    if (active && hx == 0 && g == 0 && head_ok) {
      const float l = (sh.lsum[hb][0][lane] + sh.lsum[hb][1][lane]) +
                      (sh.lsum[hb][0][lane + 32] + sh.lsum[hb][1][lane + 32]);
      reinterpret_cast<float2*>(a.ws_ml)[ws_slot] = make_float2(m_run, l);
    }
  } else {
    // O^T accumulators: lane holds head `head`, latent columns
    // 256 hx + 32 ct + 8 (r / 4) + 4 g + r % 4 in register r of tile ct.
    first_tile();
    f32x16_t acc[kColTiles];
#pragma unroll
    for (int ct = 0; ct < kColTiles; ++ct) acc[ct] = f32x16_t{};
    uint4 pv[2][2];  // weights of the tile: [token half][value, remainder]

    // A operand of column tile ct, token half j: lane (row r32, K group g)
    // gets tokens 16 j + 4 g + 0..3 and 16 j + 8 + 4 g + 0..3 of latent
    // column 256 hx + 32 ct + r32 from two transpose loads; within each
    // 16-lane group, lane i supplies row (i / 4) of the four and columns
    // 4 (i % 4) .. +3 of the group's sixteen.
    const int gi = lane & 15;
    const uint32_t v_off = (4 * g + (gi >> 2)) * kLdsRow +
                           (hx * (kDc / 2) + 16 * ((lane >> 4) & 1) + 4 * (gi & 3)) * 2;
    // The transpose loads run kPvAhead fragments ahead of their MFMAs.
    auto pv_tiles = [&](const uint8_t* tile, auto ct0_c, auto ct1_c) __attribute__((always_inline)) {
      constexpr int ct0 = decltype(ct0_c)::value, ct1 = decltype(ct1_c)::value;
      const uint8_t* vb = tile + opaque(v_off);
      uint2 w[ct1 - ct0][2][2];
#pragma unroll
      for (int ct = ct0; ct < ct1; ++ct)
#pragma unroll
        for (int j = 0; j < 2; ++j)
#pragma unroll
          for (int hh = 0; hh < 2; ++hh)
            w[ct - ct0][j][hh] = __builtin_bit_cast(uint2, __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                (lds_s16x4_t*)(vb + (16 * j + 8 * hh) * kLdsRow + 64 * ct)));
#pragma unroll
      for (int ct = ct0; ct < ct1; ++ct)
#pragma unroll
        for (int j = 0; j < 2; ++j) {
          const uint2 w0 = w[ct - ct0][j][0], w1 = w[ct - ct0][j][1];
          const bf16x8_t va = as_bf16x8(make_uint4(w0.x, w0.y, w1.x, w1.y));
          acc[ct] = mfma32(va, as_bf16x8(pv[j][0]), acc[ct]);
          acc[ct] = mfma32(va, as_bf16x8(pv[j][1]), acc[ct]);
        }
      constexpr int frags = 2 * (ct1 - ct0);
      KVD_SCHED_GROUP(kSchedDsRead, 2 * kPvAhead);
#pragma unroll
      for (int f = 0; f < frags - kPvAhead; ++f) {
        KVD_SCHED_GROUP(kSchedMfma, 2);
        KVD_SCHED_GROUP(kSchedDsRead, 2);
      }
      KVD_SCHED_GROUP(kSchedMfma, 2 * kPvAhead);
    };

    auto phase_a = [&](int t) __attribute__((always_inline)) {
      if (!active || t < 1 || t > ntiles) return;
      const float al = sh.alpha[hb][r32];
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        pv[j][0] = sh.pw[hb][j][0][lane];
        pv[j][1] = sh.pw[hb][j][1][lane];
      }
      if (__builtin_amdgcn_ballot_w64(al != 1.f)) {
#pragma unroll
        for (int ct = 0; ct < kColTiles; ++ct)
#pragma unroll
          for (int r = 0; r < 16; ++r) acc[ct][r] *= al;
      }
      pv_tiles(sh.tiles[(t - 1) % kStages], std::integral_constant<int, 0>{},
               std::integral_constant<int, kColTilesA>{});
    };
    auto phase_b = [&](int t) __attribute__((always_inline)) {
      if (!active || t < 1 || t > ntiles) return;
      pv_tiles(sh.tiles[(t - 1) % kStages], std::integral_constant<int, kColTilesA>{},
               std::integral_constant<int, kColTiles>{});
    };

    for (int t = 0; t < nsteps; t += 2) {
      phase_a(t);
      stage(t, pre[1]);
      __syncthreads();
      phase_b(t);
      __syncthreads();
      phase_a(t + 1);
      stage(t + 1, pre[0]);
      __syncthreads();
      phase_b(t + 1);
      __syncthreads();
    }
    __syncthreads();  // matches the score waves' weight-sum exchange
    if (!active || !head_ok) return;
    float* orow = a.ws_o + ws_slot * kDc + hx * (kDc / 2) + 4 * g;
#pragma unroll
    for (int ct = 0; ct < kColTiles; ++ct)
#pragma unroll
      for (int qd = 0; qd < 4; ++qd)
        *reinterpret_cast<float4*>(orow + 32 * ct + 8 * qd) =
            make_float4(acc[ct][4 * qd], acc[ct][4 * qd + 1], acc[ct][4 * qd + 2], acc[ct][4 * qd + 3]);
  }
}

}  // namespace

bool mla_supported(int num_heads, int d_c, int d_rope) {
  return d_c == kDc && d_rope == kDr && num_heads >= 16 && num_heads % 16 == 0;
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
