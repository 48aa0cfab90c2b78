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
// run on MFMA 32x32x16 with fp32 accumulation: the scores on the bf16 rows
// and queries, the value product on fp16 (weights, and the latent columns
// converted from bf16, which is exact in fp16's range).
//
// Work decomposition:
//   workgroup = (sequence b, partition p, group of 64 query heads), 8 waves,
//   two blocks of 32 heads.  The waves specialise:
//     score waves 0-1   (head block w): the full 576-wide scores of 32 heads,
//                       Q~ held in registers, then the online softmax; each
//                       writes the weights of its block to LDS;
//     value waves 2-7   (a range of 32-column tiles of the latent, both head
//                       blocks): the unnormalised output of 64 heads x their
//                       columns in registers, fed by those weights.  Wave w
//                       runs beside wave w + 4 on a SIMD; waves 4-5 (beside
//                       the score waves) take two column tiles and the
//                       others three, which with the order of each wave's
//                       staging and products balances the SIMDs over a
//                       tile.
//   Tokens come in tiles of 32 (two 16-token blocks), loaded once per
//   workgroup through the block table (rows past the sequence end read as
//   zeros) by the value waves, stored token-major in LDS and read by all 8
//   waves.  The two head groups of one (sequence, partition) are launched 8
//   workgroups apart, so they run on the same XCD and the second reads the
//   tiles from L2.
//   Scores:  S^T[token][head] = C_tile[32 x 576] . Q~^T[576 x 32] per score
//            wave, 36 MFMAs; every lane ends with one head and 16 tokens.
//   Softmax: online per head with a lazily raised reference max (raised only
//            when a score exceeds it by more than kRaise log2 units); the
//            weights enter the value MFMA rounded to fp16, the running sum
//            takes them in fp32.
//   Output:  O^T[32 x 32] += C_tile^T[32 x 32] . P^T[32 x 32] per column
//            tile, token half and head block (fp16 MFMA); the A operand (one
//            latent column per lane, tokens along K) is read from the
//            token-major tile with LDS transpose loads, converted to fp16 and
//            feeds the MFMAs of both head blocks, and each lane's accumulator
//            column is its own head, so rescaling needs no data movement
//            between lanes.
//   Pipeline: step t computes the scores and weights of tile t and the value
//   product of tile t - 1, and stages tile t + 1, with one barrier per step;
//   the weights and rescale factors alternate between two LDS buffers.
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
constexpr int kThreads = 512;             // 8 waves: 2 score + 6 value
constexpr int kBlockHeads = 32;           // heads per MFMA block
constexpr int kHeadsPerGroup = 2 * kBlockHeads;  // 64
constexpr int kKSteps = kW / 16;          // 36 score K-steps (all of 576)
constexpr int kKBatch = 6;                // K-steps whose LDS reads are in flight together
constexpr int kColTiles = kDc / 32;       // 16 column tiles of 32 latent columns
constexpr int kPvAhead = 3;               // value fragments whose loads run ahead
constexpr int kStageLanes = 3 * kWave;    // lanes that stage one 16-token block
constexpr int kLoadChunks = 6;            // 16-byte chunks per staging lane and tile
constexpr int kLoadWords = 4 * kLoadChunks;
constexpr float kRaise = 8.0f;

static_assert(kKSteps % kKBatch == 0, "batched K-steps");
static_assert(kLdsRow % 16 == 0, "16-byte aligned rows");
// Each 16-token block (18432 bytes) is fetched by three waves: 6 x 16 B per lane.
static_assert(kBlockTokens * kRowBytes == kStageLanes * kLoadChunks * 16, "tile load split");

// Column tiles of value wave w (2 .. 7): [first, first + count).
__device__ __forceinline__ int value_first_tile(int w) {
  return w == 2 ? 0 : w == 3 ? 3 : w == 4 ? 6 : w == 5 ? 8 : w == 6 ? 10 : 13;
}
__device__ __forceinline__ int value_tile_count(int w) { return (w == 4 || w == 5) ? 2 : 3; }

typedef __attribute__((ext_vector_type(16))) float f32x16_t;

__device__ __forceinline__ f32x16_t mfma32(bf16x8_t a, bf16x8_t b, f32x16_t c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

typedef __attribute__((ext_vector_type(8))) _Float16 f16x8_t;

__device__ __forceinline__ f32x16_t mfma32_f16(f16x8_t a, f16x8_t b, f32x16_t c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_f16(a, b, c, 0, 0, 0);
}

// Eight bf16 values (four words) as eight fp16 values: exact for magnitudes
// in [2^-14, 65504], the smaller ones rounded to fp16 subnormals (absolute
// error <= 2^-25), the larger ones infinite.
__device__ __forceinline__ f16x8_t bf16x8_to_f16(uint4 u) {
  const uint4 h = make_uint4(pack_f16x2(bf16_lo(u.x), bf16_hi(u.x)), pack_f16x2(bf16_lo(u.y), bf16_hi(u.y)),
                             pack_f16x2(bf16_lo(u.z), bf16_hi(u.z)), pack_f16x2(bf16_lo(u.w), bf16_hi(u.w)));
  return __builtin_bit_cast(f16x8_t, h);
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
  // fp16 weights of the tile [step parity][head block][token half][lane]
  uint4 pw[2][2][2][kWave];
  float alpha[2][2][kBlockHeads];  // rescale of the step [step parity][head block][head]
  float lsum[2][kBlockHeads];      // weight sum of each head at the end
};

__global__ __launch_bounds__(kThreads) void mla_partials_kernel(MlaLaunchDev a) {
  __shared__ __attribute__((aligned(16))) MlaShared sh;

  const int tid = threadIdx.x;
  const int lane = tid & (kWave - 1);
  const int wave = wave_uniform(tid >> 6);
  const bool score_wave = wave < 2;
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

  // The partition's block-table entries (at most 64 blocks), one per lane,
  // are requested together with the length, before it is known: lane k
  // reads entry blk0 + k of the row (0 past the row's end) and the entries
  // past the partition's last block are dropped below.
  const int t_begin = p * a.partition_tokens;
  const int blk0 = t_begin / kBlockTokens;
  int entry;
  {
    const int32_t* trow = a.block_table + static_cast<size_t>(b) * a.max_blocks_per_seq;
    const int left = wave_uniform(min(max(0, a.max_blocks_per_seq - blk0), kWave));
    const BufRsrc rt = make_rsrc(trow + min(blk0, a.max_blocks_per_seq), left * 4);
    entry = static_cast<int>(__builtin_amdgcn_raw_buffer_load_b32(rt, 4 * lane, 0, 0));
  }
  const int len_in = a.seq_lens[b];
  asm volatile("" ::: "memory");  // (both requests before either wait)
  int len = min(len_in, a.max_seq_len);
  len = min(len, a.max_blocks_per_seq * kBlockTokens);
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

  const int head0 = hg * kHeadsPerGroup;            // first head of the group
  const bool active0 = head0 < a.num_heads;         // head blocks with heads
  const bool active1 = head0 + kBlockHeads < a.num_heads;

  // Tile loads pick their block ids with readlane, and `valid` has bit j set
  // when block j of the partition lies inside the pool.  No memory reads
  // remain in the tile loop besides the tile loads themselves.
  // (Formed in each branch after its first requests: it waits for the table.)
  const int nblk = (t_end - t_begin + kBlockTokens - 1) / kBlockTokens;
  auto valid_blocks = [&]() __attribute__((always_inline)) {
    if (lane >= nblk) entry = -1;
    return __builtin_amdgcn_ballot_w64(entry >= 0 && entry < a.num_blocks);
  };

  const size_t P = a.num_partitions;
  const int nsteps = ntiles + 1;  // the value product trails the scores by one tile

  if (score_wave) {
    const int hb = wave;                       // head block
    const bool active = hb == 0 ? active0 : active1;
    const int head = head0 + hb * kBlockHeads + r32;  // this lane's head
    const bool head_ok = head < a.num_heads;
    // Q~ as the B operand: lane holds head `head`, K-slots 16 ks + 8 g .. +7.
    // A lane past the last head takes head 0's row; its results are never
    // written.  (Marked as changed after the load, so that the compiler keeps
    // it in registers rather than loading it again inside the loop.)
    u32x4_t qf[kKSteps];
    {
      const u32x4_t* qrow = reinterpret_cast<const u32x4_t*>(
          a.q + (static_cast<size_t>(b) * a.num_heads + (head_ok ? head : 0)) * kW);
#pragma unroll
      for (int ks = 0; ks < kKSteps; ++ks) qf[ks] = qrow[2 * ks + g];
    }
    const uint64_t valid = valid_blocks();
    __syncthreads();  // tile 0 staged
#pragma unroll
    for (int ks = 0; ks < kKSteps; ++ks) asm volatile("" : "+v"(qf[ks]));
    float m_run = kMinusBig;  // reference max of this lane's head (log2 units)
    float l_half = 0.f;       // this lane's share of the weight sum
    const float sl2 = a.scale * kLog2e;
    const uint32_t a_off = r32 * kLdsRow + 16 * g;  // A operand row piece

    // Valid rows of each 16-token half of tile ti (0 for a table entry
    // outside the pool, whose rows were read as zeros and must not get weight).
    auto half_valid = [&](int ti, int hv) __attribute__((always_inline)) {
      const int j = 2 * ti + hv;
      const bool ok = j < nblk && ((valid >> j) & 1);
      return ok ? min(kBlockTokens, t_end - t_begin - j * kBlockTokens) : 0;
    };

    auto step = [&](int t) __attribute__((always_inline)) {
      if (!active || t >= ntiles) return;
      const int par = t & 1;
      // A operand: lane holds token r32 of the tile, K-slots as qf.
      const uint8_t* arow = sh.tiles[t % kStages] + opaque(a_off);
      f32x16_t s = f32x16_t{};
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

      // Register r holds token 8 (r / 4) + 4 g + r % 4 of the tile.
      const int nv0 = half_valid(t, 0), nv1 = half_valid(t, 1);
      float z[16];
      float mx = -INFINITY;
      if (nv0 == kBlockTokens && nv1 == kBlockTokens) {  // (every position valid)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          z[r] = s[r] * sl2;
          mx = fmaxf(mx, z[r]);
        }
      } else {
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int tok = 8 * (r / 4) + 4 * g + (r % 4);
          const bool ok = tok < 16 ? tok < nv0 : tok - 16 < nv1;
          z[r] = ok ? s[r] * sl2 : -INFINITY;
          mx = fmaxf(mx, z[r]);
        }
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
      if (g == 0) sh.alpha[par][hb][r32] = al;
      // Weights of token half th (registers 8 th .. 8 th + 7, the K-slots of
      // the value product's K-step th), rounded to fp16 (11 bits: 8-bit
      // weights move outputs that cancel over a few positions by ~1e-3); the
      // sum takes the fp32 weights.
#pragma unroll
      for (int th = 0; th < 2; ++th) {
        uint32_t w[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const float p0 = exp2_fast(z[8 * th + 2 * e] - m_run);
          const float p1 = exp2_fast(z[8 * th + 2 * e + 1] - m_run);
          l_half += p0 + p1;
          w[e] = pack_f16x2(p0, p1);
        }
        sh.pw[par][hb][th][lane] = make_uint4(w[0], w[1], w[2], w[3]);
      }
    };

    for (int t = 0; t < nsteps; t += 2) {
      step(t);
      __syncthreads();
      step(t + 1);
      __syncthreads();
    }
    // Weight sum of the head: both half-waves (lanes l and l ^ 32 hold the
    // same head).
    auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(l_half), __float_as_uint(l_half),
                                               false, false);
    const float l = __uint_as_float(sw[0]) + __uint_as_float(sw[1]);
    if (active && g == 0 && head_ok) {
      const size_t ws_slot = (static_cast<size_t>(b) * a.num_heads + head) * P + p;
      reinterpret_cast<float2*>(a.ws_ml)[ws_slot] = make_float2(m_run, l);
    }
    // The value waves divide their sums by it (one barrier, which every wave
    // of the workgroup reaches).
    if (g == 0) sh.lsum[hb][r32] = active && head_ok ? l : 0.f;
    __syncthreads();
    return;
  }

  // A operand of column tile ct, token half j: lane (row r32, K group g)
  // gets tokens 16 j + 4 g + 0..3 and 16 j + 8 + 4 g + 0..3 of latent
  // column 32 ct + r32 from two transpose loads; within each 16-lane group,
  // lane i supplies row (i / 4) of the four and columns 4 (i % 4) .. +3 of
  // the group's sixteen.
  const int gi = lane & 15;
  const int ct0 = value_first_tile(wave);
  const uint32_t v_off = (4 * g + (gi >> 2)) * kLdsRow +
                         (32 * ct0 + 16 * ((lane >> 4) & 1) + 4 * (gi & 3)) * 2;

  // NCT column tiles from ct0: O^T accumulators acc[head block][tile], lane
  // holds head r32 of the block, latent columns 32 (ct0 + ct) + 8 (r / 4) +
  // 4 g + r % 4 in register r.
  // (The whole value path, staging included, is instantiated once per column
  // tile count, so that no register of one instance lives across the other.)
  auto run = [&](auto nct_c, auto stage_first_c) __attribute__((always_inline)) {
    constexpr int NCT = decltype(nct_c)::value;
    constexpr bool kStageFirst = decltype(stage_first_c)::value;
    // ---- Value waves: staging of the tiles, then the value products.
    // Tile loads: waves 2-4 fetch the tile's first 16-token block, waves 5-7
    // the second (a block is 16 x 1152 contiguous bytes), each lane 6 chunks of
    // 16 B, so every load instruction uses one wave-uniform buffer resource
    // whose byte count ends at the block's last valid row.
    const int half = (wave - 2) / 3;
    const int lt = ((wave - 2) % 3) * kWave + lane;
    const uint64_t valid = valid_blocks();

    // The new row's bytes in the lane that loads them from the cache block (at
    // most one 16-byte chunk per lane: a row is 72 chunks, a lane's chunks are
    // 192 apart).
    int c_sel = -1;
    uint4 new16 = make_uint4(0u, 0u, 0u, 0u);
    if (fused && half == ((rel_new / kBlockTokens) & 1)) {
      const uint8_t* src = reinterpret_cast<const uint8_t*>(a.c_new + static_cast<size_t>(b) * kW);
#pragma unroll
      for (int c = 0; c < kLoadChunks; ++c) {
        const int qi = lt + kStageLanes * c;
        if (qi / kChunks == r_new) {
          c_sel = c;
          new16 = *reinterpret_cast<const uint4*>(src + (qi % kChunks) * 16);
        }
      }
      const int jn = rel_new / kBlockTokens;  // block of the partition
      if (hg == 0 && c_sel >= 0 && ((valid >> jn) & 1)) {
        // The cache receives the caller's writable buffer on this path.
        uint8_t* dst = reinterpret_cast<uint8_t*>(const_cast<uint16_t*>(a.cache)) +
                       static_cast<size_t>(__builtin_amdgcn_readlane(entry, jn)) * kBlockTokens * kRowBytes;
        *reinterpret_cast<uint4*>(dst + (lt + kStageLanes * c_sel) * 16) = new16;
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
      for (int c = 0; c < kLoadChunks; ++c)
        buffer_load_words<4>(dst + 4 * c, r, static_cast<uint32_t>((lt + kStageLanes * c) * 16));
    };
    uint32_t st_off[kLoadChunks];  // LDS byte offsets of this lane's pieces of a tile
#pragma unroll
    for (int c = 0; c < kLoadChunks; ++c) {
      const int qi = lt + kStageLanes * c;
      st_off[c] = (half * kBlockTokens + qi / kChunks) * kLdsRow + (qi % kChunks) * 16;
    }
    // Tile tix goes to LDS; the tile holding the new row takes it from c_new.
    auto store_tile = [&](const uint32_t (&src)[kLoadWords], uint8_t* tile, int tix)
        __attribute__((always_inline)) {
      const bool sub = tix == ti_new;
#pragma unroll
      for (int c = 0; c < kLoadChunks; ++c) {
        uint4 v = make_uint4(src[4 * c], src[4 * c + 1], src[4 * c + 2], src[4 * c + 3]);
        if (sub && c == c_sel) v = new16;
        *reinterpret_cast<uint4*>(tile + opaque(st_off[c])) = v;
      }
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
    store_tile(pre[0], sh.tiles[0], 0);
    load_tile(2, pre[0]);
    __syncthreads();  // tile 0 staged

    auto stage = [&](int t, uint32_t (&slot)[kLoadWords]) __attribute__((always_inline)) {
      store_tile(slot, sh.tiles[(t + 1) % kStages], t + 1);
      load_tile(t + 3, slot);
    };

    f32x16_t acc[2][NCT];
#pragma unroll
    for (int h = 0; h < 2; ++h)
#pragma unroll
      for (int ct = 0; ct < NCT; ++ct) acc[h][ct] = f32x16_t{};

    auto step = [&](int t) __attribute__((always_inline)) {
      if (!active0 || t < 1 || t > ntiles) return;
      const int par = (t - 1) & 1;
      const float al0 = sh.alpha[par][0][r32], al1 = sh.alpha[par][1][r32];
      uint4 pv[2][2];  // fp16 weights of the tile: [head block][token half]
#pragma unroll
      for (int h = 0; h < 2; ++h)
#pragma unroll
        for (int j = 0; j < 2; ++j) pv[h][j] = sh.pw[par][h][j][lane];
      if (__builtin_amdgcn_ballot_w64(al0 != 1.f || al1 != 1.f)) {
#pragma unroll
        for (int ct = 0; ct < NCT; ++ct)
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            acc[0][ct][r] *= al0;
            acc[1][ct][r] *= al1;
          }
      }
      // The transpose loads run kPvAhead fragments ahead of their MFMAs.
      const uint8_t* vb = sh.tiles[(t - 1) % kStages] + opaque(v_off);
      uint2 w[NCT][2][2];
#pragma unroll
      for (int ct = 0; ct < NCT; ++ct)
#pragma unroll
        for (int j = 0; j < 2; ++j)
#pragma unroll
          for (int hh = 0; hh < 2; ++hh)
            w[ct][j][hh] = __builtin_bit_cast(uint2, __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                (lds_s16x4_t*)(vb + (16 * j + 8 * hh) * kLdsRow + 64 * ct)));
#pragma unroll
      for (int ct = 0; ct < NCT; ++ct)
#pragma unroll
        for (int j = 0; j < 2; ++j) {
          const uint2 w0 = w[ct][j][0], w1 = w[ct][j][1];
          const f16x8_t va = bf16x8_to_f16(make_uint4(w0.x, w0.y, w1.x, w1.y));
#pragma unroll
          for (int h = 0; h < 2; ++h)
            acc[h][ct] = mfma32_f16(va, __builtin_bit_cast(f16x8_t, pv[h][j]), acc[h][ct]);
        }
      constexpr int frags = 2 * NCT;
      KVD_SCHED_GROUP(kSchedDsRead, 2 * kPvAhead);
#pragma unroll
      for (int f = 0; f < frags - kPvAhead; ++f) {
        KVD_SCHED_GROUP(kSchedMfma, 2);
        KVD_SCHED_GROUP(kSchedDsRead, 2);
      }
      KVD_SCHED_GROUP(kSchedMfma, 2 * kPvAhead);
    };

    // Waves 2-5 stage first, so that the products of waves 4-5 reach the
    // matrix unit after the score MFMA chain beside them has started; waves
    // 6-7 run their products first, while waves 2-3 on their SIMDs stage.
    for (int t = 0; t < nsteps; t += 2) {
      if constexpr (!kStageFirst) step(t);
      stage(t, pre[1]);
      if constexpr (kStageFirst) step(t);
      __syncthreads();
      if constexpr (!kStageFirst) step(t + 1);
      stage(t + 1, pre[0]);
      if constexpr (kStageFirst) step(t + 1);
      __syncthreads();
    }
    __syncthreads();  // the score waves' weight sums
    if (!active0) return;
    // The piece's row divided by its weight sum, in fp16 (its magnitude is at
    // most that of the largest latent value).
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const int head = head0 + h * kBlockHeads + r32;
      if (head >= a.num_heads) continue;
      const float l = sh.lsum[h][r32];
      const float inv = l > 0.f ? 1.0f / l : 0.f;
      const size_t ws_slot = (static_cast<size_t>(b) * a.num_heads + head) * P + p;
      _Float16* orow = reinterpret_cast<_Float16*>(a.ws_o) + ws_slot * kDc + 32 * ct0 + 4 * g;
#pragma unroll
      for (int ct = 0; ct < NCT; ++ct)
#pragma unroll
        for (int qd = 0; qd < 4; ++qd)
          *reinterpret_cast<uint2*>(orow + 32 * ct + 8 * qd) =
              make_uint2(pack_f16x2(acc[h][ct][4 * qd] * inv, acc[h][ct][4 * qd + 1] * inv),
                         pack_f16x2(acc[h][ct][4 * qd + 2] * inv, acc[h][ct][4 * qd + 3] * inv));
    }
  };
  if (wave >= 6) run(std::integral_constant<int, 3>{}, std::false_type{});
  else if (value_tile_count(wave) == 2) run(std::integral_constant<int, 2>{}, std::true_type{});
  else run(std::integral_constant<int, 3>{}, std::true_type{});
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
