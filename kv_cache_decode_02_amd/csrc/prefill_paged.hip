// Chunked prefill / multi-token decode over the paged cache: causal attention
// of n_b new rows per sequence, on MFMA.
//
// Row i of sequence b sits at position p = L_b - n_b + i (L_b = seq_lens[b],
// which counts the new rows) and attends to positions 0..p: the causal mask
// of "单请求 KV Cache" (改动三: row i sees the past_len cached positions and the
// new rows up to its own; past_len = 0 is the triangle of a prefill, n = 1 the
// decode row) over K/V rows read through the block table ("KV-Cache——为什么AI
// 回复越来越快", 08 PagedAttention).  Unlike one decode row, a chunk of rows
// reuses every K/V tile many times, so both products are dense contractions.
//
// Work decomposition: a workgroup of 8 waves takes 128 "rows" of one (sequence,
// KV head g): row rho = (token t of the chunk, head hh of the group) with
// rho = t * r + hh, so the r query heads that share g's K/V are rows of the
// same tiles.  K/V stream through LDS in 64-token tiles (four 16-token blocks,
// double-buffered); every wave reads them for its 16 rows.  (64 tokens rather
// than 32: twice the independent score accumulators and half the barriers
// and softmax passes per token, 3% faster on MI355X.)
//   Scores: S^T[token][row] = K_tile[64 x D] . Q^T[D x 16], 4 x D/32 MFMA
//           16x16x32 bf16 per wave and tile; Q^T stays in registers (B).
//           Each lane ends with one row and 16 tokens.
//   Softmax: online per row with a lazily raised reference max (log2 units);
//           the mask drops tokens past the row's position.
//   Values: O^T[D x 16] += V_tile^T[D x 32] . P^T[32 x 16] for each 32-token
//           half of the tile; V^T comes from the token-major tile by LDS
//           transpose loads.  The weights enter as a
//           bf16 high part and a bf16 remainder (two MFMAs), about 16 bits of
//           weight, since rows over a few positions cancel to small outputs
//           that 8-bit weights would move by ~1e-3; the sum takes the fp32
//           weights.
#include "kvd_device.h"
#include "kvd_internal.h"

namespace kvd {
namespace {

constexpr int kPTile = 64;        // tokens per K/V tile
constexpr int kPWaves = 8;
constexpr int kPRows = 16 * kPWaves;  // rows per workgroup (16 per wave)
constexpr int kPThreads = 64 * kPWaves;
constexpr float kPRaise = 8.0f;

typedef __attribute__((ext_vector_type(8))) __bf16 pbf16x8_t;
typedef __attribute__((ext_vector_type(4))) float pf32x4_t;
typedef __attribute__((ext_vector_type(4))) short ps16x4_t;
typedef __attribute__((address_space(3))) ps16x4_t plds_s16x4_t;

__device__ __forceinline__ pbf16x8_t pas_bf16x8(uint32_t a, uint32_t b, uint32_t c, uint32_t d) {
  return __builtin_bit_cast(pbf16x8_t, make_uint4(a, b, c, d));
}

__device__ __forceinline__ pf32x4_t pmfma16(pbf16x8_t a, pbf16x8_t b, pf32x4_t c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

// Combination over the four 16-lane rows of the wave (lanes l, l ^ 16,
// l ^ 32, l ^ 48): every lane gets the same result.
__device__ __forceinline__ float pmax4(float x) {
  auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  x = fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
  r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float psum4(float x) {
  auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  x = __uint_as_float(r[0]) + __uint_as_float(r[1]);
  r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

template <int D>
__global__ __launch_bounds__(kPThreads) void prefill_kernel(PrefillLaunch a) {
  constexpr int KS = D / 32;           // score K-steps
  constexpr int NT = D / 16;           // output tiles over D
  constexpr int RB = D * 2;            // bytes of one token row of one head
  // Padded LDS row: 32 bytes of padding spread both the 16-byte score reads
  // (16 rows apart) and the 8-byte transpose reads (4 consecutive rows) over
  // distinct banks; with 16 bytes the transpose reads conflicted (0.44 bank
  // conflicts per LDS access, 0 with 32).
  constexpr int LROW = RB + 32;
  constexpr int CPT = RB / 16;         // 16-byte chunks per token row
  constexpr int CHUNKS = kPTile * CPT;  // 16-byte chunks per tile and tensor
  constexpr int LOADS = (CHUNKS + kPThreads - 1) / kPThreads;  // per thread
  static_assert(CHUNKS % 64 == 0 && (CHUNKS % kPThreads == 0 || CHUNKS < kPThreads),
                "whole waves load");
  static_assert((16 * CPT) % 64 == 0, "a wave's chunks lie in one block");
  __shared__ __attribute__((aligned(16))) uint8_t ktile[2][kPTile * LROW];
  __shared__ __attribute__((aligned(16))) uint8_t vtile[2][kPTile * LROW];

  const int tid = threadIdx.x;
  const int lane = tid & (kWave - 1);
  const int wave = wave_uniform(tid >> 6);
  const int col = lane & 15;
  const int kb = lane >> 4;
  const int b = blockIdx.z;
  const int g = blockIdx.y;
  const int r = a.num_q_heads / a.num_kv_heads;

  const int rb = wave_uniform(a.cu_rows[b]);
  const int n = wave_uniform(a.cu_rows[b + 1]) - rb;
  const int row0 = blockIdx.x * kPRows;
  const int L = wave_uniform(min(a.seq_lens[b], a.max_seq_len));
  const int past = L - n;
  if (n <= 0 || row0 >= n * r || past < 0) return;  // whole workgroup

  // This lane's row (the MFMA column) and the position it may see up to.
  const int rho = row0 + wave * 16 + col;
  const bool row_ok = rho < n * r;
  const int t_row = rho / r;
  const int head = g * r + rho % r;
  const int pos = row_ok ? past + t_row : -1;
  const int last_row = min(n * r, row0 + kPRows) - 1;
  const int pmax = past + last_row / r;
  const int ntiles = (pmax + kPTile) / kPTile;

  // Q^T as the B operand: row rho, dimensions 32 ks + 8 kb .. +7.
  uint32_t qf[KS][4];
  {
    const size_t qr = row_ok ? (static_cast<size_t>(rb + t_row) * a.num_q_heads + head) : 0;
    const uint32_t* qw = static_cast<const uint32_t*>(a.q) + qr * (D / 2);
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) load_words<4>(qf[ks], qw + (32 * ks + 8 * kb) / 2);
  }

  pf32x4_t acc[NT];
#pragma unroll
  for (int nt = 0; nt < NT; ++nt) acc[nt] = pf32x4_t{0.f, 0.f, 0.f, 0.f};
  float m_run = kMinusBig;
  float l_lane = 0.f;
  const float sl2 = a.scale * kLog2e;

  // Tile loads: chunk c = tid + kPThreads u of the tile is token c / CPT, 16 bytes
  // c % CPT of its row; every load instruction stays inside one 16-token
  // block, addressed by a wave-uniform buffer resource whose byte count ends
  // after the block's last position (later rows read as zeros).
  const int32_t* trow = a.block_table + static_cast<size_t>(b) * a.max_blocks_per_seq;
  const size_t tok_stride = static_cast<size_t>(a.num_kv_heads) * RB;  // bytes per token
  uint32_t kreg[LOADS][4], vreg[LOADS][4];
  auto load_tile = [&](int ti) __attribute__((always_inline)) {
#pragma unroll
    for (int u = 0; u < LOADS; ++u) {
      const int c = tid + kPThreads * u;
      if (CHUNKS < kPThreads && wave * 64 >= CHUNKS) break;  // waves past the tile
      const int tt = c / CPT, ch = c % CPT;
      const int j = wave_uniform((kPTile * ti + tt) / kBlockTokens);  // block of the sequence
      const int blk = j < a.max_blocks_per_seq && j * kBlockTokens < L ? wave_uniform(trow[j]) : -1;
      const bool ok = blk >= 0 && blk < a.num_blocks;
      const int nvalid = ok ? min(kBlockTokens, L - j * kBlockTokens) : 0;
      const size_t base = (static_cast<size_t>(ok ? blk : 0) * kBlockTokens) * tok_stride +
                          static_cast<size_t>(g) * RB;
      const BufRsrc rk = make_rsrc(static_cast<const uint8_t*>(a.k_cache) + base,
                                   nvalid * static_cast<int>(tok_stride));
      const BufRsrc rv = make_rsrc(static_cast<const uint8_t*>(a.v_cache) + base,
                                   nvalid * static_cast<int>(tok_stride));
      const uint32_t off = static_cast<uint32_t>((tt % kBlockTokens) * tok_stride + 16 * ch);
      buffer_load_words<4>(kreg[u], rk, off);
      buffer_load_words<4>(vreg[u], rv, off);
    }
  };
  auto store_tile = [&](int buf) __attribute__((always_inline)) {
#pragma unroll
    for (int u = 0; u < LOADS; ++u) {
      const int c = tid + kPThreads * u;
      if (CHUNKS < kPThreads && wave * 64 >= CHUNKS) break;
      const int tt = c / CPT, ch = c % CPT;
      *reinterpret_cast<uint4*>(&ktile[buf][tt * LROW + 16 * ch]) =
          make_uint4(kreg[u][0], kreg[u][1], kreg[u][2], kreg[u][3]);
      *reinterpret_cast<uint4*>(&vtile[buf][tt * LROW + 16 * ch]) =
          make_uint4(vreg[u][0], vreg[u][1], vreg[u][2], vreg[u][3]);
    }
  };

  auto compute = [&](int ti, int buf) __attribute__((always_inline)) {
    constexpr int MT = kPTile / 16;   // 16-token score blocks per tile
    // Scores: lane gets row col, tokens 16 mt + 4 kb + i of the tile.
    pf32x4_t s[MT];
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) s[mt] = pf32x4_t{0.f, 0.f, 0.f, 0.f};
    const uint8_t* arow = &ktile[buf][col * LROW + 16 * kb];
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      const pbf16x8_t bq = pas_bf16x8(qf[ks][0], qf[ks][1], qf[ks][2], qf[ks][3]);
#pragma unroll
      for (int mt = 0; mt < MT; ++mt) {
        const uint4 av = *reinterpret_cast<const uint4*>(arow + 16 * mt * LROW + 64 * ks);
        s[mt] = pmfma16(pas_bf16x8(av.x, av.y, av.z, av.w), bq, s[mt]);
      }
    }
    float z[MT][4];
    float mx = -INFINITY;
#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int tp = kPTile * ti + 16 * mt + 4 * kb + i;
        z[mt][i] = tp <= pos ? s[mt][i] * sl2 : -INFINITY;
        mx = fmaxf(mx, z[mt][i]);
      }
    mx = pmax4(mx);
    const bool up = mx > m_run + kPRaise;
    if (__builtin_amdgcn_ballot_w64(up)) {
      const float mn = up ? mx : m_run;
      const float alpha = exp2_fast(m_run - mn);
      l_lane *= alpha;
#pragma unroll
      for (int nt = 0; nt < NT; ++nt)
#pragma unroll
        for (int i = 0; i < 4; ++i) acc[nt][i] *= alpha;
      m_run = mn;
    }
#pragma unroll
    for (int hh = 0; hh < MT / 2; ++hh) {
      // Weights as B for the 32 tokens 32 hh ..: K-slot j < 4 is token 4 kb +
      // j, j >= 4 token 16 + 4 kb + (j - 4); high bf16 parts and remainders.
      uint32_t hi[4], lo[4];
#pragma unroll
      for (int m2 = 0; m2 < 2; ++m2)
#pragma unroll
        for (int pr = 0; pr < 2; ++pr) {
          const float p0 = exp2_fast(z[2 * hh + m2][2 * pr] - m_run);
          const float p1 = exp2_fast(z[2 * hh + m2][2 * pr + 1] - m_run);
          l_lane += p0 + p1;
          const uint32_t h = pack_bf16x2(p0, p1);
          hi[2 * m2 + pr] = h;
          lo[2 * m2 + pr] = pack_bf16x2(p0 - bf16_lo(h), p1 - bf16_hi(h));
        }
      const pbf16x8_t phi = pas_bf16x8(hi[0], hi[1], hi[2], hi[3]);
      const pbf16x8_t plo = pas_bf16x8(lo[0], lo[1], lo[2], lo[3]);
      const uint8_t* vrow0 = &vtile[buf][(32 * hh + 4 * kb + (col >> 2)) * LROW + 8 * (col & 3)];
      const uint8_t* vrow1 = vrow0 + 16 * LROW;
#pragma unroll
      for (int nt = 0; nt < NT; ++nt) {
        const ps16x4_t v0 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((plds_s16x4_t*)(vrow0 + 32 * nt));
        const ps16x4_t v1 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((plds_s16x4_t*)(vrow1 + 32 * nt));
        const uint2 w0 = __builtin_bit_cast(uint2, v0);
        const uint2 w1 = __builtin_bit_cast(uint2, v1);
        const pbf16x8_t av = pas_bf16x8(w0.x, w0.y, w1.x, w1.y);
        acc[nt] = pmfma16(av, phi, acc[nt]);
        acc[nt] = pmfma16(av, plo, acc[nt]);
      }
    }
  };

  load_tile(0);
  store_tile(0);
  __syncthreads();
  for (int ti = 0; ti < ntiles; ++ti) {
    const bool more = ti + 1 < ntiles;
    if (more) load_tile(ti + 1);
    compute(ti, ti & 1);
    if (more) store_tile((ti + 1) & 1);
    __syncthreads();
  }

  if (!row_ok) return;
  const float lsum = psum4(l_lane);
  const float inv = lsum > 0.f ? 1.0f / lsum : 0.f;
  uint16_t* orow = static_cast<uint16_t*>(a.out) +
                   (static_cast<size_t>(rb + t_row) * a.num_q_heads + head) * D + 4 * kb;
#pragma unroll
  for (int nt = 0; nt < NT; ++nt) {
    const uint32_t w0 = pack_bf16x2(acc[nt][0] * inv, acc[nt][1] * inv);
    const uint32_t w1 = pack_bf16x2(acc[nt][2] * inv, acc[nt][3] * inv);
    *reinterpret_cast<uint2*>(orow + 16 * nt) = make_uint2(w0, w1);
  }
}

}  // namespace

bool prefill_supported(int head_dim, bool bf16) { return bf16 && (head_dim == 64 || head_dim == 128); }

hipError_t launch_prefill(const PrefillLaunch& a, hipStream_t stream) {
  const int r = a.num_q_heads / a.num_kv_heads;
  const long long tiles = (static_cast<long long>(a.max_rows) * r + kPRows - 1) / kPRows;
  const dim3 grid(static_cast<unsigned>(tiles), a.num_kv_heads, a.batch);
  if (a.head_dim == 64) {
    hipLaunchKernelGGL(prefill_kernel<64>, grid, dim3(kPThreads), 0, stream, a);
  } else {
    hipLaunchKernelGGL(prefill_kernel<128>, grid, dim3(kPThreads), 0, stream, a);
  }
  return hipGetLastError();
}

}  // namespace kvd
