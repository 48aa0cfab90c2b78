// Host-side paged block allocator: reference-counted physical blocks, fork
// (shared blocks), copy-on-write when a shared last block is appended to,
// and prefix caching through chained block hashes.
//
// "KV-Cache——为什么AI回复越来越快" (08 PagedAttention: fixed-size pages,
// freed pages reused at once, copy-on-write sharing of a common prefix);
// "KV Cache（键值缓存）" (2.3: block table, sharing between parallel samples
// and beam candidates with reference counts and copy-on-write); "KV缓存原理与显存
// 估算" (知识点三: a block's key chains its parent's key, the block's tokens
// and the compatibility identity; 源码导读: reference counts say how many
// users hold a block, hashes say what computation it holds; a block whose
// count drops to zero stays matchable until its memory is reused).
//
// Allocation order: a block never cached comes first; otherwise the cached
// block with count zero that was released longest ago is evicted (its hash
// forgotten).  Every call either succeeds completely or changes nothing.
#include <limits.h>
#include <stdint.h>
#include <string.h>

#include <algorithm>
#include <deque>
#include <map>
#include <new>
#include <string>
#include <vector>

#include "../../include/kvdecode.h"

namespace kvd {
namespace {

// ---- SHA-256 (FIPS 180-4), written from the standard -------------------------

struct Sha256 {
  uint32_t h[8];
  uint64_t bits = 0;
  uint8_t buf[64];
  size_t fill = 0;

  static uint32_t rotr(uint32_t x, int n) { return (x >> n) | (x << (32 - n)); }

  Sha256() {
    static const uint32_t init[8] = {0x6a09e667u, 0xbb67ae85u, 0x3c6ef372u, 0xa54ff53au,
                                     0x510e527fu, 0x9b05688cu, 0x1f83d9abu, 0x5be0cd19u};
    memcpy(h, init, sizeof(h));
  }

  void block(const uint8_t* p) {
    static const uint32_t k[64] = {
        0x428a2f98u, 0x71374491u, 0xb5c0fbcfu, 0xe9b5dba5u, 0x3956c25bu, 0x59f111f1u,
        0x923f82a4u, 0xab1c5ed5u, 0xd807aa98u, 0x12835b01u, 0x243185beu, 0x550c7dc3u,
        0x72be5d74u, 0x80deb1feu, 0x9bdc06a7u, 0xc19bf174u, 0xe49b69c1u, 0xefbe4786u,
        0x0fc19dc6u, 0x240ca1ccu, 0x2de92c6fu, 0x4a7484aau, 0x5cb0a9dcu, 0x76f988dau,
        0x983e5152u, 0xa831c66du, 0xb00327c8u, 0xbf597fc7u, 0xc6e00bf3u, 0xd5a79147u,
        0x06ca6351u, 0x14292967u, 0x27b70a85u, 0x2e1b2138u, 0x4d2c6dfcu, 0x53380d13u,
        0x650a7354u, 0x766a0abbu, 0x81c2c92eu, 0x92722c85u, 0xa2bfe8a1u, 0xa81a664bu,
        0xc24b8b70u, 0xc76c51a3u, 0xd192e819u, 0xd6990624u, 0xf40e3585u, 0x106aa070u,
        0x19a4c116u, 0x1e376c08u, 0x2748774cu, 0x34b0bcb5u, 0x391c0cb3u, 0x4ed8aa4au,
        0x5b9cca4fu, 0x682e6ff3u, 0x748f82eeu, 0x78a5636fu, 0x84c87814u, 0x8cc70208u,
        0x90befffau, 0xa4506cebu, 0xbef9a3f7u, 0xc67178f2u};
    uint32_t w[64];
    for (int i = 0; i < 16; ++i)
      w[i] = (uint32_t(p[4 * i]) << 24) | (uint32_t(p[4 * i + 1]) << 16) |
             (uint32_t(p[4 * i + 2]) << 8) | uint32_t(p[4 * i + 3]);
    for (int i = 16; i < 64; ++i) {
      const uint32_t s0 = rotr(w[i - 15], 7) ^ rotr(w[i - 15], 18) ^ (w[i - 15] >> 3);
      const uint32_t s1 = rotr(w[i - 2], 17) ^ rotr(w[i - 2], 19) ^ (w[i - 2] >> 10);
      w[i] = w[i - 16] + s0 + w[i - 7] + s1;
    }
    uint32_t a = h[0], b = h[1], c = h[2], d = h[3], e = h[4], f = h[5], g = h[6], hh = h[7];
    for (int i = 0; i < 64; ++i) {
      const uint32_t t1 = hh + (rotr(e, 6) ^ rotr(e, 11) ^ rotr(e, 25)) + ((e & f) ^ (~e & g)) +
                          k[i] + w[i];
      const uint32_t t2 = (rotr(a, 2) ^ rotr(a, 13) ^ rotr(a, 22)) + ((a & b) ^ (a & c) ^ (b & c));
      hh = g;
      g = f;
      f = e;
      e = d + t1;
      d = c;
      c = b;
      b = a;
      a = t1 + t2;
    }
    h[0] += a; h[1] += b; h[2] += c; h[3] += d;
    h[4] += e; h[5] += f; h[6] += g; h[7] += hh;
  }

  void update(const void* data, size_t n) {
    const uint8_t* p = static_cast<const uint8_t*>(data);
    bits += uint64_t(n) * 8;
    while (n > 0) {
      const size_t take = std::min(n, size_t(64) - fill);
      memcpy(buf + fill, p, take);
      fill += take;
      p += take;
      n -= take;
      if (fill == 64) {
        block(buf);
        fill = 0;
      }
    }
  }

  void finish(uint8_t out[32]) {
    const uint64_t total = bits;
    const uint8_t one = 0x80, zero = 0;
    update(&one, 1);
    while (fill != 56) update(&zero, 1);
    uint8_t len[8];
    for (int i = 0; i < 8; ++i) len[i] = uint8_t(total >> (56 - 8 * i));
    update(len, 8);
    for (int i = 0; i < 8; ++i)
      for (int j = 0; j < 4; ++j) out[4 * i + j] = uint8_t(h[i] >> (24 - 8 * j));
  }
};

void put_u32(Sha256& s, uint32_t v) {
  const uint8_t b[4] = {uint8_t(v), uint8_t(v >> 8), uint8_t(v >> 16), uint8_t(v >> 24)};
  s.update(b, 4);
}

// ---- the pool -------------------------------------------------------------------

using Key = std::string;  // 32 hash bytes

struct Block {
  int ref = 0;
  bool cached = false;  // holds a registered hash
  Key key;
  uint64_t released = 0;  // release stamp while cached with ref == 0
};

struct Seq {
  bool live = false;
  int64_t len = 0;
  std::vector<int32_t> blocks;
};

}  // namespace
}  // namespace kvd

struct kvd_block_pool {
  int block_size = 16;
  std::vector<kvd::Block> blocks;
  std::deque<int32_t> never_cached;           // free and holding no hash
  std::map<uint64_t, int32_t> evictable;      // release stamp -> cached block with ref 0
  std::map<kvd::Key, int32_t> by_key;         // registered hash -> block
  std::vector<kvd::Seq> seqs;
  uint64_t clock = 0;
};

namespace kvd {
namespace {

int available(const kvd_block_pool* p) {
  return static_cast<int>(p->never_cached.size() + p->evictable.size());
}

// Takes a block for new contents (count 1), evicting a cached one if needed.
int32_t take_block(kvd_block_pool* p) {
  int32_t id;
  if (!p->never_cached.empty()) {
    id = p->never_cached.front();
    p->never_cached.pop_front();
  } else {
    auto it = p->evictable.begin();
    id = it->second;
    p->evictable.erase(it);
    Block& b = p->blocks[id];
    p->by_key.erase(b.key);
    b.cached = false;
    b.key.clear();
  }
  p->blocks[id].ref = 1;
  return id;
}

void hold(kvd_block_pool* p, int32_t id) {
  Block& b = p->blocks[id];
  if (b.ref == 0 && b.cached) p->evictable.erase(b.released);
  ++b.ref;
}

void drop(kvd_block_pool* p, int32_t id) {
  Block& b = p->blocks[id];
  if (--b.ref > 0) return;
  if (b.cached) {
    b.released = ++p->clock;
    p->evictable[b.released] = id;
  } else {
    p->never_cached.push_back(id);
  }
}

Seq* seq_of(kvd_block_pool* p, int s) {
  if (!p || s < 0 || s >= static_cast<int>(p->seqs.size()) || !p->seqs[s].live) return nullptr;
  return &p->seqs[s];
}

int new_seq(kvd_block_pool* p) {
  for (size_t i = 0; i < p->seqs.size(); ++i)
    if (!p->seqs[i].live) {
      p->seqs[i] = Seq();
      p->seqs[i].live = true;
      return static_cast<int>(i);
    }
  p->seqs.emplace_back();
  p->seqs.back().live = true;
  return static_cast<int>(p->seqs.size() - 1);
}

}  // namespace
}  // namespace kvd

using namespace kvd;

extern "C" {

int kvd_block_hashes(const int32_t* tokens, int64_t num_tokens, int block_size,
                     const void* identity, size_t identity_bytes, uint8_t* out) {
  if (block_size < 1 || num_tokens < 0) return KVD_ERR_SHAPE;
  if ((num_tokens > 0 && !tokens) || (identity_bytes > 0 && !identity)) return KVD_ERR_NULL;
  const int64_t full = num_tokens / block_size;
  if (full > 0 && !out) return KVD_ERR_NULL;
  for (int64_t i = 0; i < full * block_size; ++i)
    if (tokens[i] < 0) return KVD_ERR_SHAPE;
  uint8_t parent[32];
  for (int64_t j = 0; j < full; ++j) {
    Sha256 s;
    s.update("kvd-block-v1", 12);
    put_u32(s, j == 0 ? 0u : 32u);
    if (j > 0) s.update(parent, 32);
    put_u32(s, static_cast<uint32_t>(identity_bytes));
    if (identity_bytes) s.update(identity, identity_bytes);
    put_u32(s, static_cast<uint32_t>(block_size));
    for (int t = 0; t < block_size; ++t) put_u32(s, static_cast<uint32_t>(tokens[j * block_size + t]));
    s.finish(parent);
    memcpy(out + 32 * j, parent, 32);
  }
  return static_cast<int>(std::min<int64_t>(full, INT32_MAX));
}

kvd_block_pool* kvd_pool_create(int num_blocks, int block_size) {
  if (num_blocks < 1 || block_size < 1) return nullptr;
  kvd_block_pool* p = new (std::nothrow) kvd_block_pool;
  if (!p) return nullptr;
  try {
    p->block_size = block_size;
    p->blocks.resize(num_blocks);
    for (int i = 0; i < num_blocks; ++i) p->never_cached.push_back(i);
  } catch (...) {
    delete p;
    return nullptr;
  }
  return p;
}

void kvd_pool_destroy(kvd_block_pool* p) { delete p; }

int kvd_pool_available(const kvd_block_pool* p) { return p ? available(p) : KVD_ERR_NULL; }

int kvd_pool_used(const kvd_block_pool* p) {
  return p ? static_cast<int>(p->blocks.size()) - available(p) : KVD_ERR_NULL;
}

int kvd_pool_block_ref(const kvd_block_pool* p, int block) {
  if (!p) return KVD_ERR_NULL;
  if (block < 0 || block >= static_cast<int>(p->blocks.size())) return KVD_ERR_SHAPE;
  return p->blocks[block].ref;
}

int kvd_seq_create(kvd_block_pool* p) {
  if (!p) return KVD_ERR_NULL;
  try {
    return new_seq(p);
  } catch (...) {
    return KVD_ERR_NOMEM;
  }
}

int kvd_seq_fork(kvd_block_pool* p, int seq) {
  Seq* s = seq_of(p, seq);
  if (!s) return p ? KVD_ERR_SHAPE : KVD_ERR_NULL;
  try {
    const Seq copy = *s;
    const int child = new_seq(p);
    p->seqs[child].len = copy.len;
    p->seqs[child].blocks = copy.blocks;
    for (int32_t id : copy.blocks) hold(p, id);
    return child;
  } catch (...) {
    return KVD_ERR_NOMEM;
  }
}

int kvd_seq_release(kvd_block_pool* p, int seq) {
  Seq* s = seq_of(p, seq);
  if (!s) return p ? KVD_ERR_SHAPE : KVD_ERR_NULL;
  for (int32_t id : s->blocks) drop(p, id);
  *s = Seq();
  return KVD_OK;
}

int kvd_seq_append(kvd_block_pool* p, int seq, int num_tokens, int32_t* copies, int max_copies,
                   int* num_copies) {
  Seq* s = seq_of(p, seq);
  if (!s) return p ? KVD_ERR_SHAPE : KVD_ERR_NULL;
  if (num_tokens < 0 || !num_copies) return num_tokens < 0 ? KVD_ERR_SHAPE : KVD_ERR_NULL;
  *num_copies = 0;
  if (num_tokens == 0) return KVD_OK;
  const int bs = p->block_size;
  const int64_t fill = s->len % bs;  // tokens in the last block
  // A partly filled last block held by someone else is copied first.
  const bool cow = fill != 0 && p->blocks[s->blocks.back()].ref > 1;
  const int64_t need_blocks =
      (s->len + num_tokens + bs - 1) / bs - static_cast<int64_t>(s->blocks.size()) + (cow ? 1 : 0);
  if (need_blocks > available(p)) return KVD_ERR_NOMEM;
  if (cow && (!copies || max_copies < 1)) return KVD_ERR_SHAPE;
  try {
    s->blocks.reserve(s->blocks.size() + need_blocks);
  } catch (...) {
    return KVD_ERR_NOMEM;
  }
  if (cow) {
    const int32_t old = s->blocks.back();
    const int32_t fresh = take_block(p);
    copies[0] = old;
    copies[1] = fresh;
    *num_copies = 1;
    drop(p, old);
    s->blocks.back() = fresh;
  }
  while (static_cast<int64_t>(s->blocks.size()) * bs < s->len + num_tokens)
    s->blocks.push_back(take_block(p));
  s->len += num_tokens;
  return KVD_OK;
}

int64_t kvd_seq_len(const kvd_block_pool* p, int seq) {
  Seq* s = seq_of(const_cast<kvd_block_pool*>(p), seq);
  return s ? s->len : (p ? KVD_ERR_SHAPE : KVD_ERR_NULL);
}

int kvd_seq_table(const kvd_block_pool* p, int seq, int32_t* out, int capacity) {
  Seq* s = seq_of(const_cast<kvd_block_pool*>(p), seq);
  if (!s) return p ? KVD_ERR_SHAPE : KVD_ERR_NULL;
  const int n = static_cast<int>(s->blocks.size());
  if (n > 0 && (!out || capacity < n)) return KVD_ERR_SHAPE;
  std::copy(s->blocks.begin(), s->blocks.end(), out);
  return n;
}

int kvd_seq_commit_hashes(kvd_block_pool* p, int seq, const uint8_t* hashes, int num_hashes) {
  Seq* s = seq_of(p, seq);
  if (!s) return p ? KVD_ERR_SHAPE : KVD_ERR_NULL;
  if (num_hashes < 0 || (num_hashes > 0 && !hashes)) return KVD_ERR_NULL;
  const int64_t full = s->len / p->block_size;
  if (num_hashes > full) return KVD_ERR_SHAPE;
  try {
    for (int j = 0; j < num_hashes; ++j) {
      Block& b = p->blocks[s->blocks[j]];
      if (b.cached) continue;  // already registered (its own key)
      const Key key(reinterpret_cast<const char*>(hashes + 32 * j), 32);
      if (p->by_key.count(key)) continue;  // another block holds this computation
      p->by_key[key] = s->blocks[j];
      b.cached = true;
      b.key = key;
    }
  } catch (...) {
    return KVD_ERR_NOMEM;
  }
  return KVD_OK;
}

int kvd_seq_create_with_prefix(kvd_block_pool* p, const uint8_t* hashes, int num_hashes,
                               int* num_hit) {
  if (!p || !num_hit || (num_hashes > 0 && !hashes)) return KVD_ERR_NULL;
  if (num_hashes < 0) return KVD_ERR_SHAPE;
  int seq;
  try {
    seq = new_seq(p);
  } catch (...) {
    return KVD_ERR_NOMEM;
  }
  Seq& s = p->seqs[seq];
  int hit = 0;
  try {
    for (; hit < num_hashes; ++hit) {
      auto it = p->by_key.find(Key(reinterpret_cast<const char*>(hashes + 32 * hit), 32));
      if (it == p->by_key.end()) break;
      s.blocks.push_back(it->second);
      hold(p, it->second);
    }
  } catch (...) {
    for (int32_t id : s.blocks) drop(p, id);
    s = Seq();
    return KVD_ERR_NOMEM;
  }
  s.len = static_cast<int64_t>(hit) * p->block_size;
  *num_hit = hit;
  return seq;
}

}  // extern "C"
