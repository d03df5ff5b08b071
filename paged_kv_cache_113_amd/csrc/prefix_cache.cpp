// Prefix caching for the paged KV pool: host-side block identity and the
// cached block pool (control plane, no GPU work).
//
// What it implements, from the pages:
//  * block identity: SHA-256 over a full block's token ids and extra keys,
//    32 bytes ("vLLM source walkthrough: PagedAttention and continuous
//    batching", section 1.9). A block's identity must cover its whole prefix
//    (two blocks with equal tokens after different prefixes hold different
//    K/V), so each block's message starts with the previous block's hash
//    (32 zero bytes before the first block), then the tokens as
//    little-endian int32, then the extra keys;
//  * the block pool under prefix caching ("vLLM PagedAttention: from
//    fragmentation to slot mapping", block metadata and life cycle): per
//    block a reference count and an optional identity; the free queue is an
//    intrusive doubly linked list (O(1) take from the head, append at the
//    tail, unlink from the middle); a ref-0 block with an identity stays
//    hit-able in the queue; a hit takes it out of the queue (touch) and
//    counts a reference; a block taken for new data loses its identity
//    (evicted from the hash map); a block released to 0 goes to the tail
//    and keeps its identity;
//  * admission: the longest run of leading cached blocks, capped so that
//    the last token is recomputed (num_tokens - 1), is reused by reference;
//    the rest of the blocks are taken fresh (walkthrough page, sections 1.5
//    and 1.9).
//
// SHA-256 is written from its published definition (FIPS 180-4): the round
// constants are the first 32 fractional bits of the cube roots of the first
// 64 primes, the initial state those of the square roots of the first 8.
#include <array>
#include <cstring>
#include <new>
#include <unordered_map>
#include <vector>

#include "../../include/pagedkv.h"

namespace {

// ---- SHA-256 (FIPS 180-4) ------------------------------------------------------

constexpr uint32_t kRound[64] = {
    0x428a2f98u, 0x71374491u, 0xb5c0fbcfu, 0xe9b5dba5u,
    0x3956c25bu, 0x59f111f1u, 0x923f82a4u, 0xab1c5ed5u,
    0xd807aa98u, 0x12835b01u, 0x243185beu, 0x550c7dc3u,
    0x72be5d74u, 0x80deb1feu, 0x9bdc06a7u, 0xc19bf174u,
    0xe49b69c1u, 0xefbe4786u, 0x0fc19dc6u, 0x240ca1ccu,
    0x2de92c6fu, 0x4a7484aau, 0x5cb0a9dcu, 0x76f988dau,
    0x983e5152u, 0xa831c66du, 0xb00327c8u, 0xbf597fc7u,
    0xc6e00bf3u, 0xd5a79147u, 0x06ca6351u, 0x14292967u,
    0x27b70a85u, 0x2e1b2138u, 0x4d2c6dfcu, 0x53380d13u,
    0x650a7354u, 0x766a0abbu, 0x81c2c92eu, 0x92722c85u,
    0xa2bfe8a1u, 0xa81a664bu, 0xc24b8b70u, 0xc76c51a3u,
    0xd192e819u, 0xd6990624u, 0xf40e3585u, 0x106aa070u,
    0x19a4c116u, 0x1e376c08u, 0x2748774cu, 0x34b0bcb5u,
    0x391c0cb3u, 0x4ed8aa4au, 0x5b9cca4fu, 0x682e6ff3u,
    0x748f82eeu, 0x78a5636fu, 0x84c87814u, 0x8cc70208u,
    0x90befffau, 0xa4506cebu, 0xbef9a3f7u, 0xc67178f2u};
constexpr uint32_t kInit[8] = {
    0x6a09e667u, 0xbb67ae85u, 0x3c6ef372u, 0xa54ff53au,
    0x510e527fu, 0x9b05688cu, 0x1f83d9abu, 0x5be0cd19u};

inline uint32_t rotr(uint32_t x, int n) { return (x >> n) | (x << (32 - n)); }

struct Sha256 {
  uint32_t h[8];
  uint8_t buf[64];
  int fill = 0;
  uint64_t bytes = 0;

  Sha256() { std::memcpy(h, kInit, sizeof h); }

  void block(const uint8_t* p) {
    uint32_t w[64];
    for (int t = 0; t < 16; ++t)
      w[t] = (uint32_t(p[4 * t]) << 24) | (uint32_t(p[4 * t + 1]) << 16) |
             (uint32_t(p[4 * t + 2]) << 8) | uint32_t(p[4 * t + 3]);
    for (int t = 16; t < 64; ++t) {
      const uint32_t s0 = rotr(w[t - 15], 7) ^ rotr(w[t - 15], 18) ^ (w[t - 15] >> 3);
      const uint32_t s1 = rotr(w[t - 2], 17) ^ rotr(w[t - 2], 19) ^ (w[t - 2] >> 10);
      w[t] = w[t - 16] + s0 + w[t - 7] + s1;
    }
    uint32_t a = h[0], b = h[1], c = h[2], d = h[3], e = h[4], f = h[5], g = h[6], k = h[7];
    for (int t = 0; t < 64; ++t) {
      const uint32_t S1 = rotr(e, 6) ^ rotr(e, 11) ^ rotr(e, 25);
      const uint32_t ch = (e & f) ^ (~e & g);
      const uint32_t t1 = k + S1 + ch + kRound[t] + w[t];
      const uint32_t S0 = rotr(a, 2) ^ rotr(a, 13) ^ rotr(a, 22);
      const uint32_t mj = (a & b) ^ (a & c) ^ (b & c);
      const uint32_t t2 = S0 + mj;
      k = g;
      g = f;
      f = e;
      e = d + t1;
      d = c;
      c = b;
      b = a;
      a = t1 + t2;
    }
    h[0] += a; h[1] += b; h[2] += c; h[3] += d;
    h[4] += e; h[5] += f; h[6] += g; h[7] += k;
  }

  void update(const uint8_t* p, size_t n) {
    bytes += n;
    while (n > 0) {
      const size_t take = n < size_t(64 - fill) ? n : size_t(64 - fill);
      std::memcpy(buf + fill, p, take);
      fill += int(take);
      p += take;
      n -= take;
      if (fill == 64) {
        block(buf);
        fill = 0;
      }
    }
  }

  void digest(uint8_t* out) {
    const uint64_t bits = bytes * 8;
    const uint8_t one = 0x80, zero = 0;
    update(&one, 1);
    while (fill != 56) update(&zero, 1);
    uint8_t len[8];
    for (int i = 0; i < 8; ++i) len[i] = uint8_t(bits >> (56 - 8 * i));
    update(len, 8);
    for (int i = 0; i < 8; ++i) {
      out[4 * i] = uint8_t(h[i] >> 24);
      out[4 * i + 1] = uint8_t(h[i] >> 16);
      out[4 * i + 2] = uint8_t(h[i] >> 8);
      out[4 * i + 3] = uint8_t(h[i]);
    }
  }
};

// Hashes of the full blocks of `tokens`, block_size tokens each.
int64_t hash_blocks(uint8_t* out, const int32_t* tokens, int64_t n, int block_size,
                    const uint8_t* extra, int64_t extra_len) {
  const int64_t nb = n / block_size;
  uint8_t parent[32] = {0};
  std::vector<uint8_t> msg(static_cast<size_t>(block_size) * 4);
  for (int64_t b = 0; b < nb; ++b) {
    for (int i = 0; i < block_size; ++i) {
      const uint32_t t = static_cast<uint32_t>(tokens[b * block_size + i]);
      msg[4 * i] = uint8_t(t);
      msg[4 * i + 1] = uint8_t(t >> 8);
      msg[4 * i + 2] = uint8_t(t >> 16);
      msg[4 * i + 3] = uint8_t(t >> 24);
    }
    Sha256 s;
    s.update(parent, 32);
    s.update(msg.data(), msg.size());
    if (extra_len > 0) s.update(extra, static_cast<size_t>(extra_len));
    s.digest(out + 32 * b);
    std::memcpy(parent, out + 32 * b, 32);
  }
  return nb;
}

using Digest = std::array<uint8_t, 32>;
struct DigestHash {
  size_t operator()(const Digest& d) const {
    uint64_t x;
    std::memcpy(&x, d.data(), 8);  // SHA-256 output bits are uniform
    return static_cast<size_t>(x);
  }
};

}  // namespace

// ---- the cached block pool --------------------------------------------------------

struct pkv_block_pool {
  int num_blocks;
  int block_size;
  std::vector<int32_t> ref;
  std::vector<int32_t> prev, next;  // free queue links; -1 = none
  std::vector<uint8_t> queued;
  int32_t head = -1, tail = -1;
  int64_t nfree = 0;
  std::vector<Digest> ident;
  std::vector<uint8_t> has_ident;
  std::unordered_map<Digest, int32_t, DigestHash> map;

  void push_back(int32_t b) {
    prev[b] = tail;
    next[b] = -1;
    if (tail >= 0) next[tail] = b; else head = b;
    tail = b;
    queued[b] = 1;
    ++nfree;
  }
  void unlink(int32_t b) {
    if (prev[b] >= 0) next[prev[b]] = next[b]; else head = next[b];
    if (next[b] >= 0) prev[next[b]] = prev[b]; else tail = prev[b];
    prev[b] = next[b] = -1;
    queued[b] = 0;
    --nfree;
  }
  void evict(int32_t b) {
    if (has_ident[b]) {
      map.erase(ident[b]);
      has_ident[b] = 0;
    }
  }
};

namespace {

bool valid_block(const pkv_block_pool* p, int32_t b) { return b >= 0 && b < p->num_blocks; }

}  // namespace

extern "C" {

int64_t pkv_block_hashes(uint8_t* out, const int32_t* tokens, int64_t num_tokens, int block_size,
                         const uint8_t* extra, int64_t extra_len) {
  if (num_tokens < 0 || block_size < 1 || extra_len < 0) return PKV_ERR_SHAPE;
  if (num_tokens / block_size == 0) return 0;
  if (!out || !tokens || (extra_len > 0 && !extra)) return PKV_ERR_NULL;
  return hash_blocks(out, tokens, num_tokens, block_size, extra, extra_len);
}

int pkv_pool_create(pkv_block_pool** out, int num_blocks, int block_size,
                    const int32_t* initial_free) {
  if (!out) return PKV_ERR_NULL;
  *out = nullptr;
  if (num_blocks < 1 || block_size < 1) return PKV_ERR_SHAPE;
  if (initial_free) {  // must be a permutation of 0..num_blocks-1
    std::vector<uint8_t> seen(static_cast<size_t>(num_blocks), 0);
    for (int i = 0; i < num_blocks; ++i) {
      const int32_t b = initial_free[i];
      if (b < 0 || b >= num_blocks || seen[b]) return PKV_ERR_SHAPE;
      seen[b] = 1;
    }
  }
  pkv_block_pool* p = new (std::nothrow) pkv_block_pool();
  if (!p) return PKV_ERR_STATE;
  p->num_blocks = num_blocks;
  p->block_size = block_size;
  const size_t n = static_cast<size_t>(num_blocks);
  p->ref.assign(n, 0);
  p->prev.assign(n, -1);
  p->next.assign(n, -1);
  p->queued.assign(n, 0);
  p->ident.assign(n, Digest{});
  p->has_ident.assign(n, 0);
  for (int i = 0; i < num_blocks; ++i) p->push_back(initial_free ? initial_free[i] : i);
  *out = p;
  return PKV_OK;
}

void pkv_pool_destroy(pkv_block_pool* pool) { delete pool; }

int64_t pkv_pool_num_free(const pkv_block_pool* pool) {
  return pool ? pool->nfree : PKV_ERR_NULL;
}

int pkv_pool_longest_hit(const pkv_block_pool* pool, const uint8_t* hashes, int num_hashes,
                         int32_t* out_blocks) {
  if (!pool) return PKV_ERR_NULL;
  if (num_hashes < 0) return PKV_ERR_SHAPE;
  if (num_hashes == 0) return 0;
  if (!hashes || !out_blocks) return PKV_ERR_NULL;
  int k = 0;
  for (; k < num_hashes; ++k) {
    Digest d;
    std::memcpy(d.data(), hashes + 32 * static_cast<size_t>(k), 32);
    const auto it = pool->map.find(d);
    if (it == pool->map.end()) break;
    out_blocks[k] = it->second;
  }
  return k;
}

int pkv_pool_touch(pkv_block_pool* pool, const int32_t* blocks, int n) {
  if (!pool) return PKV_ERR_NULL;
  if (n < 0) return PKV_ERR_SHAPE;
  if (n > 0 && !blocks) return PKV_ERR_NULL;
  for (int i = 0; i < n; ++i)
    if (!valid_block(pool, blocks[i])) return PKV_ERR_SHAPE;
  for (int i = 0; i < n; ++i) {
    const int32_t b = blocks[i];
    if (pool->ref[b] == 0) pool->unlink(b);
    ++pool->ref[b];
  }
  return PKV_OK;
}

int pkv_pool_allocate(pkv_block_pool* pool, int n, int32_t* out_blocks) {
  if (!pool) return PKV_ERR_NULL;
  if (n < 0) return PKV_ERR_SHAPE;
  if (n == 0) return PKV_OK;
  if (!out_blocks) return PKV_ERR_NULL;
  if (n > pool->nfree) return PKV_ERR_CAPACITY;  // nothing taken
  for (int i = 0; i < n; ++i) {
    const int32_t b = pool->head;
    pool->unlink(b);
    pool->evict(b);
    pool->ref[b] = 1;
    out_blocks[i] = b;
  }
  return PKV_OK;
}

int pkv_pool_cache(pkv_block_pool* pool, int32_t block, const uint8_t* hash) {
  if (!pool || !hash) return PKV_ERR_NULL;
  if (!valid_block(pool, block)) return PKV_ERR_SHAPE;
  if (pool->ref[block] == 0) return PKV_ERR_STATE;  // only blocks in use get an identity
  if (pool->has_ident[block]) return 0;
  Digest d;
  std::memcpy(d.data(), hash, 32);
  if (pool->map.count(d)) return 0;  // the first block cached with a hash keeps it
  pool->map.emplace(d, block);
  pool->ident[block] = d;
  pool->has_ident[block] = 1;
  return 1;
}

int pkv_pool_release(pkv_block_pool* pool, const int32_t* blocks, int n) {
  if (!pool) return PKV_ERR_NULL;
  if (n < 0) return PKV_ERR_SHAPE;
  if (n > 0 && !blocks) return PKV_ERR_NULL;
  // check first, so that a bad call changes nothing: every block valid and
  // held at least as often as it is listed
  std::unordered_map<int32_t, int> count;
  for (int i = 0; i < n; ++i) {
    if (!valid_block(pool, blocks[i])) return PKV_ERR_SHAPE;
    if (++count[blocks[i]] > pool->ref[blocks[i]]) return PKV_ERR_STATE;
  }
  for (int i = 0; i < n; ++i) {
    const int32_t b = blocks[i];
    if (--pool->ref[b] == 0) pool->push_back(b);
  }
  return PKV_OK;
}

int pkv_pool_admit(pkv_block_pool* pool, const int32_t* tokens, int64_t num_tokens,
                   const uint8_t* extra, int64_t extra_len, int32_t* out_table,
                   int64_t* cached_tokens) {
  if (!pool) return PKV_ERR_NULL;
  if (num_tokens < 1 || extra_len < 0) return PKV_ERR_SHAPE;
  if (!tokens || !out_table || !cached_tokens || (extra_len > 0 && !extra)) return PKV_ERR_NULL;
  const int B = pool->block_size;
  const int64_t need_total = (num_tokens + B - 1) / B;
  if (need_total > 0x7fffffff) return PKV_ERR_SHAPE;
  // hashes of the blocks a hit may cover: full blocks before the last token
  const int64_t cap = (num_tokens - 1) / B;
  std::vector<uint8_t> h(static_cast<size_t>(cap) * 32 + 1);
  hash_blocks(h.data(), tokens, cap * B, B, extra, extra_len);
  int64_t hit = 0, revived = 0;
  for (; hit < cap; ++hit) {
    Digest d;
    std::memcpy(d.data(), h.data() + 32 * hit, 32);
    const auto it = pool->map.find(d);
    if (it == pool->map.end()) break;
    out_table[hit] = it->second;
    revived += pool->ref[it->second] == 0;
  }
  const int64_t fresh = need_total - hit;
  if (fresh > pool->nfree - revived) return PKV_ERR_CAPACITY;  // nothing changed
  for (int64_t i = 0; i < hit; ++i) {
    const int32_t b = out_table[i];
    if (pool->ref[b] == 0) pool->unlink(b);
    ++pool->ref[b];
  }
  for (int64_t i = hit; i < need_total; ++i) {
    const int32_t b = pool->head;
    pool->unlink(b);
    pool->evict(b);
    pool->ref[b] = 1;
    out_table[i] = b;
  }
  *cached_tokens = hit * B;
  return PKV_OK;
}

int pkv_pool_cache_full_blocks(pkv_block_pool* pool, const int32_t* table,
                               const int32_t* tokens, int64_t num_tokens, const uint8_t* extra,
                               int64_t extra_len) {
  if (!pool) return PKV_ERR_NULL;
  if (num_tokens < 0 || extra_len < 0) return PKV_ERR_SHAPE;
  const int64_t nb = num_tokens / pool->block_size;
  if (nb == 0) return PKV_OK;
  if (!table || !tokens || (extra_len > 0 && !extra)) return PKV_ERR_NULL;
  for (int64_t i = 0; i < nb; ++i) {
    if (!valid_block(pool, table[i])) return PKV_ERR_SHAPE;
    if (pool->ref[table[i]] == 0) return PKV_ERR_STATE;
  }
  std::vector<uint8_t> h(static_cast<size_t>(nb) * 32);
  hash_blocks(h.data(), tokens, num_tokens, pool->block_size, extra, extra_len);
  for (int64_t i = 0; i < nb; ++i)
    if (!pool->has_ident[table[i]]) pkv_pool_cache(pool, table[i], h.data() + 32 * i);
  return PKV_OK;
}

int pkv_pool_state(const pkv_block_pool* pool, int32_t* ref_out, int32_t* free_out,
                   uint8_t* cached_out) {
  if (!pool) return PKV_ERR_NULL;
  if (ref_out)
    for (int b = 0; b < pool->num_blocks; ++b) ref_out[b] = pool->ref[b];
  if (free_out) {
    int i = 0;
    for (int32_t b = pool->head; b >= 0; b = pool->next[b]) free_out[i++] = b;
  }
  if (cached_out)
    for (int b = 0; b < pool->num_blocks; ++b) cached_out[b] = pool->has_ident[b];
  return static_cast<int>(pool->nfree);
}

}  // extern "C"
