// Host KV block manager: block pool, reference counts, O(1) LRU free queue,
// prefix-hash chain and copy-on-write.  The behaviour and the pages that
// define it are stated in include/pagedkv_blocks.h.
//
// Data layout: per block a reference count, links of the doubly linked free
// queue (indices, -1 = none) and an optional 32-byte digest; a hash map from
// digest to block for the cached full blocks; a hash map from request id to
// its token ids, block table and hashing cursor.  Every operation is O(1)
// per block it touches, plus one SHA-256 per block it hashes.

#include <algorithm>
#include <array>
#include <cmath>
#include <cpuid.h>
#include <cstdlib>
#include <immintrin.h>
#include <cstring>
#include <new>
#include <string>
#include <unordered_map>
#include <vector>

#include "pagedkv.h"
#include "pagedkv_blocks.h"

namespace {

// ---------------------------------------------------------------------------
// SHA-256, FIPS 180-4.  The round constants are the first 32 bits of the
// fractional parts of the cube roots of the first 64 primes, the initial hash
// the same of the square roots of the first 8 primes: computed here from that
// definition.

struct Sha256Constants {
  uint32_t k[64];
  uint32_t h0[8];
  Sha256Constants() {
    int primes[64];
    int n = 0;
    for (int c = 2; n < 64; ++c) {
      bool prime = true;
      for (int d = 2; d * d <= c; ++d)
        if (c % d == 0) {
          prime = false;
          break;
        }
      if (prime) primes[n++] = c;
    }
    for (int i = 0; i < 64; ++i) k[i] = frac32(std::cbrt(static_cast<long double>(primes[i])));
    for (int i = 0; i < 8; ++i) h0[i] = frac32(std::sqrt(static_cast<long double>(primes[i])));
  }
  static uint32_t frac32(long double x) {
    const long double f = x - std::floor(x);
    return static_cast<uint32_t>(std::floor(std::ldexp(f, 32)));
  }
};

const Sha256Constants& sha_constants() {
  static const Sha256Constants c;
  return c;
}

inline uint32_t rotr(uint32_t x, int n) { return (x >> n) | (x << (32 - n)); }

void sha256_block(uint32_t* h, const uint8_t* p, const uint32_t* k) {
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
    const uint32_t S1 = rotr(e, 6) ^ rotr(e, 11) ^ rotr(e, 25);
    const uint32_t ch = (e & f) ^ (~e & g);
    const uint32_t t1 = hh + S1 + ch + k[i] + w[i];
    const uint32_t S0 = rotr(a, 2) ^ rotr(a, 13) ^ rotr(a, 22);
    const uint32_t maj = (a & b) ^ (a & c) ^ (b & c);
    const uint32_t t2 = S0 + maj;
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

// The same compression with the x86 SHA extensions: the state lives in two
// registers as (A, B, E, F) and (C, D, G, H); sha256rnds2 performs two rounds,
// sha256msg1 / sha256msg2 the two halves of the message schedule.
__attribute__((target("sha,sse4.1"))) void sha256_blocks_x86(uint32_t* h, const uint8_t* p,
                                                              size_t nblocks,
                                                              const uint32_t* k) {
  const __m128i swap = _mm_set_epi64x(0x0c0d0e0f08090a0bULL, 0x0405060700010203ULL);
  __m128i dcba = _mm_loadu_si128(reinterpret_cast<const __m128i*>(h));
  __m128i hgfe = _mm_loadu_si128(reinterpret_cast<const __m128i*>(h + 4));
  const __m128i cdab = _mm_shuffle_epi32(dcba, 0xB1);
  const __m128i efgh = _mm_shuffle_epi32(hgfe, 0x1B);
  __m128i abef = _mm_alignr_epi8(cdab, efgh, 8);
  __m128i cdgh = _mm_blend_epi16(efgh, cdab, 0xF0);
  for (size_t blk = 0; blk < nblocks; ++blk, p += 64) {
    const __m128i abef0 = abef, cdgh0 = cdgh;
    __m128i w[4];
#pragma GCC unroll 16
    for (int g = 0; g < 16; ++g) {
      __m128i wg;
      if (g < 4) {
        wg = _mm_shuffle_epi8(_mm_loadu_si128(reinterpret_cast<const __m128i*>(p + 16 * g)), swap);
      } else {
        const __m128i a = _mm_sha256msg1_epu32(w[g % 4], w[(g + 1) % 4]);       // W[g-4], W[g-3]
        const __m128i b = _mm_alignr_epi8(w[(g + 3) % 4], w[(g + 2) % 4], 4);   // W[g-1], W[g-2]
        wg = _mm_sha256msg2_epu32(_mm_add_epi32(a, b), w[(g + 3) % 4]);
      }
      w[g % 4] = wg;
      __m128i m = _mm_add_epi32(wg, _mm_loadu_si128(reinterpret_cast<const __m128i*>(k + 4 * g)));
      cdgh = _mm_sha256rnds2_epu32(cdgh, abef, m);
      m = _mm_shuffle_epi32(m, 0x0E);
      abef = _mm_sha256rnds2_epu32(abef, cdgh, m);
    }
    abef = _mm_add_epi32(abef, abef0);
    cdgh = _mm_add_epi32(cdgh, cdgh0);
  }
  const __m128i feba = _mm_shuffle_epi32(abef, 0x1B);
  const __m128i dchg = _mm_shuffle_epi32(cdgh, 0xB1);
  _mm_storeu_si128(reinterpret_cast<__m128i*>(h), _mm_blend_epi16(feba, dchg, 0xF0));
  _mm_storeu_si128(reinterpret_cast<__m128i*>(h + 4), _mm_alignr_epi8(dchg, feba, 8));
}

// The extensions are used when the CPU reports them (CPUID leaf 7, EBX bit
// 29), unless PKV_SHA256_PORTABLE is set in the environment.
bool cpu_has_sha() {
  static const bool has = [] {
    const char* portable = std::getenv("PKV_SHA256_PORTABLE");
    if (portable && *portable && *portable != '0') return false;
    unsigned a = 0, b = 0, c = 0, d = 0;
    return __get_cpuid_count(7, 0, &a, &b, &c, &d) && (b & (1u << 29)) != 0;
  }();
  return has;
}

void compress(uint32_t* h, const uint8_t* p, size_t nblocks, const uint32_t* k) {
  if (cpu_has_sha()) {
    sha256_blocks_x86(h, p, nblocks, k);
    return;
  }
  for (size_t b = 0; b < nblocks; ++b) sha256_block(h, p + 64 * b, k);
}

void sha256(const uint8_t* data, size_t len, uint8_t* out) {
  const Sha256Constants& c = sha_constants();
  uint32_t h[8];
  std::memcpy(h, c.h0, sizeof(h));
  size_t i = len / 64 * 64;
  compress(h, data, len / 64, c.k);
  // padding: 0x80, zeros, then the bit length as a big-endian 64-bit number
  uint8_t tail[128] = {0};
  const size_t rest = len - i;
  if (rest) std::memcpy(tail, data + i, rest);
  tail[rest] = 0x80;
  const size_t tail_len = rest + 9 <= 64 ? 64 : 128;
  const uint64_t bits = uint64_t(len) * 8;
  for (int b = 0; b < 8; ++b) tail[tail_len - 1 - b] = uint8_t(bits >> (8 * b));
  compress(h, tail, tail_len / 64, c.k);
  for (int j = 0; j < 8; ++j) {
    out[4 * j] = uint8_t(h[j] >> 24);
    out[4 * j + 1] = uint8_t(h[j] >> 16);
    out[4 * j + 2] = uint8_t(h[j] >> 8);
    out[4 * j + 3] = uint8_t(h[j]);
  }
}

// ---------------------------------------------------------------------------

constexpr int kBlock = PKV_BLOCK_SIZE;
using Digest = std::array<uint8_t, 32>;

struct DigestHasher {
  size_t operator()(const Digest& d) const {
    size_t v;
    std::memcpy(&v, d.data(), sizeof(v));   // a SHA-256 prefix is already uniform
    return v;
  }
};

void put_u32(std::string& s, uint32_t v) {
  for (int b = 0; b < 4; ++b) s.push_back(char(uint8_t(v >> (8 * b))));
}

Digest hash_block(const Digest& parent, const int32_t* tokens, const std::string& extra,
                  const std::string& salt) {
  std::string msg;
  msg.reserve(32 + 4 * kBlock + 8 + extra.size() + salt.size());
  msg.append(reinterpret_cast<const char*>(parent.data()), 32);
  for (int i = 0; i < kBlock; ++i) put_u32(msg, uint32_t(tokens[i]));
  put_u32(msg, uint32_t(extra.size()));
  msg += extra;
  put_u32(msg, uint32_t(salt.size()));
  msg += salt;
  Digest d;
  sha256(reinterpret_cast<const uint8_t*>(msg.data()), msg.size(), d.data());
  return d;
}

struct Request {
  std::vector<int32_t> tokens;   // known token ids: prompt + appended
  std::vector<int32_t> table;    // logical block -> physical block
  std::string extra, salt;
  int32_t num_tokens = 0;        // positions that own a slot
  int32_t hashed = 0;            // leading blocks whose hash is known
  Digest parent{};               // hash of block hashed - 1 (zeros before any)
};

}  // namespace

struct pkv_block_manager {
  int32_t num_blocks = 0;
  bool prefix_caching = true;
  std::vector<int32_t> ref, prev, next;
  std::vector<uint8_t> in_queue, hashed;
  std::vector<Digest> digest;
  int32_t head = -1, tail = -1, free_count = 0;
  std::unordered_map<Digest, int32_t, DigestHasher> cached;
  std::unordered_map<int64_t, Request> requests;
  std::vector<int64_t> copies;   // pending (src, dst) pairs, flattened

  // ---- the free queue
  void push_tail(int32_t b) {
    prev[b] = tail;
    next[b] = -1;
    if (tail >= 0) next[tail] = b; else head = b;
    tail = b;
    in_queue[b] = 1;
    ++free_count;
  }
  void unlink(int32_t b) {
    if (prev[b] >= 0) next[prev[b]] = next[b]; else head = next[b];
    if (next[b] >= 0) prev[next[b]] = prev[b]; else tail = prev[b];
    prev[b] = next[b] = -1;
    in_queue[b] = 0;
    --free_count;
  }
  int32_t take_free() {
    const int32_t b = head;
    unlink(b);
    if (hashed[b]) {             // reuse ends its life as a cached block
      cached.erase(digest[b]);
      hashed[b] = 0;
    }
    ref[b] = 1;
    return b;
  }
  void release(int32_t b) {
    if (--ref[b] == 0) push_tail(b);
  }

  Digest block_digest(const Request& r, int32_t j) const {
    static const std::string kNoSalt;
    return hash_block(r.parent, r.tokens.data() + int64_t(j) * kBlock, r.extra,
                      j == 0 ? r.salt : kNoSalt);
  }
};

namespace {

Request* find(pkv_block_manager* m, int64_t id) {
  auto it = m->requests.find(id);
  return it == m->requests.end() ? nullptr : &it->second;
}
const Request* find(const pkv_block_manager* m, int64_t id) {
  auto it = m->requests.find(id);
  return it == m->requests.end() ? nullptr : &it->second;
}

}  // namespace

extern "C" pkv_status pkv_bm_create(int32_t num_blocks, const int32_t* initial_order,
                                    int32_t prefix_caching, pkv_block_manager** manager) {
  if (!manager) return PKV_ERR_NULL;
  *manager = nullptr;
  if (num_blocks < 0) return PKV_ERR_SHAPE;
  pkv_block_manager* m = new (std::nothrow) pkv_block_manager;
  if (!m) return PKV_ERR_SHAPE;
  try {
    m->num_blocks = num_blocks;
    m->prefix_caching = prefix_caching != 0;
    m->ref.assign(num_blocks, 0);
    m->prev.assign(num_blocks, -1);
    m->next.assign(num_blocks, -1);
    m->in_queue.assign(num_blocks, 0);
    m->hashed.assign(num_blocks, 0);
    m->digest.assign(num_blocks, Digest{});
  } catch (...) {
    delete m;
    return PKV_ERR_SHAPE;
  }
  for (int32_t i = 0; i < num_blocks; ++i) {
    const int32_t b = initial_order ? initial_order[i] : i;
    if (b < 0 || b >= num_blocks || m->in_queue[b]) {
      delete m;
      return PKV_ERR_SHAPE;
    }
    m->push_tail(b);
  }
  *manager = m;
  return PKV_OK;
}

extern "C" void pkv_bm_destroy(pkv_block_manager* manager) { delete manager; }

extern "C" pkv_status pkv_bm_add_request(pkv_block_manager* m, int64_t id, const int32_t* prompt,
                                         int32_t n, const uint8_t* extra, int32_t extra_len,
                                         const uint8_t* salt, int32_t salt_len,
                                         int32_t* num_cached_tokens) {
  if (!m || !num_cached_tokens || (n > 0 && !prompt) || (extra_len > 0 && !extra) ||
      (salt_len > 0 && !salt))
    return PKV_ERR_NULL;
  if (n < 0 || extra_len < 0 || salt_len < 0) return PKV_ERR_SHAPE;
  if (m->requests.count(id)) return PKV_ERR_REQUEST;
  Request r;
  r.tokens.assign(prompt, prompt + n);
  if (extra_len > 0) r.extra.assign(reinterpret_cast<const char*>(extra), size_t(extra_len));
  if (salt_len > 0) r.salt.assign(reinterpret_cast<const char*>(salt), size_t(salt_len));
  if (m->prefix_caching) {
    for (int32_t j = 0; j < n / kBlock; ++j) {
      const Digest d = m->block_digest(r, j);
      auto it = m->cached.find(d);
      if (it == m->cached.end()) break;
      const int32_t b = it->second;
      if (m->ref[b] == 0) m->unlink(b);
      ++m->ref[b];
      r.table.push_back(b);
      r.parent = d;
      r.hashed = j + 1;
    }
  }
  r.num_tokens = int32_t(r.table.size()) * kBlock;
  *num_cached_tokens = r.num_tokens;
  m->requests.emplace(id, std::move(r));
  return PKV_OK;
}

extern "C" pkv_status pkv_bm_append_tokens(pkv_block_manager* m, int64_t id,
                                           const int32_t* tokens, int32_t n) {
  if (!m || (n > 0 && !tokens)) return PKV_ERR_NULL;
  if (n < 0) return PKV_ERR_SHAPE;
  Request* r = find(m, id);
  if (!r) return PKV_ERR_REQUEST;
  r->tokens.insert(r->tokens.end(), tokens, tokens + n);
  return PKV_OK;
}

extern "C" pkv_status pkv_bm_allocate(pkv_block_manager* m, int64_t id, int32_t num_new) {
  if (!m) return PKV_ERR_NULL;
  Request* r = find(m, id);
  if (!r) return PKV_ERR_REQUEST;
  if (num_new < 0) return PKV_ERR_SHAPE;
  const int64_t first = r->num_tokens, end = first + num_new;
  if (end > int64_t(r->tokens.size())) return PKV_ERR_SHAPE;
  if (num_new == 0) return PKV_OK;
  const int64_t blocks_after = (end + kBlock - 1) / kBlock;
  const int64_t need = std::max<int64_t>(0, blocks_after - int64_t(r->table.size()));
  // shared blocks in the written range (only existing table entries)
  const int64_t j_end = std::min<int64_t>((end - 1) / kBlock, int64_t(r->table.size()) - 1);
  int64_t shared = 0;
  for (int64_t j = first / kBlock; j <= j_end; ++j) shared += m->ref[r->table[j]] > 1;
  if (need + shared > m->free_count) return PKV_ERR_NO_BLOCKS;
  for (int64_t j = first / kBlock; j <= j_end; ++j) {
    const int32_t src = r->table[j];
    if (m->ref[src] <= 1) continue;
    const int32_t dst = m->take_free();
    m->copies.push_back(src);
    m->copies.push_back(dst);
    m->release(src);
    r->table[j] = dst;
  }
  for (int64_t i = 0; i < need; ++i) r->table.push_back(m->take_free());
  r->num_tokens = int32_t(end);
  if (m->prefix_caching) {
    for (int32_t j = r->hashed; j < int32_t(end / kBlock); ++j) {
      const Digest d = m->block_digest(*r, j);
      const int32_t b = r->table[j];
      if (!m->hashed[b] && m->cached.emplace(d, b).second) {
        m->digest[b] = d;
        m->hashed[b] = 1;
      }
      r->parent = d;
      r->hashed = j + 1;
    }
  }
  return PKV_OK;
}

extern "C" pkv_status pkv_bm_append_tokens_batch(pkv_block_manager* m, const int64_t* ids,
                                                 const int32_t* tokens, int32_t n) {
  if (!m || (n > 0 && (!ids || !tokens))) return PKV_ERR_NULL;
  if (n < 0) return PKV_ERR_SHAPE;
  for (int32_t i = 0; i < n; ++i)
    if (!find(m, ids[i])) return PKV_ERR_REQUEST;
  for (int32_t i = 0; i < n; ++i) find(m, ids[i])->tokens.push_back(tokens[i]);
  return PKV_OK;
}

extern "C" pkv_status pkv_bm_allocate_batch(pkv_block_manager* m, const int64_t* ids,
                                            const int32_t* num_new, int32_t n,
                                            pkv_status* status) {
  if (!m || (n > 0 && (!ids || !num_new || !status))) return PKV_ERR_NULL;
  if (n < 0) return PKV_ERR_SHAPE;
  for (int32_t i = 0; i < n; ++i) status[i] = pkv_bm_allocate(m, ids[i], num_new[i]);
  return PKV_OK;
}

extern "C" pkv_status pkv_bm_fork(pkv_block_manager* m, int64_t parent_id, int64_t child_id) {
  if (!m) return PKV_ERR_NULL;
  const Request* p = find(m, parent_id);
  if (!p || m->requests.count(child_id)) return PKV_ERR_REQUEST;
  Request c = *p;
  for (int32_t b : c.table) ++m->ref[b];
  m->requests.emplace(child_id, std::move(c));
  return PKV_OK;
}

extern "C" pkv_status pkv_bm_free_request(pkv_block_manager* m, int64_t id) {
  if (!m) return PKV_ERR_NULL;
  auto it = m->requests.find(id);
  if (it == m->requests.end()) return PKV_ERR_REQUEST;
  const std::vector<int32_t>& t = it->second.table;
  for (auto b = t.rbegin(); b != t.rend(); ++b) m->release(*b);
  m->requests.erase(it);
  return PKV_OK;
}

extern "C" int32_t pkv_bm_num_free(const pkv_block_manager* m) { return m ? m->free_count : -1; }

extern "C" int32_t pkv_bm_num_tokens(const pkv_block_manager* m, int64_t id) {
  const Request* r = m ? find(m, id) : nullptr;
  return r ? r->num_tokens : -1;
}

extern "C" int32_t pkv_bm_ref_count(const pkv_block_manager* m, int32_t block) {
  if (!m || block < 0 || block >= m->num_blocks) return -1;
  return m->ref[block];
}

extern "C" int32_t pkv_bm_table(const pkv_block_manager* m, int64_t id, int32_t* out,
                                int32_t capacity) {
  const Request* r = m ? find(m, id) : nullptr;
  if (!r) return -1;
  const int32_t n = int32_t(r->table.size());
  if (out)
    for (int32_t i = 0; i < std::min(n, capacity); ++i) out[i] = r->table[i];
  return n;
}

extern "C" int32_t pkv_bm_free_queue(const pkv_block_manager* m, int32_t* out, int32_t capacity) {
  if (!m) return -1;
  int32_t i = 0;
  for (int32_t b = m->head; b >= 0; b = m->next[b], ++i)
    if (out && i < capacity) out[i] = b;
  return i;
}

extern "C" int32_t pkv_bm_take_copies(pkv_block_manager* m, int64_t* pairs, int32_t capacity) {
  if (!m) return -1;
  const int32_t n = int32_t(m->copies.size() / 2);
  if (n > capacity || (n > 0 && !pairs)) return -n;
  std::copy(m->copies.begin(), m->copies.end(), pairs);
  m->copies.clear();
  return n;
}

extern "C" pkv_status pkv_bm_export_tables(const pkv_block_manager* m, const int64_t* ids,
                                           int32_t num, int32_t* tables, int32_t width,
                                           int32_t pad) {
  if (!m || (num > 0 && (!ids || !tables))) return PKV_ERR_NULL;
  if (num < 0 || width < 0) return PKV_ERR_SHAPE;
  for (int32_t i = 0; i < num; ++i) {
    const Request* r = find(m, ids[i]);
    if (!r) return PKV_ERR_REQUEST;
    if (int64_t(r->table.size()) > width) return PKV_ERR_SHAPE;
  }
  for (int32_t i = 0; i < num; ++i) {
    const Request* r = find(m, ids[i]);
    int32_t* row = tables + int64_t(i) * width;
    const int32_t n = int32_t(r->table.size());
    std::copy(r->table.begin(), r->table.end(), row);
    std::fill(row + n, row + width, pad);
  }
  return PKV_OK;
}

extern "C" void pkv_block_hash(const uint8_t* parent, const int32_t* tokens,
                               const uint8_t* extra, int32_t extra_len, const uint8_t* salt,
                               int32_t salt_len, uint8_t* digest) {
  Digest p;
  std::memcpy(p.data(), parent, 32);
  std::string e, s;
  if (extra_len > 0) e.assign(reinterpret_cast<const char*>(extra), size_t(extra_len));
  if (salt_len > 0) s.assign(reinterpret_cast<const char*>(salt), size_t(salt_len));
  const Digest d = hash_block(p, tokens, e, s);
  std::memcpy(digest, d.data(), 32);
}

extern "C" void pkv_sha256(const uint8_t* data, size_t len, uint8_t* digest) {
  sha256(data, len, digest);
}
