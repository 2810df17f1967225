// Host-side driver run under AddressSanitizer and UndefinedBehaviorSanitizer
// (tests/test_host_sanitize.py builds it with the library's sources, the
// sanitizers on the host code only, and runs it on the CPU).
//
// Part 1: every C-ABI entry point's host-side argument checks, each call with
// one argument wrong (null, misaligned, out-of-range size, unsupported
// dtype, arithmetic that would overflow), so that every call returns an
// error before anything is launched; fake device addresses are never
// dereferenced on the host.  Run only where no GPU is visible.
// Part 2: the host block manager on a seeded random workload of requests
// sharing prefixes, forks, appends, allocations, copy-on-write and frees,
// with its invariants checked after every operation, and its error paths.
// Part 3: SHA-256 on the FIPS 180-4 examples.
//
// Exit status 0 when every check held; a sanitizer report aborts the run.

#include <algorithm>
#include <cstdint>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <iterator>
#include <map>
#include <random>
#include <vector>

#include <hip/hip_runtime_api.h>

#include "pagedkv.h"
#include "pagedkv_blocks.h"

static int failures = 0;
#define CHECK(cond)                                                            \
  do {                                                                         \
    if (!(cond)) {                                                             \
      std::fprintf(stderr, "check failed at line %d: %s\n", __LINE__, #cond); \
      ++failures;                                                              \
    }                                                                          \
  } while (0)

static void* dev(uintptr_t a) { return reinterpret_cast<void*>(a); }
template <typename T>
static T* devp(uintptr_t a) { return reinterpret_cast<T*>(a); }

// ---------------------------------------------------------------- part 1

static void abi_checks() {
  const uintptr_t p = 0x100000, odd = 0x100008, odd4 = 0x100004;
  const int OK = PKV_OK;
  CHECK(pkv_block_size() == 16);
  CHECK(kv_bytes_per_token(32, 8, 128, 2) == 131072);
  CHECK(kv_bytes_per_token(-1, 8, 128, 2) == -1);
  CHECK(kv_bytes_per_token(1 << 30, 1 << 30, 128, 2) == -1);   // overflows int64 arithmetic
  for (int c = -3; c < 12; ++c) CHECK(pkv_status_string(static_cast<pkv_status>(c)) != nullptr);

  // slot mapping
  CHECK(compute_slot_mapping(nullptr, 4, nullptr, nullptr, 2, 10, nullptr, 5, nullptr) == PKV_ERR_NULL);
  CHECK(compute_slot_mapping(devp<int32_t>(p), 4, devp<int32_t>(p), devp<int32_t>(p), -1, 10,
                             devp<int64_t>(p), 5, nullptr) == PKV_ERR_SHAPE);
  CHECK(compute_slot_mapping(devp<int32_t>(p), 4, devp<int32_t>(p), devp<int32_t>(p), 2, 10,
                             devp<int64_t>(odd4), 5, nullptr) == PKV_ERR_ALIGN);
  CHECK(compute_slot_mapping(devp<int32_t>(p), -4, devp<int32_t>(p), devp<int32_t>(p), 2, 10,
                             devp<int64_t>(p), 5, nullptr) == PKV_ERR_SHAPE);

  // reshape_and_cache
  CHECK(reshape_and_cache(nullptr, dev(p), dev(p), dev(p), devp<int64_t>(p), 3, 2, 64, 10,
                          PKV_BF16, PKV_BF16, 1.f, 1.f, nullptr) == PKV_ERR_NULL);
  CHECK(reshape_and_cache(dev(odd), dev(p), dev(p), dev(p), devp<int64_t>(p), 3, 2, 64, 10,
                          PKV_BF16, PKV_BF16, 1.f, 1.f, nullptr) == PKV_ERR_ALIGN);
  CHECK(reshape_and_cache(dev(p), dev(p), dev(p), dev(p), devp<int64_t>(p), 3, 2, 60, 10,
                          PKV_BF16, PKV_BF16, 1.f, 1.f, nullptr) == PKV_ERR_UNSUPPORTED);
  CHECK(reshape_and_cache(dev(p), dev(p), dev(p), dev(p), devp<int64_t>(p), -1, 2, 64, 10,
                          PKV_BF16, PKV_BF16, 1.f, 1.f, nullptr) == PKV_ERR_SHAPE);
  CHECK(reshape_and_cache(dev(p), dev(p), dev(p), dev(p), devp<int64_t>(p), 3, 2, 64, 10,
                          PKV_BF16, PKV_FP8_E4M3, 0.f, 1.f, nullptr) == PKV_ERR_SHAPE);
  CHECK(reshape_and_cache(dev(p), dev(p), dev(p), dev(p), devp<int64_t>(p), 3, 2, 64, 10,
                          PKV_FP8_E4M3, PKV_FP8_E4M3, 1.f, 1.f, nullptr) == PKV_ERR_UNSUPPORTED);
  CHECK(reshape_and_cache(dev(p), dev(p), dev(p), dev(p), devp<int64_t>(p), 0, 2, 64, 10,
                          PKV_BF16, PKV_BF16, 1.f, 1.f, nullptr) == OK);

  // copy_blocks / swap_blocks: host arrays of device pointers
  void* arr[1] = {dev(p)};
  void* bad[1] = {dev(odd)};
  void* nul[1] = {nullptr};
  CHECK(copy_blocks(arr, arr, 1, devp<int64_t>(p), 2, 10, 4095, nullptr) == PKV_ERR_SHAPE);
  CHECK(copy_blocks(nullptr, arr, 1, devp<int64_t>(p), 2, 10, 4096, nullptr) == PKV_ERR_NULL);
  CHECK(copy_blocks(bad, arr, 1, devp<int64_t>(p), 2, 10, 4096, nullptr) == PKV_ERR_ALIGN);
  CHECK(copy_blocks(nul, arr, 1, devp<int64_t>(p), 2, 10, 4096, nullptr) == PKV_ERR_NULL);
  CHECK(copy_blocks(arr, arr, 1, devp<int64_t>(p), 0, 10, 4096, nullptr) == OK);
  CHECK(swap_blocks(arr, arr, arr, arr, 1, devp<int64_t>(p), 2, 10, 10, 4095, nullptr) ==
        PKV_ERR_SHAPE);
  CHECK(swap_blocks(arr, arr, nullptr, arr, 1, devp<int64_t>(p), 2, 10, 10, 4096, nullptr) ==
        PKV_ERR_NULL);
  CHECK(swap_blocks(arr, arr, bad, arr, 1, devp<int64_t>(p), 2, 10, 10, 4096, nullptr) ==
        PKV_ERR_ALIGN);
  CHECK(swap_blocks(arr, nul, arr, arr, 1, devp<int64_t>(p), 2, 10, 10, 4096, nullptr) ==
        PKV_ERR_NULL);

  // decode and its variants
  const size_t need = paged_attention_decode_workspace_size(4, 32, 8, 128, 1000, 0);
  CHECK(need > 0);
  CHECK(paged_attention_decode_workspace_size(4, 30, 8, 128, 1000, 0) == 0);
  CHECK(paged_attention_decode_workspace_size(4, 32, 8, 128, 1000, 40) == 0);
  CHECK(paged_attention_decode_num_chunks(4, 32, 8, 1000, -16) == -1);
  auto decode = [&](void* out, int32_t hq, int32_t d, pkv_dtype qd, pkv_dtype kvd, int32_t maxb,
                    int32_t part, size_t wsb, float ks) {
    return paged_attention_decode(out, dev(p), dev(p), dev(p), 100, devp<int32_t>(p), maxb,
                                  devp<int32_t>(p), 4, 1000, hq, 8, d, 0.088f, qd, kvd, ks, 1.f,
                                  part, dev(p), wsb, nullptr);
  };
  CHECK(decode(nullptr, 32, 128, PKV_BF16, PKV_BF16, 64, 0, need, 1.f) == PKV_ERR_NULL);
  CHECK(decode(dev(odd), 32, 128, PKV_BF16, PKV_BF16, 64, 0, need, 1.f) == PKV_ERR_ALIGN);
  CHECK(decode(dev(p), 30, 128, PKV_BF16, PKV_BF16, 64, 0, need, 1.f) == PKV_ERR_SHAPE);
  CHECK(decode(dev(p), 72, 128, PKV_BF16, PKV_BF16, 64, 0, need, 1.f) == PKV_ERR_UNSUPPORTED);
  CHECK(decode(dev(p), 32, 96, PKV_BF16, PKV_BF16, 64, 0, need, 1.f) == PKV_ERR_UNSUPPORTED);
  CHECK(decode(dev(p), 32, 128, PKV_F32, PKV_BF16, 64, 0, need, 1.f) == PKV_ERR_UNSUPPORTED);
  CHECK(decode(dev(p), 32, 128, PKV_BF16, PKV_BF16, 10, 0, need, 1.f) == PKV_ERR_SHAPE);
  CHECK(decode(dev(p), 32, 128, PKV_BF16, PKV_BF16, 64, 100, need, 1.f) == PKV_ERR_SHAPE);
  CHECK(decode(dev(p), 32, 128, PKV_BF16, PKV_BF16, 64, 0, need - 1, 1.f) == PKV_ERR_WORKSPACE);
  CHECK(decode(dev(p), 32, 128, PKV_BF16, PKV_FP8_E4M3, 64, 0, need, 0.f) == PKV_ERR_SHAPE);
  CHECK(paged_attention_decode_sliding(dev(p), dev(p), dev(p), dev(p), 100, devp<int32_t>(p), 63,
                                       devp<int32_t>(p), 4, 1000, 32, 8, 128, 0.088f, PKV_BF16,
                                       PKV_BF16, 1.f, 1.f, 0, 0, dev(p), need, nullptr) ==
        PKV_ERR_SHAPE);
  CHECK(paged_attention_decode_append(dev(p), dev(p), nullptr, dev(p), dev(p), dev(p), 100,
                                      devp<int32_t>(p), 63, devp<int32_t>(p), 4, 1000, 32, 8, 128,
                                      0.088f, PKV_BF16, PKV_BF16, 1.f, 1.f, 0, dev(p), need,
                                      nullptr) == PKV_ERR_NULL);
  CHECK(paged_attention_decode_append(dev(p), dev(p), dev(p), dev(p), dev(p), dev(p), 100,
                                      devp<int32_t>(p), 63, devp<int32_t>(p), 4, 1000, 32, 8, 128,
                                      0.088f, PKV_F32, PKV_F32, 1.f, 1.f, 0, dev(p), need,
                                      nullptr) == PKV_ERR_UNSUPPORTED);
  // the allocation-free variant refuses a split beyond its array before any
  // device call
  CHECK(paged_attention_decode_noalloc(dev(p), dev(p), dev(p), dev(p), 100, devp<int32_t>(p),
                                       1 << 20, devp<int32_t>(p), 1, 1 << 24, 64, 8, 128, 0.088f,
                                       PKV_BF16, PKV_BF16, 1.f, 1.f, 16, nullptr) ==
        PKV_ERR_WORKSPACE);
  CHECK(paged_attention_decode_noalloc(dev(p), dev(p), dev(p), dev(p), 100, devp<int32_t>(p),
                                       64, devp<int32_t>(p), 1, 1000, 64, 8, 128, 0.088f,
                                       PKV_BF16, PKV_BF16, 1.f, 1.f, 24, nullptr) ==
        PKV_ERR_SHAPE);

  // prefill chunk and the unified launch
  CHECK(paged_attention_prefill_chunk(nullptr, dev(p), dev(p), dev(p), 100, devp<int32_t>(p), 64,
                                      devp<int32_t>(p), devp<int32_t>(p), 3, 50, 20, 32, 8, 128,
                                      0.088f, PKV_BF16, PKV_BF16, 1.f, 1.f, nullptr) ==
        PKV_ERR_NULL);
  CHECK(paged_attention_prefill_chunk(dev(p), dev(p), dev(p), dev(p), 100, devp<int32_t>(p), 64,
                                      devp<int32_t>(p), devp<int32_t>(p), -3, 50, 20, 32, 8, 128,
                                      0.088f, PKV_BF16, PKV_BF16, 1.f, 1.f, nullptr) ==
        PKV_ERR_SHAPE);
  CHECK(paged_attention_prefill_chunk(dev(p), dev(p), dev(p), dev(p), 100, devp<int32_t>(p), 64,
                                      devp<int32_t>(p), devp<int32_t>(p), 3, 50, 20, 32, 8, 80,
                                      0.088f, PKV_BF16, PKV_BF16, 1.f, 1.f, nullptr) ==
        PKV_ERR_UNSUPPORTED);
  const size_t vneed = paged_attention_varlen_workspace_size(3, 50, 8, 128, 2000);
  CHECK(vneed > 0);
  CHECK(paged_attention_varlen_workspace_size(3, -1, 8, 128, 2000) == 0);
  CHECK(paged_attention_varlen(dev(p), dev(p), dev(p), dev(p), 100, devp<int32_t>(p), 125,
                               devp<int32_t>(p), devp<int32_t>(p), 3, 50, 2000, 32, 8, 128,
                               0.088f, PKV_BF16, PKV_BF16, dev(p), vneed - 1, nullptr) ==
        PKV_ERR_WORKSPACE);
  CHECK(paged_attention_varlen(dev(p), dev(p), dev(p), dev(p), 100, devp<int32_t>(p), 125,
                               devp<int32_t>(p), devp<int32_t>(p), 3, 50, 2000, 32, 8, 128,
                               0.088f, PKV_F32, PKV_F32, dev(p), vneed, nullptr) ==
        PKV_ERR_UNSUPPORTED);

  // int4 and nvfp4 caches
  CHECK(reshape_and_cache_int4(dev(p), dev(p), dev(p), dev(p), devp<float>(p), devp<float>(p),
                               devp<int64_t>(p), 4, 8, 130, 100, PKV_BF16, nullptr) ==
        PKV_ERR_UNSUPPORTED);
  CHECK(reshape_and_cache_int4(nullptr, dev(p), dev(p), dev(p), devp<float>(p), devp<float>(p),
                               devp<int64_t>(p), 4, 8, 128, 100, PKV_BF16, nullptr) ==
        PKV_ERR_NULL);
  CHECK(reshape_and_cache_nvfp4(dev(p), dev(p), dev(p), dev(p), dev(p), dev(p), devp<int64_t>(p),
                                4, 8, 128, 100, PKV_BF16, 0.f, 1.f, nullptr) == PKV_ERR_SHAPE);
  CHECK(paged_attention_decode_int4(dev(p), dev(p), dev(p), dev(p), devp<float>(p),
                                    devp<float>(p), 100,
                                    devp<int32_t>(p), 63, devp<int32_t>(p), 4, 1000, 32, 8, 128,
                                    0.088f, PKV_BF16, 0, dev(p), 0, nullptr) ==
        PKV_ERR_WORKSPACE);
  CHECK(paged_attention_decode_nvfp4(dev(p), dev(p), dev(p), dev(p), dev(p), dev(p), 100,
                                     devp<int32_t>(p), 63, devp<int32_t>(p), 4, 1000, 32, 8, 64,
                                     0.088f, PKV_BF16, 1.f, 1.f, 0, dev(p), need, nullptr) ==
        PKV_ERR_UNSUPPORTED);
}

// ---------------------------------------------------------------- part 2

struct Live {
  std::vector<int32_t> tokens;
};

static void block_manager_checks() {
  const int nb = 96;
  std::mt19937 rng(7);
  std::vector<int32_t> order(nb);
  for (int i = 0; i < nb; ++i) order[i] = i;
  std::shuffle(order.begin(), order.end(), rng);
  pkv_block_manager* m = nullptr;
  CHECK(pkv_bm_create(nb, order.data(), 1, &m) == PKV_OK && m != nullptr);
  std::vector<int32_t> dup = order;
  dup[0] = dup[1];
  pkv_block_manager* m2 = nullptr;
  CHECK(pkv_bm_create(nb, dup.data(), 1, &m2) == PKV_ERR_SHAPE);
  CHECK(pkv_bm_create(-1, nullptr, 1, &m2) != PKV_OK);

  // three shared prompt prefixes of 40 tokens
  std::vector<std::vector<int32_t>> prefixes(3);
  for (auto& pre : prefixes)
    for (int i = 0; i < 40; ++i) pre.push_back(int32_t(rng() % 50000));
  std::map<int64_t, Live> live;
  int64_t next_id = 1;
  std::vector<int64_t> pairs(2 * nb);
  std::vector<int32_t> table(nb);

  auto invariants = [&]() {
    // every block is either free (ref 0) or referenced; the free queue holds
    // exactly the ref-0 blocks
    int zero = 0;
    for (int b = 0; b < nb; ++b) {
      const int r = pkv_bm_ref_count(m, b);
      CHECK(r >= 0);
      zero += r == 0;
    }
    CHECK(pkv_bm_num_free(m) == zero);
    std::vector<int32_t> q(nb);
    CHECK(pkv_bm_free_queue(m, q.data(), nb) == zero);
    for (int i = 0; i < zero; ++i) CHECK(pkv_bm_ref_count(m, q[i]) == 0);
    for (auto& kv : live) {
      const int n = pkv_bm_num_tokens(m, kv.first);
      CHECK(n == int(kv.second.tokens.size()));
      const int len = pkv_bm_table(m, kv.first, table.data(), nb);
      CHECK(len >= 0 && len <= nb);
      for (int i = 0; i < len && i < nb; ++i) CHECK(table[i] >= 0 && table[i] < nb);
    }
  };

  for (int step = 0; step < 600; ++step) {
    const int op = int(rng() % 6);
    if (op == 0 || live.empty()) {                       // a new request
      Live r;
      r.tokens = prefixes[rng() % 3];
      const int extra = int(rng() % 30);
      for (int i = 0; i < extra; ++i) r.tokens.push_back(int32_t(rng() % 50000));
      const int64_t id = next_id++;
      int32_t cached = -1;
      const uint8_t salt[3] = {1, 2, 3};
      const pkv_status st = pkv_bm_add_request(m, id, r.tokens.data(), int32_t(r.tokens.size()),
                                               nullptr, 0, (rng() % 4) ? nullptr : salt,
                                               0, &cached);
      CHECK(st == PKV_OK);
      CHECK(cached >= 0 && cached % 16 == 0 && cached <= int(r.tokens.size()));
      CHECK(pkv_bm_add_request(m, id, r.tokens.data(), 1, nullptr, 0, nullptr, 0, &cached) ==
            PKV_ERR_REQUEST);
      const pkv_status a = pkv_bm_allocate(m, id, int32_t(r.tokens.size()) - cached);
      CHECK(a == PKV_OK || a == PKV_ERR_NO_BLOCKS);
      live[id] = r;
      if (a != PKV_OK) {
        CHECK(pkv_bm_free_request(m, id) == PKV_OK);
        live.erase(id);
      }
    } else {
      auto it = live.begin();
      std::advance(it, rng() % live.size());
      const int64_t id = it->first;
      if (op == 1 || op == 2) {                          // decode a token
        const int32_t t = int32_t(rng() % 50000);
        CHECK(pkv_bm_append_tokens(m, id, &t, 1) == PKV_OK);
        it->second.tokens.push_back(t);
        const pkv_status a = pkv_bm_allocate(m, id, 1);
        CHECK(a == PKV_OK || a == PKV_ERR_NO_BLOCKS);
        if (a != PKV_OK) {
          CHECK(pkv_bm_free_request(m, id) == PKV_OK);
          live.erase(id);
        }
      } else if (op == 3) {                              // parallel sampling fork
        const int64_t child = next_id++;
        CHECK(pkv_bm_fork(m, id, child) == PKV_OK);
        CHECK(pkv_bm_fork(m, id, child) != PKV_OK);
        live[child] = it->second;
      } else if (op == 4) {                              // finish
        CHECK(pkv_bm_free_request(m, id) == PKV_OK);
        CHECK(pkv_bm_free_request(m, id) == PKV_ERR_REQUEST);
        live.erase(it);
      } else {                                           // batched step over all
        std::vector<int64_t> ids;
        std::vector<int32_t> toks, ones;
        for (auto& kv : live) {
          ids.push_back(kv.first);
          toks.push_back(int32_t(rng() % 50000));
          ones.push_back(1);
        }
        CHECK(pkv_bm_append_tokens_batch(m, ids.data(), toks.data(), int32_t(ids.size())) ==
              PKV_OK);
        std::vector<pkv_status> st(ids.size());
        CHECK(pkv_bm_allocate_batch(m, ids.data(), ones.data(), int32_t(ids.size()),
                                    st.data()) == PKV_OK);
        for (size_t i = 0; i < ids.size(); ++i) {
          live[ids[i]].tokens.push_back(toks[i]);
          CHECK(st[i] == PKV_OK || st[i] == PKV_ERR_NO_BLOCKS);
          if (st[i] != PKV_OK) {
            CHECK(pkv_bm_free_request(m, ids[i]) == PKV_OK);
            live.erase(ids[i]);
          }
        }
      }
    }
    const int32_t n = pkv_bm_take_copies(m, pairs.data(), nb);
    CHECK(n >= 0);
    for (int i = 0; i < n; ++i) {
      CHECK(pairs[2 * i] >= 0 && pairs[2 * i] < nb && pairs[2 * i + 1] >= 0 &&
            pairs[2 * i + 1] < nb && pairs[2 * i] != pairs[2 * i + 1]);
    }
    invariants();
  }
  // export and the error paths of the queries
  std::vector<int64_t> ids;
  for (auto& kv : live) ids.push_back(kv.first);
  if (!ids.empty()) {
    std::vector<int32_t> tables(ids.size() * nb);
    CHECK(pkv_bm_export_tables(m, ids.data(), int32_t(ids.size()), tables.data(), nb, -1) ==
          PKV_OK);
    CHECK(pkv_bm_export_tables(m, ids.data(), int32_t(ids.size()), tables.data(), 0, -1) ==
              PKV_ERR_SHAPE ||
          pkv_bm_num_tokens(m, ids[0]) == 0);
  }
  const int64_t unknown = -12345;
  CHECK(pkv_bm_export_tables(m, &unknown, 1, table.data(), nb, -1) == PKV_ERR_REQUEST);
  CHECK(pkv_bm_num_tokens(m, unknown) == -1);
  CHECK(pkv_bm_ref_count(m, nb) == -1);
  CHECK(pkv_bm_ref_count(m, -1) == -1);
  CHECK(pkv_bm_table(m, unknown, table.data(), nb) == -1);
  CHECK(pkv_bm_allocate(m, unknown, 1) == PKV_ERR_REQUEST);
  CHECK(pkv_bm_allocate_batch(m, nullptr, nullptr, 1, nullptr) == PKV_ERR_NULL);
  for (auto& kv : live) CHECK(pkv_bm_free_request(m, kv.first) == PKV_OK);
  CHECK(pkv_bm_num_free(m) == nb);
  pkv_bm_destroy(m);
}

// ---------------------------------------------------------------- part 3

static void sha_checks() {
  struct V { const char* msg; const char* hex; };
  const V vs[] = {
      {"abc", "ba7816bf8f01cfea414140de5dae2223b00361a396177a9cb410ff61f20015ad"},
      {"", "e3b0c44298fc1c149afbf4c8996fb92427ae41e4649b934ca495991b7852b855"},
      {"abcdbcdecdefdefgefghfghighijhijkijkljklmklmnlmnomnopnopq",
       "248d6a61d20638b8e5c026930c3e6039a33ce45964ff2167f6ecedd419db06c1"}};
  for (const V& v : vs) {
    uint8_t d[32];
    pkv_sha256(reinterpret_cast<const uint8_t*>(v.msg), std::strlen(v.msg), d);
    char hex[65];
    for (int i = 0; i < 32; ++i) std::snprintf(hex + 2 * i, 3, "%02x", d[i]);
    CHECK(std::strcmp(hex, v.hex) == 0);
  }
  // a message long enough to span many blocks, hashed twice
  std::vector<uint8_t> big(100003);
  for (size_t i = 0; i < big.size(); ++i) big[i] = uint8_t(i * 131 + 7);
  uint8_t a[32], b[32];
  pkv_sha256(big.data(), big.size(), a);
  pkv_sha256(big.data(), big.size(), b);
  CHECK(std::memcmp(a, b, 32) == 0);
}

int main() {
  // Part 1 passes fake device addresses; it runs only where no GPU is
  // visible, so that a check that wrongly passed validation could not reach
  // a kernel.
  int devices = 0;
  if (hipGetDeviceCount(&devices) != hipSuccess) devices = 0;
  if (devices == 0)
    abi_checks();
  else
    std::printf("a GPU is visible: the argument checks (part 1) are not run\n");
  block_manager_checks();
  sha_checks();
  if (failures) {
    std::fprintf(stderr, "%d check(s) failed\n", failures);
    return 1;
  }
  std::printf("host sanitize driver: all checks passed\n");
  return 0;
}
