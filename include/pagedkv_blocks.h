/*
 * pagedkv_blocks.h -- C ABI of the host-side KV block manager: the block
 * pool with reference counts, the LRU free queue, the prefix-hash chain and
 * copy-on-write that decide which physical blocks each request's block
 * table names and which (src, dst) block copies a step needs.
 *
 * What it does, and where the pages define it:
 *   - The pool is a fixed set of 16-token blocks.  Free blocks sit in one
 *     LRU-ordered doubly linked queue: allocation takes the head, a released
 *     block goes to the tail and keeps its hash and contents until it is
 *     handed out again; removing a block from the middle (a prefix hit) is
 *     O(1) ("01. vLLM：从分页 KV 起家的通用推理引擎", section "KV 缓存管理与
 *     前缀缓存"; "v1/v0 区别", §4 "KV Cache 管理").
 *   - A block with a non-zero reference count is never reused (same
 *     sections).
 *   - Prefix caching: every full block is identified by a hash of its parent
 *     block's hash, its 16 token ids and extra keys (e.g. the LoRA adapter);
 *     the request's cache salt enters the first block's hash only.  A new
 *     request walks its prompt's full blocks from the first and reuses
 *     blocks while the hashes hit ("01. vLLM", same section; "vLLM 引擎解剖",
 *     section "自动前缀缓存", Fig. 4).
 *   - Copy-on-write: a request that writes into a block another request
 *     still references gets its own copy; only the writer's table changes
 *     ("vLLM 引擎解剖", section "PagedAttention：为 KV 缓存分页", the
 *     copy-on-write paragraph).  The copies are handed out as (src, dst)
 *     pairs for copy_blocks.
 *
 * Choices the pages leave open (fixed here):
 *   - Hash: SHA-256 (the pages' default algorithm) of the bytes
 *       parent digest (32 zero bytes for a request's first block)
 *       | the 16 token ids, little-endian int32
 *       | len(extra) little-endian uint32 | extra
 *       | len(salt) little-endian uint32 | salt (empty after block 0).
 *   - If the hash of a newly full block is already held by another block,
 *     the new block stays unhashed.
 *   - A request is released last block first, so the LRU queue evicts a
 *     chain from its end.
 *   - One allocation takes its copy-on-write blocks first (table order),
 *     then its new blocks; if the free queue cannot supply all of them the
 *     call fails with PKV_ERR_NO_BLOCKS and changes nothing.
 *   - Blocks are hashed when they are allocated for the tokens that fill
 *     them (their K/V are written in the same engine step).
 *
 * Host only: no GPU work, pointers are host memory.  A manager is created by
 * pkv_bm_create and owned by the caller until pkv_bm_destroy; calls on one
 * manager must not run concurrently (different managers are independent).
 * Errors are returned as pkv_status (pagedkv.h); a failing call changes
 * nothing.
 */
#ifndef PAGEDKV_BLOCKS_H
#define PAGEDKV_BLOCKS_H

#include <stddef.h>
#include <stdint.h>

#include "pagedkv.h"

#ifdef __cplusplus
extern "C" {
#endif

typedef struct pkv_block_manager pkv_block_manager;

/* A pool of num_blocks blocks.  initial_order (NULL = 0, 1, ...) gives the
 * free queue from head to tail and must be a permutation of 0..num_blocks-1
 * (else PKV_ERR_SHAPE).  prefix_caching = 0 disables hashing and hits. */
pkv_status pkv_bm_create(int32_t num_blocks, const int32_t* initial_order,
                         int32_t prefix_caching, pkv_block_manager** manager);
void pkv_bm_destroy(pkv_block_manager* manager);

/* Registers request_id (PKV_ERR_REQUEST if it exists) with its prompt token
 * ids, its extra key bytes and salt bytes (either may be NULL with length 0),
 * reuses the cached full blocks of the prompt's prefix, and stores in
 * *num_cached_tokens the number of prompt tokens whose K/V they hold
 * (a multiple of 16). */
pkv_status pkv_bm_add_request(pkv_block_manager* manager, int64_t request_id,
                              const int32_t* prompt, int32_t num_prompt_tokens,
                              const uint8_t* extra, int32_t extra_len, const uint8_t* salt,
                              int32_t salt_len, int32_t* num_cached_tokens);

/* Appends known token ids (e.g. sampled tokens) to the request. */
pkv_status pkv_bm_append_tokens(pkv_block_manager* manager, int64_t request_id,
                                const int32_t* tokens, int32_t num_tokens);

/* Gives the next num_new_tokens positions of the request a writable slot
 * (copying shared blocks, adding new ones), then hashes blocks that became
 * full.  Their token ids must be known (PKV_ERR_SHAPE otherwise). */
pkv_status pkv_bm_allocate(pkv_block_manager* manager, int64_t request_id,
                           int32_t num_new_tokens);

/* One engine step for many requests in one call: appends token i to request
 * ids[i] (a decode's sampled token), for all i, in order; PKV_ERR_REQUEST
 * (nothing appended) if an id is unknown. */
pkv_status pkv_bm_append_tokens_batch(pkv_block_manager* manager, const int64_t* ids,
                                      const int32_t* tokens, int32_t num_requests);

/* pkv_bm_allocate(ids[i], num_new_tokens[i]) for i = 0, 1, ... in order;
 * status[i] receives each result (a request that does not fit gets
 * PKV_ERR_NO_BLOCKS and the later ones are still tried).  Returns PKV_OK, or
 * PKV_ERR_NULL for missing arrays. */
pkv_status pkv_bm_allocate_batch(pkv_block_manager* manager, const int64_t* ids,
                                 const int32_t* num_new_tokens, int32_t num_requests,
                                 pkv_status* status);

/* child_id shares every block and token of parent_id (parallel sampling). */
pkv_status pkv_bm_fork(pkv_block_manager* manager, int64_t parent_id, int64_t child_id);

/* Releases the request's blocks (last block first) and forgets it. */
pkv_status pkv_bm_free_request(pkv_block_manager* manager, int64_t request_id);

/* Queries.  Each returns -1 for an unknown request or block. */
int32_t pkv_bm_num_free(const pkv_block_manager* manager);
int32_t pkv_bm_num_tokens(const pkv_block_manager* manager, int64_t request_id);
int32_t pkv_bm_ref_count(const pkv_block_manager* manager, int32_t block);
/* Writes min(length, capacity) table entries; returns the table's length. */
int32_t pkv_bm_table(const pkv_block_manager* manager, int64_t request_id, int32_t* out,
                     int32_t capacity);
/* Writes min(length, capacity) free block ids, head first; returns length. */
int32_t pkv_bm_free_queue(const pkv_block_manager* manager, int32_t* out, int32_t capacity);

/* Moves the pending copy-on-write pairs (in the order they arose) into
 * pairs [n][2] = (src, dst) and returns n; if capacity < n, takes nothing
 * and returns -n. */
int32_t pkv_bm_take_copies(pkv_block_manager* manager, int64_t* pairs, int32_t capacity);

/* Block tables of the given requests as int32 [num_requests][width], rows
 * padded with pad (PKV_ERR_SHAPE if a table is longer than width,
 * PKV_ERR_REQUEST for an unknown request). */
pkv_status pkv_bm_export_tables(const pkv_block_manager* manager, const int64_t* request_ids,
                                int32_t num_requests, int32_t* tables, int32_t width,
                                int32_t pad);

/* The block hash above (parent: 32 bytes; tokens: 16 ids); digest: 32 bytes. */
void pkv_block_hash(const uint8_t* parent, const int32_t* tokens, const uint8_t* extra,
                    int32_t extra_len, const uint8_t* salt, int32_t salt_len,
                    uint8_t* digest);

/* SHA-256 (FIPS 180-4) of len bytes into digest[32]; with the x86 SHA
 * extensions when the CPU has them, unless the environment variable
 * PKV_SHA256_PORTABLE is set (non-empty, not "0") at the first call. */
void pkv_sha256(const uint8_t* data, size_t len, uint8_t* digest);

#ifdef __cplusplus
}
#endif

#endif /* PAGEDKV_BLOCKS_H */
