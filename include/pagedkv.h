/*
 * pagedkv.h -- C ABI of the paged KV cache hot path for AMD Instinct MI355X
 * (CDNA4, gfx950).
 *
 * The KV cache of one attention layer is split into fixed physical blocks of
 * 16 token slots; each sequence reaches its blocks through a block table that
 * maps logical block j (tokens 16j .. 16j+15) to a physical block id
 * ("vLLM 引擎解剖", section "PagedAttention：为 KV 缓存分页", Fig. 2).
 *
 * Layouts (all row-major, contiguous):
 *   k_cache, v_cache  [num_blocks][num_kv_heads][16][head_dim]  cache dtype
 *   block_tables      int32 [num_seqs][max_blocks_per_seq]
 *   query / out       [num_tokens][num_q_heads][head_dim]       q dtype
 *   key / value       [num_tokens][num_kv_heads][head_dim]      source dtype
 *   slot_mapping      int64 [num_tokens]; slot = block * 16 + offset
 * Query head h reads kv head h / (num_q_heads / num_kv_heads).
 *
 * Ownership and threading: the caller allocates every buffer (device memory
 * unless stated otherwise) and keeps it alive until the work it was passed
 * to has finished on the stream.  The library allocates no memory, keeps no
 * mutable global state and may be called from several threads.  Every call
 * validates its host-side arguments synchronously, then enqueues its kernels
 * on `stream` (a hipStream_t; NULL = the null stream) and returns without
 * waiting.
 *
 * Errors: a non-zero pkv_status means nothing was enqueued (except
 * PKV_ERR_LAUNCH, reported when the runtime rejects a launch).  Device-resident
 * index data (block tables, slots, lengths, copy pairs) is not inspected on
 * the host; it must satisfy the preconditions stated per call.  Block ids
 * outside [0, num_blocks) are never dereferenced: such a block contributes
 * nothing to attention and such a slot or copy is skipped, so a violated
 * precondition gives a wrong result, never an out-of-bounds access.
 *
 * Device pointers must be 16-byte aligned.
 */
#ifndef PAGEDKV_H
#define PAGEDKV_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef int32_t pkv_status;
enum {
  PKV_OK = 0,
  PKV_ERR_NULL = 1,        /* a required pointer is NULL                    */
  PKV_ERR_ALIGN = 2,       /* a device pointer is not 16-byte aligned       */
  PKV_ERR_SHAPE = 3,       /* inconsistent or negative sizes                */
  PKV_ERR_UNSUPPORTED = 4, /* head_dim / dtype / group size not built       */
  PKV_ERR_WORKSPACE = 5,   /* decode workspace missing or too small         */
  PKV_ERR_LAUNCH = 6,      /* the HIP runtime rejected a kernel launch      */
  PKV_ERR_NO_BLOCKS = 7,   /* block manager: too few free blocks            */
  PKV_ERR_REQUEST = 8      /* block manager: unknown or duplicate request   */
};

typedef int32_t pkv_dtype;
enum {
  PKV_F32 = 0,      /* IEEE binary32                                          */
  PKV_BF16 = 1,     /* bfloat16 (upper half of a binary32)                    */
  PKV_FP8_E4M3 = 2, /* OCP fp8 E4M3 ("fn": no inf, max 448), cache dtype only */
  PKV_INT4 = 3,     /* int4 per token-head codes (see reshape_and_cache_int4),
                       cache dtype only, with separate per-row scale arrays    */
  PKV_NVFP4 = 4     /* FP4 E2M1 codes with an E4M3 scale per 16 elements and a
                       per-tensor scale (see reshape_and_cache_nvfp4), cache
                       dtype only, with separate block-scale arrays           */
};

#define PKV_BLOCK_SIZE 16

/* Tokens per physical block (16: the default block size of "vLLM 引擎解剖",
 * section "PagedAttention：为 KV 缓存分页"). */
int32_t pkv_block_size(void);

/* Static, NUL-terminated description of a status code. */
const char* pkv_status_string(pkv_status status);

/* Bytes of KV cache one token occupies over a whole model:
 * 2 (key and value) x bytes_per_elem x num_layers x num_kv_heads x head_dim
 * ("vLLM 引擎解剖", section "KV 缓存需要多少内存？", the formula of Table 1).
 * Returns -1 if any argument is negative or the product does not fit in
 * int64. Host-only, no GPU work. */
int64_t kv_bytes_per_token(int32_t num_layers, int32_t num_kv_heads,
                           int32_t head_dim, int32_t bytes_per_elem);

/*
 * compute_slot_mapping -- the cache slot of every token scheduled this step.
 *
 * One step is the unified schedule {request: num_tokens} ("vLLM 引擎解剖",
 * section "V1：统一调度预填充与解码"; "v1/v0 区别", §3.1 "Token 预算"):
 * request r brings the tokens query_start_loc[r] .. query_start_loc[r+1]-1
 * of the flattened batch, and its i-th token sits at sequence position
 * p = num_computed_tokens[r] + i.  Its slot is
 *   block_tables[r][p / 16] * 16 + p % 16            (Fig. 2 layout).
 *
 *   block_tables        int32 [num_reqs][max_blocks_per_seq], device
 *   query_start_loc     int32 [num_reqs + 1], device, non-decreasing, [0] = 0,
 *                       [num_reqs] = num_tokens
 *   num_computed_tokens int32 [num_reqs], device, >= 0
 *   slot_mapping        int64 [num_tokens], device, written
 * A position whose logical block lies beyond max_blocks_per_seq, or whose
 * block id is outside [0, num_blocks), gets slot -1.
 */
pkv_status compute_slot_mapping(const int32_t* block_tables,
                                int32_t max_blocks_per_seq,
                                const int32_t* query_start_loc,
                                const int32_t* num_computed_tokens,
                                int32_t num_reqs, int32_t num_blocks,
                                int64_t* slot_mapping, int32_t num_tokens,
                                void* stream);

/*
 * reshape_and_cache -- write each token's K and V into its cache slot.
 *
 * The forward pass computes every new token's key and value and stores them
 * in the KV cache, from where later steps read them ("vLLM 引擎解剖", section
 * "预填充、解码与三个时延指标").  For token t with slot s >= 0, for every kv head:
 *   k_cache[s / 16][head][s % 16][:] = enc(key[t][head][:])  (same for V)
 * Equal source and cache dtypes copy the bits.  An fp8 cache stores
 *   E4M3(fp32(x) / k_scale)   (v_scale for V)
 * with the division in binary32 (correctly rounded), round to nearest even,
 * saturation to +-448, NaN -> 0x7F with the sign kept, signed zero kept.
 * Negative slots are skipped.  Supported (src, cache): (F32, F32),
 * (BF16, BF16), (BF16, FP8_E4M3), (F32, FP8_E4M3).
 * Precondition: slots of one call are distinct.
 */
pkv_status reshape_and_cache(const void* key, const void* value,
                             void* k_cache, void* v_cache,
                             const int64_t* slot_mapping, int32_t num_tokens,
                             int32_t num_kv_heads, int32_t head_dim,
                             int32_t num_blocks, pkv_dtype src_dtype,
                             pkv_dtype cache_dtype, float k_scale,
                             float v_scale, void* stream);

/*
 * reshape_and_cache_from_schedule -- compute_slot_mapping and
 * reshape_and_cache in one launch: each scheduled token's slot is derived
 * from the unified schedule and its block table exactly as
 * compute_slot_mapping does (slot -1 in the same cases), stored to
 * slot_mapping if that is not NULL, and the token's K and V are written
 * there exactly as reshape_and_cache does (same encodings, negative slots
 * skipped).  Meant for the first layer of a step: later layers take the
 * stored slot_mapping to reshape_and_cache.
 *
 *   key, value, k_cache, v_cache, dtypes, scales: as reshape_and_cache
 *   block_tables, max_blocks_per_seq, query_start_loc, num_computed_tokens,
 *   num_reqs, num_blocks: as compute_slot_mapping
 *   slot_mapping    int64 [num_tokens], device, written; or NULL
 * Same supported set and preconditions as the two calls.
 */
pkv_status reshape_and_cache_from_schedule(
    const void* key, const void* value, void* k_cache, void* v_cache,
    const int32_t* block_tables, int32_t max_blocks_per_seq, const int32_t* query_start_loc,
    const int32_t* num_computed_tokens, int32_t num_reqs, int64_t* slot_mapping,
    int32_t num_tokens, int32_t num_kv_heads, int32_t head_dim, int32_t num_blocks,
    pkv_dtype src_dtype, pkv_dtype cache_dtype, float k_scale, float v_scale, void* stream);

/*
 * copy_blocks -- copy whole physical blocks, in every layer.
 *
 * Shared blocks are read-only; a sequence about to write into a block that
 * other sequences still reference gets its own copy and only its own table
 * is repointed ("vLLM 引擎解剖", section "PagedAttention：为 KV 缓存分页",
 * copy-on-write).  Such copies travel with each step as a list of
 * (src, dst) pairs ("v1/v0 区别", §2.1 "V0 引擎循环", blocks_to_copy).
 *
 *   k_caches, v_caches  HOST arrays of num_layers device pointers
 *   block_mapping       int64 [num_pairs][2] = (src, dst), device
 *   block_bytes         bytes of one block of one layer's K (or V) cache:
 *                       num_kv_heads * 16 * head_dim * element size; a
 *                       positive multiple of 16
 * For each pair and layer: K[dst] = K[src], V[dst] = V[src].
 * Precondition: destinations are distinct and none is also a source.
 */
pkv_status copy_blocks(void* const* k_caches, void* const* v_caches,
                       int32_t num_layers, const int64_t* block_mapping,
                       int32_t num_pairs, int32_t num_blocks,
                       int64_t block_bytes, void* stream);

/*
 * swap_blocks -- copy whole blocks from one cache pool into another, every
 * layer, K and V; one pool is device memory and the other host memory (the
 * other way round to swap back), or both are device memory.
 *
 * The v0 engine could preempt a request by swapping its KV blocks out to CPU
 * memory and back in later ("vLLM 引擎解剖", section "抢占：RECOMPUTE", the v0
 * SWAP mode); the swaps travelled with each step as blocks_to_swap_out /
 * blocks_to_swap_in next to blocks_to_copy ("v1/v0 区别", §2.1 "V0 引擎循环").
 * Today's engine offloads KV blocks to CPU memory
 * ("01. vLLM：从分页 KV 起家的通用推理引擎", section "KV 缓存管理与前缀缓存",
 * --kv-offloading-size).
 *
 *   src_k_caches, src_v_caches  HOST arrays of num_layers pointers to the
 *   dst_k_caches, dst_v_caches  source and destination pools, each
 *                               [num_*_blocks][num_kv_heads][16][head_dim];
 *                               device memory, or pinned host memory from
 *                               hipHostMalloc (it is read and written through
 *                               its device mapping)
 *   block_mapping  int64 [num_pairs][2] = (src block, dst block), device or
 *                  pinned host memory
 *   block_bytes    bytes of one block of one layer's K (or V) pool; a
 *                  positive multiple of 16
 * For each pair and layer: dst_K[dst] = src_K[src], dst_V[dst] = src_V[src],
 * as one kernel launch on `stream`.  A pair with an id outside its pool is
 * skipped.  Precondition: destinations are distinct; if the two pools are
 * the same memory, no destination is also a source.
 */
pkv_status swap_blocks(void* const* src_k_caches, void* const* src_v_caches,
                       void* const* dst_k_caches, void* const* dst_v_caches,
                       int32_t num_layers, const int64_t* block_mapping,
                       int32_t num_pairs, int32_t num_src_blocks,
                       int32_t num_dst_blocks, int64_t block_bytes, void* stream);

/*
 * paged_attention_decode -- one query token per sequence attends to its whole
 * paged KV history; decode streams the entire cache once per step and is
 * bound by memory bandwidth ("vLLM 引擎解剖", section "预填充、解码与三个时延指标").
 *
 * For sequence s and query head h, with L = context_lens[s] (the query's own
 * token included, its K/V already written):
 *   out[s][h] = softmax_j(q[s][h] . K_j * softmax_scale) . V_j,  j < L
 * where K_j, V_j are read through block_tables[s] and an fp8 cache element
 * c stands for value(c) * k_scale (v_scale for V).  L == 0 gives zeros.
 *
 * Work split: the blocks of all sequences are laid end to end and cut into
 * equal chunks; per kv head, a wave walks a run of consecutive chunks.
 * Each chunk of a sequence gives a (max, sum, weighted-value) partial; the
 * partials of one sequence are combined with a log-sum-exp rescale, first
 * by the wave that computed them (the chunks it walks), then by a second
 * kernel across waves, which reads them from `workspace`.  A sequence
 * walked whole by one wave is written to `out` directly.
 * partition_tokens = 0 lets the library size the chunks from the actual
 * lengths (all chunks equal, one per wave, enough waves to fill the GPU);
 * otherwise each chunk is exactly partition_tokens tokens (a positive
 * multiple of 16) of the laid-out blocks and a wave may walk several.
 * Results are bitwise reproducible for the same arguments.  The workspace is
 * caller-owned device memory of at least
 * paged_attention_decode_workspace_size(...) bytes for the same arguments;
 * its contents need no initialisation and are scratch after the call.
 *
 *   out, query          [num_seqs][num_q_heads][head_dim], q dtype
 *   context_lens        int32 [num_seqs], device, 0 <= L <= max_context_len
 *   block_tables        int32 [num_seqs][max_blocks_per_seq], device; entries
 *                       0 .. ceil(L/16)-1 are read, the rest never
 * Supported: head_dim 64 or 128; num_q_heads a multiple of num_kv_heads with
 * a group of at most 8; (q, kv) dtypes (F32, F32), (BF16, BF16),
 * (BF16, FP8_E4M3).  Accumulation is fp32; the output is rounded to the q
 * dtype (nearest even).
 */
size_t paged_attention_decode_workspace_size(int32_t num_seqs,
                                             int32_t num_q_heads,
                                             int32_t num_kv_heads,
                                             int32_t head_dim,
                                             int32_t max_context_len,
                                             int32_t partition_tokens);

/* The number of chunks (per kv head) paged_attention_decode splits the work
 * into for these arguments, or -1 when they are invalid. */
int32_t paged_attention_decode_num_chunks(int32_t num_seqs, int32_t num_q_heads,
                                          int32_t num_kv_heads,
                                          int32_t max_context_len,
                                          int32_t partition_tokens);

pkv_status paged_attention_decode(void* out, const void* query,
                                  const void* k_cache, const void* v_cache,
                                  int32_t num_blocks,
                                  const int32_t* block_tables,
                                  int32_t max_blocks_per_seq,
                                  const int32_t* context_lens,
                                  int32_t num_seqs, int32_t max_context_len,
                                  int32_t num_q_heads, int32_t num_kv_heads,
                                  int32_t head_dim, float softmax_scale,
                                  pkv_dtype q_dtype, pkv_dtype kv_dtype,
                                  float k_scale, float v_scale,
                                  int32_t partition_tokens, void* workspace,
                                  size_t workspace_bytes, void* stream);

/*
 * paged_attention_decode_noalloc -- paged_attention_decode for callers that
 * cannot allocate device memory: code under HIP graph capture, tight serving
 * loops, harnesses that forbid hipMalloc.  Same arguments, layouts, results
 * (bitwise: same kernels, same split) and errors as paged_attention_decode,
 * without the workspace: the partials live in a file-scope device array of
 * PKV_DECODE_SCRATCH_BYTES that each GPU the library runs on holds until the
 * process ends.  Its address is looked up once per device, on the first call
 * with that device current (the calling thread's current device must be the
 * one holding the tensors and running `stream`); no call allocates.
 *   PKV_ERR_WORKSPACE  the split for these arguments needs more than
 *                      PKV_DECODE_SCRATCH_BYTES (paged_attention_decode_
 *                      workspace_size gives the need); nothing is launched
 * Every call on a GPU shares that GPU's array, which keeps the last call's
 * contents (the kernels write every record before reading it, so nothing is
 * cleared): calls that overlap on one GPU -- on two streams, or from two
 * threads without ordering -- race on it and must not be made.
 */
#define PKV_DECODE_SCRATCH_BYTES (64u << 20)
pkv_status paged_attention_decode_noalloc(void* out, const void* query,
                                          const void* k_cache, const void* v_cache,
                                          int32_t num_blocks,
                                          const int32_t* block_tables,
                                          int32_t max_blocks_per_seq,
                                          const int32_t* context_lens,
                                          int32_t num_seqs, int32_t max_context_len,
                                          int32_t num_q_heads, int32_t num_kv_heads,
                                          int32_t head_dim, float softmax_scale,
                                          pkv_dtype q_dtype, pkv_dtype kv_dtype,
                                          float k_scale, float v_scale,
                                          int32_t partition_tokens, void* stream);

/*
 * paged_attention_prefill_chunk -- attention for the query rows of prompt
 * chunks scheduled this step.  A long prompt is split into chunks that share
 * steps with decodes ("vLLM 引擎解剖", section "V1：统一调度预填充与解码",
 * Fig. 3); per request the kernel needs the query length, the context
 * length and the block table ("v1/v0 区别", §3.1 "Token 预算").
 *
 * Request r owns query rows query_start_loc[r] .. query_start_loc[r+1]-1;
 * with c = num_computed_tokens[r] (tokens already in the cache before this
 * chunk, e.g. a prefix-cache hit), row i sits at position p = c + i and
 * attends causally to positions 0 .. p (inclusive) through block_tables[r]:
 *   out[row][h] = softmax_{j<=p}(q[row][h] . K_j * softmax_scale) . V_j
 * The chunk's own K/V must already be in the cache (reshape_and_cache).
 *
 *   out, query        [num_q_tokens][num_q_heads][head_dim], q dtype
 *   query_start_loc   int32 [num_reqs + 1], device, [0] = 0,
 *                     [num_reqs] = num_q_tokens, steps <= max_query_len
 *   num_computed_tokens int32 [num_reqs], device
 * Supported: head_dim 128 with (BF16, BF16) (the MFMA path); head_dim 64 or
 * 128 with (F32, F32) and (BF16, FP8_E4M3) are also accepted.  Group size
 * at most 8.  Accumulation is fp32.
 */
pkv_status paged_attention_prefill_chunk(void* out, const void* query,
                                         const void* k_cache,
                                         const void* v_cache,
                                         int32_t num_blocks,
                                         const int32_t* block_tables,
                                         int32_t max_blocks_per_seq,
                                         const int32_t* query_start_loc,
                                         const int32_t* num_computed_tokens,
                                         int32_t num_reqs,
                                         int32_t num_q_tokens,
                                         int32_t max_query_len,
                                         int32_t num_q_heads,
                                         int32_t num_kv_heads,
                                         int32_t head_dim, float softmax_scale,
                                         pkv_dtype q_dtype, pkv_dtype kv_dtype,
                                         float k_scale, float v_scale,
                                         void* stream);

/*
 * paged_attention_decode_append -- one decode step of a decode-only batch:
 * each sequence's new token (position L-1, L = context_lens[s] >= 1) is
 * written into the cache and attention over positions 0 .. L-1 follows, in
 * the same launch.  Prefill writes K and V into the cache and decode reads
 * them back ("vLLM 引擎解剖", section "预填充、解码与三个时延指标"); here the write
 * of the token a decode row brings is the reshape_and_cache of that row,
 * at the slot compute_slot_mapping gives it (block_tables[s][(L-1)/16] * 16
 * + (L-1) % 16; skipped if the block id is outside [0, num_blocks) or the
 * logical block beyond max_blocks_per_seq), encoded as reshape_and_cache
 * does.  The results equal reshape_and_cache of the new rows followed by
 * paged_attention_decode.
 *   new_key, new_value  bf16 [num_seqs][num_kv_heads][head_dim], device,
 *                       16-byte aligned; rows of sequences with L = 0 are
 *                       not read
 *   k_cache, v_cache    written at the new tokens' slots, then read
 * Supported: bf16 queries with bf16 or fp8 E4M3 caches (PKV_ERR_UNSUPPORTED
 * otherwise); other arguments, workspace and errors as
 * paged_attention_decode.  Precondition: the new tokens' slots are distinct
 * (a sequence writing into a block it shares is copied first).
 */
pkv_status paged_attention_decode_append(void* out, const void* query, const void* new_key,
                                         const void* new_value, void* k_cache, void* v_cache,
                                         int32_t num_blocks, const int32_t* block_tables,
                                         int32_t max_blocks_per_seq, const int32_t* context_lens,
                                         int32_t num_seqs, int32_t max_context_len,
                                         int32_t num_q_heads, int32_t num_kv_heads,
                                         int32_t head_dim, float softmax_scale,
                                         pkv_dtype q_dtype, pkv_dtype kv_dtype, float k_scale,
                                         float v_scale, int32_t partition_tokens,
                                         void* workspace, size_t workspace_bytes, void* stream);

/*
 * paged_attention_decode_sliding -- paged_attention_decode for sliding-window
 * layers: the query of a sequence of length L attends to positions
 * max(0, L - sliding_window) .. L-1 only (its own included; the pages note
 * that such layers' blocks outside the window can be released early, "01.
 * vLLM：从分页 KV 起家的通用推理引擎", section "KV 缓存管理与前缀缓存").
 * Blocks before the window are not read: the work split counts only the
 * window's blocks, so the cost follows min(L, window).  block_tables rows
 * must still map every logical block index up to L-1 (entries before the
 * window are never read and may be invalid).  sliding_window >= 1 (else
 * PKV_ERR_SHAPE); bf16 queries with bf16 or fp8 caches (else
 * PKV_ERR_UNSUPPORTED); other arguments, workspace and errors as
 * paged_attention_decode.
 */
pkv_status paged_attention_decode_sliding(void* out, const void* query, const void* k_cache,
                                          const void* v_cache, int32_t num_blocks,
                                          const int32_t* block_tables,
                                          int32_t max_blocks_per_seq,
                                          const int32_t* context_lens, int32_t num_seqs,
                                          int32_t max_context_len, int32_t num_q_heads,
                                          int32_t num_kv_heads, int32_t head_dim,
                                          float softmax_scale, pkv_dtype q_dtype,
                                          pkv_dtype kv_dtype, float k_scale, float v_scale,
                                          int32_t sliding_window, int32_t partition_tokens,
                                          void* workspace, size_t workspace_bytes,
                                          void* stream);

/*
 * int4 per token-head KV cache (PKV_INT4).  The pages list
 * "int4_per_token_head" among the lower-bit --kv-cache-dtype formats ("01.
 * vLLM：从分页 KV 起家的通用推理引擎", section "KV 缓存管理与前缀缓存", the
 * --kv-cache-dtype row) and fix nothing else; the encoding here: every
 * (token, kv head) row of head_dim values x has one binary32 scale
 * s = max|x| / 7 and codes q = round-half-even(x / s) in [-8, 7] (both
 * divisions in binary32; a zero row has s = 0, q = 0), stored as nibbles
 * u = q + 8, element 2i in the low nibble of byte i.  Its value is
 * (u - 8) * s.  Layouts:
 *   k_cache, v_cache   uint8 [num_blocks][num_kv_heads][16][head_dim / 2]
 *   k_scales, v_scales float [num_blocks][num_kv_heads][16]
 * A quarter of bf16's bytes per element, plus 4 bytes per row.
 *
 * reshape_and_cache_int4 -- reshape_and_cache into int4 caches: each
 * scheduled token's K and V rows are quantised as above (from bf16 or fp32
 * sources, finite values) and written with their scales at the slot; a
 * negative slot skips the token.  head_dim even and at most 128.
 */
pkv_status reshape_and_cache_int4(const void* key, const void* value, void* k_cache,
                                  void* v_cache, float* k_scales, float* v_scales,
                                  const int64_t* slot_mapping, int32_t num_tokens,
                                  int32_t num_kv_heads, int32_t head_dim, int32_t num_blocks,
                                  pkv_dtype src_dtype, void* stream);

/*
 * paged_attention_decode_int4 -- paged_attention_decode over int4 caches:
 * the result is attention over the rows' values (u - 8) * s.  The kernel
 * never widens a row with its scale: a code enters the products as the bf16
 * 128 + u, the key's scale multiplies its score and the value's scale its
 * weight, and the constant offset is taken out of both sums afterwards.
 * Same work split, workspace (paged_attention_decode_workspace_size) and
 * merge as paged_attention_decode.  Supported: bf16 queries, head_dim 128,
 * group <= 8.  Scale arrays 16-byte aligned.
 */
pkv_status paged_attention_decode_int4(void* out, const void* query, const void* k_cache,
                                       const void* v_cache, const float* k_scales,
                                       const float* v_scales, int32_t num_blocks,
                                       const int32_t* block_tables, int32_t max_blocks_per_seq,
                                       const int32_t* context_lens, int32_t num_seqs,
                                       int32_t max_context_len, int32_t num_q_heads,
                                       int32_t num_kv_heads, int32_t head_dim,
                                       float softmax_scale, pkv_dtype q_dtype,
                                       int32_t partition_tokens, void* workspace,
                                       size_t workspace_bytes, void* stream);

/*
 * nvfp4-style KV cache (PKV_NVFP4).  The pages list "nvfp4" among the
 * lower-bit --kv-cache-dtype formats ("01. vLLM：从分页 KV 起家的通用推理引擎",
 * section "KV 缓存管理与前缀缓存", the --kv-cache-dtype row) and fix nothing
 * else; the encoding here: every 16 consecutive elements of a (token, kv
 * head) row share one E4M3 block scale, and a per-tensor binary32 scale g
 * (k_scale for K, v_scale for V) sits above all blocks.  For a block x:
 *   scale code  c = E4M3(fp32(fp32(max|x| / 6) / g))   (round to nearest
 *               even, saturating at 448)
 *   element     e = E2M1(fp32(x / fp32(S * g)))         (S = value of c;
 *               nearest of 0, 0.5, 1, 1.5, 2, 3, 4, 6 with ties to the even
 *               mantissa, saturating at 6, sign kept; all codes 0 if S = 0)
 * and its value is e * S * g.  E2M1 codes are packed two per byte, element
 * 2i in the low nibble.  Layouts:
 *   k_cache, v_cache     uint8 [num_blocks][num_kv_heads][16][head_dim / 2]
 *   k_bscales, v_bscales uint8 [num_blocks][num_kv_heads][16][head_dim / 16]
 * 4.5 bits per element.
 *
 * reshape_and_cache_nvfp4 -- reshape_and_cache into nvfp4 caches: each
 * scheduled token's K and V rows (bf16 or fp32, finite) are encoded as
 * above and written with their block scales at the slot; a negative slot
 * skips the token.  head_dim a multiple of 16, at most 128; k_scale,
 * v_scale > 0.
 */
pkv_status reshape_and_cache_nvfp4(const void* key, const void* value, void* k_cache,
                                   void* v_cache, void* k_bscales, void* v_bscales,
                                   const int64_t* slot_mapping, int32_t num_tokens,
                                   int32_t num_kv_heads, int32_t head_dim, int32_t num_blocks,
                                   pkv_dtype src_dtype, float k_scale, float v_scale,
                                   void* stream);

/*
 * paged_attention_decode_nvfp4 -- paged_attention_decode over nvfp4 caches:
 * the result is attention over the values e * S * g.  Each 16-element piece
 * is widened to bf16 exactly in registers (e * S has at most six significant
 * bits); g of K multiplies the scores and g of V the output.  Same work
 * split, workspace (paged_attention_decode_workspace_size) and merge as
 * paged_attention_decode.  Supported: bf16 queries, head_dim 128,
 * group <= 8; k_scale, v_scale > 0.
 */
pkv_status paged_attention_decode_nvfp4(void* out, const void* query, const void* k_cache,
                                        const void* v_cache, const void* k_bscales,
                                        const void* v_bscales, int32_t num_blocks,
                                        const int32_t* block_tables, int32_t max_blocks_per_seq,
                                        const int32_t* context_lens, int32_t num_seqs,
                                        int32_t max_context_len, int32_t num_q_heads,
                                        int32_t num_kv_heads, int32_t head_dim,
                                        float softmax_scale, pkv_dtype q_dtype, float k_scale,
                                        float v_scale, int32_t partition_tokens,
                                        void* workspace, size_t workspace_bytes, void* stream);

/*
 * paged_attention_varlen -- the attention of one whole engine step in one
 * launch: every request's query rows, whatever their number -- one for a
 * decode, 1 + k to verify k speculative drafts, many for a prompt chunk.
 *
 * The unified scheduler has no prefill or decode phase: a request only has
 * the tokens computed so far and the tokens to reach (input + generated +
 * drafts), and a step advances each by some tokens
 * ("01. vLLM：从分页 KV 起家的通用推理引擎", section "调度器：统一的 token 预算";
 * V1 EngineCore architecture page, section "统一 token 调度"); drafts are
 * verified by the target model in one step (the "01. vLLM" page, section
 * "投机解码").
 *
 * Semantics are those of paged_attention_prefill_chunk over all requests:
 * row i of request r, at position p = num_computed_tokens[r] + i, attends to
 * positions 0 .. p through block_tables[r].  A request with at most 16 query
 * rows (tokens x group) is streamed by one wave per (request, kv head, run of
 * 64 blocks); longer requests run as chunked-prefill tiles; both kinds share
 * one kernel and run side by side, handed out through per-XCD work queues.
 * Three kernels go onto the stream: a one-workgroup plan (clears the queue
 * counters, lists the tiles and runs), the attention kernel, and a small
 * merge of the runs of requests longer than 64 blocks (log-sum-exp rule).
 *
 *   out, query, query_start_loc, num_computed_tokens, block_tables: as for
 *                   paged_attention_prefill_chunk, over all num_reqs requests
 *   max_seq_len     bound on num_computed_tokens[r] + (query rows of r)
 *   workspace       device memory of at least
 *                   paged_attention_varlen_workspace_size(...) bytes for the
 *                   same num_reqs, num_q_tokens, num_kv_heads, head_dim,
 *                   max_seq_len (0 if those are unsupported); it holds the
 *                   plan and the per-run partial results (no initial
 *                   contents needed).  Calls that share a workspace must not
 *                   overlap in time.
 * Supported: head_dim 128, (q, kv) = (BF16, BF16), group 1, 2, 4 or 8,
 * softmax_scale > 0.  Accumulation is fp32; the output is bf16.
 */
size_t paged_attention_varlen_workspace_size(int32_t num_reqs, int32_t num_q_tokens,
                                             int32_t num_kv_heads, int32_t head_dim,
                                             int32_t max_seq_len);

pkv_status paged_attention_varlen(void* out, const void* query, const void* k_cache,
                                  const void* v_cache, int32_t num_blocks,
                                  const int32_t* block_tables, int32_t max_blocks_per_seq,
                                  const int32_t* query_start_loc,
                                  const int32_t* num_computed_tokens, int32_t num_reqs,
                                  int32_t num_q_tokens, int32_t max_seq_len,
                                  int32_t num_q_heads, int32_t num_kv_heads,
                                  int32_t head_dim, float softmax_scale, pkv_dtype q_dtype,
                                  pkv_dtype kv_dtype, void* workspace,
                                  size_t workspace_bytes, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* PAGEDKV_H */
