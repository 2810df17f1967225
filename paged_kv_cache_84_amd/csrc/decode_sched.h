// Work split of paged decode over the flattened batch (shared by the vector
// and the matrix-core decode kernels and by the merge kernel).
#pragma once

#include "common.h"

namespace pkv {

// Decode cost is the number of K/V blocks read, and context lengths differ
// widely within a batch.  The batch's blocks are therefore laid end to end
// (sequence 0's blocks, then sequence 1's, ...) and cut into `num_chunks`
// equal runs of C blocks; workgroup (chunk g, kv head) attends to the blocks
// [g C, g C + C).  A run may end inside a sequence or cover several short
// ones: a sequence that lies inside one run is finished by that workgroup,
// one that spans runs leaves one partial (max, sum, weighted values) per run
// and the merge kernel combines them with the log-sum-exp rule.

PKV_DEVICE int clamp_len(int len, int max_len) { return min(max(len, 0), max_len); }
PKV_DEVICE int blocks_of(int len) { return (len + kBlock - 1) / kBlock; }

// Sliding window (window > 0): a sequence of length len attends to its last
// `window` positions only, so it reads its blocks from first_block on; the
// split below counts those blocks (window 0 = the whole context).
PKV_DEVICE int first_block(int len, int window) {
  return window > 0 && len > window ? (len - window) / kBlock : 0;
}
PKV_DEVICE int window_blocks(int len, int window) {
  return blocks_of(len) - first_block(len, window);
}

// Block counts of the batch: lane i owns the k = ceil(S / 64) consecutive
// sequences [i k, i k + k).
struct BatchScan {
  int k;        // sequences per lane
  int first;    // blocks before the lane's first sequence
  int own;      // blocks of the lane's sequences
  int own_len;  // for k == 1: the lane's sequence length (clamped)
  int total;    // blocks of the batch
};

PKV_DEVICE BatchScan scan_batch(const int32_t* lens, int num_seqs, int max_len,
                                int window = 0) {
  BatchScan b;
  const int lane = lane_id();
  b.k = (num_seqs + kWave - 1) / kWave;
  b.own = 0;
  b.own_len = 0;
  const int s0 = lane * b.k;
  for (int j = 0; j < b.k; j += 4) {
    int l4[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int sq = s0 + j + u;
      l4[u] = (j + u < b.k && sq < num_seqs) ? clamp_len(lens[sq], max_len) : 0;
    }
#pragma unroll
    for (int u = 0; u < 4; ++u) b.own += window_blocks(l4[u], window);
    if (j == 0) b.own_len = l4[0];
  }
  b.first = wave_exclusive_sum(b.own);
  b.total = __builtin_amdgcn_readlane(b.first + b.own, kWave - 1);
  return b;
}

// Length of sequence s (uniform): from the owning lane when each lane owns
// one sequence, else through the scalar cache.
PKV_DEVICE int seq_len(const BatchScan& b, const int32_t* lens, int s, int max_len) {
  return b.k == 1 ? __builtin_amdgcn_readlane(b.own_len, s) : clamp_len(lens[s], max_len);
}

// The sequence holding block `blk` of the batch (blk < total) and the number
// of blocks before it.
PKV_DEVICE void locate(const BatchScan& b, const int32_t* lens, int max_len, int blk,
                       int& s, int& before, int window = 0) {
  const uint64_t m = __ballot(b.own > 0 && b.first <= blk && blk < b.first + b.own);
  const int owner = __builtin_amdgcn_readfirstlane(int(__builtin_ctzll(m)));
  s = owner * b.k;
  before = __builtin_amdgcn_readlane(b.first, owner);
  for (;;) {
    const int n = window_blocks(seq_len(b, lens, s, max_len), window);
    if (before + n > blk) break;
    before += n;
    ++s;
  }
}

// Blocks per chunk: fixed, or the batch split evenly over the chunks (at
// least kMinChunkBlocks, so that a chunk amortises its start).
constexpr int kMinChunkBlocks = 4;
PKV_DEVICE int chunk_blocks(int total, int num_chunks, int fixed) {
  return fixed > 0 ? fixed : max((total + num_chunks - 1) / num_chunks, kMinChunkBlocks);
}

}  // namespace pkv
