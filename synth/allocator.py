"""Host block pool: reference counts, prefix sharing and copy-on-write.

The KV cache manager keeps a pool of fixed-size blocks, hands them out as
tokens arrive, counts references so that sequences with the same prefix can
point at the same physical blocks, and gives a writer its own copy of a block
that others still reference, repointing only the writer's table
("vLLM 引擎解剖", section "PagedAttention：为 KV 缓存分页"; "v1/v0 区别",
§4 "KV Cache 管理": reference counts, ref_cnt > 0 means not evictable).

This is input construction: it decides which physical blocks each sequence
owns and which (src, dst) block copies a step needs.  The copies themselves,
the slot of each token and the cache writes are the hot path's job.
"""

from collections import deque

import numpy as np

BLOCK = 16


class OutOfBlocks(RuntimeError):
    pass


class BlockPool:
    """Free blocks are taken from the head of a queue and returned to its
    tail.  ``order`` fixes the initial queue (e.g. a seeded shuffle)."""

    def __init__(self, num_blocks, order=None):
        self.num_blocks = int(num_blocks)
        self.ref = np.zeros(self.num_blocks, dtype=np.int64)
        if order is None:
            order = range(self.num_blocks)
        self.free = deque(int(b) for b in order)

    def allocate(self):
        if not self.free:
            raise OutOfBlocks("block pool exhausted")
        b = self.free.popleft()
        assert self.ref[b] == 0
        self.ref[b] = 1
        return b

    def retain(self, block):
        assert self.ref[block] > 0
        self.ref[block] += 1

    def release(self, block):
        assert self.ref[block] > 0
        self.ref[block] -= 1
        if self.ref[block] == 0:
            self.free.append(int(block))

    def num_free(self):
        return len(self.free)


class Sequence:
    """One sequence's block table and the number of tokens whose K/V are (or
    are about to be) in the cache."""

    def __init__(self, pool, table=None, num_tokens=0):
        self.pool = pool
        self.table = list(table or [])
        self.num_tokens = int(num_tokens)

    @classmethod
    def fresh(cls, pool, num_tokens):
        seq = cls(pool)
        seq.grow_to(num_tokens)
        return seq

    def grow_to(self, num_tokens):
        """Allocate blocks so that positions ``0..num_tokens-1`` have one."""
        need = (int(num_tokens) + BLOCK - 1) // BLOCK
        while len(self.table) < need:
            self.table.append(self.pool.allocate())
        self.num_tokens = max(self.num_tokens, int(num_tokens))

    def fork(self):
        """A second sequence sharing every block of this one."""
        for b in self.table:
            self.pool.retain(b)
        return Sequence(self.pool, list(self.table), self.num_tokens)

    def share_prefix(self, num_blocks):
        """A new sequence whose first ``num_blocks`` blocks are this one's."""
        for b in self.table[:num_blocks]:
            self.pool.retain(b)
        return Sequence(self.pool, list(self.table[:num_blocks]),
                        num_blocks * BLOCK)

    def prepare_write(self, first_position, count):
        """Make positions ``first_position .. first_position+count-1``
        writable: allocate missing blocks, and copy-on-write any block in that
        range that another sequence still references.  Returns the
        ``(src, dst)`` copies this needs, in table order."""
        copies = []
        last = int(first_position) + int(count) - 1
        self.grow_to(last + 1)
        for j in range(int(first_position) // BLOCK, last // BLOCK + 1):
            b = self.table[j]
            if self.pool.ref[b] > 1:
                dst = self.pool.allocate()
                copies.append((b, dst))
                self.pool.release(b)
                self.table[j] = dst
        return copies

    def free(self):
        for b in self.table:
            self.pool.release(b)
        self.table = []
        self.num_tokens = 0


def tables_array(seqs, width=None, pad=0):
    """Block tables of ``seqs`` as an int32 ``[len(seqs)][width]`` array;
    unused entries hold ``pad`` (a valid block id, never read)."""
    width = width or max([len(s.table) for s in seqs] + [1])
    out = np.full((len(seqs), width), pad, dtype=np.int32)
    for i, s in enumerate(seqs):
        out[i, :len(s.table)] = s.table
    return out
