"""Host KV block manager: the block pool, reference counts, the LRU free
queue, the prefix-hash chain and copy-on-write, written plainly.

TEST INFRASTRUCTURE ONLY (see the package docstring).

Sources ("the pages"):
  [Anatomy]   "vLLM 引擎解剖": "PagedAttention：为 KV 缓存分页" (Fig. 2 and the
              copy-on-write paragraph), "自动前缀缓存" (Fig. 4)
  [Overview]  "01. vLLM：从分页 KV 起家的通用推理引擎": "KV 缓存管理与前缀缓存"
  [V0/V1]     "v1/v0 区别": §4 "KV Cache 管理"

What the pages fix, step by step:
  * the pool is a fixed set of 16-token blocks; every free block sits in one
    LRU-ordered queue; allocation takes the block at the head, a released
    block goes back to the tail, and keeps its hash and contents until it is
    handed out again ([Overview]);
  * a block referenced by some request (ref count > 0) is never reused; a
    block whose count drops to zero waits in the free queue, still findable
    by its hash ([Overview]; [V0/V1] §4);
  * every *full* block gets a hash of (its parent block's hash, its 16 token
    ids, extra keys such as the LoRA adapter); the per-request cache salt
    enters the first block's hash only; a new request walks its prompt's
    blocks from the first and reuses blocks while the hashes hit, stopping at
    the first miss; a partial last block is never shared ([Overview];
    [Anatomy] "自动前缀缓存", Fig. 4);
  * a request that must write into a block another request still references
    gets a copy of that block, and only the writer's table changes
    ([Anatomy], copy-on-write paragraph); sharing all blocks of a request
    serves parallel sampling ([Anatomy], the "共享" paragraph).

Readings where the pages leave a step open (each listed in the design notes):
  * hash input, byte for byte: parent digest (32 zero bytes for the first
    block) | the 16 token ids as little-endian int32 | len(extra) as
    little-endian uint32 | extra | len(salt) as little-endian uint32 | salt
    (salt empty after the first block); SHA-256 (the pages' default);
  * when the hash of a newly full block is already held by another block, the
    new block stays unhashed (the cached block keeps serving hits);
  * a request is released tail first (its last block enters the free queue
    first), so the LRU queue evicts a chain from its end: a cached block is
    useless once an earlier block of its chain is gone;
  * one allocation step takes its copy-on-write blocks first (in table
    order), then its new blocks; if the free queue cannot supply all of them
    the step fails and nothing changes;
  * blocks are hashed when they are allocated for the tokens that fill them
    (the tokens' K/V are written in the same engine step).
"""

import hashlib
import struct

BLOCK_SIZE = 16
NO_PARENT = bytes(32)


def block_hash(parent, tokens, extra=b"", salt=b""):
    """SHA-256 of one full block's identity (encoding: module docstring)."""
    assert len(parent) == 32 and len(tokens) == BLOCK_SIZE
    msg = bytearray(parent)
    for t in tokens:
        msg += struct.pack("<i", int(t))
    msg += struct.pack("<I", len(extra)) + bytes(extra)
    msg += struct.pack("<I", len(salt)) + bytes(salt)
    return hashlib.sha256(bytes(msg)).digest()


class NoFreeBlocks(RuntimeError):
    pass


class Request:
    def __init__(self, tokens, extra, salt):
        self.tokens = list(tokens)     # every known token id (prompt + appended)
        self.extra = bytes(extra)
        self.salt = bytes(salt)
        self.table = []                # logical block -> physical block
        self.num_tokens = 0            # positions that own a slot
        self.hashed = 0                # leading blocks whose hash is known
        self.parent = NO_PARENT        # hash of block `hashed - 1`


class BlockManager:
    def __init__(self, num_blocks, order=None, prefix_caching=True):
        self.num_blocks = int(num_blocks)
        self.prefix_caching = bool(prefix_caching)
        self.ref = [0] * self.num_blocks
        self.hash = [None] * self.num_blocks
        self.free = [int(b) for b in (range(self.num_blocks) if order is None else order)]
        assert sorted(self.free) == list(range(self.num_blocks))
        self.cached = {}               # digest -> block
        self.requests = {}
        self.copies = []               # (src, dst) copies since the last take

    # -- the free queue: head = self.free[0], tail = self.free[-1]
    def _take_free(self):
        b = self.free.pop(0)
        if self.hash[b] is not None:   # reuse ends its life as a cached block
            del self.cached[self.hash[b]]
            self.hash[b] = None
        self.ref[b] = 1
        return b

    def _release(self, b):
        self.ref[b] -= 1
        assert self.ref[b] >= 0
        if self.ref[b] == 0:
            self.free.append(b)

    def _hash_of(self, req, j, parent):
        return block_hash(parent, req.tokens[BLOCK_SIZE * j:BLOCK_SIZE * (j + 1)], req.extra,
                          req.salt if j == 0 else b"")

    # -- requests
    def add_request(self, rid, prompt, extra=b"", salt=b""):
        """Register a request; reuse its prompt's cached prefix blocks.
        Returns the number of prompt tokens whose K/V are already cached."""
        assert rid not in self.requests
        req = Request(prompt, extra, salt)
        if self.prefix_caching:
            for j in range(len(req.tokens) // BLOCK_SIZE):
                d = self._hash_of(req, j, req.parent)
                b = self.cached.get(d)
                if b is None:
                    break
                if self.ref[b] == 0:
                    self.free.remove(b)
                self.ref[b] += 1
                req.table.append(b)
                req.parent = d
                req.hashed = j + 1
        req.num_tokens = len(req.table) * BLOCK_SIZE
        self.requests[rid] = req
        return req.num_tokens

    def append_tokens(self, rid, tokens):
        self.requests[rid].tokens.extend(int(t) for t in tokens)

    def allocate(self, rid, num_new_tokens):
        """Give positions num_tokens .. num_tokens + num_new_tokens - 1 of the
        request a writable slot: copy shared blocks in that range, add new
        blocks, then hash the blocks that became full."""
        req = self.requests[rid]
        first = req.num_tokens
        end = first + int(num_new_tokens)
        assert num_new_tokens >= 0 and end <= len(req.tokens)
        if num_new_tokens == 0:
            return
        need = -(-end // BLOCK_SIZE) - len(req.table)
        shared = [j for j in range(first // BLOCK_SIZE, len(req.table))
                  if j <= (end - 1) // BLOCK_SIZE and self.ref[req.table[j]] > 1]
        if max(need, 0) + len(shared) > len(self.free):
            raise NoFreeBlocks(f"need {max(need, 0) + len(shared)}, free {len(self.free)}")
        for j in shared:
            src = req.table[j]
            dst = self._take_free()
            self.copies.append((src, dst))
            self._release(src)
            req.table[j] = dst
        for _ in range(max(need, 0)):
            req.table.append(self._take_free())
        req.num_tokens = end
        if self.prefix_caching:
            for j in range(req.hashed, end // BLOCK_SIZE):
                d = self._hash_of(req, j, req.parent)
                b = req.table[j]
                if d not in self.cached and self.hash[b] is None:
                    self.cached[d] = b
                    self.hash[b] = d
                req.parent = d
                req.hashed = j + 1

    def fork(self, parent_id, child_id):
        """A new request sharing every block (and token) of an existing one."""
        assert child_id not in self.requests
        p = self.requests[parent_id]
        c = Request(p.tokens, p.extra, p.salt)
        c.table = list(p.table)
        c.num_tokens, c.hashed, c.parent = p.num_tokens, p.hashed, p.parent
        for b in c.table:
            self.ref[b] += 1
        self.requests[child_id] = c

    def free_request(self, rid):
        req = self.requests.pop(rid)
        for b in reversed(req.table):
            self._release(b)

    # -- queries
    def table(self, rid):
        return list(self.requests[rid].table)

    def num_tokens(self, rid):
        return self.requests[rid].num_tokens

    def num_free(self):
        return len(self.free)

    def take_copies(self):
        out, self.copies = self.copies, []
        return out
