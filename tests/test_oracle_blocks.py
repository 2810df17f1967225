"""Pins of the host block manager oracle (oracle/blocks.py) against what the
pages fix, and planted mistakes that the pins must catch.  CPU only."""

import numpy as np
import pytest

from oracle import blocks as K

B = K.BLOCK_SIZE


def ids(start, n):
    return list(range(start, start + n))


# --------------------------------------------------------------------------
# pins


def pin_fig2_tables(M=K.BlockManager):
    """[Anatomy] Fig. 2: 12 free blocks; A = 40 prompt tokens, B = 20 ->
    A: [0, 1, 2], B: [3, 4], blocks 5..11 free."""
    m = M(12, prefix_caching=False)
    m.add_request("A", ids(0, 40))
    m.allocate("A", 40)
    m.add_request("B", ids(1000, 20))
    m.allocate("B", 20)
    assert m.table("A") == [0, 1, 2]
    assert m.table("B") == [3, 4]
    assert m.free == list(range(5, 12))


def pin_fig4_chain(M=K.BlockManager):
    """[Anatomy] Fig. 4: request 2 repeats request 1's two full blocks and
    extends them; both blocks are reused, only the tail is new."""
    m = M(16)
    p1 = ids(0, 32)
    p2 = p1 + ids(500, 32)
    m.add_request(1, p1)
    m.allocate(1, 32)
    assert m.add_request(2, p2) == 32
    assert m.table(2) == m.table(1)
    assert all(m.ref[b] == 2 for b in m.table(1))
    m.allocate(2, 32)
    assert len(m.table(2)) == 4 and m.table(2)[:2] == m.table(1)
    assert not set(m.table(2)[2:]) & set(m.table(1))


def pin_partial_block_not_shared(M=K.BlockManager):
    """[Overview]: only full blocks are cached; a prefix that is not a
    multiple of 16 recomputes its last partial block."""
    m = M(8)
    m.add_request(1, ids(0, 20))
    m.allocate(1, 20)
    assert m.add_request(2, ids(0, 20)) == 16
    assert m.table(2) == m.table(1)[:1]


def pin_chain_needs_parent(M=K.BlockManager):
    """[Overview]: the hashes form a chain; a hit on a block means every
    earlier block matched.  Equal second blocks after different first blocks
    do not hit."""
    m = M(8)
    m.add_request(1, ids(0, 32))
    m.allocate(1, 32)
    assert m.add_request(2, ids(100, 16) + ids(16, 16)) == 0
    assert m.add_request(3, ids(0, 16) + ids(200, 16)) == 16
    # request 1's second block, as the first block of another prompt
    assert m.add_request(4, ids(16, 16)) == 0


def pin_extra_keys_and_salt(M=K.BlockManager):
    """[Overview]: the LoRA name (an extra key) and the cache salt enter the
    hash, so the same text under another adapter or another tenant's salt
    does not hit; the same adapter and salt do."""
    m = M(16)
    m.add_request(1, ids(0, 32), extra=b"lora-a", salt=b"tenant-1")
    m.allocate(1, 32)
    assert m.add_request(2, ids(0, 32), extra=b"lora-b", salt=b"tenant-1") == 0
    assert m.add_request(3, ids(0, 32), extra=b"lora-a", salt=b"tenant-2") == 0
    assert m.add_request(4, ids(0, 32)) == 0
    assert m.add_request(5, ids(0, 32), extra=b"lora-a", salt=b"tenant-1") == 32


def pin_lru_reuse(M=K.BlockManager):
    """[Overview]: allocation takes the queue head, release appends to the
    tail, a released block keeps its hash until it is handed out again.  With
    tail-first release a chain is evicted from its end."""
    m = M(4)
    m.add_request(1, ids(0, 32))
    m.allocate(1, 32)                       # blocks 0, 1, both hashed
    m.free_request(1)
    assert m.free == [2, 3, 1, 0]
    assert m.add_request(2, ids(0, 32)) == 32   # hits blocks still in the queue
    assert m.table(2) == [0, 1] and m.free == [2, 3]
    m.free_request(2)
    m.add_request(3, ids(900, 48))
    m.allocate(3, 48)                       # takes 2, 3, 1: block 1's hash is gone
    assert m.table(3) == [2, 3, 1]
    assert m.add_request(4, ids(0, 32)) == 16   # block 0 still hits, block 1 not
    assert m.table(4) == [0]


def pin_referenced_blocks_stay(M=K.BlockManager):
    """[V0/V1] §4: a block with ref_cnt > 0 cannot be evicted: with every
    block referenced, an allocation fails and changes nothing."""
    m = M(2)
    m.add_request(1, ids(0, 32))
    m.allocate(1, 32)
    m.add_request(2, ids(100, 16))
    with pytest.raises(K.NoFreeBlocks):
        m.allocate(2, 16)
    assert m.table(1) == [0, 1] and m.table(2) == [] and m.num_tokens(2) == 0
    assert m.free == [] and m.ref == [1, 1]


def pin_copy_on_write(M=K.BlockManager):
    """[Anatomy] copy-on-write paragraph: a writer into a block another
    sequence still references gets a copy; only the writer's table changes;
    once a block is no longer shared, writes go in place."""
    m = M(8, prefix_caching=False)
    m.add_request("p", ids(0, 20))
    m.allocate("p", 20)                     # [0, 1], block 1 half full
    m.fork("p", "c")                        # parallel sampling: share everything
    assert m.ref[0] == 2 and m.ref[1] == 2
    m.append_tokens("c", [77])
    m.allocate("c", 1)                      # position 20 lies in shared block 1
    assert m.take_copies() == [(1, 2)]
    assert m.table("c") == [0, 2] and m.table("p") == [0, 1]
    assert m.ref[1] == 1 and m.ref[0] == 2 and m.ref[2] == 1
    m.append_tokens("p", [78])
    m.allocate("p", 1)                      # block 1 is the parent's alone now
    assert m.take_copies() == []
    assert m.table("p") == [0, 1]


def _check_invariants(m):
    counts = np.zeros(m.num_blocks, dtype=np.int64)
    for r in m.requests.values():
        for b in r.table:
            counts[b] += 1
        assert len(r.table) == -(-r.num_tokens // B)
    assert list(counts) == m.ref
    assert sorted(m.free) == [b for b in range(m.num_blocks) if m.ref[b] == 0]
    assert len(set(m.free)) == len(m.free)
    for d, b in m.cached.items():
        assert m.hash[b] == d
    assert sum(h is not None for h in m.hash) == len(m.cached)


def random_trace(seed, num_blocks=48, steps=400):
    """A seeded sequence of block-manager operations over a small vocabulary
    of shared prefixes (so hits, forks, copies and evictions all occur)."""
    rng = np.random.default_rng(seed)
    prefixes = [list(rng.integers(0, 50, int(rng.integers(1, 70)))) for _ in range(6)]
    ops, live, nxt = [], [], 0
    for _ in range(steps):
        u = rng.random()
        if u < 0.3 or not live:
            p = list(prefixes[int(rng.integers(0, 6))])
            p += list(rng.integers(0, 50, int(rng.integers(0, 40))))
            extra = [b"", b"lora"][int(rng.integers(0, 2))]
            ops.append(("add", nxt, p, extra, b""))
            live.append(nxt)
            nxt += 1
        elif u < 0.65:
            r = live[int(rng.integers(0, len(live)))]
            ops.append(("step", r, int(rng.integers(1, 40)),
                        list(rng.integers(0, 50, 40))))
        elif u < 0.75:
            r = live[int(rng.integers(0, len(live)))]
            ops.append(("fork", r, nxt))
            live.append(nxt)
            nxt += 1
        else:
            r = live.pop(int(rng.integers(0, len(live))))
            ops.append(("free", r))
    return ops


def run_trace(m, ops, check=None):
    """Apply a trace; a step appends tokens as needed and allocates.  Returns
    the observable log (cached-token counts, failures, tables, copies)."""
    log = []
    for op in ops:
        if op[0] == "add":
            log.append(("add", m.add_request(op[1], op[2], extra=op[3], salt=op[4])))
        elif op[0] == "step":
            rid, n, more = op[1], op[2], op[3]
            known = len(m.requests[rid].tokens) - m.num_tokens(rid)
            if known < n:
                m.append_tokens(rid, more[:n - known])
            try:
                m.allocate(rid, n)
                log.append(("step", m.table(rid), m.take_copies()))
            except K.NoFreeBlocks:
                log.append(("step", "full"))
        elif op[0] == "fork":
            m.fork(op[1], op[2])
            log.append(("fork", m.table(op[2])))
        else:
            m.free_request(op[1])
            log.append(("free", m.num_free()))
        if check:
            check(m)
    return log


def pin_invariants_on_traces(M=K.BlockManager):
    """Reference counts equal table membership, the free queue holds exactly
    the unreferenced blocks, every cached hash names its block."""
    for seed in range(4):
        m = M(48)
        log = run_trace(m, random_trace(seed), check=_check_invariants)
        kinds = {e[0] for e in log}
        assert {"add", "step", "fork", "free"} <= kinds
        assert any(e[0] == "add" and e[1] > 0 for e in log)            # hits occur
        assert any(e[0] == "step" and e[1] != "full" and e[2] for e in log)   # copies occur


PINS = [pin_fig2_tables, pin_fig4_chain, pin_partial_block_not_shared, pin_chain_needs_parent,
        pin_extra_keys_and_salt, pin_lru_reuse, pin_referenced_blocks_stay, pin_copy_on_write,
        pin_invariants_on_traces]


@pytest.mark.parametrize("pin", PINS, ids=[p.__name__ for p in PINS])
def test_block_manager_pin(pin):
    pin()


def test_hash_encoding_is_sha256_of_the_stated_bytes():
    """The digest of a block is SHA-256 over parent | tokens | extra | salt,
    checked with an independently built message."""
    import hashlib
    import struct
    toks = list(range(100, 116))
    parent = bytes(range(32))
    msg = parent + b"".join(struct.pack("<i", t) for t in toks)
    msg += (3).to_bytes(4, "little") + b"xyz" + (2).to_bytes(4, "little") + b"s1"
    assert K.block_hash(parent, toks, b"xyz", b"s1") == hashlib.sha256(msg).digest()
    assert K.block_hash(parent, toks) != K.block_hash(K.NO_PARENT, toks)


# --------------------------------------------------------------------------
# planted mistakes


class _ReleaseHeadFirst(K.BlockManager):
    def free_request(self, rid):
        req = self.requests.pop(rid)
        for b in req.table:
            self._release(b)


class _HitStaysInQueue(K.BlockManager):
    def add_request(self, rid, prompt, extra=b"", salt=b""):
        req = K.Request(prompt, extra, salt)
        for j in range(len(req.tokens) // B):
            d = self._hash_of(req, j, req.parent)
            b = self.cached.get(d)
            if b is None:
                break
            self.ref[b] += 1
            req.table.append(b)
            req.parent, req.hashed = d, j + 1
        req.num_tokens = len(req.table) * B
        self.requests[rid] = req
        return req.num_tokens


class _KeepHashOnReuse(K.BlockManager):
    def _take_free(self):
        b = self.free.pop(0)
        self.ref[b] = 1
        return b


class _CopyEvenUnshared(K.BlockManager):
    def allocate(self, rid, num_new_tokens):
        req = self.requests[rid]
        j = req.num_tokens // B
        if num_new_tokens and j < len(req.table) and self.ref[req.table[j]] == 1:
            self.ref[req.table[j]] += 1            # pretend it is shared
        super().allocate(rid, num_new_tokens)


class _NoParentInHash(K.BlockManager):
    def _hash_of(self, req, j, parent):
        return K.block_hash(K.NO_PARENT, req.tokens[B * j:B * (j + 1)], req.extra,
                            req.salt if j == 0 else b"")


class _SaltIgnored(K.BlockManager):
    def _hash_of(self, req, j, parent):
        return K.block_hash(parent, req.tokens[B * j:B * (j + 1)], req.extra, b"")


class _AllocateFromTail(K.BlockManager):
    def _take_free(self):
        self.free.insert(0, self.free.pop())
        return super()._take_free()


MUTANTS = [_ReleaseHeadFirst, _HitStaysInQueue, _KeepHashOnReuse, _CopyEvenUnshared,
           _NoParentInHash, _SaltIgnored, _AllocateFromTail]


@pytest.mark.parametrize("mutant", MUTANTS, ids=[m.__name__ for m in MUTANTS])
def test_block_manager_mutant_is_caught(mutant):
    caught = []
    for pin in PINS:
        try:
            pin(mutant)
        except (AssertionError, K.NoFreeBlocks, KeyError, ValueError):
            caught.append(pin.__name__)
    assert caught, f"no pin catches {mutant.__name__}"
