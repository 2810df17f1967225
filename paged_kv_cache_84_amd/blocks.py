"""Host KV block manager: a thin wrapper over the C ABI of
``include/pagedkv_blocks.h`` (block pool, reference counts, O(1) LRU free
queue, prefix-hash chain, copy-on-write).  Every decision is made in the
library; this class only marshals arguments and turns status codes into
exceptions.
"""

import ctypes

import numpy as np

from ._binding import PagedKVError, library

PKV_ERR_NO_BLOCKS = 7


class NoFreeBlocks(PagedKVError):
    """The free queue cannot supply the blocks an allocation needs."""


def _check(fn, status):
    if status == PKV_ERR_NO_BLOCKS:
        raise NoFreeBlocks(fn, status, "too few free blocks")
    if status != 0:
        raise PagedKVError(fn, status, library().pkv_status_string(status).decode())


def _i32(values):
    a = np.ascontiguousarray(np.asarray(values, dtype=np.int32))
    return a, a.ctypes.data_as(ctypes.c_void_p)


def _bytes(b):
    b = bytes(b)
    return (ctypes.c_char_p(b) if b else None), len(b)


class BlockManager:
    """Same operations and names as the pages' KV cache manager: requests
    are identified by integers."""

    def __init__(self, num_blocks, order=None, prefix_caching=True):
        self._lib = library()
        handle = ctypes.c_void_p()
        if order is not None:
            order_arr, order_ptr = _i32(order)
            if order_arr.shape != (int(num_blocks),):
                raise ValueError("order must list every block once")
        else:
            order_ptr = None
        _check("pkv_bm_create", self._lib.pkv_bm_create(int(num_blocks), order_ptr,
                                                        int(bool(prefix_caching)),
                                                        ctypes.byref(handle)))
        self._h = handle
        self.num_blocks = int(num_blocks)

    def close(self):
        if getattr(self, "_h", None):
            self._lib.pkv_bm_destroy(self._h)
            self._h = None

    def __del__(self):
        self.close()

    # -- operations
    def add_request(self, rid, prompt, extra=b"", salt=b""):
        arr, ptr = _i32(prompt)
        e, el = _bytes(extra)
        s, sl = _bytes(salt)
        cached = ctypes.c_int32()
        _check("pkv_bm_add_request", self._lib.pkv_bm_add_request(
            self._h, int(rid), ptr, arr.size, e, el, s, sl, ctypes.byref(cached)))
        return cached.value

    def append_tokens(self, rid, tokens):
        arr, ptr = _i32(tokens)
        _check("pkv_bm_append_tokens",
               self._lib.pkv_bm_append_tokens(self._h, int(rid), ptr, arr.size))

    def allocate(self, rid, num_new_tokens):
        _check("pkv_bm_allocate", self._lib.pkv_bm_allocate(self._h, int(rid),
                                                            int(num_new_tokens)))

    def append_tokens_batch(self, rids, tokens):
        """One token per request (a decode step's sampled tokens)."""
        ids = np.ascontiguousarray(np.asarray(rids, dtype=np.int64))
        tok, tptr = _i32(tokens)
        assert tok.shape == ids.shape
        _check("pkv_bm_append_tokens_batch", self._lib.pkv_bm_append_tokens_batch(
            self._h, ids.ctypes.data_as(ctypes.c_void_p), tptr, ids.size))

    def allocate_batch(self, rids, num_new_tokens):
        """allocate() for every request in order; returns the per-request
        status codes (0, or 7 for a request that did not fit)."""
        ids = np.ascontiguousarray(np.asarray(rids, dtype=np.int64))
        cnt, cptr = _i32(num_new_tokens)
        assert cnt.shape == ids.shape
        status = np.zeros(ids.size, dtype=np.int32)
        _check("pkv_bm_allocate_batch", self._lib.pkv_bm_allocate_batch(
            self._h, ids.ctypes.data_as(ctypes.c_void_p), cptr, ids.size,
            status.ctypes.data_as(ctypes.c_void_p)))
        return status

    def fork(self, parent_id, child_id):
        _check("pkv_bm_fork", self._lib.pkv_bm_fork(self._h, int(parent_id), int(child_id)))

    def free_request(self, rid):
        _check("pkv_bm_free_request", self._lib.pkv_bm_free_request(self._h, int(rid)))

    # -- queries
    def num_free(self):
        return self._lib.pkv_bm_num_free(self._h)

    def num_tokens(self, rid):
        n = self._lib.pkv_bm_num_tokens(self._h, int(rid))
        if n < 0:
            raise KeyError(rid)
        return n

    def ref_count(self, block):
        return self._lib.pkv_bm_ref_count(self._h, int(block))

    def table(self, rid):
        n = self._lib.pkv_bm_table(self._h, int(rid), None, 0)
        if n < 0:
            raise KeyError(rid)
        out = np.zeros(n, dtype=np.int32)
        self._lib.pkv_bm_table(self._h, int(rid), out.ctypes.data_as(ctypes.c_void_p), n)
        return [int(b) for b in out]

    def free_queue(self):
        n = self._lib.pkv_bm_free_queue(self._h, None, 0)
        out = np.zeros(n, dtype=np.int32)
        self._lib.pkv_bm_free_queue(self._h, out.ctypes.data_as(ctypes.c_void_p), n)
        return [int(b) for b in out]

    def take_copies(self):
        n = -self._lib.pkv_bm_take_copies(self._h, None, 0)
        out = np.zeros((max(n, 0), 2), dtype=np.int64)
        got = self._lib.pkv_bm_take_copies(self._h, out.ctypes.data_as(ctypes.c_void_p), n)
        assert got == n
        return [(int(a), int(b)) for a, b in out]

    def export_tables(self, rids, width, pad=0):
        """int32 [len(rids)][width] block tables, ready for the device."""
        ids = np.ascontiguousarray(np.asarray(rids, dtype=np.int64))
        out = np.zeros((ids.size, int(width)), dtype=np.int32)
        _check("pkv_bm_export_tables", self._lib.pkv_bm_export_tables(
            self._h, ids.ctypes.data_as(ctypes.c_void_p), ids.size,
            out.ctypes.data_as(ctypes.c_void_p), int(width), int(pad)))
        return out


def block_hash(parent, tokens, extra=b"", salt=b""):
    """The library's digest of one full block (32 bytes)."""
    assert len(parent) == 32 and len(tokens) == 16
    p = ctypes.create_string_buffer(bytes(parent), 32)
    arr, ptr = _i32(tokens)
    e, el = _bytes(extra)
    s, sl = _bytes(salt)
    out = ctypes.create_string_buffer(32)
    library().pkv_block_hash(p, ptr, e, el, s, sl, out)
    return out.raw


def sha256(data):
    data = bytes(data)
    out = ctypes.create_string_buffer(32)
    library().pkv_sha256(ctypes.c_char_p(data) if data else None, len(data), out)
    return out.raw
