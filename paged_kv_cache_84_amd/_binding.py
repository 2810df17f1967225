"""ctypes marshalling for libpagedkv.so.  Argument checks and pointers only."""

import ctypes
import os

import torch

HERE = os.path.dirname(os.path.abspath(__file__))
BLOCK_SIZE = 16

PKV_F32, PKV_BF16, PKV_FP8_E4M3, PKV_INT4, PKV_NVFP4 = 0, 1, 2, 3, 4
_STATUS = {0: "ok", 1: "null pointer", 2: "misaligned pointer", 3: "bad shape",
           4: "unsupported", 5: "workspace too small", 6: "launch failed"}


class LibraryNotBuilt(RuntimeError):
    """libpagedkv.so is missing or failed to load."""


class PagedKVError(RuntimeError):
    def __init__(self, fn, status, text):
        super().__init__(f"{fn} failed: status {status} ({text})")
        self.status = status


def library_path():
    return os.environ.get("PAGEDKV_LIB", os.path.join(HERE, "libpagedkv.so"))


_lib = None

_c = ctypes
_P, _I32, _I64, _F, _SZ = _c.c_void_p, _c.c_int32, _c.c_int64, _c.c_float, _c.c_size_t
_SIGNATURES = {
    "pkv_block_size": (_I32, []),
    "pkv_status_string": (_c.c_char_p, [_I32]),
    "kv_bytes_per_token": (_I64, [_I32, _I32, _I32, _I32]),
    "compute_slot_mapping": (_I32, [_P, _I32, _P, _P, _I32, _I32, _P, _I32, _P]),
    "reshape_and_cache": (_I32, [_P, _P, _P, _P, _P, _I32, _I32, _I32, _I32, _I32,
                                 _I32, _F, _F, _P]),
    "copy_blocks": (_I32, [_P, _P, _I32, _P, _I32, _I32, _I64, _P]),
    "reshape_and_cache_from_schedule": (_I32, [_P, _P, _P, _P, _P, _I32, _P, _P, _I32, _P,
                                               _I32, _I32, _I32, _I32, _I32, _I32, _F, _F,
                                               _P]),
    "swap_blocks": (_I32, [_P, _P, _P, _P, _I32, _P, _I32, _I32, _I32, _I64, _P]),
    "paged_attention_decode_workspace_size": (_SZ, [_I32, _I32, _I32, _I32, _I32, _I32]),
    "paged_attention_decode_num_chunks": (_I32, [_I32, _I32, _I32, _I32, _I32]),
    "paged_attention_decode": (_I32, [_P, _P, _P, _P, _I32, _P, _I32, _P, _I32, _I32,
                                      _I32, _I32, _I32, _F, _I32, _I32, _F, _F, _I32,
                                      _P, _SZ, _P]),
    "paged_attention_decode_noalloc": (_I32, [_P, _P, _P, _P, _I32, _P, _I32, _P, _I32, _I32,
                                              _I32, _I32, _I32, _F, _I32, _I32, _F, _F, _I32,
                                              _P]),
    "paged_attention_decode_append": (_I32, [_P, _P, _P, _P, _P, _P, _I32, _P, _I32, _P, _I32,
                                             _I32, _I32, _I32, _I32, _F, _I32, _I32, _F, _F,
                                             _I32, _P, _SZ, _P]),
    "paged_attention_decode_sliding": (_I32, [_P, _P, _P, _P, _I32, _P, _I32, _P, _I32, _I32,
                                              _I32, _I32, _I32, _F, _I32, _I32, _F, _F, _I32,
                                              _I32, _P, _SZ, _P]),
    "reshape_and_cache_int4": (_I32, [_P, _P, _P, _P, _P, _P, _P, _I32, _I32, _I32, _I32,
                                      _I32, _P]),
    "paged_attention_decode_int4": (_I32, [_P, _P, _P, _P, _P, _P, _I32, _P, _I32, _P, _I32,
                                           _I32, _I32, _I32, _I32, _F, _I32, _I32, _P, _SZ,
                                           _P]),
    "reshape_and_cache_nvfp4": (_I32, [_P, _P, _P, _P, _P, _P, _P, _I32, _I32, _I32, _I32,
                                       _I32, _F, _F, _P]),
    "paged_attention_decode_nvfp4": (_I32, [_P, _P, _P, _P, _P, _P, _I32, _P, _I32, _P, _I32,
                                            _I32, _I32, _I32, _I32, _F, _I32, _F, _F, _I32, _P,
                                            _SZ, _P]),
    "paged_attention_varlen_workspace_size": (_SZ, [_I32, _I32, _I32, _I32, _I32]),
    "paged_attention_varlen": (_I32, [_P, _P, _P, _P, _I32, _P, _I32, _P, _P, _I32, _I32,
                                      _I32, _I32, _I32, _I32, _F, _I32, _I32, _P, _SZ, _P]),
    "paged_attention_prefill_chunk": (_I32, [_P, _P, _P, _P, _I32, _P, _I32, _P, _P,
                                             _I32, _I32, _I32, _I32, _I32, _I32, _F,
                                             _I32, _I32, _F, _F, _P]),
    # hardware ceilings (include/pagedkv_measure.h)
    "pkv_measure_hbm_read": (_I32, [_P, _I64, _P, _P]),
    "pkv_measure_mfma_bf16": (_I32, [_I32, _I32, _P, _P]),
    "pkv_measure_mfma_valu": (_I32, [_I32, _I32, _I32, _P, _P]),
    # host block manager (include/pagedkv_blocks.h)
    "pkv_bm_create": (_I32, [_I32, _P, _I32, _P]),
    "pkv_bm_destroy": (None, [_P]),
    "pkv_bm_add_request": (_I32, [_P, _I64, _P, _I32, _P, _I32, _P, _I32, _P]),
    "pkv_bm_append_tokens": (_I32, [_P, _I64, _P, _I32]),
    "pkv_bm_allocate": (_I32, [_P, _I64, _I32]),
    "pkv_bm_append_tokens_batch": (_I32, [_P, _P, _P, _I32]),
    "pkv_bm_allocate_batch": (_I32, [_P, _P, _P, _I32, _P]),
    "pkv_bm_fork": (_I32, [_P, _I64, _I64]),
    "pkv_bm_free_request": (_I32, [_P, _I64]),
    "pkv_bm_num_free": (_I32, [_P]),
    "pkv_bm_num_tokens": (_I32, [_P, _I64]),
    "pkv_bm_ref_count": (_I32, [_P, _I32]),
    "pkv_bm_table": (_I32, [_P, _I64, _P, _I32]),
    "pkv_bm_free_queue": (_I32, [_P, _P, _I32]),
    "pkv_bm_take_copies": (_I32, [_P, _P, _I32]),
    "pkv_bm_export_tables": (_I32, [_P, _P, _I32, _P, _I32, _I32]),
    "pkv_block_hash": (None, [_P, _P, _P, _I32, _P, _I32, _P]),
    "pkv_sha256": (None, [_P, _SZ, _P]),
}
EXPORTED = tuple(_SIGNATURES)


def library():
    """The loaded library (loaded once).  torch is imported first so that the
    library binds to the HIP runtime torch already uses."""
    global _lib
    if _lib is None:
        path = library_path()
        if not os.path.exists(path):
            raise LibraryNotBuilt(
                f"{path} not found; build it with python -m paged_kv_cache_84_amd.build")
        try:
            lib = ctypes.CDLL(path)
        except OSError as e:
            raise LibraryNotBuilt(f"cannot load {path}: {e}") from e
        for name, (res, args) in _SIGNATURES.items():
            fn = getattr(lib, name)
            fn.restype, fn.argtypes = res, args
        _lib = lib
    return _lib


def _check(fn, status):
    if status != 0:
        text = library().pkv_status_string(status).decode()
        raise PagedKVError(fn, status, text)


def _dtype_code(t, what):
    if t.dtype == torch.float32:
        return PKV_F32
    if t.dtype == torch.bfloat16:
        return PKV_BF16
    if t.dtype in (torch.uint8, torch.float8_e4m3fn):
        return PKV_FP8_E4M3
    raise TypeError(f"{what}: unsupported dtype {t.dtype}")


def _dev(t, what, dtype=None):
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{what} must be a torch.Tensor")
    if not t.is_cuda:
        raise ValueError(f"{what} must be on the GPU")
    if not t.is_contiguous():
        raise ValueError(f"{what} must be contiguous")
    if dtype is not None and t.dtype != dtype:
        raise TypeError(f"{what} must be {dtype}, got {t.dtype}")
    return t.data_ptr()


def _stream(t):
    return torch.cuda.current_stream(t.device).cuda_stream


def kv_bytes_per_token(num_layers, num_kv_heads, head_dim, bytes_per_elem):
    return int(library().kv_bytes_per_token(num_layers, num_kv_heads, head_dim,
                                            bytes_per_elem))


def compute_slot_mapping(block_tables, query_start_loc, num_computed_tokens,
                         num_blocks, num_tokens, out=None):
    """int64 [num_tokens] slots of the step's tokens (see the header)."""
    num_reqs = num_computed_tokens.shape[0]
    if out is None:
        out = torch.empty(num_tokens, dtype=torch.int64, device=block_tables.device)
    assert block_tables.dim() == 2 and block_tables.shape[0] >= num_reqs
    assert query_start_loc.shape[0] == num_reqs + 1 and out.shape[0] >= num_tokens
    st = library().compute_slot_mapping(
        _dev(block_tables, "block_tables", torch.int32), block_tables.shape[1],
        _dev(query_start_loc, "query_start_loc", torch.int32),
        _dev(num_computed_tokens, "num_computed_tokens", torch.int32), num_reqs,
        int(num_blocks), _dev(out, "slot_mapping", torch.int64), int(num_tokens),
        _stream(out))
    _check("compute_slot_mapping", st)
    return out


def reshape_and_cache(key, value, k_cache, v_cache, slot_mapping, k_scale=1.0,
                      v_scale=1.0):
    """Write key/value [T][Hkv][D] into the caches at the given slots."""
    t, hkv, d = key.shape
    assert value.shape == key.shape and key.dtype == value.dtype
    assert k_cache.shape == v_cache.shape and k_cache.shape[1:] == (hkv, BLOCK_SIZE, d)
    assert slot_mapping.shape[0] >= t
    st = library().reshape_and_cache(
        _dev(key, "key"), _dev(value, "value"), _dev(k_cache, "k_cache"),
        _dev(v_cache, "v_cache"), _dev(slot_mapping, "slot_mapping", torch.int64),
        t, hkv, d, k_cache.shape[0], _dtype_code(key, "key"),
        _dtype_code(k_cache, "k_cache"), float(k_scale), float(v_scale), _stream(key))
    _check("reshape_and_cache", st)


def copy_blocks(k_caches, v_caches, block_mapping):
    """Copy whole blocks (src, dst) = block_mapping[i] in every layer."""
    n = len(k_caches)
    assert len(v_caches) == n and n > 0
    shape, dtype = k_caches[0].shape, k_caches[0].dtype
    for c in list(k_caches) + list(v_caches):
        assert c.shape == shape and c.dtype == dtype
        _dev(c, "cache")
    block_bytes = k_caches[0][0].numel() * k_caches[0].element_size()
    ks = (ctypes.c_void_p * n)(*[c.data_ptr() for c in k_caches])
    vs = (ctypes.c_void_p * n)(*[c.data_ptr() for c in v_caches])
    pairs = block_mapping.reshape(-1, 2)
    st = library().copy_blocks(ks, vs, n, _dev(block_mapping, "block_mapping", torch.int64),
                               pairs.shape[0], shape[0], block_bytes,
                               _stream(k_caches[0]))
    _check("copy_blocks", st)


def _dev_or_pinned(t, what):
    """Device tensor, or pinned host tensor (reachable through its device
    mapping); contiguous."""
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{what} must be a torch.Tensor")
    if not (t.is_cuda or t.is_pinned()):
        raise ValueError(f"{what} must be on the GPU or in pinned host memory")
    if not t.is_contiguous():
        raise ValueError(f"{what} must be contiguous")
    return t.data_ptr()


def swap_blocks(src_k_caches, src_v_caches, dst_k_caches, dst_v_caches, block_mapping,
                stream_device=None):
    """dst[d] = src[s] for every (s, d) = block_mapping[i], every layer, K and
    V; pools on the GPU or in pinned host memory (see the header)."""
    n = len(src_k_caches)
    assert n > 0 and len(src_v_caches) == n and len(dst_k_caches) == n and len(dst_v_caches) == n
    s_shape, d_shape = src_k_caches[0].shape, dst_k_caches[0].shape
    assert s_shape[1:] == d_shape[1:], "source and destination blocks differ in shape"
    dtype = src_k_caches[0].dtype
    for c in list(src_k_caches) + list(src_v_caches):
        assert c.shape == s_shape and c.dtype == dtype
        _dev_or_pinned(c, "source cache")
    for c in list(dst_k_caches) + list(dst_v_caches):
        assert c.shape == d_shape and c.dtype == dtype
        _dev_or_pinned(c, "destination cache")
    block_bytes = src_k_caches[0][0].numel() * src_k_caches[0].element_size()
    arr = lambda ts: (ctypes.c_void_p * n)(*[c.data_ptr() for c in ts])
    if block_mapping.dtype != torch.int64:
        raise TypeError("block_mapping must be int64")
    pairs = block_mapping.reshape(-1, 2)
    dev = torch.device("cuda", torch.cuda.current_device()) if stream_device is None else stream_device
    st = library().swap_blocks(arr(src_k_caches), arr(src_v_caches), arr(dst_k_caches),
                               arr(dst_v_caches), n, _dev_or_pinned(block_mapping, "block_mapping"),
                               pairs.shape[0], s_shape[0], d_shape[0], block_bytes,
                               torch.cuda.current_stream(dev).cuda_stream)
    _check("swap_blocks", st)


def decode_num_chunks(num_seqs, num_q_heads, num_kv_heads, max_context_len,
                      partition_tokens=0):
    return int(library().paged_attention_decode_num_chunks(
        num_seqs, num_q_heads, num_kv_heads, max_context_len, partition_tokens))


def decode_workspace_size(num_seqs, num_q_heads, num_kv_heads, head_dim,
                          max_context_len, partition_tokens=0):
    return int(library().paged_attention_decode_workspace_size(
        num_seqs, num_q_heads, num_kv_heads, head_dim, max_context_len,
        partition_tokens))


def paged_attention_decode(query, k_cache, v_cache, block_tables, context_lens,
                           max_context_len, softmax_scale, k_scale=1.0, v_scale=1.0,
                           partition_tokens=0, out=None, workspace=None):
    """out [S][Hq][D] (q dtype) = paged decode attention (see the header)."""
    s, hq, d = query.shape
    hkv = k_cache.shape[1]
    if out is None:
        out = torch.empty_like(query)
    need = decode_workspace_size(s, hq, hkv, d, max_context_len, partition_tokens)
    if workspace is None:
        workspace = torch.zeros(max(need, 16), dtype=torch.uint8, device=query.device)
    assert block_tables.shape[0] >= s and context_lens.shape[0] >= s
    st = library().paged_attention_decode(
        _dev(out, "out", query.dtype), _dev(query, "query"), _dev(k_cache, "k_cache"),
        _dev(v_cache, "v_cache"), k_cache.shape[0],
        _dev(block_tables, "block_tables", torch.int32), block_tables.shape[1],
        _dev(context_lens, "context_lens", torch.int32), s, int(max_context_len), hq,
        hkv, d, float(softmax_scale), _dtype_code(query, "query"),
        _dtype_code(k_cache, "k_cache"), float(k_scale), float(v_scale),
        int(partition_tokens), _dev(workspace, "workspace"),
        workspace.numel() * workspace.element_size(), _stream(query))
    _check("paged_attention_decode", st)
    return out


def paged_attention_decode_noalloc(query, k_cache, v_cache, block_tables, context_lens,
                                   max_context_len, softmax_scale, out, k_scale=1.0,
                                   v_scale=1.0, partition_tokens=0):
    """paged_attention_decode with its partials in the library's per-device
    scratch array (see the header): no workspace, and nothing allocated here
    either, so `out` must be given."""
    s, hq, d = query.shape
    hkv = k_cache.shape[1]
    assert block_tables.shape[0] >= s and context_lens.shape[0] >= s
    with torch.cuda.device(query.device):
        st = library().paged_attention_decode_noalloc(
            _dev(out, "out", query.dtype), _dev(query, "query"), _dev(k_cache, "k_cache"),
            _dev(v_cache, "v_cache"), k_cache.shape[0],
            _dev(block_tables, "block_tables", torch.int32), block_tables.shape[1],
            _dev(context_lens, "context_lens", torch.int32), s, int(max_context_len), hq,
            hkv, d, float(softmax_scale), _dtype_code(query, "query"),
            _dtype_code(k_cache, "k_cache"), float(k_scale), float(v_scale),
            int(partition_tokens), _stream(query))
    _check("paged_attention_decode_noalloc", st)
    return out


def paged_attention_decode_sliding(query, k_cache, v_cache, block_tables, context_lens,
                                   max_context_len, softmax_scale, sliding_window,
                                   k_scale=1.0, v_scale=1.0, partition_tokens=0, out=None,
                                   workspace=None):
    """Decode over each sequence's last `sliding_window` tokens (see the header)."""
    s, hq, d = query.shape
    hkv = k_cache.shape[1]
    if out is None:
        out = torch.empty_like(query)
    need = decode_workspace_size(s, hq, hkv, d, max_context_len, partition_tokens)
    if workspace is None:
        workspace = torch.empty(max(need, 16), dtype=torch.uint8, device=query.device)
    assert block_tables.shape[0] >= s and context_lens.shape[0] >= s
    st = library().paged_attention_decode_sliding(
        _dev(out, "out", query.dtype), _dev(query, "query"), _dev(k_cache, "k_cache"),
        _dev(v_cache, "v_cache"), k_cache.shape[0],
        _dev(block_tables, "block_tables", torch.int32), block_tables.shape[1],
        _dev(context_lens, "context_lens", torch.int32), s, int(max_context_len), hq,
        hkv, d, float(softmax_scale), _dtype_code(query, "query"),
        _dtype_code(k_cache, "k_cache"), float(k_scale), float(v_scale), int(sliding_window),
        int(partition_tokens), _dev(workspace, "workspace"),
        workspace.numel() * workspace.element_size(), _stream(query))
    _check("paged_attention_decode_sliding", st)
    return out


def paged_attention_prefill_chunk(query, k_cache, v_cache, block_tables,
                                  query_start_loc, num_computed_tokens, max_query_len,
                                  softmax_scale, k_scale=1.0, v_scale=1.0, out=None):
    """out [Tq][Hq][D] (q dtype) = causal attention of the chunks' rows."""
    t, hq, d = query.shape
    hkv = k_cache.shape[1]
    r = num_computed_tokens.shape[0]
    if out is None:
        out = torch.empty_like(query)
    assert query_start_loc.shape[0] == r + 1 and block_tables.shape[0] >= r
    st = library().paged_attention_prefill_chunk(
        _dev(out, "out", query.dtype), _dev(query, "query"), _dev(k_cache, "k_cache"),
        _dev(v_cache, "v_cache"), k_cache.shape[0],
        _dev(block_tables, "block_tables", torch.int32), block_tables.shape[1],
        _dev(query_start_loc, "query_start_loc", torch.int32),
        _dev(num_computed_tokens, "num_computed_tokens", torch.int32), r, t,
        int(max_query_len), hq, hkv, d, float(softmax_scale),
        _dtype_code(query, "query"), _dtype_code(k_cache, "k_cache"), float(k_scale),
        float(v_scale), _stream(query))
    _check("paged_attention_prefill_chunk", st)
    return out


def varlen_workspace_size(num_reqs, num_q_tokens, num_kv_heads, head_dim, max_seq_len):
    return int(library().paged_attention_varlen_workspace_size(num_reqs, num_q_tokens,
                                                               num_kv_heads, head_dim,
                                                               max_seq_len))


def paged_attention_varlen(query, k_cache, v_cache, block_tables, query_start_loc,
                           num_computed_tokens, max_seq_len, softmax_scale, out=None,
                           workspace=None):
    """out [T][Hq][D] = causal attention of every request's rows, one launch
    (see the header).  `workspace`: device bytes for the per-run partials,
    any contents; allocated here when not given."""
    t, hq, d = query.shape
    hkv = k_cache.shape[1]
    r = num_computed_tokens.shape[0]
    if out is None:
        out = torch.empty_like(query)
    need = varlen_workspace_size(r, t, hkv, d, max_seq_len)
    if workspace is None:
        workspace = torch.empty(max(need, 16), dtype=torch.uint8, device=query.device)
    assert query_start_loc.shape[0] == r + 1 and block_tables.shape[0] >= r
    st = library().paged_attention_varlen(
        _dev(out, "out", query.dtype), _dev(query, "query"), _dev(k_cache, "k_cache"),
        _dev(v_cache, "v_cache"), k_cache.shape[0],
        _dev(block_tables, "block_tables", torch.int32), block_tables.shape[1],
        _dev(query_start_loc, "query_start_loc", torch.int32),
        _dev(num_computed_tokens, "num_computed_tokens", torch.int32), r, t,
        int(max_seq_len), hq, hkv, d, float(softmax_scale), _dtype_code(query, "query"),
        _dtype_code(k_cache, "k_cache"), _dev(workspace, "workspace"),
        workspace.numel() * workspace.element_size(), _stream(query))
    _check("paged_attention_varlen", st)
    return out


def reshape_and_cache_int4(key, value, k_cache, v_cache, k_scales, v_scales, slot_mapping):
    """Quantise key/value [T][Hkv][D] (bf16 or fp32) into int4 caches
    [NB][Hkv][16][D/2] (uint8) with scales [NB][Hkv][16] (float32)."""
    t, hkv, d = key.shape
    assert value.shape == key.shape and key.dtype == value.dtype
    assert k_cache.shape == v_cache.shape and k_cache.shape[1:] == (hkv, BLOCK_SIZE, d // 2)
    assert k_scales.shape == v_scales.shape == k_cache.shape[:3]
    st = library().reshape_and_cache_int4(
        _dev(key, "key"), _dev(value, "value"), _dev(k_cache, "k_cache", torch.uint8),
        _dev(v_cache, "v_cache", torch.uint8), _dev(k_scales, "k_scales", torch.float32),
        _dev(v_scales, "v_scales", torch.float32),
        _dev(slot_mapping, "slot_mapping", torch.int64), t, hkv, d, k_cache.shape[0],
        _dtype_code(key, "key"), _stream(key))
    _check("reshape_and_cache_int4", st)


def paged_attention_decode_int4(query, k_cache, v_cache, k_scales, v_scales, block_tables,
                                context_lens, max_context_len, softmax_scale,
                                partition_tokens=0, out=None, workspace=None):
    """Decode over int4 caches; same contract as paged_attention_decode."""
    s, hq, d = query.shape
    hkv = k_cache.shape[1]
    if out is None:
        out = torch.empty_like(query)
    need = decode_workspace_size(s, hq, hkv, d, max_context_len, partition_tokens)
    if workspace is None:
        workspace = torch.empty(max(need, 16), dtype=torch.uint8, device=query.device)
    st = library().paged_attention_decode_int4(
        _dev(out, "out", query.dtype), _dev(query, "query"),
        _dev(k_cache, "k_cache", torch.uint8), _dev(v_cache, "v_cache", torch.uint8),
        _dev(k_scales, "k_scales", torch.float32), _dev(v_scales, "v_scales", torch.float32),
        k_cache.shape[0], _dev(block_tables, "block_tables", torch.int32),
        block_tables.shape[1], _dev(context_lens, "context_lens", torch.int32), s,
        int(max_context_len), hq, hkv, d, float(softmax_scale), _dtype_code(query, "query"),
        int(partition_tokens), _dev(workspace, "workspace"),
        workspace.numel() * workspace.element_size(), _stream(query))
    _check("paged_attention_decode_int4", st)
    return out


def reshape_and_cache_nvfp4(key, value, k_cache, v_cache, k_bscales, v_bscales, slot_mapping,
                            k_scale, v_scale):
    """Encode key/value [T][Hkv][D] (bf16 or fp32) into nvfp4 caches
    [NB][Hkv][16][D/2] (uint8 E2M1 pairs) with block scales
    [NB][Hkv][16][D/16] (uint8 E4M3) under the per-tensor scales."""
    t, hkv, d = key.shape
    assert value.shape == key.shape and key.dtype == value.dtype
    assert k_cache.shape == v_cache.shape and k_cache.shape[1:] == (hkv, BLOCK_SIZE, d // 2)
    assert k_bscales.shape == v_bscales.shape == k_cache.shape[:3] + (d // 16,)
    st = library().reshape_and_cache_nvfp4(
        _dev(key, "key"), _dev(value, "value"), _dev(k_cache, "k_cache", torch.uint8),
        _dev(v_cache, "v_cache", torch.uint8), _dev(k_bscales, "k_bscales", torch.uint8),
        _dev(v_bscales, "v_bscales", torch.uint8),
        _dev(slot_mapping, "slot_mapping", torch.int64), t, hkv, d, k_cache.shape[0],
        _dtype_code(key, "key"), float(k_scale), float(v_scale), _stream(key))
    _check("reshape_and_cache_nvfp4", st)


def paged_attention_decode_nvfp4(query, k_cache, v_cache, k_bscales, v_bscales, block_tables,
                                 context_lens, max_context_len, softmax_scale, k_scale,
                                 v_scale, partition_tokens=0, out=None, workspace=None):
    """Decode over nvfp4 caches; same contract as paged_attention_decode."""
    s, hq, d = query.shape
    hkv = k_cache.shape[1]
    if out is None:
        out = torch.empty_like(query)
    need = decode_workspace_size(s, hq, hkv, d, max_context_len, partition_tokens)
    if workspace is None:
        workspace = torch.empty(max(need, 16), dtype=torch.uint8, device=query.device)
    st = library().paged_attention_decode_nvfp4(
        _dev(out, "out", query.dtype), _dev(query, "query"),
        _dev(k_cache, "k_cache", torch.uint8), _dev(v_cache, "v_cache", torch.uint8),
        _dev(k_bscales, "k_bscales", torch.uint8), _dev(v_bscales, "v_bscales", torch.uint8),
        k_cache.shape[0], _dev(block_tables, "block_tables", torch.int32),
        block_tables.shape[1], _dev(context_lens, "context_lens", torch.int32), s,
        int(max_context_len), hq, hkv, d, float(softmax_scale), _dtype_code(query, "query"),
        float(k_scale), float(v_scale), int(partition_tokens), _dev(workspace, "workspace"),
        workspace.numel() * workspace.element_size(), _stream(query))
    _check("paged_attention_decode_nvfp4", st)
    return out


def measure_hbm_read(buf, checksum):
    """Stream every byte of the device tensor `buf` (16-byte multiple) with
    the decode's load kind; `checksum` (int32 [1], device) receives the XOR
    of its 32-bit words."""
    nbytes = buf.numel() * buf.element_size()
    st = library().pkv_measure_hbm_read(_dev(buf, "buf"), nbytes,
                                        _dev(checksum, "checksum", torch.int32), _stream(buf))
    _check("pkv_measure_hbm_read", st)


def measure_mfma_bf16(iterations, result):
    """Register-only loop of bf16 MFMAs on `result.numel()` waves; each
    writes 32 * iterations into its slot of `result` (float32, device)."""
    st = library().pkv_measure_mfma_bf16(int(iterations), result.numel(),
                                         _dev(result, "result", torch.float32), _stream(result))
    _check("pkv_measure_mfma_bf16", st)


def measure_mfma_valu(iterations, mode, result):
    """MFMA loop (mode 0), the softmax-like vector work (1) or both from the
    same waves (2) on `result.numel() // 2` waves (see the header)."""
    st = library().pkv_measure_mfma_valu(int(iterations), result.numel() // 2, int(mode),
                                         _dev(result, "result", torch.float32), _stream(result))
    _check("pkv_measure_mfma_valu", st)


def reshape_and_cache_from_schedule(key, value, k_cache, v_cache, block_tables,
                                    query_start_loc, num_computed_tokens, k_scale=1.0,
                                    v_scale=1.0, slot_mapping=None):
    """compute_slot_mapping + reshape_and_cache in one launch; the slots go
    to `slot_mapping` (int64 [T]) when given."""
    t, hkv, d = key.shape
    assert value.shape == key.shape and key.dtype == value.dtype
    assert k_cache.shape == v_cache.shape and k_cache.shape[1:] == (hkv, BLOCK_SIZE, d)
    r = num_computed_tokens.shape[0]
    assert query_start_loc.shape[0] == r + 1 and block_tables.shape[0] >= r
    sm = 0 if slot_mapping is None else _dev(slot_mapping, "slot_mapping", torch.int64)
    st = library().reshape_and_cache_from_schedule(
        _dev(key, "key"), _dev(value, "value"), _dev(k_cache, "k_cache"),
        _dev(v_cache, "v_cache"), _dev(block_tables, "block_tables", torch.int32),
        block_tables.shape[1], _dev(query_start_loc, "query_start_loc", torch.int32),
        _dev(num_computed_tokens, "num_computed_tokens", torch.int32), r, sm or None, t, hkv,
        d, k_cache.shape[0], _dtype_code(key, "key"), _dtype_code(k_cache, "k_cache"),
        float(k_scale), float(v_scale), _stream(key))
    _check("reshape_and_cache_from_schedule", st)


def paged_attention_decode_append(query, new_key, new_value, k_cache, v_cache, block_tables,
                                  context_lens, max_context_len, softmax_scale, k_scale=1.0,
                                  v_scale=1.0, partition_tokens=0, out=None, workspace=None):
    """Write each sequence's new K/V row at position L-1, then decode; same
    results as reshape_and_cache of the rows followed by
    paged_attention_decode."""
    s, hq, d = query.shape
    hkv = k_cache.shape[1]
    assert new_key.shape == new_value.shape == (s, hkv, d)
    if out is None:
        out = torch.empty_like(query)
    need = decode_workspace_size(s, hq, hkv, d, max_context_len, partition_tokens)
    if workspace is None:
        workspace = torch.empty(max(need, 16), dtype=torch.uint8, device=query.device)
    st = library().paged_attention_decode_append(
        _dev(out, "out", query.dtype), _dev(query, "query"), _dev(new_key, "new_key", query.dtype),
        _dev(new_value, "new_value", query.dtype), _dev(k_cache, "k_cache"),
        _dev(v_cache, "v_cache"), k_cache.shape[0],
        _dev(block_tables, "block_tables", torch.int32), block_tables.shape[1],
        _dev(context_lens, "context_lens", torch.int32), s, int(max_context_len), hq, hkv, d,
        float(softmax_scale), _dtype_code(query, "query"), _dtype_code(k_cache, "k_cache"),
        float(k_scale), float(v_scale), int(partition_tokens), _dev(workspace, "workspace"),
        workspace.numel() * workspace.element_size(), _stream(query))
    _check("paged_attention_decode_append", st)
    return out
