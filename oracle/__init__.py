"""Plain fp64 CPU oracle for paged attention over a 16-token-block KV cache.

TEST INFRASTRUCTURE ONLY.  Only the test suite, the smoke check and the
benchmark's CPU-baseline leg may import anything from this package.  The
product path (the HIP library and its Python binding) never calls it, and this
package imports nothing from the product path: the two share no code.

What it computes, and where the pages define it:

* ``formats``   -- how stored cache elements map to real numbers (fp32, bf16,
  OCP fp8 E4M3) and the fp8 quantiser (round to nearest even, saturate to
  +-448).  The pages only name fp8 as a KV-cache dtype ("01. vLLM：从分页 KV
  起家的通用推理引擎", section "KV 缓存管理与前缀缓存", the --kv-cache-dtype row).
* ``paged``     -- slot mapping, reshape_and_cache, copy_blocks, the gather
  through a block table, decode attention, chunked-prefill attention, the
  contiguous brute force used to pin the gather, the log-sum-exp combine of
  split partitions, and the per-token KV size closed form.
  ("vLLM 引擎解剖", sections "KV 缓存需要多少内存？" (Table 1),
  "PagedAttention：为 KV 缓存分页" (Fig. 2), "V1：统一调度预填充与解码" (Fig. 3)).

* ``blocks``    -- the host block manager: pool, reference counts, LRU free
  queue, prefix-hash chain and copy-on-write ("01. vLLM", section "KV 缓存管理
  与前缀缓存"; "vLLM 引擎解剖", sections "PagedAttention：为 KV 缓存分页" and
  "自动前缀缓存" (Fig. 4); "v1/v0 区别", §4 "KV Cache 管理").

Everything is written for a reader to check by eye: explicit loops over
logical blocks and query rows, float64 arithmetic, no tiling, no fusion.

Pins: every function here is checked by ``tests/test_oracle_*.py`` against
facts fixed by the pages or by mathematics (worked examples from Fig. 2 and
Table 1, closed forms, library routines on special cases, brute force on tiny
inputs).  The only result left "parity unpinned" beyond the oracle itself is the
value of attention on the large random configurations: the pages print no
attention values.
"""

from . import blocks, formats, paged  # noqa: F401

__all__ = ["blocks", "formats", "paged"]
