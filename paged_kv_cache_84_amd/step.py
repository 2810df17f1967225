"""One engine step of the paged-attention hot path on the GPU.

The order inside a step: block copies (copy-on-write) first, then the slot of
every new token and the cache writes of all new tokens (the first layer's
write derives and stores the slots, later layers reuse them), then attention
for the chunk rows (prefill) and the decode rows, layer by layer, all on one
stream ("vLLM 引擎解剖", section "PagedAttention：为 KV 缓存分页" for the
copy-before-write rule; section "预填充、解码与三个时延指标" for write-then-read).

``DeviceStep`` takes any object with the attributes of a workload step
(block tables, unified schedule, caches, new tokens' Q/K/V, copy pairs) and
keeps device copies of everything, so that ``run()`` only launches kernels.
"""

import numpy as np
import torch

from . import _binding as B


def _i32(a, dev):
    return torch.as_tensor(np.ascontiguousarray(a, dtype=np.int32)).to(dev)


class DeviceStep:
    def __init__(self, step, device="cuda", partition_tokens=0, to_device=True):
        dev = torch.device(device)
        self.step = step
        self.device = dev
        mv = (lambda t: t.to(dev).contiguous()) if to_device else (lambda t: t)
        self.k_caches = [mv(t) for t in step.k_caches]
        self.v_caches = [mv(t) for t in step.v_caches]
        if self.k_caches[0].dtype == torch.float8_e4m3fn:
            self.k_caches = [t.view(torch.uint8) for t in self.k_caches]
            self.v_caches = [t.view(torch.uint8) for t in self.v_caches]
        self.q = [mv(t) for t in step.q]
        self.new_k = [mv(t) for t in step.new_k]
        self.new_v = [mv(t) for t in step.new_v]
        self.block_tables = _i32(step.block_tables, dev)
        self.query_start_loc = _i32(step.query_start_loc, dev)
        self.num_computed = _i32(step.num_computed, dev)
        self.copy_pairs = torch.as_tensor(
            np.ascontiguousarray(step.copy_pairs, dtype=np.int64)).to(dev)
        p = step.num_prefill_reqs
        self.num_prefill_tokens = step.num_prefill_tokens
        self.dec_tables = _i32(step.decode_block_tables, dev)
        self.dec_lens = _i32(step.decode_context_lens, dev)
        self.max_context_len = int(step.decode_context_lens.max()) if step.num_reqs > p else 0
        self.pre_tables = _i32(step.prefill_block_tables, dev)
        self.pre_qsl = _i32(step.prefill_query_start_loc, dev)
        self.pre_computed = _i32(step.prefill_num_computed, dev)
        qsl = step.query_start_loc
        self.max_query_len = int(np.max(np.diff(qsl[:p + 1]))) if p > 0 else 0
        self.num_decode = step.num_reqs - p
        self.slots = torch.empty(step.num_tokens, dtype=torch.int64, device=dev)
        self.out = [torch.empty_like(q) for q in self.q]
        self.partition_tokens = partition_tokens
        self.varlen_ws = None
        if self.num_decode > 0:
            hq, hkv, d = step.num_q_heads, step.num_kv_heads, step.head_dim
            need = B.decode_workspace_size(self.num_decode, hq, hkv, d,
                                           self.max_context_len, partition_tokens)
            self.workspace = torch.zeros(max(need, 16), dtype=torch.uint8, device=dev)
        else:
            self.workspace = None

    # --- the calls of one step -----------------------------------------
    def copy(self):
        if len(self.copy_pairs):
            B.copy_blocks(self.k_caches, self.v_caches, self.copy_pairs)

    def slot_mapping(self):
        B.compute_slot_mapping(self.block_tables, self.query_start_loc, self.num_computed,
                               self.k_caches[0].shape[0], self.step.num_tokens,
                               out=self.slots)

    def write(self, layer):
        s = self.step
        B.reshape_and_cache(self.new_k[layer], self.new_v[layer], self.k_caches[layer],
                            self.v_caches[layer], self.slots, s.k_scale, s.v_scale)

    def write_scheduled(self, layer):
        """Slots from the schedule and this layer's cache write, one launch;
        the slots are stored for the other layers."""
        s = self.step
        B.reshape_and_cache_from_schedule(
            self.new_k[layer], self.new_v[layer], self.k_caches[layer], self.v_caches[layer],
            self.block_tables, self.query_start_loc, self.num_computed, s.k_scale, s.v_scale,
            slot_mapping=self.slots)

    def write_layer(self, layer):
        """Layer 0 derives the slots while it writes; later layers use them."""
        if layer == 0:
            self.write_scheduled(0)
        else:
            self.write(layer)

    def prefill(self, layer):
        s = self.step
        t = self.num_prefill_tokens
        if t == 0:
            return
        B.paged_attention_prefill_chunk(
            self.q[layer][:t], self.k_caches[layer], self.v_caches[layer],
            self.pre_tables, self.pre_qsl, self.pre_computed, self.max_query_len,
            s.softmax_scale, s.k_scale, s.v_scale, out=self.out[layer][:t])

    def decode(self, layer):
        s = self.step
        if self.num_decode == 0:
            return
        t = self.num_prefill_tokens
        B.paged_attention_decode(
            self.q[layer][t:], self.k_caches[layer], self.v_caches[layer],
            self.dec_tables, self.dec_lens, self.max_context_len, s.softmax_scale,
            s.k_scale, s.v_scale, self.partition_tokens, out=self.out[layer][t:],
            workspace=self.workspace)

    def can_append(self):
        """True for a decode-only step whose formats the fused call takes
        (bf16 queries; bf16 caches, or fp8 E4M3 caches held as bytes)."""
        return (self.num_prefill_tokens == 0 and self.num_decode > 0 and
                self.q[0].dtype == torch.bfloat16 and
                self.k_caches[0].dtype in (torch.bfloat16, torch.uint8))

    def decode_append(self, layer):
        """This layer's new-token cache write and decode in one launch: each
        sequence's new token sits at position context_len - 1, the slot the
        block table gives it."""
        s = self.step
        B.paged_attention_decode_append(
            self.q[layer], self.new_k[layer], self.new_v[layer], self.k_caches[layer],
            self.v_caches[layer], self.dec_tables, self.dec_lens, self.max_context_len,
            s.softmax_scale, s.k_scale, s.v_scale, self.partition_tokens,
            out=self.out[layer], workspace=self.workspace)

    def run_decode_append(self):
        """A decode-only step: copies, then per layer one fused write-and-
        decode launch.  Same caches and outputs as run(); the slot array is
        not materialised."""
        if not self.can_append():
            raise ValueError("run_decode_append takes a decode-only step with bf16 queries "
                             "and bf16 or fp8 E4M3 caches")
        self.copy()
        for layer in range(len(self.k_caches)):
            self.decode_append(layer)
        return self.out

    def varlen(self, layer):
        """Attention of every request of the step (chunks and decodes) in one
        launch, written to the same output rows as prefill() + decode()."""
        s = self.step
        if self.varlen_ws is None:
            qsl = s.query_start_loc
            self.varlen_qsl = _i32(qsl, self.device)
            self.varlen_max_seq = int(np.max(s.num_computed + np.diff(qsl)))
            need = B.varlen_workspace_size(s.num_reqs, int(qsl[-1]), s.num_kv_heads, s.head_dim,
                                           self.varlen_max_seq)
            self.varlen_ws = torch.empty(max(need, 16), dtype=torch.uint8, device=self.device)
        B.paged_attention_varlen(self.q[layer], self.k_caches[layer], self.v_caches[layer],
                                 self.block_tables, self.varlen_qsl, self.num_computed,
                                 self.varlen_max_seq, s.softmax_scale, out=self.out[layer],
                                 workspace=self.varlen_ws)

    def run_varlen(self):
        """The whole step with the unified attention launch."""
        self.copy()
        for layer in range(len(self.k_caches)):
            self.write_layer(layer)
            self.varlen(layer)
        return self.out

    def run(self):
        """The whole step: copies, then per layer write (with the slots on
        layer 0) and attend."""
        self.copy()
        for layer in range(len(self.k_caches)):
            self.write_layer(layer)
            self.prefill(layer)
            self.decode(layer)
        return self.out
