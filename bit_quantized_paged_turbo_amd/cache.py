"""PagedKVCache: device memory for one layer's K/V pools, driven through the C ABI.

torch provides the allocations and the stream; appends and decodes are single calls
into libxq.so (no computation happens here).
"""
from __future__ import annotations

import torch

from . import (CacheLayout, load, xq_append_decode_attention, xq_decode_attention_balanced, xq_decode_plan,
               xq_decode_plan_balanced, xq_decode_workspace_bytes, xq_decode_workspace_bytes_balanced,
               xq_prefill_workspace_bytes,
               xq_paged_decode_attention,
               xq_paged_decode_attention_planned, xq_paged_prefill_attention,
               xq_pool_bytes, xq_quantize_append)


class PagedKVCache:
    def __init__(self, kv_dtype: int, num_kv_heads: int, page_size: int, num_pages: int,
                 device="cuda", fill_byte: int | None = None):
        load()
        self.layout = CacheLayout(kv_dtype, num_kv_heads, page_size, num_pages)
        self.pool_bytes = xq_pool_bytes(self.layout)
        if self.pool_bytes <= 0:
            raise ValueError("invalid cache layout")
        alloc = torch.empty if fill_byte is None else torch.full
        args = () if fill_byte is None else (fill_byte,)
        self.k_pool = alloc((self.pool_bytes,), *args, dtype=torch.uint8, device=device)
        self.v_pool = alloc((self.pool_bytes,), *args, dtype=torch.uint8, device=device)
        self._ws = None

    def append(self, k_new: torch.Tensor, v_new: torch.Tensor, token_seq: torch.Tensor,
               token_pos: torch.Tensor, block_tables: torch.Tensor, stream=None):
        """k_new/v_new bf16 [n, Hkv, 128]; token_seq/token_pos int32 [n]; block_tables int32 [S, P]."""
        xq_quantize_append(self.layout, k_new, v_new, int(k_new.shape[0]), token_seq, token_pos,
                           block_tables, int(block_tables.shape[1]), self.k_pool, self.v_pool,
                           stream)

    def workspace_bytes(self, batch, num_q_heads, max_context_len, num_splits=0) -> int:
        return xq_decode_workspace_bytes(self.layout, batch, num_q_heads, max_context_len,
                                         num_splits)

    def decode(self, q: torch.Tensor, block_tables: torch.Tensor, context_lens: torch.Tensor,
               max_context_len: int, softmax_scale: float, num_splits: int = 0,
               out: torch.Tensor | None = None, workspace: torch.Tensor | None = None,
               stream=None, seq_order: torch.Tensor | None = None) -> torch.Tensor:
        """q bf16 [B, Hq, 128] -> out fp32 [B, Hq, 128]. seq_order: a device int32 [B] plan
        (see plan()), or None."""
        batch, hq = int(q.shape[0]), int(q.shape[1])
        if out is None:
            out = torch.empty((batch, hq, 128), dtype=torch.float32, device=q.device)
        need = self.workspace_bytes(batch, hq, max_context_len, num_splits)
        if workspace is None and need > 0:
            if self._ws is None or self._ws.numel() < need:
                self._ws = torch.empty((need,), dtype=torch.uint8, device=q.device)
            workspace = self._ws
        wbytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
        if seq_order is None:
            xq_paged_decode_attention(self.layout, q, batch, hq, self.k_pool, self.v_pool,
                                      block_tables, int(block_tables.shape[1]), context_lens,
                                      int(max_context_len), softmax_scale, num_splits, workspace,
                                      wbytes, out, stream)
        else:
            xq_paged_decode_attention_planned(self.layout, q, batch, hq, self.k_pool, self.v_pool,
                                              block_tables, int(block_tables.shape[1]), context_lens,
                                              int(max_context_len), softmax_scale, num_splits,
                                              workspace, wbytes, out, seq_order, stream)
        return out

    def append_decode(self, k_new: torch.Tensor, v_new: torch.Tensor, q: torch.Tensor,
                      block_tables: torch.Tensor, context_lens: torch.Tensor, max_context_len: int,
                      softmax_scale: float, num_splits: int = 0, out: torch.Tensor | None = None,
                      workspace: torch.Tensor | None = None, stream=None,
                      seq_order: torch.Tensor | None = None) -> torch.Tensor:
        """One step: row b of k_new/v_new (bf16 [B, Hkv, 128]) goes to position context_lens[b] - 1,
        then the decode of q (bf16 [B, Hq, 128]) -> out fp32 [B, Hq, 128]."""
        batch, hq = int(q.shape[0]), int(q.shape[1])
        if out is None:
            out = torch.empty((batch, hq, 128), dtype=torch.float32, device=q.device)
        need = self.workspace_bytes(batch, hq, max_context_len, num_splits)
        if workspace is None and need > 0:
            if self._ws is None or self._ws.numel() < need:
                self._ws = torch.empty((need,), dtype=torch.uint8, device=q.device)
            workspace = self._ws
        wbytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
        xq_append_decode_attention(self.layout, k_new, v_new, q, batch, hq, self.k_pool, self.v_pool,
                                   block_tables, int(block_tables.shape[1]), context_lens,
                                   int(max_context_len), softmax_scale, num_splits, workspace, wbytes,
                                   out, seq_order, stream)
        return out

    def plan(self, host_context_lens, num_q_heads: int, max_context_len: int, num_splits: int = 0,
             device="cuda") -> torch.Tensor:
        """xq_decode_plan from host lengths, as a device int32 tensor for decode(seq_order=...)."""
        order = xq_decode_plan(self.layout, len(host_context_lens), num_q_heads, int(max_context_len),
                               num_splits, host_context_lens)
        return torch.tensor(order, dtype=torch.int32, device=device)

    def plan_balanced(self, host_context_lens, num_q_heads: int, max_context_len: int, device="cuda"):
        """xq_decode_plan_balanced from host lengths -> (nsplits, units int32 [2 * slots], seq_tps int32
        [batch]) on the device, for decode_balanced()."""
        ns, tps, units = xq_decode_plan_balanced(self.layout, len(host_context_lens), num_q_heads,
                                                 int(max_context_len), host_context_lens)
        return (ns, torch.tensor(units, dtype=torch.int32, device=device),
                torch.tensor(tps, dtype=torch.int32, device=device))

    def decode_balanced(self, q: torch.Tensor, block_tables: torch.Tensor, context_lens: torch.Tensor,
                        max_context_len: int, softmax_scale: float, plan, k_new=None, v_new=None,
                        out: torch.Tensor | None = None, workspace: torch.Tensor | None = None,
                        stream=None, chunk=None) -> torch.Tensor:
        """The decode with a length-aware plan (plan_balanced()); with k_new/v_new (bf16 [B, Hkv, 128])
        each sequence's new row is appended at context_lens[b] - 1 first. chunk = (k, v, token_seq,
        token_pos) appends rows of other sequences in the same launch (as append() would; none in a
        page the decode reads). -> out fp32 [B, Hq, 128]."""
        ns, units, tps = plan
        batch, hq = int(q.shape[0]), int(q.shape[1])
        if out is None:
            out = torch.empty((batch, hq, 128), dtype=torch.float32, device=q.device)
        need = xq_decode_workspace_bytes_balanced(self.layout, batch, hq, ns)
        if workspace is None and need > 0:
            if self._ws is None or self._ws.numel() < need:
                self._ws = torch.empty((need,), dtype=torch.uint8, device=q.device)
            workspace = self._ws
        wbytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
        xq_decode_attention_balanced(self.layout, q, batch, hq, self.k_pool, self.v_pool, block_tables,
                                     int(block_tables.shape[1]), context_lens, int(max_context_len),
                                     softmax_scale, ns, units, tps, k_new, v_new, workspace, wbytes, out,
                                     stream, *(() if chunk is None else
                                               (chunk[0], chunk[1], int(chunk[0].shape[0]), chunk[2], chunk[3])))
        return out

    def prefill(self, q: torch.Tensor, block_table: torch.Tensor, start_pos: int,
                softmax_scale: float, num_splits: int = 0, out: torch.Tensor | None = None,
                workspace: torch.Tensor | None = None, stream=None) -> torch.Tensor:
        """Chunk queries q bf16 [C, Hq, 128] at positions start_pos .. start_pos + C - 1 of the
        sequence whose block-table row is `block_table` (int32 [max_pages]); its rows up to the
        chunk's end must already be appended. -> out fp32 [C, Hq, 128]."""
        n, hq = int(q.shape[0]), int(q.shape[1])
        if out is None:
            out = torch.empty((n, hq, 128), dtype=torch.float32, device=q.device)
        need = xq_prefill_workspace_bytes(self.layout, n, hq, int(start_pos), num_splits)
        if workspace is None and need > 0:
            if self._ws is None or self._ws.numel() < need:
                self._ws = torch.empty((need,), dtype=torch.uint8, device=q.device)
            workspace = self._ws
        wbytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
        xq_paged_prefill_attention(self.layout, q, n, hq, self.k_pool, self.v_pool, block_table,
                                   int(block_table.shape[-1]), int(start_pos), softmax_scale,
                                   num_splits, workspace, wbytes, out, stream)
        return out
