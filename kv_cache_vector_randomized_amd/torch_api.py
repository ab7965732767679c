"""PyTorch-side convenience layer: allocates the paged cache, workspace and
outputs as torch tensors and calls the C ABI through `tq` (no compute here)."""
from __future__ import annotations

from typing import Optional

import numpy as np
import torch

from . import tq


def _dtype_code(t: torch.Tensor) -> int:
    if t.dtype == torch.bfloat16:
        return tq.TQ_BF16
    if t.dtype == torch.float32:
        return tq.TQ_F32
    raise TypeError(f"unsupported dtype {t.dtype}")


class PagedKVCache:
    """One layer's packed KV cache [num_blocks, num_kv_heads, page_bytes] (uint8) on a GPU."""

    def __init__(self, ctx: tq.Context, num_blocks: int, device="cuda", fill: Optional[int] = None):
        self.ctx = ctx
        self.num_blocks = int(num_blocks)
        shape = (self.num_blocks, ctx.cfg.num_kv_heads, ctx.page_bytes)
        if fill is None:
            self.data = torch.empty(shape, dtype=torch.uint8, device=device)
        else:
            self.data = torch.full(shape, fill, dtype=torch.uint8, device=device)
        self._ws = None

    def append(self, k: torch.Tensor, v: torch.Tensor, slot_mapping: torch.Tensor, stream=None):
        """Quantize and store k, v [N, Hkv, d] at slot_mapping (int64 [N])."""
        assert k.is_contiguous() and v.is_contiguous() and k.shape == v.shape and k.dtype == v.dtype
        assert slot_mapping.dtype == torch.int64 and slot_mapping.is_contiguous()
        assert slot_mapping.shape[0] == k.shape[0]
        self.ctx.quantize_append(k, v, slot_mapping, self.data, self.num_blocks, _dtype_code(k), k.shape[0], stream)

    def workspace(self, batch: int, max_seq_len: int) -> torch.Tensor:
        need = self.ctx.workspace_bytes(batch, max_seq_len)
        if self._ws is None or self._ws.numel() < need:
            # zero-filled once: the leading counter region must start at zero
            self._ws = torch.zeros(max(need, 16), dtype=torch.uint8, device=self.data.device)
        return self._ws

    def decode(self, q: torch.Tensor, block_tables: torch.Tensor, seq_lens: torch.Tensor, max_seq_len: int,
               softmax_scale: float, out: Optional[torch.Tensor] = None, logits: Optional[torch.Tensor] = None,
               stream=None) -> torch.Tensor:
        """Attention of q [B, Hq, d] over the cache; returns out [B, Hq, d] fp32."""
        assert q.is_contiguous() and block_tables.dtype == torch.int32 and seq_lens.dtype == torch.int32
        assert block_tables.is_contiguous() and seq_lens.is_contiguous()
        B = q.shape[0]
        if out is None:
            out = torch.empty((B, q.shape[1], q.shape[2]), dtype=torch.float32, device=q.device)
        ws = self.workspace(B, max_seq_len)
        self.ctx.decode_attention(q, _dtype_code(q), self.data, self.num_blocks, block_tables,
                                  block_tables.shape[1], seq_lens, B, max_seq_len, softmax_scale, out, ws,
                                  ws.numel(), logits_out=logits, stream=stream)
        return out

    def append_decode(self, k_new: torch.Tensor, v_new: torch.Tensor, q: torch.Tensor, block_tables: torch.Tensor,
                      seq_lens: torch.Tensor, max_seq_len: int, softmax_scale: float,
                      out: Optional[torch.Tensor] = None, logits: Optional[torch.Tensor] = None,
                      stream=None) -> torch.Tensor:
        """Store the new token k_new, v_new [B, Hkv, d] of every sequence at position
        seq_lens[b] - 1, then attend q [B, Hq, d] over the context including it."""
        assert q.is_contiguous() and k_new.is_contiguous() and v_new.is_contiguous()
        assert k_new.dtype == q.dtype and v_new.dtype == q.dtype and k_new.shape == v_new.shape
        assert k_new.shape[0] == q.shape[0]
        assert block_tables.dtype == torch.int32 and seq_lens.dtype == torch.int32
        assert block_tables.is_contiguous() and seq_lens.is_contiguous()
        B = q.shape[0]
        if out is None:
            out = torch.empty((B, q.shape[1], q.shape[2]), dtype=torch.float32, device=q.device)
        ws = self.workspace(B, max_seq_len)
        self.ctx.append_decode(k_new, v_new, q, _dtype_code(q), self.data, self.num_blocks, block_tables,
                               block_tables.shape[1], seq_lens, B, max_seq_len, softmax_scale, out, ws, ws.numel(),
                               logits_out=logits, stream=stream)
        return out

    @property
    def block_bytes(self) -> int:
        return self.ctx.cfg.num_kv_heads * self.ctx.page_bytes

    def offload_blocks(self, block_ids: torch.Tensor, host: torch.Tensor, stream=None) -> None:
        """Copy blocks block_ids (device int32 [n]) into pinned host memory `host`
        (uint8, at least n * block_bytes): block i of the list at [i*block_bytes, ...)."""
        assert block_ids.dtype == torch.int32 and block_ids.is_contiguous() and block_ids.is_cuda
        assert host.is_pinned() and host.dtype == torch.uint8 and host.numel() >= block_ids.numel() * self.block_bytes
        self.ctx.offload_blocks(self.data, self.num_blocks, block_ids, block_ids.numel(), host, stream)

    def restore_blocks(self, host: torch.Tensor, block_ids: torch.Tensor, stream=None) -> None:
        """Copy the blocks saved in pinned host memory `host` back to block_ids."""
        assert block_ids.dtype == torch.int32 and block_ids.is_contiguous() and block_ids.is_cuda
        assert host.is_pinned() and host.dtype == torch.uint8 and host.numel() >= block_ids.numel() * self.block_bytes
        self.ctx.restore_blocks(host, block_ids, block_ids.numel(), self.data, self.num_blocks, stream)

    def dequantize(self, slots: torch.Tensor, stream=None):
        """Reconstruct (k_hat, v_hat) [n, Hkv, d] fp32 for int64 slots [n]."""
        n = slots.shape[0]
        shape = (n, self.ctx.cfg.num_kv_heads, self.ctx.cfg.head_dim)
        k = torch.empty(shape, dtype=torch.float32, device=self.data.device)
        v = torch.empty(shape, dtype=torch.float32, device=self.data.device)
        self.ctx.dequantize(self.data, self.num_blocks, slots, n, k, v, stream)
        return k, v

    def dequantize_rows(self, slots: torch.Tensor, rows: Optional[torch.Tensor], k_buf: torch.Tensor,
                        v_buf: torch.Tensor, stream=None) -> None:
        """Reconstruct the tokens at int64 `slots` [n] into rows `rows` [n] (None: row i) of
        the running buffers k_buf, v_buf [rows, Hkv, d] (fp32 or bf16)."""
        assert slots.dtype == torch.int64 and slots.is_contiguous() and slots.is_cuda
        assert rows is None or (rows.dtype == torch.int64 and rows.is_contiguous() and rows.numel() == slots.numel())
        shape = (self.ctx.cfg.num_kv_heads, self.ctx.cfg.head_dim)
        assert k_buf.shape[1:] == shape and v_buf.shape == k_buf.shape and k_buf.dtype == v_buf.dtype
        assert k_buf.is_contiguous() and v_buf.is_contiguous()
        self.ctx.dequantize_rows(self.data, self.num_blocks, slots, slots.numel(), rows, k_buf, v_buf,
                                 k_buf.shape[0], _dtype_code(k_buf), stream)


def bf16_from_bits(bits: np.ndarray, device="cuda") -> torch.Tensor:
    """Upload bf16 bit patterns (uint16) as a torch.bfloat16 tensor."""
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).to(device)
