"""One Engram site on one GPU: the C-ABI calls chained over preallocated
device buffers.

``Engram.forward`` = engram_compress_hash -> engram_gather_dequant ->
engram_gated_residual on one stream, no host synchronisation, no allocation
(path "split", the default).  Path "fused" (e4m3fn tables only) replaces the
gather and the projection by engram_gather_project, which keeps the gathered
rows on chip: no [T][k_pad] bf16 row buffer, at a lower projection rate.
"""
from __future__ import annotations

from typing import Optional, Sequence

from . import (ENGRAM_DTYPE_BF16, ENGRAM_DTYPE_FP8_E4M3FN, Layout, engram_compress_hash,
               engram_gate_add, engram_gather_dequant, engram_gather_project,
               engram_gated_residual, engram_layout_create, engram_tid2eid_check)


def pad_weight(w, layout: Layout):
    """Storage layout of the wkv weight, done once at load time: the logical
    [hidden][3*H*D] bf16 matrix placed in [hidden][k_pad] with each (order, head)
    segment starting at a multiple of seg_pitch and zeros in the gaps (the
    gathered rows carry zeros there too)."""
    import torch
    info = layout.info
    hidden, K = w.shape
    cols = 3 * info.heads
    D, sp = info.row_dim, info.seg_pitch
    if K != cols * D:
        raise ValueError(f"weight has {K} columns, layout wants {cols} x {D}")
    out = torch.zeros((hidden, info.k_pad), dtype=torch.bfloat16, device=w.device)
    out.view(hidden, cols, sp)[:, :, :D].copy_(w.view(hidden, cols, D))
    return out


class Engram:
    """Device state of one Engram site: layout, compression map, tables, padded
    weight, and the per-call work buffers sized for ``max_tokens``."""

    def __init__(self, *, vocab_size: int, compressed_vocab: int, pad_token_id: int,
                 heads_per_order: int, rows: Sequence[int], row_dim: int, table_dtype: str,
                 row_pitch_bytes: int, tid2eid, tables: Sequence, scales: Optional[Sequence],
                 weight, hidden: int, hc_mult: int = 4, max_tokens: int, hash_floor: int = 0,
                 path: str = "split", stream=None):
        import torch
        if path not in ("split", "fused"):
            raise ValueError(f"unknown path {path!r}")
        if path == "fused" and table_dtype != "fp8":
            raise ValueError("the fused path reads e4m3fn tables only")
        self.path = path
        dt = ENGRAM_DTYPE_FP8_E4M3FN if table_dtype == "fp8" else ENGRAM_DTYPE_BF16
        self.layout = engram_layout_create(
            vocab_size=vocab_size, compressed_vocab=compressed_vocab, pad_token_id=pad_token_id,
            heads_per_order=heads_per_order, rows=rows, row_dim=row_dim, table_dtype=dt,
            row_pitch_bytes=row_pitch_bytes, hash_floor=hash_floor)
        info = self.layout.info
        dev = tid2eid.device
        self.tid2eid = tid2eid
        self.pad_eid = engram_tid2eid_check(self.layout, tid2eid, stream)
        self.tables = list(tables)
        self.scales = None if scales is None else list(scales)
        self.weight = pad_weight(weight, self.layout) if weight.shape[1] != info.k_pad else weight
        self.hidden = hidden
        self.hc_mult = hc_mult
        self.max_tokens = max_tokens
        self.eids = torch.empty(max_tokens, dtype=torch.int32, device=dev)
        self.row_ids = torch.empty((max_tokens, 3, info.heads), dtype=torch.int32, device=dev)
        self.rows = (torch.empty((max_tokens, info.k_pad), dtype=torch.bfloat16, device=dev)
                     if path == "split" else None)
        self.v = torch.empty((max_tokens, hidden), dtype=torch.float32, device=dev)

    @property
    def info(self):
        return self.layout.info

    def forward(self, tokens, cu_seqlens, streams, *, seq_start=None, slots=None, store=None,
                dead=None, keep=None, stream=None):
        """Adds the Engram memory of ``tokens`` into ``streams`` (bf16 [T][hc][hidden],
        in place).  With a dead mask the caller passes ``keep`` (1 = keep the gate),
        the complement of ``dead``."""
        T = tokens.numel()
        if T > self.max_tokens:
            raise ValueError(f"{T} tokens > max_tokens {self.max_tokens}")
        if dead is not None and keep is None:
            raise ValueError("a dead mask needs the matching keep mask")
        if streams.shape[0] != T:
            raise ValueError("streams must hold one row per token")
        engram_compress_hash(self.layout, self.tid2eid, tokens, cu_seqlens, self.eids,
                             self.row_ids, seq_start=seq_start, slots=slots, store=store,
                             dead=dead, stream=stream)
        if self.path == "fused":
            engram_gather_project(self.layout, self.tables, self.scales, self.row_ids, self.weight,
                                  self.v, T=T, stream=stream)
            engram_gate_add(self.layout, self.v, streams, keep=keep, T=T, stream=stream)
            return streams
        engram_gather_dequant(self.layout, self.tables, self.scales, self.row_ids, self.rows,
                              T=T, stream=stream)
        engram_gated_residual(self.layout, self.rows, self.weight, streams, self.v, keep=keep,
                              T=T, stream=stream)
        return streams
