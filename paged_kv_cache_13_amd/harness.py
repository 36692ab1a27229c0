"""Benchmark-harness helpers that sit beside the library, not inside it.

* ``gathered_rect_read``: the pages' original read, built from torch ops on the
  GPU -- gather the whole [rows, max_ctx] slot mapping into a contiguous
  history and score a [rows, heads, 1, ctx] rectangle (nanoserve "Day 60"
  page, "What I added today"; "Day 17" page, "Tomorrow").  It is the
  comparison arm of the decode-run sweep, never the product path.
* ``read_bytes`` / ``scatter_bytes``: algorithmic HBM bytes of one call, from
  host-known shapes and lengths.
"""
from __future__ import annotations

import numpy as np
import torch


def whole_history_slots(block_table: torch.Tensor, block_size: int, width: int) -> torch.Tensor:
    """[rows, width] int64 slot of every position through the block table."""
    pos = torch.arange(width, device=block_table.device)
    blk = block_table.long()[:, pos // block_size]
    return blk * block_size + (pos % block_size)


def gathered_rect_read(q, k_pool, v_pool, block_table, context_lens, scale, width=None):
    """Gather-and-reassemble read: contiguous history, masked score rectangle,
    fp32 softmax, PV.  Returns fp32 [rows, n_heads, head_dim]."""
    rows, n_heads, hd = q.shape
    nb, nkv, bs, _ = k_pool.shape
    G = n_heads // nkv
    if width is None:
        width = block_table.shape[1] * bs
    slots = whole_history_slots(block_table, bs, width)
    blk, off = slots // bs, slots % bs
    live = torch.arange(width, device=q.device)[None, :] < context_lens.long()[:, None]  # [rows, W]
    blk = torch.where(live, blk, torch.zeros_like(blk))
    off = torch.where(live, off, torch.zeros_like(off))
    K = k_pool[blk, :, off, :].float()  # [rows, W, nkv, hd]
    V = v_pool[blk, :, off, :].float()  # [rows, W, nkv, hd]
    K = torch.where(live[:, :, None, None], K, torch.zeros_like(K))
    V = torch.where(live[:, :, None, None], V, torch.zeros_like(V))
    qf = q.float().reshape(rows, nkv, G, hd)
    Kt = K.permute(0, 2, 3, 1).contiguous()   # [rows, nkv, hd, W]
    Vc = V.permute(0, 2, 1, 3).contiguous()   # [rows, nkv, W, hd]
    s = torch.matmul(qf, Kt) * scale          # [rows, nkv, G, W]
    s = torch.where(live[:, None, None, :], s, torch.full_like(s, float("-inf")))
    p = torch.softmax(s, dim=-1)
    p = torch.where(live[:, None, None, :], p, torch.zeros_like(p))  # empty rows: 0, not NaN
    o = torch.matmul(p, Vc)                   # [rows, nkv, G, hd]
    return o.reshape(rows, n_heads, hd)


def read_bytes(ctx: np.ndarray, n_heads: int, n_kv: int, head_dim: int, block_size: int,
               elem: int, out_elem: int) -> int:
    """Algorithmic HBM bytes of one decode read: every position's K and V row
    for every kv head, q and out, the block ids walked, the lengths."""
    ctx = np.asarray(ctx, dtype=np.int64)
    rows = ctx.shape[0]
    kv = int(2 * ctx.sum() * n_kv * head_dim * elem)
    qo = rows * n_heads * head_dim * (elem + out_elem)
    ids = int(4 * (-(-ctx // block_size)).sum())
    return kv + qo + ids + 4 * rows


def read_flops(ctx: np.ndarray, n_heads: int, head_dim: int) -> int:
    return int(4 * n_heads * head_dim * np.asarray(ctx, dtype=np.int64).sum())


def scatter_bytes(tokens: int, n_kv: int, head_dim: int, elem: int) -> int:
    """K and V rows read and written once each, plus the int64 slot ids."""
    return 4 * tokens * n_kv * head_dim * elem + 8 * tokens
