"""Seeded synthetic decode workloads for the paged KV cache.

This module only draws inputs: context lengths, block tables from a shuffled
free list, pool contents and queries.  It holds none of the read's arithmetic
(no scores, softmax, gather or scatter), so the HIP path and the CPU oracle can
both be fed from it without sharing any of the method.

Integer metadata (lengths, block ids, slots) comes from numpy's PCG64 stream on
the host; float payloads come from a seeded ``torch.Generator`` on the device
the tensors live on.  Slots are encoded as ``block * block_size + offset``: the
pages' slot mapping (nanoserve "Day 25" page, "What I added today") addresses a
pool of fixed-size blocks (nanoserve "Day 17" page, "Post angle").

Unused pool slots -- blocks no row owns and the positions past a row's length
in its last block -- are filled with NaN, and block-table entries past a row's
last block point at one of those NaN blocks, so a read that touches anything it
should not turns the output into NaN instead of passing silently.
"""
from __future__ import annotations

import dataclasses
import math
from typing import Optional

import numpy as np
import torch

__all__ = ["DecodeConfig", "CONFIGS", "BlockAllocator", "KVCacheExhausted",
           "DecodeBatch", "make_batch", "DecodeRun", "torch_dtype"]


class KVCacheExhausted(RuntimeError):
    """Raised when the allocator has no free block (nanoserve "Day 17" page,
    "What I learned", item 2)."""


class BlockAllocator:
    """A shuffled free list of pool block ids.

    ``allocate()`` pops the next free id, ``free(ids)`` returns ids to the list;
    ``num_free`` is the number still available.  A fresh allocator hands blocks
    out in a seeded random order, which fragments every row's block table.
    """

    def __init__(self, num_blocks: int, rng: np.random.Generator):
        self.num_blocks = int(num_blocks)
        self._free = [int(b) for b in rng.permutation(self.num_blocks)[::-1]]

    @property
    def num_free(self) -> int:
        return len(self._free)

    def allocate(self) -> int:
        if not self._free:
            raise KVCacheExhausted("no free KV block left in a pool of %d" % self.num_blocks)
        return self._free.pop()

    def free(self, ids) -> None:
        for b in ids:
            b = int(b)
            if not 0 <= b < self.num_blocks:
                raise ValueError("block id %d outside the pool" % b)
            self._free.append(b)


def torch_dtype(name: str) -> torch.dtype:
    return {"f32": torch.float32, "bf16": torch.bfloat16}[name]


@dataclasses.dataclass(frozen=True)
class DecodeConfig:
    """One synthetic decode batch shape.

    ctx: ("fixed", (n0, n1, ...)) | ("uniform", lo, hi) inclusive integers |
         ("loguniform", lo, hi): floor(exp(U[ln lo, ln hi])).
    pool: ("fixed", num_blocks) | ("factor", f): ceil(f * blocks needed).
    """
    name: str
    dtype: str
    rows: int
    n_heads: int
    n_kv_heads: int
    head_dim: int
    block_size: int
    ctx: tuple
    pool: tuple
    max_ctx: int
    value_scale: float = 1.0
    seed: int = 0

    @property
    def max_blocks_per_row(self) -> int:
        return -(-self.max_ctx // self.block_size)

    @property
    def scale(self) -> float:
        return 1.0 / math.sqrt(self.head_dim)

    def replace(self, **kw) -> "DecodeConfig":
        return dataclasses.replace(self, **kw)


# The five synthetic workloads.  Shapes follow the Llama-3-8B attention layer
# (32 query heads, 8 kv heads, head_dim 128) where the workload names it; no
# weights are involved anywhere.
CONFIGS = {
    # tiny fp32 read: two rows, lengths 16 and 64, 32-block pool
    "tiny_f32": DecodeConfig("tiny_f32", "f32", rows=2, n_heads=4, n_kv_heads=2, head_dim=16,
                             block_size=8, ctx=("fixed", (16, 64)), pool=("fixed", 32),
                             max_ctx=64, seed=1),
    # fp32 GQA batch over a fragmented 1024-block pool
    "gqa_f32": DecodeConfig("gqa_f32", "f32", rows=8, n_heads=8, n_kv_heads=2, head_dim=64,
                            block_size=16, ctx=("uniform", 128, 1024), pool=("fixed", 1024),
                            max_ctx=1024, seed=2),
    # one Llama-3-8B-shaped attention layer, bf16 pool, 64 decode rows
    "llama3_8b_layer": DecodeConfig("llama3_8b_layer", "bf16", rows=64, n_heads=32, n_kv_heads=8,
                                    head_dim=128, block_size=16, ctx=("uniform", 512, 4096),
                                    pool=("factor", 1.5), max_ctx=4096, seed=3),
    # skewed long-context batch: log-uniform lengths up to 32768
    "skewed_long": DecodeConfig("skewed_long", "bf16", rows=256, n_heads=32, n_kv_heads=8,
                                head_dim=128, block_size=32, ctx=("loguniform", 16, 32768),
                                pool=("factor", 1.5), max_ctx=32768, value_scale=0.5, seed=4),
}


def _draw_lengths(cfg: DecodeConfig, rng: np.random.Generator) -> np.ndarray:
    kind = cfg.ctx[0]
    if kind == "fixed":
        vals = np.asarray(cfg.ctx[1], dtype=np.int64)
        if vals.shape != (cfg.rows,):
            raise ValueError("fixed lengths must give one per row")
        return vals.astype(np.int32)
    if kind == "uniform":
        lo, hi = cfg.ctx[1], cfg.ctx[2]
        return rng.integers(lo, hi + 1, size=cfg.rows).astype(np.int32)
    if kind == "loguniform":
        lo, hi = cfg.ctx[1], cfg.ctx[2]
        u = rng.uniform(math.log(lo), math.log(hi), size=cfg.rows)
        return np.clip(np.floor(np.exp(u)), lo, hi).astype(np.int32)
    raise ValueError("unknown length distribution %r" % (kind,))


@dataclasses.dataclass
class DecodeBatch:
    cfg: DecodeConfig
    q: torch.Tensor             # [rows, n_heads, head_dim]
    k_pool: torch.Tensor        # [num_blocks, n_kv_heads, block_size, head_dim]
    v_pool: torch.Tensor        # [num_blocks, n_kv_heads, block_size, head_dim]
    block_table: torch.Tensor   # [rows, max_blocks_per_row] int32
    context_lens: torch.Tensor  # [rows] int32
    ctx_host: np.ndarray        # host copy of the lengths (drawn here, never read back)
    table_host: np.ndarray      # host copy of the block table
    num_blocks: int
    poison_block: int           # a NaN-filled block that unused table entries point at

    @property
    def scale(self) -> float:
        return self.cfg.scale


def _fill_normal(shape, dtype, device, gen, value_scale, chunk=1 << 26):
    """N(0, value_scale^2) draws rounded once to `dtype`, in bounded chunks."""
    out = torch.empty(shape, dtype=dtype, device=device)
    flat = out.view(-1)
    for s in range(0, flat.numel(), chunk):
        e = min(flat.numel(), s + chunk)
        tmp = torch.randn(e - s, generator=gen, device=device, dtype=torch.float32)
        if value_scale != 1.0:
            tmp.mul_(value_scale)
        flat[s:e].copy_(tmp)
    return out


def make_batch(cfg: DecodeConfig, device="cpu", seed: Optional[int] = None,
               poison: bool = True) -> DecodeBatch:
    """Draw one decode batch for `cfg` on `device` (seeded, reproducible)."""
    seed = cfg.seed if seed is None else seed
    rng = np.random.default_rng(seed)
    lens = _draw_lengths(cfg, rng)
    if int(lens.max(initial=0)) > cfg.max_ctx:
        raise ValueError("a drawn length exceeds max_ctx")
    bs = cfg.block_size
    need = [-(-int(n) // bs) for n in lens]
    if cfg.pool[0] == "fixed":
        nb = int(cfg.pool[1])
    else:
        nb = int(math.ceil(cfg.pool[1] * sum(need)))
    nb = max(nb, sum(need) + 1)  # room for at least one poison block
    alloc = BlockAllocator(nb, rng)
    mbpr = cfg.max_blocks_per_row
    table = np.empty((cfg.rows, mbpr), dtype=np.int32)
    owned = np.zeros(nb, dtype=bool)
    for r in range(cfg.rows):
        for j in range(need[r]):
            b = alloc.allocate()
            table[r, j] = b
            owned[b] = True
    poison_block = alloc.allocate()
    for r in range(cfg.rows):
        table[r, need[r]:] = poison_block

    dt = torch_dtype(cfg.dtype)
    gen = torch.Generator(device=device)
    gen.manual_seed(seed)
    q = _fill_normal((cfg.rows, cfg.n_heads, cfg.head_dim), dt, device, gen, cfg.value_scale)
    k_pool = _fill_normal((nb, cfg.n_kv_heads, bs, cfg.head_dim), dt, device, gen, cfg.value_scale)
    v_pool = _fill_normal((nb, cfg.n_kv_heads, bs, cfg.head_dim), dt, device, gen, cfg.value_scale)
    if poison:
        unused = np.ones((nb, bs), dtype=bool)
        unused[owned] = False
        for r in range(cfg.rows):
            n = int(lens[r])
            if n % bs and need[r]:
                unused[table[r, need[r] - 1], n % bs:] = True
        mask = torch.from_numpy(unused).to(device)
        k_pool.masked_fill_(mask[:, None, :, None], float("nan"))
        v_pool.masked_fill_(mask[:, None, :, None], float("nan"))
    return DecodeBatch(cfg=cfg, q=q, k_pool=k_pool, v_pool=v_pool,
                       block_table=torch.from_numpy(table).to(device),
                       context_lens=torch.from_numpy(lens).to(device),
                       ctx_host=lens, table_host=table, num_blocks=nb,
                       poison_block=poison_block)


class DecodeRun:
    """A decode run over a shared pool: a prompt per row, then one new token per
    row per step.  Each step draws the new token's K/V and query, allocates a
    block from the shuffled free list when a row's last block is full, and
    reports the slot every new token goes to; the caller scatters and reads.

    The prompt and per-step draws are seeded; the pool starts NaN-filled so a
    read of any slot that was never written shows up as NaN.
    """

    def __init__(self, rows: int, block_size: int, prompt: int, steps: int, *,
                 n_heads: int = 32, n_kv_heads: int = 8, head_dim: int = 128,
                 dtype: str = "bf16", device="cpu", seed: int = 5000,
                 pool_factor: float = 1.0, value_scale: float = 1.0):
        self.rows, self.block_size, self.prompt, self.steps = rows, block_size, prompt, steps
        self.n_heads, self.n_kv_heads, self.head_dim = n_heads, n_kv_heads, head_dim
        self.dtype, self.device, self.value_scale = torch_dtype(dtype), device, value_scale
        self.max_ctx = prompt + steps
        self.max_blocks_per_row = -(-self.max_ctx // block_size)
        # one extra block stays NaN for ever: table entries past a row's last
        # block point at it
        self.num_blocks = int(math.ceil(pool_factor * rows * self.max_blocks_per_row)) + 1
        self.rng = np.random.default_rng(seed)
        self.gen = torch.Generator(device=device)
        self.gen.manual_seed(seed)
        self.alloc = BlockAllocator(self.num_blocks, self.rng)
        self.poison_block = self.alloc.allocate()
        self.k_pool = torch.full((self.num_blocks, n_kv_heads, block_size, head_dim), float("nan"),
                                 dtype=self.dtype, device=device)
        self.v_pool = torch.full((self.num_blocks, n_kv_heads, block_size, head_dim), float("nan"),
                                 dtype=self.dtype, device=device)
        self.table_host = np.full((rows, self.max_blocks_per_row), self.poison_block,
                                  dtype=np.int32)
        self.ctx_host = np.zeros(rows, dtype=np.int32)
        self.scale = 1.0 / math.sqrt(head_dim)

    def _slots_for_next(self, count: int) -> np.ndarray:
        """Slots for the next `count` positions of every row, allocating blocks."""
        bs = self.block_size
        slots = np.empty((self.rows, count), dtype=np.int64)
        for r in range(self.rows):
            for i in range(count):
                pos = int(self.ctx_host[r]) + i
                if pos % bs == 0:
                    self.table_host[r, pos // bs] = self.alloc.allocate()
                slots[r, i] = int(self.table_host[r, pos // bs]) * bs + pos % bs
        return slots

    def _draw(self, shape):
        return _fill_normal(shape, self.dtype, self.device, self.gen, self.value_scale)

    def prefill(self):
        """(k, v, slot_mapping) for every row's prompt, token-major [rows*prompt, ...]."""
        slots = self._slots_for_next(self.prompt)
        k = self._draw((self.rows * self.prompt, self.n_kv_heads, self.head_dim))
        v = self._draw((self.rows * self.prompt, self.n_kv_heads, self.head_dim))
        self.ctx_host += self.prompt
        return k, v, torch.from_numpy(slots.reshape(-1)).to(self.device)

    def step(self):
        """(q, k_new, v_new, slot_mapping) for one decode step of every row."""
        slots = self._slots_for_next(1)
        q = self._draw((self.rows, self.n_heads, self.head_dim))
        k = self._draw((self.rows, self.n_kv_heads, self.head_dim))
        v = self._draw((self.rows, self.n_kv_heads, self.head_dim))
        self.ctx_host += 1
        return q, k, v, torch.from_numpy(slots.reshape(-1)).to(self.device)

    def block_table(self) -> torch.Tensor:
        return torch.from_numpy(self.table_host.copy()).to(self.device)

    def context_lens(self) -> torch.Tensor:
        return torch.from_numpy(self.ctx_host.copy()).to(self.device)

    def finish_row(self, r: int) -> None:
        """Return row r's blocks to the free list (free-and-reuse)."""
        used = -(-int(self.ctx_host[r]) // self.block_size)
        self.alloc.free(self.table_host[r, :used])
        self.table_host[r, :] = self.poison_block
        self.ctx_host[r] = 0
