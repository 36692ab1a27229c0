"""ctypes binding of libpkv.so (see include/pkv.h for the contract).

Argument marshalling only: shapes, dtypes and devices of torch tensors are
read on the host, raw device pointers and the current HIP stream are passed
to the C ABI, and a non-zero status becomes a ``PkvError``.  Every step of the
scatter and the read runs in the library's kernels.  PyTorch provides device
memory (including the read's workspace) and streams, nothing else.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(_HERE, "libpkv.so")

PKV_F32 = 0
PKV_BF16 = 1
_DTYPES = {torch.float32: PKV_F32, torch.bfloat16: PKV_BF16}

_lib = None


class PkvError(RuntimeError):
    """A libpkv call returned a non-zero status."""

    def __init__(self, status: int, message: str):
        super().__init__("libpkv status %d: %s" % (status, message))
        self.status = status


class AttnDesc(ctypes.Structure):
    _fields_ = [("rows", ctypes.c_int32), ("n_heads", ctypes.c_int32),
                ("n_kv_heads", ctypes.c_int32), ("head_dim", ctypes.c_int32),
                ("block_size", ctypes.c_int32), ("max_blocks_per_row", ctypes.c_int32),
                ("num_blocks", ctypes.c_int64), ("dtype", ctypes.c_int32),
                ("out_dtype", ctypes.c_int32), ("partition_tokens", ctypes.c_int32)]


class ReadStatsStruct(ctypes.Structure):
    _fields_ = [("mode", ctypes.c_int32), ("block", ctypes.c_int32), ("calls", ctypes.c_int64),
                ("rows", ctypes.c_int64), ("score_cells", ctypes.c_int64), ("held_cells", ctypes.c_int64)]


_MODES = {"gathered": 0, "streamed": 1}


def library_path() -> str:
    return _LIB_PATH


def load_library():
    """Load libpkv.so once.  A missing library is an error, never a fallback."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_LIB_PATH):
        raise ImportError("libpkv.so is not built (expected at %s); run "
                          "`python -c 'import __graft_entry__ as g; g.build()'`" % _LIB_PATH)
    lib = ctypes.CDLL(_LIB_PATH)
    vp, i32, i64, sz = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_size_t
    lib.pkv_reshape_and_cache.argtypes = [vp, vp, vp, i64, vp, vp, i64, i32, i32, i32, i32, vp]
    lib.pkv_reshape_and_cache.restype = ctypes.c_int
    lib.pkv_paged_attention.argtypes = [ctypes.POINTER(AttnDesc), vp, vp, vp, vp, vp,
                                        ctypes.c_float, vp, vp, sz, vp]
    lib.pkv_paged_attention.restype = ctypes.c_int
    lib.pkv_paged_attention_workspace_size.argtypes = [ctypes.POINTER(AttnDesc)]
    lib.pkv_paged_attention_workspace_size.restype = sz
    lib.pkv_strerror.argtypes = [ctypes.c_int]
    lib.pkv_strerror.restype = ctypes.c_char_p
    lib.pkv_version.argtypes = []
    lib.pkv_version.restype = ctypes.c_int
    lib.pkv_paged_attention_multi.argtypes = [ctypes.POINTER(AttnDesc), i32, vp, vp, vp, vp, vp,
                                              ctypes.c_float, vp, vp, sz, vp]
    lib.pkv_paged_attention_multi.restype = ctypes.c_int
    lib.pkv_paged_attention_multi_workspace_size.argtypes = [ctypes.POINTER(AttnDesc), i32]
    lib.pkv_paged_attention_multi_workspace_size.restype = sz
    lib.pkv_allocator_storage_bytes.argtypes = [i64]
    lib.pkv_allocator_storage_bytes.restype = sz
    lib.pkv_allocator_init.argtypes = [vp, vp, sz, i64, ctypes.c_uint64]
    lib.pkv_allocator_init.restype = ctypes.c_int
    lib.pkv_allocator_alloc.argtypes = [vp, i64, vp]
    lib.pkv_allocator_alloc.restype = ctypes.c_int
    lib.pkv_allocator_free.argtypes = [vp, vp, i64]
    lib.pkv_allocator_free.restype = ctypes.c_int
    lib.pkv_allocator_num_free.argtypes = [vp]
    lib.pkv_allocator_num_free.restype = i64
    lib.pkv_append_slots.argtypes = [vp, vp, i32, i32, i32, i32, vp]
    lib.pkv_append_slots.restype = ctypes.c_int
    lib.pkv_decode_step.argtypes = [ctypes.POINTER(AttnDesc), vp, vp, vp, vp, vp, vp, vp, vp,
                                    ctypes.c_float, vp, vp, sz, vp]
    lib.pkv_decode_step.restype = ctypes.c_int
    rs = ctypes.POINTER(ReadStatsStruct)
    lib.pkv_read_stats_init.argtypes = [rs, i32, i32]
    lib.pkv_read_stats_init.restype = ctypes.c_int
    lib.pkv_read_stats_record.argtypes = [rs, i32, i32, i32, i32]
    lib.pkv_read_stats_record.restype = ctypes.c_int
    lib.pkv_read_stats_record_read.argtypes = [rs, ctypes.POINTER(AttnDesc)]
    lib.pkv_read_stats_record_read.restype = ctypes.c_int
    lib.pkv_read_tile.argtypes = [ctypes.POINTER(AttnDesc)]
    lib.pkv_read_tile.restype = i32
    lib.pkv_paged_attention_noalloc.argtypes = [ctypes.POINTER(AttnDesc), vp, vp, vp, vp, vp,
                                                ctypes.c_float, vp, vp]
    lib.pkv_paged_attention_noalloc.restype = ctypes.c_int
    lib.pkv_read_stats_since.argtypes = [rs, rs, rs]
    lib.pkv_read_stats_since.restype = ctypes.c_int
    lib.pkv_read_stats_saving.argtypes = [rs]
    lib.pkv_read_stats_saving.restype = ctypes.c_double
    _lib = lib
    return lib


def _check(status: int):
    if status != 0:
        msg = load_library().pkv_strerror(status).decode()
        raise PkvError(status, msg)


def _dtype_code(t: torch.Tensor) -> int:
    try:
        return _DTYPES[t.dtype]
    except KeyError:
        raise TypeError("unsupported dtype %s (float32 or bfloat16)" % t.dtype) from None


def _require(cond: bool, msg: str):
    if not cond:
        raise ValueError(msg)


def _on_gpu(*ts):
    dev = ts[0].device
    for t in ts:
        _require(t.is_cuda, "every tensor must live on the GPU")
        _require(t.device == dev, "every tensor must live on the same GPU")
        _require(t.is_contiguous(), "every tensor must be contiguous")
    return dev


def _check_pools(k_pool, v_pool):
    _require(k_pool.dim() == 4, "k_pool must be [num_blocks, n_kv_heads, block_size, head_dim]")
    nb, nkv, bs, hd = k_pool.shape
    _require(tuple(v_pool.shape) == (nb, nkv, bs, hd),
             "v_pool must be [num_blocks, n_kv_heads, block_size, head_dim]")


def _stream_handle(device) -> int:
    return torch.cuda.current_stream(device).cuda_stream


def reshape_and_cache(k: torch.Tensor, v: torch.Tensor, slot_mapping: torch.Tensor,
                      k_pool: torch.Tensor, v_pool: torch.Tensor) -> None:
    """Scatter k, v [T, n_kv, hd] into k_pool and v_pool [nb, n_kv, bs, hd]
    at slot_mapping [T] (int64; negative = skip), on the current stream."""
    dev = _on_gpu(k, v, slot_mapping, k_pool, v_pool)
    _require(k.dim() == 3 and v.shape == k.shape, "k, v must be [T, n_kv_heads, head_dim]")
    _check_pools(k_pool, v_pool)
    _require(k_pool.shape[1] == k.shape[1] and k_pool.shape[3] == k.shape[2],
             "pools and k/v disagree on n_kv_heads or head_dim")
    _require(slot_mapping.dtype == torch.int64 and slot_mapping.shape == (k.shape[0],),
             "slot_mapping must be int64 [T]")
    dt = _dtype_code(k)
    _require(v.dtype == k.dtype and k_pool.dtype == k.dtype and v_pool.dtype == k.dtype,
             "k, v and pools must share one dtype")
    nb, nkv, bs, hd = k_pool.shape
    _check(load_library().pkv_reshape_and_cache(
        k.data_ptr(), v.data_ptr(), slot_mapping.data_ptr(), k.shape[0],
        k_pool.data_ptr(), v_pool.data_ptr(), nb, bs, nkv, hd, dt, _stream_handle(dev)))


def _desc(q, k_pool, block_table, out_dtype, partition_tokens) -> AttnDesc:
    rows, n_heads, hd = q.shape
    nb, nkv, bs, hd2 = k_pool.shape
    _require(hd == hd2, "q and pools disagree on head_dim")
    return AttnDesc(rows=rows, n_heads=n_heads, n_kv_heads=nkv, head_dim=hd, block_size=bs,
                    max_blocks_per_row=block_table.shape[1], num_blocks=nb,
                    dtype=_dtype_code(q), out_dtype=out_dtype,
                    partition_tokens=int(partition_tokens))


def workspace_size(q: torch.Tensor, k_pool: torch.Tensor, block_table: torch.Tensor,
                   out_dtype: Optional[torch.dtype] = None, partition_tokens: int = 0) -> int:
    od = _DTYPES[out_dtype or q.dtype]
    d = _desc(q, k_pool, block_table, od, partition_tokens)
    return int(load_library().pkv_paged_attention_workspace_size(ctypes.byref(d)))


def _read_args(q, k_pool, v_pool, block_table, context_lens, out, workspace, partition_tokens):
    dev = _on_gpu(q, k_pool, v_pool, block_table, context_lens, out)
    _require(q.dim() == 3, "q must be [rows, n_heads, head_dim]")
    _check_pools(k_pool, v_pool)
    _require(k_pool.dtype == q.dtype and v_pool.dtype == q.dtype, "q and pools must share one dtype")
    _require(block_table.dtype == torch.int32 and block_table.dim() == 2
             and block_table.shape[0] == q.shape[0], "block_table must be int32 [rows, max_blocks]")
    _require(context_lens.dtype == torch.int32 and context_lens.shape == (q.shape[0],),
             "context_lens must be int32 [rows]")
    _require(out.shape == q.shape, "out must be [rows, n_heads, head_dim]")
    d = _desc(q, k_pool, block_table, _dtype_code(out), partition_tokens)
    need = int(load_library().pkv_paged_attention_workspace_size(ctypes.byref(d)))
    if workspace is None:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=dev)
    else:
        _on_gpu(workspace)
    wsp = workspace.data_ptr() if need else None
    return dev, d, wsp, workspace.numel() * workspace.element_size()


def paged_attention_into(q, k_pool, v_pool, block_table, context_lens, scale, out,
                         workspace: Optional[torch.Tensor] = None,
                         partition_tokens: int = 0, stats: Optional["ReadCounters"] = None) -> torch.Tensor:
    """Paged decode read into a caller-provided `out` [rows, n_heads, hd]
    (float32 or bfloat16).  `workspace` is a uint8 GPU tensor; when None one of
    the required size is allocated by torch for this call.  `stats`, if
    given, counts the call (host arithmetic from shapes)."""
    dev, d, wsp, wsb = _read_args(q, k_pool, v_pool, block_table, context_lens, out, workspace,
                                  partition_tokens)
    _check(load_library().pkv_paged_attention(
        ctypes.byref(d), q.data_ptr(), k_pool.data_ptr(), v_pool.data_ptr(),
        block_table.data_ptr(), context_lens.data_ptr(), ctypes.c_float(scale), out.data_ptr(),
        wsp, wsb, _stream_handle(dev)))
    if stats is not None:
        stats.record_read(d)
    return out


def read_tile(q: torch.Tensor, k_pool: torch.Tensor, block_table: torch.Tensor,
              out_dtype: Optional[torch.dtype] = None, partition_tokens: int = 0) -> int:
    """Positions of one (row, head) whose scores a workgroup of the library's
    read of these shapes holds at once (pkv_read_tile)."""
    d = _desc(q, k_pool, block_table, _DTYPES[out_dtype or q.dtype], partition_tokens)
    return int(load_library().pkv_read_tile(ctypes.byref(d)))


def paged_attention_noalloc(q, k_pool, v_pool, block_table, context_lens, scale, out,
                            partition_tokens: int = 0) -> torch.Tensor:
    """The paged decode read into `out` with no workspace argument and no
    allocation: the library keeps its scratch in a static buffer of
    PKV_NOALLOC_SCRATCH_BYTES per GPU (calls overlapping on one GPU race)."""
    dev = _on_gpu(q, k_pool, v_pool, block_table, context_lens, out)
    _require(q.dim() == 3, "q must be [rows, n_heads, head_dim]")
    _check_pools(k_pool, v_pool)
    _require(k_pool.dtype == q.dtype and v_pool.dtype == q.dtype, "q and pools must share one dtype")
    _require(block_table.dtype == torch.int32 and block_table.dim() == 2
             and block_table.shape[0] == q.shape[0], "block_table must be int32 [rows, max_blocks]")
    _require(context_lens.dtype == torch.int32 and context_lens.shape == (q.shape[0],),
             "context_lens must be int32 [rows]")
    _require(out.shape == q.shape, "out must be [rows, n_heads, head_dim]")
    d = _desc(q, k_pool, block_table, _dtype_code(out), partition_tokens)
    _check(load_library().pkv_paged_attention_noalloc(
        ctypes.byref(d), q.data_ptr(), k_pool.data_ptr(), v_pool.data_ptr(), block_table.data_ptr(),
        context_lens.data_ptr(), ctypes.c_float(scale), out.data_ptr(), _stream_handle(dev)))
    return out


def workspace_size_multi(q: torch.Tensor, k_pool: torch.Tensor, block_table: torch.Tensor,
                         out_dtype: Optional[torch.dtype] = None, partition_tokens: int = 0) -> int:
    """Workspace bytes of paged_attention_multi for q [rows, query_len, H, hd]."""
    rows, qlen, n_heads, hd = q.shape
    nb, nkv, bs, _ = k_pool.shape
    d = AttnDesc(rows=rows, n_heads=n_heads, n_kv_heads=nkv, head_dim=hd, block_size=bs,
                 max_blocks_per_row=block_table.shape[1], num_blocks=nb, dtype=_dtype_code(q),
                 out_dtype=_DTYPES[out_dtype or q.dtype], partition_tokens=int(partition_tokens))
    return int(load_library().pkv_paged_attention_multi_workspace_size(ctypes.byref(d), qlen))


def paged_attention_multi(q, k_pool, v_pool, block_table, context_lens, scale, out=None,
                          workspace: Optional[torch.Tensor] = None, partition_tokens: int = 0,
                          stats: Optional["ReadCounters"] = None) -> torch.Tensor:
    """Paged read of a chunk of queries per row: q [rows, query_len, n_heads,
    hd] holds each row's last query_len positions (already in the pool and
    counted in context_lens), causal inside the chunk.  Returns (or writes
    into `out`) [rows, query_len, n_heads, hd]."""
    if out is None:
        out = torch.empty_like(q)
    dev = _on_gpu(q, k_pool, v_pool, block_table, context_lens, out)
    _require(q.dim() == 4, "q must be [rows, query_len, n_heads, head_dim]")
    _check_pools(k_pool, v_pool)
    _require(k_pool.dtype == q.dtype and v_pool.dtype == q.dtype, "q and pools must share one dtype")
    _require(block_table.dtype == torch.int32 and block_table.dim() == 2
             and block_table.shape[0] == q.shape[0], "block_table must be int32 [rows, max_blocks]")
    _require(context_lens.dtype == torch.int32 and context_lens.shape == (q.shape[0],),
             "context_lens must be int32 [rows]")
    _require(out.shape == q.shape, "out must be q's shape")
    rows, qlen, n_heads, hd = q.shape
    nb, nkv, bs, hd2 = k_pool.shape
    _require(hd == hd2, "q and pools disagree on head_dim")
    d = AttnDesc(rows=rows, n_heads=n_heads, n_kv_heads=nkv, head_dim=hd, block_size=bs,
                 max_blocks_per_row=block_table.shape[1], num_blocks=nb, dtype=_dtype_code(q),
                 out_dtype=_dtype_code(out), partition_tokens=int(partition_tokens))
    lib = load_library()
    need = int(lib.pkv_paged_attention_multi_workspace_size(ctypes.byref(d), qlen))
    if workspace is None:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=dev)
    else:
        _on_gpu(workspace)
    _check(lib.pkv_paged_attention_multi(
        ctypes.byref(d), qlen, q.data_ptr(), k_pool.data_ptr(), v_pool.data_ptr(), block_table.data_ptr(),
        context_lens.data_ptr(), ctypes.c_float(scale), out.data_ptr(), workspace.data_ptr() if need else None,
        workspace.numel() * workspace.element_size(), _stream_handle(dev)))
    if stats is not None:
        stats.record(rows, n_heads, qlen, block_table.shape[1] * bs)
    return out


def decode_step(q, k_new, v_new, slot_mapping, k_pool, v_pool, block_table, context_lens, scale,
                out=None, workspace: Optional[torch.Tensor] = None, partition_tokens: int = 0,
                stats: Optional["ReadCounters"] = None) -> torch.Tensor:
    """One decode step of every row: scatter k_new, v_new [rows, n_kv, hd] to
    slot_mapping [rows] (int64), then the paged read of q -- one library call
    on the current stream, no host synchronisation.  The read kernels append
    the new tokens themselves: one read launch per step."""
    if out is None:
        out = torch.empty_like(q)
    dev, d, wsp, wsb = _read_args(q, k_pool, v_pool, block_table, context_lens, out, workspace,
                                  partition_tokens)
    _on_gpu(k_new, v_new, slot_mapping, q)
    _require(k_new.dim() == 3 and v_new.shape == k_new.shape and k_new.shape[0] == q.shape[0]
             and k_new.shape[1] == k_pool.shape[1] and k_new.shape[2] == k_pool.shape[3],
             "k_new, v_new must be [rows, n_kv_heads, head_dim]")
    _require(k_new.dtype == q.dtype and v_new.dtype == q.dtype, "k_new, v_new must have q's dtype")
    _require(slot_mapping.dtype == torch.int64 and slot_mapping.shape == (q.shape[0],),
             "slot_mapping must be int64 [rows]")
    _check(load_library().pkv_decode_step(
        ctypes.byref(d), k_new.data_ptr(), v_new.data_ptr(), slot_mapping.data_ptr(), q.data_ptr(),
        k_pool.data_ptr(), v_pool.data_ptr(), block_table.data_ptr(), context_lens.data_ptr(),
        ctypes.c_float(scale), out.data_ptr(), wsp, wsb, _stream_handle(dev)))
    if stats is not None:
        stats.record_read(d)
    return out


class ReadCounters:
    """The library's read counters (pkv_read_stats): calls, rows, score cells
    a [rows, heads, query_len, width] rectangle is charged, cells the read
    holds, and their quotient.  Host arithmetic only."""

    def __init__(self, mode: str = "streamed", block: int = 16):
        self._s = ReadStatsStruct()
        _check(load_library().pkv_read_stats_init(ctypes.byref(self._s), _MODES[mode], int(block)))

    @classmethod
    def _wrap(cls, st: ReadStatsStruct) -> "ReadCounters":
        obj = cls.__new__(cls)
        obj._s = st
        return obj

    def record(self, rows: int, heads: int, query_len: int, width: int) -> None:
        _check(load_library().pkv_read_stats_record(ctypes.byref(self._s), rows, heads, query_len, width))

    def record_read(self, desc: AttnDesc) -> None:
        _check(load_library().pkv_read_stats_record_read(ctypes.byref(self._s), ctypes.byref(desc)))

    def snapshot(self) -> "ReadCounters":
        st = ReadStatsStruct()
        ctypes.memmove(ctypes.byref(st), ctypes.byref(self._s), ctypes.sizeof(st))
        return ReadCounters._wrap(st)

    def since(self, earlier: "ReadCounters") -> "ReadCounters":
        """The window between an earlier reading and this one; a reading of
        another read (mode or block differ) is refused."""
        out = ReadStatsStruct()
        _check(load_library().pkv_read_stats_since(ctypes.byref(self._s), ctypes.byref(earlier._s),
                                                    ctypes.byref(out)))
        return ReadCounters._wrap(out)

    mode = property(lambda self: {v: k for k, v in _MODES.items()}[self._s.mode])
    block = property(lambda self: self._s.block)
    calls = property(lambda self: self._s.calls)
    rows = property(lambda self: self._s.rows)
    score_cells = property(lambda self: self._s.score_cells)
    held_cells = property(lambda self: self._s.held_cells)

    @property
    def saving(self) -> float:
        return float(load_library().pkv_read_stats_saving(ctypes.byref(self._s)))


def paged_attention(q, k_pool, v_pool, block_table, context_lens, scale, out=None,
                    partition_tokens: int = 0, stats: Optional[ReadCounters] = None) -> torch.Tensor:
    """nanoserve-style call: returns attention output [rows, n_heads, head_dim]
    in q's dtype (or writes `out` if given)."""
    if out is None:
        out = torch.empty_like(q)
    return paged_attention_into(q, k_pool, v_pool, block_table, context_lens, scale, out,
                                partition_tokens=partition_tokens, stats=stats)


class BlockAllocatorStruct(ctypes.Structure):
    _fields_ = [("free_ids", ctypes.c_void_p), ("in_use", ctypes.c_void_p),
                ("num_blocks", ctypes.c_int64), ("num_free", ctypes.c_int64)]


class KVCacheExhausted(PkvError):
    """The pool has fewer free blocks than a call asked for."""


class BlockAllocator:
    """The library's block allocator of a shared pool (host memory): blocks
    out as sequences grow, back when they finish, reused by the next ones."""

    EXHAUSTED = 12

    def __init__(self, num_blocks: int, seed: int = 0):
        lib = load_library()
        nbytes = int(lib.pkv_allocator_storage_bytes(num_blocks))
        if nbytes == 0:
            raise ValueError("num_blocks out of range")
        import numpy as np
        self._storage = np.zeros((nbytes + 3) // 4, dtype=np.int32)  # 4-byte aligned
        self._a = BlockAllocatorStruct()
        _check(lib.pkv_allocator_init(ctypes.byref(self._a), self._storage.ctypes.data, nbytes, num_blocks,
                                      ctypes.c_uint64(seed)))

    def _call(self, status):
        if status == self.EXHAUSTED:
            raise KVCacheExhausted(status, load_library().pkv_strerror(status).decode())
        _check(status)

    @property
    def num_free(self) -> int:
        return int(load_library().pkv_allocator_num_free(ctypes.byref(self._a)))

    def allocate(self, n: int):
        import numpy as np
        ids = np.empty(max(n, 1), dtype=np.int32)
        self._call(load_library().pkv_allocator_alloc(ctypes.byref(self._a), n, ids.ctypes.data))
        return ids[:n]

    def free(self, ids) -> None:
        import numpy as np
        ids = np.ascontiguousarray(np.asarray(ids, dtype=np.int32))
        self._call(load_library().pkv_allocator_free(ctypes.byref(self._a), ids.ctypes.data, ids.size))

    def append_slots(self, table_row, block_size: int, length: int, count: int):
        """Slots (int64) of `count` positions appended at `length` to the
        sequence whose block-table row `table_row` (int32 numpy, written in
        place) is; new blocks come from this allocator."""
        import numpy as np
        assert table_row.dtype == np.int32 and table_row.flags.c_contiguous
        slots = np.empty(max(count, 1), dtype=np.int64)
        self._call(load_library().pkv_append_slots(ctypes.byref(self._a), table_row.ctypes.data,
                                                   table_row.size, block_size, length, count,
                                                   slots.ctypes.data))
        return slots[:count]
