"""Helpers for GPU-vs-oracle parity tests (not collected by pytest)."""
import numpy as np
import torch

import oracle
import paged_kv_cache_13_amd as pkv

DEV = "cuda:0"

# nanoserve "Day 25" page, "What I learned", item 2: the kernel is held to the
# reference at atol 1e-5, rtol 1e-4 (fp32).  bf16 output: atol 2e-2 (stated
# for bf16 storage with fp32 accumulation); rtol kept at 1e-4.
TOL = {torch.float32: dict(atol=1e-5, rtol=1e-4), torch.bfloat16: dict(atol=2e-2, rtol=1e-4)}


def assert_close(got, ref, atol, rtol, what=""):
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    assert got.shape == ref.shape, (got.shape, ref.shape)
    assert np.isfinite(got).all(), "%s: non-finite output at %s" % (what, np.argwhere(~np.isfinite(got))[:5])
    diff = np.abs(got - ref)
    bad = diff > atol + rtol * np.abs(ref)
    if bad.any():
        idx = np.argwhere(bad)[:5]
        raise AssertionError("%s: %d/%d elements outside atol=%g rtol=%g; max |diff| %.3g; first %s"
                             % (what, bad.sum(), bad.size, atol, rtol, diff.max(), idx.tolist()))


def gpu_read(batch, out_dtype=None, partition=0):
    out = torch.empty(batch.q.shape, dtype=out_dtype or batch.q.dtype, device=batch.q.device)
    out.fill_(float("nan"))
    pkv.paged_attention_into(batch.q, batch.k_pool, batch.v_pool, batch.block_table,
                             batch.context_lens, batch.scale, out, partition_tokens=partition)
    torch.cuda.synchronize()
    return out


def host_rows(batch, rows):
    """Host copies of q and a compact pool holding only `rows`' blocks, with the
    block table renumbered into it (paging invariance: the oracle's result does
    not depend on where the blocks live)."""
    rows = np.asarray(rows)
    bs = batch.cfg.block_size
    ids, table = [], np.zeros((len(rows), batch.table_host.shape[1]), dtype=np.int32)
    for i, r in enumerate(rows):
        need = -(-int(batch.ctx_host[r]) // bs)
        table[i, :need] = np.arange(len(ids), len(ids) + need)
        ids.extend(int(b) for b in batch.table_host[r, :need])
    if not ids:
        ids = [0]
    idx = torch.tensor(ids, dtype=torch.long, device=batch.k_pool.device)
    kp = batch.k_pool.index_select(0, idx).cpu()
    vp = batch.v_pool.index_select(0, idx).cpu()
    q = batch.q[torch.as_tensor(rows, device=batch.q.device)].cpu()
    return q, kp, vp, table, batch.ctx_host[rows].copy()


def oracle_read(batch, rows=None):
    if rows is None:
        rows = np.arange(batch.cfg.rows)
    q, kp, vp, table, lens = host_rows(batch, rows)
    return oracle.paged_attention(q, kp, vp, table, lens, batch.scale)


def oracle_read_parallel(batch, rows=None, threads=16):
    """oracle_read over many rows, the unchanged oracle called on several row
    shares at once from a thread pool (ctypes releases the GIL during the
    call).  Shares are dealt longest row first, round-robin, so they hold
    about the same number of positions."""
    import concurrent.futures

    if rows is None:
        rows = np.arange(batch.cfg.rows)
    rows = np.asarray(rows)
    order = rows[np.argsort(-batch.ctx_host[rows], kind="stable")]
    shares = [np.sort(order[i::threads]) for i in range(threads)]
    shares = [sh for sh in shares if sh.size]
    inputs = [host_rows(batch, sh) for sh in shares]
    oracle._load()
    with concurrent.futures.ThreadPoolExecutor(len(shares)) as ex:
        outs = list(ex.map(lambda a: oracle.paged_attention(a[0], a[1], a[2], a[3], a[4], batch.scale), inputs))
    ref = np.zeros((rows.size,) + outs[0].shape[1:], dtype=np.float64)
    pos = {int(r): i for i, r in enumerate(rows)}
    for sh, out in zip(shares, outs):
        for j, r in enumerate(sh):
            ref[pos[int(r)]] = out[j]
    return ref
