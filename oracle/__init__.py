"""CPU oracle for the paged KV cache -- TEST INFRASTRUCTURE ONLY.

Only ``tests/``, ``__graft_entry__.smoke()`` and ``bench.py``'s CPU-baseline leg
may import this package.  The product path (``paged_kv_cache_13_amd``) never
imports it, and the C source here shares no code with the HIP library.

What it computes is written out in ``pkv_oracle.c`` with the pages it follows
(nanoserve dev log: "Day 25: the fused read dispatches to the kernel backend",
"Day 17: paging under the sampling path ...", "Day 60: the read becomes a
choice ...").  Every entry point below is plain double-precision C; this module
only marshals arrays.

Parity pins (tests/test_oracle_pins.py): dense fp64 attention on directly
built histories, closed forms (one position, zero query, constant V, one
dominant key), invariants (block permutation, row permutation, slot-mapping vs
block-table addressing, NaN-poisoned unused slots, GQA vs replicated heads),
scatter round trip through numpy's view of the layout, the Day 60 page's
wirebench cell table, and for the multi-query read: dense causal attention,
the one-query case, and each query as a decode read of its own prefix.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "pkv_oracle.c")
_LIB = os.path.join(_HERE, "liboracle.so")

F32 = 0
BF16 = 1

_lib = None


def build(force: bool = False) -> str:
    """Compile the oracle with gcc (-O2, strict IEEE: no fast-math)."""
    if force or not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
        tmp = _LIB + ".tmp%d" % os.getpid()
        subprocess.check_call(
            ["gcc", "-O2", "-std=c99", "-fPIC", "-shared", "-fno-fast-math",
             "-ffp-contract=off", "-Wall", "-Wextra", "-o", tmp, _SRC, "-lm"])
        os.replace(tmp, _LIB)
    return _LIB


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB):
            build()
        lib = ctypes.CDLL(_LIB)
        vp, i32, i64, f64 = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_double
        lib.oracle_reshape_and_cache.argtypes = [vp, vp, vp, i64, vp, vp, i64, i32, i32, i32, i32]
        lib.oracle_paged_attention.argtypes = [i32, i32, i32, i32, i32, i32, i64, i32,
                                               vp, vp, vp, vp, vp, f64, vp]
        lib.oracle_paged_attention_slots.argtypes = [i32, i32, i32, i32, i32, i64, i32,
                                                     vp, vp, vp, vp, i64, vp, f64, vp, vp]
        lib.oracle_paged_attention_streamed.argtypes = [i32, i32, i32, i32, i32, i32, i64, i32,
                                                        vp, vp, vp, vp, vp, f64, i32, vp, vp]
        lib.oracle_paged_attention_multi.argtypes = [i32, i32, i32, i32, i32, i32, i32, i64, i32,
                                                     vp, vp, vp, vp, vp, f64, vp]
        for fn in (lib.oracle_reshape_and_cache, lib.oracle_paged_attention,
                   lib.oracle_paged_attention_slots, lib.oracle_paged_attention_streamed,
                   lib.oracle_paged_attention_multi):
            fn.restype = ctypes.c_int
        _lib = lib
    return _lib


def _raw(a):
    """Return (contiguous numpy view of the raw storage, dtype code).

    Accepts numpy float32 / uint16 (bf16 bits) arrays and torch CPU tensors of
    float32 / bfloat16.  bf16 is carried as its 16-bit pattern.
    """
    try:
        import torch
    except ImportError:  # pragma: no cover
        torch = None
    if torch is not None and isinstance(a, torch.Tensor):
        if a.device.type != "cpu":
            raise ValueError("oracle takes host tensors")
        a = a.contiguous()
        if a.dtype == torch.bfloat16:
            return a.view(torch.int16).numpy().view(np.uint16), BF16
        if a.dtype == torch.float32:
            return a.numpy(), F32
        if a.dtype in (torch.int32, torch.int64):
            return a.numpy(), None
        raise TypeError("unsupported tensor dtype %s" % a.dtype)
    a = np.ascontiguousarray(a)
    if a.dtype == np.float32:
        return a, F32
    if a.dtype == np.uint16:
        return a, BF16
    if a.dtype in (np.int32, np.int64):
        return a, None
    raise TypeError("unsupported array dtype %s" % a.dtype)


def _ptr(a):
    return a.ctypes.data_as(ctypes.c_void_p)


def _check(rc, what):
    if rc != 0:
        raise RuntimeError("%s failed with oracle status %d" % (what, rc))


def reshape_and_cache(k, v, slot_mapping, k_pool, v_pool):
    """Scatter k, v [T, n_kv, hd] into k_pool and v_pool [nb, n_kv, bs, hd]
    in place.

    Pools must be writable host arrays/tensors; they are modified in place.
    """
    kr, dt = _raw(k)
    vr, dt2 = _raw(v)
    kp, dt3 = _raw(k_pool)
    vp_, dt4 = _raw(v_pool)
    if not (dt == dt2 == dt3 == dt4) or dt is None:
        raise TypeError("k, v and pools must share one float dtype")
    sm = np.ascontiguousarray(np.asarray(slot_mapping, dtype=np.int64))
    T, n_kv, hd = kr.shape
    nb, n_kv2, bs, hd2 = kp.shape
    if ((n_kv, hd) != (n_kv2, hd2) or vr.shape != kr.shape or vp_.shape != (nb, n_kv, bs, hd)
            or sm.shape != (T,)):
        raise ValueError("shape mismatch")
    # the pools must be modified in place: refuse copies
    for orig, raw in ((k_pool, kp), (v_pool, vp_)):
        base = orig.data_ptr() if hasattr(orig, "data_ptr") else orig.ctypes.data
        if raw.ctypes.data != base:
            raise ValueError("pools must be contiguous so they can be updated in place")
    rc = _load().oracle_reshape_and_cache(_ptr(kr), _ptr(vr), _ptr(sm), T, _ptr(kp), _ptr(vp_),
                                          nb, bs, n_kv, hd, dt)
    _check(rc, "oracle_reshape_and_cache")


def _attn_common(q, k_pool, v_pool):
    qr, dt = _raw(q)
    kp, dt2 = _raw(k_pool)
    vp_, dt3 = _raw(v_pool)
    if not (dt == dt2 == dt3) or dt is None:
        raise TypeError("q and pools must share one float dtype")
    rows, n_heads, hd = qr.shape
    nb, n_kv, bs, hd2 = kp.shape
    if hd != hd2 or vp_.shape != (nb, n_kv, bs, hd):
        raise ValueError("shape mismatch: k_pool and v_pool [nb, n_kv, bs, hd]")
    return qr, kp, vp_, dt, rows, n_heads, hd, nb, n_kv, bs


def paged_attention(q, k_pool, v_pool, block_table, context_lens, scale):
    """Gathered decode read through a block table; returns float64 [rows, H, hd]."""
    qr, kp, vp_, dt, rows, n_heads, hd, nb, n_kv, bs = _attn_common(q, k_pool, v_pool)
    bt = np.ascontiguousarray(np.asarray(block_table, dtype=np.int32))
    cl = np.ascontiguousarray(np.asarray(context_lens, dtype=np.int32))
    if bt.ndim != 2 or bt.shape[0] != rows or cl.shape != (rows,):
        raise ValueError("block_table / context_lens shape mismatch")
    out = np.zeros((rows, n_heads, hd), dtype=np.float64)
    rc = _load().oracle_paged_attention(rows, n_heads, n_kv, hd, bs, bt.shape[1], nb, dt,
                                        _ptr(qr), _ptr(kp), _ptr(vp_), _ptr(bt), _ptr(cl),
                                        float(scale), _ptr(out))
    _check(rc, "oracle_paged_attention")
    return out


def paged_attention_multi(q, k_pool, v_pool, block_table, context_lens, scale):
    """Multi-query read: q [rows, query_len, H, hd] is each row's last
    query_len positions, causal inside the chunk; returns float64 of q's shape."""
    if len(q.shape) != 4:
        raise ValueError("q must be [rows, query_len, n_heads, head_dim]")
    rows, qlen, n_heads, hd = (int(x) for x in q.shape)
    qr, kp, vp_, dt, _, _, _, nb, n_kv, bs = _attn_common(q.reshape(rows * qlen, n_heads, hd), k_pool, v_pool)
    bt = np.ascontiguousarray(np.asarray(block_table, dtype=np.int32))
    cl = np.ascontiguousarray(np.asarray(context_lens, dtype=np.int32))
    if bt.ndim != 2 or bt.shape[0] != rows or cl.shape != (rows,):
        raise ValueError("block_table / context_lens shape mismatch")
    out = np.zeros((rows, qlen, n_heads, hd), dtype=np.float64)
    rc = _load().oracle_paged_attention_multi(rows, qlen, n_heads, n_kv, hd, bs, bt.shape[1], nb, dt,
                                              _ptr(qr), _ptr(kp), _ptr(vp_), _ptr(bt), _ptr(cl),
                                              float(scale), _ptr(out))
    _check(rc, "oracle_paged_attention_multi")
    return out


def paged_attention_slots(q, k_pool, v_pool, slot_mapping, context_lens, scale):
    """Gathered decode read through a whole-history slot mapping [rows, W].

    Returns (float64 out [rows, H, hd], score cells of the rectangle).
    """
    qr, kp, vp_, dt, rows, n_heads, hd, nb, n_kv, bs = _attn_common(q, k_pool, v_pool)
    sm = np.ascontiguousarray(np.asarray(slot_mapping, dtype=np.int64))
    cl = np.ascontiguousarray(np.asarray(context_lens, dtype=np.int32))
    if sm.ndim != 2 or sm.shape[0] != rows or cl.shape != (rows,):
        raise ValueError("slot_mapping / context_lens shape mismatch")
    out = np.zeros((rows, n_heads, hd), dtype=np.float64)
    cells = ctypes.c_int64(0)
    rc = _load().oracle_paged_attention_slots(rows, n_heads, n_kv, hd, bs, nb, dt,
                                              _ptr(qr), _ptr(kp), _ptr(vp_), _ptr(sm), sm.shape[1],
                                              _ptr(cl), float(scale), _ptr(out),
                                              ctypes.byref(cells))
    _check(rc, "oracle_paged_attention_slots")
    return out, int(cells.value)


def paged_attention_streamed(q, k_pool, v_pool, block_table, context_lens, scale, tile):
    """Streamed (tile-walk, online softmax) decode read.

    Returns (float64 out [rows, H, hd], held score cells summed over programs).
    """
    qr, kp, vp_, dt, rows, n_heads, hd, nb, n_kv, bs = _attn_common(q, k_pool, v_pool)
    bt = np.ascontiguousarray(np.asarray(block_table, dtype=np.int32))
    cl = np.ascontiguousarray(np.asarray(context_lens, dtype=np.int32))
    if bt.ndim != 2 or bt.shape[0] != rows or cl.shape != (rows,):
        raise ValueError("block_table / context_lens shape mismatch")
    out = np.zeros((rows, n_heads, hd), dtype=np.float64)
    held = ctypes.c_int64(0)
    rc = _load().oracle_paged_attention_streamed(rows, n_heads, n_kv, hd, bs, bt.shape[1], nb, dt,
                                                 _ptr(qr), _ptr(kp), _ptr(vp_), _ptr(bt), _ptr(cl),
                                                 float(scale), int(tile), _ptr(out),
                                                 ctypes.byref(held))
    _check(rc, "oracle_paged_attention_streamed")
    return out, int(held.value)
