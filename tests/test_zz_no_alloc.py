"""The read that allocates nothing (pkv_paged_attention_noalloc) against the
read with a caller-owned workspace (pkv_paged_attention), through the C ABI.

Both launch the same kernels with the same plan; only where the partial
slots and plan words live differs (the library's static per-GPU buffer, or
the caller's workspace).  So the outputs must agree bit for bit.  The calls
come in a row on one stream, each smaller than the one before, so a later
call runs over whatever the earlier ones left in the static buffer.
"""
import sys

import pytest
import torch

import paged_kv_cache_13_amd as pkv
from paged_kv_cache_13_amd import synth
from parity import DEV

pytestmark = pytest.mark.gpu


def note(msg):
    print(msg, file=sys.stderr, flush=True)


def cases():
    # (name, config, out dtype): the stream read of the 8B-shaped layer
    # (4.3 MB of scratch), a smaller stream read, then an fp32 partition read
    big = synth.CONFIGS["llama3_8b_layer"]
    small = big.replace(name="stream_48_rows", rows=48, ctx=("uniform", 100, 6000), max_ctx=6000, seed=31)
    return [("llama3_8b_layer", big, torch.bfloat16), ("stream_48_rows", small, torch.float32),
            ("gqa_f32", synth.CONFIGS["gqa_f32"], torch.float32)]


def test_noalloc_read_equals_the_workspace_read():
    pkv.load_library()
    for name, cfg, odt in cases():
        note("noalloc read: %s rows=%d out=%s" % (name, cfg.rows, odt))
        b = synth.make_batch(cfg, device=DEV)
        need = pkv.workspace_size(b.q, b.k_pool, b.block_table, out_dtype=odt)
        assert 0 < need <= 32 << 20, (name, need)
        ref = torch.full(b.q.shape, float("nan"), dtype=odt, device=DEV)
        ws = torch.zeros(need, dtype=torch.uint8, device=DEV)
        pkv.paged_attention_into(b.q, b.k_pool, b.v_pool, b.block_table, b.context_lens, b.scale, ref, ws)
        for call in range(2):  # twice: the second call finds the first one's words in the buffer
            got = torch.full(b.q.shape, float("nan"), dtype=odt, device=DEV)
            pkv.paged_attention_noalloc(b.q, b.k_pool, b.v_pool, b.block_table, b.context_lens, b.scale, got)
            torch.cuda.synchronize()
            assert torch.equal(got, ref), "%s call %d" % (name, call)
        del b, ref, ws, got


def test_noalloc_read_refuses_a_read_larger_than_its_buffer():
    # fp32 over 8192 rows x 32 heads: 277 MB of partials, refused before any launch
    pkv.load_library()
    cfg = synth.CONFIGS["llama3_8b_layer"]
    q = torch.zeros(8192, cfg.n_heads, cfg.head_dim, dtype=torch.float32, device=DEV)
    kp = torch.zeros(4, cfg.n_kv_heads, cfg.block_size, cfg.head_dim, dtype=torch.float32, device=DEV)
    vp = torch.zeros(4, cfg.n_kv_heads, cfg.block_size, cfg.head_dim, dtype=torch.float32, device=DEV)
    bt = torch.zeros(8192, 256, dtype=torch.int32, device=DEV)
    cl = torch.zeros(8192, dtype=torch.int32, device=DEV)
    assert pkv.workspace_size(q, kp, bt) > 32 << 20
    with pytest.raises(pkv.PkvError) as e:
        pkv.paged_attention_noalloc(q, kp, vp, bt, cl, 0.1, torch.empty_like(q))
    assert e.value.status == 13
