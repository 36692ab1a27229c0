"""C-ABI checks that need no GPU: the library loads, exports every symbol the
header declares, and refuses bad arguments on the host before any HIP call
(every case below is invalid in at least one field, so nothing is launched)."""
import ctypes
import os
import re

import pytest

from paged_kv_cache_13_amd import binding

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "pkv.h")

FAKE = 0x100000  # 16-byte aligned, never dereferenced: every call below is refused first


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(binding.library_path()):
        from paged_kv_cache_13_amd.csrc import build as b
        b.build()
    return binding.load_library()


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(pkv_[a-z_]+)\s*\(", text)))


def test_header_declares_the_entry_points():
    assert declared_functions() == ["pkv_allocator_alloc", "pkv_allocator_free", "pkv_allocator_init",
                                    "pkv_allocator_num_free", "pkv_allocator_storage_bytes",
                                    "pkv_append_slots", "pkv_decode_step", "pkv_paged_attention",
                                    "pkv_paged_attention_multi", "pkv_paged_attention_multi_workspace_size",
                                    "pkv_paged_attention_noalloc",
                                    "pkv_paged_attention_workspace_size", "pkv_read_stats_init",
                                    "pkv_read_stats_record", "pkv_read_stats_record_read",
                                    "pkv_read_stats_saving", "pkv_read_stats_since", "pkv_read_tile",
                                    "pkv_reshape_and_cache", "pkv_strerror", "pkv_version"]


def test_library_exports_every_declared_symbol(lib):
    for name in declared_functions():
        assert hasattr(lib, name), name


def test_status_strings(lib):
    for code in range(0, 14):
        assert lib.pkv_strerror(code).decode() != "unknown status"
    assert lib.pkv_strerror(0).decode() == "ok"
    assert lib.pkv_strerror(999).decode() == "unknown status"
    assert lib.pkv_version() == 300


def desc(**kw):
    d = dict(rows=64, n_heads=32, n_kv_heads=8, head_dim=128, block_size=16,
             max_blocks_per_row=256, num_blocks=14000, dtype=1, out_dtype=1, partition_tokens=0)
    d.update(kw)
    return binding.AttnDesc(**d)


def ws(lib, **kw):
    return lib.pkv_paged_attention_workspace_size(ctypes.byref(desc(**kw)))


def test_workspace_size_partition_layout(lib):
    # fp32 reads split rows into partitions of about 64 KiB of K and V: at
    # head_dim 128, 64 positions.  64 rows x 32 heads x 64 partitions -> m
    # and l (2 x 131072 floats), then 131072 rows of 128 partial sums
    assert ws(lib, dtype=0, out_dtype=0) == (2 * 131072 + 131072 * 128) * 4
    # an explicit length: 8 partitions of 512
    assert ws(lib, dtype=0, out_dtype=0, partition_tokens=512) == (2 * 16384 + 16384 * 128) * 4
    # one partition covers every row: no workspace
    assert ws(lib, dtype=0, partition_tokens=4096) == 0
    assert ws(lib, dtype=0, max_blocks_per_row=4) == 0  # 64 positions
    # partitions of one block
    assert ws(lib, dtype=0, partition_tokens=16, max_blocks_per_row=4, rows=1, n_heads=2,
              n_kv_heads=1, head_dim=16) == (2 * 8 + 8 * 16) * 4
    # odd slot count: the partial sums start 16-byte aligned
    assert ws(lib, dtype=0, rows=1, n_heads=3, n_kv_heads=1, head_dim=16, partition_tokens=16,
              max_blocks_per_row=3) == (20 + 9 * 16) * 4
    # bf16 with head_dim 16 takes the same layout: 1024-position partitions
    assert ws(lib, head_dim=16) == (2 * 8192 + 8192 * 16) * 4
    assert lib.pkv_paged_attention_workspace_size(None) == 0
    assert ws(lib, head_dim=96) == 0  # invalid descriptors need nothing


def test_workspace_size_stream_layout(lib):
    # bf16, head_dim 128: header (4 words), 1024 wave starts (2 words each),
    # 65 group prefixes, aligned; then two partial slots per persistent wave
    # (a piece that starts a cut (kv head, row) and a later piece), each of
    # align4(4 heads x 130) = 520 floats, whatever the table width
    head = 4 + 2 * 1024 + 65
    head += -head % 4
    assert ws(lib) == (head + 2 * 1024 * 520) * 4
    # the slice length does not change the slots a wave owns
    assert ws(lib, partition_tokens=512) == (head + 2 * 1024 * 520) * 4
    # the stream layout always needs its header and slots, even when no row can split
    assert ws(lib, partition_tokens=4096) == (head + 2 * 1024 * 520) * 4
    # a 32768-position table: the same slots (256 rows: 257 group prefixes)
    head256 = 4 + 2 * 1024 + 257
    head256 += -head256 % 4
    assert ws(lib, rows=256, block_size=32, max_blocks_per_row=1024) == (head256 + 2 * 1024 * 520) * 4
    # more rows than the plan kernel scans: back to partitions
    assert ws(lib, rows=9000, max_blocks_per_row=32) == 0


def test_small_batches_over_short_tables_take_partitions(lib):
    # at most 256 (row, kv head) pairs over a table of at most 4096 positions:
    # the bf16 read uses the partition layout (that of an fp32 read with the
    # same partition length).  Its default partition: one workgroup per
    # compute unit (256 pairs: one partition), within [768, 2048] positions.
    part = lambda **kw: ws(lib, dtype=0, out_dtype=0, **kw)
    assert ws(lib, rows=32) == part(rows=32, partition_tokens=2048)   # 4096 positions: two of 2048
    assert ws(lib, rows=32) == (2 * 32 * 32 * 2 + 32 * 32 * 2 * 128) * 4
    assert ws(lib, rows=32, max_blocks_per_row=48) == 0                # 768 positions: one partition
    assert ws(lib, rows=8, max_blocks_per_row=128) == part(rows=8, max_blocks_per_row=128,
                                                           partition_tokens=768)  # 64 pairs: 4 -> 768
    assert ws(lib, rows=2, max_blocks_per_row=64) == part(rows=2, max_blocks_per_row=64,
                                                          partition_tokens=768)  # 16 pairs: the floor
    # a table of at most 1024 positions takes the partition kernel at any batch
    assert ws(lib, rows=128, max_blocks_per_row=64) == part(rows=128, max_blocks_per_row=64,
                                                            partition_tokens=1024)  # one partition: 0
    assert ws(lib, rows=128, max_blocks_per_row=65) > 4 * (2 * 1024)  # 1040 positions: stream header
    # one more position, or one more row, and the stream layout comes back
    assert ws(lib, rows=32, max_blocks_per_row=257) != part(rows=32, max_blocks_per_row=257)
    assert ws(lib, rows=33) != part(rows=33)
    assert ws(lib, rows=33) > 4 * (2 * 1024)  # the stream header is there


def test_default_partitions_stated_in_the_header(lib):
    # pkv.h, pkv_attn_desc.partition_tokens: each path's default, checked
    # through the workspace it implies (m, l and head_dim partial sums per
    # (row, head, partition); 0 when one partition covers the table)
    def part_ws(rows, heads, parts, hd):
        slots = rows * heads * parts
        return 0 if parts <= 1 else (((2 * slots + 3) & ~3) + slots * hd) * 4
    # matrix-core partition read: cdiv(table, cdiv(256, rows x kv heads)),
    # clamped to [768, 2048]
    assert ws(lib, rows=16) == part_ws(16, 32, 2, 128)                          # 4096 / 2 = 2048
    assert ws(lib, rows=4) == part_ws(4, 32, 6, 128)                            # 4096 / 8 -> 768
    assert ws(lib, rows=8, max_blocks_per_row=64) == part_ws(8, 32, 2, 128)     # 1024 / 4 -> 768
    assert ws(lib, rows=64, max_blocks_per_row=48) == 0                         # 768: one partition
    assert ws(lib, rows=9000) == part_ws(9000, 32, 2, 128)                      # > 8192 rows: 4096 -> 2048
    # VALU partition read: about 64 KiB of K and V per partition
    f32 = dict(dtype=0, out_dtype=0)
    assert ws(lib, rows=8, n_heads=8, n_kv_heads=2, head_dim=64, max_blocks_per_row=64, **f32) == \
        part_ws(8, 8, 8, 64)                                                    # 128 positions
    assert ws(lib, head_dim=128, **f32) == part_ws(64, 32, 64, 128)             # 64 positions
    assert ws(lib, head_dim=16, block_size=8, max_blocks_per_row=256, **f32) == \
        part_ws(64, 32, 4, 16)                                                  # 512 positions
    assert ws(lib, head_dim=16) == part_ws(64, 32, 4, 16)                       # bf16 hd 16: 1024
    # the stream read: header and two slots per wave, whatever the slice minimum
    assert ws(lib) == ws(lib, partition_tokens=1024) > 0


def noalloc(lib, d, q=FAKE, kp=FAKE, vp=FAKE, bt=FAKE, cl=FAKE, out=FAKE):
    return lib.pkv_paged_attention_noalloc(ctypes.byref(d) if d is not None else None, q, kp, vp, bt, cl,
                                           ctypes.c_float(1.0), out, None)


def test_noalloc_read_refusals(lib):
    # every check of pkv_paged_attention except the workspace, then the
    # static scratch's size; all before any HIP call
    assert noalloc(lib, None) == 1
    assert noalloc(lib, desc(head_dim=96)) == 5
    assert noalloc(lib, desc(), q=0) == 1
    assert noalloc(lib, desc(), out=FAKE + 8) == 2
    assert noalloc(lib, desc(rows=0)) == 0  # empty: nothing to do, no scratch looked up
    # fp32, 8192 rows x 32 heads x 64 partitions of 64 positions: 277 MB of partials
    big = desc(rows=8192, dtype=0, out_dtype=0)
    assert ws(lib, rows=8192, dtype=0, out_dtype=0) > 32 << 20
    assert noalloc(lib, big) == 13
    assert lib.pkv_strerror(13).decode().startswith("the read needs more scratch")


def attn(lib, d, q=FAKE, kp=FAKE, vp=FAKE, bt=FAKE, cl=FAKE, out=FAKE, wsp=FAKE, wsb=1 << 40):
    return lib.pkv_paged_attention(ctypes.byref(d) if d is not None else None, q, kp, vp, bt, cl,
                                   ctypes.c_float(1.0), out, wsp, wsb, None)


@pytest.mark.parametrize("field,value,status", [
    ("dtype", 2, 3), ("out_dtype", -1, 3), ("head_dim", 96, 5), ("head_dim", 256, 5),
    ("block_size", 12, 6), ("block_size", 64, 6), ("n_kv_heads", 5, 4), ("n_kv_heads", 0, 4),
    ("n_heads", 256, 4),  # group 32 > 16
    ("rows", -1, 7), ("rows", 70000, 7), ("max_blocks_per_row", 0, 7), ("num_blocks", 0, 7),
    ("partition_tokens", 24, 9), ("partition_tokens", -16, 9),
])
def test_attention_refusals(lib, field, value, status):
    d = desc(**{field: value})
    assert attn(lib, d, q=0) in (status, 1)  # q NULL as well: nothing may launch
    assert attn(lib, d, q=FAKE + 4) == status  # misaligned q too: the shape check comes first


def test_attention_pointer_and_workspace_refusals(lib):
    d = desc()
    assert attn(lib, None) == 1
    for name in ("q", "kp", "vp", "bt", "cl", "out"):
        assert attn(lib, d, **{name: 0}) == 1, name
    for name in ("q", "kp", "vp", "out"):
        assert attn(lib, d, **{name: FAKE + 8}) == 2, name
    assert attn(lib, d, bt=FAKE + 2) == 2
    assert attn(lib, d, wsp=0) == 8
    assert attn(lib, d, wsb=ws(lib) - 1) == 8
    assert attn(lib, d, wsp=FAKE + 4) == 2
    # zero rows is a valid empty call and launches nothing
    assert attn(lib, desc(rows=0)) == 0


def scatter(lib, k=FAKE, v=FAKE, sm=FAKE, T=4, kp=FAKE, vp=FAKE, nb=8, bs=16, nkv=2, hd=64, dt=1):
    return lib.pkv_reshape_and_cache(k, v, sm, T, kp, vp, nb, bs, nkv, hd, dt, None)


def test_scatter_refusals(lib):
    assert scatter(lib, k=0) == 1
    assert scatter(lib, sm=0, T=0) == 1
    assert scatter(lib, dt=7) == 3
    assert scatter(lib, hd=32) == 5
    assert scatter(lib, bs=4) == 6
    assert scatter(lib, T=-1) == 7
    assert scatter(lib, nb=0) == 7
    assert scatter(lib, nkv=0) == 7
    assert scatter(lib, nb=1 << 62) == 7  # pool bytes overflow
    assert scatter(lib, k=FAKE + 4) == 2
    assert scatter(lib, sm=FAKE + 4) == 2
    assert scatter(lib, T=0) == 0  # nothing to do, nothing launched


# ---------------------------------------------------------------------------
# pkv_decode_step: every check of the scatter and of the read runs first
# ---------------------------------------------------------------------------

def step(lib, d, kn=FAKE, vn=FAKE, sl=FAKE, q=FAKE, wsb=1 << 40):
    return lib.pkv_decode_step(ctypes.byref(d), kn, vn, sl, q, FAKE, FAKE, FAKE, FAKE, ctypes.c_float(1.0),
                               FAKE, FAKE, wsb, None)


def test_decode_step_refusals(lib):
    assert step(lib, desc(), kn=0) == 1          # NULL k_new
    assert step(lib, desc(), sl=FAKE + 4) == 2   # misaligned slot mapping
    assert step(lib, desc(), q=0) == 1           # the read's own checks
    assert step(lib, desc(head_dim=96)) == 5
    assert step(lib, desc(), wsb=16) == 8        # workspace too small
    assert step(lib, desc(n_kv_heads=5000, n_heads=5000)) in (4, 7)


# ---------------------------------------------------------------------------
# read counters (host arithmetic), pinned to the Day 60 wirebench table
# ---------------------------------------------------------------------------

from test_oracle_pins import load_wirebench  # noqa: E402


@pytest.mark.parametrize("entry", load_wirebench(), ids=lambda e: "rows%d_block%s" % (e["rows"], e["block"]))
def test_read_counters_reproduce_wirebench(lib, entry):
    # 2 layers x 47 decode steps, 8 query heads (the page's tiny engine), one
    # query per row; widths 17..63 for rows 4 and 8, 9..55 for rows 2 (as in
    # the oracle's pin of the same table)
    block = entry["block"]
    c = binding.ReadCounters("gathered" if block is None else "streamed", block or 1)
    first = 17 if entry["rows"] in (4, 8) else 9
    for w in range(first, first + 47):
        for _ in range(2):
            c.record(entry["rows"], 8, 1, w)
    assert (c.calls, c.score_cells, c.held_cells) == (entry["reads"], entry["charged"], entry["held"])
    assert c.rows == entry["rows"] * entry["reads"]
    assert "%.1fx" % c.saving == entry["saving"]


def test_read_counters_window_and_refusals(lib):
    c = binding.ReadCounters("streamed", 16)
    assert c.saving == 1.0  # nothing held yet: 1, not "unmeasured"
    c.record(4, 32, 1, 1000)
    first = c.snapshot()
    c.record(4, 32, 1, 1001)
    w = c.since(first)
    assert (w.calls, w.rows, w.score_cells, w.held_cells) == (1, 4, 4 * 32 * 1001, 4 * 32 * 16)
    assert w.saving == pytest.approx(1001 / 16)
    with pytest.raises(binding.PkvError) as e:  # a reading of another read
        c.since(binding.ReadCounters("streamed", 32))
    assert e.value.status == 11
    with pytest.raises(binding.PkvError) as e:
        c.since(binding.ReadCounters("gathered", 16))
    assert e.value.status == 11
    with pytest.raises(binding.PkvError) as e:  # later minus earlier only
        first.since(c)
    assert e.value.status == 7
    g = binding.ReadCounters("gathered", 1)
    g.record(3, 8, 2, 40)
    assert g.held_cells == g.score_cells == 3 * 8 * 2 * 40 and g.saving == 1.0
    with pytest.raises(binding.PkvError):
        g.record(-1, 8, 1, 4)
    with pytest.raises(binding.PkvError):  # 2^31 x 2^31 x 2^31 x 2^31 cells overflow int64
        g.record(2 ** 31 - 1, 2 ** 31 - 1, 2 ** 31 - 1, 2 ** 31 - 1)
    assert g.calls == 1


def test_read_tile_names_what_each_read_holds(lib):
    tile = lambda **kw: lib.pkv_read_tile(ctypes.byref(desc(**kw)))
    assert tile() == 32                                   # stream read: one wave, one group
    assert tile(rows=8, max_blocks_per_row=64) == 256     # matrix-core partition read, 8 waves (128 workgroups)
    assert tile(rows=64, max_blocks_per_row=64) == 128    # 4 waves: 512 workgroups
    assert tile(dtype=0, out_dtype=0, head_dim=64) == 64  # VALU partition read, fp32
    assert tile(dtype=0, out_dtype=0, head_dim=128) == 32
    assert tile(dtype=0, out_dtype=0, head_dim=16) == 256
    assert tile(head_dim=16) == 512                       # bf16 head_dim 16: VALU
    assert tile(head_dim=96) == 0
    assert lib.pkv_read_tile(None) == 0


def test_read_counters_count_a_descriptor(lib):
    d = desc(rows=64, n_heads=32, max_blocks_per_row=256, block_size=16)
    c = binding.ReadCounters("streamed", lib.pkv_read_tile(ctypes.byref(d)))
    c.record_read(d)
    # the table's width is charged (the library never reads the lengths);
    # the stream read holds 32 positions per (row, head)
    assert (c.calls, c.rows, c.score_cells, c.held_cells) == (1, 64, 64 * 32 * 4096, 64 * 32 * 32)
    # a streamed counter of another tile width is another read's counter
    with pytest.raises(binding.PkvError) as e:
        binding.ReadCounters("streamed", 16).record_read(d)
    assert e.value.status == 11
    g = binding.ReadCounters("gathered", 1)
    g.record_read(d)
    assert g.held_cells == g.score_cells == 64 * 32 * 4096


# ---------------------------------------------------------------------------
# multi-query read: host-side plan and refusals
# ---------------------------------------------------------------------------

def multi(lib, d, qlen, q=FAKE, wsb=1 << 40):
    return lib.pkv_paged_attention_multi(ctypes.byref(d), qlen, q, FAKE, FAKE, FAKE, FAKE, ctypes.c_float(1.0),
                                         FAKE, FAKE, wsb, None)


def test_multi_query_refusals(lib):
    assert multi(lib, desc(dtype=0, out_dtype=0), 4) == 3     # fp32: not supported by this read
    assert multi(lib, desc(head_dim=16), 4) == 5
    assert multi(lib, desc(), 0) == 7
    assert multi(lib, desc(), 70000) == 7
    assert multi(lib, desc(), 4, q=0) == 1
    assert multi(lib, desc(), 4, wsb=8) == 8
    assert multi(lib, desc(partition_tokens=-32), 8) == 9
    # the multi-query partition is rounded up to 32 positions and capped at
    # 4096, so lengths the one-query read would refuse are taken: not a
    # multiple of the block size, or more than 4096 blocks
    mws = lambda d, q: lib.pkv_paged_attention_multi_workspace_size(ctypes.byref(d), q)
    assert mws(desc(partition_tokens=40), 8) == mws(desc(partition_tokens=64), 8) > 0
    assert mws(desc(partition_tokens=40), 4) == mws(desc(partition_tokens=64), 4) > 0  # stream path
    big = dict(block_size=8, max_blocks_per_row=8192, num_blocks=70000)
    assert mws(desc(partition_tokens=40000, **big), 8) == mws(desc(partition_tokens=4096, **big), 8) > 0


def test_multi_query_workspace(lib):
    ws = lambda d, q: lib.pkv_paged_attention_multi_workspace_size(ctypes.byref(d), q)
    # 4 queries x 4 heads per kv head = 16 columns: the stream path, whose
    # workspace is the one-query read's layout with 16 columns per slot --
    # header, wave starts, row prefixes, then two slots per persistent wave
    # of 16 x (128 + 2) floats
    d = desc()
    head = 4 + 2 * 1024 + 65
    head = (head + 3) & ~3
    assert ws(d, 4) == (head + 2 * 1024 * 16 * 130) * 4
    # 8 queries (32 columns), one query block per (row, kv head), <= 256
    # rows: the balanced multi-query read.  One 2-wave workgroup per slice,
    # two per compute unit (512); the stream layout for 512 slices: header,
    # slice starts, row prefixes, then two slots per slice of 32 x (128 + 2)
    # floats.  A caller's partition sets the slice minimum only.
    def balanced(rows, cols, slices):
        head = (4 + 2 * slices + rows + 1 + 3) & ~3
        return (head + 2 * slices * ((cols * 130 + 3) & ~3)) * 4
    assert ws(d, 8) == balanced(64, 32, 512)
    assert ws(desc(rows=16), 8) == balanced(16, 32, 512)
    assert ws(desc(partition_tokens=1008), 8) == balanced(64, 32, 512)
    # 64 queries (256 columns, 8 waves, one workgroup per compute unit)
    assert ws(desc(rows=16), 64) == balanced(16, 256, 256)
    # the workgroup path: two query blocks (100 queries of 4 heads: 13
    # tiles of 32 columns, blocks of 8 waves), or more than 256 rows.
    # 64 rows x 8 kv heads x 2 blocks = 1024 workgroups on 256 slots: a
    # 4096-position table wants 16384-position partitions, capped at 2048
    # for 8-wave workgroups: 2 partitions of m, l and a 128-float acc per
    # (row, query, head, partition)
    def parts(rows, q, p):
        slots = rows * q * 32 * p
        return (((2 * slots + 3) & ~3) + slots * 128) * 4
    assert ws(d, 100) == parts(64, 100, 2)
    # 300 rows, 8 queries: 2-wave workgroups stop at 1024 positions (4 parts)
    assert ws(desc(rows=300), 8) == parts(300, 8, 4)
    # a caller's partition (a multiple of the block size) is rounded up to
    # 32 positions and capped at 4096
    assert ws(desc(partition_tokens=1008), 100) == parts(64, 100, 4)
    assert ws(desc(partition_tokens=8192), 100) == 0   # capped at 4096: one partition, written directly
    assert ws(desc(max_blocks_per_row=64, partition_tokens=1024), 100) == 0
    assert ws(desc(dtype=0, out_dtype=0), 4) == 0    # refused descriptors need nothing
