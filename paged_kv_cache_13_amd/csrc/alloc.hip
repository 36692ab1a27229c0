// Host-side block allocator of the shared pool and slot mapping of appends.
//
// The pool is a fixed set of blocks shared by every sequence; a sequence
// takes a block when its length reaches a block boundary and gives all of
// its blocks back when it finishes, and the next sequences reuse them
// (nanoserve "Day 17" page, "What I added today" and "Post angle": the block
// allocator and free-and-reuse; exhaustion is an error the caller sees, the
// pages' KVCacheExhausted).  No device memory, no allocation: the caller
// provides the storage.
#include <string.h>

#include "pkv.h"

namespace {

// splitmix64 (Steele, Lea, Flood 2014): the shuffle of the initial free list.
uint64_t splitmix64(uint64_t &x) {
  uint64_t z = (x += 0x9E3779B97F4A7C15ull);
  z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
  z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
  return z ^ (z >> 31);
}

}  // namespace

extern "C" {

size_t pkv_allocator_storage_bytes(int64_t num_blocks) {
  if (num_blocks < 1 || num_blocks > INT32_MAX) return 0;
  return (size_t)num_blocks * (sizeof(int32_t) + 1);
}

int pkv_allocator_init(pkv_block_allocator *a, void *storage, size_t storage_bytes, int64_t num_blocks,
                       uint64_t seed) {
  if (!a || !storage) return PKV_ERR_NULL;
  if (num_blocks < 1 || num_blocks > INT32_MAX) return PKV_ERR_SHAPE;
  if (storage_bytes < pkv_allocator_storage_bytes(num_blocks)) return PKV_ERR_WORKSPACE;
  if (((uintptr_t)storage & 3) != 0) return PKV_ERR_ALIGN;
  a->free_ids = static_cast<int32_t *>(storage);
  a->in_use = reinterpret_cast<uint8_t *>(a->free_ids + num_blocks);
  a->num_blocks = num_blocks;
  a->num_free = num_blocks;
  // the stack pops from the top: fill it so that block 0 comes out first,
  // then (seed != 0) shuffle it (Fisher-Yates)
  for (int64_t i = 0; i < num_blocks; ++i) a->free_ids[i] = (int32_t)(num_blocks - 1 - i);
  if (seed != 0) {
    uint64_t st = seed;
    for (int64_t i = num_blocks - 1; i > 0; --i) {
      const int64_t j = (int64_t)(splitmix64(st) % (uint64_t)(i + 1));
      const int32_t t = a->free_ids[i];
      a->free_ids[i] = a->free_ids[j];
      a->free_ids[j] = t;
    }
  }
  memset(a->in_use, 0, (size_t)num_blocks);
  return PKV_OK;
}

int pkv_allocator_alloc(pkv_block_allocator *a, int64_t n, int32_t *ids) {
  if (!a || (!ids && n > 0)) return PKV_ERR_NULL;
  if (n < 0) return PKV_ERR_SHAPE;
  if (n > a->num_free) return PKV_ERR_EXHAUSTED;  // nothing is taken
  for (int64_t i = 0; i < n; ++i) {
    const int32_t b = a->free_ids[--a->num_free];
    a->in_use[b] = 1;
    ids[i] = b;
  }
  return PKV_OK;
}

int pkv_allocator_free(pkv_block_allocator *a, const int32_t *ids, int64_t n) {
  if (!a || (!ids && n > 0)) return PKV_ERR_NULL;
  if (n < 0) return PKV_ERR_SHAPE;
  // first pass: every id in range, in use and named once (marked 2 while
  // checking); on a bad id the marks are undone and nothing is freed
  for (int64_t i = 0; i < n; ++i) {
    if (ids[i] < 0 || ids[i] >= a->num_blocks || a->in_use[ids[i]] != 1) {
      for (int64_t j = 0; j < i; ++j) a->in_use[ids[j]] = 1;
      return PKV_ERR_SHAPE;
    }
    a->in_use[ids[i]] = 2;
  }
  for (int64_t i = 0; i < n; ++i) {
    a->in_use[ids[i]] = 0;
    a->free_ids[a->num_free++] = ids[i];
  }
  return PKV_OK;
}

int64_t pkv_allocator_num_free(const pkv_block_allocator *a) { return a ? a->num_free : -1; }

int pkv_append_slots(pkv_block_allocator *a, int32_t *table_row, int32_t max_blocks, int32_t block_size,
                     int32_t length, int32_t count, int64_t *slots) {
  if (!a || !table_row || (!slots && count > 0)) return PKV_ERR_NULL;
  if (block_size < 1 || max_blocks < 1 || length < 0 || count < 0) return PKV_ERR_SHAPE;
  if ((int64_t)length + count > (int64_t)max_blocks * block_size) return PKV_ERR_SHAPE;
  const int64_t first_new = ((int64_t)length + block_size - 1) / block_size;  // blocks already held
  const int64_t need = ((int64_t)length + count + block_size - 1) / block_size - first_new;
  if (need > a->num_free) return PKV_ERR_EXHAUSTED;  // nothing is taken
  if (need > 0) pkv_allocator_alloc(a, need, table_row + first_new);
  for (int32_t i = 0; i < count; ++i) {
    const int64_t pos = (int64_t)length + i;
    slots[i] = (int64_t)table_row[pos / block_size] * block_size + pos % block_size;
  }
  return PKV_OK;
}

}  // extern "C"
