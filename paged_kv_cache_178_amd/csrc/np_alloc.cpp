// Host block allocator for the paged KV cache. The cache write of "Day 20:
// the number the Triton kernel has to beat" (section "What I learned") first
// extends a sequence's block table, then stores the new K/V in their slots;
// this file is the first half, np_paged_kv_append the second.
//
// Free blocks form a stack (the back of `free_` is the top): allocation pops,
// release pushes a sequence's blocks back in reverse so its first block ends
// on top. The order is fixed by the calls alone, so tables are reproducible.

#include <cstdint>
#include <new>
#include <vector>

#include "np_paged.h"

struct np_block_allocator {
  int32_t n_blocks = 0, block_size = 0, num_seqs = 0, max_blocks = 0;
  std::vector<int32_t> free_;    // stack of free block ids, top at the back
  std::vector<int32_t> table;    // [num_seqs][max_blocks], -1 = unused
  std::vector<int32_t> lens;     // [num_seqs]
  std::vector<int32_t> used;     // blocks held per sequence
};

namespace {

bool is_pow2(int64_t x) { return x > 0 && (x & (x - 1)) == 0; }

int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }

}  // namespace

extern "C" {

np_status np_alloc_create(int32_t n_blocks, int32_t block_size, int32_t num_seqs,
                          int32_t max_blocks_per_seq, const int32_t* free_order,
                          np_block_allocator_t** out) {
  if (out == nullptr) return NP_ERR_NULL_PTR;
  *out = nullptr;
  if (n_blocks < 1 || num_seqs < 1 || max_blocks_per_seq < 1 || !is_pow2(block_size) ||
      block_size > 256)
    return NP_ERR_BAD_SHAPE;
  np_block_allocator* a = new (std::nothrow) np_block_allocator;
  if (a == nullptr) return NP_ERR_BAD_SHAPE;
  a->n_blocks = n_blocks;
  a->block_size = block_size;
  a->num_seqs = num_seqs;
  a->max_blocks = max_blocks_per_seq;
  a->free_.resize(n_blocks);
  if (free_order != nullptr) {
    // A permutation of 0 .. n_blocks-1: every id once.
    std::vector<char> seen(n_blocks, 0);
    for (int32_t i = 0; i < n_blocks; ++i) {
      const int32_t b = free_order[i];
      if (b < 0 || b >= n_blocks || seen[b]) {
        delete a;
        return NP_ERR_BAD_BLOCK_TABLE;
      }
      seen[b] = 1;
    }
  }
  // free_order[0] is handed out first, so it goes on top of the stack.
  for (int32_t i = 0; i < n_blocks; ++i)
    a->free_[n_blocks - 1 - i] = free_order ? free_order[i] : i;
  a->table.assign(static_cast<size_t>(num_seqs) * max_blocks_per_seq, -1);
  a->lens.assign(num_seqs, 0);
  a->used.assign(num_seqs, 0);
  *out = a;
  return NP_OK;
}

void np_alloc_destroy(np_block_allocator_t* alloc) { delete alloc; }

np_status np_alloc_extend(np_block_allocator_t* a, int32_t seq, int32_t new_len) {
  if (a == nullptr) return NP_ERR_NULL_PTR;
  if (seq < 0 || seq >= a->num_seqs) return NP_ERR_BAD_SHAPE;
  if (new_len < a->lens[seq] ||
      new_len > static_cast<int64_t>(a->max_blocks) * a->block_size)
    return NP_ERR_BAD_CONTEXT_LEN;
  const int64_t need = ceil_div(new_len, a->block_size) - a->used[seq];
  if (need > static_cast<int64_t>(a->free_.size())) return NP_ERR_POOL_EXHAUSTED;
  int32_t* row = a->table.data() + static_cast<size_t>(seq) * a->max_blocks;
  for (int64_t i = 0; i < need; ++i) {
    row[a->used[seq]++] = a->free_.back();
    a->free_.pop_back();
  }
  a->lens[seq] = new_len;
  return NP_OK;
}

np_status np_alloc_release(np_block_allocator_t* a, int32_t seq) {
  if (a == nullptr) return NP_ERR_NULL_PTR;
  if (seq < 0 || seq >= a->num_seqs) return NP_ERR_BAD_SHAPE;
  int32_t* row = a->table.data() + static_cast<size_t>(seq) * a->max_blocks;
  for (int32_t j = a->used[seq] - 1; j >= 0; --j) {
    a->free_.push_back(row[j]);
    row[j] = -1;
  }
  a->used[seq] = 0;
  a->lens[seq] = 0;
  return NP_OK;
}

int32_t np_alloc_free_blocks(const np_block_allocator_t* a) {
  return a ? static_cast<int32_t>(a->free_.size()) : 0;
}

const int32_t* np_alloc_block_table(const np_block_allocator_t* a) {
  return a ? a->table.data() : nullptr;
}

const int32_t* np_alloc_context_lens(const np_block_allocator_t* a) {
  return a ? a->lens.data() : nullptr;
}

}  // extern "C"
