// Device-side view of one sequence's block-table row (HIP sources only).
//
// A NULL table selects the contiguous layout: logical block j of sequence s
// is physical block s * max_blocks_per_seq + j, so a pool with
// kv_stride[0] = block_size * kv_stride[1] is a dense
// [num_seqs, max_blocks_per_seq * block_size, Hkv, d] cache (the split-KV
// decode over one contiguous KV tensor of "I Wrote the Three Attention
// Kernels That Run LLM Inference", section "2. Split-KV flash-decoding").
// Otherwise the entry is read from the table (section "3. Paged KV-cache
// attention").
//
// The launchers pass, for a NULL table, another valid int32 device array
// (context_lens) with a row stride of 0 and contig = 1: an entry is then
// always loaded, from a valid address (its first element), and masked out
// by integer arithmetic. So the table read has no branch in front of it and
// issues as early as with a real table.
#pragma once

#include <hip/hip_runtime.h>

#include <cstdint>

namespace np {

// The table is never written during a launch, so its entries are read
// through the constant address space: a wave-uniform entry then becomes a
// scalar load (s_load, counted by lgkmcnt). A vector load of the same entry
// would be counted by vmcnt, which retires in issue order, so waiting for the
// next group's entries would also wait for every K/V load issued before them.
typedef const __attribute__((address_space(4))) int32_t* ConstI32Ptr;

struct TableRow {
  const int32_t* row;
  int32_t step;         // 1, or 0 for the contiguous layout (row[0] only)
  int32_t keep;         // -1 keeps the loaded entry, 0 drops it (contiguous)
  int32_t base;         // 0, or s * max_blocks_per_seq (contiguous)
  // The entry as loaded (the stand-in's first element when contiguous).
  __device__ __forceinline__ int32_t raw(int b) const {
    return ((ConstI32Ptr)row)[b * step];
  }
  // Physical block of logical block b from its raw entry: pure arithmetic,
  // no select, so the scalar load stays where a real table's load would be
  // and can be issued long before its use.
  __device__ __forceinline__ int32_t phys(int32_t raw_entry, int b) const {
    return (raw_entry & keep) + (b & ~keep) + base;
  }
  __device__ __forceinline__ int32_t operator[](int b) const { return phys(raw(b), b); }
};

__device__ __forceinline__ TableRow table_row(const int32_t* bt, int64_t bt_stride, int s,
                                              int max_blocks, int contig) {
  const int32_t keep = contig ? 0 : -1;
  return TableRow{bt + int64_t(s) * bt_stride, contig ? 0 : 1, keep, (s * max_blocks) & ~keep};
}

}  // namespace np
