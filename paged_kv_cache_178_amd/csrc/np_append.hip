// Scatter of new K/V rows into the paged pool: the second half of the cache
// write ("Day 20: the number the Triton kernel has to beat", section "What I
// learned": extend the table, then store the new K/V in their slots). Token t of sequence s lives in slot
// t % block_size of physical block block_table[s][t / block_size] (the
// paged layout of "3. Paged KV-cache attention" in "I Wrote the Three
// Attention Kernels That Run LLM Inference"); the new rows of a sequence are
// its last positions, past_s .. context_lens[s] - 1.
//
// One wave per new row; lanes copy the row's 16-byte chunks (all KV heads) of
// K and of V with one 128-bit load and store each. The work is a copy bound by
// HBM bandwidth: 2 * Hkv * d * elt bytes read and the same written per row.

#include <hip/hip_runtime.h>

#include <cstdint>

#include "np_internal.h"
#include "np_table.h"

namespace np {

namespace {

constexpr int kAppendRowsPerWg = 4;   // one wave per new row

struct AppendParams {
  const char* k_new;
  const char* v_new;
  char* k_pool;
  char* v_pool;
  const int32_t* bt;
  const int32_t* lens;
  const int32_t* new_start;
  int64_t n_s0, n_s1;            // bytes between new rows, between their heads
  int64_t kv_s0, kv_s1, kv_s2;   // bytes between blocks, slots, heads of the pools
  int64_t bt_stride;             // elements
  int32_t bt_contig;             // 1: NULL table, contiguous layout
  int32_t hkv, block_size, n_blocks, max_blocks, chunks_per_head;
};

__global__ __launch_bounds__(kAppendRowsPerWg * kWaveSize) void paged_append_kernel(
    const AppendParams p) {
  const int s = blockIdx.y;
  const int wave = threadIdx.x / kWaveSize;
  const int lane = threadIdx.x % kWaveSize;
  const int r0 = p.new_start[s];
  const int n = p.new_start[s + 1] - r0;
  const int i = blockIdx.x * kAppendRowsPerWg + wave;
  if (i >= n) return;
  const int t = p.lens[s] - n + i;   // absolute position of the row
  if (t < 0) return;                 // context_lens < new rows: nothing to write
  const int32_t phys = table_row(p.bt, p.bt_stride, s, p.max_blocks, p.bt_contig)[t / p.block_size];
  // A table entry outside the pool (e.g. -1, never allocated) writes nothing.
  if (phys < 0 || phys >= p.n_blocks) return;
  const int slot = t % p.block_size;
  const int64_t src = int64_t(r0 + i) * p.n_s0;
  const int64_t dst = int64_t(phys) * p.kv_s0 + int64_t(slot) * p.kv_s1;
  const int total = p.hkv * p.chunks_per_head;
  for (int c = lane; c < total; c += kWaveSize) {
    const int h = c / p.chunks_per_head;
    const int64_t off = int64_t(c % p.chunks_per_head) * 16;
    const uint4 kv = *reinterpret_cast<const uint4*>(p.k_new + src + h * p.n_s1 + off);
    const uint4 vv = *reinterpret_cast<const uint4*>(p.v_new + src + h * p.n_s1 + off);
    *reinterpret_cast<uint4*>(p.k_pool + dst + h * p.kv_s2 + off) = kv;
    *reinterpret_cast<uint4*>(p.v_pool + dst + h * p.kv_s2 + off) = vv;
  }
}

bool aligned16(const void* ptr) { return reinterpret_cast<uintptr_t>(ptr) % 16 == 0; }

}  // namespace

}  // namespace np

using namespace np;

extern "C" np_status np_paged_kv_append(const np_paged_desc* desc, const np_plan_t* plan,
                                        const void* k_new, const void* v_new,
                                        const int64_t new_stride[2],
                                        const int32_t* block_table,
                                        const int32_t* context_lens,
                                        const int32_t* new_start, void* k_pool, void* v_pool,
                                        void* stream) {
  np_status st = check_desc(desc);
  if (st != NP_OK) return st;
  if (!k_new || !v_new || !new_stride || !context_lens || !new_start || !k_pool || !v_pool)
    return NP_ERR_NULL_PTR;
  st = check_contiguous(desc, block_table);
  if (st != NP_OK) return st;
  if (!aligned16(k_new) || !aligned16(v_new) || !aligned16(k_pool) || !aligned16(v_pool) ||
      reinterpret_cast<uintptr_t>(block_table) % 4 || reinterpret_cast<uintptr_t>(context_lens) % 4 ||
      reinterpret_cast<uintptr_t>(new_start) % 4)
    return NP_ERR_MISALIGNED;
  const int64_t hd = desc->head_dim;
  const int64_t elt = static_cast<int64_t>(dtype_size(desc->dtype));
  if (new_stride[1] < hd || new_stride[0] < (desc->num_kv_heads - 1) * new_stride[1] + hd)
    return NP_ERR_BAD_STRIDE;
  if ((new_stride[0] * elt) % 16 || (new_stride[1] * elt) % 16) return NP_ERR_MISALIGNED;
  st = check_plan(desc, plan, 1);
  if (st != NP_OK) return st;
  const np_plan_core& c = plan->core;
  AppendParams prm{};
  prm.k_new = static_cast<const char*>(k_new);
  prm.v_new = static_cast<const char*>(v_new);
  prm.k_pool = static_cast<char*>(k_pool);
  prm.v_pool = static_cast<char*>(v_pool);
  // A NULL table (contiguous layout) reads a stand-in row: see np_table.h.
  prm.bt = block_table ? block_table : context_lens;
  prm.bt_contig = block_table == nullptr;
  prm.lens = context_lens;
  prm.new_start = new_start;
  prm.n_s0 = new_stride[0] * elt;
  prm.n_s1 = new_stride[1] * elt;
  prm.kv_s0 = desc->kv_stride[0] * elt;
  prm.kv_s1 = desc->kv_stride[1] * elt;
  prm.kv_s2 = desc->kv_stride[2] * elt;
  prm.bt_stride = block_table ? desc->bt_stride : 0;
  prm.hkv = desc->num_kv_heads;
  prm.block_size = desc->block_size;
  prm.n_blocks = desc->n_blocks;
  prm.max_blocks = desc->max_blocks_per_seq;
  prm.chunks_per_head = static_cast<int32_t>(hd * elt / 16);   // check_desc: hd * elt % 16 == 0
  dim3 grid((c.max_rows + kAppendRowsPerWg - 1) / kAppendRowsPerWg, c.num_seqs, 1);
  paged_append_kernel<<<grid, dim3(kAppendRowsPerWg * kWaveSize), 0,
                        static_cast<hipStream_t>(stream)>>>(prm);
  return hipGetLastError() == hipSuccess ? NP_OK : NP_ERR_HIP;
}
