// Internal declarations shared by the host code (np_host.cpp, plain C++) and
// the HIP launch code. No HIP headers here: the host half builds with g++.
#pragma once

#include <cstddef>
#include <cstdint>
#include <mutex>
#include <vector>

#include "np_paged.h"
#include "np_trace.h"

namespace np {

constexpr uint32_t kPlanMagic = 0x4e50504cu;   // "NPPL"
constexpr int kWaveSize = 64;
constexpr int kDecodeWaves = 4;                // waves per decode workgroup
constexpr int kPrefillUnits = 4;               // (head, query rows) units per prefill workgroup
constexpr int kPrefillWaves = 8;               // waves per prefill workgroup: two per unit
constexpr int kPrefillRowsPerWave = 64;        // query rows of one head per wave
constexpr int kMaxGroup = 8;                   // largest Hq/Hkv with a kernel
constexpr size_t kWsAlign = 256;
constexpr int kCounterStride = 64;             // uint32 words between arrival counters
constexpr int kScheduleUniform = 1;            // decode: uniform page-aligned splits
constexpr int kScheduleStreamK = 2;            // decode: equal work per workgroup
constexpr int kSkMaxSeqs = 2048;               // stream-K: sequences per launch
constexpr int kSkDefaultCost = 4;              // stream-K: virtual blocks per segment
constexpr int kSkWaves = 8;                    // waves per stream-K decode workgroup
constexpr int kSkWgsPerCu = 1;                 // stream-K: resident decode workgroups per CU
constexpr int kSkMinUnits = 8;                 // stream-K: least units per workgroup
constexpr int kTraceStamps = NP_TRACE_STAMPS;  // trace build: phase stamps per workgroup

// Stream-K: KV heads one decode workgroup serves (the largest of 4, 2, 1 that
// divides Hkv).
constexpr int sk_heads_per_wg(int hkv) {
  return hkv % 8 == 0 ? 8 : hkv % 4 == 0 ? 4 : hkv % 2 == 0 ? 2 : 1;
}

// Sizes every launch depends on, fixed when the plan is made.
struct np_plan_core {
  int32_t dtype, num_seqs, n_q_total, hq, hkv, head_dim, block_size, max_blocks;
  int32_t group;           // Hq / Hkv
  int32_t d_pad;           // next power of two >= head_dim
  int32_t is_prefill;
  // decode
  int32_t schedule;        // kScheduleUniform or kScheduleStreamK
  int32_t blocks_per_split;  // uniform: blocks per split; stream-K: units per workgroup
  int32_t max_splits;      // over sequences (stream-K: pieces of one segment)
  int32_t sk_cost;         // stream-K: virtual units per (sequence, KV head)
  // prefill
  int32_t max_tiles;       // workgroup tiles per (sequence, KV head), max over sequences
  int32_t max_rows;        // query (or appended) rows of the longest sequence
  // launch
  uint32_t grid[3];
  uint32_t wg_size;
  uint32_t combine_wgs;     // workgroups of the separate combine kernel (0: none)
  int32_t fused_combine;    // splits merged by the last arriving workgroup
  // workspace (bytes from the workspace base)
  size_t ws_cnt_off;       // uint32 arrival counters [num_seqs][Hkv], kCounterStride apart
  size_t ws_ml_off;        // float2 (m, l) [num_seqs][Hq][max_splits] (stream-K: [2 W][G])
  size_t ws_acc_off;       // float [num_seqs][Hq][max_splits][d_pad] (stream-K: [2 W][G][d_pad])
  size_t ws_bytes;
};

}  // namespace np

struct np_plan_s {
  uint32_t magic;
  np::np_plan_core core;
  // The host lengths (and query starts) the plan was made for: launches need
  // only `core`; the work-item list, for inspection, is derived from these on
  // the first accessor call, so planning stays O(sequences).
  std::vector<int32_t> lens;
  std::vector<int32_t> q_start;
  mutable std::once_flag items_once;
  mutable std::vector<int32_t> items;   // 5 ints per active workgroup, launch order
};

namespace np {

// Descriptor-level checks shared by np_check_paged_inputs and the launchers.
np_status check_desc(const np_paged_desc* d);
// A NULL block table (the contiguous layout) needs num_seqs * max_blocks_per_seq
// blocks in the pool.
np_status check_contiguous(const np_paged_desc* d, const int32_t* block_table);
np_status check_pointers(const np_paged_desc* d, const void* q, const void* k_pool,
                         const void* v_pool, const int32_t* block_table,
                         const int32_t* context_lens, const void* out);
// The plan was made for this descriptor.
np_status check_plan(const np_paged_desc* d, const np_plan_t* plan, int want_prefill);
size_t dtype_size(int32_t dtype);

}  // namespace np
