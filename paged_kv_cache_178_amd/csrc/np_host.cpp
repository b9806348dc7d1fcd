// Host half of the library: input checks and the split/grid planner.
//
// Plain C++17 with no HIP dependency, so every integer the kernels turn into
// a pointer or a loop bound is produced and tested without a GPU ("Day 23:
// the real triton.jit paged-attention kernel", section "What I added today").

#include <algorithm>
#include <cmath>
#include <cstring>
#include <limits>
#include <new>

#include "np_internal.h"

namespace np {

size_t dtype_size(int32_t dtype) {
  switch (dtype) {
    case NP_F32: return 4;
    case NP_F16: return 2;
    case NP_BF16: return 2;
    default: return 0;
  }
}

static bool is_pow2(int64_t x) { return x > 0 && (x & (x - 1)) == 0; }

static int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }

static bool aligned(const void* p, uintptr_t a) {
  return (reinterpret_cast<uintptr_t>(p) % a) == 0;
}

np_status check_desc(const np_paged_desc* d) {
  if (d == nullptr) return NP_ERR_NULL_PTR;
  if (dtype_size(d->dtype) == 0) return NP_ERR_BAD_DTYPE;
  if (d->num_seqs < 1 || d->n_q_total < d->num_seqs || d->num_q_heads < 1 ||
      d->num_kv_heads < 1 || d->head_dim < 1 || d->n_blocks < 1 ||
      d->max_blocks_per_seq < 1 || d->reserved0 != 0 || d->reserved1 != 0)
    return NP_ERR_BAD_SHAPE;
  if (!is_pow2(d->block_size) || d->block_size > 256) return NP_ERR_BAD_SHAPE;
  if (d->num_q_heads % d->num_kv_heads != 0) return NP_ERR_BAD_GQA;
  if (!(d->scale <= 0.0f || std::isfinite(d->scale))) return NP_ERR_BAD_SHAPE;
  const int64_t hd = d->head_dim;
  // Rows must not overlap: each stride covers the extent of the dimension below.
  if (d->q_stride[1] < hd || d->q_stride[0] < (d->num_q_heads - 1) * d->q_stride[1] + hd)
    return NP_ERR_BAD_STRIDE;
  if (d->out_stride[1] < hd ||
      d->out_stride[0] < (d->num_q_heads - 1) * d->out_stride[1] + hd)
    return NP_ERR_BAD_STRIDE;
  if (d->kv_stride[2] < hd ||
      d->kv_stride[1] < (d->num_kv_heads - 1) * d->kv_stride[2] + hd ||
      d->kv_stride[0] < (d->block_size - 1) * d->kv_stride[1] +
                            (d->num_kv_heads - 1) * d->kv_stride[2] + hd)
    return NP_ERR_BAD_STRIDE;
  if (d->bt_stride < d->max_blocks_per_seq) return NP_ERR_BAD_STRIDE;
  // Every row starts on a 16-byte boundary so the kernels can use 128-bit loads.
  const int64_t elt = static_cast<int64_t>(dtype_size(d->dtype));
  const int64_t strides[] = {d->q_stride[0], d->q_stride[1], d->kv_stride[0],
                             d->kv_stride[1], d->kv_stride[2], d->out_stride[0],
                             d->out_stride[1]};
  for (int64_t s : strides)
    if ((s * elt) % 16 != 0) return NP_ERR_MISALIGNED;
  if ((hd * elt) % 16 != 0) return NP_ERR_MISALIGNED;
  return NP_OK;
}

np_status check_contiguous(const np_paged_desc* d, const int32_t* block_table) {
  // Without a table, sequence s owns physical blocks s * max_blocks_per_seq ..
  // (s + 1) * max_blocks_per_seq - 1: the pool must hold them all.
  if (block_table == nullptr &&
      int64_t(d->num_seqs) * d->max_blocks_per_seq > int64_t(d->n_blocks))
    return NP_ERR_BAD_BLOCK_TABLE;
  return NP_OK;
}

np_status check_pointers(const np_paged_desc* d, const void* q, const void* k_pool,
                         const void* v_pool, const int32_t* block_table,
                         const int32_t* context_lens, const void* out) {
  if (!q || !k_pool || !v_pool || !context_lens || !out) return NP_ERR_NULL_PTR;
  const np_status st = check_contiguous(d, block_table);
  if (st != NP_OK) return st;
  if (!aligned(q, 16) || !aligned(k_pool, 16) || !aligned(v_pool, 16) || !aligned(out, 16))
    return NP_ERR_MISALIGNED;
  if (!aligned(block_table, 4) || !aligned(context_lens, 4)) return NP_ERR_MISALIGNED;
  return NP_OK;
}

np_status check_plan(const np_paged_desc* d, const np_plan_t* plan, int want_prefill) {
  if (plan == nullptr || plan->magic != kPlanMagic) return NP_ERR_BAD_PLAN;
  const np_plan_core& c = plan->core;
  if (c.is_prefill != want_prefill || c.dtype != d->dtype || c.num_seqs != d->num_seqs ||
      c.n_q_total != d->n_q_total || c.hq != d->num_q_heads || c.hkv != d->num_kv_heads ||
      c.head_dim != d->head_dim || c.block_size != d->block_size ||
      c.max_blocks != d->max_blocks_per_seq)
    return NP_ERR_BAD_PLAN;
  return NP_OK;
}

static np_status check_host_arrays(const np_paged_desc* d, const int32_t* lens,
                                   const int32_t* q_start, const int32_t* table) {
  if (lens == nullptr) return NP_OK;
  const int64_t cap = static_cast<int64_t>(d->max_blocks_per_seq) * d->block_size;
  if (q_start == nullptr) {
    if (d->n_q_total != d->num_seqs) return NP_ERR_BAD_SHAPE;
  } else {
    if (q_start[0] != 0 || q_start[d->num_seqs] != d->n_q_total) return NP_ERR_BAD_SHAPE;
  }
  for (int32_t s = 0; s < d->num_seqs; ++s) {
    const int64_t n_q = q_start ? int64_t(q_start[s + 1]) - q_start[s] : 1;
    if (n_q < 1) return NP_ERR_BAD_SHAPE;
    if (lens[s] < n_q || lens[s] > cap) return NP_ERR_BAD_CONTEXT_LEN;
  }
  if (table == nullptr) return NP_OK;
  for (int32_t s = 0; s < d->num_seqs; ++s) {
    const int64_t used = ceil_div(lens[s], d->block_size);
    const int32_t* row = table + static_cast<int64_t>(s) * d->bt_stride;
    for (int64_t j = 0; j < used; ++j)
      if (row[j] < 0 || row[j] >= d->n_blocks) return NP_ERR_BAD_BLOCK_TABLE;
  }
  return NP_OK;
}

}  // namespace np

using namespace np;

extern "C" {

int32_t np_next_pow2(int32_t x) {
  if (x <= 1) return 1;
  int32_t p = 1;
  while (p < x && p < (1 << 30)) p <<= 1;
  return p;
}

const char* np_status_string(np_status s) {
  switch (s) {
    case NP_OK: return "ok";
    case NP_ERR_NULL_PTR: return "null pointer";
    case NP_ERR_BAD_DTYPE: return "bad dtype";
    case NP_ERR_BAD_SHAPE: return "bad shape";
    case NP_ERR_BAD_STRIDE: return "bad stride";
    case NP_ERR_MISALIGNED: return "misaligned pointer or row";
    case NP_ERR_BAD_GQA: return "num_q_heads is not a multiple of num_kv_heads";
    case NP_ERR_BAD_CONTEXT_LEN: return "bad context length";
    case NP_ERR_BAD_BLOCK_TABLE: return "block table entry out of range";
    case NP_ERR_UNSUPPORTED: return "shape valid but no kernel built for it";
    case NP_ERR_WORKSPACE_TOO_SMALL: return "workspace too small";
    case NP_ERR_BAD_PLAN: return "plan missing or made for another descriptor";
    case NP_ERR_HIP: return "HIP error";
    case NP_ERR_POOL_EXHAUSTED: return "block pool exhausted";
  }
  return "unknown status";
}

np_status np_check_paged_inputs(const np_paged_desc* desc, const void* q,
                                const void* k_pool, const void* v_pool,
                                const int32_t* block_table, const int32_t* context_lens,
                                const void* out, const int32_t* block_table_host,
                                const int32_t* context_lens_host,
                                const int32_t* q_start_host) {
  np_status st = check_desc(desc);
  if (st != NP_OK) return st;
  st = check_pointers(desc, q, k_pool, v_pool, block_table, context_lens, out);
  if (st != NP_OK) return st;
  return check_host_arrays(desc, context_lens_host, q_start_host, block_table_host);
}

namespace np {
namespace {

// Stream-K decode schedule (the kernel recomputes it on the device from the
// lengths it reads; this copy sizes the launch). A workgroup serves
// HW = sk_heads_per_wg(Hkv) KV heads at once; each (sequence, head group) is
// a segment of its blocks plus sk_cost virtual units; segments in (sequence,
// head group) order, U units in all, W workgroups of C = ceil(U / W)
// consecutive units. A piece is the part of a segment's blocks inside one
// workgroup's range.
void plan_stream_k(np_plan_core& c, const int32_t* lens, const np_plan_opts& o) {
  const int64_t cost = c.sk_cost;
  const int64_t hw = sk_heads_per_wg(c.hkv);
  const int64_t n_hg = c.hkv / hw;
  int64_t U = 0;
  for (int32_t s = 0; s < c.num_seqs; ++s) {
    const int64_t nb = std::min<int64_t>(ceil_div(lens[s], c.block_size), c.max_blocks);
    U += (nb + cost) * n_hg;
  }
  const int64_t num_cus = o.num_cus ? o.num_cus : 256;
  const int64_t per_cu = o.wgs_per_cu ? o.wgs_per_cu : kSkWgsPerCu;
  const int64_t min_units = o.min_blocks_per_split ? o.min_blocks_per_split : kSkMinUnits;
  int64_t W = std::min(num_cus * per_cu, ceil_div(U, min_units));
  W = std::max<int64_t>(1, std::min(W, U));
  const int64_t C = ceil_div(U, W);
  // The most pieces of one segment.
  int64_t max_pieces = 1;
  int64_t seg_start = 0;
  for (int32_t s = 0; s < c.num_seqs; ++s) {
    const int64_t nb = std::min<int64_t>(ceil_div(lens[s], c.block_size), c.max_blocks);
    for (int64_t hg = 0; hg < n_hg; ++hg) {
      const int64_t real_end = seg_start + std::max<int64_t>(nb, 1);
      max_pieces = std::max(max_pieces, (real_end - 1) / C - seg_start / C + 1);
      seg_start += nb + cost;
    }
  }
  c.schedule = kScheduleStreamK;
  c.blocks_per_split = static_cast<int32_t>(C);
  c.max_splits = static_cast<int32_t>(max_pieces);
  c.max_tiles = 0;
  c.max_rows = 1;
  c.grid[0] = static_cast<uint32_t>(W);
  c.grid[1] = c.grid[2] = 1;
  c.wg_size = kSkWaves * kWaveSize;
  c.fused_combine = 1;
  c.combine_wgs = 0;
  // Counters, then two partial slots per workgroup, each of HW * G query
  // heads; always present, since the device lengths decide which segments
  // are shared.
  auto round = [](size_t x) { return (x + kWsAlign - 1) / kWsAlign * kWsAlign; };
  const size_t n_part = size_t(2 * W) * hw * c.group;
  c.ws_cnt_off = 0;
  c.ws_ml_off = round(size_t(c.num_seqs) * c.hkv * kCounterStride * sizeof(uint32_t));
  c.ws_acc_off = c.ws_ml_off + round(n_part * 2 * sizeof(float));
  c.ws_bytes = c.ws_acc_off + round(n_part * c.d_pad * sizeof(float));
}

// The work-item list of a plan, in launch order of the active workgroups
// (5 ints each: sequence, KV head, split / workgroup / tile, first, end).
void build_items(const np_plan_s& plan, std::vector<int32_t>& items) {
  const np_plan_core& c = plan.core;
  const int32_t* lens = plan.lens.data();
  auto add = [&](int64_t a, int64_t b, int64_t d, int64_t e, int64_t f) {
    const int32_t item[5] = {int32_t(a), int32_t(b), int32_t(d), int32_t(e), int32_t(f)};
    items.insert(items.end(), item, item + 5);
  };
  if (c.is_prefill) {
    // One workgroup per (sequence, KV head, tile); a tile is kPrefillUnits
    // units, a unit one query head times kPrefillRowsPerWave rows, units
    // numbered head-fastest; the largest tiles are launched first.
    const int32_t* qs = plan.q_start.data();
    for (int32_t s = 0; s < c.num_seqs; ++s) {
      const int64_t n_q = int64_t(qs[s + 1]) - qs[s];
      const int64_t units = c.group * ceil_div(n_q, kPrefillRowsPerWave);
      const int64_t tiles = ceil_div(units, kPrefillUnits);
      for (int64_t x = 0; x < int64_t(c.grid[0]); ++x) {
        const int64_t tile = c.max_tiles - 1 - x / c.hkv, kvh = x % c.hkv;
        if (tile >= tiles) continue;
        const int64_t u0 = tile * kPrefillUnits;
        const int64_t u1 = std::min<int64_t>(u0 + kPrefillUnits, units);
        const int64_t r0 = (u0 / c.group) * kPrefillRowsPerWave;
        const int64_t r1 = std::min<int64_t>(((u1 - 1) / c.group + 1) * kPrefillRowsPerWave, n_q);
        add(s, kvh, tile, r0, r1);
      }
    }
  } else if (c.schedule == kScheduleStreamK) {
    const int64_t cost = c.sk_cost, hw = sk_heads_per_wg(c.hkv), n_hg = c.hkv / hw;
    const int64_t W = c.grid[0], C = c.blocks_per_split;
    std::vector<std::vector<int32_t>> by_wg(W);
    int64_t seg_start = 0;
    for (int32_t s = 0; s < c.num_seqs; ++s) {
      const int64_t nb = std::min<int64_t>(ceil_div(lens[s], c.block_size), c.max_blocks);
      for (int64_t hg = 0; hg < n_hg; ++hg) {
        const int64_t real_end = seg_start + std::max<int64_t>(nb, 1);
        for (int64_t w = seg_start / C; w <= (real_end - 1) / C; ++w) {
          const int64_t lo = std::max(seg_start, w * C) - seg_start;
          const int64_t hi = std::min(real_end, (w + 1) * C) - seg_start;
          for (int64_t k = 0; k < hw; ++k) {
            const int32_t item[5] = {s, int32_t(hg * hw + k), int32_t(w), int32_t(lo),
                                     int32_t(std::min<int64_t>(hi, nb))};
            by_wg[w].insert(by_wg[w].end(), item, item + 5);
          }
        }
        seg_start += nb + cost;
      }
    }
    for (const auto& v : by_wg) items.insert(items.end(), v.begin(), v.end());
  } else {
    // Uniform splits: blocks_per_split consecutive blocks per split.
    const int64_t bps = c.blocks_per_split;
    for (int32_t s = 0; s < c.num_seqs; ++s) {
      const int64_t nb = ceil_div(lens[s], c.block_size);
      const int64_t splits = ceil_div(nb, bps);
      for (int64_t x = 0; x < int64_t(c.grid[0]); ++x) {
        const int64_t split = x / c.hkv, kvh = x % c.hkv;
        if (split >= splits) continue;
        add(s, kvh, split, split * bps, std::min<int64_t>(split * bps + bps, nb));
      }
    }
  }
}

}  // namespace
}  // namespace np

np_status np_plan(const np_paged_desc* desc, const int32_t* lens, const int32_t* q_start,
                  const np_plan_opts* opts, np_plan_t** out) {
  if (out == nullptr || lens == nullptr) return NP_ERR_NULL_PTR;
  *out = nullptr;
  np_status st = check_desc(desc);
  if (st != NP_OK) return st;
  st = check_host_arrays(desc, lens, q_start, nullptr);
  if (st != NP_OK) return st;
  np_plan_opts o{};
  if (opts) o = *opts;
  if (o.reserved != 0 || o.num_cus < 0 || o.wgs_per_cu < 0 || o.min_blocks_per_split < 0 ||
      o.max_blocks_per_split < 0 || o.force_blocks_per_split < 0 || o.combine_mode < 0 ||
      o.combine_mode > 1 || o.schedule < 0 || o.schedule > kScheduleStreamK ||
      o.segment_cost < 0)
    return NP_ERR_BAD_SHAPE;
  // Stream-K replaces the split size and the separate combine.
  if (o.schedule == kScheduleStreamK &&
      (o.force_blocks_per_split > 0 || o.combine_mode != 0 || desc->num_seqs > kSkMaxSeqs))
    return NP_ERR_BAD_SHAPE;
  const int32_t num_cus = o.num_cus ? o.num_cus : 256;
  const int32_t wgs_per_cu = o.wgs_per_cu ? o.wgs_per_cu : 1;
  const int32_t min_bps = o.min_blocks_per_split ? o.min_blocks_per_split : 4;

  np_plan_s* plan = new (std::nothrow) np_plan_s();
  if (plan == nullptr) return NP_ERR_UNSUPPORTED;
  plan->magic = kPlanMagic;
  np_plan_core& c = plan->core;
  c.dtype = desc->dtype;
  c.num_seqs = desc->num_seqs;
  c.n_q_total = desc->n_q_total;
  c.hq = desc->num_q_heads;
  c.hkv = desc->num_kv_heads;
  c.head_dim = desc->head_dim;
  c.block_size = desc->block_size;
  c.max_blocks = desc->max_blocks_per_seq;
  c.group = c.hq / c.hkv;
  c.d_pad = np_next_pow2(c.head_dim);
  c.is_prefill = q_start != nullptr;

  bool stream_k = false;
  if (!c.is_prefill) {
    const int32_t cost = o.segment_cost ? o.segment_cost : kSkDefaultCost;
    // Units of the stream-K schedule; bounded by what the kernel can see.
    const int64_t u_bound =
        int64_t(c.num_seqs) * (int64_t(c.max_blocks) + cost) * c.hkv;
    if (o.schedule == kScheduleStreamK) {
      if (u_bound >= (int64_t(1) << 30)) {
        delete plan;
        return NP_ERR_BAD_SHAPE;
      }
      stream_k = true;
    } else if (o.schedule == 0) {
      // Stream-K pays off when the lengths are ragged (uniform splits then
      // leave a tail of long sequences); for equal lengths uniform splits are
      // already balanced and need no merge of shared segments.
      int64_t sum_nb = 0, max_nb = 0;
      for (int32_t s = 0; s < c.num_seqs; ++s) {
        const int64_t nb = ceil_div(lens[s], c.block_size);
        sum_nb += nb;
        max_nb = std::max(max_nb, nb);
      }
      const bool ragged = max_nb * 4 * c.num_seqs > sum_nb * 5;   // max > 1.25 x mean
      // ... and when the batch has enough blocks to give every workgroup of
      // the stream-K launch its least share; a small batch runs faster as
      // many small uniform splits.
      const int64_t hw = sk_heads_per_wg(c.hkv);
      const int64_t units = (sum_nb + int64_t(c.num_seqs) * cost) * (c.hkv / hw);
      const int64_t slots = int64_t(o.num_cus ? o.num_cus : 256) *
                            (o.wgs_per_cu ? o.wgs_per_cu : kSkWgsPerCu);
      const int64_t least = o.min_blocks_per_split ? o.min_blocks_per_split : kSkMinUnits;
      const bool fills = units >= slots * least;
      stream_k = c.num_seqs > 1 && ragged && fills && c.num_seqs <= kSkMaxSeqs &&
                 o.force_blocks_per_split == 0 && o.combine_mode == 0 &&
                 u_bound < (int64_t(1) << 30);
    }
    c.sk_cost = stream_k ? cost : 0;
  }
  plan->lens.assign(lens, lens + c.num_seqs);
  if (q_start) plan->q_start.assign(q_start, q_start + c.num_seqs + 1);
  if (stream_k) {
    plan_stream_k(c, lens, o);
  } else if (!c.is_prefill) {
    // Split-KV decode ("2. Split-KV flash-decoding"): page-aligned splits of a
    // uniform number of blocks, so that no split is empty and each workgroup
    // streams at most blocks_per_split blocks.
    int64_t total_blocks = 0;
    int64_t max_nb = 0;
    for (int32_t s = 0; s < c.num_seqs; ++s) {
      const int64_t nb = ceil_div(lens[s], c.block_size);
      total_blocks += nb;
      max_nb = std::max(max_nb, nb);
    }
    // A split's blocks stream as one pipelined range, so for equal lengths
    // the best split size fills the CUs once (measured from 4 to 128 Ki
    // tokens). When the lengths are ragged (the longest over 1.25x the mean)
    // smaller splits, 1024 tokens' worth by default, keep the longest
    // sequences from forming a tail.
    const bool ragged = max_nb * 4 * c.num_seqs > total_blocks * 5;
    const int64_t max_bps =
        o.max_blocks_per_split ? o.max_blocks_per_split
        : ragged               ? std::max<int64_t>(1, 1024 / desc->block_size)
                               : std::max<int64_t>(max_nb, 1);
    int64_t bps;
    if (o.force_blocks_per_split > 0) {
      bps = o.force_blocks_per_split;
    } else {
      const int64_t target_wgs = int64_t(num_cus) * wgs_per_cu;
      bps = ceil_div(total_blocks * c.hkv, target_wgs);
      bps = std::max<int64_t>(bps, min_bps);
      bps = std::min<int64_t>(bps, std::max<int64_t>(max_bps, min_bps));
    }
    bps = std::min<int64_t>(bps, std::max<int64_t>(max_nb, 1));
    c.schedule = kScheduleUniform;
    c.blocks_per_split = static_cast<int32_t>(bps);
    c.max_splits = static_cast<int32_t>(ceil_div(max_nb, bps));
    c.max_tiles = 0;
    c.max_rows = 1;
    c.grid[0] = static_cast<uint32_t>(int64_t(c.max_splits) * c.hkv);
    c.grid[1] = static_cast<uint32_t>(c.num_seqs);
    c.grid[2] = 1;
    c.wg_size = kDecodeWaves * kWaveSize;
    const bool any_split = c.max_splits > 1;
    c.fused_combine = any_split && o.combine_mode == 0;
    c.combine_wgs =
        (any_split && !c.fused_combine) ? static_cast<uint32_t>(c.num_seqs * c.hkv) : 0;
    if (any_split) {
      auto round = [](size_t x) { return (x + kWsAlign - 1) / kWsAlign * kWsAlign; };
      const size_t n_part = size_t(c.num_seqs) * c.hq * c.max_splits;
      c.ws_cnt_off = 0;
      c.ws_ml_off = round(size_t(c.num_seqs) * c.hkv * kCounterStride * sizeof(uint32_t));
      c.ws_acc_off = c.ws_ml_off + round(n_part * 2 * sizeof(float));
      c.ws_bytes = c.ws_acc_off + round(n_part * c.d_pad * sizeof(float));
    } else {
      c.ws_cnt_off = c.ws_ml_off = c.ws_acc_off = c.ws_bytes = 0;
    }
  } else {
    // Chunked prefill: one workgroup per (sequence, KV head, tile). A tile is
    // kPrefillUnits units; a unit is one query head of the group times
    // kPrefillRowsPerWave query rows. Units are numbered head-fastest. Each
    // unit has two waves, which take alternate key tiles.
    int64_t max_tiles = 0, max_rows = 0;
    for (int32_t s = 0; s < c.num_seqs; ++s) {
      const int64_t n_q = int64_t(q_start[s + 1]) - q_start[s];
      max_rows = std::max(max_rows, n_q);
      const int64_t units = c.group * ceil_div(n_q, kPrefillRowsPerWave);
      max_tiles = std::max(max_tiles, ceil_div(units, kPrefillUnits));
    }
    c.schedule = 0;
    c.blocks_per_split = 0;
    c.max_splits = 1;
    c.max_tiles = static_cast<int32_t>(max_tiles);
    c.max_rows = static_cast<int32_t>(max_rows);
    c.grid[0] = static_cast<uint32_t>(max_tiles * c.hkv);
    c.grid[1] = static_cast<uint32_t>(c.num_seqs);
    c.grid[2] = 1;
    c.wg_size = kPrefillWaves * kWaveSize;
    c.combine_wgs = 0;
    c.fused_combine = 0;
    c.ws_cnt_off = c.ws_ml_off = c.ws_acc_off = c.ws_bytes = 0;
  }
  *out = plan;
  return NP_OK;
}

void np_plan_destroy(np_plan_t* plan) {
  if (plan && plan->magic == kPlanMagic) {
    plan->magic = 0;
    delete plan;
  }
}

size_t np_plan_workspace_bytes(const np_plan_t* p) {
  return (p && p->magic == kPlanMagic) ? p->core.ws_bytes : 0;
}

int32_t np_plan_blocks_per_split(const np_plan_t* p) {
  return (p && p->magic == kPlanMagic) ? p->core.blocks_per_split : -1;
}

int32_t np_plan_max_splits(const np_plan_t* p) {
  return (p && p->magic == kPlanMagic) ? p->core.max_splits : -1;
}

int32_t np_plan_schedule(const np_plan_t* p) {
  return (p && p->magic == kPlanMagic) ? p->core.schedule : -1;
}

int32_t np_plan_is_prefill(const np_plan_t* p) {
  return (p && p->magic == kPlanMagic) ? p->core.is_prefill : -1;
}

// The work-item list is built once, on the first accessor call.
static const std::vector<int32_t>& plan_items(const np_plan_t* p) {
  std::call_once(p->items_once, [p] { build_items(*p, p->items); });
  return p->items;
}

int64_t np_plan_num_work_items(const np_plan_t* p) {
  return (p && p->magic == kPlanMagic) ? int64_t(plan_items(p).size() / 5) : -1;
}

np_status np_plan_work_item(const np_plan_t* p, int64_t index, int32_t item[5]) {
  if (p == nullptr || p->magic != kPlanMagic || item == nullptr) return NP_ERR_NULL_PTR;
  const std::vector<int32_t>& items = plan_items(p);
  if (index < 0 || index >= int64_t(items.size() / 5)) return NP_ERR_BAD_SHAPE;
  std::memcpy(item, items.data() + index * 5, 5 * sizeof(int32_t));
  return NP_OK;
}

np_status np_plan_launch_shape(const np_plan_t* p, uint32_t grid[3], uint32_t* wg_size,
                               uint32_t* combine_wgs) {
  if (p == nullptr || p->magic != kPlanMagic) return NP_ERR_BAD_PLAN;
  if (grid) std::memcpy(grid, p->core.grid, sizeof(p->core.grid));
  if (wg_size) *wg_size = p->core.wg_size;
  if (combine_wgs) *combine_wgs = p->core.combine_wgs;
  return NP_OK;
}

}  // extern "C"
