/*
 * np_paged.h -- C ABI of the paged-attention library for AMD MI355X (gfx950).
 *
 * The library computes, for every sequence s, query row i and query head h,
 *
 *     out[s,i,h,:] = sum_t softmax_t(scale * <q[s,i,h,:], K_s[t]>) * V_s[t]
 *
 * over the keys t <= past_s + i of KV head h / (Hq / Hkv), where K_s[t] and
 * V_s[t] are read through the sequence's block table from a pool of
 * fixed-size physical blocks. Sources, by page title and section:
 *
 *   - "I Wrote the Three Attention Kernels That Run LLM Inference -- in
 *     Portable Triton, on a Free Colab T4": "What is attention, really?"
 *     (the definition), "3. Paged KV-cache attention" (page lookup through
 *     the block table; GQA-aware), "2. Split-KV flash-decoding" (splitting the
 *     KV range across workgroups and merging the splits by log-sum-exp).
 *   - "Day 23: the real triton.jit paged-attention kernel": "What I added
 *     today" (every integer that becomes a pointer -- slot stride, past, grid,
 *     padded tile sizes -- is computed by plain host code that is tested
 *     without a GPU) and "What I learned", item 1 (pad head_dim to a power of
 *     two and mask the lanes past the real extent, as for the ragged tail).
 *
 * Layout (all strides in ELEMENTS; the last dimension of every tensor is
 * contiguous):
 *   q            [n_q_total, Hq, head_dim]        strides q_stride[0..1]
 *   k_pool/v_pool[n_blocks, block_size, Hkv, d]   strides kv_stride[0..2]
 *   out          [n_q_total, Hq, head_dim]        strides out_stride[0..1]
 *   block_table  int32 [num_seqs, max_blocks_per_seq], row stride bt_stride
 *   context_lens int32 [num_seqs]  -- cached tokens INCLUDING the current
 *                query tokens, whose K/V are already in the pool
 *   q_start      int32 [num_seqs + 1] (prefill only) -- rows of sequence s
 *                are q_start[s] .. q_start[s+1]-1; past_s = context_lens[s]
 *                - (q_start[s+1] - q_start[s]).
 * Token t of sequence s lives in slot t % block_size of physical block
 * block_table[s, t / block_size].
 *
 * Ownership: every device buffer is allocated by the caller. A plan is owned
 * by the library, created by np_plan and released by np_plan_destroy. The
 * library keeps no mutable global state; all calls are reentrant.
 *
 * Errors: every function returns an np_status; nothing throws or aborts
 * across this ABI. Device-side block-table entries that disagree with what
 * the host validated are undefined behaviour (the kernels clamp table reads
 * to the table's width but not entry values to the pool). Device-side
 * lengths are read by the kernels: a device context length outside
 * [1, max_blocks_per_seq * block_size], or one the plan's grid does not cover
 * (see np_paged_attention_decode and _prefill), yields NaN in the affected
 * outputs, never a silent truncation.
 */
#ifndef NP_PAGED_H
#define NP_PAGED_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum np_dtype { NP_F32 = 0, NP_F16 = 1, NP_BF16 = 2 } np_dtype;

typedef enum np_status {
  NP_OK = 0,
  NP_ERR_NULL_PTR = 1,        /* a required pointer is NULL                    */
  NP_ERR_BAD_DTYPE = 2,       /* dtype not one of np_dtype                     */
  NP_ERR_BAD_SHAPE = 3,       /* a size is < 1, block_size not a power of two,
                                 or q rows do not match the sequences          */
  NP_ERR_BAD_STRIDE = 4,      /* a stride is too small (rows would overlap)    */
  NP_ERR_MISALIGNED = 5,      /* a pointer or row is not 16-byte aligned       */
  NP_ERR_BAD_GQA = 6,         /* Hq is not a multiple of Hkv                   */
  NP_ERR_BAD_CONTEXT_LEN = 7, /* context_len < query rows or > table capacity  */
  NP_ERR_BAD_BLOCK_TABLE = 8, /* a used table entry is outside [0, n_blocks)   */
  NP_ERR_UNSUPPORTED = 9,     /* valid, but no kernel is built for this shape  */
  NP_ERR_WORKSPACE_TOO_SMALL = 10,
  NP_ERR_BAD_PLAN = 11,       /* plan missing or made for another descriptor   */
  NP_ERR_HIP = 12,            /* a HIP launch reported an error                */
  NP_ERR_POOL_EXHAUSTED = 13  /* the block allocator has too few free blocks   */
} np_status;

/*
 * Contiguous caches. Every entry point that takes a block table accepts NULL
 * for it: logical block j of sequence s is then physical block
 * s * max_blocks_per_seq + j, which needs n_blocks >= num_seqs *
 * max_blocks_per_seq (else NP_ERR_BAD_BLOCK_TABLE). With kv_stride[0] =
 * block_size * kv_stride[1] the pools are then dense
 * [num_seqs, max_blocks_per_seq * block_size, Hkv, d] tensors: the split-KV
 * decode over one contiguous KV tensor of "I Wrote the Three Attention
 * Kernels That Run LLM Inference", section "2. Split-KV flash-decoding", and
 * its fused prefill (section "1. Fused prefill attention").
 */

/* Shape and stride descriptor shared by every call. */
typedef struct np_paged_desc {
  int32_t dtype;              /* np_dtype of q, the pools and out              */
  int32_t num_seqs;
  int32_t n_q_total;          /* query rows: num_seqs for decode               */
  int32_t num_q_heads;        /* Hq                                            */
  int32_t num_kv_heads;       /* Hkv; Hq % Hkv == 0                            */
  int32_t head_dim;           /* d                                             */
  int32_t block_size;         /* slots per physical block, power of two        */
  int32_t n_blocks;           /* physical blocks in each pool                  */
  int32_t max_blocks_per_seq; /* block-table width                             */
  int32_t reserved0;          /* must be 0                                     */
  int64_t q_stride[2];        /* [row, head]                                   */
  int64_t kv_stride[3];       /* [block, slot, head]; same for K and V         */
  int64_t out_stride[2];      /* [row, head]                                   */
  int64_t bt_stride;          /* block-table row stride                        */
  float scale;                /* <= 0 selects 1/sqrt(head_dim)                 */
  int32_t reserved1;          /* must be 0                                     */
} np_paged_desc;

/* Planner knobs; pass NULL for the defaults. */
typedef struct np_plan_opts {
  int32_t num_cus;                /* compute units to fill; 0 => 256           */
  int32_t wgs_per_cu;             /* target workgroups per CU; 0 => 1          */
  int32_t min_blocks_per_split;   /* 0 => 4 (uniform); stream-K: least units
                                     per workgroup, 0 => 8                     */
  int32_t max_blocks_per_split;   /* uniform splits; 0 => no cap for equal
                                     lengths (the split fills the CUs once),
                                     1024 tokens' worth of blocks when the
                                     longest sequence has over 1.25x the mean */
  int32_t force_blocks_per_split; /* > 0: use exactly this split size          */
  int32_t combine_mode;           /* 0: the last split workgroup of each
                                     (sequence, KV head) merges the splits in
                                     the same launch; 1: a separate combine
                                     kernel does it                            */
  int32_t schedule;               /* decode work split: 0 auto (stream-K when
                                     num_seqs > 1, the longest sequence has
                                     more than 1.25x the mean blocks, the
                                     stream-K launch would be full (U >=
                                     num_cus * wgs_per_cu * min_units), and
                                     nothing above asks for uniform splits),
                                     1 uniform splits, 2 stream-K              */
  int32_t segment_cost;           /* stream-K: fixed cost of one (sequence, KV
                                     head), in blocks; 0 => 4                  */
  int32_t reserved;               /* must be 0                                 */
} np_plan_opts;

typedef struct np_plan_s np_plan_t;   /* opaque, host memory only */

/*
 * np_check_paged_inputs -- validate a call without touching the GPU.
 *
 * ("Day 23: the real triton.jit paged-attention kernel", section "What I
 * added today": every integer the kernels turn into a pointer or a bound is
 * checked by host code that runs without a GPU; the shapes checked are the
 * problem statement of "3. Paged KV-cache attention" in "I Wrote the Three
 * Attention Kernels That Run LLM Inference".)
 * Checks the descriptor, the device pointers (non-NULL, 16-byte aligned for
 * q/pools/out, 4-byte for int32 arrays; block_table may be NULL, see
 * "Contiguous caches"), strides and GQA divisibility. When
 * the host copies are given it also checks 1 <= n_q_s <= context_lens[s] <=
 * max_blocks_per_seq * block_size (with q_start_host for prefill; decode has
 * one row per sequence) and that every used table entry, columns 0 ..
 * ceil(context_lens[s] / block_size) - 1, lies in [0, n_blocks). Host arrays
 * may be NULL to skip those checks. Returns the first error found.
 */
np_status np_check_paged_inputs(const np_paged_desc* desc, const void* q,
                                const void* k_pool, const void* v_pool,
                                const int32_t* block_table,
                                const int32_t* context_lens, const void* out,
                                const int32_t* block_table_host,
                                const int32_t* context_lens_host,
                                const int32_t* q_start_host);

/*
 * np_plan -- plan the split-KV decode or the chunked prefill for one batch.
 *
 * Pure host code, deterministic: the same inputs give the same plan bit for
 * bit. context_lens_host [num_seqs] is required. q_start_host NULL makes a
 * decode plan (one query row per sequence); otherwise a prefill plan.
 *
 * Decode: every sequence's ceil(L/block_size) logical blocks are cut into
 * splits of `blocks_per_split` consecutive blocks (the last may be shorter,
 * none is empty), one workgroup per (sequence, KV head, split), following the
 * split-KV partition of "2. Split-KV flash-decoding" with page-aligned,
 * never-empty splits. blocks_per_split = clamp(ceil(total_blocks * Hkv /
 * (num_cus * wgs_per_cu)), min, max), or the forced value.
 * Decode, stream-K schedule (for batches of ragged lengths; the same
 * partition into page-aligned pieces, cut for equal work instead of equal
 * size): a workgroup serves HW KV heads together (HW = 8, 4, 2 or 1, the largest
 * dividing Hkv); each (sequence, head group) is a segment of
 * ceil(L/block_size) blocks plus segment_cost virtual units; segments are
 * laid end to end in (sequence, head group) order, U units in all, and
 * workgroup w of W = max(1, min(num_cus * wgs_per_cu, ceil(U / min_units),
 * U)) takes units [w C, (w + 1) C), C = ceil(U / W). A segment's blocks
 * inside one workgroup's range form a piece (listed as one work item per KV
 * head of the group); a segment of several pieces is merged by the last
 * piece to finish, in the same launch. The kernel recomputes the schedule
 * from the device context_lens. At most 2048 sequences;
 * force_blocks_per_split and combine_mode 1 select uniform splits.
 * Prefill: one workgroup per (sequence, KV head, tile of query rows), the
 * tiles of later rows (more keys under the causal mask) launched first.
 *
 * On success *out owns a new plan; the caller releases it with
 * np_plan_destroy after the last launch that uses it. Planning costs
 * O(num_seqs) host work; the work-item list of the accessors below is built
 * on their first call (thread-safe) and kept with the plan.
 */
np_status np_plan(const np_paged_desc* desc, const int32_t* context_lens_host,
                  const int32_t* q_start_host, const np_plan_opts* opts,
                  np_plan_t** out);

void np_plan_destroy(np_plan_t* plan);

/* Device workspace bytes the plan's launches need (0 if none). */
size_t np_plan_workspace_bytes(const np_plan_t* plan);

/* Read-only plan accessors (for tests and the benchmark). */
/* Uniform splits: blocks per split and the most splits of a sequence.
 * Stream-K: units per workgroup (C) and the most pieces of one segment. */
int32_t np_plan_blocks_per_split(const np_plan_t* plan);
int32_t np_plan_max_splits(const np_plan_t* plan);
/* Decode schedule of the plan: 1 uniform splits, 2 stream-K (0 for prefill). */
int32_t np_plan_schedule(const np_plan_t* plan);
int32_t np_plan_is_prefill(const np_plan_t* plan);
int64_t np_plan_num_work_items(const np_plan_t* plan);
/* item[0..4] = sequence, kv head, split (stream-K: workgroup; prefill: query
 * tile), first block (or first query row, relative to the sequence), end
 * block (or end row). Items are listed in launch order of the active
 * workgroups (stream-K: by workgroup, then in the order it takes them). */
np_status np_plan_work_item(const np_plan_t* plan, int64_t index, int32_t item[5]);
/* grid[0..2] and the workgroup size of the main kernel; *combine_wgs is the
 * number of workgroups of the split-combine kernel (0 if no split). */
np_status np_plan_launch_shape(const np_plan_t* plan, uint32_t grid[3],
                               uint32_t* wg_size, uint32_t* combine_wgs);

/* Host-side helper exposed for tests: smallest power of two >= x (x >= 1). */
int32_t np_next_pow2(int32_t x);

/*
 * np_paged_attention_decode -- one query token per sequence.
 *
 * (The fused paged read of "3. Paged KV-cache attention" -- each sequence's
 * K/V found block by block through its table row, GQA-aware -- with the KV
 * range of a sequence split across workgroups and merged by the log-sum-exp
 * rule of "2. Split-KV flash-decoding", both in "I Wrote the Three Attention
 * Kernels That Run LLM Inference"; the attention itself as defined in "What
 * is attention, really?" of the same page.)
 * q/out [num_seqs, Hq, d]. Launches the split-KV decode kernel and, when any
 * sequence has more than one split, the combine kernel, asynchronously on
 * `stream` (a hipStream_t; NULL = the null stream). Never allocates, never
 * synchronises. `workspace` (device, 256-byte aligned) must hold
 * np_plan_workspace_bytes(plan) bytes. Its first bytes hold one 32-bit
 * arrival counter per (sequence, KV head): they must be zero before the first
 * call that uses the workspace (allocate it zeroed) and every call leaves them
 * zero again; the rest is scratch. Two calls that share a workspace must not
 * overlap in time (same stream, or ordered by events). Checks the descriptor
 * and pointers (not
 * the device arrays' values) and that the plan was made for this descriptor.
 * Built kernels: block_size 16; head_dim a multiple of 8 (16-bit types) or 4
 * (fp32) up to 128; Hq/Hkv from 1 to 8. Other valid shapes return
 * NP_ERR_UNSUPPORTED.
 * Device lengths: the stream-K schedule is recomputed on the device from
 * context_lens, so any valid device length is attended in full. Under
 * uniform splits the grid holds max_splits * blocks_per_split blocks per
 * sequence, fixed by the host lengths the plan was made for: a sequence
 * whose device length needs more (or is below 1 or above the table
 * capacity) gets NaN in all its output heads, so a plan reused across steps
 * must be remade once a length outgrows it.
 */
np_status np_paged_attention_decode(const np_paged_desc* desc, const np_plan_t* plan,
                                    const void* q, const void* k_pool,
                                    const void* v_pool, const int32_t* block_table,
                                    const int32_t* context_lens, void* out,
                                    void* workspace, size_t workspace_bytes,
                                    void* stream);

/*
 * np_paged_attention_decode_noalloc -- np_paged_attention_decode for callers
 * that cannot allocate device memory (code under HIP graph capture, tight
 * serving loops, harnesses that forbid hipMalloc). Same arguments, checks,
 * kernels and results, without the workspace: the workspace is a
 * library-owned 8 MiB device array, one per GPU, held until the process
 * ends. A plan whose np_plan_workspace_bytes exceeds 8 MiB returns
 * NP_ERR_WORKSPACE_TOO_SMALL before anything is launched (the 64-sequence
 * stream-K plan of the Llama head shape needs 2.3 MB). The first call on a
 * device looks the array up and clears it with a fill kernel on `stream`;
 * make that first call outside graph capture to keep the clear out of a
 * captured graph. Every call on a GPU shares that GPU's array, so calls that
 * overlap in time on one GPU race: order them (one stream, or events).
 * Allocates nothing and never synchronises.
 */
np_status np_paged_attention_decode_noalloc(const np_paged_desc* desc, const np_plan_t* plan,
                                            const void* q, const void* k_pool,
                                            const void* v_pool, const int32_t* block_table,
                                            const int32_t* context_lens, void* out,
                                            void* stream);

/*
 * np_paged_attention_prefill -- a chunk of n_q_s new query rows per sequence,
 * causal: row i of sequence s sees keys t <= past_s + i ("Day 23", "What I
 * added today": past is computed on the host side of the interface; here the
 * kernel derives it from context_lens and q_start exactly as stated above).
 * QK^T and PV run on the MFMA units in bf16/fp16 with fp32 accumulation.
 * Built kernels: bf16 and fp16, head_dim 64, block_size 16, Hq/Hkv 1..8.
 * q_start is a device array [num_seqs + 1]. Same stream, allocation and
 * error rules as decode. The grid covers the query rows of the host q_start
 * the plan was made for (the longest chunk, in tiles): device rows beyond
 * it, and every row of a sequence whose device length is below its row
 * count or above the table capacity, are set to NaN.
 */
np_status np_paged_attention_prefill(const np_paged_desc* desc, const np_plan_t* plan,
                                     const void* q, const void* k_pool,
                                     const void* v_pool, const int32_t* block_table,
                                     const int32_t* context_lens, const int32_t* q_start,
                                     void* out, void* workspace, size_t workspace_bytes,
                                     void* stream);

/*
 * Writing the cache ("Day 20: the number the Triton kernel has to beat",
 * section "What I learned": each step's write first extends the sequence's
 * block table, then stores the new tokens' K/V in their slots; the read then
 * attends over them).
 *
 * Block allocator (host). A pool of n_blocks physical blocks of block_size
 * slots, handed out to num_seqs sequences whose tables hold at most
 * max_blocks_per_seq entries. Free blocks form a stack: the first
 * allocations take free_order[0], free_order[1], ... (free_order NULL means
 * 0, 1, 2, ...), and a released sequence's blocks are pushed back, its first
 * block on top, so they are reused first, in that order. Deterministic: the
 * same calls give the same tables. The allocator owns its host memory; tables
 * and lengths are read through the accessors (valid until the next call that
 * changes them) and copied to the device by the caller. Not thread-safe.
 *
 * np_alloc_extend grows sequence `seq` to `new_len` tokens (new_len >= its
 * current length, at most max_blocks_per_seq * block_size), taking
 * ceil(new_len / block_size) - (blocks it has) blocks off the stack and
 * appending them to its table row. If too few blocks are free it returns
 * NP_ERR_POOL_EXHAUSTED and changes nothing. np_alloc_release frees every
 * block of `seq` and sets its length to 0. Unused table entries hold -1.
 */
typedef struct np_block_allocator np_block_allocator_t;

np_status np_alloc_create(int32_t n_blocks, int32_t block_size, int32_t num_seqs,
                          int32_t max_blocks_per_seq, const int32_t* free_order,
                          np_block_allocator_t** out);
void np_alloc_destroy(np_block_allocator_t* alloc);
np_status np_alloc_extend(np_block_allocator_t* alloc, int32_t seq, int32_t new_len);
np_status np_alloc_release(np_block_allocator_t* alloc, int32_t seq);
int32_t np_alloc_free_blocks(const np_block_allocator_t* alloc);
/* [num_seqs][max_blocks_per_seq] row-major, -1 where unused. */
const int32_t* np_alloc_block_table(const np_block_allocator_t* alloc);
/* [num_seqs] token counts. */
const int32_t* np_alloc_context_lens(const np_block_allocator_t* alloc);

/*
 * np_paged_kv_append -- scatter new K and V rows into the pool slots of their
 * positions. For sequence s, rows new_start[s] .. new_start[s+1]-1 of k_new
 * and v_new (each [n_q_total, Hkv, d], element strides new_stride[0] between
 * rows and new_stride[1] between heads, channels contiguous, 16-byte aligned)
 * are the tokens at positions past_s + i, past_s = context_lens[s] -
 * (new_start[s+1] - new_start[s]): context_lens already counts them, as for
 * prefill (append, then attend). Token t goes to slot t % block_size of
 * physical block block_table[s][t / block_size] of k_pool and v_pool, all
 * Hkv heads and d channels; nothing else in the pools changes. The table must
 * already cover the new positions (np_alloc_extend). `plan` is a prefill plan
 * made with new_start as q_start (it fixes the launch grid); desc.n_q_total is
 * the number of new rows. Asynchronous on `stream`; never allocates. Rows of
 * the same sequence must not be written by two overlapping calls.
 */
np_status np_paged_kv_append(const np_paged_desc* desc, const np_plan_t* plan,
                             const void* k_new, const void* v_new,
                             const int64_t new_stride[2], const int32_t* block_table,
                             const int32_t* context_lens, const int32_t* new_start,
                             void* k_pool, void* v_pool, void* stream);

/*
 * Reference kernels for measurement (not part of the attention path).
 * np_probe_empty launches one empty workgroup: the per-kernel floor.
 * np_probe_stream_read reads `bytes` (a multiple of 16) from 16-byte-aligned
 * device memory `src` once, with `num_wgs` workgroups of 256 threads, and
 * writes one 32-bit word per thread to `sink` (device, at least num_wgs * 1024
 * bytes). Both are asynchronous on `stream`.
 */
np_status np_probe_empty(void* stream);
np_status np_probe_stream_read(const void* src, size_t bytes, uint32_t num_wgs, void* sink,
                               size_t sink_bytes, void* stream);
/* The same read with wg_size threads per workgroup (a multiple of 64, at most
 * 1024) and loads_per_thread (1, 2, 4, 8 or 16) 16-byte loads of a thread in
 * flight at once; sink holds num_wgs * wg_size words. The single-launch read
 * ceiling is the best time over these shapes. */
np_status np_probe_stream_read_ex(const void* src, size_t bytes, uint32_t num_wgs,
                                  uint32_t wg_size, uint32_t loads_per_thread, void* sink,
                                  size_t sink_bytes, void* stream);

/* Human-readable name of a status code (static storage). */
const char* np_status_string(np_status status);

#ifdef __cplusplus
}
#endif

#endif /* NP_PAGED_H */
