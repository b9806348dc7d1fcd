/*
 * np_trace.h -- the trace build of the paged-attention library
 * (libnp_paged_trace.so): the same C ABI as np_paged.h plus one call that
 * registers a device buffer into which the decode kernels write one record
 * per workgroup. It exists to answer "which blocks did workgroup w actually
 * read, and where did its time go" ("Day 23: the real triton.jit
 * paged-attention kernel", section "Why it matters": a planner bug shows up
 * as a wrong tile, so the tiles a program reads must be inspectable), for
 * the tests and the measurement scripts. The product library
 * libnp_paged.so has no trace code and does not export np_debug_set_trace.
 *
 * Timing in the trace build differs from the product: every timestamp first
 * waits for all of the wave's outstanding memory operations.
 */
#ifndef NP_TRACE_H
#define NP_TRACE_H

#include <stddef.h>
#include <stdint.h>

#include "np_paged.h"

#ifdef __cplusplus
extern "C" {
#endif

/*
 * Uniform-split decode kernel: NP_TRACE_UNIFORM_WORDS int32 words per
 * workgroup, at word (blockIdx.y * gridDim.x + blockIdx.x) *
 * NP_TRACE_UNIFORM_WORDS, written by thread 0 of every workgroup that
 * starts (workgroups past a sequence's last split write only word 0 = 1):
 *   [0] 1 | 2 (merged the splits) | 4 (wrote out directly)
 *   [1] hardware location (__smid(): XCC << 6 | shader engine << 4 | CU)
 *   [2] sequence  [3] KV head  [4] split  [5] first block  [6] end block
 *   [7] arrival ticket taken (the counter's previous value), -1 if none
 *   [8] splits of the sequence  [9] 0
 *   [10 + 2 i], [11 + 2 i]: low and high word of stamp i (s_memrealtime,
 *   100 MHz ticks; 0 if the workgroup did not reach it), i < NP_TRACE_STAMPS:
 *     0 start, 1 q / table / length loads arrived, 2 first group of K/V
 *     arrived (wave 0), 3 wave 0's blocks computed, 4 workgroup merged
 *     and its partial (or output) stores issued, 5 stores acknowledged,
 *     6 ticket known, 7 split merge done (merging workgroup), 8 end.
 */
#define NP_TRACE_STAMPS 9
#define NP_TRACE_UNIFORM_WORDS 32

/*
 * Stream-K decode kernel: NP_TRACE_SK_WORDS words per workgroup, at word
 * blockIdx.x * NP_TRACE_SK_WORDS:
 *   [0] pieces recorded  [1] merges recorded  [2] hardware location
 *   [3] overflow (more than NP_TRACE_SK_PIECES pieces or a merge of more
 *       than NP_TRACE_SK_SLOTS pieces; the extra entries are not recorded)
 *   [4] U (units in all)  [5] C (units per workgroup)  [6..7] 0
 *   piece i at word 8 + 8 i, i < NP_TRACE_SK_PIECES, in the order taken:
 *     sequence, head group, first block, end block, partial slot (-1 when
 *     the segment has one piece and writes out directly), pieces of the
 *     segment, arrival ticket taken (-1 when direct), first unit
 *   merge j at word NP_TRACE_SK_MERGE0 + NP_TRACE_SK_MERGE_WORDS j, j < 2:
 *     sequence, head group, pieces, first unit of the segment, workgroup of
 *     its first piece, 0, 0, 0, then the partial slot read for each piece
 *     in piece order (NP_TRACE_SK_SLOTS words).
 * A partial slot p holds (m, l) at ws_ml[p * HW * G ...] and acc after it,
 * HW * G query heads per slot (HW KV heads per workgroup).
 */
#define NP_TRACE_SK_PIECES 32
#define NP_TRACE_SK_SLOTS 768
#define NP_TRACE_SK_MERGE0 (8 + 8 * NP_TRACE_SK_PIECES)
#define NP_TRACE_SK_MERGE_WORDS (8 + NP_TRACE_SK_SLOTS)
/*
 * Stream-K timestamps (s_memrealtime, 100 MHz; low word, then high word; 0 if
 * not reached), from word NP_TRACE_SK_STAMP0 of the workgroup's record, taken
 * by wave 0 after waiting for its outstanding memory operations:
 *   [0] start  [2] schedule known (length scan done)  [4] pieces done
 *   [6] end (merges done)
 *   piece i < NP_TRACE_SK_PIECES: [8 + 4 i] start, [10 + 4 i] partial or
 *     output written (and, for a shared segment, its ticket taken)
 *   merge j < 2: [8 + 4 NP_TRACE_SK_PIECES + 4 j] start, [+ 2] end
 */
#define NP_TRACE_SK_STAMP0 (NP_TRACE_SK_MERGE0 + 2 * NP_TRACE_SK_MERGE_WORDS)
#define NP_TRACE_SK_STAMP_WORDS (8 + 4 * NP_TRACE_SK_PIECES + 8)
#define NP_TRACE_SK_WORDS 2048

/*
 * Register the trace buffer used by the decode launches that follow (device
 * memory, 4-byte aligned, `bytes` long; NULL turns tracing off). A launch
 * whose grid needs more than `bytes` returns NP_ERR_WORKSPACE_TOO_SMALL
 * before it starts. The library does not clear the buffer: clear it before
 * a launch to tell written records from stale ones. Process-wide, not
 * thread-safe.
 */
np_status np_debug_set_trace(void* buf, size_t bytes);

#ifdef __cplusplus
}
#endif

#endif /* NP_TRACE_H */
