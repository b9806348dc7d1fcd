// Chunked prefill over a paged cache (placeholder until the MFMA kernel lands).
#include <hip/hip_runtime.h>

#include "np_internal.h"

using namespace np;

extern "C" np_status np_paged_attention_prefill(const np_paged_desc* desc,
                                                const np_plan_t* plan, const void* q,
                                                const void* k_pool, const void* v_pool,
                                                const int32_t* block_table,
                                                const int32_t* context_lens,
                                                const int32_t* q_start, void* out,
                                                void* workspace, size_t workspace_bytes,
                                                void* stream) {
  (void)workspace; (void)workspace_bytes; (void)stream;
  np_status st = check_desc(desc);
  if (st != NP_OK) return st;
  st = check_pointers(desc, q, k_pool, v_pool, block_table, context_lens, out);
  if (st != NP_OK) return st;
  if (q_start == nullptr) return NP_ERR_NULL_PTR;
  st = check_plan(desc, plan, 1);
  if (st != NP_OK) return st;
  return NP_ERR_UNSUPPORTED;
}
