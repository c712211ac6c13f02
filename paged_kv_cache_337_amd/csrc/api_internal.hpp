// Internal entry points shared by the C ABI's translation units (not ABI).
#pragma once

#include <stddef.h>
#include <stdint.h>

#include <string>

#include "pa.h"

namespace pa {

// Sets the thread's error message and returns code.
int set_error(int code, const std::string& msg);

// The whole of pa_decode on a given workspace.  `noalloc` marks the entry
// point that brings its own static scratch: it skips the PA_DEBUG checks
// (which copy to pageable host memory and synchronise) and reports a
// workspace beyond the scratch as a size limit of that entry point.  `flat`
// marks the table-free comparison call: block_tables is then one first block
// id per sequence and max_blocks_per_seq is ignored.
// New tokens to write before the decode (pa_decode_step).
struct NewTokens {
  const void* k;
  const void* v;
  const int32_t* slot_mapping;
  int num_tokens;
};

// `share_plan`: device copy of pa_batch_share_plan's words for this batch
// (NULL: the device finds the sharing groups itself).
int decode_call(const pa_pool* pool, int layer, const void* q, int num_seqs, int num_q_heads,
                const int32_t* block_tables, int max_blocks_per_seq, const int32_t* context_lens,
                int max_context_len, float scale, int partition_tokens, void* workspace, size_t ws_bytes,
                void* out, void* stream, bool noalloc, bool flat = false, const NewTokens* write = nullptr,
                const int32_t* share_plan = nullptr);

}  // namespace pa
