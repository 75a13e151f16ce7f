// Internal interface between the C-ABI source files (not exported in h3k.h):
// the error message setter and the validated forward of one block or a stack.
#pragma once
#include <stdint.h>

#include "h3k.h"

namespace h3k {

// Sets the thread's h3k_last_error() message and returns `code`.
h3k_status api_fail(h3k_status code, const char* fmt, ...);

// Validates every argument, then enqueues n_blocks blocks on `stream`
// (h3k_dit_block_forward / h3k_dit_stack_forward semantics).
h3k_status api_forward(const h3k_dit_config* cfg, const h3k_dit_block_weights* blocks, int32_t n_blocks,
                       const void* x, const void* c, void* out, void* workspace, uint64_t workspace_bytes,
                       hipStream_t stream, h3k_dit_stats* stats);

}  // namespace h3k
