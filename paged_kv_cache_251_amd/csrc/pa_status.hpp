// Status reporting and internal accessors shared by the host-side translation units of
// libpagedattn.
#pragma once

#include <string>

#include "pagedattn.h"

namespace pa {

// Thread-local text of the last failure (pa_last_error).
extern thread_local std::string g_last_error;
// Record a failure and return its status.
pa_status_t fail(pa_status_t st, const char* fmt, ...) __attribute__((format(printf, 2, 3)));
// Clear the last failure and return PA_OK.
pa_status_t ok();

// Pool geometry of a block manager (block_manager.cpp).
int32_t bm_block_size(const pa_block_manager* manager);
int32_t bm_num_blocks(const pa_block_manager* manager);

}  // namespace pa
