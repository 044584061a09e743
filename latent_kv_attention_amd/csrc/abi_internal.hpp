// Host-side pieces of the C ABI layer shared between its source files.
#pragma once

#include <stddef.h>
#include <stdint.h>

#include "../../include/mla.h"

namespace mla_abi {

// Every check mla_flash_attend makes except those on its workspace; on
// MLA_OK, *ws_bytes is the workspace the call needs.
mla_status flash_check(const mla_shape* shape, const void* q_abs, int32_t q_n_frames, const void* cache,
                       const int32_t* slot_frame, const float* rope_tables, int32_t rope_t_first, int32_t rope_n_t,
                       const void* o_lat, int32_t kv_splits, size_t* ws_bytes);

// Enqueue mla_flash_attend's kernels with `workspace` (at least *ws_bytes of
// flash_check, device memory, 16-byte aligned); arguments already checked.
mla_status flash_run(const mla_shape* shape, const void* q_abs, int32_t q_n_frames, const void* cache,
                     const int32_t* slot_frame, const float* rope_tables, int32_t rope_t_first, int32_t rope_n_t,
                     void* o_lat, int32_t kv_splits, void* workspace, void* stream);

}  // namespace mla_abi
