// Internal entry points shared between the C ABI sources of libdsa.so (not
// part of the public interface).
#pragma once

#include <stddef.h>

#include "dsa.h"

namespace dsa {

// Supplies the workspace of a whole-layer call once every argument has been
// validated: receives the bytes the call needs, sets *ws and *ws_bytes, and
// returns DSA_OK or an error status (with the error recorded), in which case
// the call enqueues nothing.
typedef dsa_status (*WorkspaceProvider)(size_t need, void** ws, size_t* ws_bytes);

// dsa_forward with its workspace taken from `provider`: the same validation
// (every check runs on the host before anything is enqueued), the same
// kernels and the same results.
dsa_status forward_with_provider(const dsa_dims* dims, const void* qidx, const float* w, const void* kidx,
                                 const void* q, const void* k_cache, const void* v_cache, void* out, float* lse,
                                 int32_t* indices, uint32_t* mask, WorkspaceProvider provider, void* stream);

// Records `msg` as the thread's last error and returns `st`.
dsa_status set_error(dsa_status st, const char* msg);

}  // namespace dsa
