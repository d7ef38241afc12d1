// Host-side helpers shared by the translation units of the C ABI (internal to
// the library; the public boundary is include/paged_attn.h).
#pragma once

namespace pa {

// Record `msg` as the calling thread's pa_last_error() text and return
// `status`.
int host_fail(int status, const char* msg);

}  // namespace pa
