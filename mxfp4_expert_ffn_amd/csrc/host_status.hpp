// Error reporting shared by the host-only sources of the library: the message
// is what moe_last_error() returns on this thread until the next call.
#pragma once

namespace moe {
int host_fail(int code, const char *msg);  // records msg, returns code
int host_ok();                             // clears the message, returns MOE_OK
}  // namespace moe
