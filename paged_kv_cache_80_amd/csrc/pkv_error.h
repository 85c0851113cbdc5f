// pkv_error.h -- the library-wide last-error message, shared by the host-only
// sources (no HIP types here).
#pragma once

#include <string>

namespace pkv {

// Set / clear the message pkv_last_error() returns on this thread.
void set_last_error(const std::string& msg);
void clear_last_error();

}  // namespace pkv
