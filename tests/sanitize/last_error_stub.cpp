// last_error_stub.cpp -- the last-error plumbing of libpkv for a host-only build of
// the block allocator (csrc/block_manager.cpp) under the address and
// undefined-behaviour sanitizers; the HIP sources that normally provide it are
// not part of that build.
#include <string>

#include "pkv_error.h"

namespace {
thread_local std::string g_msg;
}

namespace pkv {
void set_last_error(const std::string& msg) { g_msg = msg; }
void clear_last_error() { g_msg.clear(); }
}  // namespace pkv

extern "C" const char* pkv_last_error(void) { return g_msg.c_str(); }
