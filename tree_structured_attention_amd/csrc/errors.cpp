// Error reporting of libtree_attn's C ABI: the thread-local last-error
// message and the mapping of exceptions to status codes.  Host-only, no HIP.
#include <cstdio>
#include <new>
#include <stdexcept>
#include <string>

#include "ta_internal.h"

namespace ta {

// The last error message of this thread, in a fixed buffer: recording an
// error never allocates, so it works when the host is out of memory.
static thread_local char g_last_error[512];

static void set_error_c(const char* msg) noexcept { std::snprintf(g_last_error, sizeof g_last_error, "%s", msg); }

void set_error(const std::string& msg) { set_error_c(msg.c_str()); }

int fail(int code, const std::string& msg) {
  set_error_c(msg.c_str());
  return code;
}

// Called from the catch-all handler of every exported function: maps the
// exception in flight to a status (host allocation failure -> capacity) so
// that none crosses the C ABI.
int fail_exception(const char* who) noexcept {
  char buf[160];
  int code = TA_ERR_INVALID_ARG;
  try {
    throw;
  } catch (const std::bad_alloc&) {
    code = TA_ERR_CAPACITY;
    std::snprintf(buf, sizeof buf, "%s: out of host memory", who);
  } catch (const std::length_error&) {
    code = TA_ERR_CAPACITY;
    std::snprintf(buf, sizeof buf, "%s: host table too large", who);
  } catch (...) {
    std::snprintf(buf, sizeof buf, "%s: internal error", who);
  }
  set_error_c(buf);
  return code;
}

}  // namespace ta

extern "C" const char* tree_attn_last_error(void) { return ta::g_last_error; }
