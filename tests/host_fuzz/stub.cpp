// Host-only stand-ins for the two helpers of the C ABI layer that the plan,
// draft-tree and pool sources call, so that they build without the HIP runtime.
#include <string>
#include "ta_internal.h"
namespace ta {
static thread_local std::string g_last_error;
void set_error(const std::string& msg) { g_last_error = msg; }
int fail(int code, const std::string& msg) { g_last_error = msg; return code; }
}
extern "C" void tree_attn_plan_destroy(ta_plan* plan) { delete plan; }
