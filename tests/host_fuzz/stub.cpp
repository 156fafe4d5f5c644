// Host-only stand-in for the one C ABI call of the HIP-facing layer that the
// plan, draft-tree and pool sources need, so that they build without the HIP
// runtime (errors.cpp, the real error reporting, is linked as it is).
#include "ta_internal.h"
extern "C" void tree_attn_plan_destroy(ta_plan* plan) { delete plan; }
