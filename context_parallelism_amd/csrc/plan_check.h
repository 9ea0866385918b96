// Validation of the forward and backward plans (host only). See
// plan_check.cpp; compiled in with -DCPATTN_CHECK_PLANS.
#pragma once

#include <cstdint>

#include "plan.h"

namespace cpattn {

// CP_OK if every record of `p` stays inside the rank's rows and keys and the
// spans expose each visible (row, key) pair exactly once; CP_EINVAL if not.
int32_t check_plan(const Meta& m, const Plan& p);
// check_plan on the dQ plan, plus the dK/dV key tiles, row blocks and bounds.
int32_t check_bwd_plan(const Meta& m, const BwdPlan& b);

}  // namespace cpattn
