// Thread-local error reporting of the C ABI (no HIP dependency, so the
// schedule and the argument checks build and run without a GPU).
#pragma once

#include <string>

#include "dfa.h"

namespace dfa {
void set_error(const std::string& msg);
dfa_status fail(dfa_status st, const std::string& msg);
}  // namespace dfa
