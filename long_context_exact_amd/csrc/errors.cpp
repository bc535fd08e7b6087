#include "errors.hpp"

namespace dfa {
namespace {
thread_local std::string g_last_error;
}

void set_error(const std::string& msg) { g_last_error = msg; }

dfa_status fail(dfa_status st, const std::string& msg) {
  g_last_error = msg;
  return st;
}
}  // namespace dfa

extern "C" const char* dfa_last_error(void) { return dfa::g_last_error.c_str(); }
