// Interface between the host-only launcher stand-ins (launch_stubs.cpp) and the
// sanitizer driver (abi_check.cpp).
#pragma once

#include <stddef.h>

#include <string>

namespace hostcheck {
extern int g_launches;            // launches recorded since reset()
extern int g_violations;          // device ranges outside every registered buffer
extern std::string g_first_violation;
void reset();
void add_alloc(const void* p, size_t n, const char* name);
bool detects_out_of_range();  // self-test of the range check
}  // namespace hostcheck
