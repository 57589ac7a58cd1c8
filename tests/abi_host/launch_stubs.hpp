// Shared state of the host-only launcher stand-ins (launch_stubs.cpp).
#pragma once

#include <cstdint>

struct StubLog {
  int launches = 0;
  const char* name = "";
  const void* p[3] = {nullptr, nullptr, nullptr};
  int fail = 0;            // make every launcher report a launch failure
  int last_error_set = 0;  // a runtime call failed and left an error behind
};
extern StubLog g_log;

constexpr uintptr_t kDevLo = 0x10000000, kDevHi = 0x20000000;
constexpr uintptr_t kPinLo = 0x30000000, kPinHi = 0x40000000;
constexpr uintptr_t kPinShift = 0x100000000ull;
