// What the recording launchers of stubs.cpp saw on their last call.
#pragma once
#include <stddef.h>
#include <stdint.h>

namespace hostcheck {
struct Record {
  char op[32];
  int B, gamma, V, r, d, mode, suppressed;
  float T;
  uint64_t round;
  bool bf16;
  void* ws;
  const void* p[10];
};
extern Record last;
extern int suppress_depth;  // live ProfSuppress objects
}  // namespace hostcheck
