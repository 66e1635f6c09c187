// Call records of the stand-in launchers (abi_stubs.cpp).
#pragma once

#include <hip/hip_runtime_api.h>

#include <string>
#include <vector>

#include "../../mixed_precision_moe_amd/csrc/internal.h"

struct Call {
  std::string name;
  const void* p[13] = {};
  int64_t i[6] = {};
  size_t off[6] = {};
  GemmArgs gemm = {};
};

extern std::vector<Call> g_calls;
extern int g_events;
