// Internal host-side declarations shared by host.cpp and model.cpp.
#pragma once
#include <vector>

#include "launch.h"

struct ExecDesc {
  int layer;  // weight layer
  int full;   // 1 = full attention, 0 = Gated-DeltaNet
  int slot;   // KV slot (full) or state slot (GDN)
  int loop, fork, merge;
};

int loop_fail(int code, const char* fmt, ...);
int loop_hip_fail(hipError_t e, const char* what);
int validate_config(const loop_config* c);
int build_schedule(const loop_config& c, std::vector<ExecDesc>& out);
