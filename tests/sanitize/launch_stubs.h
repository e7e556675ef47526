// The last launcher call the stubs in launch_stubs.cpp saw.
#pragma once
struct StubCall {
  const char* name = nullptr;
  int B = 0, T = 0, H = 0, HV = 0, K = 0, V = 0;
  const void* workspace = nullptr;
  int count = 0;
};
extern StubCall g_last;
