// State shared by the fake HIP runtime and the sanitizer driver.
#pragma once
#include <stddef.h>

struct FakeState {
  size_t quant_need = 0;  // workspace bytes the fake planner asks of call 1
  size_t gemm_need = 0;   // ... and of call 2
  int launches = 0;
  const char* last = "";
  const void* last_out = nullptr;
  const void* last_ws = nullptr;
  size_t last_ws_bytes = 0;
  int last_window[4] = {0, 0, 0, 0};
};
extern FakeState g_fake;
